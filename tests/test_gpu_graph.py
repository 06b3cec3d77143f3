"""The forward captured into a HIP graph (torch.cuda.CUDAGraph over the C
ABI's launches, which enqueue no memsets and allocate nothing): every replay
is bit-identical to the eager forward, with the program's own eager work and
synchronisations between the replays."""
import pytest
import torch

import ffn_inputs as fi
import w4a16_nvfp4_dense_amd as ffn

pytestmark = pytest.mark.gpu

# (M, K, N): the GEMV arm with activations in one and in three LDS pieces,
# the small-batch matrix-core arm (down projection in parts, with its
# reduction launch), and the 128-row arm (stream-K reduction launches).
CASES = [(1, 2048, 4096), (8, 1024, 12352), (16, 1024, 8192), (40, 512, 1024)]


def _weights(case):
    return [ffn.DeviceWeight.from_host(w) for w in (case.gate, case.up, case.down)]


@pytest.mark.parametrize("M,K,N", CASES, ids=[f"m{m}_k{k}_n{n}" for m, k, n in CASES])
@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_graph_replays_match_eager(M, K, N, noalloc):
    if noalloc and ffn.workspace_bytes(M, K, N) > 4 << 20:
        pytest.skip("workspace beyond the no-alloc scratch")
    case = fi.make_small(M, K, N, act=fi.ACT_GELU_TANH, seed=81 + M)
    other = fi.make_small(M, K, N, seed=91 + M)
    g, u, d = _weights(case)
    x = ffn.bf16_from_bits(case.x_bits)
    x2 = ffn.bf16_from_bits(other.x_bits)
    ws = torch.empty(max(ffn.workspace_bytes(M, K, N), 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")

    def run(xin, stream=None):
        if noalloc:
            return ffn.forward_noalloc(xin, g, u, d, out, case.act, stream=stream)
        return ffn.forward(xin, g, u, d, case.act, out=out, workspace=ws, stream=stream)

    eager = run(x).clone()
    eager2 = run(x2).clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(x, stream=torch.cuda.current_stream())
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        # eager work between replays, on the same buffers
        assert torch.equal(run(x2), eager2)
        torch.cuda.synchronize()
