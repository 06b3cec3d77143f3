"""ffn_nvfp4_forward_noalloc (the forward with the library's static scratch
in place of a workspace) against ffn_nvfp4_forward, through the C ABI: the
same kernels, so the outputs must be bit-identical (which also meets the
oracle bound the forward is held to). Two calls in a row, the second on a
smaller input, then the small-batch matrix-core arm (also with three token
groups and split reductions), and the rejection of a
shape whose workspace exceeds the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import ffn_inputs as fi
import oracle
import w4a16_nvfp4_dense_amd as ffn

pytestmark = pytest.mark.gpu


def _run(case):
    gate, up, down = (ffn.DeviceWeight.from_host(w) for w in (case.gate, case.up, case.down))
    x = ffn.bf16_from_bits(case.x_bits)
    ref = ffn.forward(x, gate, up, down, case.act)
    out = torch.full_like(ref, float("nan"))
    ffn.forward_noalloc(x, gate, up, down, out, case.act)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_matches_forward_twice():
    big = fi.make_config(3, M=8)                     # 5120 / 17408: h is 278,528 bytes
    out, ref = _run(big)
    assert torch.equal(out, ref)
    small = fi.make_small(2, 1024, 2048, act=fi.ACT_GELU_TANH, seed=71)
    out, ref = _run(small)
    assert torch.equal(out, ref)
    # and within the oracle bound the forward is held to
    got = ffn.bf16_to_f64(out)
    exp = oracle.ffn(small)
    assert np.all(np.abs(got - exp) <= oracle.parity_bound(exp))


def test_noalloc_small_batch_arm():
    case = fi.make_small(16, 1024, 2048, seed=72)   # matrix-core small-batch arm: h and partial sums
    assert ffn.workspace_bytes(16, 1024, 2048) <= 4 << 20
    out, ref = _run(case)
    assert torch.equal(out, ref)


def test_noalloc_three_token_groups_split():
    """Three token groups with the dual reduction split in 3 parts (K = 5120):
    the partial sums and the ready words live in the static scratch, and a
    second call finds the words the first one cleared."""
    case = fi.make_small(36, 5120, 2048, seed=73)
    assert ffn.workspace_bytes(36, 5120, 2048) <= 4 << 20
    for _ in range(2):
        out, ref = _run(case)
        assert torch.equal(out, ref)


def test_noalloc_rejects_oversized_workspace():
    M, K, N = 128, 5120, 17408                       # the 128-row arm needs about 64 MiB
    assert ffn.workspace_bytes(M, K, N) > 4 << 20
    lib = ffn.load()
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    w = ffn.WeightStruct(dummy.data_ptr(), dummy.data_ptr(), 1.0)
    rc = lib.ffn_nvfp4_forward_noalloc(dummy.data_ptr(), M, K, N, ctypes.byref(w), ctypes.byref(w),
                                       ctypes.byref(w), 0, dummy.data_ptr(), None)
    assert rc == ffn.ERR_WORKSPACE
