"""GPU parity of the small-batch matrix-core arm (9 <= M <= 40 token rows,
K and N multiples of 256) against the CPU oracle, with the
bounds of the other arms: |out - out_ref| <= 1e-2 rms(out_ref) + 1 bf16 ulp(out_ref); the dual
entry's fp32 gate/up within 1e-4 rms(ref) + 1e-6 |ref|.
"""
import numpy as np
import pytest
import torch

import ffn_inputs as fi
import oracle
import w4a16_nvfp4_dense_amd as ffn
from test_gpu_parity import assert_dual_close, assert_ffn_close, loaded

pytestmark = pytest.mark.gpu

# (M, K, N, act, seed). A round is 1024 reduction columns (16 waves x 64);
# the shapes give one-round reductions with idle waves (K = 256, 768), a short
# last round (K = 1280, N = 1280), the longest one-part reduction (K = 5120:
# five rounds), down projections split in two parts with partial sums and the
# in-order reduction (N = 6144, 8192), one to three row tiles per workgroup,
# and 9 to 16 token rows.
SMALL_BATCH = [
    (9, 256, 512, fi.ACT_SILU, 51),
    (12, 768, 1280, fi.ACT_GELU_TANH, 52),
    (16, 1280, 2048, fi.ACT_SILU, 53),
    (10, 4096, 512, fi.ACT_GELU_TANH, 54),
    (16, 2048, 8192, fi.ACT_SILU, 55),
    (13, 5120, 6144, fi.ACT_GELU_TANH, 56),
    (11, 5120, 1024, fi.ACT_SILU, 57),
    # two token groups (17 <= M <= 32): the second group from one row to
    # full, the dual projection in one part (K <= 4096) and in two (K = 5120,
    # with the paired reduction and the activation epilogue), down
    # projections in one and several parts
    (17, 256, 512, fi.ACT_SILU, 61),
    (24, 1280, 2048, fi.ACT_GELU_TANH, 62),
    (32, 4096, 1024, fi.ACT_SILU, 63),
    (20, 5120, 2048, fi.ACT_GELU_TANH, 64),
    (31, 2048, 8192, fi.ACT_SILU, 65),
    (32, 5120, 6144, fi.ACT_GELU_TANH, 66),
    # one token group with the dual projection split (K above 5120)
    (12, 5376, 1024, fi.ACT_SILU, 67),
    # down projections in more parts than the finishing workgroup loads in
    # one batch (4): 5 parts (N = 21504) with one and two token groups, and
    # 13 parts (N = 65536: three full batches and one part)
    (12, 512, 21504, fi.ACT_GELU_TANH, 69),
    (20, 256, 21504, fi.ACT_SILU, 70),
    (9, 256, 65536, fi.ACT_SILU, 71),
    # three token groups (33 <= M <= 40): one row of the third group to a
    # full batch; the dual projection in one part (2 rounds, its most),
    # two (K = 4096) and three (K = 5120, the activation epilogue after the
    # parts); the down projection in one part (3 rounds, its most), three
    # (N = 8192), seven (N = 21504) and 22 (N = 65536) parts
    (33, 256, 512, fi.ACT_SILU, 81),
    (40, 1280, 2048, fi.ACT_GELU_TANH, 82),
    (36, 5120, 2048, fi.ACT_SILU, 83),
    (40, 4096, 8192, fi.ACT_GELU_TANH, 84),
    (34, 2048, 3072, fi.ACT_SILU, 85),
    (39, 256, 21504, fi.ACT_GELU_TANH, 86),
    (35, 256, 65536, fi.ACT_SILU, 87),
    # K = 5376 (21 blocks of 256 columns): parts of unequal length, 10 and 11
    # blocks with two token groups, 7 each with three (1.75 rounds)
    (20, 5376, 1024, fi.ACT_SILU, 89),
    (37, 5376, 1024, fi.ACT_GELU_TANH, 90),
]
IDS = [f"m{m}_k{k}_n{n}_a{a}" for m, k, n, a, _ in SMALL_BATCH]


def case_of(M, K, N, act, seed):
    return fi.make_small(M, K, N, act=act, seed=seed)


@pytest.mark.parametrize("M,K,N,act,seed", SMALL_BATCH, ids=IDS)
def test_smallbatch_forward(M, K, N, act, seed):
    case = case_of(M, K, N, act, seed)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    torch.cuda.synchronize()
    assert_ffn_close(out, oracle.ffn(case), case.name)


@pytest.mark.parametrize("M,K,N,act,seed", SMALL_BATCH, ids=IDS)
def test_smallbatch_dual_entry(M, K, N, act, seed):
    case = case_of(M, K, N, act, seed)
    L = loaded(case.name, lambda: case)
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    torch.cuda.synchronize()
    g_ref, u_ref = oracle.dual(case)
    assert_dual_close(g, g_ref, "gate")
    assert_dual_close(u, u_ref, "up")


def test_smallbatch_workspace():
    """The small-batch arm keeps h = act(gate) * up and, when a projection's
    reduction is split, its fp32 partial sums and one ready word (8 bytes)
    per workgroup of the split grid."""
    r256 = lambda b: (b + 255) // 256 * 256
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert ffn.workspace_bytes(9, 256, 512) == r256(9 * 512 * 2)
    # N = 17408: 68 blocks of 256 columns in parts of at most 20: 4 parts,
    # cus / 4 groups of tiles
    assert ffn.workspace_bytes(16, 5120, 17408) == (r256(16 * 17408 * 2) + 4 * 16 * 5120 * 4
                                                    + r256(8 * 4 * (cus // 4)))
    # two token groups: the dual projection's reduction in 2 parts (K = 5120),
    # the down projection's in 4
    assert ffn.workspace_bytes(17, 5120, 17408) == (r256(17 * 17408 * 2) + 4 * 17 * 5120 * 4
                                                    + 2 * 2 * 17 * 17408 * 4
                                                    + r256(8 * max(2 * (cus // 2), 4 * (cus // 4))))
    # three token groups: the dual projection's reduction in 3 parts
    # (K = 5120), the down projection's in 6
    assert ffn.workspace_bytes(40, 5120, 17408) == (r256(40 * 17408 * 2) + 6 * 40 * 5120 * 4
                                                    + 2 * 3 * 40 * 17408 * 4
                                                    + r256(8 * max(3 * (cus // 3), 6 * (cus // 6))))
    # M = 41, or K or N not a multiple of 256: the 128-row arm with its
    # partial slots
    assert ffn.workspace_bytes(41, 5120, 17408) > 32 << 20
    assert ffn.workspace_bytes(16, 640, 1024) > 32 << 20


def test_smallbatch_rows_independent_of_batch():
    """Inside the arm a token row's result does not depend on the other rows
    of a batch with the same token-group count: its position in the token
    tile and M do not change the order of any sum."""
    case = fi.make_small(16, 2048, 6144, act=fi.ACT_GELU_TANH, seed=59)
    L = loaded(case.name, lambda: case)
    full = L.forward()
    for lo, hi in ((0, 9), (7, 16), (2, 13), (3, 15)):
        part = L.forward(L.x[lo:hi].contiguous())
        assert torch.equal(part, full[lo:hi]), (lo, hi)
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    g2, u2 = ffn.dual_gemv(L.x[4:14].contiguous(), L.gate, L.up)
    assert torch.equal(g2, g[4:14]) and torch.equal(u2, u[4:14])


def test_smallbatch_determinism():
    case = fi.make_small(14, 2048, 8192, seed=60)
    L = loaded(case.name, lambda: case)
    first = L.forward().clone()
    for _ in range(5):
        assert torch.equal(L.forward(), first)


def test_smallbatch_two_groups_rows_independent():
    """The same for two token groups (17 to 32 rows), with the dual
    projection split in parts (K = 5120)."""
    case = fi.make_small(32, 5120, 2048, act=fi.ACT_SILU, seed=68)
    L = loaded(case.name, lambda: case)
    full = L.forward()
    for lo, hi in ((0, 17), (15, 32), (3, 29), (8, 32)):
        part = L.forward(L.x[lo:hi].contiguous())
        assert torch.equal(part, full[lo:hi]), (lo, hi)


def test_smallbatch_three_groups_rows_independent():
    """The same for three token groups (33 to 40 rows), with both
    reductions split in parts (K = 5120: 3 parts; N = 8192: 3 parts)."""
    case = fi.make_small(40, 5120, 8192, act=fi.ACT_GELU_TANH, seed=88)
    L = loaded(case.name, lambda: case)
    full = L.forward()
    for lo, hi in ((0, 33), (7, 40), (3, 38), (1, 35)):
        part = L.forward(L.x[lo:hi].contiguous())
        assert torch.equal(part, full[lo:hi]), (lo, hi)


@pytest.mark.parametrize("M", [9, 16, 17, 32, 33, 40, 48, 64])
def test_config_smallbatch(M):
    """The prefill shapes (hidden 5120, intermediate 17408, SiLU) at 9 to 64
    token rows (above 40 the 128-row arm, with one or two token tiles), the
    launch configuration the bench times: the forward and the dual entry
    against the oracle on every token row."""
    case = fi.make_config(4, M=M)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    torch.cuda.synchronize()
    assert_ffn_close(out, oracle.ffn(case), case.name)
    g_ref, u_ref = oracle.dual(case)
    assert_dual_close(g, g_ref, "gate")
    assert_dual_close(u, u_ref, "up")
