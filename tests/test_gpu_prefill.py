"""GPU parity of the matrix-core arm (M > 8 token rows) against the CPU oracle.

Same bound as the decode tests: |out - out_ref| <= 1e-2 * rms(out_ref) + 1
bf16 ulp(out_ref), out_ref in double; the dual entry's fp32 outputs within
1e-4 * rms(ref) + 1e-6 * |ref| (every E2M1 x E4M3 x bf16 product is exact in
fp32 and in the matrix cores' bf16 inputs, so only the fp32 accumulation
order differs from the exact sum).
"""
import numpy as np
import pytest
import torch

import ffn_inputs as fi
import oracle
import w4a16_nvfp4_dense_amd as ffn
from test_gpu_parity import Loaded, assert_banded_close, assert_dual_close, assert_ffn_close, loaded

pytestmark = pytest.mark.gpu

DEV = "cuda"

# (M, K, N, act, seed): one to four 32-row token tiles, two and more blocks of
# 128 rows, ragged weight tiles (N not a multiple of 128, K not a multiple of
# 256), every stream-K shape from one-unit pieces to whole tiles.
PREFILL = [
    (9, 256, 512, fi.ACT_SILU, 31),         # 16 one-unit pieces: 4 pieces per dual tile
    (17, 320, 448, fi.ACT_GELU_TANH, 32),   # ragged tiles in both GEMMs
    (32, 1024, 2048, fi.ACT_SILU, 33),
    (33, 2048, 1024, fi.ACT_GELU_TANH, 34),
    (64, 512, 4096, fi.ACT_SILU, 35),
    (96, 1536, 2560, fi.ACT_SILU, 36),
    (128, 2048, 3072, fi.ACT_GELU_TANH, 37),
    (130, 512, 1024, fi.ACT_SILU, 38),      # blocks of 128 + 2 rows
    (200, 256, 384, fi.ACT_GELU_TANH, 39),  # blocks of 128 + 72 rows
]


@pytest.mark.parametrize("M,K,N,act,seed", PREFILL, ids=[f"m{m}_k{k}_n{n}_a{a}" for m, k, n, a, _ in PREFILL])
def test_prefill_forward(M, K, N, act, seed):
    case = fi.make_small(M, K, N, act=act, seed=seed)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    torch.cuda.synchronize()
    assert_ffn_close(out, oracle.ffn(case), case.name)


@pytest.mark.parametrize("M,K,N,act,seed", PREFILL[:6], ids=[f"m{m}_k{k}_n{n}" for m, k, n, a, _ in PREFILL[:6]])
def test_prefill_dual_and_down_entries(M, K, N, act, seed):
    case = fi.make_small(M, K, N, act=act, seed=seed)
    L = loaded(case.name, lambda: case)
    g_ref, u_ref = oracle.dual(case)
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    torch.cuda.synchronize()
    assert_dual_close(g, g_ref, "gate")
    assert_dual_close(u, u_ref, "up")
    g32 = g_ref.astype(np.float32)
    u32 = u_ref.astype(np.float32)
    out = ffn.down_gemv(torch.from_numpy(g32).to(DEV), torch.from_numpy(u32).to(DEV), L.down, act)
    torch.cuda.synchronize()
    h = oracle.gated_act(act, g32.astype(np.float64), u32.astype(np.float64))
    assert_ffn_close(out, oracle.down(h, case.down), "down entry")


@pytest.mark.parametrize("act", [fi.ACT_SILU, fi.ACT_GELU_TANH])
@pytest.mark.parametrize("M", [16, 128])
def test_prefill_format_coverage(act, M):
    """As the decode format-coverage test (bound widened by the propagated
    bf16 rounding of h for these extreme-range weights)."""
    case = fi.make_format_coverage(act=act, M=M)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    torch.cuda.synchronize()
    g_ref, u_ref = oracle.dual(case)
    assert_dual_close(g, g_ref, "gate")
    assert_dual_close(u, u_ref, "up")
    assert_ffn_close(out, oracle.ffn(case), case.name, extra=oracle.h_rounding_bound(case))


@pytest.mark.parametrize("act", [fi.ACT_SILU, fi.ACT_GELU_TANH])
@pytest.mark.parametrize("M", [16, 40, 128])
def test_prefill_format_coverage_onesign(act, M):
    """As the decode test of the same name: every code and finite scale in
    W_d, no cancellation, the forward at the plain output bound over the
    whole output and per band of like-magnitude outputs."""
    case = fi.make_format_coverage_onesign(act=act, M=M)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    torch.cuda.synchronize()
    ref = oracle.ffn(case)
    assert_ffn_close(out, ref, case.name)
    assert_banded_close(out, ref, case.name)


def test_prefill_determinism():
    case = fi.make_small(128, 1024, 2048, seed=41)
    L = loaded(case.name, lambda: case)
    first = L.forward().clone()
    for _ in range(5):
        assert torch.equal(L.forward(), first)


def test_prefill_rows_independent_of_batch():
    """Within the 128-row matrix-core arm (M > 64) a token row's result does
    not depend on the batch it is in (its position in a token tile or the tile
    count)."""
    case = fi.make_small(128, 1024, 1536, act=fi.ACT_GELU_TANH, seed=42)
    L = loaded(case.name, lambda: case)
    full = L.forward()
    for lo, hi in ((0, 65), (60, 128), (5, 105), (20, 120)):
        part = L.forward(L.x[lo:hi].contiguous())
        assert torch.equal(part, full[lo:hi]), (lo, hi)


def test_prefill_degenerate_weights():
    case = fi.make_small(40, 256, 512, seed=43)
    L = loaded(case.name, lambda: case)
    zero = ffn.DeviceWeight(torch.zeros_like(L.gate.codes), L.gate.scales, 1.0)
    assert torch.count_nonzero(ffn.forward(L.x, zero, L.up, L.down)) == 0
    neg = ffn.DeviceWeight(L.down.codes, L.down.scales, -case.down.scale2)
    assert torch.equal(ffn.forward(L.x, L.gate, L.up, neg), -L.forward())


def test_prefill_nan_scale_propagates():
    case = fi.make_small(12, 256, 512, seed=44)
    case.down.scales[7, 2] = 0xFF
    L = Loaded(case)
    out = ffn.bf16_to_f64(L.forward())
    ref = oracle.ffn(case)
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    assert np.isnan(ref).any() and not np.isnan(ref).all()


# ------------------------------------------------------------ full size


def test_config_prefill():
    """Prefill config at full size (M = 128, hidden 5120, intermediate 17408):
    the forward against the oracle on every token row, and the dual entry's
    gate and up on every row."""
    case = fi.make_config(4)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    torch.cuda.synchronize()
    assert_ffn_close(out, oracle.ffn(case), case.name)
    g_ref, u_ref = oracle.dual(case)
    assert_dual_close(g, g_ref, "gate")
    assert_dual_close(u, u_ref, "up")
