"""GPU parity of the block-scaled FP8 (W8A16) FFN against the CPU oracle
(needs an MI355X).

Bounds as for NVFP4: the FFN output within 1e-2 * rms(out_ref) + 1 bf16 ulp
of the double reference; the dual GEMV's fp32 outputs within
1e-4 * rms(ref) + 1e-6 * |ref| (every product of an E4M3 value and a bf16
input is exact in fp32; a 16-column sum is multiplied by its fp32 block scale
once, so only fp32 rounding of sums and of that product can differ).
"""
import numpy as np
import pytest
import torch

import ffn_inputs as fi
import oracle
import w4a16_nvfp4_dense_amd as ffn

pytestmark = pytest.mark.gpu


class Loaded:
    def __init__(self, case):
        self.case = case
        self.gate = ffn.Fp8DeviceWeight.from_host(case.gate)
        self.up = ffn.Fp8DeviceWeight.from_host(case.up)
        self.down = ffn.Fp8DeviceWeight.from_host(case.down)
        self.x = ffn.bf16_from_bits(case.x_bits)

    def forward(self, x=None):
        return ffn.fp8_forward(self.x if x is None else x, self.gate, self.up, self.down, self.case.act)

    def dual(self, x=None):
        return ffn.fp8_dual_gemv(self.x if x is None else x, self.gate, self.up)


_cache = {}


def loaded(key, make):
    if key not in _cache:
        _cache.clear()
        _cache[key] = Loaded(make())
    return _cache[key]


def assert_ffn_close(out_gpu, out_ref, what, extra=None):
    got = ffn.bf16_to_f64(out_gpu)
    bound = oracle.parity_bound(out_ref)
    if extra is not None:
        bound = bound + extra
    err = np.abs(got - out_ref)
    bad = ~(err <= bound)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside bound; first at {i}: gpu {got[i]!r} "
                             f"ref {out_ref[i]!r} bound {bound[i]!r}; "
                             f"max err/rms {np.max(err) / np.sqrt(np.mean(out_ref ** 2)):.3e}")


def assert_dual_close(got, ref, what):
    got = got.double().cpu().numpy()
    rms = np.sqrt(np.mean(ref ** 2))
    bound = 1e-4 * rms + 1e-6 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"{what}: max err/rms {np.max(err) / rms:.3e}"


# Shapes: ragged block grids (K, N not multiples of 128), chunk counts that
# leave lanes idle in the last step, 1 to 21 chunks per lane, every batch
# size up to 8 (each in one launch per projection), activations in LDS pieces
# (M = 8 with long down rows), one and two workgroups per compute unit.
SMALL = [
    # (M, K, N, act, seed)
    (1, 256, 512, fi.ACT_SILU, 1),
    (1, 16, 16, fi.ACT_SILU, 2),             # one chunk per row, one block
    (3, 400, 336, fi.ACT_GELU_TANH, 3),      # 25 / 21 chunks, ragged 128-blocks both ways
    (2, 1040, 1200, fi.ACT_SILU, 4),         # 65 / 75 chunks: one live lane in the last step
    (8, 2048, 3072, fi.ACT_SILU, 5),
    (5, 1536, 2576, fi.ACT_GELU_TANH, 6),    # 5 rows
    (6, 3072, 1040, fi.ACT_SILU, 7),         # 6 rows
    (7, 1024, 6160, fi.ACT_GELU_TANH, 8),    # 7 rows
    (4, 4096, 14336, fi.ACT_SILU, 9),        # down: 14 chunks per lane
    (8, 4096, 14336, fi.ACT_GELU_TANH, 10),  # down: activations staged in two pieces
    (8, 2064, 24576, fi.ACT_SILU, 11),       # down: 24 chunks per lane, three pieces
    (1, 24576, 272, fi.ACT_SILU, 12),        # dual: 24 chunks per lane, fewer rows than CUs
]


@pytest.mark.parametrize("M,K,N,act,seed", SMALL, ids=[f"m{m}_k{k}_n{n}_a{a}" for m, k, n, a, _ in SMALL])
def test_fp8_forward_and_entries(M, K, N, act, seed):
    print(f"\nfp8 case M={M} K={K} N={N} act={act} seed={seed}", flush=True)
    case = fi.make_fp8_ffn(f"fp8_m{M}_k{K}_n{N}", M, K, N, act=act, seed=seed)
    L = Loaded(case)
    out = L.forward()
    ref = oracle.fp8_ffn(case)
    assert_ffn_close(out, ref, case.name)
    # dual entry against the oracle's gate/up
    g, u = L.dual()
    gr, ur = oracle.fp8_dual(case)
    assert_dual_close(g, gr, "gate")
    assert_dual_close(u, ur, "up")
    # down entry (activation fused into its load) from the GPU's gate/up is
    # the forward bit for bit (same fp32 gate/up, same one rounding of h)
    d = ffn.fp8_down_gemv(g, u, L.down, act)
    assert torch.equal(d, out)
    # ... and from the oracle's gate/up rounded to fp32 it meets the bound
    g32 = torch.from_numpy(gr.astype(np.float32)).cuda()
    u32 = torch.from_numpy(ur.astype(np.float32)).cuda()
    d2 = ffn.fp8_down_gemv(g32, u32, L.down, act)
    h = oracle.gated_act(act, gr.astype(np.float32).astype(np.float64), ur.astype(np.float32).astype(np.float64))
    assert_ffn_close(d2, oracle.fp8_linear(h, case.down), case.name + " down entry")


@pytest.mark.parametrize("act", [fi.ACT_SILU, fi.ACT_GELU_TANH])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_fp8_format_coverage(act, M):
    """Every finite E4M3FN byte in every weight, ragged block grids: the dual
    entry at the fp32 bound (this checks the decoding of every code), the FFN
    at the output bound widened by the propagated bound of h's one bf16
    rounding (these weights span 2^-9 to 448 within a block)."""
    case = fi.make_fp8_format_coverage(act=act, M=M)
    L = Loaded(case)
    g, u = L.dual()
    gr, ur = oracle.fp8_dual(case)
    assert_dual_close(g, gr, "gate")
    assert_dual_close(u, ur, "up")
    assert_ffn_close(L.forward(), oracle.fp8_ffn(case), case.name, extra=oracle.fp8_h_rounding_bound(case))


def test_fp8_determinism_and_batch_rows():
    """Ten repeats are bit-identical; row m of a batch equals the M = 1 call on
    that row, for batches of 2, 3, 5 and 8."""
    case = fi.make_fp8_ffn("fp8_det", 8, 2048, 6144, seed=21)
    L = Loaded(case)
    first = L.forward()
    for _ in range(9):
        assert torch.equal(L.forward(), first)
    singles = [L.forward(L.x[m:m + 1]) for m in range(8)]
    for Mb in (2, 3, 5, 8):
        out = L.forward(L.x[:Mb].contiguous())
        for m in range(Mb):
            assert torch.equal(out[m:m + 1], singles[m]), (Mb, m)


def test_fp8_nan_code_and_zero_weights():
    """A NaN code (0x7F) reaches exactly the outputs it touches; zero codes
    give zero outputs."""
    case = fi.make_fp8_ffn("fp8_nan", 2, 512, 384, seed=22)
    case.gate.codes[5, 300] = 0x7F
    L = Loaded(case)
    g, u = L.dual()
    g = g.cpu().numpy()
    assert np.all(np.isnan(g[:, 5]))
    assert np.all(np.isfinite(np.delete(g, 5, axis=1)))
    assert np.all(np.isfinite(u.cpu().numpy()))
    zero = fi.make_fp8_ffn("fp8_zero", 3, 512, 384, seed=23)
    for w in (zero.gate, zero.up, zero.down):
        w.codes[:] = 0
    out = Loaded(zero).forward()
    assert torch.count_nonzero(out) == 0


def test_fp8_empty_batch():
    case = fi.make_fp8_ffn("fp8_empty", 1, 256, 512, seed=24)
    L = Loaded(case)
    x0 = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    assert L.forward(x0).shape == (0, 256)


@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_fp8_config_decode_and_verify(M):
    """The decode shape (K = 5120, N = 17408) with FP8 weights at M = 1 and
    the verify batches M = 2, 3, 8, against the oracle on every element."""
    print(f"\nfp8 config M={M}", flush=True)
    L = loaded("fp8_cfg", lambda: fi.make_fp8_config(M=8))
    case = fi.make_fp8_config(M=M)
    x = ffn.bf16_from_bits(case.x_bits)
    out = L.forward(x)
    assert_ffn_close(out, oracle.fp8_ffn(L.case.with_x(case.x_bits)), case.name)


def test_fp8_config_gelu():
    """The GELU-tanh shape (K = 5376, N = 21504: 21 chunks per lane in the
    down GEMV) with FP8 weights, M = 1."""
    case = fi.make_fp8_ffn("fp8_gelu_m1", 1, 5376, 21504, act=fi.ACT_GELU_TANH, sigma=0.5,
                           seed=fi.SEED_BASE + 52)
    L = Loaded(case)
    assert_ffn_close(L.forward(), oracle.fp8_ffn(case), case.name)
