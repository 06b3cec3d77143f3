"""GPU parity of the HIP library against the CPU oracle (needs an MI355X).

Every comparison is element by element on the same seeded inputs. The FFN
output bound is |out - out_ref| <= 1e-2 * rms(out_ref) + 1 bf16 ulp(out_ref)
(out_ref in double); the dual GEMV's fp32 outputs must be within
1e-4 * rms(ref) + 1e-6 * |ref| of the double reference (only fp32
accumulation-order error is possible there, since every product of an E2M1
value, an E4M3 scale and a bf16 input is exact in fp32).
"""
import numpy as np
import pytest
import torch

import ffn_inputs as fi
import oracle
import w4a16_nvfp4_dense_amd as ffn

pytestmark = pytest.mark.gpu

DEV = "cuda"


class Loaded:
    """A case with its weights on the device."""

    def __init__(self, case):
        self.case = case
        self.gate = ffn.DeviceWeight.from_host(case.gate)
        self.up = ffn.DeviceWeight.from_host(case.up)
        self.down = ffn.DeviceWeight.from_host(case.down)
        self.x = ffn.bf16_from_bits(case.x_bits)

    def forward(self, x=None):
        return ffn.forward(self.x if x is None else x, self.gate, self.up, self.down, self.case.act)


_cache = {}


def loaded(key, make):
    if key not in _cache:
        _cache.clear()  # keep at most one large case resident
        _cache[key] = Loaded(make())
    return _cache[key]


def assert_ffn_close(out_gpu, out_ref, what, extra=None):
    """`extra` (elementwise) widens the bound, for the format-coverage weights
    only: see oracle.h_rounding_bound."""
    got = ffn.bf16_to_f64(out_gpu) if torch.is_tensor(out_gpu) else out_gpu
    bound = oracle.parity_bound(out_ref)
    if extra is not None:
        bound = bound + extra
    err = np.abs(got - out_ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside bound; first at {tuple(i)}: "
                             f"gpu {got[tuple(i)]!r} ref {out_ref[tuple(i)]!r} bound {bound[tuple(i)]!r}; "
                             f"max err/rms {np.max(err) / np.sqrt(np.mean(out_ref ** 2)):.3e}")


def assert_banded_close(out_gpu, out_ref, what, band=32):
    """The FFN output bound applied to each band of `band` consecutive output
    columns as if it were the whole output (rms over the band), so columns
    of small magnitude are checked at their own scale rather than at the
    scale of the largest ones."""
    got = ffn.bf16_to_f64(out_gpu) if torch.is_tensor(out_gpu) else out_gpu
    for b0 in range(0, out_ref.shape[1], band):
        sl = slice(b0, b0 + band)
        assert_ffn_close(got[:, sl], out_ref[:, sl], f"{what} columns {b0}..{b0 + band - 1}")


def assert_dual_close(got, ref, what):
    got = got.double().cpu().numpy()
    rms = np.sqrt(np.mean(ref ** 2))
    bound = 1e-4 * rms + 1e-6 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"{what}: max err/rms {np.max(err) / rms:.3e}"


# Small and mid-size shapes: several tiles, ragged chunk counts, every lane
# width (chunk counts divisible by 64, 32, 16, 8 and by none of them), LDS
# staging in one piece and in several pieces.
SMALL = [
    # (M, K, N, act, seed)
    (1, 256, 512, fi.ACT_SILU, 1),
    (1, 32, 32, fi.ACT_SILU, 2),
    (1, 96, 160, fi.ACT_GELU_TANH, 3),      # chunk counts 3 and 5: partly masked lanes
    (2, 160, 96, fi.ACT_SILU, 4),
    (3, 2048, 1024, fi.ACT_SILU, 5),        # 64 chunks per row: a full wave per row
    (1, 1024, 2048, fi.ACT_GELU_TANH, 6),
    (4, 512, 4096, fi.ACT_SILU, 7),
    (5, 480, 800, fi.ACT_GELU_TANH, 8),     # 15 and 25 chunks
    (6, 1536, 544, fi.ACT_SILU, 9),
    (7, 256, 3072, fi.ACT_SILU, 10),
    (8, 5120, 2048, fi.ACT_SILU, 11),       # several LDS pieces for M = 8
    (8, 1056, 8224, fi.ACT_GELU_TANH, 12),  # 33 and 257 chunks: ragged, several pieces
    # many-wave kernel (33 or more chunks per row, activations in LDS)
    (1, 1056, 2080, fi.ACT_SILU, 13),       # 33 / 65 chunks: partly masked last lane chunk
    (2, 2080, 1056, fi.ACT_GELU_TANH, 14),
    (1, 4096, 96, fi.ACT_SILU, 15),         # fewer rows than compute units
    (2, 2048, 20000, fi.ACT_SILU, 16),      # 79 rows per CU; 625-chunk down rows from LDS
    (1, 12288, 4096, fi.ACT_GELU_TANH, 17), # 6 chunks per lane
    (5, 1056, 12288, fi.ACT_GELU_TANH, 18), # down: 6 chunks per lane, 5 rows in one launch
    (7, 4096, 18432, fi.ACT_SILU, 19),      # down: 9 chunks per lane, 7 rows staged in two pieces
    (6, 12288, 1056, fi.ACT_SILU, 20),      # dual: 6 chunks per lane, 6 rows in one launch
    (3, 24576, 1056, fi.ACT_GELU_TANH, 21), # dual: 12 chunks per lane, 8-wave workgroups
    # activations staged in pieces of steps (M x steps x 4 KB over the LDS budget)
    (4, 1056, 21504, fi.ACT_GELU_TANH, 27), # down: 11 steps in pieces of 6 + 5
    (8, 2080, 12352, fi.ACT_SILU, 28),      # down: 386 chunks, 7 steps in pieces of 4 + 3
]


@pytest.mark.parametrize("M,K,N,act,seed", SMALL, ids=[f"m{m}_k{k}_n{n}_a{a}" for m, k, n, a, _ in SMALL])
def test_forward_small(M, K, N, act, seed):
    case = fi.make_small(M, K, N, act=act, seed=seed)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    torch.cuda.synchronize()
    assert_ffn_close(out, oracle.ffn(case), case.name)


@pytest.mark.parametrize("M,K,N,act,seed", SMALL[:8], ids=[f"m{m}_k{k}_n{n}" for m, k, n, a, _ in SMALL[:8]])
def test_dual_and_down_entries(M, K, N, act, seed):
    case = fi.make_small(M, K, N, act=act, seed=seed)
    L = loaded(case.name, lambda: case)
    g_ref, u_ref = oracle.dual(case)
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    torch.cuda.synchronize()
    assert_dual_close(g, g_ref, "gate")
    assert_dual_close(u, u_ref, "up")
    # The down entry on the oracle's gate/up rounded to fp32, against the
    # oracle's down projection of act(gate) * up from those same inputs.
    g32 = g_ref.astype(np.float32)
    u32 = u_ref.astype(np.float32)
    out = ffn.down_gemv(torch.from_numpy(g32).to(DEV), torch.from_numpy(u32).to(DEV), L.down, act)
    torch.cuda.synchronize()
    h = oracle.gated_act(act, g32.astype(np.float64), u32.astype(np.float64))
    assert_ffn_close(out, oracle.down(h, case.down), "down entry")


@pytest.mark.parametrize("act", [fi.ACT_SILU, fi.ACT_GELU_TANH])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_format_coverage(act, M):
    """All 16 E2M1 codes, all 254 finite E4M3 scales (negative, subnormal,
    448), scale2 not a power of two. The decoding is checked through the dual
    entry at the fp32 bound; the FFN output bound adds the propagated bound of
    the one bf16 rounding of h, which these weights (E4M3 scales spanning
    2^-9 .. 448 in W_d) can blow up through cancellation."""
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
@pytest.mark.parametrize("M", [1, 3, 8])
def test_format_coverage_onesign(act, M):
    """All 16 E2M1 codes and all 254 finite E4M3 scales in W_d, with every
    product of an output's sum of one sign (so nothing cancels): the forward
    and the down entry at the plain output bound, over the whole output and
    over each band of like-magnitude outputs (the subnormal-scale rows
    included), with no allowance for the rounding of h."""
    case = fi.make_format_coverage_onesign(act=act, M=M)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    torch.cuda.synchronize()
    g_ref, u_ref = oracle.dual(case)
    assert_dual_close(g, g_ref, "gate")
    assert_dual_close(u, u_ref, "up")
    ref = oracle.ffn(case)
    assert_ffn_close(out, ref, case.name)
    assert_banded_close(out, ref, case.name)
    g32, u32 = g_ref.astype(np.float32), u_ref.astype(np.float32)
    d = ffn.down_gemv(torch.from_numpy(g32).to(DEV), torch.from_numpy(u32).to(DEV), L.down, act)
    torch.cuda.synchronize()
    d_ref = oracle.down(oracle.gated_act(act, g32.astype(np.float64), u32.astype(np.float64)), case.down)
    assert_ffn_close(d, d_ref, "down entry")
    assert_banded_close(d, d_ref, "down entry")


def test_determinism_and_entry_composition():
    case = fi.make_small(3, 1024, 2048, seed=21)
    L = loaded(case.name, lambda: case)
    first = L.forward().clone()
    for _ in range(10):
        assert torch.equal(L.forward(), first)
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    out2 = ffn.down_gemv(g, u, L.down, case.act)
    torch.cuda.synchronize()
    assert torch.equal(out2, first), "forward must equal dual + down bit for bit"


def test_batch_rows_match_single_row():
    """Row m of an M-row call is bit-identical to the M = 1 call on x[m]."""
    case = fi.make_small(8, 1536, 3072, act=fi.ACT_GELU_TANH, seed=22)
    L = loaded(case.name, lambda: case)
    full = L.forward()
    for M in (2, 3, 5):
        part = L.forward(L.x[:M].contiguous())
        assert torch.equal(part, full[:M])
    for m in range(8):
        one = L.forward(L.x[m:m + 1].contiguous())
        assert torch.equal(one[0], full[m]), m


def test_degenerate_weights():
    case = fi.make_small(2, 256, 512, seed=23)
    L = loaded(case.name, lambda: case)
    zero = ffn.DeviceWeight(torch.zeros_like(L.gate.codes), L.gate.scales, 1.0)
    out = ffn.forward(L.x, zero, L.up, L.down)
    assert torch.count_nonzero(out) == 0  # SiLU(0) * up = 0
    s0 = ffn.DeviceWeight(L.down.codes, L.down.scales, 0.0)
    assert torch.count_nonzero(ffn.forward(L.x, L.gate, L.up, s0)) == 0
    # a negative scale2 on the down projection flips the sign exactly
    neg = ffn.DeviceWeight(L.down.codes, L.down.scales, -case.down.scale2)
    assert torch.equal(ffn.forward(L.x, L.gate, L.up, neg), -L.forward())
    # zero activations
    z = torch.zeros_like(L.x)
    assert torch.count_nonzero(ffn.forward(z, L.gate, L.up, L.down)) == 0


def _scales_at_offset(w, off):
    """The same scales in a buffer that starts `off` bytes past an aligned
    allocation (the ABI only asks for 2-byte alignment for M <= 8)."""
    buf = torch.zeros(w.scales.numel() + 16, dtype=torch.uint8, device=DEV)
    view = buf[off:off + w.scales.numel()].view(w.scales.shape)
    view.copy_(w.scales)
    return ffn.DeviceWeight(w.codes, view, w.scale2)


@pytest.mark.parametrize("M", [1, 2, 3])
def test_scales_two_byte_aligned(M):
    case = fi.make_small(M, 1056, 2080, act=fi.ACT_GELU_TANH, seed=26)
    L = loaded(case.name, lambda: case)
    ref = L.forward()
    g, u, d = (_scales_at_offset(w, 2) for w in (L.gate, L.up, L.down))
    assert g.scales.data_ptr() % 4 == 2
    out = ffn.forward(L.x, g, u, d, case.act)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert_ffn_close(out, oracle.ffn(case), case.name)


def test_nan_scale_propagates():
    """A NaN scale byte (0x7F) in W_g makes that gate NaN, hence every output
    NaN, in the oracle and on the GPU."""
    case = fi.make_small(1, 256, 512, seed=24)
    case.gate.scales[5, 3] = 0x7F
    L = Loaded(case)
    out = ffn.bf16_to_f64(L.forward())
    ref = oracle.ffn(case)
    assert np.all(np.isnan(ref))
    assert np.all(np.isnan(out))


def test_empty_batch():
    case = fi.make_small(1, 256, 512, seed=25)
    L = loaded(case.name, lambda: case)
    x0 = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    out = L.forward(x0)
    assert out.shape == (0, 256)


# ------------------------------------------------------------ full sizes


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_config_decode(idx):
    case = fi.make_config(idx)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    torch.cuda.synchronize()
    g_ref, u_ref = oracle.dual(case)
    assert_dual_close(g, g_ref, "gate")
    assert_dual_close(u, u_ref, "up")
    assert_ffn_close(out, oracle.ffn(case), case.name)


@pytest.mark.parametrize("M", [2, 3, 8])
def test_config_verify(M):
    case = fi.make_config(3, M=M)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    torch.cuda.synchronize()
    assert_ffn_close(out, oracle.ffn(case), case.name)
    for m in range(M):
        assert torch.equal(L.forward(L.x[m:m + 1].contiguous())[0], out[m])


# (config, M): the down entry at the decode and verify shapes, where a lane
# takes 9 (N = 17408) or 11 (N = 21504) chunks and an 8-row batch stages its
# activations in three pieces.
DOWN_FULL = [(1, 1), (2, 1), (3, 2), (3, 3), (3, 8)]


@pytest.mark.parametrize("idx,M", DOWN_FULL, ids=[f"config{i}_m{m}" for i, m in DOWN_FULL])
def test_config_down_entry(idx, M):
    """The activation-fused down entry at full size, every element: from the
    oracle's gate and up rounded to fp32, against the oracle's down
    projection of act(gate) * up from those same inputs. Then, on the GPU's
    own gate and up, the down entry equals the forward bit for bit."""
    case = fi.make_config(idx, M=M) if idx == 3 else fi.make_config(idx)
    L = loaded(case.name, lambda: case)
    g_ref, u_ref = oracle.dual(case)
    g32, u32 = g_ref.astype(np.float32), u_ref.astype(np.float32)
    out = ffn.down_gemv(torch.from_numpy(g32).to(DEV), torch.from_numpy(u32).to(DEV), L.down, case.act)
    torch.cuda.synchronize()
    h = oracle.gated_act(case.act, g32.astype(np.float64), u32.astype(np.float64))
    assert_ffn_close(out, oracle.down(h, case.down), f"{case.name} down entry")
    g, u = ffn.dual_gemv(L.x, L.gate, L.up)
    assert torch.equal(ffn.down_gemv(g, u, L.down, case.act), L.forward()), "forward != dual + down"


@pytest.mark.parametrize("M", [5, 6, 7])
def test_verify_batch_one_launch(M):
    """Verify batches of 5 to 7 rows at the decode shape (one launch per
    projection): every element against the oracle, every row bit-identical
    to the M = 1 call on it."""
    case = fi.make_config(3, M=M)
    L = loaded(case.name, lambda: case)
    out = L.forward()
    torch.cuda.synchronize()
    assert_ffn_close(out, oracle.ffn(case), case.name)
    for m in range(M):
        assert torch.equal(L.forward(L.x[m:m + 1].contiguous())[0], out[m]), m
