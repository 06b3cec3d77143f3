"""GPU parity of the W4A4 prefill arm against the W4A4 oracle (needs an MI355X).

The integer steps are compared bit for bit: the NVFP4 -> MXFP4 weight
requantisation and the per-call MXFP4 quantisation of the activations (read
back from the workspace, where the entry points document it). The dual GEMM's
fp32 outputs are held to 1e-4 * rms(ref) + 1e-6 * |ref| (products of MXFP4
values are exact in fp32; only the accumulation order differs), the hybrid
FFN to the FFN output bound. Against the lossless W4A16 oracle the arm is only
expected to correlate (cosine), as the pages describe it as lossy.
"""
import numpy as np
import pytest
import torch

import ffn_inputs as fi
import oracle
import w4a16_nvfp4_dense_amd as ffn

pytestmark = pytest.mark.gpu


def _r256(b):
    return (b + 255) // 256 * 256


class Loaded:
    def __init__(self, case):
        self.case = case
        self.gate = ffn.DeviceWeight.from_host(case.gate)
        self.up = ffn.DeviceWeight.from_host(case.up)
        self.down = ffn.DeviceWeight.from_host(case.down)
        self.gmx = ffn.w4a4_prepare_weight(self.gate)
        self.umx = ffn.w4a4_prepare_weight(self.up)
        self.x = ffn.bf16_from_bits(case.x_bits)
        # the oracle's requantised weights (checked equal to the GPU's below)
        self.ogmx = oracle.mx_requant(case.gate)
        self.oumx = oracle.mx_requant(case.up)


def assert_dual_close(got, ref, what):
    got = got.double().cpu().numpy()
    rms = np.sqrt(np.mean(ref ** 2))
    bound = 1e-4 * rms + 1e-6 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"{what}: max err/rms {np.max(err) / rms:.3e}"


def assert_ffn_close(out_gpu, out_ref, what):
    got = ffn.bf16_to_f64(out_gpu)
    bound = oracle.parity_bound(out_ref)
    err = np.abs(got - out_ref)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside bound, max err/rms " \
                          f"{np.max(err) / np.sqrt(np.mean(out_ref ** 2)):.3e}"


def assert_requant_exact(L):
    np.testing.assert_array_equal(L.gmx.codes.cpu().numpy(), L.ogmx.codes)
    np.testing.assert_array_equal(L.gmx.scales.cpu().numpy(), L.ogmx.e8m0)
    np.testing.assert_array_equal(L.umx.codes.cpu().numpy(), L.oumx.codes)
    np.testing.assert_array_equal(L.umx.scales.cpu().numpy(), L.oumx.e8m0)


SHAPES = [
    # (M, K, N, act, seed)
    (1, 256, 64, fi.ACT_SILU, 1),
    (17, 512, 128, fi.ACT_GELU_TANH, 2),    # tokens not a multiple of 32
    (45, 1024, 320, fi.ACT_SILU, 3),
    (128, 2048, 1024, fi.ACT_SILU, 4),
    (200, 768, 448, fi.ACT_GELU_TANH, 5),   # two token groups, two down blocks
    # Wider N: rows per workgroup R = ceil(N / 256 compute units) on MI355X,
    # in NF fragments of 32 B rows (gate and up interleaved); the last
    # workgroup holds fewer rows when R does not divide N.
    (40, 512, 5184, fi.ACT_SILU, 6),        # R = 21 (NF 2), last workgroup 18 rows
    (130, 256, 9024, fi.ACT_GELU_TANH, 7),  # R = 36 (NF 3), last 24 rows, two token groups
    (5, 256, 15424, fi.ACT_SILU, 8),        # R = 61 (NF 4), last 52 rows
    (7, 256, 17984, fi.ACT_GELU_TANH, 9),   # R = 71 (NF 5), last 21 rows
    (8, 256, 21504, fi.ACT_SILU, 10),       # R = 84 (NF 6, 3 ring stages), 256 workgroups
]


@pytest.mark.parametrize("M,K,N,act,seed", SHAPES, ids=[f"m{m}_k{k}_n{n}_a{a}" for m, k, n, a, _ in SHAPES])
def test_w4a4_parity(M, K, N, act, seed):
    print(f"\nw4a4 case M={M} K={K} N={N} act={act}", flush=True)
    case = fi.make_small(M, K, N, act=act, seed=seed)
    case.x_bits[0, :64] = 0  # a block of zeros (shared exponent 0)
    L = Loaded(case)
    assert_requant_exact(L)
    ws = torch.zeros(ffn.w4a4_workspace_bytes(M, K, N), dtype=torch.uint8, device="cuda")
    g, u = ffn.w4a4_dual_gemm(L.x, L.gmx, L.umx, workspace=ws)
    torch.cuda.synchronize()
    # the activations' MXFP4 form, as the workspace documents it
    xc, xe = oracle.mx_quantize_bf16(case.x_bits)
    wsn = ws.cpu().numpy()
    np.testing.assert_array_equal(wsn[:M * K // 2].reshape(M, K // 2), xc)
    off = _r256(M * K // 2)
    np.testing.assert_array_equal(wsn[off:off + M * K // 32].reshape(M, K // 32), xe)
    gr, ur = oracle.w4a4_dual(case, L.ogmx, L.oumx)
    assert_dual_close(g, gr, "gate")
    assert_dual_close(u, ur, "up")
    out = ffn.w4a4_forward(L.x, L.gmx, L.umx, L.down, act)
    assert_ffn_close(out, oracle.w4a4_ffn(case, L.ogmx, L.oumx), case.name)
    # repeatable
    assert torch.equal(ffn.w4a4_forward(L.x, L.gmx, L.umx, L.down, act), out)


def test_w4a4_format_coverage():
    """Every E2M1 code and every finite E4M3 scale in the NVFP4 weights: the
    requantisation bit for bit, the dual at the fp32 bound."""
    case = fi.make_format_coverage(M=40)
    L = Loaded(case)
    assert_requant_exact(L)
    g, u = ffn.w4a4_dual_gemm(L.x, L.gmx, L.umx)
    gr, ur = oracle.w4a4_dual(case, L.ogmx, L.oumx)
    assert_dual_close(g, gr, "gate")
    assert_dual_close(u, ur, "up")


def test_w4a4_prefill_config():
    """The prefill shape (M = 128, K = 5120, N = 17408): requantisation bit
    for bit on both weights, and the dual GEMM and the hybrid forward on every
    token row against the oracle. Against the lossless W4A16 oracle, the
    rows correlate (cosine > 0.95)."""
    case = fi.make_config(4, M=128)
    L = Loaded(case)
    assert_requant_exact(L)
    g, u = ffn.w4a4_dual_gemm(L.x, L.gmx, L.umx)
    out = ffn.w4a4_forward(L.x, L.gmx, L.umx, L.down, case.act)
    torch.cuda.synchronize()
    gr, ur = oracle.w4a4_dual(case, L.ogmx, L.oumx)
    assert_dual_close(g, gr, "gate")
    assert_dual_close(u, ur, "up")
    ref = oracle.w4a4_ffn(case, L.ogmx, L.oumx)
    assert_ffn_close(out, ref, "w4a4 forward")
    lossless = oracle.ffn(case)
    got = ffn.bf16_to_f64(out)
    cos = float(np.sum(got * lossless) / np.linalg.norm(got) / np.linalg.norm(lossless))
    print(f"\nw4a4 vs w4a16 cosine over all rows: {cos:.5f}", flush=True)
    assert cos > 0.95


# ------------------------------------------------------------ all three projections on 4 bits


def _fp4_offsets(M, K, N):
    """Offsets of h [M, N] bf16 and of mx(h) (codes, exponents) in the
    workspace of ffn_w4a4_down_gemm / ffn_w4a4_forward_fp4 (include/ffn_w4a4.h
    orders it mx(x), h, mx(h), partial sums, ready words)."""
    h = _r256(M * K // 2) + _r256(M * K // 32)
    hc = h + _r256(M * N * 2)
    he = hc + _r256(M * N // 2)
    return h, hc, he


def assert_down_close(out_gpu, ref, what):
    """A 4-bit down projection: exact products summed in fp32, scaled and
    rounded once to bf16: within one bf16 ulp of the exact value plus
    1e-4 * rms for the fp32 sums."""
    got = ffn.bf16_to_f64(out_gpu)
    rms = np.sqrt(np.mean(ref ** 2))
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * rms
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"{what}: {(err > bound).sum()} outside, max err/rms {np.max(err) / rms:.3e}"


DOWN_SHAPES = [
    # (M, N (reduction), K (output rows), seed); the reduction is split in P
    # parts with P = min(8, 256 // ceil(K / 64), N / 256) on 256 compute units
    (1, 256, 256, 21),      # P = 1: no split
    (17, 1024, 512, 22),    # P = 4
    (128, 2048, 5120, 23),  # P = 3 (80 row blocks of 64)
    (100, 4352, 2560, 24),  # P = 6: the finisher reads 5 parts in 3 batches
    (200, 768, 1024, 25),   # P = 3, two blocks of 128 tokens
    (33, 2048, 1024, 26),   # P = 8
]


@pytest.mark.parametrize("M,N,K,seed", DOWN_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k, _ in DOWN_SHAPES])
def test_w4a4_down_parity(M, N, K, seed):
    """The down projection on 4 bits: mx(h) bit for bit from the same bf16 h,
    the output within one bf16 ulp (+1e-4 rms) of the oracle."""
    print(f"\nw4a4 down case M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(seed)
    h_bits = fi.f32_to_bf16_bits((rng.normal(size=(M, N)) * np.exp(rng.uniform(-3, 3, size=(M, 1)))).astype(np.float32))
    h_bits[0, :32] = 0  # a block of zeros
    w = fi.make_small(1, N, K, seed=seed).gate  # an NVFP4 weight [K, N]
    dmx = ffn.w4a4_prepare_weight(ffn.DeviceWeight.from_host(w))
    odmx = oracle.mx_requant(w)
    np.testing.assert_array_equal(dmx.codes.cpu().numpy(), odmx.codes)
    np.testing.assert_array_equal(dmx.scales.cpu().numpy(), odmx.e8m0)
    h = ffn.bf16_from_bits(h_bits)
    ws = torch.zeros(ffn.w4a4_fp4_workspace_bytes(M, K, N), dtype=torch.uint8, device="cuda")
    out = ffn.w4a4_down_gemm(h, dmx, workspace=ws)
    torch.cuda.synchronize()
    _, hc, he = _fp4_offsets(M, K, N)
    qc, qe = oracle.mx_quantize_bf16(h_bits)
    wsn = ws.cpu().numpy()
    np.testing.assert_array_equal(wsn[hc:hc + M * N // 2].reshape(M, N // 2), qc)
    np.testing.assert_array_equal(wsn[he:he + M * N // 32].reshape(M, N // 32), qe)
    assert_down_close(out, oracle.w4a4_down(h_bits, odmx), "w4a4 down")
    assert torch.equal(ffn.w4a4_down_gemm(h, dmx, workspace=ws), out)  # repeatable, workspace reused


def _check_fp4_forward(case, L, out, ws):
    """The GPU's own h (read back from the workspace): its MXFP4 form bit for
    bit and the output within one bf16 ulp of the oracle's down projection of
    that h; h itself within the FFN bound of the oracle's act(gate) * up; and
    the whole forward within the FFN bound of the oracle's all-4-bit FFN,
    which quantises its own h (rounded once from double): an h element whose
    GPU and oracle values straddle a rounding boundary takes a neighbouring
    code there, which the bound covers."""
    M, K, N = case.M, case.K, case.N
    wsn = ws.cpu().numpy()
    ho, hc, he = _fp4_offsets(M, K, N)
    h_bits = wsn[ho:ho + M * N * 2].view(np.uint16).reshape(M, N).copy()
    qc, qe = oracle.mx_quantize_bf16(h_bits)
    np.testing.assert_array_equal(wsn[hc:hc + M * N // 2].reshape(M, N // 2), qc)
    np.testing.assert_array_equal(wsn[he:he + M * N // 32].reshape(M, N // 32), qe)
    odmx = oracle.mx_requant(case.down)
    assert_down_close(out, oracle.w4a4_down(h_bits, odmx), "down of the GPU's h")
    gr, ur = oracle.w4a4_dual(case, L.ogmx, L.oumx)
    h_ref = oracle.gated_act(case.act, gr, ur)
    h_err = np.abs(fi.bf16_bits_to_f32(h_bits).astype(np.float64) - h_ref)
    assert np.all(h_err <= oracle.parity_bound(h_ref)), "h"
    assert_ffn_close(out, oracle.w4a4_ffn_fp4(case, L.ogmx, L.oumx, odmx), case.name)


FP4_SHAPES = [
    (1, 256, 256, fi.ACT_SILU, 31),
    (17, 512, 512, fi.ACT_GELU_TANH, 32),
    (45, 1024, 768, fi.ACT_SILU, 33),
    (128, 2048, 1024, fi.ACT_SILU, 34),
    (200, 768, 512, fi.ACT_GELU_TANH, 35),   # two token groups and two down blocks
    (40, 512, 5376, fi.ACT_SILU, 36),        # wider intermediate (dual R = 21)
]


@pytest.mark.parametrize("M,K,N,act,seed", FP4_SHAPES, ids=[f"m{m}_k{k}_n{n}_a{a}" for m, k, n, a, _ in FP4_SHAPES])
def test_w4a4_forward_fp4(M, K, N, act, seed):
    print(f"\nw4a4 fp4 forward case M={M} K={K} N={N} act={act}", flush=True)
    case = fi.make_small(M, K, N, act=act, seed=seed)
    L = Loaded(case)
    dmx = ffn.w4a4_prepare_weight(L.down)
    ws = torch.zeros(ffn.w4a4_fp4_workspace_bytes(M, K, N), dtype=torch.uint8, device="cuda")
    out = ffn.w4a4_forward_fp4(L.x, L.gmx, L.umx, dmx, act, workspace=ws)
    torch.cuda.synchronize()
    _check_fp4_forward(case, L, out, ws)
    assert torch.equal(ffn.w4a4_forward_fp4(L.x, L.gmx, L.umx, dmx, act, workspace=ws), out)


def test_w4a4_fp4_prefill_config():
    """The prefill shape (M = 128, K = 5120, N = 17408) with all three
    projections on 4 bits, every token row; against the lossless W4A16 oracle
    the rows correlate (cosine > 0.95)."""
    case = fi.make_config(4, M=128)
    L = Loaded(case)
    dmx = ffn.w4a4_prepare_weight(L.down)
    ws = torch.zeros(ffn.w4a4_fp4_workspace_bytes(case.M, case.K, case.N), dtype=torch.uint8, device="cuda")
    out = ffn.w4a4_forward_fp4(L.x, L.gmx, L.umx, dmx, case.act, workspace=ws)
    torch.cuda.synchronize()
    _check_fp4_forward(case, L, out, ws)
    lossless = oracle.ffn(case)
    got = ffn.bf16_to_f64(out)
    cos = float(np.sum(got * lossless) / np.linalg.norm(got) / np.linalg.norm(lossless))
    print(f"\nall-4-bit vs w4a16 cosine over all rows: {cos:.5f}", flush=True)
    assert cos > 0.95
