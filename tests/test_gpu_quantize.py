"""GPU parity of the BF16 -> NVFP4 quantiser (ffn_nvfp4_quantize) against the
CPU oracle (needs an MI355X).

The quantiser's outputs are integers decided by fp32 arithmetic that both
sides take in the same order, so codes, scale bytes and scale2 must be
bit-exact. Then a quantise -> FFN round trip: weights quantised on the GPU
drive the forward, against the oracle FFN on the oracle's quantisation of the
same bf16 weights.
"""
import numpy as np
import pytest
import torch

import ffn_inputs as fi
import oracle
import w4a16_nvfp4_dense_amd as ffn

pytestmark = pytest.mark.gpu


def _gpu_quantize(bits):
    w = ffn.bf16_from_bits(bits)
    codes, scales, s2 = ffn.quantize(w)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), float(s2.cpu()[0])


def _assert_same(bits, what):
    rows, cols = bits.shape
    print(f"quantize {what}: {rows} x {cols}", flush=True)
    gc, gs, g2 = _gpu_quantize(bits)
    oc, osc, o2 = oracle.quantize(bits)
    assert np.float32(g2) == np.float32(o2), (what, g2, o2)
    bad_s = np.argwhere(gs != osc)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale bytes differ, first {tuple(bad_s[0])}: " \
                            f"gpu {gs[tuple(bad_s[0])]:#x} oracle {osc[tuple(bad_s[0])]:#x}"
    bad_c = np.argwhere(gc != oc)
    assert bad_c.size == 0, f"{what}: {len(bad_c)} code bytes differ, first {tuple(bad_c[0])}: " \
                            f"gpu {gc[tuple(bad_c[0])]:#x} oracle {oc[tuple(bad_c[0])]:#x}"
    return gc, gs, g2


@pytest.mark.parametrize("rows,cols,seed", [
    (1, 32, 1),        # one row, two blocks
    (37, 96, 2),       # ragged: rows and blocks not multiples of a workgroup
    (128, 512, 3),
    (300, 5120, 4),    # rows of the decode hidden size
    (64, 17408, 5),    # rows of the decode intermediate size
])
def test_quantize_bit_exact(rows, cols, seed):
    _assert_same(fi.make_dense_bf16(rows, cols, seed), f"normal seed {seed}")


def test_quantize_full_gate_shape():
    """The decode gate/up weight shape (17408 x 5120), whole, in the launch
    configuration the benchmark times."""
    _assert_same(fi.make_dense_bf16(17408, 5120, 6), "full 17408 x 5120")


def test_quantize_zero_and_tiny():
    z = np.zeros((16, 64), dtype=np.uint16)
    gc, gs, g2 = _assert_same(z, "zeros")
    assert g2 == 0.0 and not gc.any() and not gs.any()
    # one huge element: every other block's scale underflows E4M3 (subnormal
    # scale bytes and zero blocks), and its own block saturates at 448
    rng = np.random.default_rng(8)
    f = (rng.standard_normal((24, 256)) * 10.0 ** rng.uniform(-5, 1, size=(24, 1))).astype(np.float32)
    f[5, 77] = 3.0e4
    f[11, 16:32] = 0.0                                   # an all-zero block
    f[13, 32:48] = 1e-8                                  # a block far below the rest
    gc, gs, g2 = _assert_same(fi.f32_to_bf16_bits(f), "wide range")
    assert gs[5, 77 // 16] == 0x7E and gs[11, 1] == 0
    assert ((gs > 0) & (gs < 0x08)).any(), "no subnormal scale byte exercised"


def test_quantize_exact_grid_and_ties():
    """Weights that are exactly E2M1 x E4M3 x 2^-4 (one +-6 per block, one
    block scale 448) come back exactly; and values halfway between E2M1
    neighbours take the even code on both sides."""
    rng = np.random.default_rng(9)
    e2 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
    rows, cols = 16, 128
    idx = rng.integers(0, 16, size=(rows, cols))
    for r in range(rows):
        for b in range(cols // 16):
            idx[r, b * 16 + rng.integers(16)] = 7
    sb = rng.integers(0x08, 0x7F, size=(rows, cols // 16))
    sb[3, 2] = 0x7E
    sv = torch.from_numpy(sb.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    w = e2[idx] * np.repeat(sv, 16, axis=1) * 2.0 ** -4
    bits = fi.f32_to_bf16_bits(w.astype(np.float32))
    gc, gs, g2 = _assert_same(bits, "exact grid")
    assert g2 == 2.0 ** -4
    np.testing.assert_array_equal(gs, sb.astype(np.uint8))
    # midpoints: blocks of scale 1.0 (max 6 sets it), other elements at
    # 0.25, 0.75, ..., 5 times the unit
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 6.0, -6.0])
    blk = np.tile(mids, (8, 4)) * 2.0 ** -4
    blk[0, 0] = 6 * 448 * 2.0 ** -4   # sets scale2 = 2^-4 through amax
    blk[0, 1:16] = 0.0
    _assert_same(fi.f32_to_bf16_bits(blk.astype(np.float32)), "midpoints")


def test_quantize_deterministic():
    bits = fi.make_dense_bf16(256, 1024, 10)
    w = ffn.bf16_from_bits(bits)
    a = ffn.quantize(w)
    b = ffn.quantize(w)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("act", [fi.ACT_SILU, fi.ACT_GELU_TANH])
def test_quantize_then_ffn(act):
    """bf16 weights quantised on the GPU drive the FFN; the oracle quantises
    the same weights (bit-identical bytes, checked) and runs its FFN."""
    M, K, N = 3, 512, 1536
    gb = fi.make_dense_bf16(N, K, 11)
    ub = fi.make_dense_bf16(N, K, 12)
    db = fi.make_dense_bf16(K, N, 13)
    dev = [ffn.quantize_weight(ffn.bf16_from_bits(b)) for b in (gb, ub, db)]
    host = []
    for b, d in zip((gb, ub, db), dev):
        oc, osc, o2 = oracle.quantize(b)
        np.testing.assert_array_equal(d.codes.cpu().numpy(), oc)
        np.testing.assert_array_equal(d.scales.cpu().numpy(), osc)
        assert np.float32(d.scale2) == np.float32(o2)
        host.append(fi.Nvfp4Weight(oc, osc, o2))
    x_bits = fi.f32_to_bf16_bits(np.random.default_rng(14).standard_normal((M, K)).astype(np.float32))
    case = fi.FfnCase("quantised", M, K, N, act, x_bits, host[0], host[1], host[2])
    out = ffn.forward(ffn.bf16_from_bits(x_bits), dev[0], dev[1], dev[2], act)
    torch.cuda.synchronize()
    ref = oracle.ffn(case)
    got = ffn.bf16_to_f64(out)
    bound = oracle.parity_bound(ref)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / np.sqrt(np.mean(ref ** 2))))
