"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each ``pin_*`` function checks the oracle against something it does not
contain: the OCP format tables, torch's own float8 decoder, closed forms of
the activations, exact rational arithmetic, numpy's float64 matmul on cases
where every sum is exact, and the generator's closed-form moments. The
mutation test at the end compiles deliberately broken copies of the oracle
source (on the CPU) and checks that some pin catches each one.
"""
import math
import os
import re
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import ffn_inputs as fi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                rows.append((a, float(b)))
    return rows


def _same_float(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


# ---------------------------------------------------------------- formats


def pin_e2m1_table(orc):
    table = orc.e2m1_table()
    for code, val in _read_table("e2m1_values.txt"):
        assert _same_float(table[int(code)], val), (code, table[int(code)], val)
    assert table.sum() == 0.0
    assert np.sum(table ** 2) == 137.0


def pin_e4m3_vs_torch(orc):
    table = orc.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        assert _same_float(table[b], ref[b]) or (table[b] == 0 and ref[b] == 0 and
                                                 math.copysign(1, table[b]) == math.copysign(1, ref[b])), \
            (hex(b), table[b], ref[b])


def pin_e4m3_anchors_and_order(orc):
    table = orc.e4m3_table()
    for hx, val in _read_table("e4m3_anchors.txt"):
        assert _same_float(table[int(hx, 16)], val), (hx, table[int(hx, 16)], val)
    pos = table[:0x7F]
    assert np.all(np.diff(pos) > 0), "E4M3 magnitudes must increase with the byte"
    assert np.isfinite(table).sum() == 254
    assert np.nanmax(np.abs(table)) == 448.0
    for b in range(0x7F):
        assert _same_float(table[b | 0x80], -table[b])


def pin_byte_nibble_order(orc):
    """Bytes 0..255 as one row of codes: every ordered pair of E2M1 values
    appears once, and byte 0x21 decodes to (0.5, 1.0): the even column is
    the low nibble."""
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    scales = np.full((1, 32), 0x38, dtype=np.uint8)  # 1.0
    w = orc.dequant(fi.Nvfp4Weight(codes, scales, 1.0))[0]
    e2 = [v for _, v in _read_table("e2m1_values.txt")]
    pairs = {(float(w[2 * j]), math.copysign(1, w[2 * j]), float(w[2 * j + 1]), math.copysign(1, w[2 * j + 1]))
             for j in range(256)}
    assert len(pairs) == 256
    assert (w[2 * 0x21], w[2 * 0x21 + 1]) == (0.5, 1.0)
    assert (w[2 * 0x7F], w[2 * 0x7F + 1]) == (-6.0, 6.0)
    assert (w[2 * 0xF0], w[2 * 0xF0 + 1]) == (0.0, -6.0)
    assert sorted(set(float(v) for v in w)) == sorted(set(e2)), "value set is the E2M1 set"


def pin_scale_blocks(orc):
    """Scale byte j of a row applies to columns 16j..16j+15 of that row."""
    rng = np.random.default_rng(3)
    rows, cols = 4, 64
    codes = np.full((rows, cols // 2), 0x22, dtype=np.uint8)  # every element 1.0
    scales = rng.choice(fi.finite_e4m3_bytes(), size=(rows, cols // 16)).astype(np.uint8)
    w = orc.dequant(fi.Nvfp4Weight(codes, scales, 1.0))
    ref = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(w, np.repeat(ref, 16, axis=1))


def _independent_dequant(w):
    """Dequantise with a separate route: nibble unpack by numpy, the E2M1
    values from the OCP table fixture, E4M3 scales decoded by torch."""
    e2 = np.array([v for _, v in _read_table("e2m1_values.txt")])
    lo = w.codes & 0x0F
    hi = w.codes >> 4
    idx = np.stack([lo, hi], axis=-1).reshape(w.codes.shape[0], -1)
    sc = torch.from_numpy(np.ascontiguousarray(w.scales)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return e2[idx] * np.repeat(sc, 16, axis=1) * float(np.float32(w.scale2))


def pin_dequant_independent(orc):
    case = fi.make_format_coverage()
    for w in (case.gate, case.up, case.down):
        np.testing.assert_array_equal(orc.dequant(w), _independent_dequant(w))


# ------------------------------------------------------------ activations


def pin_activations(orc):
    S, G = fi.ACT_SILU, fi.ACT_GELU_TANH
    assert orc.act(S, 0.0) == 0.0 and orc.act(G, 0.0) == 0.0
    xs = np.concatenate([np.linspace(-12, 12, 97), [1e-8, -1e-8, 0.5, -3.7, 30.0, -30.0]])
    for x in xs:
        # Odd-part identities f(x) - f(-x) = x hold for both gates.
        assert abs(orc.act(S, x) - orc.act(S, -x) - x) <= 1e-13 * max(1.0, abs(x))
        assert abs(orc.act(G, x) - orc.act(G, -x) - x) <= 1e-13 * max(1.0, abs(x))
        # Library routines: x * expit(x); torch's tanh-approximate GELU in float64.
        assert abs(orc.act(S, x) - x * scipy.special.expit(x)) <= 1e-14 * max(1.0, abs(x))
        tg = torch.nn.functional.gelu(torch.tensor(x, dtype=torch.float64), approximate="tanh").item()
        assert abs(orc.act(G, x) - tg) <= 1e-14 * max(1.0, abs(x))
    assert abs(orc.act(S, 50.0) - 50.0) < 1e-15 * 50 + 1e-18
    assert abs(orc.act(S, -50.0)) < 1e-19
    assert orc.act(G, 10.0) == 10.0 and abs(orc.act(G, -10.0)) < 1e-30
    assert orc.act(S, 1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


def pin_gated_act(orc):
    rng = np.random.default_rng(5)
    g = rng.normal(size=64) * 4
    u = rng.normal(size=64)
    for kind in (fi.ACT_SILU, fi.ACT_GELU_TANH):
        h = orc.gated_act(kind, g, u)
        for i in range(64):
            assert h[i] == orc.act(kind, g[i]) * u[i]
    # The product is act(gate) * up, not act(up) * gate.
    h = orc.gated_act(fi.ACT_SILU, np.array([2.0]), np.array([-1.0]))
    assert h[0] == pytest.approx(-2.0 * scipy.special.expit(2.0), rel=1e-15)


# ------------------------------------------------------------ linear part


def _one_hot_weight(rows, cols, pick, value_code=0x2):
    """Row r holds code `value_code` at column pick[r]; scale 1.0; scale2 1."""
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    for r, c in enumerate(pick):
        codes[r, c // 2] |= (value_code << 4) if c % 2 else value_code
    scales = np.full((rows, cols // 16), 0x38, dtype=np.uint8)
    return fi.Nvfp4Weight(codes, scales, 1.0)


def pin_one_hot_selects(orc):
    rng = np.random.default_rng(11)
    K, N, M = 96, 40, 3
    pick = rng.integers(0, K, size=N)
    wg = _one_hot_weight(N, K, pick)
    wu = _one_hot_weight(N, K, rng.integers(0, K, size=N), value_code=0xA)  # -1.0
    x_bits = fi.f32_to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    x = fi.bf16_bits_to_f32(x_bits).astype(np.float64)
    case = fi.FfnCase("onehot", M, K, N, fi.ACT_SILU, x_bits, wg, wu, wg)
    gate, up = orc.dual(case)
    np.testing.assert_array_equal(gate, x[:, pick])
    # Doubling scale2 doubles the output exactly.
    case2 = fi.FfnCase("onehot2", M, K, N, fi.ACT_SILU, x_bits,
                       fi.Nvfp4Weight(wg.codes, wg.scales, 2.0), wu, wg)
    g2, _ = orc.dual(case2)
    np.testing.assert_array_equal(g2, 2.0 * gate)


def pin_down_orientation(orc):
    """W_d is [K, N]: out[m, j] = h[m, pick[j]] for a one-hot W_d."""
    rng = np.random.default_rng(12)
    K, N, M = 64, 96, 2
    pick = rng.integers(0, N, size=K)
    wd = _one_hot_weight(K, N, pick)
    h = rng.normal(size=(M, N))
    out = orc.down(h, wd)
    np.testing.assert_array_equal(out, h[:, pick])


def pin_ternary_exact_vs_numpy(orc):
    """Codes in {0, +1, -1} with unit scales: every partial sum of bf16
    inputs is exact in double, so the oracle must equal numpy's matmul
    bit for bit."""
    rng = np.random.default_rng(21)
    M, K, N = 3, 512, 64
    tern = np.array([0x0, 0x2, 0xA], dtype=np.uint8)
    lo = rng.choice(tern, size=(N, K // 2))
    hi = rng.choice(tern, size=(N, K // 2))
    w = fi.Nvfp4Weight((lo | (hi << 4)).astype(np.uint8), np.full((N, K // 16), 0x38, np.uint8), 1.0)
    x_bits = fi.f32_to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    x = fi.bf16_bits_to_f32(x_bits).astype(np.float64)
    wd = np.where(lo == 0x2, 1.0, np.where(lo == 0xA, -1.0, 0.0))
    wdh = np.where(hi == 0x2, 1.0, np.where(hi == 0xA, -1.0, 0.0))
    dense = np.stack([wd, wdh], axis=-1).reshape(N, K)
    ref = x @ dense.T
    np.testing.assert_array_equal(orc.linear(x, w), ref)


def pin_matches_numpy_matmul(orc):
    """General weights: the oracle agrees with numpy's float64 matmul over an
    independently dequantised matrix to double rounding."""
    case = fi.make_format_coverage(M=2)
    x = fi.bf16_bits_to_f32(case.x_bits).astype(np.float64)
    for w in (case.gate, case.up):
        ref = x @ _independent_dequant(w).T
        got = orc.linear(x, w)
        scale = np.abs(x) @ np.abs(_independent_dequant(w)).T
        assert np.all(np.abs(got - ref) <= 1e-12 * scale + 1e-300)


def _exact_x_bits(rng, shape):
    """bf16 values k/64 with |k| < 256: all partial sums stay exact in double."""
    k = rng.integers(-255, 256, size=shape)
    return fi.f32_to_bf16_bits((k / 64.0).astype(np.float32))


def pin_fraction_brute_force(orc):
    """Exact rational gate/up for tiny shapes; the double result must be exact."""
    rng = np.random.default_rng(31)
    M, K, N = 2, 64, 16
    fin = fi.finite_e4m3_bytes()
    # keep scales >= 2^-6 so every product and sum is exact in double
    fin = fin[(fin & 0x78) != 0]

    def weight(rows, cols):
        return fi.Nvfp4Weight(rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8),
                              rng.choice(fin, size=(rows, cols // 16)).astype(np.uint8), 0.375)

    wg, wu = weight(N, K), weight(N, K)
    x_bits = _exact_x_bits(rng, (M, K))
    case = fi.FfnCase("frac", M, K, N, fi.ACT_SILU, x_bits, wg, wu, weight(K, N))
    gate, up = orc.dual(case)
    e2 = [Fraction(v) for _, v in _read_table("e2m1_values.txt")]
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xf = [[Fraction(float(v)) for v in row] for row in fi.bf16_bits_to_f32(x_bits)]
    for w, got in ((wg, gate), (wu, up)):
        for m in range(M):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    byte = int(w.codes[n, k // 2])
                    code = byte & 15 if k % 2 == 0 else byte >> 4
                    acc += e2[code] * Fraction(float(e4[w.scales[n, k // 16]])) * xf[m][k]
                acc *= Fraction(0.375)
                assert Fraction(got[m, n]) == acc, (m, n)


def pin_down_fraction_bound(orc):
    """Down projection over double inputs: within the standard bound
    n*u*sum|w h| of the exact rational result."""
    rng = np.random.default_rng(41)
    K, N, M = 8, 48, 2
    wd = fi.Nvfp4Weight(rng.integers(0, 256, size=(K, N // 2), dtype=np.uint8),
                        rng.choice(fi.finite_e4m3_bytes(), size=(K, N // 16)).astype(np.uint8), 0.7)
    h = rng.normal(size=(M, N)) * 3
    out = orc.down(h, wd)
    dense = _independent_dequant(wd)
    u = 2.0 ** -53
    for m in range(M):
        for j in range(K):
            exact = sum(Fraction(float(dense[j, n])) * Fraction(float(h[m, n])) for n in range(N))
            bound = N * u * float(np.sum(np.abs(dense[j] * h[m]))) * 1.01
            assert abs(float(Fraction(out[m, j]) - exact)) <= bound


def pin_ffn_composition(orc):
    """The whole FFN equals down(act(gate) * up) assembled from library
    routines (numpy matmul, scipy expit, torch gelu) to double rounding."""
    for act in (fi.ACT_SILU, fi.ACT_GELU_TANH):
        case = fi.make_small(2, 128, 96, act=act, seed=51, scale2=0.25)
        out = orc.ffn(case)
        x = fi.bf16_bits_to_f32(case.x_bits).astype(np.float64)
        g = x @ _independent_dequant(case.gate).T
        u = x @ _independent_dequant(case.up).T
        if act == fi.ACT_SILU:
            h = g * scipy.special.expit(g) * u
        else:
            h = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy() * u
        ref = h @ _independent_dequant(case.down).T
        scale = np.abs(h) @ np.abs(_independent_dequant(case.down)).T
        assert np.all(np.abs(out - ref) <= 1e-10 * scale)
        # row subset gives the same rows
        np.testing.assert_array_equal(orc.ffn(case, rows=np.array([1])), out[1:2])


# ------------------------------------------------------------ quantiser


def _bits_of(values):
    """bf16 bit patterns of float values that are exact in bf16."""
    f = np.asarray(values, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def pin_e2m1_encode_grid(orc):
    """Every E2M1 value (from the OCP table fixture, -0 included) encodes to
    its own code; each midpoint goes to its even neighbour; beyond 6
    saturates; the sign bit is the input's (small negatives give -0)."""
    table = _read_table("e2m1_values.txt")
    for code, val in table:
        assert orc.e2m1_encode(val) == int(code), (code, val)
    assert orc.e2m1_encode(0.0) == 0 and orc.e2m1_encode(0.2) == 0
    assert orc.e2m1_encode(-0.0) == 8 and orc.e2m1_encode(-0.2) == 8
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for m, k in mids.items():
        assert orc.e2m1_encode(m) == k, (m, orc.e2m1_encode(m))
        assert orc.e2m1_encode(-m) == k | 8, (-m, orc.e2m1_encode(-m))
        lo = float(np.nextafter(np.float32(m), np.float32(0)))
        hi = float(np.nextafter(np.float32(m), np.float32(10)))
        vals = sorted((abs(v), int(c)) for c, v in table if int(c) < 8)
        below = max(c for v, c in vals if v < m)
        above = min(c for v, c in vals if v > m)
        assert orc.e2m1_encode(lo) == below and orc.e2m1_encode(hi) == above, m
    for v in (6.0001, 7.0, 1e30):
        assert orc.e2m1_encode(v) == 7 and orc.e2m1_encode(-v) == 15


def pin_e4m3_encode_vs_torch(orc):
    """Nearest-even E4M3 of values up to 448 agrees with torch's float8
    conversion (an independent implementation): every finite byte's own
    value, the midpoints between neighbours, and random values; above 448
    the encoder saturates to 0x7E."""
    rng = np.random.default_rng(17)
    vals = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    rand = np.concatenate([rng.uniform(0, 448, 2000), 2.0 ** rng.uniform(-12, 8.8, 2000)]).astype(np.float32)
    probe = np.concatenate([vals, mids, rand, np.float32([0.0, 2 ** -10, 2 ** -10 * 1.0001, 447.9, 448.0])])
    probe = probe[probe <= 448.0]
    ref = torch.from_numpy(probe).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in probe])
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(probe[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]
    for v in (448.5, 464.0, 480.0, 1e6):
        assert orc.e4m3_encode(v) == 0x7E


def pin_quantize_zero(orc):
    codes, scales, s2 = orc.quantize(np.zeros((3, 64), dtype=np.uint16))
    assert s2 == 0.0 and not codes.any() and not scales.any()


def _exact_nvfp4_weight(rng, rows, cols, scale2_exp=-4):
    """A weight whose every element is e2m1 x e4m3 x 2^scale2_exp with one
    element of each block at +-6 times the block scale, and one block scale
    448: the quantiser's rule must give back exactly these codes and scales
    and scale2 = 2^scale2_exp."""
    e2 = np.array([v for _, v in _read_table("e2m1_values.txt")])
    nb = cols // 16
    code_idx = rng.integers(0, 16, size=(rows, cols))
    pos = rng.integers(0, 16, size=(rows, nb))
    for r in range(rows):
        for b in range(nb):
            code_idx[r, b * 16 + pos[r, b]] = 7 if rng.random() < 0.5 else 15  # +-6
    finite = np.arange(1, 0x7F)  # non-zero, non-negative finite scale bytes
    sbytes = rng.choice(finite, size=(rows, nb))
    sbytes[rng.integers(rows), rng.integers(nb)] = 0x7E
    sval = torch.from_numpy(sbytes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    w = e2[code_idx] * np.repeat(sval, 16, axis=1) * 2.0 ** scale2_exp
    return _bits_of(w), w, sbytes.astype(np.uint8)


def pin_quantize_exact_roundtrip(orc):
    rng = np.random.default_rng(23)
    bits, w, sbytes = _exact_nvfp4_weight(rng, 24, 256)
    codes, scales, s2 = orc.quantize(bits)
    assert s2 == 2.0 ** -4, s2
    np.testing.assert_array_equal(scales, sbytes)
    back = orc.dequant(fi.Nvfp4Weight(codes, scales, s2))
    np.testing.assert_array_equal(back, w)


def pin_quantize_error_bound(orc):
    """Random weights: scale2 maps the largest magnitude to 6 * 448 (the block
    holding it gets scale byte 0x7E), and every element is reproduced to
    within one block unit (half the widest E2M1 step, 2) of the block scale."""
    rng = np.random.default_rng(29)
    rows, cols = 40, 512
    f = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-6, 3, size=(rows, 1)))).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)  # truncated to bf16
    wv = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, scales, s2 = orc.quantize(bits)
    amax = np.abs(wv).max()
    assert s2 == float(np.float32(amax) / np.float32(2688.0))
    r, c = np.unravel_index(np.argmax(np.abs(wv)), wv.shape)
    assert scales[r, c // 16] == 0x7E
    back = orc.dequant(fi.Nvfp4Weight(codes, scales, s2))
    sv = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    unit = np.repeat(sv, 16, axis=1) * s2
    assert np.all(np.abs(back - wv) <= unit * (1 + 1e-6) + 1e-300)
    assert np.all(scales < 0x7F)


# ------------------------------------------------------------ FP8 weights


def _torch_e4m3(codes):
    """E4M3FN bytes decoded by torch's float8 type (a route independent of the
    oracle's table)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _fp8_dense(w):
    """Dense float64 [rows, cols]: torch-decoded codes times the block grid
    expanded with numpy (block (i, j) covers rows 128i.., columns 128j..)."""
    grid = np.repeat(np.repeat(w.block_scale.astype(np.float64), 128, axis=0), 128, axis=1)
    return _torch_e4m3(w.codes) * grid[: w.rows, : w.cols]


def _fp8_one_hot(rows, cols, pick, code=0x38):
    """Row r holds `code` (0x38 = 1.0) at column pick[r]; block (i, j) has
    the scale 2**(i - 2 * j), distinct for every block of the grid."""
    codes = np.zeros((rows, cols), dtype=np.uint8)
    codes[np.arange(rows), pick] = code
    gr, gc = (rows + 127) // 128, (cols + 127) // 128
    bs = np.array([[2.0 ** (i - 2 * j) for j in range(gc)] for i in range(gr)], dtype=np.float32)
    return fi.Fp8Weight(codes, bs)


def pin_fp8_block_indexing(orc):
    """A one-hot FP8 weight with a distinct power-of-two scale per 128 x 128
    block, ragged in both directions: gate[m, n] = x[m, pick[n]] * 2**(n//128 -
    2 * (pick[n]//128)) exactly, and a [K, N] down weight picks from h the same
    way."""
    rng = np.random.default_rng(61)
    M, K, N = 2, 400, 300
    pick = rng.integers(0, K, size=N)
    wg = _fp8_one_hot(N, K, pick)
    wu = _fp8_one_hot(N, K, rng.integers(0, K, size=N), code=0xB8)  # -1.0
    x_bits = fi.f32_to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    x = fi.bf16_bits_to_f32(x_bits).astype(np.float64)
    case = fi.Fp8FfnCase("fp8_onehot", M, K, N, fi.ACT_SILU, x_bits, wg, wu, _fp8_one_hot(K, N, np.zeros(K, int)))
    gate, up = orc.fp8_dual(case)
    n = np.arange(N)
    np.testing.assert_array_equal(gate, x[:, pick] * 2.0 ** (n // 128 - 2 * (pick // 128)))
    np.testing.assert_array_equal(up, -x[:, wu.codes.argmax(axis=1)] * 2.0 ** (n // 128 - 2 * (wu.codes.argmax(axis=1) // 128)))
    pick_d = rng.integers(0, N, size=K)
    h = rng.normal(size=(M, N))
    out = orc.fp8_linear(h, _fp8_one_hot(K, N, pick_d))
    j = np.arange(K)
    np.testing.assert_array_equal(out, h[:, pick_d] * 2.0 ** (j // 128 - 2 * (pick_d // 128)))


def pin_fp8_dequant_vs_torch(orc):
    """Every finite E4M3FN byte, ragged grids: the oracle's dequantised weight
    equals torch's float8 decode times the numpy-expanded block grid, bit for
    bit (an E4M3 value times an fp32 value is exact in double)."""
    case = fi.make_fp8_format_coverage()
    for w in (case.gate, case.up, case.down):
        assert len(np.unique(w.codes)) == 254
        np.testing.assert_array_equal(orc.fp8_dequant(w), _fp8_dense(w))


def pin_fp8_exact_vs_numpy(orc):
    """Codes in {0, +-1, +-2} and power-of-two block scales: every partial sum
    of bf16 inputs is exact in double, so the oracle equals numpy's float64
    matmul bit for bit, including over a ragged last block."""
    rng = np.random.default_rng(62)
    M, K, N = 3, 320, 136
    codes = rng.choice(np.array([0x00, 0x38, 0xB8, 0x40, 0xC0], dtype=np.uint8), size=(N, K))
    bs = (2.0 ** rng.integers(-3, 4, size=((N + 127) // 128, (K + 127) // 128))).astype(np.float32)
    w = fi.Fp8Weight(codes, bs)
    x_bits = fi.f32_to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    x = fi.bf16_bits_to_f32(x_bits).astype(np.float64)
    np.testing.assert_array_equal(orc.fp8_linear(x, w), x @ _fp8_dense(w).T)


def pin_fp8_fraction_bound(orc):
    """Random finite codes and random fp32 block scales over two ragged block
    columns and rows: the oracle's gate and up are within the standard bound
    n*u*sum|w x| of the exact rational results."""
    rng = np.random.default_rng(63)
    M, K, N = 2, 160, 130
    fin = fi.finite_e4m3_bytes()

    def weight(rows, cols):
        grid = ((rows + 127) // 128, (cols + 127) // 128)
        return fi.Fp8Weight(rng.choice(fin, size=(rows, cols)).astype(np.uint8),
                            rng.uniform(0.1, 3.0, size=grid).astype(np.float32))

    wg, wu = weight(N, K), weight(N, K)
    x_bits = _exact_x_bits(rng, (M, K))
    case = fi.Fp8FfnCase("fp8_frac", M, K, N, fi.ACT_SILU, x_bits, wg, wu, weight(K, N))
    gate, up = orc.fp8_dual(case)
    xf = fi.bf16_bits_to_f32(x_bits).astype(np.float64)
    u = 2.0 ** -53
    for w, got in ((wg, gate), (wu, up)):
        e4 = _torch_e4m3(w.codes)
        for m in range(M):
            for n in range(0, N, 3):
                terms = [Fraction(float(e4[n, k])) * Fraction(float(w.block_scale[n // 128, k // 128]))
                         * Fraction(float(xf[m, k])) for k in range(K)]
                exact = sum(terms)
                bound = K * u * float(sum(abs(t) for t in terms)) * 1.01
                assert abs(float(Fraction(got[m, n]) - exact)) <= bound, (m, n)


def pin_fp8_ffn_composition(orc):
    """The whole FP8 FFN equals down(act(gate) * up) assembled from torch's
    float8 decode, numpy matmul, scipy expit and torch's gelu, to double
    rounding; a row subset gives the same rows."""
    for act in (fi.ACT_SILU, fi.ACT_GELU_TANH):
        case = fi.make_fp8_ffn("fp8_comp", 3, 192, 160, act=act, seed=64)
        out = orc.fp8_ffn(case)
        x = fi.bf16_bits_to_f32(case.x_bits).astype(np.float64)
        g = x @ _fp8_dense(case.gate).T
        u = x @ _fp8_dense(case.up).T
        if act == fi.ACT_SILU:
            h = g * scipy.special.expit(g) * u
        else:
            h = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy() * u
        ref = h @ _fp8_dense(case.down).T
        scale = np.abs(h) @ np.abs(_fp8_dense(case.down)).T
        assert np.all(np.abs(out - ref) <= 1e-10 * scale)
        np.testing.assert_array_equal(orc.fp8_ffn(case, rows=np.array([2])), out[2:3])


# ------------------------------------------------------------ W4A4 (MXFP4)

_E2M1 = None


def _e2m1_table():
    global _E2M1
    if _E2M1 is None:
        _E2M1 = np.array([v for _, v in _read_table("e2m1_values.txt")])
    return _E2M1


def _mx_decode(codes, e8m0):
    """MXFP4 -> float64 with the OCP E2M1 value table fixture and numpy
    (element 2j is the low nibble of byte j; 2^(byte - 127) per 32)."""
    t = _e2m1_table()
    vals = np.stack([t[codes & 15], t[codes >> 4]], axis=-1).reshape(codes.shape[0], -1)
    return vals * np.repeat(np.ldexp(1.0, e8m0.astype(np.int64) - 127), 32, axis=1)


def pin_mx_exponent_rule(orc):
    """The shared exponent is floor(log2(amax)) - 2 (math.frexp here), clamped
    to [-127, 127]; anchors: amax 1 -> -2, 4 -> 0, 6 -> 0, 7.99 -> 0, 3.99 -> -1,
    0.75 -> -3, 0 -> 0."""
    for amax, want in ((1.0, -2), (4.0, 0), (6.0, 0), (7.99, 0), (3.99, -1), (0.75, -3), (0.0, 0),
                       (2.0 ** -130, -127), (2.0 ** 200, 127)):
        assert orc.mx_block_exponent(amax) == want, (amax, orc.mx_block_exponent(amax), want)
    rng = np.random.default_rng(71)
    for amax in np.exp(rng.uniform(-60, 60, size=200)):
        m, e = math.frexp(amax)
        assert orc.mx_block_exponent(amax) == max(-127, min(127, e - 1 - 2))


def pin_mx_quantize_nearest(orc):
    """Every element decodes to a nearest point of the E2M1 grid times the
    block's scale, ties to the even code, saturating at 6, sign kept; brute
    force over the fixture table in numpy."""
    rng = np.random.default_rng(72)
    v = rng.normal(size=(6, 256)) * np.exp(rng.uniform(-8, 8, size=(6, 1)))
    v[0, :32] = 0.0
    v[1, 5] = -1e-30
    codes, e8m0 = orc.mx_quantize(v)
    t = _e2m1_table()
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            se = 0 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 3))
            assert e8m0[r, b] == se + 127
            for j in range(32):
                c = 32 * b + j
                byte = codes[r, c // 2]
                code = byte & 15 if c % 2 == 0 else byte >> 4
                q = float(np.float32(blk[j] / 2.0 ** se))
                a = abs(q)
                if a >= 6:
                    assert code & 7 == 7
                else:
                    d = np.abs(t[:8] - a)
                    best = np.flatnonzero(d == d.min())
                    assert (code & 7) in best, (r, c, q, code)
                    if len(best) == 2:
                        assert (code & 7) % 2 == 0
                assert (code >> 3) == (1 if math.copysign(1.0, q) < 0 else 0)


def pin_mx_grid_roundtrip(orc):
    """Blocks built as E2M1 values x 2^s with a largest magnitude of 4 or 6
    come back exactly: codes, and E8M0 = s + 127."""
    rng = np.random.default_rng(73)
    rows, cols = 4, 128
    codes = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    codes[:, ::32] = rng.choice([6, 7, 14, 15], size=(rows, cols // 32))  # +-4 or +-6 in every block
    s = rng.integers(-20, 20, size=(rows, cols // 32))
    v = _e2m1_table()[codes] * np.repeat(np.ldexp(1.0, s), 32, axis=1)
    mc, me = orc.mx_quantize(v)
    np.testing.assert_array_equal(me, (s + 127).astype(np.uint8))
    np.testing.assert_array_equal(_mx_decode(mc, me), v)


def _aligned_nvfp4(rng, rows, cols):
    """An NVFP4 weight whose two E4M3 scales in each 32-block are one power of
    two and whose block maximum is 4 or 6: exactly MXFP4-representable."""
    codes = rng.integers(0, 16, size=(rows, cols)).astype(np.uint8)
    codes[:, ::32] = rng.choice([6, 7, 14, 15], size=(rows, cols // 32))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    e = rng.integers(-6, 3, size=(rows, cols // 32))
    sc = np.repeat(((e + 7) << 3).astype(np.uint8), 2, axis=1)  # E4M3 2^e, same for both halves
    return fi.Nvfp4Weight(packed, sc, 0.75)


def pin_mx_requant(orc):
    """Requantising an exactly representable NVFP4 weight keeps every value;
    on general weights every requantised value is the nearest-grid MXFP4 of
    the NVFP4 value (checked through the quantiser pinned above, on the
    independently dequantised weight)."""
    rng = np.random.default_rng(74)
    w = _aligned_nvfp4(rng, 8, 256)
    mx = orc.mx_requant(w)
    assert mx.scale2 == 0.75
    np.testing.assert_array_equal(_mx_decode(mx.codes, mx.e8m0), _independent_dequant(fi.Nvfp4Weight(w.codes, w.scales, 1.0)))
    g = fi.make_small(1, 256, 96, seed=75).gate
    mx = orc.mx_requant(g)
    c2, e2 = orc.mx_quantize(_independent_dequant(fi.Nvfp4Weight(g.codes, g.scales, 1.0)))
    np.testing.assert_array_equal(mx.codes, c2)
    np.testing.assert_array_equal(mx.e8m0, e2)


def pin_w4a4_reduces_to_w4a16(orc):
    """Activations exactly on each block's MXFP4 grid and exactly
    representable weights: the W4A4 gate/up equal the W4A16 oracle's bit for
    bit (both sum the same exact products in the same order)."""
    rng = np.random.default_rng(76)
    M, K, N = 3, 256, 64
    wg, wu = _aligned_nvfp4(rng, N, K), _aligned_nvfp4(rng, N, K)
    xc = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    xc[:, ::32] = 7
    xs = rng.integers(-4, 4, size=(M, K // 32))
    xv = _e2m1_table()[xc] * np.repeat(np.ldexp(1.0, xs), 32, axis=1)
    x_bits = fi.f32_to_bf16_bits(xv.astype(np.float32))
    assert np.array_equal(fi.bf16_bits_to_f32(x_bits).astype(np.float64), xv)
    case = fi.FfnCase("w4a4_exact", M, K, N, fi.ACT_SILU, x_bits, wg, wu, _aligned_nvfp4(rng, K, N))
    g4, u4 = orc.w4a4_dual(case, orc.mx_requant(wg), orc.mx_requant(wu))
    g, u = orc.dual(case)
    np.testing.assert_array_equal(g4, g)
    np.testing.assert_array_equal(u4, u)


def pin_w4a4_matches_numpy(orc):
    """General activations and weights: W4A4 gate/up equal scale2 times numpy's
    float64 matmul of the independently decoded MXFP4 operands, to double
    rounding; the whole hybrid FFN equals the W4A16 down GEMV (oracle.down,
    pinned above) of act(gate) * up from scipy/torch."""
    for act in (fi.ACT_SILU, fi.ACT_GELU_TANH):
        case = fi.make_small(2, 192, 160, act=act, seed=77, scale2=0.375)
        gm, um = orc.mx_requant(case.gate), orc.mx_requant(case.up)
        g4, u4 = orc.w4a4_dual(case, gm, um)
        xc, xe = orc.mx_quantize_bf16(case.x_bits)
        xa = _mx_decode(xc, xe)
        for mx, got in ((gm, g4), (um, u4)):
            wd = _mx_decode(mx.codes, mx.e8m0)
            ref = 0.375 * (xa @ wd.T)
            assert np.all(np.abs(got - ref) <= 1e-12 * (np.abs(xa) @ np.abs(wd).T) + 1e-300)
        if act == fi.ACT_SILU:
            h = g4 * scipy.special.expit(g4) * u4
        else:
            h = torch.nn.functional.gelu(torch.from_numpy(g4), approximate="tanh").numpy() * u4
        ref = h @ _independent_dequant(case.down).T
        out = orc.w4a4_ffn(case, gm, um)
        assert np.all(np.abs(out - ref) <= 1e-10 * (np.abs(h) @ np.abs(_independent_dequant(case.down)).T))
        np.testing.assert_array_equal(orc.w4a4_ffn(case, gm, um, rows=np.array([1])), out[1:2])


def _bf16_bits_of_f32(f):
    """float32 -> bf16 bit patterns, nearest with ties to even (the usual
    integer form: add 0x7FFF plus the kept lowest bit, truncate), for finite
    values."""
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def pin_bf16_round(orc):
    """The oracle's bf16 rounding (h of the all-W4A4 FFN): ties to even at the
    binade's spacing, signed zero, the subnormal spacing 2^-133, overflow to
    infinity past halfway above the largest finite bf16; and, on float32
    inputs (where one rounding from double equals one from float32), the
    integer rounding of the bit pattern."""
    r = orc.bf16_round_bits
    assert r(1.0) == 0x3F80
    assert r(1.0 + 2.0 ** -8) == 0x3F80          # tie: even (1.0) wins
    assert r(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie: even (1 + 2^-6) wins
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -20) == 0x3F81
    assert r(-2.5) == 0xC020
    assert r(0.0) == 0x0000 and r(-0.0) == 0x8000
    assert r(2.0 ** -133) == 0x0001 and r(2.0 ** -134) == 0x0000 and r(0.75 * 2.0 ** -133) == 0x0001
    big = float(np.uint32(0x7F7F0000).view(np.float32))  # the largest finite bf16, 3.3895e38
    assert r(big) == 0x7F7F and r(3.38e38) == 0x7F7E      # below the midpoint 3.3829e38 to 0x7F7F
    assert r(3.4e38) == 0x7F80 and r(-3.4e38) == 0xFF80   # past halfway to 2^128
    rng = np.random.default_rng(78)
    f = (rng.normal(size=4000) * np.exp(rng.uniform(-40, 40, size=4000))).astype(np.float32)
    want = _bf16_bits_of_f32(f)
    got = np.array([r(float(v)) for v in f], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


def _random_mx(rng, rows, cols, scale2):
    codes = rng.integers(0, 256, size=(rows, cols // 2)).astype(np.uint8)
    e8m0 = rng.integers(120, 131, size=(rows, cols // 32)).astype(np.uint8)
    return fi.MxWeight(codes, e8m0, scale2)


def pin_w4a4_down(orc):
    """The down projection on 4 bits. h already on each block's MXFP4 grid
    (largest magnitude 4 or 6 times 2^s): quantising it is the identity, and
    the result is scale2 times numpy's float64 product of h with the
    independently decoded MXFP4 weight. General h: the same with h replaced
    by the quantiser's output (the quantiser is pinned above)."""
    rng = np.random.default_rng(79)
    M, N, K = 3, 256, 96
    w = _random_mx(rng, K, N, 0.625)
    wd = _mx_decode(w.codes, w.e8m0)
    hc = rng.integers(0, 16, size=(M, N)).astype(np.uint8)
    hc[:, ::32] = rng.choice([6, 7, 14, 15], size=(M, N // 32))
    hs = rng.integers(-8, 8, size=(M, N // 32))
    hv = _e2m1_table()[hc] * np.repeat(np.ldexp(1.0, hs), 32, axis=1)
    h_bits = fi.f32_to_bf16_bits(hv.astype(np.float32))
    assert np.array_equal(fi.bf16_bits_to_f32(h_bits).astype(np.float64), hv)
    got = orc.w4a4_down(h_bits, w)
    ref = 0.625 * (hv @ wd.T)
    assert np.all(np.abs(got - ref) <= 1e-12 * (np.abs(hv) @ np.abs(wd).T))
    h_bits = fi.f32_to_bf16_bits(rng.normal(size=(M, N)).astype(np.float32))
    qc, qe = orc.mx_quantize_bf16(h_bits)
    ha = _mx_decode(qc, qe)
    got = orc.w4a4_down(h_bits, w)
    assert np.all(np.abs(got - 0.625 * (ha @ wd.T)) <= 1e-12 * (np.abs(ha) @ np.abs(wd).T))


def pin_w4a4_ffn_fp4(orc):
    """The all-W4A4 FFN, through exact symmetries that a dropped or misplaced
    term breaks: negating W_d (sign bits of its codes) or W_u negates the
    output exactly (h = act(gate) * up is odd in up, and bf16 rounding and
    MXFP4 quantisation keep signs), and doubling scale2_d doubles it; its
    rows do not depend on the other rows."""
    for act in (fi.ACT_SILU, fi.ACT_GELU_TANH):
        case = fi.make_small(3, 256, 512, act=act, seed=80, scale2=0.5)
        gm, um, dm = orc.mx_requant(case.gate), orc.mx_requant(case.up), orc.mx_requant(case.down)
        out = orc.w4a4_ffn_fp4(case, gm, um, dm)
        assert np.isfinite(out).all() and np.abs(out).max() > 0
        neg = lambda w: fi.MxWeight((w.codes ^ 0x88).astype(np.uint8), w.e8m0, w.scale2)
        np.testing.assert_array_equal(orc.w4a4_ffn_fp4(case, gm, um, neg(dm)), -out)
        np.testing.assert_array_equal(orc.w4a4_ffn_fp4(case, gm, neg(um), dm), -out)
        d2 = fi.MxWeight(dm.codes, dm.e8m0, 2 * dm.scale2)
        np.testing.assert_array_equal(orc.w4a4_ffn_fp4(case, gm, um, d2), 2 * out)
        np.testing.assert_array_equal(orc.w4a4_ffn_fp4(case, gm, um, dm, rows=np.array([2])), out[2:3])


PINS = [pin_e2m1_table, pin_e4m3_vs_torch, pin_e4m3_anchors_and_order, pin_byte_nibble_order,
        pin_scale_blocks, pin_dequant_independent, pin_activations, pin_gated_act,
        pin_one_hot_selects, pin_down_orientation, pin_ternary_exact_vs_numpy,
        pin_matches_numpy_matmul, pin_fraction_brute_force, pin_down_fraction_bound,
        pin_ffn_composition, pin_e2m1_encode_grid, pin_e4m3_encode_vs_torch, pin_quantize_zero,
        pin_quantize_exact_roundtrip, pin_quantize_error_bound, pin_fp8_block_indexing,
        pin_fp8_dequant_vs_torch, pin_fp8_exact_vs_numpy, pin_fp8_fraction_bound, pin_fp8_ffn_composition,
        pin_mx_exponent_rule, pin_mx_quantize_nearest, pin_mx_grid_roundtrip, pin_mx_requant,
        pin_w4a4_reduces_to_w4a16, pin_w4a4_matches_numpy, pin_bf16_round, pin_w4a4_down, pin_w4a4_ffn_fp4]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle.default())


# ------------------------------------------------------------ generator


def test_generator_moments():
    """rms(gate) follows from the draw: E[e2m1^2] = 137/16, E[scale^2] over
    2^u, u uniform on {-6..0}, is (1/7) sum 4^u; so rms = sqrt(K * 137/16 *
    E[s^2]) * scale2 * sigma."""
    case = fi.make_small(4, 1024, 2048, seed=61, scale2=0.5)
    gate, up = oracle.dual(case)
    es2 = sum(4.0 ** u for u in range(-6, 1)) / 7.0
    x = fi.bf16_bits_to_f32(case.x_bits).astype(np.float64)
    expect = math.sqrt(case.K * (137 / 16) * es2 * np.mean(x ** 2)) * 0.5
    for a in (gate, up):
        got = math.sqrt(np.mean(a ** 2))
        assert abs(got / expect - 1) < 0.05, (got, expect)
    # codes uniform over all 16 nibbles, scales over exactly 7 bytes
    assert set(np.unique(case.gate.scales)) == {(u + 7) << 3 for u in range(-6, 1)}
    nib = np.concatenate([(case.gate.codes & 15).ravel(), (case.gate.codes >> 4).ravel()])
    counts = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(counts - 1 / 16) < 0.01)


def test_generator_deterministic_and_shapes():
    a = fi.make_config(0)
    b = fi.make_config(0)
    np.testing.assert_array_equal(a.gate.codes, b.gate.codes)
    np.testing.assert_array_equal(a.x_bits, b.x_bits)
    assert a.gate.codes.shape == (512, 128) and a.gate.scales.shape == (512, 16)
    assert a.down.codes.shape == (256, 256) and a.down.scales.shape == (256, 32)
    assert a.weight_bytes == 221184


def test_fp8_generator_shapes_and_recipe():
    """The FP8 draw: row-major codes, ceil-128 block grids, no NaN byte, the
    recipe's magnitude fields only, scales in [2**-10, 2**-9), deterministic."""
    a = fi.make_fp8_ffn("a", 2, 640, 1000, seed=5)
    b = fi.make_fp8_ffn("b", 2, 640, 1000, seed=5)
    for wa, wb, shape in ((a.gate, b.gate, (1000, 640)), (a.up, b.up, (1000, 640)), (a.down, b.down, (640, 1000))):
        assert wa.codes.shape == shape and wa.codes.dtype == np.uint8
        assert wa.block_scale.shape == ((shape[0] + 127) // 128, (shape[1] + 127) // 128)
        assert wa.block_scale.dtype == np.float32
        assert np.all((wa.codes & 0x7F) < fi.FP8_RECIPE_MAGS)
        assert np.all((wa.block_scale >= 2.0 ** -10) & (wa.block_scale < 2.0 ** -9))
        np.testing.assert_array_equal(wa.codes, wb.codes)
        np.testing.assert_array_equal(wa.block_scale, wb.block_scale)
    np.testing.assert_array_equal(a.x_bits, b.x_bits)
    c = fi.make_fp8_config(M=1)
    assert (c.K, c.N, c.M) == (5120, 17408, 1)
    assert c.gate.block_scale.shape == (136, 40) and c.down.block_scale.shape == (40, 136)


def test_format_coverage_case():
    c = fi.make_format_coverage()
    allsc = np.concatenate([c.gate.scales.ravel(), c.up.scales.ravel(), c.down.scales.ravel()])
    assert set(np.unique(allsc)) == set(fi.finite_e4m3_bytes().tolist())
    nib = np.concatenate([(c.gate.codes & 15).ravel(), (c.gate.codes >> 4).ravel()])
    assert set(np.unique(nib)) == set(range(16))


def test_golden_tiny_config():
    """Regression pin of the oracle on the tiny config, written by
    tests/golden/make_golden.py (which calls only the oracle)."""
    path = os.path.join(GOLDEN, "tiny_silu_m1_out.txt")
    ref = np.loadtxt(path, dtype=np.float64).reshape(1, -1)
    out = oracle.ffn(fi.make_config(0))
    np.testing.assert_allclose(out, ref, rtol=1e-15, atol=0)


# ------------------------------------------------------------ mutations


MUTANTS = {
    "nibble_order": ("(c % 2 == 0) ? (byte & 0x0F) : (byte >> 4)", "(c % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e2m1_sign": ("return s ? -mag : mag;\n}\n\n/* E4M3FN", "return mag;\n}\n\n/* E4M3FN"),
    "e4m3_bias": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3_subnormal": ("ldexp(m / 8.0, -6)", "ldexp(1.0 + m / 8.0, -6)"),
    "e4m3_nan": ("if (e == 15 && m == 7)\n        return NAN;", "if (0)\n        return NAN;"),
    "scale_block": ("(size_t)(c / 16)]", "(size_t)(c / 32)]"),
    "scale2_dropped": ("e2m1[code] * e4m3[sb] * scale2", "e2m1[code] * e4m3[sb]"),
    "silu_sign": ("g / (1.0 + exp(-g))", "g / (1.0 + exp(g))"),
    "gelu_coeff": ("0.044715 * g * g * g", "0.044715 * g * g"),
    "gate_up_swapped": ("h[i] = oracle_act(act, gate[i]) * up[i];", "h[i] = oracle_act(act, up[i]) * gate[i];"),
    "dropped_last_term": ("for (int c = 0; c < cols; ++c)\n            acc += weight_at",
                          "for (int c = 0; c < cols - 1; ++c)\n            acc += weight_at"),
    "row_index": ("codes[(size_t)r * (size_t)(cols / 2)", "codes[(size_t)(r / 2) * (size_t)(cols / 2)"),
    "q_e2m1_ties_odd": ("if (d < bd || (d == bd && (k & 1) == 0 && (best & 1) == 1)) {\n            best = k;",
                        "if (d < bd || (d == bd && (k & 1) == 1 && (best & 1) == 0)) {\n            best = k;"),
    "q_e4m3_ties_odd": ("if (d < bd || (d == bd && (b & 1) == 0 && (best & 1) == 1)) {",
                        "if (d < bd || (d == bd && (b & 1) == 1 && (best & 1) == 0)) {"),
    "q_e2m1_sign": ("return signbit(q) ? (best | 8) : best;", "return best;"),
    "q_scale_rule": ("amax / 2688.0f", "amax / 448.0f"),
    "q_block_max": ("for (int j = 0; j < 16; ++j) {\n                const float v", "for (int j = 0; j < 15; ++j) {\n                const float v"),
    "q_pack_nibble": ("(c % 2 == 0) ? code : (code << 4)", "(c % 2 == 0) ? (code << 4) : code"),
    "q_e2m1_saturation": ("return signbit(q) ? 15 : 7;", "return signbit(q) ? 14 : 6;"),
    "q_e4m3_range": ("for (int b = 0; b < 127; ++b) {", "for (int b = 0; b < 126; ++b) {"),
    "mx_exp_offset": ("int se = (e - 1) - 2;", "int se = (e - 1) - 1;"),
    "mx_exp_round": ("int se = (e - 1) - 2;", "int se = e - 2;"),
    "mx_zero_scale": ("            const int se = oracle_mx_block_exponent(amax);\n            e8m0[(size_t)r * nb + b] = (uint8_t)(se + 127);",
                      "            const int se = oracle_mx_block_exponent(amax);\n            e8m0[(size_t)r * nb + b] = (uint8_t)(se + 126);"),
    "mx_requant_scale_dropped": ("    oracle_dequant(codes, scales, 1.0f, rows, cols, v);\n    oracle_mx_quantize(v, rows, cols, mx_codes",
                                 "    oracle_dequant(codes, scales, 1.0f, rows, cols, v);\n    for (size_t i = 0; i < (size_t)rows * cols; ++i) v[i] = v[i] > 0 ? 1.0 : (v[i] < 0 ? -1.0 : 0.0);\n    oracle_mx_quantize(v, rows, cols, mx_codes"),
    "mx_act_nibbles": ("const int ac = (c % 2 == 0) ? (ab & 0x0F) : (ab >> 4);", "const int ac = (c % 2 == 0) ? (ab >> 4) : (ab & 0x0F);"),
    "w4a4_scale2_dropped": ("            gate[i] *= (double)g_scale2;", "            gate[i] *= 1.0;"),
    "w4a4_down_scale2": ("u_scale2, gate, up) == 0) {\n        oracle_gated_act(act, gate, up, mn, gate);\n        oracle_down(gate, M, N, K, d_codes, d_scales, d_scale2, out);",
                         "u_scale2, gate, up) == 0) {\n        oracle_gated_act(act, gate, up, mn, gate);\n        oracle_down(gate, M, N, K, d_codes, d_scales, 1.0f, out);"),
    "fp8_block_cols": ("(size_t)(c / 128)]", "(size_t)(c / 64)]"),
    "fp8_block_rows": ("(size_t)(r / 128) * (size_t)bcols", "(size_t)(r / 256) * (size_t)bcols"),
    "fp8_grid_stride": ("int bcols = (cols + 127) / 128;", "int bcols = cols / 128;"),
    "fp8_scale_dropped": ("c]] * (double)bs[", "c]] + 0.0 * (double)bs["),
    "fp8_up_from_gate": ("oracle_fp8_linear_f64(x, M, K, N, uw, ubs, up);", "oracle_fp8_linear_f64(x, M, K, N, gw, gbs, up);"),
    "fp8_down_from_up": ("oracle_fp8_linear_f64(gate, M, N, K, dw, dbs, out);",
                         "oracle_fp8_linear_f64(gate, M, N, K, uw, ubs, out);"),
    "fp8_dropped_last_term": ("for (int c = 0; c < cols; ++c)\n            acc += fp8_weight_at",
                              "for (int c = 1; c < cols; ++c)\n            acc += fp8_weight_at"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    """A plausible mistake planted in a copy of the oracle (CPU only) must make
    at least one pin fail."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ffn_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    mpath = tmp_path / f"mut_{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(mpath), out=str(tmp_path / f"mut_{name}.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"


@pytest.mark.parametrize("act", [fi.ACT_SILU, fi.ACT_GELU_TANH])
def test_h_rounding_bound_covers_bf16_h(act):
    """The format-coverage FFN bound: storing h = act(gate) * up in bf16 (with
    gate and up in fp32) stays within parity_bound + h_rounding_bound of the
    exact result, here simulated with torch's bf16 rounding."""
    import torch

    case = fi.make_format_coverage(act=act, M=128)
    g, u = oracle.dual(case)
    h = oracle.gated_act(act, g.astype(np.float32).astype(np.float64), u.astype(np.float32).astype(np.float64))
    hb = torch.from_numpy(h).to(torch.bfloat16).double().numpy()
    staged = oracle.down(hb, case.down)
    ref = oracle.ffn(case)
    extra = oracle.h_rounding_bound(case)
    assert np.all(np.abs(staged - ref) <= oracle.parity_bound(ref) + extra)
    assert np.all(extra >= 0) and np.all(np.isfinite(extra))
