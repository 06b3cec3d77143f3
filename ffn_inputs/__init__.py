"""Seeded synthetic inputs for the NVFP4 W4A16 gated FFN.

This module only draws random bytes and random bf16 activations. It holds none
of the FFN's arithmetic (no decoding of codes or scales, no products, no
activation functions), so both the CPU oracle and the GPU library can take
their inputs from here without sharing any of the method.

Storage layout of one NVFP4 weight of logical shape [rows, cols] (the layout
described on the dense_ffn.rs page, in the docs of the int8 requant helper of
``DenseFfnLayer``: packed E2M1 ``[N, K/2]``, per-16 E4M3 ``[N, K/16]``, one
per-tensor F32 ``weight_scale_2``):

* ``codes``  uint8 ``[rows, cols/2]``: two 4-bit codes per byte, the code of
  the even column in the low nibble (the reading taken where the pages are
  silent);
* ``scales`` uint8 ``[rows, cols/16]``: one E4M3 byte per 16 consecutive
  columns of a row;
* ``scale2`` a Python float (an fp32 value).

Workload recipe (synthetic stand-ins for the checkpoints the pages run):

* codes: bytes uniform on 0..255, i.e. two independent uniform nibbles;
* scales: ``2**u`` with ``u`` uniform on {-6..0}, stored as the exact E4M3
  byte ``(u + 7) << 3``;
* scale2: 1.0 for the tiny case, ``2**-4`` otherwise;
* x: fp32 normal times sigma, rounded to bf16 (round to nearest even);
* draw order: gate codes, gate scales, up codes, up scales, down codes, down
  scales, then x.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

SEED_BASE = 20261202

ACT_SILU = 0
ACT_GELU_TANH = 1
ACT_NAMES = {ACT_SILU: "silu", ACT_GELU_TANH: "gelu_tanh"}


@dataclasses.dataclass
class Nvfp4Weight:
    """One NVFP4 weight of logical shape [rows, cols] (see module docstring)."""

    codes: np.ndarray   # uint8 [rows, cols // 2]
    scales: np.ndarray  # uint8 [rows, cols // 16]
    scale2: float

    @property
    def rows(self) -> int:
        return int(self.codes.shape[0])

    @property
    def cols(self) -> int:
        return int(self.codes.shape[1]) * 2

    @property
    def nbytes(self) -> int:
        return int(self.codes.nbytes + self.scales.nbytes)


@dataclasses.dataclass
class FfnCase:
    """Inputs of one gated-FFN call: out[M,K] = W_d (act(W_g x) * (W_u x))."""

    name: str
    M: int
    K: int          # hidden size
    N: int          # intermediate size
    act: int        # ACT_SILU or ACT_GELU_TANH
    x_bits: np.ndarray  # uint16 [M, K], bf16 bit patterns
    gate: Nvfp4Weight   # [N, K]
    up: Nvfp4Weight     # [N, K]
    down: Nvfp4Weight   # [K, N]

    def with_x(self, x_bits: np.ndarray, name: Optional[str] = None) -> "FfnCase":
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        return dataclasses.replace(self, x_bits=x_bits, M=int(x_bits.shape[0]),
                                   name=name or self.name)

    @property
    def weight_bytes(self) -> int:
        return self.gate.nbytes + self.up.nbytes + self.down.nbytes


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Only finite inputs are expected here (normal draws)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw_weight(rng: np.random.Generator, rows: int, cols: int, scale2: float) -> Nvfp4Weight:
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    u = rng.integers(-6, 1, size=(rows, cols // 16), dtype=np.int16)
    scales = ((u + 7) << 3).astype(np.uint8)
    return Nvfp4Weight(codes=codes, scales=scales, scale2=float(scale2))


def _draw_x(rng: np.random.Generator, M: int, K: int, sigma: float) -> np.ndarray:
    x = rng.standard_normal(size=(M, K), dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(x)


def make_ffn(name: str, M: int, K: int, N: int, act: int, sigma: float, scale2: float,
             seed: int, x_seed: Optional[int] = None) -> FfnCase:
    """Draw one case. Weights come from ``seed``; x from the same stream, or
    from ``x_seed`` when given (so batched cases can reuse a weight set)."""
    if K % 32 or N % 32:
        raise ValueError("K and N must be multiples of 32")
    rng = np.random.Generator(np.random.PCG64(seed))
    gate = _draw_weight(rng, N, K, scale2)
    up = _draw_weight(rng, N, K, scale2)
    down = _draw_weight(rng, K, N, scale2)
    if x_seed is not None:
        rng = np.random.Generator(np.random.PCG64(x_seed))
    x_bits = _draw_x(rng, M, K, sigma)
    return FfnCase(name=name, M=M, K=K, N=N, act=act, x_bits=x_bits, gate=gate, up=up, down=down)


# The five workloads: tiny SwiGLU, decode SwiGLU, decode GELU-tanh,
# speculative-verify batch, prefill batch.
CONFIG_NAMES = ["tiny_silu_m1", "decode_silu_m1", "decode_gelu_m1", "verify_silu", "prefill_silu_m128"]


def make_config(index: int, M: Optional[int] = None) -> FfnCase:
    """Build config ``index`` (0..4). ``M`` picks the row count for config 3
    (2, 3 and 8 are the verify batches; 4 to 7 the others a batch of up to 8
    can take; default 8) and may override the row count of config 4."""
    seed = SEED_BASE + index
    if index == 0:
        return make_ffn(CONFIG_NAMES[0], 1, 256, 512, ACT_SILU, 1.0, 1.0, seed)
    if index == 1:
        return make_ffn(CONFIG_NAMES[1], 1, 5120, 17408, ACT_SILU, 1.0, 2.0 ** -4, seed)
    if index == 2:
        return make_ffn(CONFIG_NAMES[2], 1, 5376, 21504, ACT_GELU_TANH, 0.5, 2.0 ** -4, seed)
    if index in (3, 4):
        m = M if M is not None else (8 if index == 3 else 128)
        if index == 3 and not 2 <= m <= 8:
            raise ValueError("verify config takes 2 <= M <= 8")
        # Reuse config 1's weights; x from its own seed per row count.
        return make_ffn(f"{CONFIG_NAMES[index]}_m{m}", m, 5120, 17408, ACT_SILU, 1.0, 2.0 ** -4,
                        SEED_BASE + 1, x_seed=SEED_BASE + index + 100 * m)
    raise ValueError(f"no config {index}")


def make_small(M: int, K: int, N: int, act: int = ACT_SILU, seed: int = 7, sigma: float = 1.0,
               scale2: float = 2.0 ** -4) -> FfnCase:
    """A small random case of any shape (K, N multiples of 32)."""
    return make_ffn(f"small_m{M}_k{K}_n{N}_{ACT_NAMES[act]}", M, K, N, act, sigma, scale2, seed)


def finite_e4m3_bytes() -> np.ndarray:
    """All 254 E4M3FN byte values except the two NaN encodings (0x7F, 0xFF)."""
    b = np.arange(256, dtype=np.uint16)
    return b[(b & 0x7F) != 0x7F].astype(np.uint8)


def make_format_coverage(act: int = ACT_SILU, seed: int = 99, M: int = 1) -> FfnCase:
    """Every E2M1 code and every finite E4M3 scale byte appear, and scale2 is
    not a power of two. Shape K=512, N=256."""
    K, N = 512, 256
    rng = np.random.Generator(np.random.PCG64(seed))
    fin = finite_e4m3_bytes()

    def weight(rows: int, cols: int, s2: float) -> Nvfp4Weight:
        nbytes = rows * cols // 2
        codes = np.resize(rng.permutation(256).astype(np.uint8), nbytes)
        rng.shuffle(codes)
        nsc = rows * cols // 16
        scales = np.resize(rng.permutation(fin), nsc)
        return Nvfp4Weight(codes=codes.reshape(rows, cols // 2),
                           scales=scales.reshape(rows, cols // 16).astype(np.uint8), scale2=s2)

    gate = weight(N, K, 0.7)
    up = weight(N, K, 1.3)
    down = weight(K, N, 0.3)
    x_bits = _draw_x(rng, M, K, 1.0)
    return FfnCase(name=f"format_coverage_{ACT_NAMES[act]}_m{M}", M=M, K=K, N=N, act=act,
                   x_bits=x_bits, gate=gate, up=up, down=down)


def make_format_coverage_onesign(act: int = ACT_SILU, seed: int = 97, M: int = 1) -> FfnCase:
    """Format coverage without cancellation: W_d holds every E2M1 code and
    every finite E4M3 scale byte (negative, subnormal and 448 included), yet
    every nonzero product in an output's sum has that output's sign, so the
    one bf16 rounding of h cannot be amplified by cancellation. Shape K=512,
    N=256.

    Built from byte structure only: the sign is bit 3 of an E2M1 code and
    bit 7 of an E4M3 byte, and E4M3 magnitudes increase with the low 7 bits.
    x >= 0; row n of W_g and of W_u share one sign s_n (each code's sign bit
    is set so that code sign times scale sign is s_n), so gate and up have
    the same sign and h = act(gate) * up >= 0 (SiLU and GELU-tanh keep the
    sign of their input); their scales are +-2^-2 .. +-1. Row j of W_d has
    one sign t_j the same way, and its 16 scale bytes are consecutive in the
    magnitude-sorted list of all scale bytes, so rows 32 b .. 32 b + 31 hold
    scales within a few binades of each other ("bands" of like magnitude,
    rows of band b smaller than those of band b + 1)."""
    K, N = 512, 256
    rng = np.random.Generator(np.random.PCG64(seed))
    fin = finite_e4m3_bytes()

    def onesign(rows: int, cols: int, scales: np.ndarray, signs: np.ndarray, s2: float) -> Nvfp4Weight:
        mags = rng.integers(0, 8, size=(rows, cols), dtype=np.uint8)
        # element (r, c): its block's scale sign bit, flipped when the row is negative
        neg = ((scales >> 7).astype(np.uint8)[:, np.arange(cols) // 16] ^ (signs[:, None] < 0)).astype(np.uint8)
        nib = mags | (neg << 3)
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        return Nvfp4Weight(codes=codes, scales=scales.astype(np.uint8), scale2=s2)

    sn = rng.choice(np.array([-1, 1], dtype=np.int8), size=N)
    small = lambda rows, cols: (rng.choice(np.array([0x28, 0x30, 0x38], dtype=np.uint8), size=(rows, cols // 16))
                                | (rng.integers(0, 2, size=(rows, cols // 16), dtype=np.uint8) << 7))
    gate = onesign(N, K, small(N, K), sn, 0.02)
    up = onesign(N, K, small(N, K), sn, 0.03)
    nsc = K * N // 16
    sc = np.resize(rng.permutation(fin), nsc)
    sc = sc[np.argsort(sc & 0x7F, kind="stable")].reshape(K, N // 16)
    tj = rng.choice(np.array([-1, 1], dtype=np.int8), size=K)
    down = onesign(K, N, sc, tj, 0.3)
    x = np.abs(rng.standard_normal(size=(M, K), dtype=np.float32))
    return FfnCase(name=f"format_coverage_onesign_{ACT_NAMES[act]}_m{M}", M=M, K=K, N=N, act=act,
                   x_bits=f32_to_bf16_bits(x), gate=gate, up=up, down=down)


@dataclasses.dataclass
class Fp8Weight:
    """One block-scaled FP8 weight of logical shape [rows, cols] (the format
    the qwen35_dense.rs page describes for native FP8 checkpoints):

    * ``codes`` uint8 ``[rows, cols]``: one E4M3FN byte per element, row-major;
    * ``block_scale`` float32 ``[ceil(rows/128), ceil(cols/128)]``: one fp32
      multiplier per 128 x 128 block, row-major.
    """

    codes: np.ndarray        # uint8 [rows, cols]
    block_scale: np.ndarray  # float32 [ceil(rows/128), ceil(cols/128)]

    @property
    def rows(self) -> int:
        return int(self.codes.shape[0])

    @property
    def cols(self) -> int:
        return int(self.codes.shape[1])

    @property
    def nbytes(self) -> int:
        return int(self.codes.nbytes + self.block_scale.nbytes)


@dataclasses.dataclass
class Fp8FfnCase:
    """Inputs of one gated FFN over FP8 weights (same shapes as FfnCase)."""

    name: str
    M: int
    K: int
    N: int
    act: int
    x_bits: np.ndarray  # uint16 [M, K], bf16 bit patterns
    gate: Fp8Weight     # [N, K]
    up: Fp8Weight       # [N, K]
    down: Fp8Weight     # [K, N]

    def with_x(self, x_bits: np.ndarray, name: Optional[str] = None) -> "Fp8FfnCase":
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        return dataclasses.replace(self, x_bits=x_bits, M=int(x_bits.shape[0]),
                                   name=name or self.name)

    @property
    def weight_bytes(self) -> int:
        return self.gate.nbytes + self.up.nbytes + self.down.nbytes


def _draw_fp8_weight(rng: np.random.Generator, rows: int, cols: int, mags: int) -> Fp8Weight:
    """Codes: uniform over the finite E4M3FN bytes whose magnitude field
    (low 7 bits) is below ``mags`` (a random sign, no NaN); block scales: fp32
    uniform on [2**-10, 2**-9), so not powers of two."""
    sign = rng.integers(0, 2, size=(rows, cols), dtype=np.uint8) << 7
    mag = rng.integers(0, mags, size=(rows, cols), dtype=np.uint8)
    codes = (sign | mag).astype(np.uint8)
    grid = ((rows + 127) // 128, (cols + 127) // 128)
    bs = (rng.uniform(1.0, 2.0, size=grid) * 2.0 ** -10).astype(np.float32)
    return Fp8Weight(codes=codes, block_scale=bs)


# Magnitude fields 0..0x77 span +-[0, 240]: every exponent, so every decode
# path, appears, while values stay in the range block-scaled checkpoints use
# (their per-block absmax maps to at most 448 = field 0x7E).
FP8_RECIPE_MAGS = 0x78


def make_fp8_ffn(name: str, M: int, K: int, N: int, act: int = ACT_SILU, sigma: float = 1.0,
                 seed: int = 11, x_seed: Optional[int] = None, mags: int = FP8_RECIPE_MAGS) -> Fp8FfnCase:
    """Draw one FP8 case: gate, up, down codes and block scales in that order,
    then x (from ``x_seed`` when given). Any K, N >= 1 are allowed here; the
    library states its own shape limits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    gate = _draw_fp8_weight(rng, N, K, mags)
    up = _draw_fp8_weight(rng, N, K, mags)
    down = _draw_fp8_weight(rng, K, N, mags)
    if x_seed is not None:
        rng = np.random.Generator(np.random.PCG64(x_seed))
    x_bits = _draw_x(rng, M, K, sigma)
    return Fp8FfnCase(name=name, M=M, K=K, N=N, act=act, x_bits=x_bits, gate=gate, up=up, down=down)


def make_fp8_config(M: int = 1, act: int = ACT_SILU) -> Fp8FfnCase:
    """The decode workload of the dense layer with FP8 weights: K=5120,
    N=17408 (the shape of the NVFP4 decode workload), ``M`` rows."""
    return make_fp8_ffn(f"fp8_decode_{ACT_NAMES[act]}_m{M}", M, 5120, 17408, act, 1.0,
                        SEED_BASE + 50, x_seed=SEED_BASE + 51 + 100 * M)


def make_fp8_format_coverage(act: int = ACT_SILU, seed: int = 98, M: int = 1) -> Fp8FfnCase:
    """Every finite E4M3FN byte (254 of them) appears in every weight, and the
    block grids are ragged (K=384+64, N=256+32). Block scales as in the recipe."""
    K, N = 448, 288
    rng = np.random.Generator(np.random.PCG64(seed))
    fin = finite_e4m3_bytes()

    def weight(rows: int, cols: int) -> Fp8Weight:
        codes = np.resize(rng.permutation(fin), rows * cols)
        rng.shuffle(codes)
        grid = ((rows + 127) // 128, (cols + 127) // 128)
        bs = (rng.uniform(1.0, 2.0, size=grid) * 2.0 ** -10).astype(np.float32)
        return Fp8Weight(codes=codes.reshape(rows, cols).astype(np.uint8), block_scale=bs)

    gate, up, down = weight(N, K), weight(N, K), weight(K, N)
    x_bits = _draw_x(rng, M, K, 1.0)
    return Fp8FfnCase(name=f"fp8_format_coverage_{ACT_NAMES[act]}_m{M}", M=M, K=K, N=N, act=act,
                      x_bits=x_bits, gate=gate, up=up, down=down)


@dataclasses.dataclass
class MxWeight:
    """An MXFP4 weight of logical shape [rows, cols] (the W4A4 arm's operand
    layout): E2M1 codes [rows, cols/2] (element 2j in the low nibble of byte
    j), one E8M0 exponent byte per 32 consecutive elements [rows, cols/32]
    (value 2^(byte - 127)), and the per-tensor fp32 scale2 carried over from
    the NVFP4 weight it was requantised from."""

    codes: np.ndarray   # uint8 [rows, cols // 2]
    e8m0: np.ndarray    # uint8 [rows, cols // 32]
    scale2: float

    @property
    def rows(self) -> int:
        return int(self.codes.shape[0])

    @property
    def cols(self) -> int:
        return int(self.codes.shape[1]) * 2


def make_dense_bf16(rows: int, cols: int, seed: int, spread: float = 4.0) -> np.ndarray:
    """Seeded dense bf16 weight bits [rows, cols] (the quantiser's input): a
    normal draw times a per-row factor e^u, u uniform on [-spread, spread / 2]
    (rows of different magnitude, so block scales spread over the E4M3
    range), rounded to bf16 (nearest, ties to even)."""
    rng = np.random.default_rng(SEED_BASE + 7919 * seed + 11)
    f = rng.standard_normal((rows, cols)).astype(np.float32)
    f *= np.exp(rng.uniform(-spread, spread / 2, size=(rows, 1))).astype(np.float32)
    return f32_to_bf16_bits(f)


def weight_copies(w: Nvfp4Weight, n: int) -> List[Nvfp4Weight]:
    """``n`` byte-identical copies (used to defeat cache reuse in timing)."""
    return [Nvfp4Weight(w.codes.copy(), w.scales.copy(), w.scale2) for _ in range(n)]
