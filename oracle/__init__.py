"""CPU oracle for the NVFP4 W4A16 gated FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never calls it, and it
shares no code with the GPU library.

The arithmetic lives in ``ffn_oracle.c`` (plain C, double precision, sums in
ascending index order); this module only compiles it with gcc and marshals
numpy arrays into it. Every function here takes an ``ffn_inputs.FfnCase`` or
plain numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ffn_oracle.c")
LIB_PATH = os.path.join(_HERE, "libffn_oracle.so")


def build(force: bool = True, src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP over outputs)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-ffp-contract=off",
               src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """ctypes view of one compiled copy of ffn_oracle.c."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            build(force=False, out=lib_path)
        lib = ctypes.CDLL(lib_path)
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e2m1_value.argtypes = [_I]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [_I]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_act.restype = ctypes.c_double
        lib.oracle_act.argtypes = [_I, ctypes.c_double]
        lib.oracle_dequant.restype = None
        lib.oracle_dequant.argtypes = [_P, _P, _F, _I, _I, _P]
        lib.oracle_linear_f64.restype = None
        lib.oracle_linear_f64.argtypes = [_P, _I, _I, _I, _P, _P, _F, _P]
        lib.oracle_dual.restype = _I
        lib.oracle_dual.argtypes = [_P, _I, _I, _I, _P, _P, _F, _P, _P, _F, _P, _P]
        lib.oracle_gated_act.restype = None
        lib.oracle_gated_act.argtypes = [_I, _P, _P, ctypes.c_size_t, _P]
        lib.oracle_down.restype = None
        lib.oracle_down.argtypes = [_P, _I, _I, _I, _P, _P, _F, _P]
        lib.oracle_ffn.restype = _I
        lib.oracle_ffn.argtypes = [_P, _I, _I, _I, _I, _P, _P, _F, _P, _P, _F, _P, _P, _F, _P]
        lib.oracle_num_threads.restype = _I
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [_I]
        lib.oracle_e2m1_encode.restype = _I
        lib.oracle_e2m1_encode.argtypes = [_F]
        lib.oracle_e4m3_encode.restype = _I
        lib.oracle_e4m3_encode.argtypes = [_F]
        lib.oracle_quantize.restype = None
        lib.oracle_quantize.argtypes = [_P, _I, _I, _P, _P, _P]
        lib.oracle_fp8_dequant.restype = None
        lib.oracle_fp8_dequant.argtypes = [_P, _P, _I, _I, _P]
        lib.oracle_fp8_linear_f64.restype = None
        lib.oracle_fp8_linear_f64.argtypes = [_P, _I, _I, _I, _P, _P, _P]
        lib.oracle_fp8_dual.restype = _I
        lib.oracle_fp8_dual.argtypes = [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P]
        lib.oracle_fp8_ffn.restype = _I
        lib.oracle_fp8_ffn.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
        lib.oracle_mx_value.restype = ctypes.c_double
        lib.oracle_mx_value.argtypes = [_I, _I]
        lib.oracle_mx_block_exponent.restype = _I
        lib.oracle_mx_block_exponent.argtypes = [ctypes.c_double]
        lib.oracle_mx_quantize.restype = None
        lib.oracle_mx_quantize.argtypes = [_P, _I, _I, _P, _P]
        lib.oracle_mx_quantize_bf16.restype = _I
        lib.oracle_mx_quantize_bf16.argtypes = [_P, _I, _I, _P, _P]
        lib.oracle_mx_requant_nvfp4.restype = _I
        lib.oracle_mx_requant_nvfp4.argtypes = [_P, _P, _I, _I, _P, _P]
        lib.oracle_mx_linear_f64.restype = None
        lib.oracle_mx_linear_f64.argtypes = [_P, _P, _I, _I, _P, _P, _I, _P]
        lib.oracle_w4a4_dual.restype = _I
        lib.oracle_w4a4_dual.argtypes = [_P, _I, _I, _I, _P, _P, ctypes.c_float, _P, _P, ctypes.c_float, _P, _P]
        lib.oracle_w4a4_ffn.restype = _I
        lib.oracle_w4a4_ffn.argtypes = [_P, _I, _I, _I, _I, _P, _P, ctypes.c_float, _P, _P, ctypes.c_float,
                                        _P, _P, ctypes.c_float, _P]
        lib.oracle_bf16_round_bits.restype = ctypes.c_uint16
        lib.oracle_bf16_round_bits.argtypes = [ctypes.c_double]
        lib.oracle_w4a4_down.restype = _I
        lib.oracle_w4a4_down.argtypes = [_P, _I, _I, _I, _P, _P, ctypes.c_float, _P]
        lib.oracle_w4a4_ffn_fp4.restype = _I
        lib.oracle_w4a4_ffn_fp4.argtypes = [_P, _I, _I, _I, _I, _P, _P, ctypes.c_float, _P, _P, ctypes.c_float,
                                            _P, _P, ctypes.c_float, _P]
        self.lib = lib
        self.path = lib_path

    def e2m1_value(self, code: int) -> float:
        return self.lib.oracle_e2m1_value(int(code))

    def e4m3_value(self, byte: int) -> float:
        return self.lib.oracle_e4m3_value(int(byte))

    def bf16_value(self, bits: int) -> float:
        return self.lib.oracle_bf16_value(int(bits))

    def act(self, kind: int, g: float) -> float:
        return self.lib.oracle_act(int(kind), float(g))

    def e2m1_table(self) -> np.ndarray:
        return np.array([self.e2m1_value(i) for i in range(16)], dtype=np.float64)

    def e4m3_table(self) -> np.ndarray:
        return np.array([self.e4m3_value(i) for i in range(256)], dtype=np.float64)

    def dequant(self, w) -> np.ndarray:
        """Dequantised weight [rows, cols] in double."""
        codes = _c(w.codes, np.uint8)
        scales = _c(w.scales, np.uint8)
        rows, cols = codes.shape[0], codes.shape[1] * 2
        out = np.empty((rows, cols), dtype=np.float64)
        self.lib.oracle_dequant(_ptr(codes), _ptr(scales), float(w.scale2), rows, cols, _ptr(out))
        return out

    def linear(self, a: np.ndarray, w) -> np.ndarray:
        """y[m, r] = sum_c W[r, c] a[m, c] with a in double."""
        a = _c(a, np.float64)
        codes = _c(w.codes, np.uint8)
        scales = _c(w.scales, np.uint8)
        M, cols = a.shape
        rows = codes.shape[0]
        assert codes.shape[1] * 2 == cols
        y = np.empty((M, rows), dtype=np.float64)
        self.lib.oracle_linear_f64(_ptr(a), M, cols, rows, _ptr(codes), _ptr(scales),
                                   float(w.scale2), _ptr(y))
        return y

    def dual(self, case) -> Tuple[np.ndarray, np.ndarray]:
        """(gate, up), each [M, N] in double."""
        x = _c(case.x_bits, np.uint16)
        g, u = case.gate, case.up
        gate = np.empty((case.M, case.N), dtype=np.float64)
        up = np.empty((case.M, case.N), dtype=np.float64)
        gc, gs, uc, us = (_c(a, np.uint8) for a in (g.codes, g.scales, u.codes, u.scales))
        rc = self.lib.oracle_dual(_ptr(x), case.M, case.K, case.N,
                                  _ptr(gc), _ptr(gs), float(g.scale2),
                                  _ptr(uc), _ptr(us), float(u.scale2), _ptr(gate), _ptr(up))
        if rc != 0:
            raise MemoryError("oracle_dual")
        return gate, up

    def gated_act(self, kind: int, gate: np.ndarray, up: np.ndarray) -> np.ndarray:
        gate = _c(gate, np.float64)
        up = _c(up, np.float64)
        h = np.empty_like(gate)
        self.lib.oracle_gated_act(int(kind), _ptr(gate), _ptr(up), gate.size, _ptr(h))
        return h

    def down(self, h: np.ndarray, w) -> np.ndarray:
        """out[m, j] = sum_n W_d[j, n] h[m, n]."""
        h = _c(h, np.float64)
        codes = _c(w.codes, np.uint8)
        scales = _c(w.scales, np.uint8)
        M, N = h.shape
        K = codes.shape[0]
        out = np.empty((M, K), dtype=np.float64)
        self.lib.oracle_down(_ptr(h), M, N, K, _ptr(codes), _ptr(scales), float(w.scale2), _ptr(out))
        return out

    def ffn(self, case, rows: Optional[np.ndarray] = None) -> np.ndarray:
        """out [M, K] in double; with ``rows`` only those rows of x are
        computed (rows of the FFN are independent): [len(rows), K]."""
        x = _c(case.x_bits if rows is None else case.x_bits[np.asarray(rows)], np.uint16)
        M = x.shape[0]
        g, u, d = case.gate, case.up, case.down
        arrs = [_c(a, np.uint8) for a in (g.codes, g.scales, u.codes, u.scales, d.codes, d.scales)]
        out = np.empty((M, case.K), dtype=np.float64)
        rc = self.lib.oracle_ffn(_ptr(x), M, case.K, case.N, int(case.act),
                                 _ptr(arrs[0]), _ptr(arrs[1]), float(g.scale2),
                                 _ptr(arrs[2]), _ptr(arrs[3]), float(u.scale2),
                                 _ptr(arrs[4]), _ptr(arrs[5]), float(d.scale2), _ptr(out))
        if rc != 0:
            raise MemoryError("oracle_ffn")
        return out

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        """Threads of later calls (results do not depend on it)."""
        self.lib.oracle_set_num_threads(int(n))

    def e2m1_encode(self, q: float) -> int:
        return self.lib.oracle_e2m1_encode(float(q))

    def e4m3_encode(self, s: float) -> int:
        return self.lib.oracle_e4m3_encode(float(s))

    def quantize(self, w_bits: np.ndarray):
        """BF16 weight bits [rows, cols] -> (codes [rows, cols/2], scales
        [rows, cols/16], scale2 as an fp32 value)."""
        w = _c(w_bits, np.uint16)
        rows, cols = w.shape
        assert cols % 16 == 0
        codes = np.empty((rows, cols // 2), dtype=np.uint8)
        scales = np.empty((rows, cols // 16), dtype=np.uint8)
        s2 = np.zeros(1, dtype=np.float32)
        self.lib.oracle_quantize(_ptr(w), rows, cols, _ptr(codes), _ptr(scales), _ptr(s2))
        return codes, scales, float(s2[0])


    # ------------------------------------------------------------ FP8
    # An ffn_inputs.Fp8Weight: E4M3 bytes [rows, cols] and an fp32 block-scale
    # grid [ceil(rows/128), ceil(cols/128)].

    def fp8_dequant(self, w) -> np.ndarray:
        codes = _c(w.codes, np.uint8)
        bs = _c(w.block_scale, np.float32)
        rows, cols = codes.shape
        out = np.empty((rows, cols), dtype=np.float64)
        self.lib.oracle_fp8_dequant(_ptr(codes), _ptr(bs), rows, cols, _ptr(out))
        return out

    def fp8_linear(self, a: np.ndarray, w) -> np.ndarray:
        a = _c(a, np.float64)
        codes = _c(w.codes, np.uint8)
        bs = _c(w.block_scale, np.float32)
        M, cols = a.shape
        rows = codes.shape[0]
        assert codes.shape[1] == cols
        y = np.empty((M, rows), dtype=np.float64)
        self.lib.oracle_fp8_linear_f64(_ptr(a), M, cols, rows, _ptr(codes), _ptr(bs), _ptr(y))
        return y

    def fp8_dual(self, case) -> Tuple[np.ndarray, np.ndarray]:
        x = _c(case.x_bits, np.uint16)
        g, u = case.gate, case.up
        gate = np.empty((case.M, case.N), dtype=np.float64)
        up = np.empty((case.M, case.N), dtype=np.float64)
        gw, uw = _c(g.codes, np.uint8), _c(u.codes, np.uint8)
        gb, ub = _c(g.block_scale, np.float32), _c(u.block_scale, np.float32)
        rc = self.lib.oracle_fp8_dual(_ptr(x), case.M, case.K, case.N, _ptr(gw), _ptr(gb), _ptr(uw), _ptr(ub),
                                      _ptr(gate), _ptr(up))
        if rc != 0:
            raise MemoryError("oracle_fp8_dual")
        return gate, up

    def fp8_ffn(self, case, rows: Optional[np.ndarray] = None) -> np.ndarray:
        x = _c(case.x_bits if rows is None else case.x_bits[np.asarray(rows)], np.uint16)
        M = x.shape[0]
        g, u, d = case.gate, case.up, case.down
        ws = [_c(t.codes, np.uint8) for t in (g, u, d)]
        bs = [_c(t.block_scale, np.float32) for t in (g, u, d)]
        out = np.empty((M, case.K), dtype=np.float64)
        rc = self.lib.oracle_fp8_ffn(_ptr(x), M, case.K, case.N, int(case.act), _ptr(ws[0]), _ptr(bs[0]),
                                     _ptr(ws[1]), _ptr(bs[1]), _ptr(ws[2]), _ptr(bs[2]), _ptr(out))
        if rc != 0:
            raise MemoryError("oracle_fp8_ffn")
        return out


    # ------------------------------------------------------------ W4A4 (MXFP4)

    def mx_value(self, code: int, e8m0: int) -> float:
        return float(self.lib.oracle_mx_value(int(code), int(e8m0)))

    def mx_block_exponent(self, amax: float) -> int:
        return int(self.lib.oracle_mx_block_exponent(float(amax)))

    def mx_quantize(self, v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """float64 [rows, cols] -> (codes uint8 [rows, cols/2], e8m0 uint8 [rows, cols/32])."""
        v = _c(v, np.float64)
        rows, cols = v.shape
        codes = np.zeros((rows, cols // 2), dtype=np.uint8)
        e8m0 = np.zeros((rows, cols // 32), dtype=np.uint8)
        self.lib.oracle_mx_quantize(_ptr(v), rows, cols, _ptr(codes), _ptr(e8m0))
        return codes, e8m0

    def mx_quantize_bf16(self, x_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        x = _c(x_bits, np.uint16)
        M, K = x.shape
        codes = np.zeros((M, K // 2), dtype=np.uint8)
        e8m0 = np.zeros((M, K // 32), dtype=np.uint8)
        if self.lib.oracle_mx_quantize_bf16(_ptr(x), M, K, _ptr(codes), _ptr(e8m0)) != 0:
            raise MemoryError("oracle_mx_quantize_bf16")
        return codes, e8m0

    def mx_requant(self, w):
        """An NVFP4 weight (ffn_inputs.Nvfp4Weight) requantised to MXFP4
        (ffn_inputs.MxWeight, scale2 carried over)."""
        import ffn_inputs
        codes = _c(w.codes, np.uint8)
        scales = _c(w.scales, np.uint8)
        rows, cols = w.rows, w.cols
        mc = np.zeros((rows, cols // 2), dtype=np.uint8)
        me = np.zeros((rows, cols // 32), dtype=np.uint8)
        if self.lib.oracle_mx_requant_nvfp4(_ptr(codes), _ptr(scales), rows, cols, _ptr(mc), _ptr(me)) != 0:
            raise MemoryError("oracle_mx_requant_nvfp4")
        return ffn_inputs.MxWeight(mc, me, float(w.scale2))

    def mx_linear(self, a_codes, a_e8m0, w_codes, w_e8m0) -> np.ndarray:
        ac, ae, wc, we = (_c(t, np.uint8) for t in (a_codes, a_e8m0, w_codes, w_e8m0))
        M, cols = ac.shape[0], ac.shape[1] * 2
        rows = wc.shape[0]
        y = np.empty((M, rows), dtype=np.float64)
        self.lib.oracle_mx_linear_f64(_ptr(ac), _ptr(ae), M, cols, _ptr(wc), _ptr(we), rows, _ptr(y))
        return y

    def w4a4_dual(self, case, gate_mx, up_mx) -> Tuple[np.ndarray, np.ndarray]:
        x = _c(case.x_bits, np.uint16)
        M = x.shape[0]
        gate = np.empty((M, case.N), dtype=np.float64)
        up = np.empty((M, case.N), dtype=np.float64)
        gc, ge, uc, ue = (_c(t, np.uint8) for t in (gate_mx.codes, gate_mx.e8m0, up_mx.codes, up_mx.e8m0))
        rc = self.lib.oracle_w4a4_dual(_ptr(x), M, case.K, case.N, _ptr(gc), _ptr(ge), float(gate_mx.scale2),
                                       _ptr(uc), _ptr(ue), float(up_mx.scale2), _ptr(gate), _ptr(up))
        if rc != 0:
            raise MemoryError("oracle_w4a4_dual")
        return gate, up

    def w4a4_ffn(self, case, gate_mx, up_mx, rows: Optional[np.ndarray] = None) -> np.ndarray:
        x = _c(case.x_bits if rows is None else case.x_bits[np.asarray(rows)], np.uint16)
        M = x.shape[0]
        gc, ge, uc, ue = (_c(t, np.uint8) for t in (gate_mx.codes, gate_mx.e8m0, up_mx.codes, up_mx.e8m0))
        dc, ds = _c(case.down.codes, np.uint8), _c(case.down.scales, np.uint8)
        out = np.empty((M, case.K), dtype=np.float64)
        rc = self.lib.oracle_w4a4_ffn(_ptr(x), M, case.K, case.N, int(case.act), _ptr(gc), _ptr(ge),
                                      float(gate_mx.scale2), _ptr(uc), _ptr(ue), float(up_mx.scale2), _ptr(dc),
                                      _ptr(ds), float(case.down.scale2), _ptr(out))
        if rc != 0:
            raise MemoryError("oracle_w4a4_ffn")
        return out


    def bf16_round_bits(self, v: float) -> int:
        return int(self.lib.oracle_bf16_round_bits(float(v)))

    def w4a4_down(self, h_bits: np.ndarray, down_mx) -> np.ndarray:
        """scale2_d * (mx(h) . mx(W_d)) for bf16 h [M, N] (bit patterns) and an
        MXFP4 down weight [K, N]."""
        h = _c(h_bits, np.uint16)
        M, N = h.shape
        dc, de = _c(down_mx.codes, np.uint8), _c(down_mx.e8m0, np.uint8)
        K = dc.shape[0]
        out = np.empty((M, K), dtype=np.float64)
        rc = self.lib.oracle_w4a4_down(_ptr(h), M, N, K, _ptr(dc), _ptr(de), float(down_mx.scale2), _ptr(out))
        if rc != 0:
            raise MemoryError("oracle_w4a4_down")
        return out

    def w4a4_ffn_fp4(self, case, gate_mx, up_mx, down_mx, rows: Optional[np.ndarray] = None) -> np.ndarray:
        x = _c(case.x_bits if rows is None else case.x_bits[np.asarray(rows)], np.uint16)
        M = x.shape[0]
        gc, ge, uc, ue, dc, de = (_c(t, np.uint8) for t in (gate_mx.codes, gate_mx.e8m0, up_mx.codes, up_mx.e8m0,
                                                             down_mx.codes, down_mx.e8m0))
        out = np.empty((M, case.K), dtype=np.float64)
        rc = self.lib.oracle_w4a4_ffn_fp4(_ptr(x), M, case.K, case.N, int(case.act), _ptr(gc), _ptr(ge),
                                          float(gate_mx.scale2), _ptr(uc), _ptr(ue), float(up_mx.scale2), _ptr(dc),
                                          _ptr(de), float(down_mx.scale2), _ptr(out))
        if rc != 0:
            raise MemoryError("oracle_w4a4_ffn_fp4")
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(LIB_PATH)
    return _default


def e2m1_table() -> np.ndarray:
    return default().e2m1_table()


def e4m3_table() -> np.ndarray:
    return default().e4m3_table()


def dequant(w) -> np.ndarray:
    return default().dequant(w)


def linear(a: np.ndarray, w) -> np.ndarray:
    return default().linear(a, w)


def dual(case):
    return default().dual(case)


def gated_act(kind: int, gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    return default().gated_act(kind, gate, up)


def down(h: np.ndarray, w) -> np.ndarray:
    return default().down(h, w)


def ffn(case, rows=None) -> np.ndarray:
    return default().ffn(case, rows)


def num_threads() -> int:
    return default().num_threads()


def e2m1_encode(q: float) -> int:
    return default().e2m1_encode(q)


def e4m3_encode(s: float) -> int:
    return default().e4m3_encode(s)


def quantize(w_bits: np.ndarray):
    return default().quantize(w_bits)


def fp8_dequant(w) -> np.ndarray:
    return default().fp8_dequant(w)


def fp8_linear(a: np.ndarray, w) -> np.ndarray:
    return default().fp8_linear(a, w)


def fp8_dual(case):
    return default().fp8_dual(case)


def fp8_ffn(case, rows=None) -> np.ndarray:
    return default().fp8_ffn(case, rows)


def mx_quantize_bf16(x_bits):
    return default().mx_quantize_bf16(x_bits)


def mx_requant(w):
    return default().mx_requant(w)


def w4a4_dual(case, gate_mx, up_mx):
    return default().w4a4_dual(case, gate_mx, up_mx)


def w4a4_ffn(case, gate_mx, up_mx, rows=None) -> np.ndarray:
    return default().w4a4_ffn(case, gate_mx, up_mx, rows)


def w4a4_down(h_bits, down_mx) -> np.ndarray:
    return default().w4a4_down(h_bits, down_mx)


def w4a4_ffn_fp4(case, gate_mx, up_mx, down_mx, rows=None) -> np.ndarray:
    return default().w4a4_ffn_fp4(case, gate_mx, up_mx, down_mx, rows)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v|: 2^(floor(log2|v|) - 7), floored at the
    smallest bf16 subnormal 2^-133."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    u = np.ldexp(1.0, (e - 7).astype(np.int64))
    u = np.where(a > 0, u, 0.0)
    return np.maximum(u, 2.0 ** -133)


def parity_bound(out_ref: np.ndarray, rms_ref: Optional[float] = None,
                 rel: float = 1e-2) -> np.ndarray:
    """Per-element bound for a bf16 GPU output against the double reference:
    rel * rms(out_ref) + one bf16 ulp of the reference value."""
    if rms_ref is None:
        rms_ref = float(np.sqrt(np.mean(np.square(out_ref))))
    return rel * rms_ref + ulp_bf16(out_ref)


def fp8_h_rounding_bound(case) -> np.ndarray:
    """h_rounding_bound for an FP8 case: 2^-8 * sum_n |W_d[j, n]| |h[m, n]|."""
    g, u = default().fp8_dual(case)
    h = default().gated_act(case.act, g, u)
    wd = np.abs(default().fp8_dequant(case.down))
    return (2.0 ** -8) * (np.abs(h) @ wd.T)


def h_rounding_bound(case) -> np.ndarray:
    """First-order bound [M, K] of what rounding h = act(gate) * up to bf16
    (once, to nearest) can move out = W_d h: 2^-8 * sum_n |W_d[j, n]| |h[m, n]|
    (bf16 keeps 8 significant bits, so one rounding is off by at most 2^-8 of
    the value). It only matters for weights with extreme dynamic range, where
    out is a small difference of large terms."""
    g, u = default().dual(case)
    h = default().gated_act(case.act, g, u)
    wd = np.abs(default().dequant(case.down))
    return (2.0 ** -8) * (np.abs(h) @ wd.T)
