"""Python binding of libffn_nvfp4 (MI355X / gfx950 NVFP4 W4A16 gated FFN).

Argument marshalling only: every step of the FFN runs in the HIP kernels of
``lib/libffn_nvfp4.so`` through its C ABI (``include/ffn_nvfp4.h``). PyTorch
is used for device memory and streams. There is no fallback: if the library
is missing or a call fails, an exception is raised.

The functions mirror the C entry points:

* :func:`forward`    -- ``ffn_nvfp4_forward``   out = W_d (act(W_g x) * (W_u x))
* :func:`forward_noalloc` -- ``ffn_nvfp4_forward_noalloc`` the same with the
  library's static scratch instead of a workspace (allocates nothing)
* :func:`dual_gemv`  -- ``ffn_nvfp4_dual_gemv`` gate, up = W_g x, W_u x (fp32)
* :func:`down_gemv`  -- ``ffn_nvfp4_down_gemv`` out = W_d bf16(act(gate) * up)
* :func:`workspace_bytes` -- ``ffn_nvfp4_workspace_bytes``
* :func:`quantize`   -- ``ffn_nvfp4_quantize``  bf16 weight -> NVFP4 codes, scales, scale2
* :func:`quantize_workspace_bytes` -- ``ffn_nvfp4_quantize_workspace_bytes``

and, for block-scaled FP8 weights (``include/ffn_fp8.h``):

* :func:`fp8_forward`    -- ``ffn_fp8_forward``
* :func:`fp8_dual_gemv`  -- ``ffn_fp8_dual_gemv``
* :func:`fp8_down_gemv`  -- ``ffn_fp8_down_gemv``
* :func:`fp8_workspace_bytes` -- ``ffn_fp8_workspace_bytes``

the streaming-read ceiling the decode GEMVs are measured against
(``include/ffn_diag.h``):

* :func:`diag_read` -- ``ffn_diag_read`` one launch reading device buffers once

and the W4A4 prefill arm over MXFP4 operands (``include/ffn_w4a4.h``):

* :func:`w4a4_prepare_weight` -- ``ffn_w4a4_prepare_weight`` NVFP4 -> MXFP4 (once)
* :func:`w4a4_dual_gemm`  -- ``ffn_w4a4_dual_gemm``
* :func:`w4a4_forward`    -- ``ffn_w4a4_forward``
* :func:`w4a4_workspace_bytes` -- ``ffn_w4a4_workspace_bytes``
* :func:`w4a4_down_gemm`  -- ``ffn_w4a4_down_gemm`` (the down projection on 4 bits)
* :func:`w4a4_forward_fp4` -- ``ffn_w4a4_forward_fp4`` (all three projections on 4 bits)
* :func:`w4a4_fp4_workspace_bytes` -- ``ffn_w4a4_fp4_workspace_bytes``
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "lib", "libffn_nvfp4.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "ffn_nvfp4.h")
FP8_HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "ffn_fp8.h")
W4A4_HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "ffn_w4a4.h")
DIAG_HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "ffn_diag.h")

ACT_SILU = 0
ACT_GELU_TANH = 1

OK = 0
ERR_NULL = -1
ERR_ALIGN = -2
ERR_SHAPE = -3
ERR_BATCH = -4
ERR_ACT = -5
ERR_WORKSPACE = -6
ERR_LAUNCH = -7
ERR_SCALE2 = -8


class FfnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({strerror(status)})")


class WeightStruct(ctypes.Structure):
    """ffn_nvfp4_weight: device codes, device scales, host fp32 scale2."""

    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("scale2", ctypes.c_float)]


class Fp8WeightStruct(ctypes.Structure):
    """ffn_fp8_weight: device codes, device fp32 block-scale grid."""

    _fields_ = [("codes", ctypes.c_void_p), ("block_scale", ctypes.c_void_p)]


class MxWeightStruct(ctypes.Structure):
    """ffn_mxfp4_weight: device codes, device E8M0 bytes, host fp32 scale2."""

    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("scale2", ctypes.c_float)]


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_WP = ctypes.POINTER(WeightStruct)
_FP = ctypes.POINTER(Fp8WeightStruct)
_MP = ctypes.POINTER(MxWeightStruct)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m w4a16_nvfp4_dense_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    lib.ffn_nvfp4_version.restype = _I
    lib.ffn_nvfp4_version.argtypes = []
    lib.ffn_nvfp4_strerror.restype = ctypes.c_char_p
    lib.ffn_nvfp4_strerror.argtypes = [_I]
    lib.ffn_nvfp4_workspace_bytes.restype = ctypes.c_size_t
    lib.ffn_nvfp4_workspace_bytes.argtypes = [_I, _I, _I]
    lib.ffn_nvfp4_forward.restype = _I
    lib.ffn_nvfp4_forward.argtypes = [_P, _I, _I, _I, _WP, _WP, _WP, _I, _P, ctypes.c_size_t, _P, _P]
    lib.ffn_nvfp4_forward_noalloc.restype = _I
    lib.ffn_nvfp4_forward_noalloc.argtypes = [_P, _I, _I, _I, _WP, _WP, _WP, _I, _P, _P]
    lib.ffn_nvfp4_dual_gemv.restype = _I
    lib.ffn_nvfp4_dual_gemv.argtypes = [_P, _I, _I, _I, _WP, _WP, _P, _P, _P]
    lib.ffn_nvfp4_down_gemv.restype = _I
    lib.ffn_nvfp4_down_gemv.argtypes = [_P, _P, _I, _I, _I, _WP, _I, _P, _P]
    lib.ffn_nvfp4_quantize_workspace_bytes.restype = ctypes.c_size_t
    lib.ffn_nvfp4_quantize_workspace_bytes.argtypes = [_I, _I]
    lib.ffn_nvfp4_quantize.restype = _I
    lib.ffn_nvfp4_quantize.argtypes = [_P, _I, _I, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.ffn_fp8_workspace_bytes.restype = ctypes.c_size_t
    lib.ffn_fp8_workspace_bytes.argtypes = [_I, _I, _I]
    lib.ffn_fp8_forward.restype = _I
    lib.ffn_fp8_forward.argtypes = [_P, _I, _I, _I, _FP, _FP, _FP, _I, _P, ctypes.c_size_t, _P, _P]
    lib.ffn_fp8_dual_gemv.restype = _I
    lib.ffn_fp8_dual_gemv.argtypes = [_P, _I, _I, _I, _FP, _FP, _P, _P, _P]
    lib.ffn_fp8_down_gemv.restype = _I
    lib.ffn_fp8_down_gemv.argtypes = [_P, _P, _I, _I, _I, _FP, _I, _P, _P]
    lib.ffn_w4a4_prepare_weight.restype = _I
    lib.ffn_w4a4_prepare_weight.argtypes = [_WP, _I, _I, _P, _P, _P]
    lib.ffn_w4a4_workspace_bytes.restype = ctypes.c_size_t
    lib.ffn_w4a4_workspace_bytes.argtypes = [_I, _I, _I]
    lib.ffn_w4a4_dual_gemm.restype = _I
    lib.ffn_w4a4_dual_gemm.argtypes = [_P, _I, _I, _I, _MP, _MP, _P, _P, _P, ctypes.c_size_t, _P]
    lib.ffn_diag_read.restype = _I
    lib.ffn_diag_read.argtypes = [ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_size_t), _I, _P, _P]
    lib.ffn_w4a4_forward.restype = _I
    lib.ffn_w4a4_forward.argtypes = [_P, _I, _I, _I, _MP, _MP, _WP, _I, _P, ctypes.c_size_t, _P, _P]
    lib.ffn_w4a4_fp4_workspace_bytes.restype = ctypes.c_size_t
    lib.ffn_w4a4_fp4_workspace_bytes.argtypes = [_I, _I, _I]
    lib.ffn_w4a4_down_gemm.restype = _I
    lib.ffn_w4a4_down_gemm.argtypes = [_P, _I, _I, _I, _MP, _P, _P, ctypes.c_size_t, _P]
    lib.ffn_w4a4_forward_fp4.restype = _I
    lib.ffn_w4a4_forward_fp4.argtypes = [_P, _I, _I, _I, _MP, _MP, _MP, _I, _P, ctypes.c_size_t, _P, _P]
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> Sequence[str]:
    """Names of the functions a public header declares."""
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ffn_(?:nvfp4|fp8|w4a4|diag)_[a-z_0-9]+)\s*\(", text)))


def version() -> int:
    return load().ffn_nvfp4_version()


def strerror(status: int) -> str:
    return load().ffn_nvfp4_strerror(int(status)).decode()


def workspace_bytes(M: int, K: int, N: int) -> int:
    return int(load().ffn_nvfp4_workspace_bytes(int(M), int(K), int(N)))


# ------------------------------------------------------------ torch marshalling


@dataclasses.dataclass
class DeviceWeight:
    """An NVFP4 weight resident on the GPU: codes uint8 [rows, cols/2],
    scales uint8 [rows, cols/16] (both torch tensors on the device) and the
    per-tensor scale2 (host float)."""

    codes: "object"
    scales: "object"
    scale2: float

    @property
    def rows(self) -> int:
        return int(self.codes.shape[0])

    @property
    def cols(self) -> int:
        return int(self.codes.shape[1]) * 2

    def struct(self) -> WeightStruct:
        return WeightStruct(self.codes.data_ptr(), self.scales.data_ptr(), float(self.scale2))

    @classmethod
    def from_host(cls, w, device="cuda") -> "DeviceWeight":
        """From an object with numpy ``codes``, ``scales`` and ``scale2``."""
        import torch
        return cls(torch.from_numpy(w.codes).to(device), torch.from_numpy(w.scales).to(device),
                   float(w.scale2))


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _record(stream, *tensors) -> None:
    """Tensors allocated inside a binding belong to the current stream's
    pool; when the call was enqueued on another stream, mark them as used
    there so the caching allocator cannot hand their memory out again before
    that stream's kernels are done."""
    import torch
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if int(s.cuda_stream) == int(torch.cuda.current_stream().cuda_stream):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def _check_tensor(t, dtype, shape, name, device=None):
    import torch
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(status: int, what: str) -> None:
    if status != OK:
        raise FfnError(status, what)


def _check_nvfp4_weight(w: "DeviceWeight", rows: int, cols: int, name: str, device) -> None:
    """An NVFP4 weight of logical shape [rows, cols]: contiguous uint8 codes
    [rows, cols/2] and scales [rows, cols/16] on the device of the call (the C
    ABI sees only pointers, so a mismatched weight would be read out of
    bounds)."""
    import torch
    if cols % 16:
        raise ValueError(f"{name}: {cols} columns is not a multiple of 16")
    _check_tensor(w.codes, torch.uint8, (rows, cols // 2), f"{name}.codes", device)
    _check_tensor(w.scales, torch.uint8, (rows, cols // 16), f"{name}.scales", device)


def forward(x, gate: DeviceWeight, up: DeviceWeight, down: DeviceWeight, act: int = ACT_SILU,
            out=None, workspace=None, stream=None):
    """out[M, K] (bf16) = W_d (act(W_g x) * (W_u x)) for x bf16 [M, K]."""
    import torch
    M, K = x.shape
    N = gate.rows
    _check_tensor(x, torch.bfloat16, (M, K), "x")
    _check_nvfp4_weight(gate, N, K, "gate", x.device)
    _check_nvfp4_weight(up, N, K, "up", x.device)
    _check_nvfp4_weight(down, K, N, "down", x.device)
    new_out = out is None
    if new_out:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    _check_tensor(out, torch.bfloat16, (M, K), "out", x.device)
    need = workspace_bytes(M, K, N)
    new_ws = workspace is None
    if new_ws:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    g, u, d = gate.struct(), up.struct(), down.struct()
    rc = load().ffn_nvfp4_forward(x.data_ptr(), M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                  int(act), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  out.data_ptr(), _stream_handle(stream))
    _check(rc, "ffn_nvfp4_forward")
    _record(stream, out if new_out else None, workspace if new_ws else None)
    return out


def forward_noalloc(x, gate: DeviceWeight, up: DeviceWeight, down: DeviceWeight, out, act: int = ACT_SILU,
                    stream=None):
    """:func:`forward` through ``ffn_nvfp4_forward_noalloc``: the caller
    passes ``out`` (bf16 [M, K]); no device memory is allocated, by the
    library or here."""
    import torch
    M, K = x.shape
    N = gate.rows
    _check_tensor(x, torch.bfloat16, (M, K), "x")
    _check_nvfp4_weight(gate, N, K, "gate", x.device)
    _check_nvfp4_weight(up, N, K, "up", x.device)
    _check_nvfp4_weight(down, K, N, "down", x.device)
    _check_tensor(out, torch.bfloat16, (M, K), "out", x.device)
    g, u, d = gate.struct(), up.struct(), down.struct()
    rc = load().ffn_nvfp4_forward_noalloc(x.data_ptr(), M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                          int(act), out.data_ptr(), _stream_handle(stream))
    _check(rc, "ffn_nvfp4_forward_noalloc")
    return out


def dual_gemv(x, gate: DeviceWeight, up: DeviceWeight, gate_out=None, up_out=None, stream=None):
    """(gate, up) fp32 [M, N] = (scale2_g W_g x, scale2_u W_u x)."""
    import torch
    M, K = x.shape
    N = gate.rows
    _check_tensor(x, torch.bfloat16, (M, K), "x")
    _check_nvfp4_weight(gate, N, K, "gate", x.device)
    _check_nvfp4_weight(up, N, K, "up", x.device)
    new_g, new_u = gate_out is None, up_out is None
    if new_g:
        gate_out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if new_u:
        up_out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check_tensor(gate_out, torch.float32, (M, N), "gate_out", x.device)
    _check_tensor(up_out, torch.float32, (M, N), "up_out", x.device)
    g, u = gate.struct(), up.struct()
    rc = load().ffn_nvfp4_dual_gemv(x.data_ptr(), M, K, N, ctypes.byref(g), ctypes.byref(u),
                                    gate_out.data_ptr(), up_out.data_ptr(), _stream_handle(stream))
    _check(rc, "ffn_nvfp4_dual_gemv")
    _record(stream, gate_out if new_g else None, up_out if new_u else None)
    return gate_out, up_out


def down_gemv(gate_in, up_in, down: DeviceWeight, act: int = ACT_SILU, out=None, stream=None):
    """out[M, K] (bf16) = W_d bf16(act(gate) * up) with the activation fused
    into the down GEMV's input load."""
    import torch
    M, N = gate_in.shape
    K = down.rows
    _check_tensor(gate_in, torch.float32, (M, N), "gate_in")
    _check_tensor(up_in, torch.float32, (M, N), "up_in", gate_in.device)
    _check_nvfp4_weight(down, K, N, "down", gate_in.device)
    new_out = out is None
    if new_out:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=gate_in.device)
    _check_tensor(out, torch.bfloat16, (M, K), "out", gate_in.device)
    d = down.struct()
    rc = load().ffn_nvfp4_down_gemv(gate_in.data_ptr(), up_in.data_ptr(), M, N, K, ctypes.byref(d), int(act),
                                    out.data_ptr(), _stream_handle(stream))
    _check(rc, "ffn_nvfp4_down_gemv")
    _record(stream, out if new_out else None)
    return out


def quantize_workspace_bytes(rows: int, cols: int) -> int:
    return int(load().ffn_nvfp4_quantize_workspace_bytes(int(rows), int(cols)))


def quantize(w, codes=None, scales=None, scale2=None, workspace=None, stream=None):
    """NVFP4 of the bf16 weight w [rows, cols]: (codes uint8 [rows, cols/2],
    scales uint8 [rows, cols/16], scale2 fp32 [1]), all on w's device."""
    import torch
    rows, cols = w.shape
    _check_tensor(w, torch.bfloat16, (rows, cols), "w")
    dev = w.device
    fresh = []
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        fresh.append(codes)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        fresh.append(scales)
    if scale2 is None:
        scale2 = torch.empty(1, dtype=torch.float32, device=dev)
        fresh.append(scale2)
    _check_tensor(codes, torch.uint8, (rows, cols // 2), "codes", dev)
    _check_tensor(scales, torch.uint8, (rows, cols // 16), "scales", dev)
    _check_tensor(scale2, torch.float32, (1,), "scale2", dev)
    need = quantize_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
        fresh.append(workspace)
    rc = load().ffn_nvfp4_quantize(w.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(),
                                   scale2.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(rc, "ffn_nvfp4_quantize")
    _record(stream, *fresh)
    return codes, scales, scale2


def quantize_weight(w, stream=None) -> DeviceWeight:
    """:func:`quantize` as a DeviceWeight (waits for the result to read
    scale2 back to the host)."""
    codes, scales, scale2 = quantize(w, stream=stream)
    return DeviceWeight(codes, scales, float(scale2.cpu()[0]))


def bf16_from_bits(bits, device="cuda"):
    """A bf16 torch tensor on ``device`` from a numpy uint16 array of bf16 bits."""
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_to_f64(t):
    """A bf16 torch tensor as a float64 numpy array (exact)."""
    return t.float().cpu().double().numpy()


# ------------------------------------------------------------ FP8 weights


@dataclasses.dataclass
class Fp8DeviceWeight:
    """A block-scaled FP8 weight resident on the GPU: codes uint8 [rows, cols]
    (E4M3FN bytes) and block_scale float32 [ceil(rows/128), ceil(cols/128)]."""

    codes: "object"
    block_scale: "object"

    @property
    def rows(self) -> int:
        return int(self.codes.shape[0])

    @property
    def cols(self) -> int:
        return int(self.codes.shape[1])

    def struct(self) -> Fp8WeightStruct:
        return Fp8WeightStruct(self.codes.data_ptr(), self.block_scale.data_ptr())

    @classmethod
    def from_host(cls, w, device="cuda") -> "Fp8DeviceWeight":
        """From an object with numpy ``codes`` and ``block_scale``."""
        import torch
        return cls(torch.from_numpy(w.codes).to(device), torch.from_numpy(w.block_scale).to(device))


def _check_fp8_weight(w: Fp8DeviceWeight, rows: int, cols: int, name: str, device=None) -> None:
    import torch
    _check_tensor(w.codes, torch.uint8, (rows, cols), f"{name}.codes", device)
    _check_tensor(w.block_scale, torch.float32, ((rows + 127) // 128, (cols + 127) // 128), f"{name}.block_scale",
                  device)


def fp8_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(load().ffn_fp8_workspace_bytes(int(M), int(K), int(N)))


def fp8_forward(x, gate: Fp8DeviceWeight, up: Fp8DeviceWeight, down: Fp8DeviceWeight, act: int = ACT_SILU,
                out=None, workspace=None, stream=None):
    """out[M, K] (bf16) = W_d (act(W_g x) * (W_u x)) over FP8 weights."""
    import torch
    M, K = x.shape
    N = gate.rows
    _check_tensor(x, torch.bfloat16, (M, K), "x")
    _check_fp8_weight(gate, N, K, "gate", x.device)
    _check_fp8_weight(up, N, K, "up", x.device)
    _check_fp8_weight(down, K, N, "down", x.device)
    new_out = out is None
    if new_out:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    _check_tensor(out, torch.bfloat16, (M, K), "out", x.device)
    need = fp8_workspace_bytes(M, K, N)
    new_ws = workspace is None
    if new_ws:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    g, u, d = gate.struct(), up.struct(), down.struct()
    rc = load().ffn_fp8_forward(x.data_ptr(), M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                int(act), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                out.data_ptr(), _stream_handle(stream))
    _check(rc, "ffn_fp8_forward")
    _record(stream, out if new_out else None, workspace if new_ws else None)
    return out


def fp8_dual_gemv(x, gate: Fp8DeviceWeight, up: Fp8DeviceWeight, gate_out=None, up_out=None, stream=None):
    """(gate, up) fp32 [M, N] = (W_g x, W_u x) over FP8 weights."""
    import torch
    M, K = x.shape
    N = gate.rows
    _check_tensor(x, torch.bfloat16, (M, K), "x")
    _check_fp8_weight(gate, N, K, "gate", x.device)
    _check_fp8_weight(up, N, K, "up", x.device)
    new_g, new_u = gate_out is None, up_out is None
    if new_g:
        gate_out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if new_u:
        up_out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check_tensor(gate_out, torch.float32, (M, N), "gate_out", x.device)
    _check_tensor(up_out, torch.float32, (M, N), "up_out", x.device)
    g, u = gate.struct(), up.struct()
    rc = load().ffn_fp8_dual_gemv(x.data_ptr(), M, K, N, ctypes.byref(g), ctypes.byref(u),
                                  gate_out.data_ptr(), up_out.data_ptr(), _stream_handle(stream))
    _check(rc, "ffn_fp8_dual_gemv")
    _record(stream, gate_out if new_g else None, up_out if new_u else None)
    return gate_out, up_out


def fp8_down_gemv(gate_in, up_in, down: Fp8DeviceWeight, act: int = ACT_SILU, out=None, stream=None):
    """out[M, K] (bf16) = W_d bf16(act(gate) * up) over an FP8 W_d, with the
    activation fused into the down GEMV's input load."""
    import torch
    M, N = gate_in.shape
    K = down.rows
    _check_tensor(gate_in, torch.float32, (M, N), "gate_in")
    _check_tensor(up_in, torch.float32, (M, N), "up_in", gate_in.device)
    _check_fp8_weight(down, K, N, "down", gate_in.device)
    new_out = out is None
    if new_out:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=gate_in.device)
    _check_tensor(out, torch.bfloat16, (M, K), "out", gate_in.device)
    d = down.struct()
    rc = load().ffn_fp8_down_gemv(gate_in.data_ptr(), up_in.data_ptr(), M, N, K, ctypes.byref(d), int(act),
                                  out.data_ptr(), _stream_handle(stream))
    _check(rc, "ffn_fp8_down_gemv")
    _record(stream, out if new_out else None)
    return out


# ------------------------------------------------------------ W4A4 (MXFP4)


@dataclasses.dataclass
class MxDeviceWeight:
    """An MXFP4 weight on the GPU: codes uint8 [rows, cols/2], E8M0 scales
    uint8 [rows, cols/32], and the host fp32 scale2."""

    codes: "object"
    scales: "object"
    scale2: float

    @property
    def rows(self) -> int:
        return int(self.codes.shape[0])

    @property
    def cols(self) -> int:
        return int(self.codes.shape[1]) * 2

    def struct(self) -> MxWeightStruct:
        return MxWeightStruct(self.codes.data_ptr(), self.scales.data_ptr(), float(self.scale2))


def _check_mx_weight(w: MxDeviceWeight, rows: int, cols: int, name: str, device) -> None:
    """An MXFP4 weight of logical shape [rows, cols]: contiguous uint8 codes
    [rows, cols/2] and E8M0 bytes [rows, cols/32] on the device of the call."""
    import torch
    if cols % 32:
        raise ValueError(f"{name}: {cols} columns is not a multiple of 32")
    _check_tensor(w.codes, torch.uint8, (rows, cols // 2), f"{name}.codes", device)
    _check_tensor(w.scales, torch.uint8, (rows, cols // 32), f"{name}.scales", device)


def w4a4_prepare_weight(w: DeviceWeight, stream=None) -> MxDeviceWeight:
    """Requantise an NVFP4 weight to MXFP4 on the GPU (asynchronous)."""
    import torch
    rows, cols = w.rows, w.cols
    dev = w.codes.device
    _check_nvfp4_weight(w, rows, cols, "w", dev)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    st = w.struct()
    rc = load().ffn_w4a4_prepare_weight(ctypes.byref(st), rows, cols, codes.data_ptr(), scales.data_ptr(),
                                        _stream_handle(stream))
    _check(rc, "ffn_w4a4_prepare_weight")
    _record(stream, codes, scales)
    return MxDeviceWeight(codes, scales, float(w.scale2))


def w4a4_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(load().ffn_w4a4_workspace_bytes(int(M), int(K), int(N)))


def w4a4_dual_gemm(x, gate: MxDeviceWeight, up: MxDeviceWeight, gate_out=None, up_out=None, workspace=None,
                   stream=None):
    """(gate, up) fp32 [M, N] over MXFP4 activations and weights."""
    import torch
    M, K = x.shape
    N = gate.rows
    _check_tensor(x, torch.bfloat16, (M, K), "x")
    _check_mx_weight(gate, N, K, "gate", x.device)
    _check_mx_weight(up, N, K, "up", x.device)
    fresh = []
    if gate_out is None:
        gate_out = torch.empty((M, N), dtype=torch.float32, device=x.device)
        fresh.append(gate_out)
    if up_out is None:
        up_out = torch.empty((M, N), dtype=torch.float32, device=x.device)
        fresh.append(up_out)
    _check_tensor(gate_out, torch.float32, (M, N), "gate_out", x.device)
    _check_tensor(up_out, torch.float32, (M, N), "up_out", x.device)
    if workspace is None:
        workspace = torch.empty(max(w4a4_workspace_bytes(M, K, N), 1), dtype=torch.uint8, device=x.device)
        fresh.append(workspace)
    g, u = gate.struct(), up.struct()
    rc = load().ffn_w4a4_dual_gemm(x.data_ptr(), M, K, N, ctypes.byref(g), ctypes.byref(u), gate_out.data_ptr(),
                                   up_out.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(rc, "ffn_w4a4_dual_gemm")
    _record(stream, *fresh)
    return gate_out, up_out


def w4a4_forward(x, gate: MxDeviceWeight, up: MxDeviceWeight, down: DeviceWeight, act: int = ACT_SILU, out=None,
                 workspace=None, stream=None):
    """out[M, K] (bf16): W4A4 gate and up, then the NVFP4 down projection."""
    import torch
    M, K = x.shape
    N = gate.rows
    _check_tensor(x, torch.bfloat16, (M, K), "x")
    _check_mx_weight(gate, N, K, "gate", x.device)
    _check_mx_weight(up, N, K, "up", x.device)
    _check_nvfp4_weight(down, K, N, "down", x.device)
    fresh = []
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
        fresh.append(out)
    _check_tensor(out, torch.bfloat16, (M, K), "out", x.device)
    if workspace is None:
        workspace = torch.empty(max(w4a4_workspace_bytes(M, K, N), 1), dtype=torch.uint8, device=x.device)
        fresh.append(workspace)
    g, u, d = gate.struct(), up.struct(), down.struct()
    rc = load().ffn_w4a4_forward(x.data_ptr(), M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), int(act),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(), out.data_ptr(),
                                 _stream_handle(stream))
    _check(rc, "ffn_w4a4_forward")
    _record(stream, *fresh)
    return out


def w4a4_fp4_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(load().ffn_w4a4_fp4_workspace_bytes(int(M), int(K), int(N)))


def w4a4_down_gemm(h, down: MxDeviceWeight, out=None, workspace=None, stream=None):
    """out[M, K] (bf16) = scale2 * (mx(h) . mx(W_d)) for h [M, N] bf16 and an
    MXFP4 down weight [K, N]."""
    import torch
    M, N = h.shape
    K = down.rows
    _check_tensor(h, torch.bfloat16, (M, N), "h")
    _check_mx_weight(down, K, N, "down", h.device)
    fresh = []
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=h.device)
        fresh.append(out)
    _check_tensor(out, torch.bfloat16, (M, K), "out", h.device)
    if workspace is None:
        workspace = torch.empty(max(w4a4_fp4_workspace_bytes(M, K, N), 1), dtype=torch.uint8, device=h.device)
        fresh.append(workspace)
    d = down.struct()
    rc = load().ffn_w4a4_down_gemm(h.data_ptr(), M, N, K, ctypes.byref(d), out.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(rc, "ffn_w4a4_down_gemm")
    _record(stream, *fresh)
    return out


def w4a4_forward_fp4(x, gate: MxDeviceWeight, up: MxDeviceWeight, down: MxDeviceWeight, act: int = ACT_SILU,
                     out=None, workspace=None, stream=None):
    """out[M, K] (bf16): all three projections on 4 bits (MXFP4 weights and
    activations, h quantised before the down projection)."""
    import torch
    M, K = x.shape
    N = gate.rows
    _check_tensor(x, torch.bfloat16, (M, K), "x")
    _check_mx_weight(gate, N, K, "gate", x.device)
    _check_mx_weight(up, N, K, "up", x.device)
    _check_mx_weight(down, K, N, "down", x.device)
    fresh = []
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
        fresh.append(out)
    _check_tensor(out, torch.bfloat16, (M, K), "out", x.device)
    if workspace is None:
        workspace = torch.empty(max(w4a4_fp4_workspace_bytes(M, K, N), 1), dtype=torch.uint8, device=x.device)
        fresh.append(workspace)
    g, u, d = gate.struct(), up.struct(), down.struct()
    rc = load().ffn_w4a4_forward_fp4(x.data_ptr(), M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                     int(act), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     out.data_ptr(), _stream_handle(stream))
    _check(rc, "ffn_w4a4_forward_fp4")
    _record(stream, *fresh)
    return out


# ------------------------------------------------------------ measurement aid


class DiagRead:
    """Prepared arguments of ``ffn_diag_read`` over a list of device tensors
    (contiguous, sizes multiples of 16 bytes): ``launch(stream)`` enqueues one
    read of all of them."""

    def __init__(self, tensors):
        import torch
        if not 1 <= len(tensors) <= 8:
            raise ValueError("1 to 8 buffers")
        for t in tensors:
            if t.device.type != "cuda" or not t.is_contiguous():
                raise ValueError("buffers must be contiguous GPU tensors")
        self._keep = list(tensors)
        self.n = len(tensors)
        self.bytes = sum(t.numel() * t.element_size() for t in tensors)
        self._ptrs = (_P * self.n)(*[t.data_ptr() for t in tensors])
        self._sizes = (ctypes.c_size_t * self.n)(*[t.numel() * t.element_size() for t in tensors])
        self._sink = torch.zeros(1, dtype=torch.int32, device=tensors[0].device)

    def launch(self, stream=None) -> None:
        rc = load().ffn_diag_read(self._ptrs, self._sizes, self.n, self._sink.data_ptr(), _stream_handle(stream))
        _check(rc, "ffn_diag_read")


def diag_read(tensors, stream=None) -> None:
    """One streaming read of every byte of ``tensors`` (see ``ffn_diag.h``)."""
    DiagRead(tensors).launch(stream)
