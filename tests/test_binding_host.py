"""The Python binding rejects mismatched weights before any pointer reaches
the C ABI (the ABI sees only pointers, so a transposed or short weight would
be read out of bounds). Runs on the CPU with stand-in tensors that carry a
GPU device, dtype and shape but no memory: every case must fail in the
checks, before a data pointer is taken."""
import pytest
import torch

import w4a16_nvfp4_dense_amd as ffn


class Fake:
    """Shape, dtype, device and contiguity of a GPU tensor, nothing else."""

    def __init__(self, shape, dtype=torch.uint8, device="cuda:0", contiguous=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self._contiguous = contiguous

    def is_contiguous(self):
        return self._contiguous

    def data_ptr(self):
        raise AssertionError("a data pointer was taken before the checks failed")


M, K, N = 2, 256, 512


def nv(rows, cols, **kw):
    return ffn.DeviceWeight(Fake((rows, cols // 2), **kw), Fake((rows, cols // 16), **kw), 1.0)


def x_of(m=M, k=K):
    return Fake((m, k), torch.bfloat16)


def good():
    return nv(N, K), nv(N, K), nv(K, N)


@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_forward_transposed_weight(which):
    g, u, d = good()
    if which == "gate":
        g = nv(K, N)
    elif which == "up":
        u = nv(K, N)
    else:
        d = nv(N, K)
    with pytest.raises(ValueError):
        ffn.forward(x_of(), g, u, d, out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))


def test_forward_wrong_scales():
    g, u, d = good()
    d = ffn.DeviceWeight(d.codes, Fake((K, N // 32)), 1.0)
    with pytest.raises(ValueError, match="down.scales"):
        ffn.forward(x_of(), g, u, d, out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))


def test_forward_non_contiguous_and_dtype():
    g, u, d = good()
    g = ffn.DeviceWeight(Fake((N, K // 2), contiguous=False), g.scales, 1.0)
    with pytest.raises(ValueError, match="contiguous"):
        ffn.forward(x_of(), g, u, d, out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))
    g, u, d = good()
    u = ffn.DeviceWeight(Fake((N, K // 2), torch.int8), u.scales, 1.0)
    with pytest.raises(ValueError, match="up.codes"):
        ffn.forward(x_of(), g, u, d, out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))


def test_forward_weight_on_other_device():
    g, u, d = good()
    d = nv(K, N, device="cuda:1")
    with pytest.raises(ValueError, match="must be on"):
        ffn.forward(x_of(), g, u, d, out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))


def test_forward_cpu_weight():
    g, u, d = good()
    g = nv(N, K, device="cpu")
    with pytest.raises(ValueError, match="GPU tensor"):
        ffn.forward(x_of(), g, u, d, out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))


def test_dual_and_down_check_weights():
    g, u, d = good()
    with pytest.raises(ValueError):
        ffn.dual_gemv(x_of(), g, nv(N, 2 * K), gate_out=Fake((M, N), torch.float32),
                      up_out=Fake((M, N), torch.float32))
    with pytest.raises(ValueError):
        ffn.down_gemv(Fake((M, N), torch.float32), Fake((M, N), torch.float32), nv(K, N // 2),
                      out=Fake((M, K), torch.bfloat16))
    with pytest.raises(ValueError, match="up_in"):
        ffn.down_gemv(Fake((M, N), torch.float32), Fake((M, N + 32), torch.float32), d,
                      out=Fake((M, K), torch.bfloat16))


def test_w4a4_checks_weights():
    mx = lambda r, c: ffn.MxDeviceWeight(Fake((r, c // 2)), Fake((r, c // 32)), 1.0)
    g, u = mx(N, K), mx(N, K)
    bad = ffn.MxDeviceWeight(Fake((N, K // 2)), Fake((N, K // 16)), 1.0)
    with pytest.raises(ValueError, match="scales"):
        ffn.w4a4_dual_gemm(x_of(), g, bad, gate_out=Fake((M, N), torch.float32), up_out=Fake((M, N), torch.float32),
                           workspace=Fake((1,)))
    with pytest.raises(ValueError, match="down"):
        ffn.w4a4_forward(x_of(), g, u, nv(N, K), out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))
    w = ffn.DeviceWeight(Fake((N, K // 2)), Fake((N, K // 32)), 1.0)
    with pytest.raises(ValueError, match="w.scales"):
        ffn.w4a4_prepare_weight(w)
    # all three projections on 4 bits: the down weight is MXFP4 [K, N]
    with pytest.raises(ValueError, match="down"):
        ffn.w4a4_forward_fp4(x_of(), g, u, mx(N, K), out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))
    with pytest.raises(ValueError, match="down"):
        ffn.w4a4_down_gemm(Fake((M, N), torch.bfloat16), mx(K, N + 32), out=Fake((M, K), torch.bfloat16),
                           workspace=Fake((1,)))
    with pytest.raises(ValueError, match="h"):
        ffn.w4a4_down_gemm(Fake((M, N), torch.float32), mx(K, N), out=Fake((M, K), torch.bfloat16),
                           workspace=Fake((1,)))


def test_fp8_checks_weights():
    f8 = lambda r, c: ffn.Fp8DeviceWeight(Fake((r, c)), Fake(((r + 127) // 128, (c + 127) // 128), torch.float32))
    with pytest.raises(ValueError):
        ffn.fp8_forward(x_of(), f8(N, K), f8(N, K), f8(N, K), out=Fake((M, K), torch.bfloat16), workspace=Fake((1,)))
