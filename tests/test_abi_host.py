"""Host-only checks of the C ABI (no GPU): the library loads, exports every
function the header declares, and rejects invalid arguments before anything
is launched. Every call here fails validation (or is the empty M = 0 call),
so no HIP work is ever enqueued; fake device addresses are never touched.
"""
import ctypes

import pytest

import w4a16_nvfp4_dense_amd as ffn

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def W(codes=FAKE, scales=FAKE + 0x10000, scale2=1.0):
    return ffn.WeightStruct(codes, scales, scale2)


def fwd(x=FAKE, M=1, K=256, N=512, g=None, u=None, d=None, act=0, ws=FAKE + 0x200000, wsb=1 << 20,
        out=FAKE + 0x400000):
    g = g or W()
    u = u or W()
    d = d or W()
    return ffn.load().ffn_nvfp4_forward(x, M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), act,
                                        ws, wsb, out, 0)


def dual(x=FAKE, M=1, K=256, N=512, g=None, u=None, go=FAKE + 0x200000, uo=FAKE + 0x400000):
    g = g or W()
    u = u or W()
    return ffn.load().ffn_nvfp4_dual_gemv(x, M, K, N, ctypes.byref(g), ctypes.byref(u), go, uo, 0)


def down(gi=FAKE, ui=FAKE + 0x200000, M=1, N=512, K=256, d=None, act=0, out=FAKE + 0x400000):
    d = d or W()
    return ffn.load().ffn_nvfp4_down_gemv(gi, ui, M, N, K, ctypes.byref(d), act, out, 0)


def test_exports_every_header_symbol():
    lib = ffn.load()
    names = ffn.header_functions()
    assert set(names) == {"ffn_nvfp4_forward", "ffn_nvfp4_forward_noalloc", "ffn_nvfp4_dual_gemv",
                          "ffn_nvfp4_down_gemv", "ffn_nvfp4_workspace_bytes", "ffn_nvfp4_strerror",
                          "ffn_nvfp4_version", "ffn_nvfp4_quantize", "ffn_nvfp4_quantize_workspace_bytes"}
    fp8 = ffn.header_functions(ffn.FP8_HEADER_PATH)
    assert set(fp8) == {"ffn_fp8_forward", "ffn_fp8_dual_gemv", "ffn_fp8_down_gemv", "ffn_fp8_workspace_bytes"}
    w4 = ffn.header_functions(ffn.W4A4_HEADER_PATH)
    assert set(w4) == {"ffn_w4a4_prepare_weight", "ffn_w4a4_workspace_bytes", "ffn_w4a4_dual_gemm",
                       "ffn_w4a4_forward", "ffn_w4a4_fp4_workspace_bytes", "ffn_w4a4_down_gemm",
                       "ffn_w4a4_forward_fp4"}
    diag = ffn.header_functions(ffn.DIAG_HEADER_PATH)
    assert set(diag) == {"ffn_diag_read"}
    for n in list(names) + list(fp8) + list(w4) + list(diag):
        assert hasattr(lib, n), n


def test_noalloc_rejects_oversized_workspace_before_any_launch():
    """Shapes whose workspace exceeds the 4 MiB static scratch are refused
    before anything touches a device (the 128-row arm, and M <= 8 never)."""
    lib = ffn.load()
    w = W()
    assert ffn.workspace_bytes(128, 5120, 17408) > 4 << 20
    rc = lib.ffn_nvfp4_forward_noalloc(FAKE, 128, 5120, 17408, ctypes.byref(w), ctypes.byref(w), ctypes.byref(w),
                                       0, FAKE + 0x400000, 0)
    assert rc == ffn.ERR_WORKSPACE
    assert ffn.workspace_bytes(8, 65536, 65536) <= 4 << 20


def test_diag_read_validation():
    lib = ffn.load()
    P = ctypes.c_void_p
    S = ctypes.c_size_t

    def call(ptrs, sizes, n=None, sink=FAKE):
        n = len(ptrs) if n is None else n
        return lib.ffn_diag_read((P * max(1, len(ptrs)))(*ptrs), (S * max(1, len(sizes)))(*sizes), n, sink, 0)

    assert call([FAKE], [16], n=0) == ffn.ERR_SHAPE
    assert call([FAKE] * 9, [16] * 9) == ffn.ERR_SHAPE
    assert call([FAKE], [24]) == ffn.ERR_SHAPE
    assert call([FAKE + 8], [16]) == ffn.ERR_ALIGN
    assert call([FAKE], [16], sink=FAKE + 2) == ffn.ERR_ALIGN
    assert call([FAKE], [16], sink=0) == ffn.ERR_NULL
    assert call([0], [16]) == ffn.ERR_NULL
    assert lib.ffn_diag_read(None, None, 1, FAKE, 0) == ffn.ERR_NULL
    assert call([0, 0], [0, 0]) == ffn.OK  # nothing to read: no launch


def test_version_strerror_workspace():
    assert ffn.version() >= 100
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert ffn.strerror(s) and ffn.strerror(s) != "unknown status"
    assert ffn.strerror(-99) == "unknown status"
    assert ffn.workspace_bytes(1, 5120, 17408) == 17408 * 2
    assert ffn.workspace_bytes(8, 5120, 17408) == 8 * 17408 * 2
    assert ffn.workspace_bytes(0, 256, 512) == 0
    assert ffn.workspace_bytes(1, 250, 512) == 0
    # small-batch arm (9 <= M <= 40, K and N multiples of 256): h, the down
    # projection's partial sums when its reduction is split (N = 17408: 4
    # parts), the dual projection's when its reduction is split (two token
    # groups at K = 5120: 2 parts), and one 8-byte ready word per workgroup
    # of the larger split grid (about one workgroup per compute unit; 256
    # compute units assumed where no device is visible)
    r256 = lambda b: (b + 255) // 256 * 256
    flags = lambda grid: r256(8 * grid)
    assert ffn.workspace_bytes(9, 256, 512) == 9 * 512 * 2
    assert ffn.workspace_bytes(16, 5120, 17408) == 16 * 17408 * 2 + 4 * 16 * 5120 * 4 + flags(4 * 64)
    assert ffn.workspace_bytes(17, 5120, 17408) == (r256(17 * 17408 * 2) + 4 * 17 * 5120 * 4
                                                    + 2 * 2 * 17 * 17408 * 4 + flags(256))
    assert ffn.workspace_bytes(32, 4096, 8192) == r256(32 * 8192 * 2) + 2 * 32 * 4096 * 4 + flags(2 * 128)
    # dual reduction in 2 parts over 32 row tiles (512 rows): a grid of 64
    assert ffn.workspace_bytes(16, 5376, 512) == r256(16 * 512 * 2) + 2 * 2 * 16 * 512 * 4 + flags(2 * 32)
    # three token groups (33 <= M <= 40): the dual reduction in parts of at
    # most 2 rounds (K = 5120: 3 parts, 256 // 3 = 85 tile groups), the down
    # reduction in parts of at most 3 (N = 17408: 6 parts, 42 groups)
    assert ffn.workspace_bytes(33, 5120, 17408) == (r256(33 * 17408 * 2) + 6 * 33 * 5120 * 4
                                                    + 2 * 3 * 33 * 17408 * 4 + flags(max(3 * 85, 6 * 42)))
    assert ffn.workspace_bytes(40, 256, 512) == 40 * 512 * 2
    # 128-row matrix-core arm (M > 40, or K or N not a multiple of 256): h for
    # one block of 128 rows and the partial slots
    ws41 = ffn.workspace_bytes(41, 256, 512)
    assert ws41 > 41 * 512 * 2 and ws41 % 256 == 0 and ws41 > 32 << 20
    assert ffn.workspace_bytes(16, 640, 1024) > 32 << 20
    assert ffn.workspace_bytes(128, 5120, 17408) == ffn.workspace_bytes(4096, 5120, 17408)
    assert ffn.workspace_bytes(128, 5120, 17408) >= 128 * 17408 * 2
    assert ffn.workspace_bytes(9, 96, 512) == 0   # the arm needs K, N multiples of 64
    assert ffn.workspace_bytes(65537, 256, 512) == 0
    assert ffn.workspace_bytes(3, 96, 160) % 256 == 0


@pytest.mark.parametrize("call", [fwd, dual, down])
def test_null_pointers(call):
    if call is fwd:
        assert fwd(x=0) == ffn.ERR_NULL
        assert fwd(out=0) == ffn.ERR_NULL
        assert fwd(ws=0) == ffn.ERR_NULL
        assert fwd(g=W(codes=0)) == ffn.ERR_NULL
        assert fwd(d=W(scales=0)) == ffn.ERR_NULL
    elif call is dual:
        assert dual(x=0) == ffn.ERR_NULL
        assert dual(go=0) == ffn.ERR_NULL
        assert dual(u=W(codes=0)) == ffn.ERR_NULL
    else:
        assert down(gi=0) == ffn.ERR_NULL
        assert down(out=0) == ffn.ERR_NULL
        assert down(d=W(codes=0)) == ffn.ERR_NULL


def test_misaligned():
    assert fwd(x=FAKE + 2) == ffn.ERR_ALIGN
    assert fwd(out=FAKE + 0x400008) == ffn.ERR_ALIGN
    assert fwd(ws=FAKE + 4) == ffn.ERR_ALIGN
    assert fwd(g=W(codes=FAKE + 8)) == ffn.ERR_ALIGN
    assert fwd(u=W(scales=FAKE + 1)) == ffn.ERR_ALIGN
    assert dual(go=FAKE + 4) == ffn.ERR_ALIGN
    assert down(ui=FAKE + 0x200004) == ffn.ERR_ALIGN
    # scales need 2-byte alignment up to M = 8 (this one fails later, on M),
    # 8-byte alignment on the matrix-core arms
    assert fwd(g=W(scales=FAKE + 2), M=-1) == ffn.ERR_BATCH
    assert fwd(g=W(scales=FAKE + 2), M=9, wsb=1 << 30) == ffn.ERR_ALIGN
    assert fwd(g=W(scales=FAKE + 4), M=9, wsb=1 << 30) == ffn.ERR_ALIGN
    assert dual(u=W(scales=FAKE + 6), M=64) == ffn.ERR_ALIGN
    assert dual(u=W(scales=FAKE + 4), M=17) == ffn.ERR_ALIGN
    assert down(d=W(scales=FAKE + 2), M=128) == ffn.ERR_ALIGN


@pytest.mark.parametrize("K,N", [(0, 512), (256, 0), (250, 512), (256, 500), (-32, 512), (65568, 512),
                                 (256, 70000)])
def test_bad_shapes(K, N):
    assert fwd(K=K, N=N) == ffn.ERR_SHAPE
    assert dual(K=K, N=N) == ffn.ERR_SHAPE
    assert down(K=K, N=N) == ffn.ERR_SHAPE


@pytest.mark.parametrize("M", [-1, -100, 65537, 1 << 24])
def test_unsupported_batch(M):
    assert fwd(M=M) == ffn.ERR_BATCH
    assert dual(M=M) == ffn.ERR_BATCH
    assert down(M=M) == ffn.ERR_BATCH


@pytest.mark.parametrize("K,N", [(96, 512), (256, 480), (320, 96)])
def test_prefill_needs_multiples_of_64(K, N):
    # M <= 8 takes any multiple of 32; the matrix-core arm (M > 8) needs 64
    assert fwd(M=9, K=K, N=N, wsb=1 << 30) == ffn.ERR_SHAPE
    assert dual(M=16, K=K, N=N) == ffn.ERR_SHAPE
    assert down(M=128, K=K, N=N) == ffn.ERR_SHAPE


def test_bad_act_and_workspace_and_scale2():
    assert fwd(act=2) == ffn.ERR_ACT
    assert fwd(act=-1) == ffn.ERR_ACT
    assert down(act=7) == ffn.ERR_ACT
    assert fwd(wsb=ffn.workspace_bytes(1, 256, 512) - 1) == ffn.ERR_WORKSPACE
    assert fwd(M=2, wsb=ffn.workspace_bytes(1, 256, 512)) == ffn.ERR_WORKSPACE
    assert fwd(M=9, wsb=ffn.workspace_bytes(9, 256, 512) - 256) == ffn.ERR_WORKSPACE
    assert fwd(g=W(scale2=float("nan"))) == ffn.ERR_SCALE2
    assert dual(u=W(scale2=float("inf"))) == ffn.ERR_SCALE2
    assert down(d=W(scale2=float("-inf"))) == ffn.ERR_SCALE2


def test_empty_batch_is_a_noop():
    # M = 0: nothing to compute; output/workspace pointers may be NULL.
    assert fwd(M=0, x=0, out=0, ws=0, wsb=0) == ffn.OK
    assert dual(M=0, x=0, go=0, uo=0) == ffn.OK
    assert down(M=0, gi=0, ui=0, out=0) == ffn.OK
    # ...but the rest is still validated
    assert fwd(M=0, K=100) == ffn.ERR_SHAPE
    assert fwd(M=0, act=5) == ffn.ERR_ACT
    assert dual(M=0, g=W(codes=0)) == ffn.ERR_NULL


# ------------------------------------------------------------ quantiser


def quant(w=FAKE, rows=64, cols=256, codes=FAKE + 0x200000, scales=FAKE + 0x400000, s2=FAKE + 0x500000,
          ws=FAKE + 0x600000, wsb=1 << 16):
    return ffn.load().ffn_nvfp4_quantize(w, rows, cols, codes, scales, s2, ws, wsb, 0)


def test_quantize_workspace_bytes():
    assert ffn.quantize_workspace_bytes(17408, 5120) == 8192
    assert ffn.quantize_workspace_bytes(1, 32) == 8192
    for rows, cols in [(0, 256), (64, 0), (64, 48), (65537, 256), (64, 65568), (-1, 256)]:
        assert ffn.quantize_workspace_bytes(rows, cols) == 0


def test_quantize_validation():
    assert quant(w=0) == ffn.ERR_NULL
    assert quant(codes=0) == ffn.ERR_NULL
    assert quant(scales=0) == ffn.ERR_NULL
    assert quant(s2=0) == ffn.ERR_NULL
    assert quant(ws=0) == ffn.ERR_NULL
    assert quant(w=FAKE + 8) == ffn.ERR_ALIGN
    assert quant(codes=FAKE + 0x200004) == ffn.ERR_ALIGN
    assert quant(s2=FAKE + 0x500002) == ffn.ERR_ALIGN
    assert quant(ws=FAKE + 0x600002) == ffn.ERR_ALIGN
    assert quant(wsb=8191) == ffn.ERR_WORKSPACE
    for rows, cols in [(0, 256), (64, 0), (64, 48), (65537, 256), (64, 65568)]:
        assert quant(rows=rows, cols=cols) == ffn.ERR_SHAPE
    # shape is checked before pointers
    assert quant(rows=0, w=0) == ffn.ERR_SHAPE


# ------------------------------------------------------------ FP8 entry points


def F8(codes=FAKE, bs=FAKE + 0x10000):
    return ffn.Fp8WeightStruct(codes, bs)


def f8fwd(x=FAKE, M=1, K=256, N=512, g=None, u=None, d=None, act=0, ws=FAKE + 0x200000, wsb=1 << 20,
          out=FAKE + 0x400000):
    g, u, d = g or F8(), u or F8(), d or F8()
    return ffn.load().ffn_fp8_forward(x, M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), act,
                                      ws, wsb, out, 0)


def f8dual(x=FAKE, M=1, K=256, N=512, g=None, u=None, go=FAKE + 0x200000, uo=FAKE + 0x400000):
    g, u = g or F8(), u or F8()
    return ffn.load().ffn_fp8_dual_gemv(x, M, K, N, ctypes.byref(g), ctypes.byref(u), go, uo, 0)


def f8down(gi=FAKE, ui=FAKE + 0x200000, M=1, N=512, K=256, d=None, act=0, out=FAKE + 0x400000):
    d = d or F8()
    return ffn.load().ffn_fp8_down_gemv(gi, ui, M, N, K, ctypes.byref(d), act, out, 0)


def test_fp8_workspace_bytes():
    assert ffn.fp8_workspace_bytes(1, 5120, 17408) == 17408 * 2
    assert ffn.fp8_workspace_bytes(8, 5120, 17408) == 8 * 17408 * 2
    assert ffn.fp8_workspace_bytes(3, 400, 336) == 2048  # 3 * 336 * 2 = 2016, rounded up to 256
    assert ffn.fp8_workspace_bytes(0, 256, 512) == 0
    assert ffn.fp8_workspace_bytes(9, 256, 512) == 0      # the FP8 path covers M <= 8
    assert ffn.fp8_workspace_bytes(1, 264, 512) == 0      # K not a multiple of 16
    assert ffn.fp8_workspace_bytes(1, 256, 24592) == 0    # N above 24576
    assert ffn.fp8_workspace_bytes(1, 24576, 16) == 32 * 8


@pytest.mark.parametrize("call", [f8fwd, f8dual, f8down])
def test_fp8_validation(call):
    kw = {"K": 256, "N": 512}
    # NULL and misaligned weights
    key = {"f8fwd": "g", "f8dual": "g", "f8down": "d"}[call.__name__]
    assert call(**{key: F8(codes=0)}) == ffn.ERR_NULL
    assert call(**{key: F8(bs=0)}) == ffn.ERR_NULL
    assert call(**{key: F8(codes=FAKE + 8)}) == ffn.ERR_ALIGN
    assert call(**{key: F8(bs=FAKE + 0x10002)}) == ffn.ERR_ALIGN
    # shapes: multiples of 16 up to 24576
    for K, N in ((0, 512), (256, 0), (264, 512), (256, 520), (24592, 512), (256, 24592), (-16, 512)):
        assert call(K=K, N=N) == ffn.ERR_SHAPE, (K, N)
    # batches: 0..8 only
    for M in (-1, 9, 16, 128):
        assert call(M=M, **kw) == ffn.ERR_BATCH, M
    # the empty call validates weights and shape, then launches nothing
    assert call(M=0, **kw) == ffn.OK
    if call is f8fwd:
        assert f8fwd(M=0, x=0, out=0, ws=0) == ffn.OK
        assert f8fwd(x=0) == ffn.ERR_NULL
        assert f8fwd(ws=0) == ffn.ERR_NULL
        assert f8fwd(x=FAKE + 8) == ffn.ERR_ALIGN
        assert f8fwd(ws=FAKE + 0x200008) == ffn.ERR_ALIGN
        assert f8fwd(act=2) == ffn.ERR_ACT
        assert f8fwd(wsb=512 * 2 - 1) == ffn.ERR_WORKSPACE
        assert f8fwd(M=2, wsb=1024) == ffn.ERR_WORKSPACE
    elif call is f8dual:
        assert f8dual(M=0, x=0, go=0, uo=0) == ffn.OK
        assert f8dual(go=0) == ffn.ERR_NULL
        assert f8dual(uo=FAKE + 0x400004) == ffn.ERR_ALIGN
    else:
        assert f8down(M=0, gi=0, ui=0, out=0) == ffn.OK
        assert f8down(ui=0) == ffn.ERR_NULL
        assert f8down(out=FAKE + 0x400002) == ffn.ERR_ALIGN
        assert f8down(act=-1) == ffn.ERR_ACT
        assert f8down(M=0, act=7) == ffn.ERR_ACT


# ------------------------------------------------------------ W4A4 entry points


def MX(codes=FAKE, scales=FAKE + 0x10000, scale2=1.0):
    return ffn.MxWeightStruct(codes, scales, scale2)


def w4fwd(x=FAKE, M=1, K=256, N=64, g=None, u=None, d=None, act=0, ws=FAKE + 0x200000, wsb=1 << 24,
          out=FAKE + 0x400000):
    g, u, d = g or MX(), u or MX(), d or W()
    return ffn.load().ffn_w4a4_forward(x, M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), act,
                                       ws, wsb, out, 0)


def w4dual(x=FAKE, M=1, K=256, N=64, g=None, u=None, go=FAKE + 0x200000, uo=FAKE + 0x400000,
           ws=FAKE + 0x600000, wsb=1 << 24):
    g, u = g or MX(), u or MX()
    return ffn.load().ffn_w4a4_dual_gemm(x, M, K, N, ctypes.byref(g), ctypes.byref(u), go, uo, ws, wsb, 0)


def test_w4a4_workspace_bytes():
    r = lambda b: (b + 255) // 256 * 256
    partials = ffn.w4a4_workspace_bytes(1, 256, 64) - r(128) - r(8) - r(128)
    assert partials > 0 and partials % 256 == 0
    assert ffn.w4a4_workspace_bytes(128, 5120, 17408) == r(128 * 2560) + r(128 * 160) + r(128 * 17408 * 2) + partials
    assert ffn.w4a4_workspace_bytes(0, 256, 64) == 0
    assert ffn.w4a4_workspace_bytes(1, 128, 64) == 0     # K must be a multiple of 256
    assert ffn.w4a4_workspace_bytes(1, 256, 96) == 0     # N must be a multiple of 64
    assert ffn.w4a4_workspace_bytes(65537, 256, 64) == 0


@pytest.mark.parametrize("call", [w4fwd, w4dual])
def test_w4a4_validation(call):
    assert call(g=MX(codes=0)) == ffn.ERR_NULL
    assert call(u=MX(scales=0)) == ffn.ERR_NULL
    assert call(g=MX(codes=FAKE + 8)) == ffn.ERR_ALIGN
    assert call(g=MX(scales=FAKE + 0x10004)) == ffn.ERR_ALIGN
    assert call(g=MX(scale2=float("inf"))) == ffn.ERR_SCALE2
    for K, N in ((128, 64), (256, 96), (0, 64), (256, 0), (65792, 64)):
        assert call(K=K, N=N) == ffn.ERR_SHAPE, (K, N)
    assert call(M=-1) == ffn.ERR_BATCH
    assert call(M=65537) == ffn.ERR_BATCH
    assert call(M=0, x=0) == ffn.OK
    assert call(x=0) == ffn.ERR_NULL
    assert call(x=FAKE + 8) == ffn.ERR_ALIGN
    assert call(wsb=100) == ffn.ERR_WORKSPACE
    if call is w4fwd:
        assert w4fwd(act=3) == ffn.ERR_ACT
        assert w4fwd(d=W(scales=FAKE + 0x10002)) == ffn.ERR_ALIGN
        assert w4fwd(d=W(codes=0)) == ffn.ERR_NULL
        assert w4fwd(d=W(scale2=float("nan"))) == ffn.ERR_SCALE2
    else:
        assert w4dual(go=0) == ffn.ERR_NULL
        assert w4dual(ws=0) == ffn.ERR_NULL


def w4fp4(x=FAKE, M=1, K=256, N=256, g=None, u=None, d=None, act=0, ws=FAKE + 0x200000, wsb=1 << 24,
          out=FAKE + 0x400000):
    g, u, d = g or MX(), u or MX(), d or MX()
    return ffn.load().ffn_w4a4_forward_fp4(x, M, K, N, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), act,
                                           ws, wsb, out, 0)


def w4down(h=FAKE, M=1, N=256, K=256, d=None, out=FAKE + 0x400000, ws=FAKE + 0x200000, wsb=1 << 24):
    d = d or MX()
    return ffn.load().ffn_w4a4_down_gemm(h, M, N, K, ctypes.byref(d), out, ws, wsb, 0)


def test_w4a4_fp4_workspace_bytes():
    """mx(x), h, mx(h), the down projection's partial sums and ready words:
    at K = 5120 the reduction is split in 3 parts over 80 row blocks of 64
    (256 compute units assumed where no device is visible)."""
    r = lambda b: (b + 255) // 256 * 256
    M, K, N = 128, 5120, 17408
    want = (r(M * K // 2) + r(M * K // 32) + r(M * N * 2) + r(M * N // 2) + r(M * N // 32)
            + r(3 * 128 * K * 4) + r(3 * 80 * 8))
    assert ffn.w4a4_fp4_workspace_bytes(M, K, N) == want
    # one 256-column piece: no split, no partial sums
    assert ffn.w4a4_fp4_workspace_bytes(1, 256, 256) == r(128) + r(8) + r(512) + r(128) + r(8)
    assert ffn.w4a4_fp4_workspace_bytes(1, 256, 320) == 0   # N must be a multiple of 256 here
    assert ffn.w4a4_fp4_workspace_bytes(0, 256, 256) == 0


@pytest.mark.parametrize("call", [w4fp4, w4down])
def test_w4a4_fp4_validation(call):
    wkey = "d" if call is w4down else "g"
    assert call(**{wkey: MX(codes=0)}) == ffn.ERR_NULL
    assert call(**{wkey: MX(codes=FAKE + 8)}) == ffn.ERR_ALIGN
    assert call(**{wkey: MX(scale2=float("inf"))}) == ffn.ERR_SCALE2
    assert call(d=MX(scales=FAKE + 0x10004)) == ffn.ERR_ALIGN
    for K, N in ((128, 256), (256, 320), (256, 64), (0, 256), (65792, 256)):
        assert call(K=K, N=N) == ffn.ERR_SHAPE, (K, N)
    assert call(M=-1) == ffn.ERR_BATCH
    assert call(wsb=100) == ffn.ERR_WORKSPACE
    assert call(ws=0) == ffn.ERR_NULL
    assert call(out=FAKE + 8) == ffn.ERR_ALIGN
    if call is w4fp4:
        assert w4fp4(act=3) == ffn.ERR_ACT
        assert w4fp4(M=0, x=0) == ffn.OK
        assert w4fp4(x=0) == ffn.ERR_NULL
    else:
        assert w4down(M=0, h=0) == ffn.OK
        assert w4down(h=0) == ffn.ERR_NULL
        assert w4down(h=FAKE + 8) == ffn.ERR_ALIGN


def test_w4a4_prepare_validation():
    lib = ffn.load()
    w = W()
    call = lambda rows=64, cols=256, mc=FAKE + 0x200000, ms=FAKE + 0x300000, wt=w: \
        lib.ffn_w4a4_prepare_weight(ctypes.byref(wt), rows, cols, mc, ms, 0)
    assert call(mc=0) == ffn.ERR_NULL
    assert call(wt=W(codes=0)) == ffn.ERR_NULL
    assert call(cols=48) == ffn.ERR_SHAPE
    assert call(rows=0) == ffn.ERR_SHAPE
    assert call(mc=FAKE + 0x200008) == ffn.ERR_ALIGN
    assert call(wt=W(scales=FAKE + 0x10001)) == ffn.ERR_ALIGN


def test_traffic_summaries_match_sources():
    """Every committed HBM-counter summary names the kernel sources it was
    measured on by digest; bench.py reports its traffic only while they
    match. A source change that leaves the kernel's instructions unchanged
    must re-stamp the digest (after checking the assembly), any other must
    re-take the counters: either way this keeps the reported traffic alive."""
    import glob
    import json
    import os
    from w4a16_nvfp4_dense_amd import profiling
    files = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                          "profiles", "traffic_*.json")))
    assert files
    for f in files:
        t = json.load(open(f))
        assert t["source_digest"] == profiling.source_digest(t.get("source_files")), os.path.basename(f)
