"""Benchmark of the NVFP4 W4A16 gated FFN on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one FFN forward (dual gate+up GEMV, then the down GEMV with the
activation fused into its input load) over one batch of synthetic input. The
default workload is the M=1 SwiGLU decode FFN (hidden 5120, intermediate
17408). Weights are rotated over several byte-identical copies so the 256 MB
Infinity Cache cannot serve repeated reads; all inputs are resident in HBM
before the timed region.

Prints ONE JSON line on stdout. `value` is the achieved algorithmic HBM
bandwidth of the whole forward (bytes the method must move / time), with
`us_per_forward` beside it; `roofline` reports the dominant kernel (the dual
GEMV, 2/3 of the bytes) timed with HIP events on the stream it runs on, around
a batch of back-to-back launches; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "µs/FFN forward + achieved HBM GB/s (% of peak), NVFP4 SwiGLU decode M=1"

WORKLOADS = {
    # name: (config index, M)
    "tiny_silu_m1": (0, 1),
    "decode_silu_m1": (1, 1),
    "decode_gelu_m1": (2, 1),
    "verify_silu_m2": (3, 2),
    "verify_silu_m3": (3, 3),
    "verify_silu_m4": (3, 4),
    "verify_silu_m5": (3, 5),
    "verify_silu_m6": (3, 6),
    "verify_silu_m7": (3, 7),
    "verify_silu_m8": (3, 8),
    "prefill_silu_m128": (4, 128),
    # small batches (9 <= M <= 40) on the prefill shapes: the small-batch arm
    "smallbatch_silu_m9": (4, 9),
    "smallbatch_silu_m16": (4, 16),
    "smallbatch_silu_m17": (4, 17),
    "smallbatch_silu_m32": (4, 32),
    "smallbatch_silu_m33": (4, 33),
    "smallbatch_silu_m40": (4, 40),
    # 41 <= M <= 64: the 128-row matrix-core arm (one or two token tiles)
    "smallbatch_silu_m48": (4, 48),
    "smallbatch_silu_m64": (4, 64),
    "prefill_silu_m96": (4, 96),
}
SMALL_BATCH_MAX_M = 40  # above this the forward runs the 128-row matrix-core arm
# The BF16 -> NVFP4 quantiser (ffn_nvfp4_quantize) on one weight of the decode
# gate/up shape; timed like the forward, reported on its own line.
QUANT_WORKLOADS = {"quantize_17408x5120": (17408, 5120)}
QUANT_METRIC = "µs per BF16->NVFP4 weight quantise + achieved HBM GB/s (% of peak)"
# The same FFN over block-scaled FP8 weights (ffn_fp8_forward, E4M3 codes and
# fp32 128 x 128 block scales) on the decode shape; reported on its own line.
FP8_WORKLOADS = {"fp8_decode_silu_m1": 1, "fp8_verify_silu_m2": 2, "fp8_verify_silu_m3": 3,
                 "fp8_verify_silu_m8": 8}
FP8_METRIC = "µs/FFN forward + achieved HBM GB/s (% of peak), block-scaled FP8 SwiGLU"
# The W4A4 prefill arm on the prefill shape, each its own line: the hybrid
# (ffn_w4a4_forward: MXFP4 gate/up on FP4 matrix cores, NVFP4 down on the bf16
# arm) and all three projections on 4 bits (ffn_w4a4_forward_fp4).
W4A4_WORKLOADS = {"w4a4_prefill_silu_m128": (128, False), "w4a4fp4_prefill_silu_m128": (128, True)}
W4A4_METRIC = "µs/FFN forward + achieved TFLOP/s, W4A4 (MXFP4 gate/up) prefill SwiGLU"
W4A4_FP4_METRIC = "µs/FFN forward + achieved TFLOP/s, W4A4 (MXFP4 gate/up/down) prefill SwiGLU"
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lead_spin(n_launch_calls):
    """Starts a timed region with the GPU busy: a bounded spin kernel
    (torch.cuda._sleep, on the current stream) runs while the host enqueues
    the region's start event and launches, so the region holds the launches
    back to back and not the host's latency to issue the first one after the
    synchronisation. About 15 us per enqueued call plus 50 us, at most 20 ms
    (cycles counted at ~2 GHz); the spin itself is outside the region."""
    import torch
    us = min(20000.0, 50.0 + 15.0 * n_launch_calls)
    torch.cuda._sleep(int(us * 2000))


def timed_ms(fn, n, stream, warmup=0):
    """Milliseconds for fn(0) .. fn(n - 1), enqueued back to back on `stream`
    (the current stream), between HIP events on that stream, after `warmup`
    untimed calls and a synchronisation."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    lead_spin(n)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def roofline_bound(flops, nbytes, peak_tflops, peak_gbs=8000.0):
    """'mfma' when the arithmetic intensity is at or above the ridge point of
    the matrix peak over HBM bandwidth, else 'hbm'."""
    return "mfma" if flops / nbytes >= peak_tflops * 1e12 / (peak_gbs * 1e9) else "hbm"


def algorithmic_bytes(M, K, N):
    """Bytes each launch must move at minimum: NVFP4 codes + E4M3 scales of
    the weights it streams, its activation input and its output. The forward
    passes h = act(gate) * up between its two kernels as bf16 [M, N]."""
    w1 = N * K // 2 + N * K // 16          # one [N, K] (or [K, N]) NVFP4 weight
    return {
        "weights": 3 * w1,
        "forward": 3 * w1 + 2 * M * K + 2 * M * N + 2 * M * N + 2 * M * K,
        # the dual GEMV entry as timed for the roofline: fp32 gate and up out
        "dual_f32": 2 * w1 + 2 * M * K + 2 * M * N * 4,
        "down_h": w1 + 2 * M * N + 2 * M * K,
    }


def measured_traffic(workload, what="dual_gemv"):
    """HBM bytes per launch of the dual GEMV (or, with what="forward", per
    forward summed over its kernels) from the committed counter summary
    (profiles/traffic_<what>_<workload>.json), or None when there is none or
    the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{what}_{workload}.json")
    if not os.path.exists(path):
        return None
    from w4a16_nvfp4_dense_amd import profiling
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != profiling.source_digest(t.get("source_files")):
        log(f"[bench] {path} was measured on other kernel sources: traffic not reported")
        return None
    return t


def cpu_baseline(case, seconds):
    import numpy as np
    import oracle

    orc = oracle.default()
    b = algorithmic_bytes(case.M, case.K, case.N)["forward"]
    orc.ffn(case)  # warm
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.ffn(case)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    us = el / n * 1e6
    return {"value": round(b / (us * 1e-6) / 1e9, 3), "unit": "GB/s", "us_per_forward": round(us, 1),
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{n} full forwards of the same workload (fp64 C oracle, OpenMP over output rows), "
                      f"{el:.1f} s"}


def calibration_copy(dev):
    """A plain 64 MiB device-to-device copy (three times), the reference that
    scales FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(64 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def fp8_algorithmic_bytes(M, K, N):
    """As algorithmic_bytes for FP8 weights: one code byte per element and an
    fp32 scale per 128 x 128 block."""
    w1 = N * K + 4 * ((N + 127) // 128) * ((K + 127) // 128)
    return {
        "weights": 3 * w1,
        "forward": 3 * w1 + 2 * M * K + 2 * M * N + 2 * M * N + 2 * M * K,
        "dual_f32": 2 * w1 + 2 * M * K + 2 * M * N * 4,
    }


def fp8_cpu_baseline(case, seconds):
    import oracle

    orc = oracle.default()
    b = fp8_algorithmic_bytes(case.M, case.K, case.N)["forward"]
    orc.fp8_ffn(case)
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.fp8_ffn(case)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    us = el / n * 1e6
    return {"value": round(b / (us * 1e-6) / 1e9, 3), "unit": "GB/s", "us_per_forward": round(us, 1),
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{n} full FP8 forwards of the same workload (fp64 C oracle, OpenMP over output rows), "
                      f"{el:.1f} s"}


def bench_fp8(args):
    import torch

    import ffn_inputs as fi
    import w4a16_nvfp4_dense_amd as ffn

    lib = ffn.load()
    M = FP8_WORKLOADS[args.workload]
    case = fi.make_fp8_config(M=M)
    K, N, act = case.K, case.N, case.act
    nbytes = fp8_algorithmic_bytes(M, K, N)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copies = [tuple(ffn.Fp8DeviceWeight.from_host(w, dev) for w in (case.gate, case.up, case.down))
              for _ in range(args.copies)]
    structs = [tuple(w.struct() for w in c) for c in copies]
    refs = [tuple(ctypes.byref(s) for s in c) for c in structs]
    x = ffn.bf16_from_bits(case.x_bits, dev)
    out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ws_bytes = ffn.fp8_workspace_bytes(M, K, N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    gate_out = torch.empty((M, N), dtype=torch.float32, device=dev)
    up_out = torch.empty((M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    xp, op, wp, gp, upp = x.data_ptr(), out.data_ptr(), ws.data_ptr(), gate_out.data_ptr(), up_out.data_ptr()
    nc = len(refs)

    def step(i):
        g, u, d = refs[i % nc]
        rc = lib.ffn_fp8_forward(xp, M, K, N, g, u, d, act, wp, ws_bytes, op, sh)
        if rc:
            raise ffn.FfnError(rc, "ffn_fp8_forward")

    def dual(i):
        g, u, _ = refs[i % nc]
        rc = lib.ffn_fp8_dual_gemv(xp, M, K, N, g, u, gp, upp, sh)
        if rc:
            raise ffn.FfnError(rc, "ffn_fp8_dual_gemv")

    outs = []
    for i in range(nc):
        step(i)
        outs.append(out.clone())
    torch.cuda.synchronize()
    assert all(torch.equal(o, outs[0]) for o in outs), "weight copies disagree"
    if args.calibrate_copy:
        calibration_copy(dev)

    def timed(fn, n):
        return timed_ms(fn, n, stream, args.warmup)

    ms_total = timed(step, args.steps)
    ms_per_step = ms_total / args.steps
    us = ms_per_step * 1e3
    gbs = nbytes["forward"] / (us * 1e-6) / 1e9
    nk = min(args.steps, 1000)
    dual_us = timed(dual, nk) / nk * 1e3
    dual_gbs = nbytes["dual_f32"] / (dual_us * 1e-6) / 1e9
    log(f"[bench] {args.workload}: {us:.2f} us/forward, {gbs:.1f} GB/s algorithmic "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f}); dual GEMV {dual_us:.2f} us, {dual_gbs:.1f} GB/s")
    traffic = measured_traffic(args.workload)
    result = {
        "metric": FP8_METRIC, "value": round(gbs, 2), "unit": "GB/s", "us_per_forward": round(us, 3),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{case.name}: gated FFN forward, M={M}, hidden K={K}, intermediate N={N}, "
                               f"act={fi.ACT_NAMES[act]}, block-scaled FP8 weights rotated over {nc} copies",
                   "M": M, "K": K, "N": N, "act": fi.ACT_NAMES[act],
                   "algorithmic_bytes_per_forward": nbytes["forward"]},
        "roofline": {"kernel": "FP8 dual gate+up GEMV (ffn_fp8_dual_gemv entry point: fp8_gemv_kernel, gate and "
                               "up fp32 out)",
                     "bound": "hbm", "achieved": round(dual_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dual_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic["bytes"]),
                     "us_per_launch": round(dual_us, 3), "algorithmic_bytes_per_launch": nbytes["dual_f32"]},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = fp8_cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bench_w4a4(args):
    import numpy as np
    import torch

    import ffn_inputs as fi
    import w4a16_nvfp4_dense_amd as ffn

    lib = ffn.load()
    M, fp4 = W4A4_WORKLOADS[args.workload]
    case = fi.make_config(4, M=M)
    K, N, act = case.K, case.N, case.act
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copies = []
    for _ in range(args.copies):
        g, u, d = (ffn.DeviceWeight.from_host(w, dev) for w in (case.gate, case.up, case.down))
        copies.append((ffn.w4a4_prepare_weight(g), ffn.w4a4_prepare_weight(u),
                       ffn.w4a4_prepare_weight(d) if fp4 else d))
    torch.cuda.synchronize()
    structs = [(g.struct(), u.struct(), d.struct()) for g, u, d in copies]
    refs = [tuple(ctypes.byref(x) for x in st) for st in structs]
    x = ffn.bf16_from_bits(case.x_bits, dev)
    out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ws_bytes = ffn.w4a4_fp4_workspace_bytes(M, K, N) if fp4 else ffn.w4a4_workspace_bytes(M, K, N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    h_in = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gate_out = torch.empty((M, N), dtype=torch.float32, device=dev)
    up_out = torch.empty((M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    nc = len(refs)

    def step(i):
        g, u, d = refs[i % nc]
        fn = lib.ffn_w4a4_forward_fp4 if fp4 else lib.ffn_w4a4_forward
        rc = fn(x.data_ptr(), M, K, N, g, u, d, act, ws.data_ptr(), ws_bytes, out.data_ptr(), sh)
        if rc:
            raise ffn.FfnError(rc, "ffn_w4a4_forward_fp4" if fp4 else "ffn_w4a4_forward")

    def down4(i):
        _, _, d = refs[i % nc]
        rc = lib.ffn_w4a4_down_gemm(h_in.data_ptr(), M, N, K, d, out.data_ptr(), ws.data_ptr(), ws_bytes, sh)
        if rc:
            raise ffn.FfnError(rc, "ffn_w4a4_down_gemm")

    def dual(i):
        g, u, _ = refs[i % nc]
        rc = lib.ffn_w4a4_dual_gemm(x.data_ptr(), M, K, N, g, u, gate_out.data_ptr(), up_out.data_ptr(),
                                    ws.data_ptr(), ws_bytes, sh)
        if rc:
            raise ffn.FfnError(rc, "ffn_w4a4_dual_gemm")

    outs = []
    for i in range(nc):
        step(i)
        outs.append(out.clone())
    torch.cuda.synchronize()
    assert all(torch.equal(o, outs[0]) for o in outs), "weight copies disagree"
    if args.calibrate_copy:
        calibration_copy(dev)

    def timed(fn, n):
        return timed_ms(fn, n, stream, args.warmup)

    steps = min(args.steps, 500)
    ms_per_step = timed(step, steps) / steps
    us = ms_per_step * 1e3
    flops = 2.0 * 3 * M * K * N
    tflops = flops / (us * 1e-6) / 1e12
    dual_us = timed(dual, steps) / steps * 1e3
    down_us = None
    if fp4:
        h_in.copy_(ffn.bf16_from_bits(fi.f32_to_bf16_bits(np.random.default_rng(5).normal(
            size=(M, N)).astype(np.float32)), dev))
        down_us = timed(down4, steps) / steps * 1e3
    dual_flops = 2.0 * 2 * M * K * N
    dual_tflops = dual_flops / (dual_us * 1e-6) / 1e12
    # the dual entry's bytes: both MXFP4 weights (codes + E8M0 per 32), x in
    # bf16, fp32 gate and up out
    dual_bytes = 2 * N * K // 2 + 2 * N * K // 32 + 2 * M * K + 8 * M * N
    dual_gbs = dual_bytes / (dual_us * 1e-6) / 1e9
    bound = roofline_bound(dual_flops, dual_bytes, MFMA_FP4_PEAK_TFLOPS)
    traffic = measured_traffic("w4a4_prefill_silu_m128")  # the same dual entry in both workloads
    log(f"[bench] {args.workload}: {us:.2f} us/forward, {tflops:.1f} TFLOP/s; W4A4 dual GEMM (with the activation "
        f"quantisation) {dual_us:.2f} us, {dual_tflops:.1f} TFLOP/s ({100 * dual_tflops / MFMA_FP4_PEAK_TFLOPS:.1f}% "
        f"of the FP4 peak)")
    if fp4:
        down_bytes = K * N // 2 + K * N // 32 + 2 * M * N + 2 * M * K
        log(f"[bench] W4A4 down GEMM entry (with the quantisation of h): {down_us:.2f} us, "
            f"{2.0 * M * K * N / (down_us * 1e-6) / 1e12:.1f} TFLOP/s, {down_bytes / (down_us * 1e-6) / 1e9:.1f} GB/s")
    down_desc = "MXFP4 down requantised from NVFP4, h quantised to MXFP4" if fp4 else "NVFP4 down"
    result = {
        "metric": W4A4_FP4_METRIC if fp4 else W4A4_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s",
        "us_per_forward": round(us, 3),
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4" if fp4 else "fp4 (gate/up), bf16 (down)",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: gated FFN forward, M={M}, hidden K={K}, intermediate N={N}, "
                               f"act={fi.ACT_NAMES[act]}, MXFP4 gate/up requantised from NVFP4, {down_desc}, "
                               f"rotated over {nc} copies",
                   "M": M, "K": K, "N": N, "act": fi.ACT_NAMES[act], "flops_per_forward": flops},
        "roofline": {"kernel": "W4A4 dual GEMM entry (ffn_w4a4_dual_gemm: mx_quant_bf16_kernel + w4a4_gemm_kernel, "
                               "fp32 gate and up out)",
                     "bound": bound,
                     "achieved": round(dual_gbs if bound == "hbm" else dual_tflops, 2),
                     "peak": HBM_PEAK_GBS if bound == "hbm" else MFMA_FP4_PEAK_TFLOPS,
                     "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                     "frac": round(dual_gbs / HBM_PEAK_GBS if bound == "hbm" else dual_tflops / MFMA_FP4_PEAK_TFLOPS,
                                   4),
                     "traffic": None if traffic is None else round(traffic["bytes"]),
                     "us_per_launch": round(dual_us, 3), "flops_per_launch": dual_flops,
                     "algorithmic_bytes_per_launch": dual_bytes,
                     "intensity_flop_per_byte": round(dual_flops / dual_bytes, 1),
                     "tflops": round(dual_tflops, 2),
                     "frac_of_fp4_peak": round(dual_tflops / MFMA_FP4_PEAK_TFLOPS, 4)},
    }
    if fp4:
        result["down_gemm_us"] = round(down_us, 3)
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        gm, um = orc.mx_requant(case.gate), orc.mx_requant(case.up)
        dm = orc.mx_requant(case.down) if fp4 else None
        rows = np.array([0])
        sub = case.with_x(case.x_bits[rows])
        one = (lambda: orc.w4a4_ffn_fp4(sub, gm, um, dm)) if fp4 else (lambda: orc.w4a4_ffn(sub, gm, um))
        one()
        n = 0
        t0 = time.perf_counter()
        while True:
            one()
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        row_flops = 2.0 * 3 * K * N
        result["cpu_baseline"] = {"value": round(n * row_flops / el / 1e12, 6), "unit": "TFLOP/s",
                                  "us_per_token_row": round(el / n * 1e6, 1), "cores": orc.num_threads(),
                                  "kind": "oracle",
                                  "sample": f"{n} single-token-row {'all-4-bit ' if fp4 else ''}W4A4 forwards of the same "
                                            f"weights (fp64 C oracle, "
                                            f"OpenMP over outputs), {el:.1f} s"}
    print(json.dumps(result), flush=True)


def quant_bytes(rows, cols):
    """Bytes the two passes must move: the bf16 weight read by the absmax pass
    and again by the quantise pass, then the codes, scale bytes and scale2."""
    n = rows * cols
    return 2 * (2 * n) + n // 2 + n // 16 + 4


def bench_quantize(args):
    import torch
    import ffn_inputs as fi
    import w4a16_nvfp4_dense_amd as ffn

    lib = ffn.load()
    rows, cols = QUANT_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bits = fi.make_dense_bf16(rows, cols, 1)
    # byte-identical copies rotated over, so the Infinity Cache cannot serve repeats
    ws_in = [ffn.bf16_from_bits(bits, dev) for _ in range(args.copies)]
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    s2 = torch.empty(1, dtype=torch.float32, device=dev)
    wsb = ffn.quantize_workspace_bytes(rows, cols)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    q = lib.ffn_nvfp4_quantize
    ptrs = [w.data_ptr() for w in ws_in]
    cp, sp, s2p, wp = codes.data_ptr(), scales.data_ptr(), s2.data_ptr(), ws.data_ptr()
    nc = len(ptrs)

    def step(i):
        rc = q(ptrs[i % nc], rows, cols, cp, sp, s2p, wp, wsb, sh)
        if rc:
            raise ffn.FfnError(rc, "ffn_nvfp4_quantize")

    outs = []
    for i in range(nc):
        step(i)
        outs.append((codes.clone(), scales.clone(), s2.clone()))
    torch.cuda.synchronize()
    assert all(all(torch.equal(a, b) for a, b in zip(o, outs[0])) for o in outs), "input copies disagree"
    if args.calibrate_copy:
        calibration_copy(dev)
    steps = min(args.steps, 1000)
    t0 = time.perf_counter()
    ms_per_step = timed_ms(step, steps, stream, args.warmup) / steps
    wall = time.perf_counter() - t0
    us = ms_per_step * 1e3
    nbytes = quant_bytes(rows, cols)
    gbs = nbytes / (us * 1e-6) / 1e9
    traffic = measured_traffic(args.workload, "quantize")
    if traffic is not None:
        log(f"[bench] measured HBM traffic of both passes: {traffic['bytes'] / 1e6:.2f} MB per quantise "
            f"({traffic['bytes'] / nbytes:.4f} x algorithmic)")
    log(f"[bench] {args.workload}: {us:.2f} us/quantise, {gbs:.1f} GB/s algorithmic "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f}); host wall {wall * 1e3 / steps * 1e3:.2f} us/step")
    result = {
        "metric": QUANT_METRIC, "value": round(gbs, 2), "unit": "GB/s", "us_per_quantise": round(us, 3),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.workload}: BF16 weight [{rows}, {cols}] (normal values, per-row factors "
                               f"e^U[-4,2]) to NVFP4, inputs rotated over {nc} copies",
                   "rows": rows, "cols": cols, "algorithmic_bytes_per_quantise": nbytes},
        "roofline": {"kernel": "whole quantise (absmax pass + quantise pass)", "bound": "hbm",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic["bytes"]), "us_per_launch": round(us, 3),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
        n = 0
        tq = time.perf_counter()
        while True:
            orc.quantize(bits)
            n += 1
            el = time.perf_counter() - tq
            if el >= args.cpu_seconds:
                break
        cus = el / n * 1e6
        result["cpu_baseline"] = {"value": round(nbytes / (cus * 1e-6) / 1e9, 3), "unit": "GB/s",
                                  "us_per_quantise": round(cus, 1), "cores": 1, "kind": "oracle",
                                  "sample": f"{n} full quantises of the same weight (C oracle, one thread), "
                                            f"{el:.1f} s"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_silu_m1",
                    choices=sorted(WORKLOADS) + sorted(QUANT_WORKLOADS) + sorted(FP8_WORKLOADS)
                    + sorted(W4A4_WORKLOADS))
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated over")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="time the forward and the roofline kernel only (no trial median, read-ceiling or graph "
                         "legs): for runs under a profiler")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 64 MiB device-to-device copy (untimed), the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import ffn_inputs as fi
    import w4a16_nvfp4_dense_amd as ffn

    if args.workload in QUANT_WORKLOADS:
        bench_quantize(args)
        return
    if args.workload in FP8_WORKLOADS:
        bench_fp8(args)
        return
    if args.workload in W4A4_WORKLOADS:
        bench_w4a4(args)
        return
    bench_nvfp4(args)


def packed_weights(case, dev):
    """One weight copy as a single device allocation: the codes and scales of
    W_g, W_u and W_d back to back (each piece 256-byte aligned), so that the
    bytes a forward streams are one contiguous range (W_g and W_u first) that
    the read-ceiling leg can stream the same way. Returns (buffer, gate, up,
    down) with DeviceWeights viewing into the buffer."""
    import numpy as np
    import torch
    import w4a16_nvfp4_dense_amd as ffn

    pieces = []
    for w in (case.gate, case.up, case.down):
        pieces += [w.codes, w.scales]
    offs, at = [], 0
    for a in pieces:
        offs.append(at)
        at = (at + a.nbytes + 255) // 256 * 256
    host = np.zeros(at, dtype=np.uint8)
    for a, o in zip(pieces, offs):
        host[o:o + a.nbytes] = np.ascontiguousarray(a).reshape(-1)
    buf = torch.from_numpy(host).to(dev)
    views = [buf[o:o + a.nbytes].view(a.shape) for a, o in zip(pieces, offs)]
    ws = [ffn.DeviceWeight(views[2 * i], views[2 * i + 1], float(w.scale2))
          for i, w in enumerate((case.gate, case.up, case.down))]
    return buf, ws[0], ws[1], ws[2], offs[4]


def single_thread_oracle_us(trials=5):
    """Median over `trials` runs of one full forward of the oracle on one
    thread, for the tiny, decode SwiGLU and decode GELU-tanh configs."""
    import statistics
    import ffn_inputs as fi
    import oracle

    orc = oracle.default()
    threads = orc.num_threads()
    orc.set_num_threads(1)
    out = {}
    try:
        for idx in (0, 1, 2):
            case = fi.make_config(idx)
            ts = []
            for _ in range(trials):
                t0 = time.perf_counter()
                orc.ffn(case)
                ts.append((time.perf_counter() - t0) * 1e6)
            out[case.name] = round(statistics.median(ts), 1)
    finally:
        orc.set_num_threads(threads)
    return out


def bench_nvfp4(args):
    import statistics

    import torch

    import ffn_inputs as fi
    import w4a16_nvfp4_dense_amd as ffn

    lib = ffn.load()
    idx, M = WORKLOADS[args.workload]
    case = fi.make_config(idx, M=M) if idx in (3, 4) else fi.make_config(idx)
    K, N = case.K, case.N
    nbytes = algorithmic_bytes(M, K, N)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    copies, bufs = [], []
    for _ in range(args.copies):
        buf, g, u, d, down_at = packed_weights(case, dev)
        copies.append((g, u, d))
        bufs.append((buf, down_at))
    x = ffn.bf16_from_bits(case.x_bits, dev)
    out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    ws_bytes = ffn.workspace_bytes(M, K, N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    gate_out = torch.empty((M, N), dtype=torch.float32, device=dev)
    up_out = torch.empty((M, N), dtype=torch.float32, device=dev)
    structs = [(g.struct(), u.struct(), d.struct()) for g, u, d in copies]
    refs = [(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d)) for g, u, d in structs]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    xp, op, wp = x.data_ptr(), out.data_ptr(), ws.data_ptr()
    gp, upp = gate_out.data_ptr(), up_out.data_ptr()
    fwd = lib.ffn_nvfp4_forward
    dual = lib.ffn_nvfp4_dual_gemv
    act = case.act
    nc = len(refs)

    def step(i, handle=None):
        g, u, d = refs[i % nc]
        rc = fwd(xp, M, K, N, g, u, d, act, wp, ws_bytes, op, sh if handle is None else handle)
        if rc:
            raise ffn.FfnError(rc, "ffn_nvfp4_forward")

    def dual_step(i):
        g, u, _ = refs[i % nc]
        rc = dual(xp, M, K, N, g, u, gp, upp, sh)
        if rc:
            raise ffn.FfnError(rc, "ffn_nvfp4_dual_gemv")

    # copies are byte-identical, so every copy must give the same output
    outs = []
    for i in range(nc):
        step(i)
        outs.append(out.clone())
    torch.cuda.synchronize()
    assert all(torch.equal(o, outs[0]) for o in outs), "weight copies disagree"

    if args.calibrate_copy:
        calibration_copy(dev)

    # The timed region: W warmup forwards, then exactly K forwards.
    t0 = time.perf_counter()
    ms_total = timed_ms(step, args.steps, stream, args.warmup)
    wall = time.perf_counter() - t0
    ms_per_step = ms_total / args.steps
    us = ms_per_step * 1e3
    gbs = nbytes["forward"] / (us * 1e-6) / 1e9
    log(f"[bench] {args.workload}: {us:.2f} us/forward, {gbs:.1f} GB/s algorithmic "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f}); host wall {wall * 1e6 / args.steps:.2f} us/step")
    # Context: five more trials of 200 forwards each, median.
    trials = [] if args.profile_run else [timed_ms(step, 200, stream) / 200 * 1e3 for _ in range(5)]
    us_med5 = statistics.median(trials) if trials else None
    if trials:
        log(f"[bench] 5 trials of 200 forwards: median {us_med5:.2f} us (" +
            ", ".join(f"{t:.2f}" for t in trials) + ")")

    result = {
        # the headline metric names its workload (decode SwiGLU M = 1); the
        # other workloads name theirs
        "metric": METRIC if args.workload == "decode_silu_m1" else
        METRIC.replace("SwiGLU decode M=1", f"{'SwiGLU' if act == fi.ACT_SILU else 'GELU-tanh'} {args.workload}"),
        "value": round(gbs, 2),
        "unit": "GB/s",
        "us_per_forward": round(us, 3),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{case.name}: gated FFN forward, M={M}, hidden K={K}, intermediate N={N}, "
                        f"act={fi.ACT_NAMES[act]}, NVFP4 weights rotated over {nc} copies",
            "M": M, "K": K, "N": N, "act": fi.ACT_NAMES[act],
            "algorithmic_bytes_per_forward": nbytes["forward"],
        },
        "us_per_forward_median5": None if us_med5 is None else round(us_med5, 3),
        "us_per_forward_trials": [round(t, 3) for t in trials],
    }

    if M > 16:
        # Matrix-core arms beyond one token group: the roofline is the whole
        # forward (its kernels are not all reachable through the dual entry),
        # against HBM or the bf16 MFMA peak, whichever its arithmetic
        # intensity (three [M, K] x [K, N]-sized products over the forward's
        # bytes) makes the bound.
        flops = 2.0 * 3 * M * K * N
        tflops = flops / (us * 1e-6) / 1e12
        bound = roofline_bound(flops, nbytes["forward"], MFMA_BF16_PEAK_TFLOPS)
        arm = "small-batch GEMMs" if M <= SMALL_BATCH_MAX_M else "128-row GEMMs"
        log(f"[bench] {args.workload}: {tflops:.1f} TFLOP/s ({100 * tflops / MFMA_BF16_PEAK_TFLOPS:.1f}% of "
            f"{MFMA_BF16_PEAK_TFLOPS:.0f}); bound by {bound}")
        traffic = measured_traffic(args.workload, "forward")
        if traffic is not None:
            log(f"[bench] measured HBM traffic of the forward's kernels: {traffic['bytes'] / 1e6:.2f} MB per forward "
                f"({traffic['bytes'] / nbytes['forward']:.4f} x algorithmic)")
        result["roofline"] = {
            "kernel": f"whole forward ({arm}: dual GEMM + down GEMM on bf16 matrix cores)",
            "bound": bound,
            "achieved": round(gbs if bound == "hbm" else tflops, 2),
            "peak": HBM_PEAK_GBS if bound == "hbm" else MFMA_BF16_PEAK_TFLOPS,
            "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
            "frac": round(gbs / HBM_PEAK_GBS if bound == "hbm" else tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None if traffic is None else round(traffic["bytes"]), "flops_per_forward": flops,
            "tflops": round(tflops, 2),
            "intensity_flop_per_byte": round(flops / nbytes["forward"], 1)}
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return

    # Dominant kernel: the dual GEMV (GEMM for the small-batch arm), timed
    # with events on its stream around a batch of back-to-back launches
    # (rotating the weight copies).
    nk = min(args.steps, 1000)
    dual_us = timed_ms(dual_step, nk, stream, args.warmup) / nk * 1e3
    dual_gbs = nbytes["dual_f32"] / (dual_us * 1e-6) / 1e9
    log(f"[bench] dual {'GEMV' if M <= 8 else 'GEMM'}: {dual_us:.2f} us/launch, {dual_gbs:.1f} GB/s")
    traffic = measured_traffic(args.workload)
    if traffic is not None:
        log(f"[bench] measured HBM traffic of the dual GEMV: {traffic['bytes'] / 1e6:.2f} MB per launch "
            f"({traffic['bytes'] / nbytes['dual_f32']:.4f} x algorithmic)")
    result["roofline"] = {
        "kernel": ("dual gate+up GEMV (ffn_nvfp4_dual_gemv entry point: wave_gemv_kernel, gate and up fp32 out)"
                   if M <= 8 else
                   "dual gate+up GEMM (ffn_nvfp4_dual_gemv entry point: smallm_gemm_kernel, gate and up fp32 out)"),
        "bound": "hbm",
        "achieved": round(dual_gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(dual_gbs / HBM_PEAK_GBS, 4),
        "traffic": None if traffic is None else round(traffic["bytes"]),
        "us_per_launch": round(dual_us, 3),
        "algorithmic_bytes_per_launch": nbytes["dual_f32"],
    }

    if args.profile_run:
        print(json.dumps(result), flush=True)
        return

    # Streaming-read ceiling (context, not `value`): a trivial kernel with the
    # GEMVs' load width reading the same weight bytes (each copy is one
    # contiguous range), as one launch over all three weights and as two
    # launches (W_g + W_u, then W_d), rotating copies.
    one = [ffn.DiagRead([buf]) for buf, _ in bufs]
    two = [(ffn.DiagRead([buf[:at]]), ffn.DiagRead([buf[at:]])) for buf, at in bufs]
    r1 = timed_ms(lambda i: one[i % nc].launch(stream), 200, stream, 20) / 200 * 1e3

    def two_step(i):
        a, b = two[i % nc]
        a.launch(stream)
        b.launch(stream)

    r2 = timed_ms(two_step, 200, stream, 20) / 200 * 1e3
    rd = timed_ms(lambda i: two[i % nc][0].launch(stream), 200, stream, 20) / 200 * 1e3
    wbytes = one[0].bytes
    log(f"[bench] read ceiling of the {wbytes / 1e6:.1f} MB of weights: one launch {r1:.2f} us "
        f"({wbytes / r1 / 1e3:.1f} GB/s), two launches {r2:.2f} us; the dual GEMV's bytes alone {rd:.2f} us")
    result["read_ceiling"] = {
        "weight_bytes": wbytes,
        "one_launch_us": round(r1, 3), "one_launch_GBs": round(wbytes / r1 / 1e3, 1),
        "two_launch_us": round(r2, 3), "dual_bytes_us": round(rd, 3),
        "forward_frac_of_one_launch": round(r1 / us, 4),
        "forward_frac_of_two_launch": round(r2 / us, 4),
        "dual_frac_of_its_read": round(rd / dual_us, 4),
    }

    if M <= 8:
        # The same forwards replayed from a HIP graph (one capture of one
        # forward per weight copy), checked against the eager output.
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(nc):
                step(i, side.cuda_stream)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for i in range(nc):
                step(i, cap)
        torch.cuda.synchronize()
        out.zero_()
        reps = max(1, 200 // nc)
        g_ms = timed_ms(lambda i: graph.replay(), reps, stream, 5)
        graph_us = g_ms / (reps * nc) * 1e3
        assert torch.equal(out, outs[0]), "graph replay disagrees with the eager forward"
        log(f"[bench] HIP graph replay: {graph_us:.2f} us/forward")
        result["graph_us_per_forward"] = round(graph_us, 3)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
        if args.workload == "decode_silu_m1":
            result["cpu_baseline"]["single_thread_us_median5"] = single_thread_oracle_us()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
