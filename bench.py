"""Benchmark of the NVFP4 W4A4 linear hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input: run-time
NVFP4 quantization of the bf16 activations under the calibrated input scale, then the
block-scaled W4A4 GEMM with bf16 output (the fused linear). Weights are quantized
offline and the global scales calibrated before the timed region, as a deployed layer
does. Inputs are resident in HBM when timing starts.

Prints one JSON line (rank 0) with the step throughput in TFLOP/s (2*M*N*K per step),
the dominant kernel's roofline (GEMM vs the f16 dense MFMA peak), the quantize kernel's
HBM bandwidth on rotated buffers (for the workload's activation and for a large
4608 x 12288 activation), context rows (the GEMM at every M = 4608 FLUX shape and a
4-image batch, short activations, hipBLASLt bf16 at the same shape, the MXFP8, rowwise
FP8 and W4A16 paths) and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload attn_out] [--gpus 1]
                    [--no-context] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s + % MFMA peak at FLUX shapes; quantize GB/s % HBM peak"
PEAK_F16_TFLOPS = 2516.6  # MI355X dense f16/bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
QUANT_BYTES_PER_ELEM = 2.5625  # 2 B bf16 in + 0.5 B codes + 1/16 B scale out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock ramps for tens of milliseconds after idle: the first 50 attn_out steps
    # average ~45% longer than the steady state reached after ~500 steps, so the default
    # warm-up runs well past that before the timed steps.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="attn_out")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context rows (other shapes, hipBLASLt, MXFP8, fp8r, W4A16)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--rotate-mb", type=int, default=1024,
                    help="bytes of rotated activation buffers for the quantize bandwidth leg")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run 3 plain device copies of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    return ap.parse_args()


KERNEL_SOURCES = ["gemm.hip", "gemm_common.hpp", "kernels.hpp", "quantize.hip", "quant_common.hpp",
                  "codec.hpp"]
PEAK_FP8_TFLOPS = 5033.2  # MI355X dense fp8 MFMA


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "nvfp4_block_scaled_02_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per GEMM launch from the committed counter summary, if it was taken
    on the current kernel sources for this workload (else None)."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, d, ags, wgs, seconds):
    """The oracle as it stands on the workload's activation rows, full weights: chunks of
    rows in order (wrapping round to row 0 after the last) until about `seconds` of CPU
    work; scaled to TFLOP/s of the same 2*rows*N*K count."""
    import numpy as np

    from oracle import nvfp4_oracle as O

    try:
        from threadpoolctl import threadpool_info

        blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max(blas) if blas else 1
    except Exception:  # threadpoolctl missing: report the affinity size
        cores = len(os.sched_getaffinity(0))
    wp, ws = O.quantize(d["w"], wgs)  # offline weight quantization, not timed
    rows_done, t_total, chunk, r0 = 0, 0.0, 64, 0
    while t_total < seconds:
        r1 = min(wl.M, r0 + chunk)
        t0 = time.perf_counter()
        ap, as_ = O.quantize(d["x"][r0:r1], ags)
        O.gemm_ref(ap, as_, ags, wp, ws, wgs, with_abs=False)
        t_total += time.perf_counter() - t0
        rows_done += r1 - r0
        r0 = 0 if r1 == wl.M else r1
        chunk = min(chunk * 2, 1024)
    flops = 2.0 * rows_done * wl.N * wl.K
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{rows_done} activation rows ({rows_done / wl.M:.2f} passes over the {wl.M} rows) "
                  f"x full [{wl.N}x{wl.K}] weights: NumPy quantize (1 thread) + float64 GEMM "
                  f"reference ({cores} BLAS threads), {t_total:.1f} s",
    }


def time_launches(fn, n, stream):
    """Average ms of n back-to-back launches of fn on `stream` (HIP events on that
    stream), after 3 untimed ones."""
    import torch

    for _ in range(3):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def context_legs(nv, lib, stream, n):
    """Context rows (not the metric): every M = 4608 FLUX linear of the workload set, short
    activations, hipBLASLt bf16 at the metric's shape, and the MXFP8, rowwise FP8 and W4A16
    paths.
    Operands are device-generated N(0, 1) activations and N(0, 0.02) weights, quantized
    by the library; GEMM times are warm (operands resident)."""
    import torch

    from workloads import make

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(7)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    out = {"gemm": {}, "short_activations": {}}

    def operands(M, N, K):
        x = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
        w = (torch.randn((N, K), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
        ags, wgs = nv.calibrate(x), nv.calibrate(w)
        ap, as_ = nv.quantize(x, ags)
        wp, ws = nv.quantize(w, wgs)
        return x, w, ags, wgs, ap, as_, wp, ws

    def nvfp4_gemm_ms(M, N, K, ops):
        _, _, ags, wgs, ap, as_, wp, ws = ops
        o = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        args = (P(ap), P(as_), ctypes.c_float(ags), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(o), sp)
        return time_launches(lambda: lib.nvfp4_gemm(*args), n, stream)

    for name in ["attn_out", "mlp_up_static", "qkv", "mlp_down", "batch4_up"]:
        wl = make(name)
        M, N, K = wl.M, wl.N, wl.K
        ops = operands(M, N, K)
        ms = nvfp4_gemm_ms(M, N, K, ops)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out["gemm"][name] = {"M": M, "N": N, "K": K, "kernel": nv.gemm_plan(M, N, K),
                             "avg_ms": round(ms, 5), "TFLOP/s": round(tf, 1),
                             "frac_f16_peak": round(tf / PEAK_F16_TFLOPS, 4)}
        if name == "attn_out":
            x, w, ags, wgs, ap, as_, wp, ws = ops
            # hipBLASLt bf16 GEMM of the unquantized operands at the same shape
            wt = w.t().contiguous()
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ms_b = time_launches(lambda: torch.matmul(x, wt, out=y), n, stream)
            out["hipblaslt_bf16_matmul"] = {"shape": [M, N, K], "avg_ms": round(ms_b, 5),
                                            "TFLOP/s": round(2.0 * M * N * K / (ms_b * 1e-3) / 1e12, 1)}
            # MXFP8 path (E4M3 elements, E8M0 scales per 32) on the same operands
            ac, asx = nv.mxfp8_quantize(x)
            wc, wsx = nv.mxfp8_quantize(w)
            y8 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            a8 = (P(ac), P(asx), P(wc), P(wsx), M, N, K, P(y8), sp)
            ms8 = time_launches(lambda: lib.nvfp4_mxfp8_gemm(*a8), n, stream)
            q8 = (P(x), M, K, P(ac), P(asx), sp)
            msq8 = time_launches(lambda: lib.nvfp4_mxfp8_quantize(*q8), n, stream)
            tf8 = 2.0 * M * N * K / (ms8 * 1e-3) / 1e12
            out["mxfp8"] = {"shape": [M, N, K], "gemm_avg_ms": round(ms8, 5), "gemm_TFLOP/s": round(tf8, 1),
                            "frac_fp8_peak": round(tf8 / PEAK_FP8_TFLOPS, 4),
                            "quantize_avg_ms_warm": round(msq8, 5),
                            "quantize_GB/s_warm": round((2 + 1 + 1 / 32) * M * K / (msq8 * 1e-3) / 1e9, 1)}
            # rowwise FP8 (fp8r): E4M3 with one fp32 scale per row, unit-scaled fp8 MFMA
            rc, rs = nv.fp8r_quantize(x)
            wrc, wrs = nv.fp8r_quantize(w)
            yr = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ar = (P(rc), P(rs), P(wrc), P(wrs), M, N, K, P(yr), sp)
            msr = time_launches(lambda: lib.nvfp4_fp8r_gemm(*ar), n, stream)
            qr = (P(x), M, K, P(rc), P(rs), sp)
            msqr = time_launches(lambda: lib.nvfp4_fp8r_quantize(*qr), n, stream)
            tfr = 2.0 * M * N * K / (msr * 1e-3) / 1e12
            out["fp8r"] = {"shape": [M, N, K], "gemm_avg_ms": round(msr, 5), "gemm_TFLOP/s": round(tfr, 1),
                           "frac_fp8_peak": round(tfr / PEAK_FP8_TFLOPS, 4),
                           "quantize_avg_ms_warm": round(msqr, 5),
                           "quantize_GB/s_warm": round((3 * M * K + 4 * M) / (msqr * 1e-3) / 1e9, 1)}
            del rc, rs, wrc, wrs, yr
            # W4A16: NVFP4 weights, bf16 activations
            y16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            a16 = (P(x), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y16), sp)
            ms16 = time_launches(lambda: lib.nvfp4_gemm_w4a16(*a16), n, stream)
            out["w4a16"] = {"shape": [M, N, K], "avg_ms": round(ms16, 5),
                            "TFLOP/s": round(2.0 * M * N * K / (ms16 * 1e-3) / 1e12, 1)}
            del x, w, wt, y, ac, asx, wc, wsx, y8, y16
        del ops
    # short activations: the weights dominate the bytes (K/2 + K/16 bytes per weight row)
    N, K = 3072, 3072
    w = (torch.randn((N, K), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    wgs = nv.calibrate(w)
    wp, ws = nv.quantize(w, wgs)
    for M in (1, 17, 256, 1000):
        x = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
        ags = nv.calibrate(x)
        ap, as_ = nv.quantize(x, ags)
        ms = nvfp4_gemm_ms(M, N, K, (x, w, ags, wgs, ap, as_, wp, ws))
        y16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        a16 = (P(x), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y16), sp)
        ms16 = time_launches(lambda: lib.nvfp4_gemm_w4a16(*a16), n, stream)
        # the whole linear (quantize + GEMM, one fused kernel where the plan says so)
        nb = nv.linear_workspace_bytes(M, K)
        work = torch.empty(nb, dtype=torch.uint8, device=dev)
        al = (P(x), ctypes.c_float(ags), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y16),
              P(work), ctypes.c_size_t(nb), sp)
        msl = time_launches(lambda: lib.nvfp4_linear(*al), n, stream)
        wbytes = N * (K // 2 + K // 16)
        out["short_activations"][f"M={M}"] = {
            "N": N, "K": K, "kernel": nv.gemm_plan(M, N, K), "w4a4_avg_ms": round(ms, 5),
            "w4a4_weight_GB/s": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "linear": nv.linear_plan(M, N, K), "linear_avg_ms": round(msl, 5),
            "w4a16_avg_ms": round(ms16, 5),
            "TFLOP/s": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 2)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   f"--gpus {args.gpus} is not supported"}))
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_block_scaled_02_amd as nv
    from workloads import make

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    lib = nv.load_library()
    dev = torch.device("cuda:0")
    wl = make(args.workload)
    M, N, K = wl.M, wl.N, wl.K
    d = wl.generate()

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x = to_dev(d["x"])
    w = to_dev(d["w"])
    # offline: weight global scale + weight quantization; activation input scale
    wgs = nv.calibrate(w)
    wq, wsc = nv.quantize(w, wgs)
    ags = nv.calibrate(to_dev(d["calib"])) if "calib" in d else nv.calibrate(x)
    del w
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    work = torch.empty(nv.linear_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    qp, qs = nv.workspace_views(work, M, K)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    xa, qpa, qsa, wqa, wsa, oa = P(x), P(qp), P(qs), P(wq), P(wsc), P(out)
    f_ags, f_wgs = ctypes.c_float(ags), ctypes.c_float(wgs)

    def step():
        s1 = lib.nvfp4_quantize(xa, M, K, f_ags, qpa, qsa, sp)
        s2 = lib.nvfp4_gemm(qpa, qsa, f_ags, wqa, wsa, f_wgs, M, N, K, oa, sp)
        if s1 or s2:
            raise RuntimeError(f"status {s1} {s2}")

    # untimed warm-up; its first 50 steps are timed separately to show the clock ramp
    n_first = min(50, args.warmup)
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for i in range(args.warmup):
        step()
        if i + 1 == n_first:
            w1.record(stream)
    torch.cuda.synchronize()
    first_ms = w0.elapsed_time(w1) / n_first if n_first else None

    # Timed region 1: K whole steps (quantize + GEMM), events only at its two ends.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12

    # Timed region 2: the dominant kernel alone, K back-to-back launches on the same
    # stream (its average launch duration, for the roofline).
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    for _ in range(args.steps):
        if lib.nvfp4_gemm(qpa, qsa, f_ags, wqa, wsa, f_wgs, M, N, K, oa, sp):
            raise RuntimeError("gemm failed")
    g1.record(stream)
    torch.cuda.synchronize()
    g_ms = g0.elapsed_time(g1) / args.steps
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12

    # quantize bandwidth on rotated buffers (beyond the 256 MB Infinity Cache)
    n_rot = max(2, int(args.rotate_mb * 2**20 // (M * K * 2)))
    xs = [x] + [x.clone() for _ in range(n_rot - 1)]
    outs = [(torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
             torch.empty((M, K // 16), dtype=torch.uint8, device=dev)) for _ in range(n_rot)]
    ptrs = [(P(a), P(b), P(c)) for a, (b, c) in zip(xs, outs)]
    for i in range(n_rot):
        lib.nvfp4_quantize(ptrs[i][0], M, K, f_ags, ptrs[i][1], ptrs[i][2], sp)
    qa, qb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_q = max(args.steps, 4 * n_rot)
    torch.cuda.synchronize()
    qa.record(stream)
    for i in range(n_q):
        a, b, c = ptrs[i % n_rot]
        lib.nvfp4_quantize(a, M, K, f_ags, b, c, sp)
    qb.record(stream)
    torch.cuda.synchronize()
    q_rot_ms = qa.elapsed_time(qb) / n_q
    q_gbs = QUANT_BYTES_PER_ELEM * M * K / (q_rot_ms * 1e-3) / 1e9
    del xs, outs

    # quantize bandwidth on a large activation (the 4608 x 12288 input of a FLUX MLP down
    # projection), rotated the same way
    LM, LK = 4608, 12288
    n_rot_l = max(2, int(args.rotate_mb * 2**20 // (LM * LK * 2)))
    gen = torch.Generator(device=dev).manual_seed(5)
    xl = [torch.randn((LM, LK), device=dev, generator=gen).to(torch.bfloat16) for _ in range(n_rot_l)]
    ol = [(torch.empty((LM, LK // 2), dtype=torch.uint8, device=dev),
           torch.empty((LM, LK // 16), dtype=torch.uint8, device=dev)) for _ in range(n_rot_l)]
    f_lgs = ctypes.c_float(nv.calibrate(xl[0]))
    pl = [(P(a), P(b), P(c)) for a, (b, c) in zip(xl, ol)]
    for i in range(n_rot_l):
        lib.nvfp4_quantize(pl[i][0], LM, LK, f_lgs, pl[i][1], pl[i][2], sp)
    n_ql = max(args.steps, 4 * n_rot_l)
    torch.cuda.synchronize()
    qa.record(stream)
    for i in range(n_ql):
        a, b, c = pl[i % n_rot_l]
        lib.nvfp4_quantize(a, LM, LK, f_lgs, b, c, sp)
    qb.record(stream)
    torch.cuda.synchronize()
    ql_ms = qa.elapsed_time(qb) / n_ql
    ql_gbs = QUANT_BYTES_PER_ELEM * LM * LK / (ql_ms * 1e-3) / 1e9
    del xl, ol

    if args.copy_calibration_mb:
        # Known-size reference for the hardware byte counters: a plain device copy of
        # N MiB whose source was evicted from the caches by a larger fill in between.
        nbytes = args.copy_calibration_mb * 2**20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        evict = torch.empty(2 * nbytes // 4, dtype=torch.float32, device=dev)
        for _ in range(3):
            evict.fill_(0.0)
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, evict

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "warmup_first_steps_ms_per_step": round(first_ms, 5) if first_ms else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: NVFP4 W4A4 linear, x bf16 [M={M}, K={K}] "
                        f"({wl.description}), W [N={N}, K={K}], bf16 out",
            "global_batch": M,
            "seq_len": None,
            "parallelism": "none (1 GPU)",
            "M": M, "N": N, "K": K,
        },
        "roofline": {
            "kernel": "nvfp4 block-scaled GEMM (f16 MFMA after exact E2M1xE4M3 decode)",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_F16_TFLOPS, 4),
            "traffic": measured_traffic(wl.name),
            "kernel_source_hash": kernel_source_hash(),
            "avg_ms": round(g_ms, 5),
        },
        "quantize": {
            "rotated_avg_ms": round(q_rot_ms, 5),
            "achieved": round(q_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(q_gbs / PEAK_HBM_GBS, 4),
            "bytes_per_launch": int(QUANT_BYTES_PER_ELEM * M * K),
            "rotated_buffers": n_rot,
            "large": {
                "shape": [LM, LK],
                "rotated_avg_ms": round(ql_ms, 5),
                "achieved": round(ql_gbs, 1),
                "frac": round(ql_gbs / PEAK_HBM_GBS, 4),
                "rotated_buffers": n_rot_l,
            },
        },
        "precision": "E2M1 x E4M3 operands decoded exactly to f16, f16 MFMA, fp32 accumulate, "
                     "bf16 output",
    }
    if not args.no_context:
        del x, qp, qs, work, out
        torch.cuda.empty_cache()
        result["context"] = context_legs(nv, lib, stream, max(10, args.steps // 2))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, d, ags, wgs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
