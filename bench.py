"""Benchmark of the NVFP4 W4A4 linear hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input: run-time
NVFP4 quantization of the bf16 activations under the calibrated input scale, then the
block-scaled W4A4 GEMM with bf16 output. Weights are quantized offline and the global
scales calibrated before the timed region, as a deployed layer does. Inputs are resident
in HBM when timing starts.

Phases, in order (the GPU clock takes tens of milliseconds to rise after idle, so the
settle phase runs by wall time, whatever --warmup says):

1. settle: whole steps until at least --settle-seconds and --settle-min-steps have
   passed (reported as its own field, with the step time of its last chunk);
2. warm-up: --warmup untimed steps;
3. timed: --steps whole steps between two HIP events on the launch stream -> `value`;
4. roofline leg: the GEMM alone, back-to-back launches on the same stream (its average
   launch duration, for the roofline against the f16 dense MFMA peak);
5. quantize bandwidth on rotated buffers (beyond the 256 MB Infinity Cache) for the three
   large activations [4608, 3072], [4608, 12288] and [18432, 3072], each beside a rotated
   device-to-device copy moving the same bytes (the copy ceiling);
6. context rows: the fused linear (quantize + GEMM) and the GEMM alone for every
   M = 4608 FLUX linear and the 4-image batch, hipBLASLt bf16 at the metric's shape, the
   MXFP8, rowwise FP8 and W4A16 paths, and short activations (for 1 and 17 rows also on
   rotated weights, read from HBM);
7. the CPU oracle timed on a bounded sample.

The GFX clock is sampled (amdsmi, its own thread) throughout and reported per leg; the
memory clock is read once at the end.

    python bench.py [--steps K] [--warmup W] [--workload attn_out] [--gpus 1]
                    [--no-context] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s + % MFMA peak at FLUX shapes; quantize GB/s % HBM peak"
PEAK_F16_TFLOPS = 2516.6  # MI355X dense f16/bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_FP8_TFLOPS = 5033.2  # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
QUANT_BYTES_PER_ELEM = 2.5625  # 2 B bf16 in + 0.5 B codes + 1/16 B scale out
QUANT_SHAPES = [(4608, 3072), (4608, 12288), (18432, 3072)]  # the large FLUX activations
LINEAR_WORKLOADS = ["attn_out", "mlp_up_static", "qkv", "mlp_down", "batch4_up"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-seconds", type=float, default=1.5,
                    help="wall time of whole steps run before the warm-up (clock ramp)")
    ap.add_argument("--settle-min-steps", type=int, default=500)
    ap.add_argument("--roofline-launches", type=int, default=1000,
                    help="back-to-back GEMM launches of the roofline leg (at least --steps)")
    ap.add_argument("--workload", default="attn_out")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context rows (other shapes, hipBLASLt, MXFP8, fp8r, W4A16)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--rotate-mb", type=int, default=1024,
                    help="bytes of rotated buffers for the quantize and copy bandwidth legs")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run 3 plain device copies of this many MiB (a known-size "
                         "reference for hardware byte counters)")
    return ap.parse_args()


KERNEL_SOURCES = ["gemm.hip", "gemm_common.hpp", "kernels.hpp", "quantize.hip", "quant_common.hpp",
                  "codec.hpp"]


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


class ClockSampler:
    """Samples the GPU's GFX clock (MHz) from amdsmi every `interval` seconds on its own
    thread; `window(t0, t1)` summarises the samples taken between two host times. The
    GPU is matched to amdsmi's device list by PCI bus; without amdsmi (or a readable
    clock) every summary is None."""

    def __init__(self, interval: float = 0.004):
        self.interval = interval
        self.samples: list[tuple[float, float]] = []
        self.source = None
        self._stop = threading.Event()
        self._thread = None
        self._read = None
        self._read_mem = None
        try:
            self._setup()
        except Exception as e:  # no amdsmi, no permission, no device: report, never fail
            self.source = f"unavailable ({type(e).__name__})"
            self._read = None

    def _setup(self):
        import amdsmi
        import torch

        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        if not handles:
            raise RuntimeError("no amdsmi devices")
        props = torch.cuda.get_device_properties(0)
        handle, matched = handles[0], False
        for hd in handles:
            try:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(hd)  # "dddd:bb:dd.f"
                dom, bus = bdf.split(":")[0], bdf.split(":")[1]
                if int(bus, 16) == props.pci_bus_id and int(dom, 16) == props.pci_domain_id:
                    handle, matched = hd, True
                    break
            except Exception:
                continue

        def from_metrics():
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            v = m.get("current_gfxclks")
            vals = [float(c) for c in (v if isinstance(v, (list, tuple)) else [])
                    if isinstance(c, (int, float)) and 0 < c < 10000]
            if vals:
                return sum(vals) / len(vals)
            c = m.get("current_gfxclk")
            return float(c) if isinstance(c, (int, float)) and 0 < c < 10000 else None

        def from_clock_info():
            c = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX).get("clk")
            return float(c) if isinstance(c, (int, float)) and 0 < c < 10000 else None

        def mem_clock():
            c = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.MEM).get("clk")
            return float(c) if isinstance(c, (int, float)) and 0 < c < 100000 else None

        self._read_mem = mem_clock
        for name, fn in (("amdsmi gpu_metrics current_gfxclk(s)", from_metrics),
                         ("amdsmi clock_info GFX", from_clock_info)):
            try:
                if fn() is not None:
                    self._read, self.source = fn, name + ("" if matched else " (device not matched by PCI bus)")
                    return
            except Exception:
                continue
        raise RuntimeError("no readable GFX clock")

    def start(self):
        if self._read is None:
            return self

        def run():
            while not self._stop.is_set():
                try:
                    v = self._read()
                    if v is not None:
                        self.samples.append((time.perf_counter(), v))
                except Exception:
                    pass
                self._stop.wait(self.interval)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=1.0)

    def memory_clock_mhz(self):
        """One reading of the memory clock (MHz), or None where it cannot be read."""
        try:
            return self._read_mem() if self._read_mem is not None else None
        except Exception:
            return None

    def window(self, t0: float, t1: float):
        v = [c for t, c in self.samples if t0 <= t <= t1]
        if not v:
            return None
        # (amdsmi refreshes its metrics every few ms to tens of ms, so consecutive samples
        # often repeat a value: "distinct" counts the different readings)
        return {"mean_mhz": round(sum(v) / len(v), 1), "min_mhz": round(min(v), 1),
                "max_mhz": round(max(v), 1), "samples": len(v), "distinct": len(set(v))}


def cpu_baseline(wl, d, ags, wgs, seconds):
    """The oracle as it stands on the workload's activation rows, full weights: chunks of
    rows in order (wrapping round to row 0 after the last) until about `seconds` of CPU
    work; scaled to TFLOP/s of the same 2*rows*N*K count."""
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


class Timer:
    """HIP events on one stream around back-to-back launches, with the host times of the
    region for the clock sampler."""

    def __init__(self, stream, clock: ClockSampler):
        import torch

        self.torch, self.stream, self.clock = torch, stream, clock

    def launches(self, fn, n: int, warm: int, warm_seconds: float = 0.0):
        """Average ms of n back-to-back launches of fn on the stream, after `warm` untimed
        ones and, with warm_seconds, more untimed ones until that much wall time has passed
        (the GPU clock takes milliseconds to rise again after memory-bound work); returns
        (ms, clock summary of the timed launches)."""
        torch = self.torch
        for _ in range(warm):
            fn()
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < warm_seconds:
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(self.stream)
        for _ in range(n):
            fn()
        b.record(self.stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return a.elapsed_time(b) / n, self.clock.window(t0, t1)


def settle(step, stream, seconds: float, min_steps: int, chunk: int = 50):
    """Whole steps in chunks of `chunk` until `seconds` of wall time and `min_steps` steps
    have passed; returns the settle record (the last chunk's ms per step)."""
    import torch

    t_start = time.perf_counter()
    steps, last_ms = 0, None
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while True:
        a.record(stream)
        for _ in range(chunk):
            step()
        b.record(stream)
        b.synchronize()
        steps += chunk
        last_ms = a.elapsed_time(b) / chunk
        if steps >= min_steps and time.perf_counter() - t_start >= seconds:
            break
    return {"seconds": round(time.perf_counter() - t_start, 3), "steps": steps,
            "last_chunk_steps": chunk, "last_chunk_ms_per_step": round(last_ms, 5)}


def bandwidth_legs(nv, lib, timer, sp, rotate_mb, n_min, gen):
    """Quantize on rotated buffers for each large activation, and a rotated device copy
    moving the same bytes (1.28125 B per element each way = the quantize's 2.5625 B of
    traffic per element)."""
    import torch

    dev = torch.device("cuda:0")
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    out = []
    for (M, K) in QUANT_SHAPES:
        n_rot = max(2, int(rotate_mb * 2**20 // (M * K * 2)))
        xs = [torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16) for _ in range(n_rot)]
        f_gs = ctypes.c_float(nv.calibrate(xs[0]))
        ob = [(torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
               torch.empty((M, K // 16), dtype=torch.uint8, device=dev)) for _ in range(n_rot)]
        ptrs = [(P(a), P(b), P(c)) for a, (b, c) in zip(xs, ob)]
        it = [0]

        def q():
            a, b, c = ptrs[it[0] % n_rot]
            it[0] += 1
            if lib.nvfp4_quantize(a, M, K, f_gs, b, c, sp):
                raise RuntimeError("quantize failed")

        n = max(n_min, 4 * n_rot)
        ms, clk = timer.launches(q, n, warm=2 * n_rot)
        nbytes = QUANT_BYTES_PER_ELEM * M * K
        del xs, ob, ptrs
        # copy of the same traffic, rotated the same way
        cbytes = M * K * 41 // 32
        n_crot = max(2, int(rotate_mb * 2**20 // (2 * cbytes)))
        srcs = [torch.empty(cbytes, dtype=torch.uint8, device=dev).fill_(1) for _ in range(n_crot)]
        dsts = [torch.empty(cbytes, dtype=torch.uint8, device=dev) for _ in range(n_crot)]
        jt = [0]

        def cp():
            i = jt[0] % n_crot
            jt[0] += 1
            dsts[i].copy_(srcs[i])

        nc = max(n_min, 4 * n_crot)
        cms, cclk = timer.launches(cp, nc, warm=2 * n_crot)
        del srcs, dsts
        torch.cuda.empty_cache()
        out.append({
            "shape": [M, K], "rotated_buffers": n_rot, "launches": n,
            "avg_ms": round(ms, 5), "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_per_launch": int(nbytes), "clock": clk,
            "copy_same_bytes": {"bytes_each_way": cbytes, "rotated_buffers": n_crot,
                                "avg_ms": round(cms, 5),
                                "GB/s": round(2 * cbytes / (cms * 1e-3) / 1e9, 1),
                                "frac": round(2 * cbytes / (cms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                "clock": cclk},
        })
    return out


def context_legs(nv, lib, timer, stream, n, rotate_weights_mb=512):
    """Context rows (not the metric). The fused linear (quantize + GEMM: nvfp4_linear) and
    the GEMM alone on every M = 4608 FLUX linear and the 4-image batch, on the seeded
    workload tensors (the static-scale MLP up-projection keeps its offline scale);
    hipBLASLt bf16, MXFP8, rowwise FP8 and W4A16 at the metric's shape; short activations
    (weights dominate the bytes). All operands resident (warm), except the rows for 1 and
    17 activation rows, which also cycle through copies of the weights totalling
    `rotate_weights_mb` (HBM-bound: the weights' bytes are the work)."""
    import numpy as np
    import torch

    from workloads import make

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(7)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    warm = max(20, n // 4)
    out = {"linear": {}, "short_activations": {}}

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    for name in LINEAR_WORKLOADS:
        wl = make(name)
        M, N, K = wl.M, wl.N, wl.K
        d = wl.generate()
        x, w = to_dev(d["x"]), to_dev(d["w"])
        wgs = nv.calibrate(w)
        wp, ws = nv.quantize(w, wgs)
        ags = nv.calibrate(to_dev(d["calib"])) if "calib" in d else nv.calibrate(x)
        del d
        nb = nv.linear_workspace_bytes(M, K)
        work = torch.empty(nb, dtype=torch.uint8, device=dev)
        ap, as_ = nv.workspace_views(work, M, K)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        al = (P(x), ctypes.c_float(ags), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y),
              P(work), ctypes.c_size_t(nb), sp)
        ms_l, clk_l = timer.launches(lambda: lib.nvfp4_linear(*al), n, warm, warm_seconds=0.3)
        ag = (P(ap), P(as_), ctypes.c_float(ags), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y), sp)
        ms_g, clk_g = timer.launches(lambda: lib.nvfp4_gemm(*ag), n, warm, warm_seconds=0.3)
        fl = 2.0 * M * N * K
        out["linear"][name] = {
            "M": M, "N": N, "K": K, "gemm_kernel": nv.gemm_plan(M, N, K),
            "static_activation_scale": bool(wl.static_scale),
            "linear_avg_ms": round(ms_l, 5), "linear_TFLOP/s": round(fl / (ms_l * 1e-3) / 1e12, 1),
            "linear_frac_f16_peak": round(fl / (ms_l * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
            "gemm_avg_ms": round(ms_g, 5), "gemm_TFLOP/s": round(fl / (ms_g * 1e-3) / 1e12, 1),
            "gemm_frac_f16_peak": round(fl / (ms_g * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
            "gemm_share_of_linear": round(ms_g / ms_l, 4), "clock_linear": clk_l, "clock_gemm": clk_g}
        if name == "attn_out":
            # hipBLASLt bf16 GEMM of the unquantized operands at the same shape
            wt = w.t().contiguous()
            ms_b, _ = timer.launches(lambda: torch.matmul(x, wt, out=y), n, warm, warm_seconds=0.2)
            out["hipblaslt_bf16_matmul"] = {"shape": [M, N, K], "avg_ms": round(ms_b, 5),
                                            "TFLOP/s": round(fl / (ms_b * 1e-3) / 1e12, 1)}
            del wt
            # MXFP8 path (E4M3 elements, E8M0 scales per 32) on the same operands
            ac, asx = nv.mxfp8_quantize(x)
            wc, wsx = nv.mxfp8_quantize(w)
            a8 = (P(ac), P(asx), P(wc), P(wsx), M, N, K, P(y), sp)
            ms8, _ = timer.launches(lambda: lib.nvfp4_mxfp8_gemm(*a8), n, warm, warm_seconds=0.2)
            q8 = (P(x), M, K, P(ac), P(asx), sp)
            msq8, _ = timer.launches(lambda: lib.nvfp4_mxfp8_quantize(*q8), n, warm)
            out["mxfp8"] = {"shape": [M, N, K], "gemm_avg_ms": round(ms8, 5),
                            "gemm_TFLOP/s": round(fl / (ms8 * 1e-3) / 1e12, 1),
                            "frac_fp8_peak": round(fl / (ms8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                            "quantize_avg_ms_warm": round(msq8, 5),
                            "quantize_GB/s_warm": round((2 + 1 + 1 / 32) * M * K / (msq8 * 1e-3) / 1e9, 1)}
            del ac, asx, wc, wsx
            # rowwise FP8 (fp8r): E4M3 with one fp32 scale per row, unit-scaled fp8 MFMA
            rc, rs = nv.fp8r_quantize(x)
            wrc, wrs = nv.fp8r_quantize(w)
            ar = (P(rc), P(rs), P(wrc), P(wrs), M, N, K, P(y), sp)
            msr, _ = timer.launches(lambda: lib.nvfp4_fp8r_gemm(*ar), n, warm, warm_seconds=0.2)
            qr = (P(x), M, K, P(rc), P(rs), sp)
            msqr, _ = timer.launches(lambda: lib.nvfp4_fp8r_quantize(*qr), n, warm)
            out["fp8r"] = {"shape": [M, N, K], "gemm_avg_ms": round(msr, 5),
                           "gemm_TFLOP/s": round(fl / (msr * 1e-3) / 1e12, 1),
                           "frac_fp8_peak": round(fl / (msr * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                           "quantize_avg_ms_warm": round(msqr, 5),
                           "quantize_GB/s_warm": round((3 * M * K + 4 * M) / (msqr * 1e-3) / 1e9, 1)}
            del rc, rs, wrc, wrs
            # W4A16: NVFP4 weights, bf16 activations
            a16 = (P(x), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y), sp)
            ms16, _ = timer.launches(lambda: lib.nvfp4_gemm_w4a16(*a16), n, warm, warm_seconds=0.2)
            out["w4a16"] = {"shape": [M, N, K], "kernel": nv.gemm_w4a16_plan(M, N, K),
                            "avg_ms": round(ms16, 5), "TFLOP/s": round(fl / (ms16 * 1e-3) / 1e12, 1)}
        del x, w, wp, ws, work, ap, as_, y
        torch.cuda.empty_cache()
    # short activations: the weights dominate the bytes (K/2 + K/16 bytes per weight row)
    N, K = 3072, 3072
    w = (torch.randn((N, K), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    wgs = nv.calibrate(w)
    wp, ws = nv.quantize(w, wgs)
    for M in (1, 17, 256, 1000):
        x = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
        ags = nv.calibrate(x)
        ap, as_ = nv.quantize(x, ags)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ag = (P(ap), P(as_), ctypes.c_float(ags), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y), sp)
        ms, _ = timer.launches(lambda: lib.nvfp4_gemm(*ag), n, warm)
        a16 = (P(x), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y), sp)
        ms16, _ = timer.launches(lambda: lib.nvfp4_gemm_w4a16(*a16), n, warm)
        nb = nv.linear_workspace_bytes(M, K)
        work = torch.empty(nb, dtype=torch.uint8, device=dev)
        al = (P(x), ctypes.c_float(ags), P(wp), P(ws), ctypes.c_float(wgs), M, N, K, P(y),
              P(work), ctypes.c_size_t(nb), sp)
        msl, _ = timer.launches(lambda: lib.nvfp4_linear(*al), n, warm)
        wbytes = N * (K // 2 + K // 16)
        row = {
            "N": N, "K": K, "kernel": nv.gemm_plan(M, N, K), "w4a4_avg_ms": round(ms, 5),
            "w4a4_weight_GB/s": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "linear": nv.linear_plan(M, N, K), "linear_avg_ms": round(msl, 5),
            "w4a16_kernel": nv.gemm_w4a16_plan(M, N, K), "w4a16_avg_ms": round(ms16, 5),
            "TFLOP/s": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 2)}
        if M <= 17:
            # HBM-bound on the weights: cycle through copies of the quantized weights
            # totalling beyond the 256 MB Infinity Cache, so each launch reads them from HBM
            n_rot = max(2, -(-rotate_weights_mb * 2**20 // wbytes))
            sets = [(wp.clone(), ws.clone()) for _ in range(n_rot)]
            args_r = [(P(ap), P(as_), ctypes.c_float(ags), P(a), P(b), ctypes.c_float(wgs), M, N, K,
                       P(y), sp) for a, b in sets]
            it = [0]

            def rot():
                if lib.nvfp4_gemm(*args_r[it[0] % n_rot]):
                    raise RuntimeError("gemm failed")
                it[0] += 1

            ms_r, _ = timer.launches(rot, max(n, 2 * n_rot), n_rot)
            abytes = M * (K // 2 + K // 16) + 2 * M * N  # activation codes + bf16 output
            row["w4a4_rotated_weights"] = {
                "weight_sets": n_rot, "avg_ms": round(ms_r, 5),
                "weight_GB/s": round(wbytes / (ms_r * 1e-3) / 1e9, 1),
                "bytes_per_launch": wbytes + abytes,
                "frac_hbm_peak": round((wbytes + abytes) / (ms_r * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            del sets, args_r
        out["short_activations"][f"M={M}"] = row
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   f"--gpus {args.gpus} is not supported (the hot path is "
                                   "measured on one GPU's share; see DESIGN.md for sharding)"}))
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

    def gemm_only():
        if lib.nvfp4_gemm(qpa, qsa, f_ags, wqa, wsa, f_wgs, M, N, K, oa, sp):
            raise RuntimeError("gemm failed")

    clock = ClockSampler().start()
    timer = Timer(stream, clock)

    # 1. clock settle (wall time, independent of --warmup), 2. warm-up
    t_s0 = time.perf_counter()
    settle_rec = settle(step, stream, args.settle_seconds, args.settle_min_steps)
    settle_rec["clock"] = clock.window(t_s0, time.perf_counter())
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # 3. Timed region: K whole steps (quantize + GEMM), events only at its two ends.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12

    # 4. The dominant kernel alone, back-to-back launches on the same stream (its average
    # launch duration, for the roofline).
    n_roof = max(args.steps, args.roofline_launches)
    g_ms, g_clk = timer.launches(gemm_only, n_roof, warm=0)
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12

    # 5. quantize bandwidth (and the copy ceiling) on rotated buffers
    gen = torch.Generator(device=dev).manual_seed(5)
    del x, qp, qs, work, out
    torch.cuda.empty_cache()
    bw = bandwidth_legs(nv, lib, timer, sp, args.rotate_mb, max(args.steps, 200), gen)

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

    q0 = bw[0]
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "settle": settle_rec,
        "clock_timed_steps": clock.window(h0, h1),
        "clock_source": clock.source,
        "memory_clock_mhz": clock.memory_clock_mhz(),
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
            "launches": n_roof,
            "clock": g_clk,
        },
        "quantize": {
            "rotated_avg_ms": q0["avg_ms"],
            "achieved": q0["achieved"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": q0["frac"],
            "bytes_per_launch": q0["bytes_per_launch"],
            "shapes": bw,
        },
        "precision": "E2M1 x E4M3 operands decoded exactly to f16, f16 MFMA, fp32 accumulate, "
                     "bf16 output",
    }
    if not args.no_context:
        result["context"] = context_legs(nv, lib, timer, stream, max(200, args.steps // 2))
    clock.stop()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, d, ags, wgs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
