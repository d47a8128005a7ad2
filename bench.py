"""Benchmark of the exact block-quantized decode GEMV on one MI355X.

A step is one pass of the whole hot path over one synthetic activation row: quantize the
f32 row and run the GEMV over the packed matrix.  At one column that is one launch of
qg_quantize_gemv (--two-launch: qg_quantize_act then qg_gemv_q); batched workloads run
qg_quantize_act then qg_gemm_q.  Everything runs on one stream with inputs resident in HBM.
The default workload is the Llama-8B-shaped FFN up-projection, 14336 x 4096 Q4_K-style,
PerBlock scaling, fresh activations every step, and the weights are read cold: each step
uses the next of C copies of the image (C * 33 MB >= 512 MB, twice the 256 MB Infinity
Cache).

Timing:
  * ms_per_step: the K timed steps are captured in HIP graphs (one graph node per kernel)
    and replayed between two events after a synchronize; whole-job weight GB/s = K * image
    bytes / elapsed.
  * roofline.achieved: algorithmic bytes per launch of the step's dominant kernel (the
    fused kernel, or the GEMV/GEMM kernel) over that kernel's duration, from HIP events
    around replays of a graph of kernel-only launches over the same rotated-cold copies (on
    the stream they run on).  The median of single eager launches timed by events the
    launch itself records (hipExtLaunchKernelGGL, qg_time_next_launch) is reported beside it.
  * measured_ceiling: qg_stream_read, a plain read with the GEMV's load pattern, over the same
    bytes per launch and rotated copies (what one launch of this size can reach), and over
    2 GiB (the sustained rate).
  * cpu_baseline: the CPU oracle on the same workload, all rows, fresh activations, for
    about --cpu-seconds of wall time on every core it may use (at most OMP_NUM_THREADS),
    then half that on one thread; the host's core counts and CPU model beside them.

Prints one JSON line.  --gpus above 1 is refused: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM traffic of the GEMV kernel per launch, from two rocprofv3 --pmc passes (FETCH_SIZE,
# then WRITE_SIZE, medians in KiB per dispatch), each scaled by what the same counter reads
# for a plain device copy of 256 MiB (FETCH_SIZE 131083.5 KiB, WRITE_SIZE 262144 KiB).
# A figure is reported only while the kernel sources still hash to the value it was taken
# on; the commands and readings are kept under profiles/.
COPY_BYTES = 268435456
FETCH_FACTOR = COPY_BYTES / (131083.5 * 1024)
WRITE_FACTOR = COPY_BYTES / (262144.0 * 1024)
KERNEL_SOURCES = ("block_format_gemv_amd/csrc/gemv.hip", "block_format_gemv_amd/csrc/qg_device.hpp",
                  "block_format_gemv_amd/csrc/qg_internal.hpp")
MEASURED_TRAFFIC = {
    # (workload, dominant kernel): medians per dispatch, kernel sources hash
    ("q4k_ffn_up_14336x4096", "fused"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 16240.5, "write_kib": 61.0625},
    ("q4k_ffn_up_14336x4096", "gemv"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 16184.5, "write_kib": 56.0},
    ("q4k_attn_4096x4096", "fused"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 4716.5, "write_kib": 21.0625},
    ("q4k_attn_4096x4096", "gemv"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 4659.0, "write_kib": 16.0},
    ("q4k_sub32_14336x4096", "fused"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 16264.4375, "write_kib": 61.5},
    ("q4k_sub32_14336x4096", "gemv"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 16209.0, "write_kib": 56.0},
    ("q6k_output_128256x4096", "fused"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 210541.0, "write_kib": 506.0625},
    ("q6k_output_128256x4096", "gemv"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 210487.0, "write_kib": 501.0},
    ("q8_0_ffn_up_14336x4096", "fused"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 30580.5, "write_kib": 61.5},
    ("q8_0_ffn_up_14336x4096", "gemv"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 30526.0, "write_kib": 56.0},
    ("q4_0_ffn_up_14336x4096", "fused"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 16244.5, "write_kib": 61.5},
    ("q4_0_ffn_up_14336x4096", "gemv"): {"kernel_sha": "ee861e45e0dbc1ee", "fetch_kib": 16195.5, "write_kib": 56.0},
}

# The batched GEMM kernels (several columns): HBM traffic as above, and for the int8
# matrix-core kernel its matrix-core use, from rocprofv3 --pmc passes:
# SQ_INSTS_VALU_MFMA_MOPS_I8 (int8 matrix operations / 512 over the chip) and MfmaUtil (the
# matrix units' busy cycles over the dispatch's active cycles times the SIMDs); medians per
# dispatch, reported only while the sources (the GEMV kernels, which hold the several-column
# kernel, and the matrix-core kernels) still hash to the value they were taken on.
GEMM_SOURCES = KERNEL_SOURCES + ("block_format_gemv_amd/csrc/gemm_mfma.hip",)
MFMA_PEAK_TOPS = 5000.0     # dense int8 matrix-core peak of the part, TOP/s
MEASURED_GEMM = {
    "q4k_gemm_n2_4096x4096": {"kernel_sha": "0798631ed8d0ef3a", "fetch_kib": 4687.5, "write_kib": 32.0, "mops_i8": 3145728.0, "mfma_util_pct": 2.43},
    "q4k_gemm_n8_4096x4096": {"kernel_sha": "0798631ed8d0ef3a", "fetch_kib": 4785.0, "write_kib": 128.0, "mops_i8": 3145728.0, "mfma_util_pct": 2.2},
    "q4k_gemm_n64_4096x4096": {"kernel_sha": "0798631ed8d0ef3a", "fetch_kib": 5724.5, "write_kib": 1024.0, "mops_i8": 12582912.0, "mfma_util_pct": 5.95},
    "q4k_gemm_n2_14336x4096": {"kernel_sha": "0798631ed8d0ef3a", "fetch_kib": 16220.0, "write_kib": 112.0},
    "q4k_gemm_n8_14336x4096": {"kernel_sha": "0798631ed8d0ef3a", "fetch_kib": 16328.5, "write_kib": 448.0, "mops_i8": 11010048.0, "mfma_util_pct": 5.27},
    "q4k_gemm_n64_14336x4096": {"kernel_sha": "0798631ed8d0ef3a", "fetch_kib": 17589.625, "write_kib": 3584.0625, "mops_i8": 44040192.0, "mfma_util_pct": 14.15},
}


def kernel_sha(sources=KERNEL_SOURCES) -> str:
    import hashlib

    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    t = MEASURED_GEMM.get(workload) if kernel == "gemm" else MEASURED_TRAFFIC.get((workload, kernel))
    if not t or t["kernel_sha"] != kernel_sha(GEMM_SOURCES if kernel == "gemm" else KERNEL_SOURCES):
        return None
    return round(t["fetch_kib"] * 1024 * FETCH_FACTOR + t["write_kib"] * 1024 * WRITE_FACTOR)


def measured_mfma(workload: str):
    t = MEASURED_GEMM.get(workload)
    if not t or "mops_i8" not in t or t["kernel_sha"] != kernel_sha(GEMM_SOURCES):
        return None
    return {"int8_ops_per_launch": t["mops_i8"] * 512, "mfma_util_pct": t["mfma_util_pct"]}


METRIC = "quantized GEMV weight-stream HBM GB/s (% of peak) and rows/s at 1 GPU"

WORKLOADS = {
    # name: (format, rows, cols, scaling, columns); rows a tuple = several matrices (named by
    # workloads.gen.llama_q4k) sharing one activation row in one launch
    "q4k_ffn_up_14336x4096": ("q4k", 14336, 4096, 0, 1),
    "q4k_ffn_gate_up_2x14336x4096": ("q4k", (("gate", 14336), ("ffn", 14336)), 4096, 0, 1),
    "q4k_attn_qkv_6144x4096": ("q4k", (("attn", 4096), ("k", 1024), ("v", 1024)), 4096, 0, 1),
    "q4k_attn_4096x4096": ("q4k", 4096, 4096, 0, 1),
    "q6k_output_128256x4096": ("q6k", 128256, 4096, 0, 1),
    "q8_0_ffn_up_14336x4096": ("q8_0", 14336, 4096, 0, 1),
    "q4_0_ffn_up_14336x4096": ("q4_0", 14336, 4096, 0, 1),
    "q4k_sub32_14336x4096": ("q4k", 14336, 4096, 1, 1),
    "q4k_gemm_n2_14336x4096": ("q4k", 14336, 4096, 0, 2),
    "q4k_gemm_n8_14336x4096": ("q4k", 14336, 4096, 0, 8),
    "q4k_gemm_n16_14336x4096": ("q4k", 14336, 4096, 0, 16),
    "q4k_gemm_n32_14336x4096": ("q4k", 14336, 4096, 0, 32),
    "q4k_gemm_n64_14336x4096": ("q4k", 14336, 4096, 0, 64),
    "q4k_gemm_n64_4096x4096": ("q4k", 4096, 4096, 0, 64),
    "q4k_gemm_n8_4096x4096": ("q4k", 4096, 4096, 0, 8),
    "q4k_gemm_n2_4096x4096": ("q4k", 4096, 4096, 0, 2),
    # int8 KV cache (attention of one decode step): ("kv", query heads, KV heads, positions,
    # head size, query scaling)
    "kv_decode_32h_8kv_4096pos_128hd": ("kv", 32, 8, 4096, 128, 0),
}
KV_METRIC = "int8 KV-cache attention stream GB/s at 1 GPU"
DEFAULT = "q4k_ffn_up_14336x4096"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1600)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    p.add_argument("--cold-bytes", type=float, default=512e6, help="rotate over at least this many weight bytes")
    p.add_argument("--warm", action="store_true", help="one copy of the weights (cache-resident)")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--kernel-launches", type=int, default=1600)
    p.add_argument("--two-launch", action="store_true",
                   help="time the step as qg_quantize_act + qg_gemv_q instead of qg_quantize_gemv")
    p.add_argument("--tune", action="append", default=[], metavar="KEY=VALUE",
                   help="a speed-only tuning knob (qg_set_tuning): waves_per_wg, mfma_min_cols, mfma_col_tiles, "
                        "mfma_form, cols_kernel, mfma_tables, gemm_row_tiles, gemv_quarter; output bits do not depend on "
                        "them")
    p.add_argument("--kernel-only", type=int, default=0, metavar="K",
                   help="only launch the step's dominant kernel K times (eager, over the rotated copies) and exit: "
                        "for rocprofv3 counter passes")
    p.add_argument("--ceiling-sweep", action="store_true",
                   help="only sweep plain-read launch shapes (qg_stream_read_shape) and a library read kernel "
                        "(torch's amax) over the 4096x4096 and 14336x4096 Q4_K-style image sizes, cold; "
                        "print a markdown table and exit")
    p.add_argument("--copy-probe", type=float, default=0,
                   help="only run 20 device-to-device copies of this many bytes (counter calibration) and exit")
    return p.parse_args()


def copy_probe(nbytes: int) -> None:
    """A plain copy kernel of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "copies": 20}), flush=True)


def ceiling_sweep() -> None:
    """Plain reads of the two Q4_K-style image sizes (9,437,184 and 33,030,144 bytes) in many
    launch shapes, each launch reading the next of the copies of a 1 GiB buffer (cold, as the
    benchmark reads weights); per shape the time per launch from events around graph replays.
    Beside our own read kernel, torch's amax over the same bytes (viewed as int32) is timed the
    same way: a read kernel this library did not write."""
    import torch

    import block_format_gemv_amd as qg

    dev = torch.device("cuda:0")
    big = torch.randint(0, 1 << 30, ((1 << 30) // 4,), dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.Stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    graph_len = 32

    def per_launch_us(fn, copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(graph_len):
                fn(i % copies)
        for _ in range(3):
            g.replay()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        reps = 8
        with torch.cuda.stream(s):
            torch.cuda.synchronize()
            t0.record(s)
            for _ in range(reps):
                g.replay()
            t1.record(s)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / (reps * graph_len)

    lines = ["| image bytes | read kernel | waves/WG | KiB/wave | workgroups | loads | us/launch | GB/s | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    results = []
    for nbytes in (9437184, 33030144):
        copies = (1 << 30) // nbytes
        views = [big.view(torch.uint8)[c * nbytes:(c + 1) * nbytes] for c in range(copies)]
        shapes = []
        for w in (4, 8, 16):
            for k in (1, 2, 4, 9, 16):
                shapes.append((w, k, 0, 0))
        for w in (4, 8, 16):
            for k in (1, 4, 9):
                for wgs in (cus, 2 * cus, 4 * cus, 8 * cus):
                    shapes.append((w, k, wgs, 0))
        shapes += [(16, 9, 0, 1), (4, 4, 0, 1), (8, 4, 2 * cus, 1)]
        for w, k, wgs, flags in shapes:
            def fn(c, w=w, k=k, wgs=wgs, flags=flags):
                qg.qg_stream_read_shape(views[c], nbytes, w, k, wgs, flags, 0x9E3779B9, sink, s)
            us = per_launch_us(fn, copies)
            nwg = wgs if wgs else -(-(-(-nbytes // 1024) // k) // w)
            gbs = nbytes / (us * 1e-6) / 1e9
            results.append((nbytes, "qg_stream_read_shape", w, k, nwg, "grid-stride" if wgs else "one pass",
                            "ordinary" if flags else "non-temporal", us, gbs))
        def gemv_pattern(c):
            qg.qg_stream_read(views[c], nbytes, 0x9E3779B9, sink, s)
        us = per_launch_us(gemv_pattern, copies)
        results.append((nbytes, "qg_stream_read (the GEMV's pattern)", 16, 9, -(-(-(-nbytes // 1024) // 9) // 16),
                        "one pass", "non-temporal", us, nbytes / (us * 1e-6) / 1e9))
        # torch's reduction, eager (it is kept out of graphs: it may clear a semaphore with a
        # memset): a long read first, so that the launches queue up behind it and each pair of
        # events brackets its kernels back to back
        ints = [v.view(torch.int32) for v in views]
        outs = [torch.empty((), dtype=torch.int32, device=dev) for _ in range(copies)]
        ts = []
        with torch.cuda.stream(s):
            torch.amax(ints[0], dim=0, out=outs[0])
            torch.cuda.synchronize()
            qg.qg_stream_read(big, big.numel() * 4, 0x9E3779B9, sink, s)
            evs = []
            for i in range(24):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(s)
                torch.amax(ints[i % copies], dim=0, out=outs[i % copies])
                e1.record(s)
                evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs[4:])
        us = ts[len(ts) // 2]
        results.append((nbytes, "torch.amax (int32 view, eager, median)", "-", "-", "-", "library", "-", us,
                        nbytes / (us * 1e-6) / 1e9))
    for nbytes, kern, w, k, nwg, mode, loads, us, gbs in results:
        lines.append(f"| {nbytes} | {kern} | {w} | {k} | {nwg} ({mode}) | {loads} | {us:.3f} | {gbs:.1f} | "
                     f"{100 * gbs / HBM_PEAK_GBS:.1f} |")
    print("\n".join(lines), flush=True)
    best = {}
    for r in results:
        if r[0] not in best or r[7] < best[r[0]][7]:
            best[r[0]] = r
    print(json.dumps({"ceiling_sweep_best": {str(k): {"kernel": v[1], "waves_per_wg": v[2], "kib_per_wave": v[3],
                                                      "workgroups": v[4], "mode": v[5], "us": round(v[7], 3),
                                                      "frac_of_peak": round(v[8] / HBM_PEAK_GBS, 4)}
                                             for k, v in best.items()}}), flush=True)


class Hip:
    """The few HIP runtime calls bench.py makes itself (events)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.L.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert self.L.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return float(ms.value)

    def destroy(self, e):
        self.L.hipEventDestroy(ctypes.c_void_p(e))


def make_inputs(wl, n_act):
    """(list of matrices' fields, activation rows)"""
    from workloads import gen

    fmt, rows, cols, mode, ncol = wl
    if isinstance(rows, tuple):
        fields = [gen.llama_q4k(name) for name, _ in rows]
    elif fmt == "q4k":
        fields = [gen.q4k_fields(rows, cols, gen.SEED_ATTN_W if rows == 4096 else gen.SEED_FFN_W)]
    elif fmt == "q8_0":
        fields = [gen.q8_0_fields(rows, cols, gen.SEED_Q8_W)]
    elif fmt == "q4_0":
        fields = [gen.q4_0_fields(rows, cols, gen.SEED_Q4_0_W)]
    else:
        fields = [gen.output_q6k()[0]]
    if ncol > 1:
        xs = [gen.act_normal(ncol, cols, gen.SEED_BATCH_X + ncol + 1000 * k) for k in range(n_act)]
    elif mode == 1:
        xs = [gen.sub32_act(k, cols)[0] for k in range(n_act)]
    elif fmt == "q6k":
        xs = [gen.act_normal(1, cols, gen.SEED_OUT_X + 1000 * k) for k in range(n_act)]
    else:
        xs = [gen.decode_act(k, cols) for k in range(n_act)]
    return fields, xs


def host_threads():
    """The host description a CPU baseline carries and the thread count of its all-cores run:
    every core this process may run on, but no more than OMP_NUM_THREADS when that is set (a
    host shared by several GPUs gives each its share through it)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = avail
    if omp and omp.isdigit() and int(omp) > 0:
        threads = min(avail, int(omp))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    host = {"nproc": os.cpu_count(), "affinity_cpus": avail, "omp_num_threads": omp, "cpu_model": model}
    return threads, host


def timed_runs(step, seconds):
    """step(k) repeated for about `seconds` of wall time; (steps, seconds taken)."""
    t0 = time.perf_counter()
    steps = 0
    while True:
        step(steps)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return steps, dt


def cpu_baseline(mats, xs, mode, seconds, image_bytes):
    """The oracle on the same workload, whole steps with fresh activations: once on all the
    threads host_threads() allows (the reported value) and once on one thread."""
    import oracle

    threads, host = host_threads()
    outs = []

    def step(k):
        x = xs[k % len(xs)]
        c, m, e, _ = oracle.quantize(x, mode, block=oracle.act_block(mats[0]["fmt"], mode))
        out = np.concatenate([oracle.gemm(f, c, m, e, mode).reshape(xs[0].shape[0], -1) for f in mats], axis=1)
        if k < 2 and len(outs) < 2:
            outs.append(out)

    total_rows = sum(f["rows"] for f in mats)
    rows = total_rows * xs[0].shape[0]
    what = f"quantize + all {total_rows} rows x {xs[0].shape[0]} column(s)"
    oracle.set_threads(1)
    s1, d1 = timed_runs(step, seconds / 2)
    oracle.set_threads(threads)
    steps, dt = timed_runs(step, seconds)
    return {
        "value": round(steps * image_bytes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{steps} whole steps ({what}) of the same workload with fresh activations on {threads} "
                  f"threads, {dt:.1f} s",
        "rows_per_s": round(steps * rows / dt, 1),
        "single_thread": {"value": round(s1 * image_bytes / d1 / 1e9, 3), "unit": "GB/s", "threads": 1,
                          "sample": f"{s1} whole steps ({what}) on one thread, {d1:.1f} s",
                          "rows_per_s": round(s1 * rows / d1, 1)},
        "host": host,
    }, outs


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(int(args.copy_probe))
        return
    if args.ceiling_sweep:
        ceiling_sweep()
        return
    import torch

    import block_format_gemv_amd as qg

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tuned = {}
    for kv in args.tune:
        key, _, val = kv.partition("=")
        qg.qg_set_tuning(getattr(qg, "TUNE_" + key.upper()), int(val))
        tuned[key] = int(val)
    wl = WORKLOADS[args.workload]
    if wl[0] == "kv":
        kv_main(args, wl, torch, qg, Hip())
        return
    fmt_s, _, cols, mode, ncol = wl
    fmt = qg.FMT_CODES[fmt_s]
    dev = torch.device("cuda:0")
    hip = Hip()

    n_act = 64
    mats, xs = make_inputs(wl, n_act)
    nmat = len(mats)
    mrows = [int(f["rows"]) for f in mats]
    rows = sum(mrows)
    hosts = [qg.pack(f) for f in mats]
    sizes = [h.nbytes for h in hosts]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    image_bytes = int(offs[-1])
    copies = 1 if args.warm else max(1, int(np.ceil(args.cold_bytes / image_bytes)))
    # each copy is one buffer holding the matrices back to back (image sizes are multiples of 16)
    base = torch.from_numpy(np.concatenate(hosts)).to(dev)
    bufs = [base] + [base.clone() for _ in range(copies - 1)]
    images = [[b[int(offs[m]):int(offs[m + 1])] for m in range(nmat)] for b in bufs]
    x_dev = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in xs]
    slots = max(copies, 16)
    acts = [qg.alloc_act(ncol, cols, mode, dev, fmt) for _ in range(slots)]
    outs = [torch.empty((ncol, rows), dtype=torch.float32, device=dev) for _ in range(slots)]
    # per-matrix output views (one column): out[0, row offset of matrix m ...]
    ro = np.concatenate([[0], np.cumsum(mrows)]).astype(np.int64)
    mouts = [[o.view(-1)[int(ro[m]):int(ro[m + 1])] for m in range(nmat)] for o in outs]
    act_bytes = ncol * (cols + 4 * qg._nsc(fmt, mode, cols) + 4 * (cols // 16))
    out_bytes = 4 * ncol * rows
    fused = ncol == 1 and not args.two_launch
    if nmat > 1 and ncol != 1:
        raise SystemExit("several matrices are benchmarked with one activation column")

    def quantize(i, stream=None):
        a = acts[i % slots]
        qg.qg_quantize_act(fmt, mode, ncol, cols, x_dev[i % n_act], a.codes, a.scales, a.csums, None, stream)

    def multiply(i, stream=None):
        a = acts[i % slots]
        if nmat > 1:
            qg.qg_gemv_q_multi(fmt, mode, mrows, cols, images[i % copies], a.codes, a.scales, a.csums,
                               mouts[i % slots], stream)
        else:
            qg.qg_gemm_q(fmt, mode, rows, cols, ncol, images[i % copies][0], a.codes, a.scales, a.csums,
                         outs[i % slots], stream)

    def fused_call(i, stream=None):
        a = acts[i % slots]
        if nmat > 1:
            qg.qg_quantize_gemv_multi(fmt, mode, mrows, cols, images[i % copies], x_dev[i % n_act], a.codes,
                                      a.scales, a.csums, None, mouts[i % slots], stream)
        else:
            qg.qg_quantize_gemv(fmt, mode, rows, cols, images[i % copies][0], x_dev[i % n_act], a.codes, a.scales,
                                a.csums, None, outs[i % slots], stream)

    def two_launch(i, stream=None):
        quantize(i, stream)
        multiply(i, stream)

    if ncol == 1 and fmt_s in ("q8_0", "q4_0"):
        kernel_label = ("gemv1_b32_kernel<..., SRC_F32> (one-launch quantize + GEMV)" if fused
                        else "gemv1_b32_kernel<..., SRC_CODES> (GEMV of a quantized row)")
    elif ncol == 1 and fmt_s == "q4k" and mode == 0 and cols <= 16 * 256 and not tuned.get("waves_per_wg") and (
            tuned.get("gemv_quarter") == 1 or (not tuned.get("gemv_quarter") and sum((r + 63) // 64 for r in mrows) < 128)):
        # the library's 16-row workgroups (launch_one_any: fewer than 128 row groups in the launch)
        kernel_label = ("gemv1_quarter_kernel<SRC_F32> (one-launch quantize + GEMV, 16-row workgroups)" if fused
                        else "gemv1_quarter_kernel<SRC_CODES> (GEMV of a quantized row, 16-row workgroups)")
    elif ncol == 1:
        kernel_label = ("gemv1_kernel<..., SRC_F32> (one-launch quantize + GEMV)" if fused
                        else "gemv1_kernel<..., SRC_CODES> (GEMV of a quantized row)")
    elif fmt_s == "q4k" and mode == 0 and ncol >= (tuned.get("mfma_min_cols") or (2 if rows < 8192 else 5)):
        # the library's choice of matrix-core form (qg_gemm_q, launch_gemm_mfma)
        form = tuned.get("mfma_form") or (1 if cols <= 16 * 256 and ncol <= 16 else 3 if rows < 8192
                                          else 4 if cols <= 16 * 256 else 2)
        kernel_label = {1: "gemm_staged_q4k (matrix cores, columns staged in LDS, one block per wave)",
                        2: "gemm_mfma_q4k (matrix cores, shared operands)",
                        3: "gemm_split_q4k (matrix cores, one block per wave)",
                        4: "gemm_resident_q4k (matrix cores, columns resident in LDS, one row tile per wave)"}[form]
    elif cols <= 16 * 256 and not tuned.get("cols_kernel") and fmt_s in ("q4k", "q6k"):
        kernel_label = "gemv1_cols_kernel (one-column machinery, up to 8 columns a wave)"
    else:
        kernel_label = "gemv_kernel (several columns staged in LDS)"
    step = fused_call if fused else two_launch
    # the step's dominant kernel: the fused kernel (reads x, writes the quantized row once)
    # or the GEMV/GEMM kernel (reads the quantized row)
    kernel_fn = fused_call if fused else multiply
    if fused:
        algo_bytes = image_bytes + 4 * cols + act_bytes + out_bytes
    else:
        algo_bytes = image_bytes + act_bytes + out_bytes

    if args.kernel_only:
        torch.cuda.synchronize()
        for i in range(args.kernel_only):
            kernel_fn(i)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": args.kernel_only, "workload": args.workload, "kernel": kernel_label}), flush=True)
        return

    # eager first pass, then a bitwise check of step 0 against the oracle on sampled rows
    torch.cuda.synchronize()
    step(0)
    torch.cuda.synchronize()
    first = outs[0].cpu().numpy().copy()

    # HIP graphs of `gsteps` calls each, replayed between two events on the stream they run on
    gsteps = slots
    s = torch.cuda.Stream()

    def graph_of(fn, nsteps, offset=0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(nsteps):
                fn(offset + i)
        return g

    def replay_ms(graphs_in_order):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            torch.cuda.synchronize()
            t0.record(s)
            for g in graphs_in_order:
                g.replay()
            t1.record(s)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    def per_call_us(fn, launches):
        g = graph_of(fn, gsteps)
        for _ in range(4):
            g.replay()
        reps = max(1, launches // gsteps)
        return replay_ms([g] * reps) * 1e3 / (reps * gsteps), reps

    # the timed K steps: exactly K steps of graph replays
    full = graph_of(step, gsteps)
    rest = args.steps % gsteps
    tail = graph_of(step, rest) if rest else None
    torch.cuda.synchronize()
    for _ in range(max(1, -(-args.warmup // gsteps))):
        full.replay()
    torch.cuda.synchronize()
    ms_total = replay_ms([full] * (args.steps // gsteps) + ([tail] if tail is not None else []))
    ms_per_step = ms_total / args.steps

    # the dominant kernel's duration as the workload runs it (graph of kernel-only launches
    # over the same rotated cold copies)
    k_us, reps = per_call_us(kernel_fn, args.kernel_launches)
    achieved = algo_bytes / (k_us * 1e-6) / 1e9
    extra = {}
    if fused:
        # the same step as two launches, and the GEMV kernel alone, for comparison
        extra["two_launch_us_per_step"] = round(per_call_us(two_launch, args.kernel_launches // 4)[0], 3)
        gemv_us = per_call_us(multiply, args.kernel_launches // 4)[0]
        extra["gemv_kernel_us"] = round(gemv_us, 3)
        extra["gemv_kernel_frac_of_peak"] = round((image_bytes + act_bytes + out_bytes) / (gemv_us * 1e-6) / 1e9
                                                  / HBM_PEAK_GBS, 4)

    # the measured ceiling: a plain streaming read (qg_stream_read, the GEMV's load pattern and
    # nothing else) of the same bytes per launch over the same rotated copies, and of 2 GiB
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def read_same(i, stream=None):
        qg.qg_stream_read(bufs[i % copies], image_bytes, 0x9E3779B9, sink, stream)

    ceil_us = per_call_us(read_same, args.kernel_launches // 4)[0]
    big = torch.ones(2 << 30, dtype=torch.uint8, device=dev)

    def read_big(i, stream=None):
        qg.qg_stream_read(big, big.numel(), 0x9E3779B9, sink, stream)

    big_us = per_call_us(read_big, 3 * gsteps)[0]
    del big
    ceiling = {
        "kernel": "qg_stream_read",
        "same_bytes_us": round(ceil_us, 3),
        "same_bytes_GBs": round(image_bytes / (ceil_us * 1e-6) / 1e9, 1),
        "same_bytes_frac_of_peak": round(image_bytes / (ceil_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "read_2GiB_GBs": round((2 << 30) / (big_us * 1e-6) / 1e9, 1),
        "kernel_vs_same_bytes_ceiling": round(ceil_us / k_us, 4),
    }

    # secondary: single eager launches, each bracketed by events the launch itself records
    evs = [(hip.event(), hip.event()) for _ in range(64)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        qg.qg_time_next_launch(e0, e1)
        kernel_fn(i)
    torch.cuda.synchronize()
    k_ms = np.array([hip.elapsed_ms(e0, e1) for e0, e1 in evs])[8:]
    for e0, e1 in evs:
        hip.destroy(e0)
        hip.destroy(e1)

    value = args.steps * image_bytes / (ms_total * 1e-3) / 1e9
    record = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "format": fmt_s,
            "rows": rows if nmat == 1 else mrows,
            "matrices": nmat,
            "cols": cols,
            "act_scaling": "perblock" if mode == 0 else "sub32",
            "columns": ncol,
            "weights": "cold, rotating over %d copies (%.0f MB)" % (copies, copies * image_bytes / 1e6)
                       if copies > 1 else "warm, one copy (cache-resident)",
            **({"tuning": tuned} if tuned else {}),
            "step": (("qg_quantize_gemv_multi" if nmat > 1 else "qg_quantize_gemv") + " (one launch)" if fused
                     else "qg_quantize_act + " + ("qg_gemv_q_multi" if nmat > 1 else "qg_gemm_q"))
                    + ", HIP graph replay",
        },
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "rows_per_s": round(rows * ncol / (ms_per_step * 1e-3), 1),
        "kernel_us": round(k_us, 3),
        "kernel_timing": f"HIP events around {reps} replays of a graph of {gsteps} launches",
        "kernel_us_eager_launch_events_median": round(float(np.median(k_ms)) * 1e3, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload, "fused" if fused else "gemv" if ncol == 1 else "gemm"),
            "kernel": kernel_label,
            "algorithmic_bytes_per_launch": algo_bytes,
        },
    }
    if "matrix cores" in kernel_label:
        # the int8 matrix-core roofline: the dense contraction is 2*rows*cols*columns operations;
        # the kernels issue three int8 products per weight (the sub-scale split into its high and
        # low 3 bits, and the offset) over columns padded to 16
        useful = 2.0 * rows * cols * ncol
        issued = 3 * 2.0 * rows * cols * (-(-ncol // 16) * 16)
        mm = measured_mfma(args.workload)
        record["roofline_matrix_cores"] = {
            "bound": "mfma",
            "achieved": round(useful / (k_us * 1e-6) / 1e12, 2),
            "peak": MFMA_PEAK_TOPS,
            "unit": "TOP/s",
            "frac": round(useful / (k_us * 1e-6) / 1e12 / MFMA_PEAK_TOPS, 4),
            "issued_ops_per_launch": issued,
            "issued_frac": round(issued / (k_us * 1e-6) / 1e12 / MFMA_PEAK_TOPS, 4),
            "counters": mm,
        }
    record["measured_ceiling"] = ceiling
    record.update(extra)
    if not args.no_cpu:
        cb, cpu_outs = cpu_baseline(mats, xs, mode, args.cpu_seconds, image_bytes)
        record["cpu_baseline"] = cb
        record["parity_step0"] = bool(np.array_equal(cpu_outs[0].reshape(-1).view(np.uint32),
                                                     first.reshape(-1).view(np.uint32)))
    print(json.dumps(record), flush=True)


def kv_main(args, wl, torch, qg, hip):
    """One decode step of attention over an int8 KV cache: the step appends the new
    position's key and value rows to the cache (qg_kv_cache_rows), quantizes the query heads
    (qg_kv_quantize_heads), scores them against every cached key (qg_kv_scores) and forms the
    weighted sum of the cached values in two passes (qg_kv_weighted_with_workspace; the
    one-pass qg_kv_weighted is timed beside it) with given attention weights (the softmax
    between the two is the caller's and is not timed).  The caches rotate over copies of at
    least --cold-bytes, like the GEMV's weights."""
    from workloads import gen

    _, nh, nkv, npos, hd, mode = wl
    dev = torch.device("cuda:0")
    keys, vals, query, weights = gen.kv_decode(nh, nkv, npos, hd)
    rows = nkv * npos
    ks = torch.zeros(rows, dtype=torch.int16, device=dev)
    kc = torch.zeros((rows, hd), dtype=torch.int8, device=dev)
    vs = torch.zeros(rows, dtype=torch.int16, device=dev)
    vc = torch.zeros((rows, hd), dtype=torch.int8, device=dev)
    qg.qg_kv_cache_rows(rows, hd, torch.from_numpy(keys.reshape(-1, hd)).to(dev), ks, kc)
    qg.qg_kv_cache_rows(rows, hd, torch.from_numpy(vals.reshape(-1, hd)).to(dev), vs, vc)
    cache_bytes = 2 * (rows * hd + 2 * rows)
    copies = 1 if args.warm else max(1, int(np.ceil(args.cold_bytes / cache_bytes)))
    caches = [(ks, kc, vs, vc)] + [(ks.clone(), kc.clone(), vs.clone(), vc.clone()) for _ in range(copies - 1)]
    n_q = 64
    qs = [torch.from_numpy(gen.act_normal(nh, hd, gen.SEED_KV + 10 + k)).to(dev) for k in range(n_q)]
    new_rows = [torch.from_numpy(gen.kv_rows(2 * nkv, hd, gen.SEED_KV + 200 + k)).to(dev) for k in range(n_q)]
    probs = torch.from_numpy(weights).to(dev)
    nb = 1 if mode == qg.PERBLOCK else hd // 32
    slots = 16
    new_s = [torch.zeros(2 * nkv, dtype=torch.int16, device=dev) for _ in range(slots)]
    new_c = [torch.zeros((2 * nkv, hd), dtype=torch.int8, device=dev) for _ in range(slots)]
    qc = [torch.zeros((nh, hd), dtype=torch.int8, device=dev) for _ in range(slots)]
    qsc = [torch.zeros((nh, nb), dtype=torch.int32, device=dev) for _ in range(slots)]
    sc = [torch.zeros((nh, npos), dtype=torch.float32, device=dev) for _ in range(slots)]
    out = [torch.zeros((nh, hd), dtype=torch.float32, device=dev) for _ in range(slots)]

    def append(i, stream=None):
        qg.qg_kv_cache_rows(2 * nkv, hd, new_rows[i % n_q], new_s[i % slots], new_c[i % slots], stream)

    def quant(i, stream=None):
        qg.qg_kv_quantize_heads(mode, nh, hd, qs[i % n_q], qc[i % slots], qsc[i % slots], None, stream)

    def scores(i, stream=None):
        k = caches[i % copies]
        qg.qg_kv_scores(mode, nh, nkv, npos, hd, qc[i % slots], qsc[i % slots], k[0], k[1], sc[i % slots], stream)

    ws = [torch.empty(qg.qg_kv_weighted_workspace(nh, npos, hd), dtype=torch.uint8, device=dev)
          for _ in range(2)]

    def weighted(i, stream=None):
        k = caches[i % copies]
        qg.qg_kv_weighted_with_workspace(nh, nkv, npos, hd, probs, k[2], k[3], out[i % slots], ws[i % 2], stream)

    def weighted_one_pass(i, stream=None):
        k = caches[i % copies]
        qg.qg_kv_weighted(nh, nkv, npos, hd, probs, k[2], k[3], out[i % slots], stream)

    def step(i, stream=None):
        append(i, stream)
        quant(i, stream)
        scores(i, stream)
        weighted(i, stream)

    # algorithmic bytes: every cached code and scale read once (per KV head), the weights,
    # the query, the scores written once, the output; the append's rows in and out
    b_scores = rows * hd + 2 * rows + nh * hd * 4 + nh * npos * 4
    b_weighted = nh * npos * 4 + rows * hd + 2 * rows + nh * hd * 4
    b_step = b_scores + b_weighted + 2 * nkv * hd * (4 + 1) + 2 * 2 * nkv + nh * hd * (4 + 1)
    gsteps = slots
    s = torch.cuda.Stream()

    def graph_of(fn, nsteps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(nsteps):
                fn(i)
        return g

    def replay_ms(graphs):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            torch.cuda.synchronize()
            t0.record(s)
            for g in graphs:
                g.replay()
            t1.record(s)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    def per_call_us(fn, launches):
        g = graph_of(fn, gsteps)
        for _ in range(4):
            g.replay()
        reps = max(1, launches // gsteps)
        return replay_ms([g] * reps) * 1e3 / (reps * gsteps)

    torch.cuda.synchronize()
    step(0)
    torch.cuda.synchronize()
    first_sc = sc[0].cpu().numpy().copy()
    first_out = out[0].cpu().numpy().copy()
    full = graph_of(step, gsteps)
    rest = args.steps % gsteps
    tail = graph_of(step, rest) if rest else None
    for _ in range(max(1, -(-args.warmup // gsteps))):
        full.replay()
    torch.cuda.synchronize()
    ms_total = replay_ms([full] * (args.steps // gsteps) + ([tail] if tail is not None else []))
    ms_per_step = ms_total / args.steps
    us_scores = per_call_us(scores, args.kernel_launches)
    us_weighted = per_call_us(weighted, args.kernel_launches)
    us_weighted_one = per_call_us(weighted_one_pass, args.kernel_launches // 4)
    us_quant = per_call_us(quant, args.kernel_launches // 4)
    us_append = per_call_us(append, args.kernel_launches // 4)
    dom = ("kv_scores_kernel", us_scores, b_scores) if us_scores >= us_weighted else \
        ("kv_weighted_pieces_kernel + kv_weighted_fold_kernel", us_weighted, b_weighted)
    achieved = dom[2] / (dom[1] * 1e-6) / 1e9
    value = b_step / (ms_per_step * 1e-3) / 1e9
    record = {
        "metric": KV_METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "query_heads": nh, "kv_heads": nkv, "positions": npos, "head_size": hd,
            "query_scaling": "perblock" if mode == 0 else "sub32",
            "cache": "cold, rotating over %d copies (%.0f MB)" % (copies, copies * cache_bytes / 1e6)
                     if copies > 1 else "warm, one copy (cache-resident)",
            "step": "qg_kv_cache_rows + qg_kv_quantize_heads + qg_kv_scores + qg_kv_weighted_with_workspace, "
                    "HIP graph replay",
        },
        "algorithmic_bytes_per_step": b_step,
        "kernels_us": {"kv_scores": round(us_scores, 3), "kv_weighted_two_pass": round(us_weighted, 3),
                       "kv_weighted_one_pass": round(us_weighted_one, 3),
                       "kv_quantize_heads": round(us_quant, 3), "kv_cache_rows": round(us_append, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom[0],
                     "algorithmic_bytes_per_launch": dom[2]},
    }
    if not args.no_cpu:
        import oracle

        threads, host = host_threads()
        kh, kcc = oracle.kv_cache_rows(keys.reshape(-1, hd))
        vh, vcc = oracle.kv_cache_rows(vals.reshape(-1, hd))
        kh, kcc = kh.reshape(nkv, npos), kcc.reshape(nkv, npos, hd)
        vh, vcc = vh.reshape(nkv, npos), vcc.reshape(nkv, npos, hd)
        q0 = qs[0].cpu().numpy()
        parity = None

        def step(k):
            nonlocal parity
            qn = qs[k % n_q].cpu().numpy() if k else q0
            oracle.kv_cache_rows(new_rows[k % n_q].cpu().numpy())
            c, m_, e_ = oracle.kv_quantize_heads(qn, mode)
            sc_o = oracle.kv_scores(mode, c, m_, e_, kh, kcc)
            out_o = oracle.kv_weighted(weights, vh, vcc)
            if k == 0 and parity is None:
                parity = bool(np.array_equal(sc_o.view(np.uint32), first_sc.view(np.uint32))
                              and np.array_equal(out_o.view(np.uint32), first_out.view(np.uint32)))

        what = "append, quantize, all scores, weighted sum"
        oracle.set_threads(1)
        s1, d1 = timed_runs(step, args.cpu_seconds / 2)
        oracle.set_threads(threads)
        steps, dt = timed_runs(step, args.cpu_seconds)
        record["cpu_baseline"] = {"value": round(steps * b_step / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"{steps} whole steps ({what}) of the same workload on {threads} "
                                            f"threads, {dt:.1f} s",
                                  "single_thread": {"value": round(s1 * b_step / d1 / 1e9, 3), "unit": "GB/s",
                                                    "threads": 1,
                                                    "sample": f"{s1} whole steps ({what}) on one thread, {d1:.1f} s"},
                                  "host": host}
        record["parity_step0"] = parity
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
