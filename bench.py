#!/usr/bin/env python3
"""Benchmark of the grouped MXFP4 GEMM hot path on one MI355X.

One step = one training step of an MoE expert layer (FC1 of a gated FFN:
32 experts, 4096 tokens x top-8 = 32768 routed rows, K = 4096, N = 3072,
seeded Dirichlet(0.5) routing with empty experts) through every row of the
hot path, all in the library's HIP kernels:

  quantize: X (= A), W and dY, each row-wise and column-wise segment-padded
            in one read (the dual-output quantizer; W with splits N per
            expert gives the forward's W and dgrad's W along N)
  forward : grouped forward (TN)
  dgrad   : grouped input gradient (NN)
  wgrad   : grouped variable-K weight gradient (NT) accumulated in place into
            an fp32 main_grad [32, 3072, 4096]
(--separate-quant: the six single-output quantizer launches instead)

value = GEMM flops of the step (3 x 2 * sum(m_g) * N * K) / step time, in
TFLOPS. Every kernel is also timed alone with HIP events on the stream it is
launched on; the dominant kernel's roofline is reported against MI355X's
published peaks (MXFP4 dense MFMA 10.1 PFLOP/s, HBM3E 8 TB/s).

workloads: on the default run, the a8w4 forward (128 experts, 65536 routed
rows, K=7168, N=2048, MXFP8 x MXFP4) and the blockwise FP8 forward + weight
gradient (64 experts, 32768 rows, K=7168, N=4096) are timed the same way after
the headline and reported under this key, each with its own metric (TFLOPS,
% of the FP8 MFMA peak) and per-kernel times (--no-extra skips them).

Inputs are drawn on the device from one seeded generator per tensor, with
synth's per-tensor seeds (A 1, W 2, dY 3, main_grad 4) and the routing splits
of synth (seed 0).

cpu_baseline: the CPU oracle (NumPy fp64) timed on a bounded sample of the
same step -- one expert with 8192 tokens at the full K and N, all three
passes including quantization -- on this host's cores.

roofline.traffic: HBM bytes per launch of the dominant kernel, read from the
committed rocprofv3 summary profiles/<kernel>_<workload>_traffic.txt (FETCH_SIZE and
WRITE_SIZE per dispatch, each scaled by the same counter's reading for a plain
1 GiB copy); null when that summary was taken from a different kernel source.
kernels.<gemm>.rocprof_mfma_busy_pct (fc1): MFMA-busy of that GEMM from the
committed summary profiles/gemm_fc1_mfma_busy.txt (SQ_VALU_MFMA_BUSY_CYCLES
over GRBM_GUI_ACTIVE x SIMDs), null likewise.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
                       [--workload fc1|a8w4|a8w4_bwd|blockwise|blockwise_dgrad] [--separate-quant]
                       [--codes auto|kblock|rows] [--weight-scales block|mfma] [--rotate N]
       python bench.py --copy-only            (calibration copy for --pmc runs)
       python bench.py --summarize KERNEL STATS_CSV FETCH_CSV WRITE_CSV
                       COPY_FETCH_CSV COPY_WRITE_CSV   (writes the summary text)
       python bench.py --summarize-mfma PMC_CSV        (MFMA-busy summary of the fc1 GEMMs)
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "grouped MXFP4 GEMM TFLOPS (fwd/dgrad/wgrad) and % of MFMA peak, 1 MI355X"
PEAK_MXFP4_TFLOPS = 10100.0   # MI355X dense MXFP4 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=1,
                    help="independent copies of every input and output buffer, cycled step by step (3 or more: "
                         "no step finds the previous step's data in the 256 MB MALL or the L2s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="fc1: skip the a8w4 and blockwise workloads timed beside the headline")
    ap.add_argument("--passes", default="all", help="profiling aid: fwd, dgrad, wgrad or all")
    ap.add_argument("--workload", default="fc1", choices=["fc1", "a8w4", "a8w4_bwd", "blockwise", "blockwise_dgrad"],
                    help="fc1: the a4w4 training step (default, the headline); a8w4: the MXFP8 x MXFP4 forward; "
                         "a8w4_bwd: its input and weight gradients; blockwise: the blockwise FP8 forward + "
                         "weight gradient; blockwise_dgrad: the blockwise input gradient")
    ap.add_argument("--copy-only", action="store_true", help="run only a 1 GiB device copy (counter calibration)")
    ap.add_argument("--codes", default="auto", choices=["auto", "kblock", "rows"],
                    help="MX code layout of the forward / input-gradient operands: 64-byte K blocks "
                         "(MXGG_KBLOCK_ROWS / _COLS) or plain rows; auto: K blocks for the training "
                         "steps (fc1, a8w4_bwd), rows for the a8w4 forward, whose row-wise quantizer "
                         "writes rows faster than it saves in the GEMM")
    ap.add_argument("--weight-scales", default="block", choices=["block", "mfma"],
                    help="fc1: the weights' MX scales block-major or in the MFMA layout")
    ap.add_argument("--separate-quant", action="store_true",
                    help="fc1: single-output quantizers instead of the dual-output ones")
    ap.add_argument("--summarize-mfma", metavar="PMC_CSV",
                    help="print the MFMA-busy summary of the workload's GEMMs from a rocprofv3 counter csv")
    ap.add_argument("--summarize", nargs=6, metavar=("KERNEL", "STATS", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="print the profile summary of KERNEL from rocprofv3 csv outputs")
    return ap.parse_args()


# --- profile summaries --------------------------------------------------------
CSRC = os.path.join(ROOT, "moe_grouped_block_mx_amd", "csrc")
KERNEL_SOURCES = {  # bench kernel name -> (profiled kernel name prefix, source files)
    "fwd": ("void mxgg::grouped_fwd_kernel", ["gemm_mx.hip", "device_common.hpp", "launch.hpp"]),
    "dgrad": ("void mxgg::grouped_dgrad_kernel", ["gemm_mx.hip", "device_common.hpp", "launch.hpp"]),
    "wgrad": ("void mxgg::grouped_wgrad_kernel", ["gemm_mx.hip", "device_common.hpp", "launch.hpp"]),
}
COPY_BYTES = 1 << 30


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_summary_path(kernel, workload="fc1"):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")


def read_traffic(kernel, workload="fc1"):
    """(fetch, write) HBM bytes per launch from the committed summary, or None."""
    path = traffic_summary_path(kernel, workload)
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash(kernel):
        return None
    return float(kv["hbm_fetch_bytes_per_launch"]), float(kv["hbm_write_bytes_per_launch"])


def _counter_per_dispatch(path, name_prefix, counter, pick=None):
    """Counter values (summed over the dispatch's entries) of every dispatch whose
    kernel name starts with name_prefix, in dispatch order."""
    per = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            if not row["Kernel_Name"].startswith(name_prefix) or row["Counter_Name"] != counter:
                continue
            if pick is not None and not pick(row):
                continue
            d = int(row["Dispatch_Id"])
            per[d] = per.get(d, 0.0) + float(row["Counter_Value"])
    return [per[d] for d in sorted(per)]


def summarize(kernel, stats_csv, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload="fc1"):
    prefix = KERNEL_SOURCES[kernel][0]
    wl = "" if workload == "fc1" else f" --workload {workload}"
    sfx = "" if workload == "fc1" else f"_{workload}"
    stats = None
    with open(stats_csv, newline="") as fh:
        for row in csv.DictReader(fh):
            if row["Name"].startswith(prefix):
                stats = row if stats is None else stats
    fetch = _counter_per_dispatch(fetch_csv, prefix, "FETCH_SIZE")
    write = _counter_per_dispatch(write_csv, prefix, "WRITE_SIZE")
    copy_pick = lambda r: "copy" in r["Kernel_Name"].lower()
    cf = _counter_per_dispatch(copy_fetch_csv, "", "FETCH_SIZE", copy_pick)
    cw = _counter_per_dispatch(copy_write_csv, "", "WRITE_SIZE", copy_pick)
    kib = 1024.0
    f_scale = COPY_BYTES / (float(np.median(cf)) * kib)
    w_scale = COPY_BYTES / (float(np.median(cw)) * kib)
    fetch_b = float(np.median(fetch)) * kib * f_scale
    write_b = float(np.median(write)) * kib * w_scale
    lines = [
        f"kernel: {kernel}",
        f"workload: {WORKLOAD_TITLES[workload]} (bench.py{wl or ' default step'})",
        "# commands (GPU run, R = repository root, OUT = an output directory, each rocprofv3 pass in its own process):",
        "#   cd /tmp && export TMPDIR=/tmp",
        f"#   rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_stats{sfx} -o run"
        f" -- python3 $R/bench.py{wl} --steps 5 --warmup 2 --no-cpu-baseline",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/prof_fetch{sfx} -o run"
        f" -- python3 $R/bench.py{wl} --steps 3 --warmup 1 --no-cpu-baseline",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/prof_write{sfx} -o run"
        f" -- python3 $R/bench.py{wl} --steps 3 --warmup 1 --no-cpu-baseline",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/prof_cfetch -o run"
        " -- python3 $R/bench.py --copy-only",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/prof_cwrite -o run"
        " -- python3 $R/bench.py --copy-only",
        f"#   python3 $R/bench.py --summarize {kernel} <prof_stats{sfx} kernel_stats.csv> <prof_fetch{sfx}"
        f" counter_collection.csv> <prof_write{sfx} ...> <prof_cfetch ...> <prof_cwrite ...>{wl}",
        f"source_sha256_16: {source_hash(kernel)}",
        f"kernel_name_prefix: {prefix}",
        f"stats_calls: {stats['Calls'] if stats else 'n/a'}",
        f"stats_average_ns: {stats['AverageNs'] if stats else 'n/a'}",
        f"stats_min_ns: {stats['MinNs'] if stats else 'n/a'}",
        f"stats_max_ns: {stats['MaxNs'] if stats else 'n/a'}",
        f"fetch_size_kib_per_dispatch_median: {float(np.median(fetch)):.1f}",
        f"write_size_kib_per_dispatch_median: {float(np.median(write)):.1f}",
        f"copy_calibration_bytes: {COPY_BYTES}",
        f"copy_fetch_size_kib_median: {float(np.median(cf)):.1f}",
        f"copy_write_size_kib_median: {float(np.median(cw)):.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"hbm_fetch_bytes_per_launch: {fetch_b:.0f}",
        f"hbm_write_bytes_per_launch: {write_b:.0f}",
        f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
    ]
    return "\n".join(lines) + "\n"


SIMDS = 256 * 4  # MI355X: 256 compute units x 4 SIMDs
WORKLOAD_TITLES = {
    "fc1": "MoE FC1 a4w4, 32 experts, 32768 routed rows, K=4096, N=3072",
    "a8w4": "a8w4 forward, 128 experts, 65536 routed rows, K=7168, N=2048",
    "a8w4_bwd": "a8w4 backward (MXFP8 x MXFP4 input gradient, MXFP8 weight gradient), 128 experts, 65536 rows",
    "blockwise": "blockwise FP8 forward and weight gradient, 64 experts, 32768 rows, K=7168, N=4096",
    "blockwise_dgrad": "blockwise FP8 input gradient, 64 experts, 32768 rows, K=7168, N=4096",
}


def mfma_summary_path():
    return os.path.join(ROOT, "profiles", "gemm_fc1_mfma_busy.txt")


def summarize_mfma(pmc_csv, workload="fc1"):
    """MFMA-busy of the fc1 GEMMs from one rocprofv3 pass over
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: busy cycles summed over the
    SIMDs / (GPU-active cycles x SIMDs), the MfmaUtil definition of
    rocprofiler-sdk for gfx950, median over the dispatches. rocprofv3 reports
    each counter summed over its instances, so GRBM_GUI_ACTIVE (one per XCD)
    is divided by the XCD count; XCD and SIMD counts come from the run's
    agent_info.csv."""
    xcc, simds = 8, SIMDS
    info = os.path.join(os.path.dirname(pmc_csv), os.path.basename(pmc_csv).replace("counter_collection", "agent_info"))
    if os.path.exists(info):
        with open(info, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Agent_Type") == "GPU":
                    xcc, simds = int(row["Num_Xcc"]), int(row["Simd_Count"])
    def per_dispatch(prefix, counter, reduce_fn):
        vals = {}
        with open(pmc_csv, newline="") as fh:
            for row in csv.DictReader(fh):
                if row["Kernel_Name"].startswith(prefix) and row["Counter_Name"] == counter:
                    vals.setdefault(int(row["Dispatch_Id"]), []).append(float(row["Counter_Value"]))
        return [reduce_fn(vals[d]) for d in sorted(vals)]

    def durations_ns(prefix):
        dur = {}
        with open(pmc_csv, newline="") as fh:
            for row in csv.DictReader(fh):
                if row["Kernel_Name"].startswith(prefix):
                    dur[int(row["Dispatch_Id"])] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
        return [dur[d] for d in sorted(dur)]
    wl_flag = "" if workload == "fc1" else f" --workload {workload}"
    prof_dir = "prof_mfma" if workload == "fc1" else f"prof_mfma_{workload}"
    lines = [
        f"workload: {WORKLOAD_TITLES[workload]} (bench.py{wl_flag or ' default step'})",
        "# commands (GPU run, R = repository root, OUT = an output directory):",
        "#   cd /tmp && export TMPDIR=/tmp",
        "#   rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $OUT/"
        f"{prof_dir} -o run -- python3 $R/bench.py{wl_flag} --steps 3 --warmup 1 --no-cpu-baseline",
        f"#   python3 $R/bench.py --summarize-mfma <{prof_dir} counter_collection.csv>{wl_flag}",
        f"# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcc} XCDs x {simds} SIMDs), median over dispatches",
        "# (busy cycles accrue per MFMA issued, padding rows included: 32 for a 32x32x64 FP4 MFMA, 64 with an",
        "#  E4M3 operand; the active cycles run at the shader clock under load, so busy x clock / 2.4 GHz is the",
        "#  fraction of that format's peak rate)",
    ]
    # every mxgg GEMM kernel of the run, by name
    names = []
    with open(pmc_csv, newline="") as fh:
        for row in csv.DictReader(fh):
            n = row["Kernel_Name"]
            if n.startswith(("void mxgg::grouped_fwd_kernel", "void mxgg::grouped_dgrad_kernel",
                             "void mxgg::grouped_wgrad_kernel")) and n not in names:
                names.append(n)
    lines.append("# per kernel: dispatches, median mfma_busy %, kernel")
    for n in names:
        busy = per_dispatch(n, "SQ_VALU_MFMA_BUSY_CYCLES", sum)
        active = per_dispatch(n, "GRBM_GUI_ACTIVE", max)
        util = [100.0 * b / (a / xcc * simds) for b, a in zip(busy, active)]
        lines.append(f"#   {len(util):3d} {float(np.median(util)):6.2f}  {n[:140]}")
    if workload != "fc1":
        return "\n".join(lines) + "\n"
    for kernel in ("fwd", "dgrad", "wgrad"):
        prefix = KERNEL_SOURCES[kernel][0]
        busy = per_dispatch(prefix, "SQ_VALU_MFMA_BUSY_CYCLES", sum)
        active = per_dispatch(prefix, "GRBM_GUI_ACTIVE", max)
        util = [100.0 * b / (a / xcc * simds) for b, a in zip(busy, active)]
        dur = durations_ns(prefix)
        # shader clock while the kernel ran: active cycles per XCD over the
        # dispatch's duration (under counter collection)
        sclk = [a / xcc / d for a, d in zip(active, dur) if d > 0]
        lines += [f"{kernel}_source_sha256_16: {source_hash(kernel)}",
                  f"{kernel}_dispatches: {len(util)}",
                  f"{kernel}_mfma_busy_cycles_median: {float(np.median(busy)):.0f}",
                  f"{kernel}_gpu_active_cycles_per_xcd_median: {float(np.median(active)) / xcc:.0f}",
                  f"{kernel}_sclk_ghz_median: {float(np.median(sclk)):.3f}",
                  f"{kernel}_mfma_busy_pct_median: {float(np.median(util)):.2f}"]
    return "\n".join(lines) + "\n"


def read_mfma_busy(kernel):
    """MFMA-busy percent of an fc1 GEMM from the committed summary, or None
    when it was taken from a different kernel source."""
    path = mfma_summary_path()
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get(f"{kernel}_source_sha256_16") != source_hash(kernel):
        return None
    return float(kv[f"{kernel}_mfma_busy_pct_median"])


def copy_only():
    import torch
    dev = torch.device("cuda:0")
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def cpu_baseline(seconds_hint=20.0):
    """The oracle on a bounded sample: one expert with 8192 tokens, K=4096,
    N=3072; fwd + dgrad + wgrad including every quantization."""
    from threadpoolctl import threadpool_info

    from oracle import grouped as og
    from oracle import mx as omx
    from synth import bf16_normal

    m, K, N = 8192, 4096, 3072
    a = bf16_normal((m, K), 1.0, seed=1)
    w = bf16_normal((N, K), 0.02, seed=2)
    dy = bf16_normal((m, N), 1.0, seed=3)
    t0 = time.perf_counter()
    aq, as_ = omx.quantize_rowwise(a, "mxfp4")
    wq, ws = omx.quantize_rowwise(w, "mxfp4")
    og.grouped_fwd(omx.dequantize_rowwise(aq, as_, "mxfp4"), omx.dequantize_rowwise(wq, ws, "mxfp4")[None], [m])
    dq, ds = omx.quantize_rowwise(dy, "mxfp4")
    wcq, wcs = omx.quantize_colwise_segpad(w, [N], "mxfp4")
    og.grouped_dgrad(omx.dequantize_rowwise(dq, ds, "mxfp4"), omx.dequantize_rowwise(wcq, wcs, "mxfp4"), [m])
    dcq, dcs = omx.quantize_colwise_segpad(dy, [m], "mxfp4")
    xcq, xcs = omx.quantize_colwise_segpad(a, [m], "mxfp4")
    og.grouped_wgrad(omx.dequantize_rowwise(dcq, dcs, "mxfp4"), omx.dequantize_rowwise(xcq, xcs, "mxfp4"), [m])
    t = time.perf_counter() - t0
    flops = 3 * 2.0 * m * N * K
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / t / 1e12, "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "seconds": round(t, 3),
            "sample": f"one expert, {m} tokens, K={K}, N={N}: fwd+dgrad+wgrad incl. MX quantization, "
                      f"NumPy fp64 oracle (OpenBLAS {threads} threads, host has {os.cpu_count()} cpus)"}


def build_workload(name, dev, separate_quant=False, weight_scales="block", codes="auto"):
    """Device inputs, the op list and the per-op algorithmic work of one step.

    Returns dict(ops=[(name, kind, fn)], bytes_alg={op: bytes}, flops={op: flops},
    config={...}, peak_tflops=..., dtype=...)."""
    import torch

    import moe_grouped_block_mx_amd as mxg
    from synth import SEED_A, SEED_DY, SEED_MAIN_GRAD, SEED_W, WORKLOADS, splits_for

    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)

    def gen_for(seed):
        # one seeded generator per tensor, with the per-tensor seeds of synth
        # (drawn on the device: the host PCG64 streams of the tests would take
        # minutes at these sizes)
        return torch.Generator(device=dev).manual_seed(seed)

    def normal(shape, std=1.0, seed=SEED_A):
        x = torch.randn(shape, generator=gen_for(seed), device=dev, dtype=torch.float32)
        return (x * std).to(torch.bfloat16) if std != 1.0 else x.to(torch.bfloat16)

    def fp32_normal(shape, seed=SEED_MAIN_GRAD):
        return torch.randn(shape, generator=gen_for(seed), device=dev, dtype=torch.float32)

    # MX code layout: 64-byte K blocks (u8 [bytes per row / 64, rows, 64]) or rows
    if codes == "auto":
        codes = "rows" if name == "a8w4" else "kblock"
    kr = mxg.KBLOCK_ROWS if codes == "kblock" else 0
    kc = mxg.KBLOCK_COLS if codes == "kblock" else 0

    def codes_buf(rows, row_bytes, blocked):
        return torch.empty((row_bytes // 64, rows, 64) if blocked else (rows, row_bytes), **u8)

    if name == "fc1":
        wl = WORKLOADS["fc1"]
        G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
        sp = splits_for("fc1")
        a, w = normal((M, K), seed=SEED_A), normal((G * N, K), wl["w_std"], seed=SEED_W)
        dy, main_grad = normal((M, N), seed=SEED_DY), fp32_normal((G, N, K))
        mpad = mxg.segpad_rows(sp, "mxfp4")
        # MX scales are block-major: [blocks of 32 along the contraction, rows
        # rounded up to a multiple of 4]
        R4 = mxg.mx_scale_stride(M)
        aq, as_ = codes_buf(M, K // 2, kr), torch.empty((K // 32, R4), **u8)
        # the weights' scales block-major, or in the MFMA layout ([K/128,
        # G*N*4] row-wise, [G*N/128, K*4] column-wise)
        lay = mxg.LAYOUT_MFMA if weight_scales == "mfma" else mxg.LAYOUT_BLOCK_MAJOR
        wfmt = mxg.MXFP4 | lay
        xf, dyf = mxg.MXFP4 | kr, mxg.MXFP4 | kr  # activations: blocked row-wise codes, plain column codes
        ws_shape = (K // 128, G * N * 4) if lay else (K // 32, G * N)
        wcs_shape = (G * N // 128, K * 4) if lay else (G * N // 32, K)
        wq, ws = codes_buf(G * N, K // 2, kr), torch.empty(ws_shape, **u8)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        dq, ds = codes_buf(M, N // 2, kr), torch.empty((N // 32, R4), **u8)
        wcq, wcs = codes_buf(K, G * N // 2, kc), torch.empty(wcs_shape, **u8)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dcq, dcs = torch.empty((N, mpad // 2), **u8), torch.empty((mpad // 32, N), **u8)
        xcq, xcs = torch.empty((K, mpad // 2), **u8), torch.empty((mpad // 32, K), **u8)
        wsp = [N] * G
        dual_ops = [
            ("quant_X_dual", "quant", lambda: mxg.quantize_dual(a, sp, xf, q_row=aq, s_row=as_, q_col=xcq,
                                                                s_col=xcs)),
            ("quant_W_dual", "quant", lambda: mxg.quantize_dual(w, wsp, wfmt | kr | kc, q_row=wq, s_row=ws,
                                                                q_col=wcq, s_col=wcs)),
            ("fwd", "gemm", lambda: mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=xf, w_fmt=wfmt | kr, out=y)),
            ("quant_dY_dual", "quant", lambda: mxg.quantize_dual(dy, sp, dyf, q_row=dq, s_row=ds, q_col=dcq,
                                                                 s_col=dcs)),
            ("dgrad", "gemm", lambda: mxg.grouped_dgrad(dq, ds, wcq, wcs, sp, N, K, fmt=wfmt | kr | kc, dx=dx)),
            ("wgrad", "gemm", lambda: mxg.grouped_wgrad(dcq, dcs, xcq, xcs, sp, N, K, mpad, main_grad,
                                                        accumulate=True)),
        ]
        ops = [
            ("quant_A_row", "quant", lambda: mxg.quantize_rowwise(a, xf, q=aq, scales=as_)),
            ("quant_W_row", "quant", lambda: mxg.quantize_rowwise(w, wfmt | kr, q=wq, scales=ws)),
            ("fwd", "gemm", lambda: mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=xf, w_fmt=wfmt | kr, out=y)),
            ("quant_dY_row", "quant", lambda: mxg.quantize_rowwise(dy, dyf, q=dq, scales=ds)),
            ("quant_W_col", "quant", lambda: mxg.quantize_colwise_segpad(w, [N] * G, wfmt | kc, q=wcq, scales=wcs)),
            ("dgrad", "gemm", lambda: mxg.grouped_dgrad(dq, ds, wcq, wcs, sp, N, K, fmt=wfmt | kr | kc, dx=dx)),
            ("quant_dY_col", "quant", lambda: mxg.quantize_colwise_segpad(dy, sp, "mxfp4", q=dcq, scales=dcs)),
            ("quant_X_col", "quant", lambda: mxg.quantize_colwise_segpad(a, sp, "mxfp4", q=xcq, scales=xcs)),
            ("wgrad", "gemm", lambda: mxg.grouped_wgrad(dcq, dcs, xcq, xcs, sp, N, K, mpad, main_grad,
                                                        accumulate=True)),
        ]
        nz = int((sp > 0).sum())
        q4 = 0.5 + 1 / 32
        bytes_alg = {
            "quant_A_row": M * K * (2 + q4), "quant_W_row": G * N * K * (2 + q4),
            "fwd": M * K * q4 + nz * N * K * q4 + M * N * 2,
            "quant_dY_row": M * N * (2 + q4), "quant_W_col": G * N * K * (2 + q4),
            "dgrad": M * N * q4 + nz * N * K * q4 + M * K * 2,
            "quant_dY_col": M * N * 2 + mpad * N * q4, "quant_X_col": M * K * 2 + mpad * K * q4,
            "wgrad": mpad * (N + K) * q4 + nz * N * K * 4 * 2,
            "quant_X_dual": M * K * (2 + q4) + mpad * K * q4, "quant_W_dual": G * N * K * (2 + 2 * q4),
            "quant_dY_dual": M * N * (2 + q4) + mpad * N * q4,
        }
        if not separate_quant:
            ops = dual_ops
        config = {"workload": "MoE FC1 a4w4 training step (fwd+dgrad+wgrad with MX quantization)",
                  "quantizers": "separate" if separate_quant else "dual-output",
                  "weight_scales": "MFMA layout" if lay else "block-major",
                  "codes": "64-byte K blocks (fwd/dgrad operands)" if kr else "rows",
                  "experts": G, "rows": M, "K": K, "N": N, "nonempty_experts": nz,
                  "max_split": int(sp.max()), "mpad": mpad, "routing": "Dirichlet(0.5), 3 zeroed, seed 0"}
        return dict(ops=ops, bytes_alg=bytes_alg, flops={"fwd": 2.0 * M * N * K, "dgrad": 2.0 * M * N * K,
                                                          "wgrad": 2.0 * M * N * K},
                    config=config, peak_tflops=PEAK_MXFP4_TFLOPS, dtype="mxfp4", hbm_gemms={"wgrad"},
                    metric=METRIC)

    if name == "a8w4":
        wl = WORKLOADS["a8w4"]
        G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
        sp = splits_for("a8w4")
        a, w = normal((M, K), seed=SEED_A), normal((G * N, K), wl["w_std"], seed=SEED_W)
        aq, as_ = codes_buf(M, K, kr), torch.empty((K // 32, mxg.mx_scale_stride(M)), **u8)
        wq, ws = codes_buf(G * N, K // 2, kr), torch.empty((K // 32, G * N), **u8)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        af, wf = mxg.MXFP8 | kr, mxg.MXFP4 | kr
        ops = [
            ("quant_A_row", "quant", lambda: mxg.quantize_rowwise(a, af, q=aq, scales=as_)),
            ("quant_W_row", "quant", lambda: mxg.quantize_rowwise(w, wf, q=wq, scales=ws)),
            ("fwd", "gemm", lambda: mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt=af, w_fmt=wf, out=y)),
        ]
        nz = int((sp > 0).sum())
        bytes_alg = {"quant_A_row": M * K * (2 + 1 + 1 / 32), "quant_W_row": G * N * K * (2 + 0.5 + 1 / 32),
                     "fwd": M * K * (1 + 1 / 32) + nz * N * K * (0.5 + 1 / 32) + M * N * 2}
        config = {"workload": "MoE a8w4 forward (MXFP8 activations x MXFP4 weights, with quantization)",
                  "codes": "64-byte K blocks" if kr else "rows", "experts": G, "rows": M, "K": K, "N": N, "nonempty_experts": nz, "max_split": int(sp.max()),
                  "routing": "Zipf(1.1), 8 zeroed, seed 0"}
        return dict(ops=ops, bytes_alg=bytes_alg, flops={"fwd": 2.0 * M * N * K}, config=config,
                    peak_tflops=PEAK_FP8_TFLOPS, dtype="mxfp8xmxfp4", hbm_gemms=set(),
                    metric="grouped a8w4 GEMM TFLOPS (fwd) and % of FP8 MFMA peak, 1 MI355X")

    if name == "a8w4_bwd":
        # the backward of a8w4 training at the a8w4 shapes: dY quantized to
        # MXFP8 both ways, W along N to MXFP4, X column-wise to MXFP8
        wl = WORKLOADS["a8w4"]
        G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
        sp = splits_for("a8w4")
        mpad = mxg.segpad_rows(sp, "mxfp8")
        a, w = normal((M, K), seed=SEED_A), normal((G * N, K), wl["w_std"], seed=SEED_W)
        dy, main_grad = normal((M, N), seed=SEED_DY), fp32_normal((G, N, K))
        R4 = mxg.mx_scale_stride(M)
        dq, ds = codes_buf(M, N, kr), torch.empty((N // 32, R4), **u8)
        dcq, dcs = torch.empty((N, mpad), **u8), torch.empty((mpad // 32, N), **u8)
        wcq, wcs = codes_buf(K, G * N // 2, kc), torch.empty((G * N // 32, K), **u8)
        xcq, xcs = torch.empty((K, mpad), **u8), torch.empty((mpad // 32, K), **u8)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        ops = [
            ("quant_dY_dual", "quant", lambda: mxg.quantize_dual(dy, sp, mxg.MXFP8 | kr, q_row=dq, s_row=ds,
                                                                 q_col=dcq, s_col=dcs)),
            ("quant_W_col", "quant", lambda: mxg.quantize_colwise_segpad(w, [N] * G, mxg.MXFP4 | kc, q=wcq,
                                                                         scales=wcs)),
            ("dgrad", "gemm", lambda: mxg.grouped_dgrad(dq, ds, wcq, wcs, sp, N, K, fmt=mxg.MXFP8 | kr | kc,
                                                        dx=dx)),
            ("quant_X_col", "quant", lambda: mxg.quantize_colwise_segpad(a, sp, "mxfp8", q=xcq, scales=xcs)),
            ("wgrad", "gemm", lambda: mxg.grouped_wgrad(dcq, dcs, xcq, xcs, sp, N, K, mpad, main_grad,
                                                        accumulate=True, fmt="mxfp8")),
        ]
        nz = int((sp > 0).sum())
        q8, q4 = 1 + 1 / 32, 0.5 + 1 / 32
        bytes_alg = {"quant_dY_dual": M * N * (2 + q8) + mpad * N * q8, "quant_W_col": G * N * K * (2 + q4),
                     "dgrad": M * N * q8 + nz * N * K * q4 + M * K * 2,
                     "quant_X_col": M * K * 2 + mpad * K * q8,
                     "wgrad": mpad * (N + K) * q8 + nz * N * K * 4 * 2}
        config = {"workload": "MoE a8w4 backward (input gradient MXFP8 x MXFP4, weight gradient MXFP8 x MXFP8 "
                              "with fp32 main_grad accumulate, with quantization)",
                  "codes": "64-byte K blocks (dgrad operands)" if kr else "rows", "experts": G, "rows": M, "K": K, "N": N, "nonempty_experts": nz, "max_split": int(sp.max()),
                  "mpad": mpad, "routing": "Zipf(1.1), 8 zeroed, seed 0"}
        return dict(ops=ops, bytes_alg=bytes_alg, flops={"dgrad": 2.0 * M * N * K, "wgrad": 2.0 * M * N * K},
                    config=config, peak_tflops=PEAK_FP8_TFLOPS, dtype="mxfp8xmxfp4", hbm_gemms={"wgrad"},
                    metric="grouped a8w4 backward GEMM TFLOPS (dgrad/wgrad) and % of FP8 MFMA peak, 1 MI355X")

    if name == "blockwise_dgrad":
        # the blockwise input gradient at the blockwise shapes: dY 1x128 along
        # N, and the 128x128 weight blocks transposed (same codes and scales)
        wl = WORKLOADS["blockwise"]
        G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
        sp = splits_for("blockwise")
        w, dy = normal((G * N, K), wl["w_std"], seed=SEED_W), normal((M, N), seed=SEED_DY)
        wq, ws = mxg.quantize_rowwise(w, "fp8_128x128_p2")
        del w
        # blockwise codes in 64-byte K blocks, 1x128 scales block-major
        dq, ds = torch.empty((N // 64, M, 64), **u8), torch.empty((N // 128, M), **f32)
        tq, ts = torch.empty((N // 64, G * K, 64), **u8), torch.empty((G * K // 128, N // 128), **f32)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        ops = [
            ("quant_dY_1x128", "quant", lambda: mxg.quantize_rowwise(dy, "fp8_1x128_p2", q=dq, scales=ds)),
            ("transpose_W", "quant", lambda: mxg.transpose_128x128(wq, ws, G, N, K, wt_q=tq, wt_s=ts)),
            ("dgrad", "gemm", lambda: mxg.grouped_dgrad(dq, ds, tq, ts, sp, N, K, fmt="fp8_1x128_p2", dx=dx)),
        ]
        nz = int((sp > 0).sum())
        q8 = 1 + 4 / 128
        bytes_alg = {"quant_dY_1x128": M * N * (2 + q8), "transpose_W": G * N * K * 2 + G * N * K / 16384 * 8,
                     "dgrad": M * N * q8 + nz * N * K + M * K * 2}
        config = {"workload": "MoE blockwise FP8 input gradient (1x128 dY x transposed 128x128 weight blocks, "
                              "power-of-two scales)",
                  "experts": G, "rows": M, "K": K, "N": N, "nonempty_experts": nz, "max_split": int(sp.max()),
                  "routing": "Dirichlet(1), seed 0"}
        return dict(ops=ops, bytes_alg=bytes_alg, flops={"dgrad": 2.0 * M * N * K}, config=config,
                    peak_tflops=PEAK_FP8_TFLOPS, dtype="fp8_e4m3", hbm_gemms=set(),
                    metric="grouped blockwise FP8 input-gradient GEMM TFLOPS and % of FP8 MFMA peak, 1 MI355X")

    if name == "blockwise":
        wl = WORKLOADS["blockwise"]
        G, M, K, N = wl["G"], wl["M"], wl["K"], wl["N"]
        sp = splits_for("blockwise")
        a, w = normal((M, K), seed=SEED_A), normal((G * N, K), wl["w_std"], seed=SEED_W)
        dy = normal((M, N), seed=SEED_DY)
        mpad = mxg.segpad_rows(sp, "fp8_1x128")
        # blockwise codes in 64-byte K blocks, 1x128 scales block-major
        aq, as_ = torch.empty((K // 64, M, 64), **u8), torch.empty((K // 128, M), **f32)
        wq, ws = torch.empty((K // 64, G * N, 64), **u8), torch.empty((G * N // 128, K // 128), **f32)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        # column-wise 1x128 codes in 64-byte K blocks, scales block-major
        dcq, dcs = torch.empty((mpad // 64, N, 64), **u8), torch.empty((mpad // 128, N), **f32)
        xcq, xcs = torch.empty((mpad // 64, K, 64), **u8), torch.empty((mpad // 128, K), **f32)
        dw = torch.empty((G, N, K), dtype=torch.bfloat16, device=dev)
        ops = [
            # power-of-two scales (the blockwise default), declared by the _p2
            # formats so the forward and the weight gradient apply them inside
            # the MFMA
            # X both ways from one read (the blockwise dual quantizer)
            ("quant_X_dual", "quant", lambda: mxg.quantize_dual(a, sp, "fp8_1x128_p2", q_row=aq, s_row=as_, q_col=xcq,
                                                                s_col=xcs)),
            ("quant_W_128x128", "quant", lambda: mxg.quantize_rowwise(w, "fp8_128x128_p2", q=wq, scales=ws)),
            ("fwd", "gemm", lambda: mxg.grouped_fwd(aq, as_, wq, ws, sp, N, K, a_fmt="fp8_1x128_p2",
                                                    w_fmt="fp8_128x128_p2", out=y)),
            ("quant_dY_col", "quant", lambda: mxg.quantize_colwise_segpad(dy, sp, "fp8_1x128_p2", q=dcq, scales=dcs)),
            ("wgrad", "gemm", lambda: mxg.grouped_wgrad(dcq, dcs, xcq, xcs, sp, N, K, mpad, dw, accumulate=False,
                                                        fmt="fp8_1x128_p2")),
        ]
        nz = int((sp > 0).sum())
        q8 = 1 + 4 / 128
        bytes_alg = {"quant_X_dual": M * K * (2 + q8) + mpad * K * q8, "quant_W_128x128": G * N * K * (2 + 1),
                     "fwd": M * K * q8 + nz * N * K * 1 + M * N * 2,
                     "quant_dY_col": M * N * 2 + mpad * N * q8,
                     "wgrad": mpad * (N + K) * q8 + G * N * K * 2}
        config = {"workload": "MoE blockwise FP8 forward + weight gradient (1x128 / 128x128 fp32 scales, "
                              "power-of-two; bf16 weight gradient, overwrite)",
                  "experts": G, "rows": M, "K": K, "N": N, "nonempty_experts": nz, "max_split": int(sp.max()),
                  "mpad": mpad, "routing": "Dirichlet(1), seed 0"}
        return dict(ops=ops, bytes_alg=bytes_alg, flops={"fwd": 2.0 * M * N * K, "wgrad": 2.0 * M * N * K},
                    config=config, peak_tflops=PEAK_FP8_TFLOPS, dtype="fp8_e4m3", hbm_gemms={"wgrad"},
                    metric="grouped blockwise FP8 GEMM TFLOPS (fwd/wgrad) and % of FP8 MFMA peak, 1 MI355X")
    raise SystemExit(f"unknown workload {name!r}")


def measure(W, args, dev, sets=None):
    """Warm-up, then `steps` timed steps of the workload's ops between device
    synchronizations, then `steps` more with HIP events around every launch on
    the stream it is launched on. With `sets` (independent copies of the
    workload's buffers), step i runs on copy i % len(sets). Returns (seconds
    per step, per-kernel dict, roofline dict of the kernel with the largest
    time)."""
    import torch

    ops, bytes_alg, flops = W["ops"], W["bytes_alg"], W["flops"]
    op_sets = [X["ops"] for X in sets] if sets else [ops]
    stream = torch.cuda.current_stream(dev)
    ev = {name: [] for name, _, _ in ops}
    n_step = [0]

    def step(record):
        cur = op_sets[n_step[0] % len(op_sets)]
        n_step[0] += 1
        for name, _, fn in cur:
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev[name].append((e0, e1))
            else:
                fn()

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(False)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()

    per = {}
    for name, kind, _ in ops:
        ms = [e0.elapsed_time(e1) for e0, e1 in ev[name]]
        d = float(np.mean(ms)) * 1e-3
        entry = {"ms": round(d * 1e3, 4), "ms_median": round(float(np.median(ms)), 4),
                 "ms_min": round(float(np.min(ms)), 4)}
        entry["GBs_alg"] = round(bytes_alg[name] / d / 1e9, 1)
        entry["frac_hbm"] = round(bytes_alg[name] / d / 1e9 / PEAK_HBM_GBS, 4)
        if kind == "gemm":
            entry["TFLOPS"] = round(flops[name] / d / 1e12, 1)
            entry["pct_mfma_peak"] = round(100 * flops[name] / d / 1e12 / W["peak_tflops"], 2)
        per[name] = entry

    dom = max(per, key=lambda k: per[k]["ms"])
    dkind = dict((n, k) for n, k, _ in ops)[dom]
    d = per[dom]["ms"] * 1e-3
    if dkind == "gemm" and dom not in W["hbm_gemms"]:
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(flops[dom] / d / 1e12, 1),
                "peak": W["peak_tflops"], "unit": "TFLOP/s"}
        per_unit = flops[dom]
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(bytes_alg[dom] / d / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        per_unit = bytes_alg[dom]
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["per_launch_algorithmic"] = per_unit
    return t_step, per, roof


# workloads timed beside the headline one on the default run (their own
# metrics, on the same JSON line)
EXTRA_WORKLOADS = ("a8w4", "blockwise")


def main():
    args = parse()
    if args.summarize:
        sys.stdout.write(summarize(*args.summarize, workload=args.workload))
        return
    if args.summarize_mfma:
        sys.stdout.write(summarize_mfma(args.summarize_mfma, args.workload))
        return
    if args.copy_only:
        copy_only()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the path would shard by expert (each GPU running these "
                                   "kernels on its own experts), which is not implemented here",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Ws = [build_workload(args.workload, dev, args.separate_quant, args.weight_scales, args.codes)
          for _ in range(args.rotate)]
    if args.passes != "all":
        keep = {"fwd": {"quant_A_row", "quant_W_row", "quant_X_dual", "quant_W_dual", "fwd"},
                "dgrad": {"quant_dY_row", "quant_W_col", "quant_dY_dual", "quant_W_dual", "dgrad"},
                "wgrad": {"quant_dY_col", "quant_X_col", "quant_X_dual", "quant_dY_dual", "wgrad"}}[args.passes]
        for X in Ws:
            X["ops"] = [o for o in X["ops"] if o[0] in keep]
    W = Ws[0]
    flops = W["flops"]
    t_step, per, roof = measure(W, args, dev, Ws)
    if args.workload == "fc1" and args.passes == "all" and not args.separate_quant:
        for name in per:
            if "TFLOPS" in per[name]:
                per[name]["rocprof_mfma_busy_pct"] = read_mfma_busy(name)
    step_flops = sum(flops[n] for n, k, _ in W["ops"] if k == "gemm")
    value = step_flops / t_step / 1e12
    tr = read_traffic(roof["kernel"]) if (args.passes == "all" and args.workload == "fc1") else None
    roof["traffic"] = None if tr is None else round(tr[0] + tr[1])
    per_unit = roof.pop("per_launch_algorithmic")
    roof["per_launch_algorithmic"] = per_unit

    config = dict(W["config"])
    config["passes"] = args.passes
    config["buffer_sets"] = args.rotate
    out = {
        "metric": W["metric"],
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W["dtype"],
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "kernels": per,
        "pct_mfma_peak_step": round(100 * value / W["peak_tflops"], 2),
    }
    if args.workload == "fc1" and args.passes == "all" and not args.separate_quant and not args.no_extra:
        # the a8w4 forward and the blockwise FP8 forward + weight gradient at
        # their own workload sizes, against the FP8 MFMA peak
        del W, Ws
        torch.cuda.empty_cache()
        extra = {}
        for name in EXTRA_WORKLOADS:
            Xs = [build_workload(name, dev, codes=args.codes) for _ in range(args.rotate)]
            X = Xs[0]
            t_x, per_x, roof_x = measure(X, args, dev, Xs)
            tr_x = read_traffic(roof_x["kernel"], name)
            roof_x["traffic"] = None if tr_x is None else round(tr_x[0] + tr_x[1])
            fl = sum(X["flops"][n] for n, k, _ in X["ops"] if k == "gemm")
            extra[name] = {"metric": X["metric"], "value": round(fl / t_x / 1e12, 2), "unit": "TFLOPS",
                           "ms_per_step": round(t_x * 1e3, 4), "dtype": X["dtype"],
                           "config": dict(X["config"], buffer_sets=args.rotate),
                           "pct_mfma_peak_step": round(100 * fl / t_x / 1e12 / X["peak_tflops"], 2),
                           "roofline": roof_x, "kernels": per_x}
            del X, Xs
            torch.cuda.empty_cache()
        out["workloads"] = extra
    if not args.no_cpu_baseline and args.workload == "fc1":
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
