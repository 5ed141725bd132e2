"""Throughput of the RVQ hot path (encode + decode) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batched]

One step = ``rvq_prepare_codebooks`` (codebooks scaled and rounded to fp16,
with their half-norms), ``rvq_encode_prepared`` (codes + final residual;
fp16 scores with exact re-rank, batches of up to 8192 frames with every
stage's codebook split over a workgroup's wavefronts) and ``rvq_decode``
(codes -> reconstruction) over the whole batch,
inputs and outputs resident in HBM. Before the steps, the side
measurements run (about a second of GPU load, so the clocks have settled
when the steps start): the ceilings of this GPU from ``librvq_probe.so``
(random 256 B row gathers from a table of the decode's working set, fp16
and fp32 matrix cores, a 1 GiB copy and fill), the decode alone warm and
after a 1 GiB flush (median and min of 20), and the fp32-scored encode.
Then W untimed steps (100 by default), then K timed steps (100) between
``torch.cuda.synchronize()`` calls. Per-launch kernel times come from HIP
events recorded on the stream the kernels run on (torch's current
stream, which is the stream handed to the C ABI): around every timed
encode (the roofline's kernel), and around the preparation and the decode
on 20 instrumented steps after the timed ones, since each recorded event
adds a few microseconds between the kernels of a step.

Prints one JSON line with the throughput, the roofline of the dominant
kernel (the encode on the fp16 matrix cores: spec and measured peaks,
contraction dtype, the float64 decision), the same encode with fp32 scores
against the fp32 matrix-core roofline, the decode's HBM roofline with its
row-gather ceiling and warm / cold times, sampled parity against the CPU
oracle, and the oracle's own throughput on a bounded sample of the same
workload (``cpu_baseline``).

``--summarize-profiles DIR`` turns the rocprofv3 runs listed in
PROFILE_COMMANDS into the summaries under ``profiles/``.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

_ROOT = os.path.dirname(os.path.abspath(__file__))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import rvq_workloads as W  # noqa: E402

METRIC = "RVQ encode + decode frames/sec (Q=8,K=1024,D=64 fp32); % MFMA / HBM roofline"
PEAK_FP32_MFMA_TFLOPS = 157.3      # MI355X dense fp32 matrix peak
PEAK_BF16_MFMA_TFLOPS = 2500.0     # MI355X dense bf16 (and fp16) matrix peak
PEAK_F16_MFMA_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E
N_XCD, N_SIMD = 8, 1024            # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
COPY_BYTES = 512 << 20             # size of the counter-calibration copy
FLUSH_BYTES = 1 << 30             # written between cold decode launches to evict L2 / MALL
SPLIT_MAX_FRAMES = 8192    # prepared encodes of up to this many frames take the split-codebook kernel

CSRC = os.path.join(_ROOT, "residual_vector_quantization_amd", "csrc")
# kernel kind -> sources whose text defines it (hashed to detect stale counters)
KERNEL_SOURCES = {
    "encode_f16": ["encode_f16.hip", "encode_common.h", "prepared.h"],
    "encode_f16_split": ["encode_f16.hip", "encode_common.h", "prepared.h"],
    "encode_fp32": ["encode.hip", "encode_common.h"],
    "decode": ["decode.hip"],
    "linear_in": ["linear.hip"],
    "linear_out": ["linear.hip"],
    "linear_out_touch": ["linear.hip"],
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks settle after roughly 50 ms of load: 3 warm-up + 20 timed
    # steps measured the batched step 17% slower than 100 + 100 or 200 + 200
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="batched", choices=list(W.WORKLOADS))
    p.add_argument("--fp32-steps", type=int, default=20,
                   help="launches of the fp32-scored encode timed before the main steps")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the CPU-oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain elementwise copy of 512 MiB (for HBM counter scaling)")
    p.add_argument("--gather-probe", metavar="OUT_MD",
                   help="run the ceiling probes (row gathers over 0.25..16 MiB tables, matrix cores, HBM copy), "
                        "write a summary to OUT_MD, then exit")
    p.add_argument("--no-probes", action="store_true",
                   help="skip the live ceiling probes and the cold / warm decode timing")
    p.add_argument("--gather-sweep", metavar="OUT_MD",
                   help="time rvq_decode at Q=32, N=720000 over codebook sizes 0.25..16 MiB, write a "
                        "summary of the row-gather rates to OUT_MD, then exit")
    p.add_argument("--summarize-trace", metavar="DIR",
                   help="turn a rocprofv3 --kernel-trace --stats CSV directory of --workload into "
                        "profiles/<workload>_rocprof.md (per-kernel times and rates), then exit")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="turn rocprofv3 CSV output under DIR (trace/, fetch/, write/, mfma/) into the "
                        "summaries under profiles/, then exit")
    return p.parse_args()


def _code_only(text):
    """Source text without comments and blank lines: edits to comments leave the hash alone."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    return "\n".join(ln for ln in lines if ln.strip())


def source_hash(kind, read=None):
    """SHA-256 of the code (comments stripped) of the sources that define a kernel kind."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        text = read(name) if read else open(os.path.join(CSRC, name)).read()
        h.update(_code_only(text).encode())
    return h.hexdigest()


def recorded_traffic(kind, workload):
    """HBM bytes per launch from a committed counter summary, or None if the kernel changed since."""
    path = os.path.join(_ROOT, "profiles", f"{kind}_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_hash(kind):
        return None
    return rec.get("traffic_bytes_per_launch")


# ---------------------------------------------------------------- profiles

PROFILE_COMMANDS = """cd /tmp && export TMPDIR=/tmp   # R = repository root
rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof_{wl}/trace -o bench -- python3 $R/bench.py --workload {wl} --no-cpu-baseline --no-probes
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof_{wl}/fetch -o bench -- python3 $R/bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --no-probes --calibrate-copy
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof_{wl}/write -o bench -- python3 $R/bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --no-probes --calibrate-copy
rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE --output-format csv -d $R/gpurun_out/prof_{wl}/mfma -o bench -- python3 $R/bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --no-probes
rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_MFMA SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $R/gpurun_out/prof_{wl}/valu -o bench -- python3 $R/bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --no-probes
python3 $R/bench.py --workload {wl} --summarize-profiles $R/gpurun_out/prof_{wl}"""


def _csv(dirname, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(dirname, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {dirname}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _kernel_of(name):
    if "linear_in_kernel" in name:
        return "linear_in"
    if "linear_out_kernel" in name or "linear_out_split_kernel" in name or "linear_out_res_kernel" in name:
        return "linear_out"
    if "touch_kernel" in name:
        return "linear_out_touch"   # fc2's inputs read once ahead of it
    if "encode_f16_kernel" in name:
        return "encode_f16"
    if "encode_f16_ksplit_kernel" in name:
        return "encode_f16_split"
    if "encode_bf16_ksplit_kernel" in name or "encode_bf16_kernel" in name:
        return "encode_bf16_onthefly"   # codebooks split in every workgroup (no prepared layout)
    if "encode_kernel" in name:
        return "encode_fp32"
    if "decode_kernel" in name or "decode_tiled_kernel" in name:
        return "decode"
    if "prepare_kernel" in name:
        return "prepare"
    if "elementwise" in name and "MulFunctor" in name:
        return "copy"
    if "gather_probe_kernel" in name:
        return "calib_gather"
    return None


def _counter_means(rows, counter):
    """Mean value of `counter` per dispatch, for each kernel kind (copy: the calibration mul)."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        kind = _kernel_of(r["Kernel_Name"])
        if kind:
            per.setdefault(kind, {}).setdefault(r["Dispatch_Id"], 0.0)
            per[kind][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def summarize_profiles(w, src_dir):
    """Writes profiles/encode_decode_<workload>_rocprof.md and <kernel>_<workload>_hbm_counters.json."""
    out_dir = os.path.join(_ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    cmds = PROFILE_COMMANDS.format(wl=w.name)
    n, q, k, d = w.n_frames, w.n_stages, w.n_codes, w.dim
    enc_flop = 2.0 * q * k * d * n
    dec_bytes = (4.0 * q + 4.0 * d) * n

    stats = _csv(os.path.join(src_dir, "trace"), "kernel_stats.csv")
    lines = [f"# rocprofv3: encode + decode, workload `{w.name}`", "",
             f"Workload: {w.description}.", "", "Commands (the summary is the last line's output):", "",
             "```", cmds, "```", "",
             "## Kernel trace", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    avg = {}
    for r in stats:
        kind = _kernel_of(r["Name"]) or r["Name"][:40]
        a = float(r["AverageNs"]) / 1e3
        avg[kind] = a
        lines.append(f"| {kind} | {r['Calls']} | {a:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines.append("")
    # the bench times only its last `steps` launches (after the warm-up), so the
    # same average over the trace's last launches is what its line reports
    trace_rows = _csv(os.path.join(src_dir, "trace"), "kernel_trace.csv")
    steps = 100
    for kind in ("encode_f16", "decode", "prepare"):
        durs = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                for r in trace_rows if _kernel_of(r["Kernel_Name"]) == kind]
        durs.sort()
        if len(durs) > steps:
            tail = [d for _, d in durs[-steps:]]
            lines.append(f"- {kind}: average over the last {steps} launches (the timed steps) "
                         f"{sum(tail) / len(tail) / 1e3:.1f} us; over all {len(durs)} launches "
                         f"{sum(d for _, d in durs) / len(durs) / 1e3:.1f} us")
    if "encode_f16" in avg:
        t = avg["encode_f16"]
        lines.append(f"- encode_f16 (prepared codebooks): {enc_flop:.4g} flop per launch (2QKD per frame, "
                     f"on the fp16 matrix cores) / {t:.1f} us = {enc_flop / t / 1e6:.1f} TFLOP/s "
                     f"({enc_flop / t / 1e6 / PEAK_F16_MFMA_TFLOPS:.1%} of {PEAK_F16_MFMA_TFLOPS:.0f} fp16; "
                     f"{enc_flop / t / 1e6 / PEAK_FP32_MFMA_TFLOPS:.2f}x the {PEAK_FP32_MFMA_TFLOPS} fp32 matrix "
                     f"peak); matrix steps issued {enc_flop * (d + 16) / d:.4g} flop (2QK(D+16) per frame, "
                     f"the half-norm step included).")
    if "encode_fp32" in avg:
        t = avg["encode_fp32"]
        lines.append(f"- encode_fp32: {enc_flop:.4g} flop per launch (2QKD per frame) / {t:.1f} us = "
                     f"{enc_flop / t / 1e6:.1f} TFLOP/s ({enc_flop / t / 1e6 / PEAK_FP32_MFMA_TFLOPS:.1%} "
                     f"of {PEAK_FP32_MFMA_TFLOPS} fp32 MFMA).")
    if "decode" in avg:
        t = avg["decode"]
        lines.append(f"- decode: {dec_bytes:.4g} bytes per launch ((4Q+4D) per frame) / {t:.1f} us = "
                     f"{dec_bytes / t / 1e3:.0f} GB/s ({dec_bytes / t / 1e3 / PEAK_HBM_GBPS:.1%} of "
                     f"{PEAK_HBM_GBPS:.0f} GB/s HBM).")
    if w.hidden:
        lin_bytes = (4.0 * w.hidden + 4.0 * d) * n
        lin_flop = 2.0 * w.hidden * d * n
        for kind, what in (("linear_in", "fc, hidden -> 64: h rows in, latent rows out"),
                           ("linear_out", "fc2, 64 -> hidden: latent rows in, h rows out")):
            if kind in avg:
                t = avg[kind]
                lines.append(f"- {kind} ({what}): {lin_bytes:.4g} bytes per launch ((4 hidden + 4D) per frame) / "
                             f"{t:.1f} us = {lin_bytes / t / 1e3:.0f} GB/s ({lin_bytes / t / 1e3 / PEAK_HBM_GBPS:.1%} "
                             f"of {PEAK_HBM_GBPS:.0f} GB/s HBM); {lin_flop / t / 1e6:.1f} TFLOP/s of fp32 work "
                             f"(2 hidden D per frame).")
        if "linear_out" in avg and "linear_out_touch" in avg:
            t = avg["linear_out"] + avg["linear_out_touch"]
            lines.append(f"- fc2 with the read of its inputs ahead of it (linear_out_touch, {avg['linear_out_touch']:.1f}"
                         f" us): {t:.1f} us = {lin_bytes / t / 1e3:.0f} GB/s "
                         f"({lin_bytes / t / 1e3 / PEAK_HBM_GBPS:.1%} of {PEAK_HBM_GBPS:.0f} GB/s HBM).")

    fetch = _counter_means(_csv(os.path.join(src_dir, "fetch"), "counter_collection.csv"), "FETCH_SIZE")
    write = _counter_means(_csv(os.path.join(src_dir, "write"), "counter_collection.csv"), "WRITE_SIZE")
    f_scale = COPY_BYTES / (fetch["copy"] * 1024.0)
    w_scale = COPY_BYTES / (write["copy"] * 1024.0)
    # the same fetch scale checked on a gather pattern: every 256 B row of a 1 GiB table read once
    g_scale = (1 << 30) / (fetch["calib_gather"] * 1024.0) if "calib_gather" in fetch else None
    enc_algo = (4.0 * d + 4.0 * d + 4.0 * q) * n + 4.0 * q * k * d
    # the prepared encodes read the prepared codebooks: fp16 rows with their half-norm parts (144 B),
    # stage maxima and exponent, besides the fp32 rows of the picks
    kp = -(-k // 256) * 256
    prep16_bytes = q * (kp * 144 + 4 * (kp // 256) + 4)
    hid = w.hidden or 0
    algo = {"encode_f16": enc_algo + prep16_bytes, "encode_f16_split": enc_algo + prep16_bytes,
            "encode_fp32": enc_algo, "decode": dec_bytes + 4.0 * q * k * d,
            # fc: h rows in, latent rows out (weights 256 KiB, read once); fc2 the reverse
            "linear_in": (4.0 * hid + 4.0 * d) * n + 4.0 * hid * d,
            "linear_out": (4.0 * hid + 4.0 * d) * n + 4.0 * hid * d,
            "linear_out_touch": 4.0 * d * n}
    lines += ["", "## HBM counters (per launch)", "",
              f"A 512 MiB elementwise copy reads FETCH_SIZE = {fetch['copy']:.0f} KiB and WRITE_SIZE = "
              f"{write['copy']:.0f} KiB, so readings are scaled by {f_scale:.3f} (fetch) and "
              f"{w_scale:.3f} (write)." + (
                  f" Check on a gather pattern (every 256 B row of a 1 GiB table read once, in a scattered "
                  f"order): FETCH_SIZE = {fetch['calib_gather']:.0f} KiB for 1048576 KiB read, a scale of "
                  f"{g_scale:.3f}." if g_scale else ""), "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB | algorithmic MB |",
              "|---|---|---|---|---|---|"]
    for kind in KERNEL_SOURCES:
        if kind not in fetch or kind not in write:
            continue
        rd = fetch[kind] * 1024.0 * f_scale
        wr = write[kind] * 1024.0 * w_scale
        lines.append(f"| {kind} | {fetch[kind]:.0f} | {write[kind]:.0f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{algo[kind] / 1e6:.1f} |")
        json.dump({"kernel": kind, "workload": w.name, "source_sha256": source_hash(kind),
                   "fetch_kib": fetch[kind], "write_kib": write[kind],
                   "copy_scale_fetch": f_scale, "copy_scale_write": w_scale,
                   "traffic_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": algo[kind],
                   "commands": cmds},
                  open(os.path.join(out_dir, f"{kind}_{w.name}_hbm_counters.json"), "w"), indent=1)

    mf = _csv(os.path.join(src_dir, "mfma"), "counter_collection.csv")
    names = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_VALU_MFMA_MOPS_F16",
             "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE")
    means = {name: _counter_means(mf, name) for name in names}
    lines += ["", "## Matrix-core counters (per launch)", ""]
    for kind in ("encode_f16", "encode_f16_split", "encode_fp32", "linear_in", "linear_out"):
        c = {name: means[name].get(kind) for name in names}
        if c["GRBM_GUI_ACTIVE"] is None:
            continue
        active = c["GRBM_GUI_ACTIVE"] / N_XCD
        lines += [f"{kind}:",
                  f"- MFMA busy: {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (active * N_SIMD):.1%} of SIMD cycles "
                  f"(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x {N_SIMD} SIMDs))",
                  f"- MFMA flop counted: fp32 {c['SQ_INSTS_VALU_MFMA_MOPS_F32'] * 512:.4g}, "
                  f"fp16 {c['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512:.4g} (algorithmic 2QKD = {enc_flop:.4g})",
                  f"- instructions: VALU {c['SQ_INSTS_VALU']:.4g} of which MFMA {c['SQ_INSTS_MFMA']:.4g}",
                  f"- LDS bank-conflict cycles / LDS active cycles: "
                  f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1):.1%}", ""]
    vdir = os.path.join(src_dir, "valu")
    if os.path.isdir(vdir):
        vf = _csv(vdir, "counter_collection.csv")
        vnames = ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_WAIT_INST_ANY",
                  "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
        vm = {name: _counter_means(vf, name) for name in vnames}
        lines += ["## Instruction-issue counters (per launch)", ""]
        for kind in ("encode_f16", "encode_fp32", "linear_in", "linear_out"):
            c = {name: vm[name].get(kind) for name in vnames}
            if c["GRBM_GUI_ACTIVE"] is None:
                continue
            active = c["GRBM_GUI_ACTIVE"] / N_XCD
            lines += [f"{kind}:",
                      f"- instructions: VALU {c['SQ_INSTS_VALU']:.4g} (MFMA {c['SQ_INSTS_MFMA']:.4g}), "
                      f"SALU {c['SQ_INSTS_SALU']:.4g}, LDS {c['SQ_INSTS_LDS']:.4g}",
                      f"- VALU issue: {c['SQ_INSTS_VALU'] * 4 / (active * N_SIMD):.1%} of SIMD cycles "
                      f"(4 cycles per wavefront instruction on a 16-lane SIMD; SQ_INSTS_VALU x 4 / "
                      f"(GRBM_GUI_ACTIVE per XCD x {N_SIMD} SIMDs))",
                      f"- waves waiting on a dependency or counter: "
                      f"{c['SQ_WAIT_INST_ANY'] / max(c['SQ_WAVE_CYCLES'], 1):.1%} of wave cycles "
                      f"(SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)", ""]
    path = os.path.join(out_dir, f"encode_decode_{w.name}_rocprof.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print("wrote", path)


# ------------------------------------------- per-kernel summary (any workload)

def _trace_work(w):
    """Algorithmic work per launch of each kernel of a workload: name -> (amount, unit, what)."""
    n, q, k, d, hid = w.n_frames, w.n_stages, w.n_codes, w.dim, w.hidden
    qe = 1 if w.per_stage else q   # per-stage workloads launch the encode once per stage
    work = {
        "encode_f16_kernel": (2.0 * qe * k * d * n, "flop",
                              "fp16 matrix flop, 2KD per frame" if w.per_stage else
                              "fp16 matrix flop, 2QKD per frame"),
        "encode_bf16_kernel": (3 * 2.0 * qe * k * d * n, "flop",
                               "bf16 matrix flop, 3 x 2KD per frame" if w.per_stage else
                               "bf16 matrix flop, 3 x 2QKD per frame"),
        "encode_bf16_ksplit_kernel": (3 * 2.0 * qe * k * d * n, "flop",
                                      "bf16 matrix flop, 3 x 2KD per frame" if w.per_stage else
                                      "bf16 matrix flop, 3 x 2QKD per frame"),
        "encode_f16_ksplit_kernel": (2.0 * qe * k * d * n, "flop",
                                     "fp16 matrix flop, 2KD per frame" if w.per_stage else
                                     "fp16 matrix flop, 2QKD per frame"),
        "encode_kernel": (2.0 * q * k * d * n, "flop", "fp32 matrix flop, 2QKD per frame"),
        "decode_kernel": ((4.0 * q + 4.0 * d) * n, "B", "HBM, (4Q+4D) per frame"),
        "decode_tiled_kernel": ((4.0 * q + 4.0 * d) * n, "B", "HBM, (4Q+4D) per frame"),
    }
    if w.hidden:
        work.update({
            "linear_in_kernel": (2.0 * hid * 64 * n, "flop", "fp32 matrix flop, 2 hidden 64 per frame"),
            "linear_out_kernel": (2.0 * hid * 64 * n, "flop", "fp32 matrix flop, 2 hidden 64 per frame"),
            "linear_out_split_kernel": (2.0 * hid * 64 * n, "flop", "fp32 matrix flop, 2 hidden 64 per frame"),
            "linear_out_res_kernel": (2.0 * hid * 64 * n, "flop", "fp32 matrix flop, 2 hidden 64 per frame"),
            "touch_kernel": (4.0 * 64 * n, "B", "HBM, fc2's input rows read once ahead of it (4D per frame)"),
            "update_kernel": (8.0 * hid * n, "B", "HBM, residual read + write (8 hidden per frame)"),
            "proj8_kernel": (8.0 * hid * n, "B", "HBM, residual read + write (8 hidden per frame)"),
            "projected_decode_kernel": ((4.0 * q + 4.0 * hid) * n, "B", "HBM, (4Q + 4 hidden) per frame"),
            "projected_decode_tiled_kernel": ((4.0 * q + 4.0 * hid) * n, "B", "HBM, (4Q + 4 hidden) per frame"),
            "table_kernel": (2.0 * k * hid * d, "flop", "float64 flop, 2 K hidden D per stage"),
            "cosine_argmin_kernel": (2.0 * k * d * n, "flop", "fp32 flop, 2KD per frame"),
            "cosine_fused_kernel": ((2.0 * hid * d + 2.0 * k * d) * q * n, "flop",
                                    "fp32 flop, Q (2 hidden D + 2KD) per frame; HBM 8 hidden B per frame"),
        })
    return work


def summarize_trace(w, src_dir):
    out_dir = os.path.join(_ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    stats = _csv(src_dir, "kernel_stats.csv")
    work = _trace_work(w)
    cmd = ("cd /tmp && export TMPDIR=/tmp   # R = repository root\n"
           f"rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/tr_{w.name} -o t -- "
           f"python3 $R/bench.py --workload {w.name} --steps 5 --no-cpu-baseline --no-probes\n"
           f"python3 $R/bench.py --workload {w.name} --summarize-trace $R/gpurun_out/tr_{w.name}")
    lines = [f"# rocprofv3: kernel trace, workload `{w.name}`", "", f"Workload: {w.description}.", "",
             "Commands:", "", "```", cmd, "```", "",
             "8 steps ran (3 warmup + 5 timed). Rates are algorithmic work per launch / average duration.", "",
             "| kernel | calls | average (us) | share | work per launch | rate |", "|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"]
        short = name.split("(")[0] if not name.startswith(("void ", "rvq::")) else name
        base = next((key for key in sorted(work, key=len, reverse=True) if key + "<" in name or key + "(" in name),
                    None)
        a = float(r["AverageNs"]) / 1e3
        if base:
            i = name.index(base)
            j = name.find("(", i)
            label = name[i:j if j >= 0 else len(name)]
        else:
            label = short[:48]
        if base:
            amt, unit, what = work[base]
            rate = f"{amt / a / 1e6:.1f} TFLOP/s" if unit == "flop" else f"{amt / a / 1e3:.0f} GB/s"
            lines.append(f"| {label} | {r['Calls']} | {a:.1f} | {float(r['Percentage']):.1f}% | "
                         f"{amt:.4g} {unit} ({what}) | {rate} |")
        else:
            lines.append(f"| {label} | {r['Calls']} | {a:.1f} | {float(r['Percentage']):.1f}% | | |")
    path = os.path.join(out_dir, f"{w.name}_rocprof.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print("wrote", path)


# ------------------------------------------------------------ gather sweep

def gather_sweep(out_md):
    """Decode time vs codebook footprint at a fixed number of row gathers (Q=32 x 720000 frames)."""
    import torch
    import residual_vector_quantization_amd as rvq
    dev = torch.device("cuda:0")
    n, q = 720000, 32
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rows = []
    for k in (32, 128, 256, 512, 1024, 2048):
        books = torch.from_numpy(W.codebooks(q, k, 64, 0.85, 1)).to(dev)
        codes = torch.from_numpy(W.random_codes(n, q, k, seed=3)).to(dev)
        out = torch.empty((n, 64), dtype=torch.float32, device=dev)
        ts = []
        for rep in range(10):
            torch.cuda.synchronize()
            ev[0].record()
            rvq.rvq_decode(codes, books, out=out)
            ev[1].record()
            torch.cuda.synchronize()
            if rep >= 2:
                ts.append(ev[0].elapsed_time(ev[1]))
        ms = float(np.median(ts))
        kernel = "decode_tiled_kernel" if q * k * 256 >= 4 << 20 else "decode_kernel"
        rec = {"K": k, "codebook_MiB": q * k * 256 / 2 ** 20, "kernel": kernel, "ms": ms,
               "gather_TBps": n * q * 256 / (ms * 1e-3) / 1e12,
               "hbm_GBps": (4.0 * q + 256.0) * n / (ms * 1e-3) / 1e9}
        print(json.dumps(rec), flush=True)
        rows.append(rec)
    lines = ["# Decode row-gather rate vs codebook size", "",
             "Q = 32 stages, N = 720000 frames, D = 64, uniform random codes (seed 3); every frame "
             "gathers Q rows of 256 B, so each launch moves 5.9 GB of codebook rows out of L2 / MALL "
             "and 0.28 GB to and from HBM (codes in, reconstruction out). Median of 8 timed launches "
             "(HIP events).", "",
             "Command: `python3 bench.py --gather-sweep gpurun_out/decode_gather_sweep.md`", "",
             "| K | codebook MiB | kernel | ms | row gathers TB/s | HBM GB/s |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['K']} | {r['codebook_MiB']:.2f} | {r['kernel']} | {r['ms']:.3f} | "
                     f"{r['gather_TBps']:.1f} | {r['hbm_GBps']:.0f} |")
    lines += ["", f"Best row-gather rate: {max(r['gather_TBps'] for r in rows):.1f} TB/s."]
    os.makedirs(os.path.dirname(os.path.abspath(out_md)), exist_ok=True)
    open(out_md, "w").write("\n".join(lines) + "\n")


# ------------------------------------------------------------ ceilings

class Probes:
    """The ceiling probes of librvq_probe.so (row gathers, matrix cores), timed with HIP events on torch's
    current stream, plus a plain device copy for the HBM rate."""

    def __init__(self):
        import ctypes
        import torch
        path = os.path.join(_ROOT, "residual_vector_quantization_amd", "librvq_probe.so")
        if not os.path.exists(path):
            raise SystemExit(f"{path} is missing; build with `python -m residual_vector_quantization_amd.build`")
        self.lib = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        self.lib.rvqprobe_gather_rows.argtypes = [vp, i64, i64, i32, i32, vp, vp]
        self.lib.rvqprobe_mfma.argtypes = [i32, i32, i32, vp, vp]
        self.lib.rvqprobe_read.argtypes = [vp, i64, i32, vp, vp]
        self.torch = torch
        self.dev = torch.device("cuda:0")

    def _time(self, fn, reps):
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        return float(np.median(ts)), float(np.min(ts))

    def gather(self, table_bytes, n_rows, reps=20):
        """Random 256 B row gathers out of a table of table_bytes (rounded up to a power of two of rows):
        (TB/s at the median launch, TB/s at the fastest)."""
        torch = self.torch
        rows = 1 << max(0, (int(table_bytes) // 256 - 1).bit_length())
        table = torch.rand(rows * 64, device=self.dev)
        n_groups = 1 << 18
        per_group = max(8, -(-int(n_rows) // n_groups + 7) // 8 * 8)
        sink = torch.empty(n_groups * 64, device=self.dev)
        stream = torch.cuda.current_stream().cuda_stream

        def run():
            if self.lib.rvqprobe_gather_rows(table.data_ptr(), rows, n_groups, per_group, 0, sink.data_ptr(),
                                             stream):
                raise SystemExit("rvqprobe_gather_rows failed")
        med, mn = self._time(run, reps)
        moved = 256.0 * n_groups * per_group
        return moved / med / 1e12, moved / mn / 1e12

    def permuted_gather_once(self, table_bytes):
        """Every 256 B row of a table_bytes table read once in a scattered order (counter calibration)."""
        torch = self.torch
        rows = int(table_bytes) // 256
        table = torch.ones(rows * 64, device=self.dev)
        n_groups = 1 << 18
        sink = torch.empty(n_groups * 64, device=self.dev)
        torch.cuda.synchronize()
        if self.lib.rvqprobe_gather_rows(table.data_ptr(), rows, n_groups, rows // n_groups, 1, sink.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream):
            raise SystemExit("rvqprobe_gather_rows failed")
        torch.cuda.synchronize()

    def mfma(self, fp16, reps=5):
        """Back-to-back matrix-core products on every SIMD: TFLOP/s (median launch, fastest)."""
        torch = self.torch
        blocks, iters = 1024, (2000 if fp16 else 1000)
        sink = torch.empty(blocks * 256, device=self.dev)
        stream = torch.cuda.current_stream().cuda_stream

        def run():
            if self.lib.rvqprobe_mfma(1 if fp16 else 0, blocks, iters, sink.data_ptr(), stream):
                raise SystemExit("rvqprobe_mfma failed")
        med, mn = self._time(run, reps)
        flop = blocks * 4 * 4 * iters * (32768.0 if fp16 else 4096.0)
        return flop / med / 1e12, flop / mn / 1e12

    def copy(self, reps=10):
        """A 1 GiB device-to-device copy: GB/s of HBM traffic (read + write)."""
        torch = self.torch
        a = torch.ones(FLUSH_BYTES // 4, device=self.dev)
        b = torch.empty_like(a)
        med, mn = self._time(lambda: b.copy_(a), reps)
        del a, b
        return 2.0 * FLUSH_BYTES / med / 1e9, 2.0 * FLUSH_BYTES / mn / 1e9

    def read(self, reps=10, blocks=2048):
        """1 GiB read by a grid-stride sum (one store per thread): GB/s read."""
        torch = self.torch
        a = torch.ones(FLUSH_BYTES // 4, device=self.dev)
        sink = torch.empty(blocks * 256, device=self.dev)
        stream = torch.cuda.current_stream().cuda_stream

        def run():
            if self.lib.rvqprobe_read(a.data_ptr(), a.numel(), blocks, sink.data_ptr(), stream):
                raise SystemExit("rvqprobe_read failed")
        med, mn = self._time(run, reps)
        del a, sink
        return FLUSH_BYTES / med / 1e9, FLUSH_BYTES / mn / 1e9

    def fill(self, reps=10):
        """A 1 GiB device fill: GB/s written."""
        torch = self.torch
        a = torch.empty(FLUSH_BYTES // 4, device=self.dev)
        med, mn = self._time(lambda: a.fill_(1.0), reps)
        del a
        return FLUSH_BYTES / med / 1e9, FLUSH_BYTES / mn / 1e9


def time_decode(rvq, codes, books, out, reps=20):
    """rvq_decode timed alone with HIP events: warm (right after a launch on the same data) and cold (after
    writing a 1 GiB buffer, which evicts L2 and MALL); median and min in ms of each."""
    import torch
    flush = torch.empty(FLUSH_BYTES // 4, device=codes.device)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    res = {}
    for mode in ("warm", "cold"):
        ts = []
        for _ in range(reps):
            if mode == "cold":
                flush.fill_(1.0)
            else:
                rvq.rvq_decode(codes, books, out=out)
            ev[0].record()
            rvq.rvq_decode(codes, books, out=out)
            ev[1].record()
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        res[mode] = {"median_ms": float(np.median(ts)), "min_ms": float(np.min(ts))}
    del flush
    return res


def gather_probe(out_md):
    """The row-gather ceiling over table sizes 0.25..16 MiB (5.9 GB of rows each) and the matrix-core and
    copy ceilings; writes a summary to out_md."""
    pr = Probes()
    rows = []
    for mib in (0.25, 1, 2, 4, 8, 16):
        med, best = pr.gather(mib * 2 ** 20, 720000 * 32)
        rec = {"table_MiB": mib, "gather_TBps_median": med, "gather_TBps_best": best}
        print(json.dumps(rec), flush=True)
        rows.append(rec)
    f16 = pr.mfma(True)
    f32 = pr.mfma(False)
    cp = pr.copy()
    fl = pr.fill()
    rd = pr.read()
    print(json.dumps({"mfma_f16_TFLOPs": f16, "mfma_f32_TFLOPs": f32, "copy_GBps": cp, "fill_GBps": fl,
                      "read_GBps": rd}), flush=True)
    lines = ["# Ceiling probes (row gathers, matrix cores, HBM copy)", "",
             "`librvq_probe.so` (`csrc/probes.hip`), HIP events on the launch stream; median and best of the "
             "timed launches.", "",
             "Command: `python3 bench.py --gather-probe gpurun_out/ceilings.md`", "",
             "## Random 256 B row gathers",
             "",
             "16 lanes x 16 B per row (the decode's access pattern), row index from an in-kernel hash (no "
             "dependent load), 8 row loads in flight per lane, no store per row; 2^18 groups of 16 lanes, "
             "5.9 GB of rows per launch (720,000 frames x 32 stages).", "",
             "| table MiB | TB/s (median) | TB/s (best) |", "|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['table_MiB']} | {r['gather_TBps_median']:.1f} | {r['gather_TBps_best']:.1f} |")
    lines += ["", "## Matrix cores and HBM", "",
              "| probe | median | best | published |", "|---|---|---|---|",
              f"| v_mfma_f32_32x32x16_f16, 4 chains per wavefront, 16 wavefronts per CU | {f16[0]:.0f} TFLOP/s | "
              f"{f16[1]:.0f} TFLOP/s | {PEAK_F16_MFMA_TFLOPS:.0f} TFLOP/s |",
              f"| v_mfma_f32_32x32x2_f32, same | {f32[0]:.1f} TFLOP/s | {f32[1]:.1f} TFLOP/s | "
              f"{PEAK_FP32_MFMA_TFLOPS} TFLOP/s |",
              f"| 1 GiB device copy (read + write) | {cp[0]:.0f} GB/s | {cp[1]:.0f} GB/s | {PEAK_HBM_GBPS:.0f} GB/s |",
              f"| 1 GiB device fill (write only) | {fl[0]:.0f} GB/s | {fl[1]:.0f} GB/s | {PEAK_HBM_GBPS:.0f} GB/s |",
              f"| 1 GiB read, grid-stride sum of 16 B loads (read only; 2048 workgroups of 256) | {rd[0]:.0f} GB/s | "
              f"{rd[1]:.0f} GB/s | {PEAK_HBM_GBPS:.0f} GB/s |"]
    os.makedirs(os.path.dirname(os.path.abspath(out_md)), exist_ok=True)
    open(out_md, "w").write("\n".join(lines) + "\n")


def calibrate_counters(dev):
    """Kernels of a known size for the HBM counters: an elementwise copy (streaming read + write) and a
    scattered read of every 256 B row of a 1 GiB table once (gather pattern, read only)."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    del a, b
    Probes().permuted_gather_once(1 << 30)


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(w, x, books, codes_gpu, target_s):
    """Times the CPU oracle (encode + decode) on a seeded frame sample; also checks parity there."""
    import oracle
    o = oracle.get()
    probe = W.sample_frames(w.n_frames, min(w.n_frames, 1024), seed=7)
    t0 = time.perf_counter()
    o.encode(x[probe], books)
    rate = probe.size / max(time.perf_counter() - t0, 1e-6)
    count = int(min(w.n_frames, max(probe.size, rate * target_s)))
    idx = W.sample_frames(w.n_frames, count, seed=8)
    xs = x[idx]
    t0 = time.perf_counter()
    oc, _, best, second = o.encode(xs, books)
    o.decode(oc, books)
    dt = time.perf_counter() - t0
    threads = o.last_threads
    mism = (codes_gpu[idx] != oc).any(axis=1)
    tie = oracle.near_tie(best, second).any(axis=1)
    parity = {"frames_checked": int(idx.size), "code_mismatch_frames": int(mism.sum()),
              "mismatch_not_near_tie": int((mism & ~tie).sum()),
              "near_tie_frames_in_sample": int(tie.sum())}
    base = {"value": idx.size / dt, "unit": "frames/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{idx.size} of {w.n_frames} frames (seeded uniform sample incl. first/last 64), "
                      f"encode + decode, {dt:.1f} s wall"}
    return base, parity


# --------------------------------------------------------------- benches

def bench_projected(args, w):
    """Codebook preparation, then fc -> encode -> decode -> fc2, per step (rvq_project_roundtrip)."""
    import torch
    import residual_vector_quantization_amd as rvq
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    w_in, b_in, w_out, b_out = W.projection_weights(w)
    h = W.hidden_states(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = {k: torch.from_numpy(v).to(dev) for k, v in
         dict(h=h, w_in=w_in, b_in=b_in, w_out=w_out, b_out=b_out, books=books).items()}
    n, q, k, d, hid = w.n_frames, w.n_stages, w.n_codes, w.dim, w.hidden
    out = (torch.empty((n, q), dtype=torch.int32, device=dev), torch.empty((n, d), device=dev),
           torch.empty((n, d), device=dev), torch.empty((n, hid), device=dev))
    prep = torch.empty(rvq.rvq_prepared_bytes(q, k, d), dtype=torch.uint8, device=dev)

    def step():
        rvq.rvq_prepare_codebooks(t["books"], prep)
        rvq.rvq_project_roundtrip(t["h"], t["w_in"], t["b_in"], t["books"], t["w_out"], t["b_out"], out=out,
                                  prepared=prep)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(args.steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    if args.calibrate_copy:
        calibrate_counters(dev)
    lin_flop = 2 * 2.0 * hid * d * n
    enc_flop = 2.0 * q * k * d * n
    rec = {"metric": "RVQ projected round trip frames/sec (fc 1024->64, Q=8 K=1024 D=64 RVQ, fc2 64->1024; fp32)",
           "value": n * args.steps / wall, "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "frames": n, "hidden": hid, "Q": q, "K": k, "D": d,
                      "recipe": w.description},
           "step_ms_events": ms,
           "fp32_equivalent_tflops": (lin_flop + enc_flop) / (ms * 1e-3) / 1e12}
    print(json.dumps(rec), flush=True)


def bench_stage_projected(args, w):
    """Per-stage projected RVQ: table (and codebook) preparation + encode + decode per step."""
    import torch
    import residual_vector_quantization_amd as rvq
    import oracle
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    w_in, b_in, w_out, b_out = W.stage_projection_weights(w)
    h = W.hidden_states(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = {k: torch.from_numpy(v).to(dev) for k, v in
         dict(h=h, w_in=w_in, b_in=b_in, w_out=w_out, b_out=b_out, books=books).items()}
    n, q, k, d, hid = w.n_frames, w.n_stages, w.n_codes, w.dim, w.hidden
    table = torch.empty((q, k, hid), device=dev)
    units = torch.empty((q, k, d), dtype=torch.float64, device=dev) if w.normalized else None
    out = (torch.empty((n, q), dtype=torch.int32, device=dev), torch.empty((q, n, d), device=dev),
           torch.empty((n, hid), device=dev))
    recon = torch.empty((n, hid), device=dev)
    prep = None if w.normalized else torch.empty(rvq.rvq_prepared_bytes(q, k, d), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        rvq.rvq_projected_prepare(t["books"], t["w_out"], t["b_out"], table)
        if w.normalized:
            rvq.rvq_cosine_prepare(t["books"], units)
        else:
            rvq.rvq_prepare_codebooks(t["books"], prep)
        if ev is not None:
            ev[1].record()
        if w.normalized:
            rvq.rvq_cosine_encode(t["h"], t["w_in"], t["b_in"], units, table, out=out)
        else:
            rvq.rvq_projected_encode(t["h"], t["w_in"], t["b_in"], t["books"], table, out=out, prepared=prep)
        if ev is not None:
            ev[2].record()
        rvq.rvq_projected_decode(out[0], table, out=recon)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep_ms, enc_ms, dec_ms = (float(np.mean([e[j].elapsed_time(e[j + 1]) for e in events])) for j in range(3))
    # encode work per frame: Q in-projections (2*H*D) and Q score sets (2*K*D) on the matrix cores;
    # HBM per frame and stage: residual read + write and one gathered table row (H floats each)
    proj_flop = 2.0 * q * hid * d * n
    score_flop = 2.0 * q * k * d * n
    metric = (f"RVQ normalized (cosine) per-stage projected encode + decode frames/sec (H={hid}, Q={q}, K={k}, "
              f"D={d}; fp32)" if w.normalized else
              f"RVQ per-stage projected encode + decode frames/sec (H={hid}, Q={q}, K={k}, D={d}; fp32)")
    rec = {"metric": metric,
           "value": n * args.steps / wall, "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "frames": n, "hidden": hid, "Q": q, "K": k, "D": d,
                      "recipe": w.description},
           "prepare_ms": prep_ms, "encode_ms": enc_ms, "decode_ms": dec_ms,
           "encode_fp32_equivalent_tflops": (proj_flop + score_flop) / (enc_ms * 1e-3) / 1e12,
           "decode_hbm": {"achieved": (4.0 * q + 4.0 * hid) * n / (dec_ms * 1e-3) / 1e9, "unit": "GB/s",
                          "peak": PEAK_HBM_GBPS, "work_per_launch": "(4Q + 4H) B per frame",
                          "row_gathers_TBps": 4.0 * hid * q * n / (dec_ms * 1e-3) / 1e12}}
    if not args.no_cpu_baseline:
        codes_h = out[0].cpu().numpy()
        o = oracle.get()
        probe = W.sample_frames(n, 256, seed=7)
        t1 = time.perf_counter()
        o.projected_encode(h[probe], w_in, b_in, books, w_out, b_out, normalize=w.normalized)
        rate = probe.size / max(time.perf_counter() - t1, 1e-6)
        idx = W.sample_frames(n, int(min(n, max(probe.size, rate * args.cpu_seconds))), seed=8)
        t1 = time.perf_counter()
        oc, _, _, best, second = o.projected_encode(h[idx], w_in, b_in, books, w_out, b_out,
                                                    normalize=w.normalized)
        o.projected_decode(oc, books, w_out, b_out)
        dt = time.perf_counter() - t1
        mism = (codes_h[idx] != oc).any(axis=1)
        ties = oracle.near_tie(best, second)
        exempt = 0
        if mism.any():
            bad = np.nonzero(mism)[0]
            exempt = int(ties[bad, np.argmax(codes_h[idx][bad] != oc[bad], axis=1)].sum())
        rec["cpu_baseline"] = {"value": idx.size / dt, "unit": "frames/s", "cores": int(o.last_threads),
                               "kind": "oracle",
                               "sample": f"{idx.size} of {n} frames (seeded uniform sample incl. first/last 64), "
                                         f"{'normalized ' if w.normalized else ''}projected encode + decode, "
                                         f"{dt:.1f} s wall"}
        rec["parity_sample"] = {"frames_checked": int(idx.size), "code_mismatch_frames": int(mism.sum()),
                                "mismatch_first_stage_near_tie": exempt,
                                "near_tie_frames_in_sample": int(ties.any(axis=1).sum()),
                                "note": "oracle on its own float64 projections vs GPU codes"}
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(W.WORKLOADS[args.workload], args.summarize_profiles)
        return
    if args.gather_sweep:
        gather_sweep(args.gather_sweep)
        return
    if args.gather_probe:
        gather_probe(args.gather_probe)
        return
    if args.summarize_trace:
        summarize_trace(W.WORKLOADS[args.workload], args.summarize_trace)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(frames shard with no exchange, so N GPUs would each run this same kernel on N/G frames)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import residual_vector_quantization_amd as rvq

    w = W.WORKLOADS[args.workload]
    if w.projected:
        return bench_projected(args, w)
    if w.per_stage:
        return bench_stage_projected(args, w)
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    x, _ = W.latents(w, books)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xg = torch.from_numpy(x).to(dev)
    bg = torch.from_numpy(books).to(dev)
    codes = torch.empty((w.n_frames, w.n_stages), dtype=torch.int32, device=dev)
    residual = torch.empty_like(xg)
    out = torch.empty_like(xg)
    torch.cuda.synchronize()

    prepared = torch.empty(rvq.rvq_prepared_bytes(w.n_stages, w.n_codes, w.dim), dtype=torch.uint8,
                           device=dev)

    def step(ev=None):
        # codebooks prepared (every step), encode from them, decode the codes
        if ev is not None:
            ev[0].record()
        rvq.rvq_prepare_codebooks(bg, prepared)
        if ev is not None:
            ev[1].record()
        rvq.rvq_encode_prepared(xg, bg, prepared, out=(codes, None, residual))
        if ev is not None:
            ev[2].record()
        rvq.rvq_decode(codes, bg, out=out)
        if ev is not None:
            ev[3].record()

    n, q, k, d = w.n_frames, w.n_stages, w.n_codes, w.dim
    # Side measurements first (they also bring the GPU to its sustained clocks before the timed steps):
    # the ceilings of this GPU, the decode alone warm and cold, the fp32-scored encode.
    step()
    torch.cuda.synchronize()
    ceil = dec_alone = None
    if not args.no_probes:
        pr = Probes()
        # the frame-parallel decode gathers from the whole codebook, the stage-ordered one (codebooks of
        # 4 MiB and more) from the few stages in flight: probe tables of those sizes, long enough launches
        table = 4.0 * q * k * d if 4 * q * k * d < 4 << 20 else 2 << 20
        probe_rows = max(n * q, 1 << 24)
        ceil = {"gather_TBps": pr.gather(table, probe_rows), "mfma_f16_TFLOPs": pr.mfma(True),
                "mfma_f32_TFLOPs": pr.mfma(False), "copy_GBps": pr.copy(), "fill_GBps": pr.fill()}
        dec_alone = time_decode(rvq, codes, bg, out)
    # the same encode with fp32 matrix-core scores (identical results), timed separately
    fp32_ms = None
    if args.fp32_steps > 0:
        c32 = torch.empty_like(codes)
        r32 = torch.empty_like(xg)
        rvq.rvq_encode_scored(xg, bg, "fp32", out=(c32, None, r32))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(args.fp32_steps):
            rvq.rvq_encode_scored(xg, bg, "fp32", out=(c32, None, r32))
        ev[1].record()
        torch.cuda.synchronize()
        fp32_ms = ev[0].elapsed_time(ev[1]) / args.fp32_steps
        if not torch.equal(c32, codes):
            raise SystemExit("fp32 scoring and the prepared encode disagree")
        rvq.rvq_encode(xg, bg, codes=c32, residual_out=r32)
        torch.cuda.synchronize()
        if not torch.equal(c32, codes):
            raise SystemExit("rvq_encode and rvq_encode_prepared disagree")

    # the encode's launch-to-launch settling: 40 back-to-back launches timed one by one (a fresh
    # process's first launches run up to 1.3x slower while the clocks adjust to this kernel)
    settle = None
    if not args.no_probes:
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(40)]
        for e in sev:
            e[0].record()
            rvq.rvq_encode_prepared(xg, bg, prepared, out=(codes, None, residual))
            e[1].record()
        torch.cuda.synchronize()
        st = [e[0].elapsed_time(e[1]) for e in sev]
        settle = {"launches": 40, "first_ms": st[0], "median_2_10_ms": float(np.median(st[1:10])),
                  "median_11_30_ms": float(np.median(st[10:30])), "median_31_40_ms": float(np.median(st[30:]))}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed steps record events around the encode only (each recorded event is one more packet on
    # the stream, a few microseconds between the kernels); the codebook preparation and the decode
    # are timed on separate instrumented steps right after.
    enc_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        rvq.rvq_prepare_codebooks(bg, prepared)
        enc_events[i][0].record()
        rvq.rvq_encode_prepared(xg, bg, prepared, out=(codes, None, residual))
        enc_events[i][1].record()
        rvq.rvq_decode(codes, bg, out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in enc_events]))
    n_inst = min(args.steps, 20)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_inst)]
    for i in range(n_inst):
        step(events[i])
    torch.cuda.synchronize()
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))
    codes_h = codes.cpu().numpy()

    if args.calibrate_copy:
        calibrate_counters(dev)

    ms_per_step = wall * 1e3 / args.steps
    value = n * args.steps / wall
    enc_flop = 2.0 * q * k * d * n
    wide = n > SPLIT_MAX_FRAMES
    # one fp16 product per dimension; the method's 2QKD flop on the fp16 peak
    mm_work, mm_what = enc_flop, f"2*Q*K*D*N = {enc_flop:.4g} flop on fp16 matrix cores"
    mm_kernel = (("encode_f16_kernel" if wide else
                  "encode_f16_ksplit_kernel (codebook split over a workgroup's wavefronts)") +
                 ", prepared codebooks (v_mfma_f32_32x32x16_f16, one product per dimension + a half-norm "
                 "step; exact float64 re-rank of candidates)")
    mm_tflops = mm_work / (enc_ms * 1e-3) / 1e12
    dec_bytes = (4.0 * q + 4.0 * d) * n
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    gather_tbps = 4.0 * d * q * n / (dec_ms * 1e-3) / 1e12
    dec_kernel = "decode_tiled_kernel" if 4 * q * k * d >= 4 << 20 else "decode_kernel"
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "frames": n, "Q": q, "K": k, "D": d,
                   "scoring": "fp16 + exact re-rank",
                   "recipe": w.description},
        "audio_seconds_per_s": value / w.frame_rate_hz,
        "prepare_ms": prep_ms,
        "encode_ms": enc_ms,
        "decode_ms": dec_ms,
        "timing": "value and ms_per_step: wall clock over the timed steps (prepare + encode + decode, "
                  "synchronized on both sides); encode_ms: HIP events around each timed encode; "
                  "prepare_ms and decode_ms: HIP events on 20 instrumented steps after the timed ones",
        "roofline": {"bound": "mfma", "kernel": mm_kernel,
                     "achieved": mm_tflops, "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": mm_tflops / PEAK_F16_MFMA_TFLOPS,
                     "traffic": recorded_traffic("encode_f16" if wide else "encode_f16_split", w.name),
                     "work_per_launch": mm_what,
                     "contraction_dtype": "fp16",
                     "decision": "float64 re-rank of every candidate within the proven fp16 error bound; "
                                 "codes equal the oracle's float64 argmin",
                     "limiter": ("vector-ALU issue, not the matrix cores: every score's packed (score, index) "
                                 "key is updated on the VALU (about 3 instructions per score, half the SIMD "
                                 "cycles in the rocprofv3 issue counters against a quarter for the matrix "
                                 "cores)" if wide else "latency: one four-wavefront workgroup per CU and 32 frames "
                                 "each, with the merge of the wavefronts' keys and the decision between "
                                 "stages"),
                     "results_dtype": "f32 residual and reconstruction, i32 codes"},
        "encode_fp32_equivalent": {"achieved": enc_flop / (enc_ms * 1e-3) / 1e12, "peak": PEAK_FP32_MFMA_TFLOPS,
                                   "unit": "TFLOP/s", "work_per_launch": f"2*Q*K*D*N = {enc_flop:.4g} flop"},
        "decode_roofline": {"bound": "hbm", "kernel": dec_kernel, "achieved": dec_gbps,
                            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": dec_gbps / PEAK_HBM_GBPS,
                            "traffic": recorded_traffic("decode", w.name),
                            "work_per_launch": f"(4Q+4D)*N = {dec_bytes:.4g} B",
                            "row_gathers": {"achieved": gather_tbps, "unit": "TB/s",
                                            "work_per_launch": f"4*D*Q*N = {4.0 * d * q * n:.4g} B "
                                                               "of codebook rows from L2 / MALL"}},
    }
    if ceil is not None:
        g_med = ceil["gather_TBps"][0]
        rg = rec["decode_roofline"]["row_gathers"]
        rg.update({"ceiling": g_med, "frac": gather_tbps / g_med,
                   "ceiling_source": f"rvqprobe_gather_rows (librvq_probe.so) on this GPU: random 256 B rows from "
                                     f"a {table / 2 ** 20:g} MiB table (the decode's working set), no dependent "
                                     f"loads, about {256 * probe_rows / 1e9:.1f} GB per launch, median launch"})
        f16_med, f32_med = ceil["mfma_f16_TFLOPs"][0], ceil["mfma_f32_TFLOPs"][0]
        # bf16 and fp16 share the dense matrix-core rate, so the fp16 probe serves both
        rec["roofline"].update({"peak_measured": f16_med, "frac_measured": mm_tflops / f16_med,
                                "peak_measured_source": "rvqprobe_mfma: back-to-back v_mfma_f32_32x32x16_f16 "
                                                        "on every SIMD, this GPU"})
        rec["encode_fp32_equivalent"].update({"peak_measured": f32_med})
        cp_med = ceil["copy_GBps"][0]
        rec["decode_roofline"].update({"peak_measured": cp_med, "frac_measured": dec_gbps / cp_med,
                                       "peak_measured_source": "1 GiB device copy (read + write), this GPU"})
        for mode, t in dec_alone.items():
            rec["decode_roofline"][mode] = {
                "median_ms": t["median_ms"], "min_ms": t["min_ms"],
                "hbm_GBps_median": dec_bytes / (t["median_ms"] * 1e-3) / 1e9,
                "row_gathers_TBps_median": 4.0 * d * q * n / (t["median_ms"] * 1e-3) / 1e12,
                "timing": "rvq_decode alone, 20 launches, HIP events" +
                          (", each after writing 1 GiB (L2 and MALL evicted)" if mode == "cold" else
                           ", each right after a launch on the same data")}
        rec["ceilings_measured"] = {k_: {"median": v[0], "best": v[1]} for k_, v in ceil.items()}
    if settle is not None:
        rec["encode_settling"] = settle
    if fp32_ms is not None:
        t32 = enc_flop / (fp32_ms * 1e-3) / 1e12
        rec["encode_fp32_scoring"] = {"kernel": "encode_kernel (v_mfma_f32_32x32x2_f32)", "ms": fp32_ms,
                                      "bound": "mfma", "achieved": t32, "peak": PEAK_FP32_MFMA_TFLOPS,
                                      "unit": "TFLOP/s", "frac": t32 / PEAK_FP32_MFMA_TFLOPS,
                                      "traffic": recorded_traffic("encode_fp32", w.name),
                                      "codes_equal_to_default": True}
        if ceil is not None:
            rec["encode_fp32_scoring"].update({"peak_measured": ceil["mfma_f32_TFLOPs"][0],
                                               "frac_measured": t32 / ceil["mfma_f32_TFLOPs"][0]})
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(w, x, books, codes_h, args.cpu_seconds)
        rec["cpu_baseline"] = base
        rec["parity_sample"] = parity
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
