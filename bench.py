"""Throughput of the RVQ hot path (encode + decode) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batched]

One step = ``rvq_encode`` (codes + final residual) followed by
``rvq_decode`` (codes -> reconstruction) over the whole batch, inputs and
outputs resident in HBM. W untimed steps, then K timed steps between
``torch.cuda.synchronize()`` calls. Per-launch kernel times come from HIP
events recorded on the stream the kernels run on (torch's current stream,
which is the stream handed to the C ABI).

Prints one JSON line with the throughput, the roofline of the dominant
kernel (encode, fp32 matrix cores), the decode's HBM roofline, sampled
parity against the CPU oracle, and the oracle's own throughput on a bounded
sample of the same workload (``cpu_baseline``).
"""

import argparse
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
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="batched", choices=list(W.WORKLOADS))
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the CPU-oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain elementwise copy of 512 MiB (for HBM counter scaling)")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="turn rocprofv3 CSV output under DIR (trace/, fetch/, write/, mfma/) into the "
                        "summaries under profiles/, then exit")
    return p.parse_args()


def recorded_traffic(kernel_source, summary):
    """HBM bytes per launch from a committed counter summary, or None if the kernel changed since."""
    import hashlib
    path = os.path.join(_ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(_ROOT, "residual_vector_quantization_amd", "csrc", kernel_source)
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
        return None
    return rec.get("traffic_bytes_per_launch")


PROFILE_COMMANDS = """cd /tmp && export TMPDIR=/tmp   # R = repository root
rocprofv3 --kernel-trace --stats --output-format csv -d $R/gpurun_out/prof/trace -o bench -- python3 $R/bench.py --workload {wl} --steps 20 --no-cpu-baseline
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/gpurun_out/prof/fetch -o bench -- python3 $R/bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --calibrate-copy
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/gpurun_out/prof/write -o bench -- python3 $R/bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --calibrate-copy
rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_BUSY_CU_CYCLES SQ_INSTS_VALU SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE --output-format csv -d $R/gpurun_out/prof/mfma -o bench -- python3 $R/bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline
python3 $R/bench.py --workload {wl} --summarize-profiles $R/gpurun_out/prof"""

# MI355X: 8 XCDs, 256 CUs, 4 SIMDs per CU.
N_XCD, N_SIMD = 8, 1024
COPY_BYTES = 512 << 20


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
    if "encode_kernel" in name:
        return "encode"
    if "decode_kernel" in name:
        return "decode"
    if "elementwise" in name and "MulFunctor" in name:
        return "copy"
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
    """Writes profiles/<kernel>_<workload>_* from the four rocprofv3 runs under src_dir."""
    import hashlib
    out_dir = os.path.join(_ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    cmds = PROFILE_COMMANDS.format(wl=w.name)
    n, q, k, d = w.n_frames, w.n_stages, w.n_codes, w.dim

    stats = _csv(os.path.join(src_dir, "trace"), "kernel_stats.csv")
    lines = [f"# Kernel trace: encode + decode, workload `{w.name}`", "",
             f"Workload: {w.description}.", "", "Commands (the summary is the last line's output):", "",
             "```", cmds, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    avg = {}
    for r in stats:
        kind = _kernel_of(r["Name"]) or r["Name"][:40]
        a = float(r["AverageNs"]) / 1e3
        avg[kind] = a
        lines.append(f"| {kind} | {r['Calls']} | {a:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    enc_flop = 2.0 * q * k * d * n
    dec_bytes = (4.0 * q + 4.0 * d) * n
    lines += ["", f"Encode: {enc_flop:.4g} algorithmic flop per launch (2QKD per frame) / "
                  f"{avg['encode']:.1f} us = {enc_flop / avg['encode'] / 1e6:.1f} TFLOP/s "
                  f"({enc_flop / avg['encode'] / 1e6 / PEAK_FP32_MFMA_TFLOPS:.1%} of {PEAK_FP32_MFMA_TFLOPS} fp32 MFMA).",
              f"Decode: {dec_bytes:.4g} algorithmic bytes per launch ((4Q+4D) per frame) / "
              f"{avg['decode']:.1f} us = {dec_bytes / avg['decode'] / 1e3:.0f} GB/s "
              f"({dec_bytes / avg['decode'] / 1e3 / PEAK_HBM_GBPS:.1%} of {PEAK_HBM_GBPS:.0f} GB/s HBM)."]

    fetch = _counter_means(_csv(os.path.join(src_dir, "fetch"), "counter_collection.csv"), "FETCH_SIZE")
    write = _counter_means(_csv(os.path.join(src_dir, "write"), "counter_collection.csv"), "WRITE_SIZE")
    f_scale = COPY_BYTES / (fetch["copy"] * 1024.0)
    w_scale = COPY_BYTES / (write["copy"] * 1024.0)
    algo = {"encode": (4.0 * d + 4.0 * d + 4.0 * q) * n + 4.0 * q * k * d, "decode": dec_bytes + 4.0 * q * k * d}
    lines += ["", "## HBM counters (per launch)", "",
              f"A 512 MiB elementwise copy reads FETCH_SIZE = {fetch['copy']:.0f} KiB and WRITE_SIZE = "
              f"{write['copy']:.0f} KiB, so counter readings are scaled by {f_scale:.3f} (fetch) and "
              f"{w_scale:.3f} (write).", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB | algorithmic MB |",
              "|---|---|---|---|---|---|"]
    for kind, src in (("encode", "encode.hip"), ("decode", "decode.hip")):
        rd = fetch[kind] * 1024.0 * f_scale
        wr = write[kind] * 1024.0 * w_scale
        lines.append(f"| {kind} | {fetch[kind]:.0f} | {write[kind]:.0f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{algo[kind] / 1e6:.1f} |")
        sha = hashlib.sha256(open(os.path.join(_ROOT, "residual_vector_quantization_amd", "csrc", src),
                                  "rb").read()).hexdigest()
        json.dump({"kernel": kind, "workload": w.name, "source_sha256": sha,
                   "fetch_kib": fetch[kind], "write_kib": write[kind],
                   "copy_scale_fetch": f_scale, "copy_scale_write": w_scale,
                   "traffic_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": algo[kind],
                   "commands": cmds},
                  open(os.path.join(out_dir, f"{kind}_{w.name}_hbm_counters.json"), "w"), indent=1)

    mf = _csv(os.path.join(src_dir, "mfma"), "counter_collection.csv")
    c = {name: _counter_means(mf, name).get("encode") for name in
         ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU",
          "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE")}
    active = c["GRBM_GUI_ACTIVE"] / N_XCD
    lines += ["", "## Encode matrix-core counters (per launch)", "",
              f"- MFMA busy: {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (active * N_SIMD):.1%} of SIMD cycles "
              f"(SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x {N_SIMD} SIMDs))",
              f"- MFMA fp32 flop counted: {c['SQ_INSTS_VALU_MFMA_MOPS_F32'] * 512:.4g} "
              f"(algorithmic {enc_flop:.4g})",
              f"- VALU instructions (incl. MFMA): {c['SQ_INSTS_VALU']:.4g}",
              f"- LDS bank-conflict cycles / LDS active cycles: "
              f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1):.1%}"]
    path = os.path.join(out_dir, f"encode_decode_{w.name}_rocprof.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print("wrote", path)


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


def bench_projected(args, w):
    """fc -> encode -> decode -> fc2 per step (rvq_project_roundtrip); all three kernels are fp32 MFMA."""
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

    def step():
        rvq.rvq_project_roundtrip(t["h"], t["w_in"], t["b_in"], t["books"], t["w_out"], t["b_out"], out=out)

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
    flop = (2.0 * q * k * d + 2 * 2.0 * hid * d) * n
    tflops = flop / (ms * 1e-3) / 1e12
    rec = {"metric": "RVQ projected round trip frames/sec (fc 1024->64, Q=8 K=1024 D=64 RVQ, fc2 64->1024; fp32)",
           "value": n * args.steps / wall, "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "frames": n, "hidden": hid, "Q": q, "K": k, "D": d,
                      "recipe": w.description},
           "roofline": {"bound": "mfma", "kernel": "linear_in + encode + linear_out (fp32 MFMA)",
                        "achieved": tflops, "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                        "frac": tflops / PEAK_FP32_MFMA_TFLOPS, "traffic": None,
                        "work_per_launch": f"(2QKD + 4*H*D)*N = {flop:.4g} flop"}}
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(W.WORKLOADS[args.workload], args.summarize_profiles)
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

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        rvq.rvq_encode(xg, bg, codes=codes, residual_out=residual)
        if ev is not None:
            ev[1].record()
        rvq.rvq_decode(codes, bg, out=out)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))

    n, q, k, d = w.n_frames, w.n_stages, w.n_codes, w.dim
    ms_per_step = wall * 1e3 / args.steps
    value = n * args.steps / wall
    enc_flop = 2.0 * q * k * d * n
    enc_tflops = enc_flop / (enc_ms * 1e-3) / 1e12
    dec_bytes = (4.0 * q + 4.0 * d) * n
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9

    if args.calibrate_copy:
        a = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b

    codes_h = codes.cpu().numpy()
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
                   "recipe": w.description},
        "audio_seconds_per_s": value / w.frame_rate_hz,
        "encode_ms": enc_ms,
        "decode_ms": dec_ms,
        "roofline": {"bound": "mfma", "kernel": "encode_kernel (fp32 v_mfma_f32_32x32x2_f32)",
                     "achieved": enc_tflops, "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": enc_tflops / PEAK_FP32_MFMA_TFLOPS,
                     "traffic": recorded_traffic("encode.hip", f"encode_{w.name}_hbm_counters.json"),
                     "work_per_launch": f"2*Q*K*D*N = {enc_flop:.4g} flop"},
        "decode_roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": dec_gbps,
                            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": dec_gbps / PEAK_HBM_GBPS,
                            "traffic": recorded_traffic("decode.hip", f"decode_{w.name}_hbm_counters.json"),
                            "work_per_launch": f"(4Q+4D)*N = {dec_bytes:.4g} B"},
    }
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(w, x, books, codes_h, args.cpu_seconds)
        rec["cpu_baseline"] = base
        rec["parity_sample"] = parity
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
