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
    p.add_argument("--workload", default="batched", choices=[k for k, v in W.WORKLOADS.items() if not v.projected])
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the CPU-oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain elementwise copy of 512 MiB (for HBM counter scaling)")
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(frames shard with no exchange, so N GPUs would each run this same kernel on N/G frames)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import residual_vector_quantization_amd as rvq

    w = W.WORKLOADS[args.workload]
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
