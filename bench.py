"""Throughput of the GDN large-beam decode path on one MI355X.

One step = one pass of the whole hot path over one batch: the L = 4 decode
steps (ancestry update, shared-context projections, record replay, current
transition, output and append) of 8 requests x 512 beams, H = 32 heads,
d_k = d_v = 128, on seeded synthetic inputs already resident in HBM.

Prints one JSON line: beam-steps/s, the roofline of the decode kernel
(algorithmic bytes per launch over its HIP-event-timed mean duration, against
8 TB/s), and the FP64 CPU oracle timed on a bounded sample of the same
workload on the host cores.
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from linear_attention_beam_gdn_amd import accounting, configs  # noqa: E402

METRIC = "GDN beam-steps/sec (H=32,dk=dv=128,512 beams) + % of HBM roofline"
HBM_PEAK_GBS = 8000.0
WORKLOAD = configs.LARGE

_CPU_INPUTS = None
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_beam_fused_gdn_large_beam_hbm_traffic.json")


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    when the kernel sources have changed since those counters were taken."""
    import hashlib

    try:
        rec = json.load(open(TRAFFIC_RECORD))
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, ValueError, KeyError):
        return None
    return float(rec["traffic_bytes_per_launch"]) if h.hexdigest() == rec["sources_sha256"] else None


def _single_thread():
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)


def _oracle_pair(rh):
    import oracle.gdn_oracle as O

    r, h = rh
    O.beam_decode(_CPU_INPUTS["S0"], _CPU_INPUTS["steps"], requests=[r], heads=[h])
    return rh


def cpu_baseline(inp, n_pairs, workers):
    """Time the FP64 oracle on n_pairs (request, head) pairs of the workload
    (all beams and steps of each), in a pool of single-threaded workers."""
    global _CPU_INPUTS
    _CPU_INPUTS = inp
    w = WORKLOAD
    pairs = [(r, h) for r in range(w.R) for h in range(w.H)][:n_pairs]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_single_thread) as pool:
        list(pool.imap_unordered(_oracle_pair, pairs))
    dt = time.perf_counter() - t0
    beam_steps = w.W * w.L * len(pairs) / w.H  # a beam-step covers all H heads
    return {
        "value": beam_steps / dt,
        "unit": "beam-steps/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{len(pairs)} of {w.R * w.H} (request, head) pairs, all {w.W} beams x {w.L} "
                  f"steps each ({w.W * w.L * len(pairs)} beam-head-steps), {dt:.1f} s wall",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=32)
    ap.add_argument("--cpu-workers", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the warm-up, run a plain device copy of this many MiB three times "
                         "(a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path shards by request and head with no "
              "exchange, so a multi-GPU figure is not produced here", file=sys.stderr)
        sys.exit(2)

    w = WORKLOAD
    inp = w.inputs()
    cpu = None
    if not args.no_cpu_baseline:  # before the GPU is touched: the pool forks
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        cpu = cpu_baseline(inp, args.cpu_pairs, workers)

    import torch

    from linear_attention_beam_gdn_amd import binding as B

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    B.lib()
    steps = [B.upload(st, dev) for st in inp["steps"]]
    store = B.Store(w.R, w.W, w.H, w.dk, w.dv, w.L, S=torch.from_numpy(inp["S0"]).to(dev))
    outs = [torch.empty(w.R, w.W, w.H, w.dv, dtype=torch.float32, device=dev) for _ in range(w.L)]
    stream = torch.cuda.current_stream()

    def one_pass(ev=None):
        for t, d in enumerate(steps):
            if ev is not None:
                ev[t][0].record(stream)
            B.decode_step(store, t, w.W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"],
                          d["beta"], o=outs[t], stream=stream)
            if ev is not None:
                ev[t][1].record(stream)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()

    # Timed region: K passes back to back, bracketed by synchronisation.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        one_pass()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)

    # Per-launch durations of the decode kernel, from HIP events recorded on
    # the launch stream around every launch (a second live loop of K passes;
    # the events themselves add a few microseconds between launches).
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(w.L)]
           for _ in range(args.steps)]
    for k in range(args.steps):
        one_pass(evs[k])
    torch.cuda.synchronize()
    launch_ms = np.array([[e[0].elapsed_time(e[1]) for e in ev] for ev in evs])  # [K, L]

    # algorithmic bytes per launch (unique-record model, from the lineage itself)
    anc = store.anc.cpu().numpy()
    step_bytes, gather_bytes = [], []
    for t in range(w.L):
        uniq = sum(accounting.unique_ancestors(anc[t, r, :, :t], w.W) for r in range(w.R))
        kw = dict(R=w.R, H=w.H, dk=w.dk, dv=w.dv, W_t=w.W, t=t)
        step_bytes.append(accounting.beam_step_bytes(unique_records=uniq, **kw))
        gather_bytes.append(accounting.beam_step_bytes(**kw))
    mean_bytes = float(np.mean(step_bytes))
    mean_launch_s = float(launch_ms.mean()) * 1e-3
    achieved = mean_bytes / mean_launch_s / 1e9

    beam_steps = w.R * w.W * w.L * args.steps
    line = {
        "metric": METRIC,
        "value": beam_steps / (total_ms * 1e-3),
        "unit": "beam-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; bf16 q/k/v, FP32 state, gates and records)",
        "config": {"workload": w.name, "R": w.R, "W": w.W, "H": w.H, "dk": w.dk, "dv": w.dv,
                   "L": w.L, "hot_parent_fraction": w.hot_frac, "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "kernel": "k_beam_fused<128,128,t> (t = 0..L-1, one launch per decode step)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "bytes_per_launch": mean_bytes,
            "bytes_per_launch_per_beam_gather": float(np.mean(gather_bytes)),
            "launch_us": [float(x) * 1e3 for x in launch_ms.mean(0)],
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
