"""Throughput of the GDN large-beam decode path on one MI355X.

One step = one pass of the whole hot path over one batch: the L = 4 decode
steps (ancestry update, shared-context projections, record replay, current
transition, output and append) of 8 requests x 512 beams, H = 32 heads,
d_k = d_v = 128, on seeded synthetic inputs already resident in HBM.

Prints one JSON line: beam-steps/s, the roofline of the decode kernel
(algorithmic bytes per launch over its mean kernel time, taken by HIP events
that the runtime records around each launch after a cache-evicting read-only
sweep, against 8 TB/s; beside it the same launches back to back with no sweep,
and the timed loop's own rate, launch gaps included), and the FP64 CPU oracle
timed on a bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import dataclasses
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense
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


def host_cores():
    """(cores this process may run on, cores the machine reports)."""
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    return allowed, os.cpu_count() or allowed


# host cores a one-GPU share of the GPU machines holds; a pool never exceeds it
HOST_SHARE = 16


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
    allowed, total = host_cores()
    return {
        "value": beam_steps / dt,
        "unit": "beam-steps/s",
        "cores": workers,
        "cores_available": allowed,
        "cores_reported": total,
        "kind": "oracle",
        "sample": f"{len(pairs)} of {w.R * w.H} (request, head) pairs, all {w.W} beams x {w.L} "
                  f"steps each ({w.W * w.L * len(pairs)} beam-head-steps), {dt:.1f} s wall, "
                  f"one single-threaded worker per core",
    }


_PAD_CYCLES = []


def _pad(torch, stream):
    """Queue about 0.3 ms of untimed GPU work that touches no memory (torch's
    clock-spin kernel), so that the host issues the launches that follow
    while the GPU is still busy and no event pair brackets host-side launch
    latency.  The spin length is calibrated once against HIP events."""
    if not _PAD_CYCLES:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        torch.cuda._sleep(1_000_000)
        b.record(stream)
        torch.cuda.synchronize()
        us = max(a.elapsed_time(b) * 1e3, 1.0)
        _PAD_CYCLES.append(int(min(max(1_000_000 * 300.0 / us, 1e4), 1e8)))
    torch.cuda._sleep(_PAD_CYCLES[0])


def _queued(torch, stream, calls, flush=False):
    """Duration (us) of each call, issued back to back on the launch stream
    behind the untimed pad, each bracketed by a HIP event pair recorded on
    that stream.  With ``flush``, a 1 GiB read-only sweep runs (outside the
    event pair) before every call, so that each starts with the 256 MB
    Infinity Cache holding none of its data and no dirty line of other work
    (``flush="copy"``: a 1 GiB device copy instead, whose dirty lines drain
    during the call)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
    _pad(torch, stream)
    for (a, b), fn in zip(ev, calls):
        if flush == "copy":
            _copy_flush(torch)
        elif flush:
            _flush(torch)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def _queued_kernel(torch, stream, calls, flush=False):
    """As _queued, for calls that take a pair of timing events and hand it to
    their kernel launch (gdn_beam_decode_step_timed): the runtime records the
    pair as the kernel starts and completes, so each duration is the kernel's
    execution alone, without event commands of its own in the stream or a
    system-scope fence (KernelEvents)."""
    from linear_attention_beam_gdn_amd.measure import stream as S

    ev = S.KernelEvents(len(calls))
    try:
        _pad(torch, stream)
        for pair, fn in zip(ev.pairs, calls):
            if flush == "copy":
                _copy_flush(torch)
            elif flush:
                _flush(torch)
            fn(pair)
        torch.cuda.synchronize()
        return ev.elapsed_us()
    finally:
        ev.close()


_FLUSH_BUF = []
_COPY_BUF = []


def _copy_flush(torch):
    """A 1 GiB device copy on the current stream: evicts the Infinity Cache but
    leaves up to its size of dirty lines, written back during the next kernel."""
    if not _COPY_BUF:
        src = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
        _COPY_BUF.extend([src, torch.empty_like(src)])
    _COPY_BUF[1].copy_(_COPY_BUF[0])


def _flush(torch):
    """Evict the Infinity Cache on the current stream: a 1 GiB read-only
    sweep (leaves no dirty line behind to be written back during the next
    kernel)."""
    if not _FLUSH_BUF:
        from linear_attention_beam_gdn_amd.measure import stream as S

        _FLUSH_BUF.append(S.ReadFlush(torch))
    _FLUSH_BUF[0](torch.cuda.current_stream())


def _bw(nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bytes": float(nbytes), "us": us, "achieved_GBps": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}


# streaming rates of this GPU at several read:write mixes, from the
# hand-written reference kernel (set by main())
_STREAM_RATES = {}


def mix_rate(read_frac):
    """Streaming rate (GB/s) of a read fraction, piecewise linear between the
    measured mixes, or None before they exist."""
    if not _STREAM_RATES:
        return None
    from linear_attention_beam_gdn_amd.measure import stream as S

    return float(S.rate_at(_STREAM_RATES, read_frac))


def beam_precision(wl):
    """Arithmetic of the kernel that decodes a beam workload: how S0 (and, for
    channel decay, the FP32 probes) reach the matrix cores, and the resulting
    relative accuracy of the shared-context projection."""
    if wl.channel_decay:
        return ("S0 and the FP32 probes (decays folded in) each as two bf16 planes, hi*hi + hi*lo + lo*hi "
                "MFMA products, FP32 accumulation and replay: about 2^-17 relative")
    if wl.dk > 128:
        return ("S0 as two bf16 planes (hi + lo), bf16 q and k (exact plane products), FP32 accumulation "
                "and replay: about 2^-18 relative")
    return ("S0 as three bf16 planes (hi + mid + lo), bf16 q and k (exact plane products), FP32 "
            "accumulation and replay: about 2^-27 relative, below FP32 rounding")


SEQ_PRECISION = "FP32 FMAs on the FP32 base (no plane split), FP32 replay and fold"


def beam_row(B, torch, dev, stream, wl, reps):
    """The L decode steps of a beam workload: per-launch durations and
    bandwidth under the unique-record byte model."""
    inp = wl.inputs()
    steps = [B.upload(st, dev) for st in inp["steps"]]
    store = B.Store(wl.R, wl.W, wl.H, wl.dk, wl.dv, wl.L, channel_decay=wl.channel_decay,
                    S=torch.from_numpy(inp["S0"]).to(dev), Hk=wl.Hk)
    outs = [torch.empty(wl.R, wl.W, wl.H, wl.dv, dtype=torch.float32, device=dev) for _ in range(wl.L)]

    def launch(t, ev=None):
        d = steps[t]
        B.decode_step(store, t, wl.W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                      o=outs[t], stream=stream, events=ev)

    for _ in range(2):
        for t in range(wl.L):
            launch(t)
    torch.cuda.synchronize()
    # keep the step order: step t reads step t-1's records.  As for the
    # headline's roofline launches, a 1 GiB read-only sweep runs (untimed)
    # before every launch, and the runtime brackets each kernel with timing
    # events; the same launches back to back, where each one also drains the
    # previous one's dirty lines from the Infinity Cache, and the flushed
    # launches timed between event commands of their own, are reported beside.
    calls = [(lambda ev, t=t: launch(t, ev)) for _ in range(reps) for t in range(wl.L)]
    # one round untimed first: the first round of swept launches after a
    # workload's buffers are new runs 1-3 % slower than every later one
    _queued_kernel(torch, stream, calls, flush=True)
    d = _queued_kernel(torch, stream, calls, flush=True)
    d_b2b = _queued_kernel(torch, stream, calls)
    d_pair = _queued(torch, stream, [(lambda t=t: launch(t)) for _ in range(reps) for t in range(wl.L)], flush=True)
    us = [float(np.mean(d[t::wl.L])) for t in range(wl.L)]
    us_b2b = [float(np.mean(d_b2b[t::wl.L])) for t in range(wl.L)]
    us_pair = [float(np.mean(d_pair[t::wl.L])) for t in range(wl.L)]
    anc = store.anc.cpu().numpy()
    per = []
    for t in range(wl.L):
        uniq = sum(accounting.unique_ancestors(anc[t, r, :, :t], wl.W) for r in range(wl.R))
        nbytes = accounting.beam_step_bytes(R=wl.R, H=wl.H, dk=wl.dk, dv=wl.dv, W_t=wl.W, t=t,
                                            channel_decay=wl.channel_decay, unique_records=uniq, Hk=wl.Hk)
        per.append(_bw(nbytes, us[t]))
        wb = accounting.beam_step_write_bytes(R=wl.R, H=wl.H, dk=wl.dk, dv=wl.dv, W_t=wl.W, t=t,
                                              channel_decay=wl.channel_decay, Hk=wl.Hk)
        per[-1]["read_fraction"] = 1.0 - wb / nbytes
    tot_b, tot_us, tot_us_b2b = sum(p["bytes"] for p in per), sum(us), sum(us_b2b)
    out = {"workload": wl.name, "precision": beam_precision(wl), "decode_steps": wl.L,
           "cache": "Infinity Cache flushed (1 GiB read-only sweep) before every timed launch",
           "timing": "kernel time as the runtime brackets the launch (gdn_beam_decode_step_timed)",
           "beam_steps_per_s": wl.R * wl.W * wl.L / (tot_us * 1e-6),
           "launch_us": us, **{k: v for k, v in _bw(tot_b / wl.L, tot_us / wl.L).items() if k != "us"},
           "launch_us_event_pair": us_pair,
           "back_to_back": {"launch_us": us_b2b, "beam_steps_per_s": wl.R * wl.W * wl.L / (tot_us_b2b * 1e-6),
                            **{k: v for k, v in _bw(tot_b / wl.L, tot_us_b2b / wl.L).items() if k != "us"}}}
    # the L launches captured in a HIP graph, replayed back to back (what a
    # caller that replays whole decode passes sees; launch-bound shapes gain)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(wl.L):
            d = steps[t]
            B.decode_step(store, t, wl.W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"], o=outs[t])
    graph.replay()
    torch.cuda.synchronize()
    g_us = float(np.mean(_queued(torch, stream, [graph.replay] * reps)))
    del graph
    out["graph_replay"] = {"us_per_pass": g_us, "beam_steps_per_s": wl.R * wl.W * wl.L / (g_us * 1e-6),
                           **{k: v for k, v in _bw(tot_b / wl.L, g_us / wl.L).items() if k != "us"}}
    if _STREAM_RATES:
        out["read_fraction"] = [p["read_fraction"] for p in per]
        out["frac_of_mix_matched"] = (sum(p["bytes"] / (mix_rate(p["read_fraction"]) * 1e9) for p in per)
                                      / (tot_us * 1e-6))
    return out


# OneLA's printed operator latencies at its Qwen geometry (unnamed GPU; context only):
# R = 16 from §4.3 (GDN attention, largest shape), R = 4 from §4.4 (recurrent-state path)
ONELA_MS = {16: {3: 0.212, 7: 0.990}, 4: {3: 0.0755, 7: 0.308}}


def onela_latency_row(B, torch, dev, stream, wl, reps):
    """Decode latency of O - 1 back-to-back steps (O = 3 and 7 output tokens)
    at OneLA's Qwen geometry, beside the page's own figure for the shape."""
    inp = wl.inputs()
    steps = [B.upload(st, dev) for st in inp["steps"]]
    store = B.Store(wl.R, wl.W, wl.H, wl.dk, wl.dv, wl.L, S=torch.from_numpy(inp["S0"]).to(dev))
    outs = [torch.empty(wl.R, wl.W, wl.H, wl.dv, dtype=torch.float32, device=dev) for _ in range(wl.L)]

    def launch(t):
        d = steps[t]
        B.decode_step(store, t, wl.W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                      o=outs[t], stream=stream)

    for _ in range(2):
        for t in range(wl.L):
            launch(t)
    torch.cuda.synchronize()
    out = {"workload": wl.name}
    for O in (3, 7):
        T = O - 1
        tot = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            _pad(torch, stream)
            a.record(stream)
            for t in range(T):
                launch(t)
            b.record(stream)
            torch.cuda.synchronize()
            tot.append(a.elapsed_time(b))
        ms = float(np.median(tot))
        out[f"O={O}"] = {"decode_calls": T, "ms": ms, "beam_steps_per_s": wl.R * wl.W * T / (ms * 1e-3),
                         "page_ms": ONELA_MS[wl.R][O]}
    return out


def sequence_row(B, torch, dev, stream, wl):
    """Bounded-log decoding of independent sequences: every token's decode
    (log length token mod M) and the merge after every M tokens."""
    seq = wl.inputs()
    store = B.Store(wl.R, 1, wl.H, wl.dk, wl.dv, wl.M, channel_decay=wl.channel_decay,
                    S=torch.from_numpy(seq["S0"]).to(dev), plain_update=wl.plain_update)
    toks = [B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")}, dev)
            for i in range(wl.T)]
    zero = torch.zeros(wl.R, 1, dtype=torch.int32, device=dev)
    o = torch.empty(wl.R, 1, wl.H, wl.dv, dtype=torch.float32, device=dev)

    def decode(i):
        d = toks[i]
        B.decode_step(store, i % wl.M, 1, zero, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o=o, stream=stream)

    calls, kinds = [], []
    for i in range(wl.T):
        calls.append(lambda i=i: decode(i))
        kinds.append(i % wl.M)
        if i % wl.M == wl.M - 1:
            calls.append(lambda: B.log_merge(store, wl.M, 0, stream=stream))
            kinds.append(-1)
    # one untimed pass first (the first launch of a kernel also loads its code
    # object; a pass over T = a multiple of M tokens leaves the log empty)
    for fn in calls:
        fn()
    torch.cuda.synchronize()
    d = _queued(torch, stream, calls)
    dec_us = [float(np.mean([x for x, k in zip(d, kinds) if k == j])) for j in range(wl.M)]
    merge_us = float(np.mean([x for x, k in zip(d, kinds) if k == -1]))
    d = _queued(torch, stream, calls, flush=True)
    dec_us_fl = [float(np.mean([x for x, k in zip(d, kinds) if k == j])) for j in range(wl.M)]
    merge_us_fl = float(np.mean([x for x, k in zip(d, kinds) if k == -1]))

    # the same tokens with the merge fused into the decode that fills the log
    fstore = B.Store(wl.R, 1, wl.H, wl.dk, wl.dv, wl.M, channel_decay=wl.channel_decay,
                     S=torch.from_numpy(seq["S0"]).to(dev), plain_update=wl.plain_update)

    def fused(i):
        d = toks[i]
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        if i % wl.M == wl.M - 1:
            B.decode_merge_step(fstore, i % wl.M, *args, o=o, stream=stream)
        else:
            B.decode_step(fstore, i % wl.M, 1, zero, *args, o=o, stream=stream)

    fcalls = [(lambda i=i: fused(i)) for i in range(wl.T)]
    for fn in fcalls:
        fn()
    torch.cuda.synchronize()
    df = _queued(torch, stream, fcalls)
    fdec_us = [float(np.mean(df[j::wl.M])) for j in range(wl.M)]
    df = _queued(torch, stream, fcalls, flush=True)
    fdec_us_fl = [float(np.mean(df[j::wl.M])) for j in range(wl.M)]
    df = _queued(torch, stream, fcalls, flush="copy")
    fdec_us_cfl = [float(np.mean(df[j::wl.M])) for j in range(wl.M)]

    # one merge cycle of the fused path captured in a HIP graph and replayed
    # (the replays keep decoding the cycle's M tokens on the evolving base)
    gstore = B.Store(wl.R, 1, wl.H, wl.dk, wl.dv, wl.M, channel_decay=wl.channel_decay,
                     S=torch.from_numpy(seq["S0"]).to(dev), plain_update=wl.plain_update)
    gout = torch.empty_like(o)

    def gcycle():
        for i in range(wl.M):
            d = toks[i]
            args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
            if i == wl.M - 1:
                B.decode_merge_step(gstore, i, *args, o=gout)
            else:
                B.decode_step(gstore, i, 1, zero, *args, o=gout)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gcycle()
    graph.replay()
    torch.cuda.synchronize()
    n_rep = max(1, wl.T // wl.M)
    graph_cycle_us = float(np.mean(_queued(torch, stream, [graph.replay] * n_rep)))
    dec_b = [accounting.sequence_token_bytes(R=wl.R, H=wl.H, dk=wl.dk, dv=wl.dv, log_len=j,
                                             channel_decay=wl.channel_decay, plain=wl.plain_update)
             for j in range(wl.M)]
    mrg_b = accounting.merge_bytes(R=wl.R, H=wl.H, dk=wl.dk, dv=wl.dv, n_rec=wl.M, channel_decay=wl.channel_decay,
                                   plain=wl.plain_update)
    cycle_us = sum(dec_us) + merge_us
    fdm_b = accounting.decode_merge_bytes(R=wl.R, H=wl.H, dk=wl.dk, dv=wl.dv, log_len=wl.M - 1,
                                          channel_decay=wl.channel_decay, plain=wl.plain_update)
    fcycle_us = sum(fdec_us)
    fcycle_b = sum(dec_b[:-1]) + fdm_b
    fcycle_us_fl = sum(fdec_us_fl)
    cycle_us_fl = sum(dec_us_fl) + merge_us_fl
    return {"workload": wl.name, "precision": SEQ_PRECISION,
            "sequence_steps_per_s": wl.R * wl.M / (fcycle_us_fl * 1e-6),
            "us_per_token_amortised": fcycle_us_fl / wl.M,
            # every launch after a read-only cache-flushing sweep (as the headline is timed)
            "fused_cycle_flushed": {**_bw(fcycle_b, fcycle_us_fl), "us_by_log_length": fdec_us_fl,
                                    "decode_merge": _bw(fdm_b, fdec_us_fl[-1])},
            # every launch after a 1 GiB copy instead, whose dirty lines drain during the launch
            "fused_cycle_after_copy_flush": {**_bw(fcycle_b, sum(fdec_us_cfl)), "us_by_log_length": fdec_us_cfl},
            "separate_flushed": {"sequence_steps_per_s": wl.R * wl.M / (cycle_us_fl * 1e-6),
                                 "merge": _bw(mrg_b, merge_us_fl),
                                 "cycle": _bw(sum(dec_b) + mrg_b, cycle_us_fl)},
            # the same launches back to back with no flush: part of the 268 MB
            # base can still sit in the Infinity Cache from the previous token
            "fused_cycle_warm": {**_bw(fcycle_b, fcycle_us), "us_by_log_length": fdec_us,
                                 "decode_merge": _bw(fdm_b, fdec_us[-1])},
            "fused_cycle_graph_replay_warm": _bw(fcycle_b, graph_cycle_us),
            "separate_warm": {"sequence_steps_per_s": wl.R * wl.M / (cycle_us * 1e-6),
                              "decode": {**_bw(float(np.mean(dec_b)), float(np.mean(dec_us))),
                                         "us_by_log_length": dec_us},
                              "merge": _bw(mrg_b, merge_us),
                              "cycle": _bw(sum(dec_b) + mrg_b, cycle_us)}}


def merge_interval_row(B, torch, dev, stream, wl, intervals):
    """The bounded-log workload at several log capacities M (DeltaLog Figure 9
    sweeps M = 4 and 8): amortised time per token and bandwidth of one merge
    cycle, merge fused into the decode that fills the log and separate."""
    out = {}
    for m in intervals:
        r = sequence_row(B, torch, dev, stream, dataclasses.replace(wl, M=m))
        out[f"M={m}"] = {"us_per_token_amortised": r["us_per_token_amortised"],
                         "achieved_GBps": r["fused_cycle_flushed"]["achieved_GBps"],
                         "frac_of_peak": r["fused_cycle_flushed"]["frac_of_peak"],
                         "separate_us_per_token_amortised": r["separate_flushed"]["cycle"]["us"] / m,
                         "warm_us_per_token_amortised": r["fused_cycle_warm"]["us"] / m}
    return out


def split_replay_row(B, torch, dev, stream, wl, intervals=(4, 8), splits=(1, 2, 4)):
    """DeltaLog's split-replay ablation (Figure 9): the bounded-log workload
    with d_v cut into value tiles, the replay preparation formed once per
    (sequence, head) and shared through a workspace, or repeated by every
    tile; per-token latency amortised over one merge cycle (the merge fused
    into the token that fills the log), timed per call with a cache flush
    before each, and the same cycle captured in a HIP graph and replayed
    (as the page times it; back to back, no flush)."""
    seq = wl.inputs()
    toks = [B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")}, dev)
            for i in range(max(intervals))]
    o = torch.empty(wl.R, 1, wl.H, wl.dv, dtype=torch.float32, device=dev)
    out = {"workload": wl.name, "precision": SEQ_PRECISION}
    for m in intervals:
        row = {}
        for n in splits:
            for shared in (False, True):
                if n == 1 and shared:
                    continue
                store = B.Store(wl.R, 1, wl.H, wl.dk, wl.dv, m, channel_decay=wl.channel_decay,
                                S=torch.from_numpy(seq["S0"]).to(dev), plain_update=wl.plain_update)
                ws = (torch.empty(B.split_workspace_bytes(store) // 4, dtype=torch.float32, device=dev)
                      if shared else None)

                def call(i, store=store, ws=ws, n=n, shared=shared):
                    # on the current stream (the capture stream inside graph capture)
                    d = toks[i]
                    B.decode_step_split(store, i, n, shared, i == m - 1, d["q"], d["k"], d["v"], d["alpha"],
                                        d["beta"], o=o, workspace=ws)

                calls = [(lambda i=i: call(i)) for i in range(m)]
                for fn in calls:
                    fn()
                torch.cuda.synchronize()
                fl = _queued(torch, stream, calls, flush=True)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for fn in calls:
                        fn()
                graph.replay()
                torch.cuda.synchronize()
                g_us = float(np.mean(_queued(torch, stream, [graph.replay] * 8)))
                key = "unsplit" if n == 1 else f"{n}_tiles_{'shared' if shared else 'repeated'}_preparation"
                row[key] = {"us_per_token_flushed": sum(fl) / m, "us_per_token_graph_replay": g_us / m,
                            "us_by_log_length_flushed": fl}
                del store, ws, graph
        out[f"M={m}"] = row
    return out


def materialize_row(B, torch, dev, stream, wl, n_items, reps):
    """Dense states of n_items beams after the last step of a beam workload."""
    inp = wl.inputs()
    store = B.Store(wl.R, wl.W, wl.H, wl.dk, wl.dv, wl.L, channel_decay=wl.channel_decay,
                    S=torch.from_numpy(inp["S0"]).to(dev), Hk=wl.Hk)
    for t, st in enumerate(inp["steps"]):
        d = B.upload(st, dev)
        B.decode_step(store, t, wl.W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"], stream=stream)
    rng = np.random.default_rng(0)
    pairs = np.stack([np.arange(n_items) % wl.R, rng.integers(0, wl.W, n_items)], 1).astype(np.int32)
    rb = torch.from_numpy(pairs).to(dev)
    out = torch.empty(n_items, wl.H, wl.dk, wl.dv, dtype=torch.float32, device=dev)
    B.materialize(store, wl.L - 1, rb, out=out, stream=stream)
    calls = [lambda: B.materialize(store, wl.L - 1, rb, out=out, stream=stream)] * reps
    us = float(np.mean(_queued(torch, stream, calls, flush=True)))  # each after the read-only sweep
    us_b2b = float(np.mean(_queued(torch, stream, calls)))
    rec = accounting.record_bytes(wl.dk, wl.dv, wl.channel_decay)
    reqs = len(set(pairs[:, 0].tolist()))
    nbytes = reqs * wl.H * 4 * wl.dk * wl.dv + n_items * wl.H * (4 * wl.dk * wl.dv + wl.L * rec)
    return {"workload": f"{wl.name}: {n_items} beams after step {wl.L - 1}", **_bw(nbytes, us),
            "back_to_back": _bw(nbytes, us_b2b)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=32)
    ap.add_argument("--cpu-workers", type=int, default=0)
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other path rows (channel decay, bounded log, materialise)")
    ap.add_argument("--rows", default="",
                    help="comma-separated subset of the rows to run (default: all of them)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming-rate reference kernels (for profiler runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the rows and the warm-up, run a plain device copy of this many MiB three times "
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
        workers = args.cpu_workers or min(HOST_SHARE, host_cores()[0])
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

    def one_step(t, ev=None):
        d = steps[t]
        B.decode_step(store, t, w.W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"], o=outs[t],
                      stream=stream, events=ev)

    def one_pass():
        for t in range(w.L):
            one_step(t)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The other rows run first.  This GPU raises its clocks over the first
    # tens of milliseconds of sustained work (measured: a cold device's first
    # 20 headline passes take about 350 us each, against 323 us once it has
    # run decode work for 20 ms), so the headline's warm-up passes and timed
    # passes below find it at the clocks it holds under a steady decode load.
    row_results = None
    if not args.no_rows:
        reps = max(3, min(args.steps, 10))
        rows = {
            "single_request_beam_decode": lambda: beam_row(B, torch, dev, stream, configs.SINGLE, reps),
            "channel_decay_beam_decode": lambda: beam_row(B, torch, dev, stream, configs.KDA, reps),
            "shared_key_heads_beam_decode": lambda: beam_row(B, torch, dev, stream, configs.SHARED_KEYS, reps),
            "wide_state_beam_decode": lambda: beam_row(B, torch, dev, stream, configs.WIDE, reps),
            "channel_decay_wide_value_beam_decode": lambda: beam_row(B, torch, dev, stream, configs.KDA_WIDE, reps),
            # chains to the OneLA operator suite's longest (T = 6): the same
            # workloads decoded for seven steps, t = 0 .. 6
            "long_chain_beam_decode": lambda: beam_row(B, torch, dev, stream, dataclasses.replace(WORKLOAD, L=7), reps),
            "wide_state_long_chain_beam_decode": lambda: beam_row(B, torch, dev, stream,
                                                                  dataclasses.replace(configs.WIDE, L=7), reps),
            "channel_decay_long_chain_beam_decode": lambda: beam_row(B, torch, dev, stream,
                                                                     dataclasses.replace(configs.KDA, L=7), reps),
            "bounded_log_decode_and_merge": lambda: sequence_row(B, torch, dev, stream, configs.DELTALOG),
            "bounded_log_merge_interval": lambda: merge_interval_row(B, torch, dev, stream, configs.DELTALOG,
                                                                     (4, 8, 16)),
            "rwkv6_bounded_log": lambda: sequence_row(B, torch, dev, stream, configs.RWKV6),
            "kda_bounded_log": lambda: sequence_row(B, torch, dev, stream, configs.KDA_LOG),
            "split_replay_gdn": lambda: split_replay_row(B, torch, dev, stream, configs.DELTALOG),
            "split_replay_kda": lambda: split_replay_row(B, torch, dev, stream, configs.KDA_LOG),
            "split_replay_rwkv6": lambda: split_replay_row(B, torch, dev, stream, configs.RWKV6),
            "materialize": lambda: materialize_row(B, torch, dev, stream, WORKLOAD, 64, reps),
            "onela_qwen_geometry_latency_r4": lambda: onela_latency_row(B, torch, dev, stream, configs.QWEN_R4, reps),
            "onela_qwen_geometry_latency_r16": lambda: onela_latency_row(B, torch, dev, stream, configs.QWEN_R16, reps),
        }
        pick = [r for r in args.rows.split(",") if r] or list(rows)
        unknown = [r for r in pick if r not in rows]
        if unknown:
            sys.exit(f"unknown rows {unknown}; choose from {sorted(rows)}")
        # light and sequence rows first, the beam decode rows last (ending
        # with the headline geometry's long chains) right before the headline;
        # the results keep the order above
        first = ("single_request_beam_decode", "onela_qwen_geometry_latency_r4",
                 "onela_qwen_geometry_latency_r16", "materialize", "bounded_log_decode_and_merge",
                 "bounded_log_merge_interval", "rwkv6_bounded_log", "kda_bounded_log", "split_replay_gdn",
                 "split_replay_kda", "split_replay_rwkv6")
        last = ("long_chain_beam_decode",)
        order = ([r for r in pick if r in first] + [r for r in pick if r not in first and r not in last]
                 + [r for r in pick if r in last])
        done = {name: rows[name]() for name in order}
        row_results = {name: done[name] for name in pick}

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()

    # Timed region: K passes back to back, bracketed by synchronisation.  The
    # untimed pad ahead of the start event lets the host queue the first
    # launches before the GPU reaches them, so the host's latency in issuing
    # the first launch is not inside the region.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _pad(torch, stream)
    start.record(stream)
    for _ in range(args.steps):
        one_pass()
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)

    # The same passes captured in a HIP graph and replayed (context: on this
    # stack a replayed pass has been no faster than the launches above).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t, d in enumerate(steps):
            B.decode_step(store, t, w.W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                          o=outs[t])
    for _ in range(args.warmup):
        graph.replay()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _pad(torch, stream)
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1)
    del graph

    # What this GPU streams: the hand-written reference kernel at read:write
    # mixes from writes only to reads only (fully coalesced 16-byte accesses
    # over 2 GiB, best of several launch shapes and store kinds); the 1:1 mix
    # is the device copy.  torch's own copy kernel is timed beside it.
    from linear_attention_beam_gdn_amd.measure import stream as S

    stream_rates = {} if args.no_ceilings else S.all_rates(torch, stream)
    copy_gbps = stream_rates["r1w1"]["GBps"] if stream_rates else float("nan")
    src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    torch_copy_gbps = 2 * src.numel() * 4 / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9

    # Per-launch durations of the decode kernel (a second live loop of K
    # passes): HIP events on the launch stream that the runtime records as
    # each kernel starts and completes (gdn_beam_decode_step_timed), created
    # without the system-scope fence a default event adds, so that they time
    # the kernel as rocprofv3's kernel trace does.  A 1 GiB read-only sweep
    # runs, untimed, before every launch, so that each launch starts with the
    # 256 MB Infinity Cache holding none of its data and no dirty line of
    # other work.  Beside: the same launches between default event commands
    # recorded around each (which add their own cost to every launch), and
    # after a 1 GiB copy instead of the sweep (whose dirty lines drain during
    # the launch).
    def timed_passes(flush, kernel=True):
        if kernel:
            calls = [(lambda ev, t=t: one_step(t, ev)) for _ in range(args.steps) for t in range(w.L)]
            us = _queued_kernel(torch, stream, calls, flush=flush)
        else:
            calls = [(lambda t=t: one_step(t)) for _ in range(args.steps) for t in range(w.L)]
            us = _queued(torch, stream, calls, flush=flush)
        return np.array(us).reshape(args.steps, w.L) * 1e-3  # [K, L] ms

    timed_passes(True)  # untimed round (as in the rows)
    launch_ms = timed_passes(True)
    launch_ms_pair = timed_passes(True, kernel=False)
    launch_ms_copy = timed_passes("copy")
    # and back to back with no sweep (the steady state of the timed loop:
    # each launch meets what the previous one left in the caches)
    launch_ms_b2b = timed_passes(False)
    del src, dst
    # what any launch timed the same way costs: a near-empty launch after the
    # same sweep, bracketed by the runtime, and between event commands
    empty_us = S.empty_kernel_us(torch, stream)
    empty_pair_us = S.empty_launch_us(torch, stream)

    # algorithmic bytes per launch (unique-record model, from the lineage itself)
    anc = store.anc.cpu().numpy()
    step_bytes, gather_bytes = [], []
    for t in range(w.L):
        uniq = sum(accounting.unique_ancestors(anc[t, r, :, :t], w.W) for r in range(w.R))
        kw = dict(R=w.R, H=w.H, dk=w.dk, dv=w.dv, W_t=w.W, t=t)
        step_bytes.append(accounting.beam_step_bytes(unique_records=uniq, **kw))
        gather_bytes.append(accounting.beam_step_bytes(**kw))
    mean_bytes = float(np.mean(step_bytes))
    # each launch's read fraction, and the streaming rate of that mix on this
    # GPU (piecewise linear between the measured mixes); frac_of_mix_matched
    # is the time those rates would take for the launches' bytes over the
    # launches' measured time
    write_bytes = [accounting.beam_step_write_bytes(R=w.R, H=w.H, dk=w.dk, dv=w.dv, W_t=w.W, t=t)
                   for t in range(w.L)]
    read_frac = [1.0 - wb / sb for wb, sb in zip(write_bytes, step_bytes)]
    _STREAM_RATES.update(stream_rates)
    mix_rates = [mix_rate(f) for f in read_frac] if stream_rates else [float("nan")] * len(read_frac)
    mix_s = sum(b_ / (r * 1e9) for b_, r in zip(step_bytes, mix_rates))
    mfma_flops = 3 * 2 * 2 * w.dk * w.dv * w.R * w.W * w.H
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
            "precision": beam_precision(w),
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            # what this GPU streams beside the nominal peak: the hand-written
            # reference kernel's device copy, and each read:write mix
            "copy_GBps": copy_gbps,
            "frac_of_copy": achieved / copy_gbps,
            "torch_copy_GBps": torch_copy_gbps,
            "stream_GBps": {k: v["GBps"] for k, v in stream_rates.items()},
            "read_fraction": read_frac,
            "mix_matched_GBps": mix_rates,
            "frac_of_mix_matched": mix_s / (float(launch_ms.mean(0).sum()) * 1e-3),
            "cache": "Infinity Cache flushed (1 GiB read-only sweep) before every timed launch",
            "timing": ("kernel time as the runtime brackets each launch (gdn_beam_decode_step_timed: "
                       "hipExtLaunchKernel events without a system-scope fence), as rocprofv3's kernel "
                       "trace times it"),
            "launch_us_event_pair": [float(x) * 1e3 for x in launch_ms_pair.mean(0)],
            "frac_event_pair": mean_bytes / (float(launch_ms_pair.mean()) * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "launch_us_after_copy_flush": [float(x) * 1e3 for x in launch_ms_copy.mean(0)],
            "launch_us_back_to_back": [float(x) * 1e3 for x in launch_ms_b2b.mean(0)],
            "frac_back_to_back": mean_bytes / (float(launch_ms_b2b.mean()) * 1e-3) / 1e9 / HBM_PEAK_GBS,
            # the timed loop's own rate: every launch's bytes over the wall
            # clock of the back-to-back passes, the gaps between launches included
            "frac_sustained": w.L * mean_bytes / (total_ms / args.steps * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "bytes_per_launch": mean_bytes,
            "bytes_per_launch_per_beam_gather": float(np.mean(gather_bytes)),
            "launch_us": [float(x) * 1e3 for x in launch_ms.mean(0)],
            "empty_launch_us": empty_us,
            "empty_launch_us_event_pair": empty_pair_us,
            # the S0^T [q | k] contraction on the matrix cores: three bf16 planes
            # x two probes x 2 d_k d_v FLOP per beam-head, over the same launches
            "mfma_tflops": mfma_flops / mean_launch_s / 1e12,
            "mfma_frac_of_bf16_peak": mfma_flops / mean_launch_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        },
        "value_graph_replay": beam_steps / (graph_ms * 1e-3),
        "cpu_baseline": cpu,
    }
    if row_results is not None:
        line["rows"] = row_results
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
