"""Where a headline decode launch spends its time: per-workgroup clock stamps.

Runs a beam workload (by default the large-beam one: 8 requests x 512 beams,
H = 32, d_k = d_v = 128, four decode steps; or any scalar- or channel-decay
beam workload whose chunks hold all its beams) on libgdnbeam_stamps.so, the
library built with the fused kernels' clock stamps compiled in (lane 0 of one
consumer wave per workgroup reads the 100 MHz real-time clock at entry, after
each prologue barrier and after its last tile).  Each launch runs after a 1 GiB read-only
sweep that evicts the Infinity Cache, with its kernel time taken as the
benchmark takes it (HIP events the runtime records as the kernel starts and
completes).  Prints a markdown summary: per step, the median time of each
phase boundary after the first workgroup's entry, the tile loop's length, the
spread of the exits, and the part of the kernel time that no workgroup
covers.

    python -m linear_attention_beam_gdn_amd.measure.stamps [--reps N] [--out FILE] [--workload NAME]
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

PKG = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

NAMES = ["entry", "Q (schedule inputs in)", "P (schedule built)", "S (S0 staged)", "A (tile 0 in)",
         "loop start (tile 0 prepared)", "last tile done"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--out", default="")
    ap.add_argument("--workload", default="gdn_large_beam",
                    help="a beam workload whose chunks hold all its beams (one chunk per slice)")
    args = ap.parse_args()

    import torch

    from linear_attention_beam_gdn_amd import binding as B
    from linear_attention_beam_gdn_amd import build, configs

    B.LIB_PATH = build.STAMPS_LIB
    L = B.lib()
    w = configs.BY_NAME[args.workload]
    kda = w.channel_decay
    read = L.gdn_kda_stamps_read if kda else L.gdn_stamps_read
    read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    read.restype = ctypes.c_int
    L.gdn_stamps_clock_khz.argtypes = []
    L.gdn_stamps_clock_khz.restype = ctypes.c_int

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    # value slices per (request, head): 128 value rows each, or 256 for
    # channel decay with d_v >= 256 and chains of at most three records
    nvs = w.dv // 128 if w.dv > 128 else 1
    if kda and w.dv >= 256:
        if w.L > 4:
            raise SystemExit("channel decay at d_v >= 256: the slice width changes past t = 3; use L <= 4")
        nvs = w.dv // 256
    tb = 8 if kda else 16  # beams per tile
    inp = w.inputs()
    steps = [B.upload(st, dev) for st in inp["steps"]]
    store = B.Store(w.R, w.W, w.H, w.dk, w.dv, w.L, S=torch.from_numpy(inp["S0"]).to(dev), Hk=w.Hk,
                    channel_decay=kda)
    outs = [torch.empty(w.R, w.W, w.H, w.dv, dtype=torch.float32, device=dev) for _ in range(w.L)]
    stream = torch.cuda.current_stream()
    # at most one workgroup per (request, head, value slice) with every beam in
    # one chunk (fewer where a workgroup takes two heads); the reader clears
    # the stamps, so rows of workgroups a launch did not have read zero
    n_wg = w.R * w.H * nvs

    def launch(t, ev=None):
        d = steps[t]
        B.decode_step(store, t, w.W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                      o=outs[t], stream=stream, events=ev)

    for _ in range(2):
        for t in range(w.L):
            launch(t)
    torch.cuda.synchronize()
    khz = L.gdn_stamps_clock_khz()
    tick_us = 1e3 / khz
    from linear_attention_beam_gdn_amd.measure import stream as S

    flush = S.ReadFlush(torch)
    buf = np.zeros((n_wg, 16), np.uint64)
    if read(buf.ctypes.data, n_wg) != 0:  # clears what the warm-up launches wrote
        raise RuntimeError("gdn_stamps_read failed")
    rows = {t: [] for t in range(w.L)}
    for _ in range(args.reps):
        for t in range(w.L):
            flush(stream)
            ev = S.KernelEvents(1)
            try:
                launch(t, ev.pairs[0])
                torch.cuda.synchronize()
                kernel_us = ev.elapsed_us()[0]
            finally:
                ev.close()
            rc = read(buf.ctypes.data, n_wg)
            if rc != 0:
                raise RuntimeError(f"gdn_stamps_read returned {rc}")
            rows[t].append((kernel_us, buf.copy()))

    live = np.stack([r[1] for r in rows[0]])[0, :, 0] != 0  # workgroups the launches had
    for t in range(w.L):
        rows[t] = [(ev, st[live]) for ev, st in rows[t]]
    n_wg = int(live.sum())
    kname = "k_beam_fused_kda" if kda else "k_beam_fused"
    lines = [f"Clock stamps of `{kname}<{w.dk},{w.dv},t>` at `{w.name}` ({w.R} x {w.W} beams, H = {w.H}, "
             f"d_k = {w.dk}, d_v = {w.dv}; {n_wg} workgroups), "
             f"{args.reps} launches per step, each after a 1 GiB read-only cache-flushing sweep; real-time clock "
             f"{khz / 1e3:.0f} MHz; times in us after the first workgroup's entry, medians over "
             f"workgroups and launches; kernel time as the runtime's events bracket the launch.", ""]
    hdr = "| step | kernel time | " + " | ".join(NAMES[1:]) + " | loop (median) | loop p10-p90 | " \
          "exit spread (last - median) | first entry to last exit | kernel time - that |"
    lines += [hdr, "|" + "---|" * (hdr.count("|") - 1)]
    xcd_rows = []
    for t in range(w.L):
        ev = np.array([r[0] for r in rows[t]])
        st = np.stack([r[1] for r in rows[t]]).astype(np.int64)  # [reps, wg, 8]
        t0 = st[:, :, 0].min(axis=1, keepdims=True)
        rel = (st[:, :, :7] - t0[..., None]) * tick_us
        if t == 0:
            rel[:, :, 1] = np.nan  # no barrier Q without a chain
        med = [np.nanmedian(rel[:, :, i]) for i in range(1, 7)]
        loop = (st[:, :, 6] - st[:, :, 5]) * tick_us
        last = rel[:, :, 6].max(axis=1)
        spread = last - np.median(rel[:, :, 6], axis=1)
        gap = ev - last
        lines.append(f"| {t} | {np.median(ev):.1f} | " + " | ".join(f"{m:.1f}" for m in med) +
                     f" | {np.median(loop):.1f} | {np.percentile(loop, 10):.1f}-{np.percentile(loop, 90):.1f} | "
                     f"{np.median(spread):.1f} | {np.median(last):.1f} | {np.median(gap):.1f} |")
        xcd = (st[:, :, 7] >> 32) & 0xF
        per = {int(x): float(np.median(rel[:, :, 6][xcd == x])) for x in np.unique(xcd)}
        xcd_rows.append((t, per))
    nt = w.W // tb * (w.R * w.H * nvs // n_wg)  # tiles per workgroup (two heads' worth where paired)
    if kda:
        lines += ["", "Work and waits inside the tile loop, us per tile (medians over workgroups and launches; "
                  f"{nt} tiles of {tb} beams per workgroup): each consumer wave prepares its share of tile i + 1 (probes, "
                  "record weights, appends), then finishes tile i (matrix-core products, replay, stores), and all meet "
                  "at a barrier; a DMA wave waits until the tile prepared next has landed.", "",
                  "| step | consumer wave 0: preparation | consumer wave 0: finishing | consumer wave 0: at barrier | "
                  "last consumer wave: work | last consumer wave: at barrier | DMA wave 0: waiting | "
                  "DMA wave 1: waiting |", "|---|---|---|---|---|---|---|---|"]
        for t in range(w.L):
            st = np.stack([r[1] for r in rows[t]]).astype(np.int64)
            f = lambda i: float(np.median(st[:, :, i])) * tick_us / nt
            lines.append(f"| {t} | {f(8):.2f} | {f(9):.2f} | {f(10):.2f} | {f(13):.2f} | {f(14):.2f} | "
                         f"{f(11):.2f} | {f(12):.2f} |")
    else:
        lines += ["", "Work and waits inside the tile loop, us per tile (medians over workgroups and launches; "
                  f"{nt} tiles of {tb} beams per workgroup): the dot wave forms tile i + 1's dot products and decay "
                  "weights while the consumers take tile i, and both then meet at a barrier; a DMA wave waits until "
                  "the tile the dot wave takes next has landed.", "",
                  "| step | dot wave: tile 0 (prologue) | dot wave: work per tile | dot wave: at barrier | "
                  "consumer wave 0: work per tile | consumer wave 0: at barrier | DMA wave 0: waiting | "
                  "DMA wave 1: waiting |", "|---|---|---|---|---|---|---|---|"]
        for t in range(w.L):
            st = np.stack([r[1] for r in rows[t]]).astype(np.int64)
            f = lambda i, n: float(np.median(st[:, :, i])) * tick_us / n
            lines.append(f"| {t} | {f(9, 1):.2f} | {f(8, nt - 1):.2f} | {f(13, nt):.2f} | {f(10, nt):.2f} | "
                         f"{f(14, nt):.2f} | {f(11, nt):.2f} | {f(12, nt):.2f} |")
    lines += ["", "Median exit (last tile done) per XCD, us after the first entry:", "",
              "| step | " + " | ".join(f"XCD {x}" for x in sorted(xcd_rows[0][1])) + " |",
              "|---|" + "---|" * len(xcd_rows[0][1])]
    for t, per in xcd_rows:
        lines.append(f"| {t} | " + " | ".join(f"{per[x]:.1f}" for x in sorted(per)) + " |")
    text = "\n".join(lines)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
