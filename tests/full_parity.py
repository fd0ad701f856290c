"""Full-size parity: the FP64 oracle on every (request, head) pair of a
workload, compared with the HIP path's outputs.

Test infrastructure.  A GPU test runs the HIP path, writes its outputs into a
directory as .npy files and then runs this file as a separate program (a
child process).  The child never touches the GPU, so it can fork a pool of
single-threaded workers over the host cores; each worker regenerates nothing:
it inherits the seeded inputs from the child's main process, slices out one
(request, head) pair (or a block of sequence pairs) and runs the oracle on
that slice alone.  Pairs are independent in the method (a request's shared
state, records and ancestry are private to it, and every quantity is per
head), so the oracle on a slice computes exactly what it computes for that
pair inside the whole workload.  Each worker returns the largest per-slice
relative error (infinity norm of the difference over that of the oracle's
slice) of o_t, delta_t and, for sequences, the merged bases; the child writes
them, with the worst pair, as JSON.

    python tests/full_parity.py beam <workload> <dir>  [--over JSON]
    python tests/full_parity.py seq  <workload> <dir>  [--over JSON]

Files read from <dir>:
    beam: o_<t>.npy, d_<t>.npy   FP32 [R, W_t, H, d_v] for t = 0 .. L-1
    seq:  o.npy, d.npy           FP32 [T, R, H, d_v]  (d: the record of each token)
          S_<m>.npy              FP32 [R, H, d_k, d_v] base after the m-th merge
and result.json is written there.
"""

from __future__ import annotations

import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# the host cores this run may use (16 per GPU on the GPU machines, whatever the
# machine reports in total)
MAX_WORKERS = 16

_INP = None  # the workload's inputs, inherited by the forked workers
_DIR = None
_SPEC = None


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


def _rel(x, ref):
    """max over slices (last axis) of |x - ref|_inf / |ref|_inf."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(x - ref).max(axis=-1)
    n = np.abs(ref).max(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(n > 0, d / np.where(n > 0, n, 1), np.where(d > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0


def _init():
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)


def _beam_pair(rh):
    import oracle.gdn_oracle as O

    r, h = rh
    steps = _INP["steps"]
    H = steps[0]["v"].shape[2]
    hk = h // (H // steps[0]["q"].shape[2])  # the value head's key head
    S0 = _INP["S0"][r:r + 1, h:h + 1]
    sl = []
    for st in steps:
        d = dict(q=st["q"][r:r + 1, :, hk:hk + 1], k=st["k"][r:r + 1, :, hk:hk + 1],
                 v=st["v"][r:r + 1, :, h:h + 1], alpha=st["alpha"][r:r + 1, :, h:h + 1],
                 beta=st["beta"][r:r + 1, :, h:h + 1])
        if "parent" in st:
            d["parent"] = st["parent"][r:r + 1]
        sl.append(d)
    ref = O.beam_decode(S0, sl, rule=_SPEC.get("rule", "delta"))
    eo = ed = 0.0
    for t in range(len(steps)):
        o = np.load(os.path.join(_DIR, f"o_{t}.npy"), mmap_mode="r")[r, :, h]
        d = np.load(os.path.join(_DIR, f"d_{t}.npy"), mmap_mode="r")[r, :, h]
        eo = max(eo, _rel(o, ref["o"][t][0, :, 0]))
        ed = max(ed, _rel(d, ref["delta"][t][0, :, 0]))
    return r, h, eo, ed


def _seq_block(pairs):
    import oracle.gdn_oracle as O

    M = _SPEC["M"]
    ref = O.sequence_decode(_INP["S0"], _INP["tokens"], M, pairs=pairs, rule=_SPEC.get("rule", "delta"))
    rs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    o = np.load(os.path.join(_DIR, "o.npy"), mmap_mode="r")
    d = np.load(os.path.join(_DIR, "d.npy"), mmap_mode="r")
    eo = _rel(o[:, rs, hs], ref["o"])
    ed = _rel(d[:, rs, hs], ref["delta"])
    es = 0.0
    for m in range(ref["bases"].shape[0]):
        S = np.load(os.path.join(_DIR, f"S_{m}.npy"), mmap_mode="r")[rs, hs]
        es = max(es, _rel(S.reshape(len(pairs), -1), ref["bases"][m].reshape(len(pairs), -1)))
    return pairs[0], eo, ed, es


def _main(argv):
    global _INP, _DIR, _SPEC
    import multiprocessing as mp

    from linear_attention_beam_gdn_amd import configs

    kind, name, _DIR = argv[:3]
    over = json.loads(argv[4]) if len(argv) > 4 and argv[3] == "--over" else {}
    w = configs.BY_NAME[name]
    if over:
        import dataclasses

        w = dataclasses.replace(w, **over)
    t0 = time.perf_counter()
    _INP = w.inputs()
    nw = workers()
    print(f"[full-parity] {w.name}: inputs in {time.perf_counter() - t0:.1f} s, {nw} workers", flush=True)
    ctx = mp.get_context("fork")
    res = {"workload": w.name, "workers": nw}
    if kind == "beam":
        _SPEC = {"rule": "delta"}
        items = [(r, h) for r in range(w.R) for h in range(w.H)]
        fn = _beam_pair
    else:
        _SPEC = {"M": w.M, "rule": w.rule}
        allp = [(r, h) for r in range(w.R) for h in range(w.H)]
        blk = max(1, len(allp) // (4 * nw))
        items = [allp[i:i + blk] for i in range(0, len(allp), blk)]
        fn = _seq_block
    worst = {"o": (0.0, None), "delta": (0.0, None), "base": (0.0, None)}
    done = 0
    t1 = time.perf_counter()
    with ctx.Pool(nw, initializer=_init) as pool:
        for out in pool.imap_unordered(fn, items):
            key = out[:2] if kind == "beam" else out[0]
            errs = out[2:] if kind == "beam" else out[1:]
            for name_, e in zip(("o", "delta", "base"), errs):
                if e > worst[name_][0]:
                    worst[name_] = (e, list(map(int, key)))
            done += 1
            if done % max(1, len(items) // 8) == 0:
                print(f"[full-parity] {done}/{len(items)} items, {time.perf_counter() - t1:.1f} s", flush=True)
    res["pairs"] = w.R * w.H
    res["seconds"] = time.perf_counter() - t0
    res["worst"] = {k: {"rel_err": v[0], "pair": v[1]} for k, v in worst.items() if v[1] is not None}
    with open(os.path.join(_DIR, "result.json"), "w") as f:
        json.dump(res, f)
    print(f"[full-parity] done: {json.dumps(res)}", flush=True)


def run(kind: str, name: str, outdir: str, over: dict | None = None, timeout: float = 600) -> dict:
    """Run the checker as a child program on the outputs in ``outdir``."""
    cmd = [sys.executable, os.path.abspath(__file__), kind, name, outdir]
    if over:
        cmd += ["--over", json.dumps(over)]
    env = dict(os.environ)
    env["OMP_NUM_THREADS"] = "1"
    p = subprocess.run(cmd, env=env, timeout=timeout, capture_output=True, text=True)
    sys.stdout.write(p.stdout)
    if p.returncode != 0:
        raise RuntimeError(f"full-parity checker failed ({p.returncode}):\n{p.stdout}\n{p.stderr}")
    with open(os.path.join(outdir, "result.json")) as f:
        return json.load(f)


if __name__ == "__main__":
    _main(sys.argv[1:])
