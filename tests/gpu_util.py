"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs, and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

from linear_attention_beam_gdn_amd import binding as B

TOL = 1e-4  # max relative error (per-slice infinity norm) against the FP64 oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_slices(x, ref, mask=None):
    """max over slices (last axis) of |x - ref|_inf / |ref|_inf, skipping
    slices where ref is NaN (not computed by the oracle)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    keep = ~np.isnan(ref).any(axis=-1)
    if mask is not None:
        keep &= mask
    if not keep.any():
        raise AssertionError("nothing to compare")
    d = np.abs(x - ref).max(axis=-1)[keep]
    n = np.abs(ref).max(axis=-1)[keep]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(n > 0, d / np.where(n > 0, n, 1), np.where(d > 0, np.inf, 0.0))
    return float(r.max())


def rel_states(x, ref):
    """max over (item, head) of |x - ref|_inf / |ref|_inf for [n,H,dk,dv]."""
    x = np.asarray(x, np.float64).reshape(x.shape[0], x.shape[1], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], ref.shape[1], -1)
    return rel_slices(x, ref)


def run_beam(inp, channel=False, L_max=None, W_max=None, S=None):
    """Decode every step of ``inp`` through the C ABI; returns (store, [o_t])."""
    S0 = inp["S0"]
    R, H, dk, dv = S0.shape
    widths = [st["q"].shape[1] for st in inp["steps"]]
    W_max = W_max or max(widths)
    L_max = L_max or len(inp["steps"])
    S_dev = torch.from_numpy(np.ascontiguousarray(S0)).cuda() if S is None else S
    Hk = inp["steps"][0]["q"].shape[2]  # key heads (== H unless value heads share them)
    store = B.Store(R, W_max, H, dk, dv, L_max, channel_decay=channel, S=S_dev, Hk=Hk)
    outs = []
    for t, st in enumerate(inp["steps"]):
        d = B.upload(st)
        o = B.decode_step(store, t, widths[t], d.get("parent"), d["q"], d["k"], d["v"],
                          d["alpha"], d["beta"])
        outs.append(o)
    torch.cuda.synchronize()
    return store, [o.cpu().numpy() for o in outs]


def record_slots(store, t, W_t):
    """[R, W_t] record slot of each beam at step t: with scalar decay and
    beams (W_max > 1) a step stores a beam's record at its order key, the
    last entry of its ancestry row, from step 1 on; otherwise at its index."""
    idx = np.tile(np.arange(W_t, dtype=np.int64), (store.R, 1))
    if t == 0 or store.channel_decay or store.W_max == 1:
        return idx
    keys = store.anc[t, :, :W_t, store.L_max - 1].cpu().numpy().astype(np.int64)
    for r in range(store.R):  # the keys of a step's beams are a permutation of its slots
        assert np.array_equal(np.sort(keys[r]), np.arange(W_t)), f"step {t}: order keys are not a permutation"
    return keys


def step_records(store, t, W_t, widths=None):
    """(delta [R,W_t,H,dv], k bits [R,W_t,Hk,dk], alpha, anc [R,W_t,t]) at
    step t, per beam index: each beam's record read at its slot, and the
    ancestry rows' slots mapped back to the ancestors' beam indices (the
    pages' h_t).  ``widths``: W_j of every step j <= t (default W_t)."""
    widths = [W_t] * (t + 1) if widths is None else list(widths)
    sl = record_slots(store, t, W_t)
    rows = np.arange(store.R)[:, None]
    d = store.rec_delta[t].cpu().numpy()[rows, sl]
    k = store.rec_k[t].view(torch.int16).cpu().numpy().view(np.uint16)[rows, sl]
    a = store.rec_alpha[t].cpu().numpy()[rows, sl]
    anc = store.anc[t, :, :W_t, :t].cpu().numpy().astype(np.int64)
    for j in range(t):
        slj = record_slots(store, j, widths[j])
        inv = np.full((store.R, store.W_max), -1, np.int64)
        inv[rows, slj] = np.arange(widths[j])[None, :]
        anc[:, :, j] = inv[rows, anc[:, :, j]]
    return d, k, a, anc.astype(np.int32)
