"""Seeded synthetic inputs for the GDN large-beam decode path.

This module only draws random numbers and encodes them in the storage formats
the path consumes (bf16 bit patterns, FP32, int32 parent pointers).  It holds
none of the method's arithmetic: no state update, no replay, no ancestry
recursion.  Both the HIP path and the CPU oracle are fed from the arrays it
returns, so the two sides see bit-identical inputs.

Recipe (the distributions follow the workload descriptions of the OneLA page,
§4.1, and of the DeltaLog page, Table 3):

* ``S0``: i.i.d. normal with the stated standard deviation, rounded to FP32.
* per step ``t`` the draws happen in this fixed order:
  q, k, v (standard normal), the alpha logit, the beta logit, then (t >= 1)
  the parent selection.
* q and k are L2-normalised over d_k in FP64, then rounded FP64 -> FP32 -> bf16
  (round-to-nearest-even at each step).  v is rounded the same way.  Nothing
  is renormalised afterwards, so |k| differs from 1 by at most about 2^-8.
* alpha = exp(-softplus(x)) and beta = sigmoid(x), computed in FP64, rounded
  to FP32.  With per-channel decay alpha has one value per d_k channel.
* parent pointers:
  - ``uniform``: pi_t(b) uniform over the previous step's beams;
  - ``topk``: every parent proposes E children scored parent_score + N(0,1);
    the W best survive (ties to the lower flat candidate index), the parent
    of a survivor is its flat index // E, and survivors are ordered by rank;
  - ``topk_hot``: ``topk``, then one hot parent per request and step is drawn
    and written over the parent of floor(frac * W) beams chosen without
    replacement (skewed ancestry with heavy fan-out).
  - ``zero``: W == 1 sequences (every step extends beam 0).
"""

from __future__ import annotations

import numpy as np

__all__ = ["bf16_bits", "bf16_bits_to_f32", "make_inputs", "make_sequence_inputs"]


def bf16_bits(x) -> np.ndarray:
    """Round to FP32 (RNE), then to bf16 (RNE); return the raw uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to FP32 (a storage-format decode)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _draw_token_inputs(rng, lead, dk, dv, channel_decay, Hk=None):
    """q, k, v, alpha, beta for a block of tokens with leading shape ``lead``
    (its last axis the value heads); q and k get ``Hk`` key heads instead
    when given."""
    lead_k = lead if Hk is None else lead[:-1] + (Hk,)
    q = bf16_bits(_unit_rows(rng.standard_normal(lead_k + (dk,))))
    k = bf16_bits(_unit_rows(rng.standard_normal(lead_k + (dk,))))
    v = bf16_bits(rng.standard_normal(lead + (dv,)))
    a_shape = lead + ((dk,) if channel_decay else ())
    alpha = np.exp(-_softplus(rng.standard_normal(a_shape))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal(lead)))).astype(np.float32)
    return q, k, v, alpha, beta


def _select_parents(rng, mode, R, W_prev, W, score, expand, hot_frac):
    """Parent pointers pi_t [R, W] and the survivors' cumulative scores."""
    if mode == "uniform":
        return rng.integers(0, W_prev, size=(R, W)).astype(np.int32), score
    if mode == "zero":
        return np.zeros((R, W), np.int32), score
    if mode not in ("topk", "topk_hot"):
        raise ValueError(f"unknown parent mode {mode!r}")
    cand = np.repeat(score, expand, axis=1) + rng.standard_normal((R, W_prev * expand))
    parent = np.empty((R, W), np.int32)
    new_score = np.empty((R, W), np.float64)
    for r in range(R):
        order = np.argsort(-cand[r], kind="stable")[:W]
        parent[r] = order // expand
        new_score[r] = cand[r, order]
    if mode == "topk_hot":
        n_hot = int(np.floor(hot_frac * W))
        for r in range(R):
            hot = rng.integers(0, W_prev)
            idx = rng.choice(W, size=n_hot, replace=False)
            parent[r, idx] = hot
    return parent, new_score


def make_inputs(*, R, H, dk, dv, W, L, s0_std, seed, parents="topk",
                channel_decay=False, expand=8, hot_frac=0.3, widths=None,
                alpha_const=None, beta_const=None, Hk=None):
    """Inputs for an L-step beam decode.

    Returns a dict with ``S0`` (FP32 [R,H,dk,dv]) and ``steps``: a list of L
    dicts holding ``q``, ``k`` (bf16 bits [R,W_t,H,dk]), ``v`` (bf16 bits
    [R,W_t,H,dv]), ``alpha`` (FP32 [R,W_t,H] or [R,W_t,H,dk]), ``beta`` (FP32
    [R,W_t,H]) and, for t >= 1, ``parent`` (int32 [R,W_t]).  ``widths`` gives a
    per-step beam width W_t (default: W at every step).  ``alpha_const`` and
    ``beta_const`` replace the drawn gates by constants (the draws still
    happen, so the other inputs are unchanged).  ``Hk`` (a divisor of H) gives
    q and k that many key heads, shared by H / Hk value heads each.
    """
    if Hk is not None and (Hk < 1 or H % Hk):
        raise ValueError("Hk must divide H")
    rng = np.random.default_rng(seed)
    widths = list(widths) if widths is not None else [W] * L
    if len(widths) != L:
        raise ValueError("widths must have L entries")
    S0 = (rng.standard_normal((R, H, dk, dv)) * s0_std).astype(np.float32)
    steps = []
    score = np.zeros((R, widths[0]), np.float64)
    for t in range(L):
        Wt = widths[t]
        q, k, v, alpha, beta = _draw_token_inputs(rng, (R, Wt, H), dk, dv, channel_decay, Hk)
        if alpha_const is not None:
            alpha = np.full_like(alpha, alpha_const)
        if beta_const is not None:
            beta = np.full_like(beta, beta_const)
        step = dict(q=q, k=k, v=v, alpha=alpha, beta=beta)
        if t >= 1:
            step["parent"], score = _select_parents(
                rng, parents, R, widths[t - 1], Wt, score, expand, hot_frac)
        steps.append(step)
    return dict(S0=S0, steps=steps)


def make_sequence_inputs(*, R, H, dk, dv, T, s0_std, seed, channel_decay=False, Hk=None):
    """Inputs for T tokens of R independent sequences (no beams).

    ``S0`` is the FP32 dense base [R,H,dk,dv]; ``tokens`` holds q, k, v, alpha,
    beta with a leading token axis: q/k [T,R,Hk,dk] (Hk = H by default),
    v [T,R,H,dv], ...
    """
    if Hk is not None and (Hk < 1 or H % Hk):
        raise ValueError("Hk must divide H")
    rng = np.random.default_rng(seed)
    S0 = (rng.standard_normal((R, H, dk, dv)) * s0_std).astype(np.float32)
    cols = {n: [] for n in ("q", "k", "v", "alpha", "beta")}
    for _ in range(T):
        q, k, v, alpha, beta = _draw_token_inputs(rng, (R, H), dk, dv, channel_decay, Hk)
        for n, a in zip(cols, (q, k, v, alpha, beta)):
            cols[n].append(a)
    return dict(S0=S0, tokens={n: np.stack(a) for n, a in cols.items()})
