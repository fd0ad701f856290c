"""FP64 CPU oracle for the GDN large-beam decode path.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The HIP library never calls it, and it
imports nothing from the HIP side; both are fed the same seeded input arrays.

What it computes is the plain definition the two pages reach by other means:

* OneLA ("Scaling Linear-Attention Decoding to Large Beams in Generative
  Recommendation") states that projection replay reproduces the original GDN
  computation (§3.2) and that every beam's records are found through the
  ancestry index (§3.3).  So the reference result for beam b at step t is the
  eager dense GDN recurrence (§2.2 equation) applied from the shared
  post-prefill state to the beam's full chain of ancestral inputs, then to its
  own step-t inputs.
* DeltaLog ("Deferred Materialization of Recurrent States for Linear Attention
  Decoding") states that the model observes the same dense state as eager
  decoding (abstract).  So the reference for bounded-log decoding of
  independent sequences is eager token-by-token decoding, and the expected
  base after a merge is the eager state at that token.

Orientation.  OneLA writes S in R^{d_v x d_k} with o = S q.  Here every state
is stored as its transpose, an array [d_k, d_v], so the same recurrence reads
    S_t = alpha_t * S_{t-1} + k_t delta_t^T,
    delta_t = beta_t * (v_t - (alpha_t S_{t-1})^T k_t),      o_t = S_t^T q_t.
For per-channel decay (the KDA row of DeltaLog Table 1: transform
D(lambda_t) S_{t-1}, update pair (k_t, beta_t (v_t - k_t^T S_{t-1})), diagonal
decay), alpha_t is a d_k vector that scales the rows of S before the delta
correction.  The RWKV6 row of the same table keeps the diagonal decay but its
update pair is (k_t, v_t): no delta correction, so S_t = D(a_t) S_{t-1} +
k_t v_t^T, the record's update vector is v_t itself and beta is not used
(``rule="plain"`` below; the readout stays o_t = S_t^T q_t).

Key heads.  OneLA's operator suite (§4.1) pairs H_K key heads with H_V value
heads, H_V a multiple of H_K.  When q and k carry fewer heads than v, value
head h reads the q and k of key head h // (H_V / H_K); everything else stays
per value head, and each value head's recurrence is the one above.

Every array is converted to float64 exactly (bf16 bit patterns and FP32 values
widen without rounding) and all arithmetic is FP64.  Batching over beams uses
numpy broadcasting only; there is no blocking, fusion or reordering.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "decay", "transition", "readout", "ancestry",
    "beam_decode", "beam_states", "beam_decode_replay", "sequence_decode",
]


# --------------------------------------------------------------------------
# input decoding (storage formats -> float64, exact)
# --------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (the top 16 bits of an FP32)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _key_head(step, h):
    """Key head of value head h.  With H_K key heads and H_V = g H_K value
    heads (OneLA §4.1 geometries), value heads g*i .. g*i + g-1 share key
    head i: q and k carry H_K heads, everything else H_V."""
    H, Hk = step["v"].shape[2], step["q"].shape[2]
    return h // (H // Hk)


def _token(step, r, rows, h):
    """(q, k, v, alpha, beta) of request r, beam slots ``rows``, value head h."""
    hk = _key_head(step, h)
    q = bf16_to_f64(step["q"][r, rows, hk])
    k = bf16_to_f64(step["k"][r, rows, hk])
    v = bf16_to_f64(step["v"][r, rows, h])
    alpha = np.asarray(step["alpha"][r, rows, h], dtype=np.float64)
    beta = np.asarray(step["beta"][r, rows, h], dtype=np.float64)
    return q, k, v, alpha, beta


# --------------------------------------------------------------------------
# one eager transition (OneLA §2.2 equation; DeltaLog Table 1, GDN/KDA rows)
# --------------------------------------------------------------------------

def decay(S, alpha):
    """alpha * S for a scalar gate per state, diag(alpha) S for a d_k vector.

    S: [N, d_k, d_v]; alpha: [N] (scalar decay) or [N, d_k] (channel decay).
    """
    if alpha.ndim == 1:
        return alpha[:, None, None] * S
    return alpha[:, :, None] * S


def readout(S, x):
    """S^T x for each state: [N, d_k, d_v] x [N, d_k] -> [N, d_v]."""
    return np.matmul(x[:, None, :], S)[:, 0, :]


def transition(S, k, v, alpha, beta, rule="delta"):
    """One eager step on a batch of states; returns (S_t, delta_t).

    rule "delta" (GDN, KDA): the decayed state is corrected towards v along k,
    and the transition record's update vector is delta_t = beta_t (v_t -
    decayed^T k_t) (OneLA §3.2, GTR equation), so that S_t = decayed +
    k_t delta_t^T.  rule "plain" (RWKV6 row of DeltaLog Table 1): the update
    pair is (k_t, v_t), so delta_t = v_t and S_t = decayed + k_t v_t^T.
    """
    S_dec = decay(S, alpha)
    if rule == "plain":
        delta = np.array(v, dtype=np.float64, copy=True)
    elif rule == "delta":
        delta = beta[:, None] * (v - readout(S_dec, k))
    else:
        raise ValueError(rule)
    return S_dec + k[:, :, None] * delta[:, None, :], delta


# --------------------------------------------------------------------------
# ancestry index (OneLA §3.3 equation)
# --------------------------------------------------------------------------

def ancestry(parents, R, W0):
    """Physical slots of every beam's ancestors.

    ``parents[t]`` is the int array pi_t [R, W_t] for t >= 1 (``parents[0]`` is
    ignored; W0 is the beam count at step 0).  Returns ``anc`` with anc[t] an
    int64 array [R, W_t, t]: anc[t][r, b, j] = h_t(b, j), the slot written at
    step j by beam b's ancestor.  A child copies its parent's indices for the
    depths before t-1 and records the parent itself at depth t-1.
    """
    anc = [np.zeros((R, W0, 0), dtype=np.int64)]
    for t in range(1, len(parents)):
        pi = np.asarray(parents[t], dtype=np.int64)
        prev = anc[t - 1]
        Wt = pi.shape[1]
        row = np.empty((R, Wt, t), dtype=np.int64)
        for r in range(R):
            row[r, :, : t - 1] = prev[r, pi[r], :]
            row[r, :, t - 1] = pi[r]
        anc.append(row)
    return anc


def _anc_of(steps):
    R, W0 = steps[0]["q"].shape[:2]
    return ancestry([s.get("parent") for s in steps], R, W0)


# --------------------------------------------------------------------------
# eager dense decode of beams (the reference for o_t, delta_t and S_{t,b})
# --------------------------------------------------------------------------

def _eager_chain(S0, steps, anc, t, r, h, beams, rule="delta"):
    """Dense states and delta_t of ``beams`` of request r, head h after step t.

    Starts from the shared state S0[r, h] and applies, in order, the inputs of
    the ancestor at each depth j < t (slot anc[t][r, b, j] of step j), then the
    beam's own step-t inputs.
    """
    beams = np.asarray(beams, dtype=np.int64)
    S = np.repeat(S0[r, h][None].astype(np.float64), len(beams), axis=0)
    for j in range(t):
        slot = anc[t][r, beams, j]
        _, k, v, alpha, beta = _token(steps[j], r, slot, h)
        S, _ = transition(S, k, v, alpha, beta, rule)
    q, k, v, alpha, beta = _token(steps[t], r, beams, h)
    S, delta = transition(S, k, v, alpha, beta, rule)
    return S, delta, q


def beam_decode(S0, steps, *, requests=None, heads=None, rule="delta"):
    """Eager reference for every decode step.

    S0: FP32 [R, H, d_k, d_v]; steps: list of per-step input dicts (see the
    input generator).  Returns dict(anc=..., o=[...], delta=[...]) where o[t]
    and delta[t] are float64 [R, W_t, H, d_v]; entries of requests/heads not
    selected are NaN.
    """
    R, H, _, dv = S0.shape
    anc = _anc_of(steps)
    requests = range(R) if requests is None else requests
    heads = range(H) if heads is None else heads
    o_all, d_all = [], []
    for t, step in enumerate(steps):
        Wt = step["q"].shape[1]
        o = np.full((R, Wt, H, dv), np.nan)
        d = np.full((R, Wt, H, dv), np.nan)
        for r in requests:
            for h in heads:
                S, delta, q = _eager_chain(S0, steps, anc, t, r, h, np.arange(Wt), rule)
                o[r, :, h] = readout(S, q)
                d[r, :, h] = delta
        o_all.append(o)
        d_all.append(d)
    return dict(anc=anc, o=o_all, delta=d_all)


def beam_states(S0, steps, t, pairs, *, heads=None, rule="delta"):
    """Dense states S_{t,b} [n, H, d_k, d_v] (float64) for (r, b) ``pairs``."""
    R, H, dk, dv = S0.shape
    anc = _anc_of(steps)
    heads = range(H) if heads is None else heads
    out = np.full((len(pairs), H, dk, dv), np.nan)
    for i, (r, b) in enumerate(pairs):
        for h in heads:
            S, _, _ = _eager_chain(S0, steps, anc, t, r, h, [b], rule)
            out[i, h] = S[0]
    return out


# --------------------------------------------------------------------------
# FP64 projection replay (OneLA §3.2 replay equations), used to check that
# replay and eager agree; KDA: the decay moves onto the d_k-side probe
# --------------------------------------------------------------------------

def beam_decode_replay(S0, steps, *, requests=None, heads=None, rule="delta"):
    """Projection replay over records (alpha_j, delta_j, k_j), in FP64.

    Scalar decay follows OneLA's recursion: u^(-1) = S_ctx^T x,
    u^(j) = alpha_j u^(j-1) + delta_j (k_j . x) for 0 <= j < t, then
    delta_t = beta_t (v_t - alpha_t u_k^(t-1)), o_t = alpha_t u_q^(t-1) +
    delta_t (k_t . q_t).  Channel decay unrolls S_j^T y = S_{j-1}^T (a_j * y) +
    delta_j (k_j . y) from the current step down to S_ctx.  Records are the
    replay's own deltas of earlier steps.  With the plain rule the update
    vector is v_t itself (no projection of k_t is needed).
    """
    R, H, _, dv = S0.shape
    anc = _anc_of(steps)
    requests = range(R) if requests is None else requests
    heads = range(H) if heads is None else heads
    o_all, d_all = [], []
    for t, step in enumerate(steps):
        Wt = step["q"].shape[1]
        o = np.full((R, Wt, H, dv), np.nan)
        d = np.full((R, Wt, H, dv), np.nan)
        for r in requests:
            for h in heads:
                S_ctx = S0[r, h].astype(np.float64)
                q, k, v, alpha, beta = _token(step, r, np.arange(Wt), h)
                chain = []
                for j in range(t):
                    slot = anc[t][r, :, j]
                    _, k_j, _, a_j, _ = _token(steps[j], r, slot, h)
                    chain.append((a_j, d_all[j][r, slot, h], k_j))
                if alpha.ndim == 1:
                    u_q, u_k = q @ S_ctx, k @ S_ctx
                    for a_j, delta_j, k_j in chain:
                        u_q = a_j[:, None] * u_q + delta_j * np.sum(k_j * q, 1)[:, None]
                        u_k = a_j[:, None] * u_k + delta_j * np.sum(k_j * k, 1)[:, None]
                    delta = v if rule == "plain" else beta[:, None] * (v - alpha[:, None] * u_k)
                    o_t = alpha[:, None] * u_q + delta * np.sum(k * q, 1)[:, None]
                else:
                    def project(x):
                        y = alpha * x
                        acc = np.zeros((Wt, dv))
                        for a_j, delta_j, k_j in reversed(chain):
                            acc += delta_j * np.sum(k_j * y, 1)[:, None]
                            y = a_j * y
                        return acc + y @ S_ctx
                    delta = v if rule == "plain" else beta[:, None] * (v - project(k))
                    o_t = project(q) + delta * np.sum(k * q, 1)[:, None]
                o[r, :, h] = o_t
                d[r, :, h] = delta
        o_all.append(o)
        d_all.append(d)
    return dict(anc=anc, o=o_all, delta=d_all)


# --------------------------------------------------------------------------
# independent sequences, token by token (DeltaLog reference)
# --------------------------------------------------------------------------

def sequence_decode(S0, tokens, merge_every, *, pairs=None, rule="delta"):
    """Eager decoding of independent sequences.

    S0: FP32 [R, H, d_k, d_v]; tokens: dict of arrays with a leading token axis
    (q/k [T, R, H, d_k], v [T, R, H, d_v], alpha [T, R, H] or [T, R, H, d_k],
    beta [T, R, H]).  ``pairs`` restricts to (r, h) pairs (default: all).
    Returns dict(pairs, o [T, n, d_v], delta [T, n, d_v], bases [T // M, n,
    d_k, d_v]) where bases[m] is the dense state after token (m + 1) * M - 1,
    i.e. what the base must hold once the m-th full log has been merged.
    """
    R, H, _, _ = S0.shape
    if pairs is None:
        pairs = [(r, h) for r in range(R) for h in range(H)]
    rs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    hks = hs // (tokens["v"].shape[2] // tokens["q"].shape[2])  # key head of each value head
    S = S0[rs, hs].astype(np.float64)
    T = tokens["q"].shape[0]
    o, d, bases = [], [], []
    for i in range(T):
        q = bf16_to_f64(tokens["q"][i][rs, hks])
        k = bf16_to_f64(tokens["k"][i][rs, hks])
        v = bf16_to_f64(tokens["v"][i][rs, hs])
        alpha = np.asarray(tokens["alpha"][i][rs, hs], dtype=np.float64)
        beta = np.asarray(tokens["beta"][i][rs, hs], dtype=np.float64)
        S, delta = transition(S, k, v, alpha, beta, rule)
        o.append(readout(S, q))
        d.append(delta)
        if (i + 1) % merge_every == 0:
            bases.append(S.copy())
    return dict(pairs=pairs, o=np.stack(o), delta=np.stack(d),
                bases=np.stack(bases) if bases else np.zeros((0,) + S.shape))
