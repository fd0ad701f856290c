"""Algorithmic byte and FLOP counts for the GDN beam decode path.

These count what the method must move, not what a dense per-beam design
would move.  Per (beam, head) and step, with A = 1 for scalar decay and
A = d_k for channel decay:

* inputs  q, k (bf16), v (bf16), alpha (FP32 x A), beta (FP32):
          in  = 2 d_k + 2 d_k + 2 d_v + 4 A + 4
* output  o (FP32):                         out = 4 d_v
* record  (alpha FP32 x A, delta FP32 d_v, k bf16 d_k), appended once and
          read back by every descendant:   rec = 4 A + 4 d_v + 2 d_k
          (the plain rule, RWKV6, keeps its update vector v_t in bf16 and
          reads no beta: rec = 4 A + 2 d_v + 2 d_k, in = ... without the 4)
* shared state, read once per (request, head) per step: 4 d_k d_v.

Ancestor records read at step t are counted two ways:
* unique-record model: each distinct ancestor record of a request counted
  once (records are immutable and shared between beams), the minimum;
* per-beam-gather model: t records per beam.

The record layout (alpha, update vector, key) is the transition record of
OneLA §3.2; the capacity and write figures of OneLA §4.4 (Figure 8b) follow
from the same counting with the page's own record size (see ``onela_fig8b``).
"""

from __future__ import annotations

import numpy as np

MiB = float(1 << 20)


def record_bytes(dk, dv, channel_decay=False, plain=False):
    A = dk if (channel_decay or plain) else 1
    return 4 * A + (2 if plain else 4) * dv + 2 * dk


def input_bytes(dk, dv, channel_decay=False, plain=False):
    A = dk if (channel_decay or plain) else 1
    return 4 * dk + 2 * dv + 4 * A + (0 if plain else 4)


def output_bytes(dv):
    return 4 * dv


def unique_ancestors(anc_row, W_t):
    """Distinct ancestor slots per depth of one request's beams.

    anc_row: int array [W >= W_t, >= t]; returns the sum over depths j < t of
    the number of distinct anc_row[:W_t, j].
    """
    t = anc_row.shape[1]
    return int(sum(len(np.unique(anc_row[:W_t, j])) for j in range(t)))


def beam_step_bytes(*, R, H, dk, dv, W_t, t, channel_decay=False, unique_records=None, Hk=None):
    """Algorithmic bytes of one decode step (all requests and heads).

    ``unique_records``: total distinct ancestor records over requests (the
    unique-record model); ``None`` selects the per-beam-gather model.
    ``Hk``: key heads when value heads share them (q, k and the record key are
    stored once per key head); ``None`` means one key head per value head.
    """
    Hk = H if Hk is None else Hk
    A = dk if channel_decay else 1
    rec_v, rec_k = 4 * A + 4 * dv, 2 * dk  # record parts per value head / per key head
    per_beam = H * (2 * dv + 4 * A + 4 + output_bytes(dv) + rec_v) + Hk * (4 * dk + rec_k)
    chain = (R * W_t * t) if unique_records is None else unique_records
    # parent pointer + parent's t-1 indices read, own t indices written
    ancestry = 4 * R * W_t * 2 * t
    return R * H * 4 * dk * dv + R * W_t * per_beam + chain * (H * rec_v + Hk * rec_k) + ancestry


def beam_step_write_bytes(*, R, H, dk, dv, W_t, t, channel_decay=False, Hk=None):
    """The written part of ``beam_step_bytes``: outputs, appended records and
    the step's ancestry rows (the rest of a step's bytes are reads)."""
    Hk = H if Hk is None else Hk
    A = dk if channel_decay else 1
    return R * W_t * (H * (output_bytes(dv) + 4 * A + 4 * dv) + Hk * 2 * dk) + 4 * R * W_t * t


def beam_step_flops(*, R, H, dk, dv, W_t, t):
    """FLOPs of one step: 2 x (2 d_k d_v) for S0^T [q|k], 4 (d_k + d_v) per
    ancestor (two dot products, two axpys), and the current transition."""
    per = 4 * dk * dv + t * 4 * (dk + dv) + 2 * dk + 6 * dv
    return R * W_t * H * per


def sequence_token_bytes(*, R, H, dk, dv, log_len, channel_decay=False, plain=False):
    """One W = 1 decode token with ``log_len`` records in the log."""
    rec = record_bytes(dk, dv, channel_decay, plain)
    per = input_bytes(dk, dv, channel_decay, plain) + output_bytes(dv) + rec + log_len * rec
    return R * H * (4 * dk * dv + per)


def merge_bytes(*, R, H, dk, dv, n_rec, channel_decay=False, plain=False):
    """Fold n_rec records into the dense base: base read + written + records."""
    return R * H * (2 * 4 * dk * dv + n_rec * record_bytes(dk, dv, channel_decay, plain))


def decode_merge_bytes(*, R, H, dk, dv, log_len, channel_decay=False, plain=False):
    """The decode that fills the log with the merge in the same pass: the
    token's bytes (base read once, the log's log_len records read once, the
    new record appended) and the base written back.  The fold takes the same
    log_len records the replay reads, plus the record the step appends, so
    it moves no record a second time."""
    return (sequence_token_bytes(R=R, H=H, dk=dk, dv=dv, log_len=log_len, channel_decay=channel_decay, plain=plain)
            + R * H * 4 * dk * dv)


def onela_fig8b(*, R, W, H, K, V, O, record_bytes_per_head):
    """Capacity and write figures as OneLA §4.4 counts them.

    T = O - 1 decode calls; persistent capacity = one FP32 context state per
    request and head plus all T x W transition records; state writes = the
    records; FullState keeps (and rewrites at every call) a dense FP32 state
    per beam.  Returns MiB and ratios.
    """
    T = O - 1
    ctx = R * H * K * V * 4
    records = R * W * H * T * record_bytes_per_head
    full_capacity = R * W * H * K * V * 4
    full_writes = T * full_capacity
    return dict(
        capacity_mib=(ctx + records) / MiB,
        writes_mib=records / MiB,
        full_capacity_mib=full_capacity / MiB,
        capacity_ratio=full_capacity / (ctx + records),
        write_ratio=full_writes / records,
    )
