"""The byte model against the capacity and write figures printed on the OneLA
page (§4.4, Figure 8b), and against its own definitions."""

import json
import os

import numpy as np
from linear_attention_beam_gdn_amd import accounting as A

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _matches_printed(x, printed, digits=3):
    """x rounds to ``printed`` at the page's 3 significant digits (halves up)."""
    ulp = 10.0 ** (np.floor(np.log10(abs(printed))) - digits + 1)
    return abs(x - printed) <= 0.5 * ulp + 1e-9


def test_fig8b_capacity_and_writes():
    g = json.load(open(os.path.join(GOLDEN, "onela_fig8b_state_bytes.json")))
    geo = g["geometry"]
    for row in g["printed"]:
        got = A.onela_fig8b(R=geo["R"], W=geo["W"], H=geo["H"], K=geo["K"], V=geo["V"],
                            O=row["O"], record_bytes_per_head=g["record_bytes_per_head"])
        assert _matches_printed(got["capacity_mib"], row["capacity_mib"]), got
        assert _matches_printed(got["writes_mib"], row["writes_mib"]), got
        assert _matches_printed(got["capacity_ratio"], row["capacity_reduction_vs_fullstate"]), got
        assert round(got["write_ratio"]) == row["write_reduction_vs_fullstate"]


def test_record_and_input_sizes():
    assert A.record_bytes(128, 128) == 772
    assert A.record_bytes(128, 128, channel_decay=True) == 1280
    assert A.input_bytes(128, 128) == 776
    assert A.input_bytes(128, 128, channel_decay=True) == 1284


def test_large_beam_step_bytes_per_beam_gather():
    # 8 requests x 512 beams, H = 32, d_k = d_v = 128, 4 steps
    tot = sum(A.beam_step_bytes(R=8, H=32, dk=128, dv=128, W_t=512, t=t) for t in range(4))
    anc = sum(4 * 8 * 512 * 2 * t for t in range(4))
    assert tot - anc == 4 * 286_785_536 + 6 * 101_187_584


def test_shared_key_heads_step_bytes():
    # the same beams with 32 value heads on 16 key heads: q, k and the record
    # key (4 d_k + 2 d_k bytes per beam, 2 d_k per ancestor) counted per key head
    kw = dict(R=8, H=32, dk=128, dv=128, W_t=512)
    tot = sum(A.beam_step_bytes(t=t, Hk=16, **kw) for t in range(4))
    anc = sum(4 * 8 * 512 * 2 * t for t in range(4))
    assert tot - anc == 4 * 236_453_888 + 6 * 84_410_368
    for t in range(4):
        assert A.beam_step_bytes(t=t, Hk=32, **kw) == A.beam_step_bytes(t=t, **kw)
        assert A.beam_step_bytes(t=t, Hk=32, channel_decay=True, **kw) == \
            A.beam_step_bytes(t=t, channel_decay=True, **kw)


def test_unique_ancestors():
    row = np.array([[0, 1], [0, 1], [0, 2], [3, 2]])
    assert A.unique_ancestors(row, 4) == 2 + 2
    assert A.unique_ancestors(row, 2) == 1 + 1


def test_bounded_log_run_bytes():
    # 128 sequences, H/d_k/d_v = 32/128/128, log capacity M = 8 (DeltaLog
    # Table 3), 64 tokens: 8 full cycles of log lengths 0..7.  A merge cycle
    # either merges separately (base read + written + 8 records read again)
    # or folds the log in the decode that fills it (base written; the fold
    # takes the records that decode already reads and appends).
    kw = dict(R=128, H=32, dk=128, dv=128)
    tokens = 8 * sum(A.sequence_token_bytes(log_len=j, **kw) for j in range(8))
    separate = tokens + 8 * A.merge_bytes(n_rec=8, **kw)
    fused = 8 * (sum(A.sequence_token_bytes(log_len=j, **kw) for j in range(7))
                 + A.decode_merge_bytes(log_len=7, **kw))
    assert separate == 22_925_541_376
    assert fused == 20_575_682_560
    # per cycle: one base read and the merge's second read of the 8 records
    assert separate - fused == 8 * 128 * 32 * (4 * 128 * 128 + 8 * A.record_bytes(128, 128, False, False))


def test_step_write_bytes_are_the_written_part():
    """Outputs (4 d_v), appended records (4A + 4 d_v per value head, 2 d_k per
    key head) and the step's ancestry rows are written; taking them from the
    total leaves the reads: S0, the inputs, the ancestral records and the
    ancestry read."""
    for ch, Hk in ((False, None), (True, None), (False, 8)):
        R, H, dk, dv, W, t, uniq = 3, 16, 128, 256, 40, 2, 57
        hk = H if Hk is None else Hk
        Ach = dk if ch else 1
        total = A.beam_step_bytes(R=R, H=H, dk=dk, dv=dv, W_t=W, t=t, channel_decay=ch, unique_records=uniq, Hk=Hk)
        writes = A.beam_step_write_bytes(R=R, H=H, dk=dk, dv=dv, W_t=W, t=t, channel_decay=ch, Hk=Hk)
        reads = (R * H * 4 * dk * dv + R * W * (H * (2 * dv + 4 * Ach + 4) + hk * 4 * dk)
                 + uniq * (H * (4 * Ach + 4 * dv) + hk * 2 * dk) + 4 * R * W * t)
        assert writes == R * W * (H * (4 * dv + 4 * Ach + 4 * dv) + hk * 2 * dk) + 4 * R * W * t
        assert total - writes == reads
