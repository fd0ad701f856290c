"""The timed decode entry point (gdn_beam_decode_step_timed): the same bits as
gdn_beam_decode_step on every kernel family a decode step can dispatch, with
both events recorded by the runtime around the step's kernel."""

import numpy as np
import pytest
import torch

from gpu_util import log
from linear_attention_beam_gdn_amd import binding as B
from linear_attention_beam_gdn_amd import synth
from linear_attention_beam_gdn_amd.measure import stream as S

pytestmark = pytest.mark.gpu


def run(inp, channel, timed):
    """Every step of ``inp`` through the C ABI, timed or not; returns (store,
    [o_t], [us_t])."""
    S0 = inp["S0"]
    R, H, dk, dv = S0.shape
    widths = [st["q"].shape[1] for st in inp["steps"]]
    store = B.Store(R, max(widths), H, dk, dv, len(widths), channel_decay=channel,
                    S=torch.from_numpy(np.ascontiguousarray(S0)).cuda(), Hk=inp["steps"][0]["q"].shape[2])
    ev = S.KernelEvents(len(widths)) if timed else None
    try:
        outs = []
        for t, st in enumerate(inp["steps"]):
            d = B.upload(st)
            outs.append(B.decode_step(store, t, widths[t], d.get("parent"), d["q"], d["k"], d["v"], d["alpha"],
                                      d["beta"], events=ev.pairs[t] if timed else None))
        torch.cuda.synchronize()
        us = ev.elapsed_us() if timed else []
    finally:
        if ev is not None:
            ev.close()
    return store, [o.cpu().numpy() for o in outs], us


# (label, make_inputs arguments, channel decay, GDN_BEAM_GENERIC)
CASES = [
    ("scalar decay, fused kernel", dict(R=2, H=4, dk=128, dv=128, W=64, L=4), False, None),
    ("scalar decay, d_k = 256 x d_v = 512 value slices", dict(R=1, H=2, dk=256, dv=512, W=48, L=3), False, None),
    ("channel decay, two heads per workgroup", dict(R=16, H=32, dk=128, dv=128, W=16, L=3), True, None),
    ("channel decay, one head per workgroup", dict(R=2, H=2, dk=128, dv=128, W=40, L=3), True, None),
    ("scalar decay, general kernel", dict(R=2, H=2, dk=64, dv=64, W=40, L=3), False, "1"),
    ("sequences (one beam each), sequence kernel", dict(R=4, H=4, dk=128, dv=128, W=1, L=4), False, None),
]


@pytest.mark.parametrize("label,kw,channel,generic", CASES, ids=[c[0] for c in CASES])
def test_timed_step_same_bits(label, kw, channel, generic, monkeypatch):
    log(f"[timed] {label}: {kw}")
    if generic is not None:
        monkeypatch.setenv("GDN_BEAM_GENERIC", generic)
    inp = synth.make_inputs(s0_std=0.05, seed=11, parents="topk" if kw["W"] > 1 else "zero",
                            channel_decay=channel, **kw)
    st0, o0, _ = run(inp, channel, False)
    st1, o1, us = run(inp, channel, True)
    for t in range(len(o0)):
        assert np.array_equal(o0[t], o1[t]), (label, t)
    for name in ("rec_delta", "rec_k", "rec_alpha", "anc"):
        assert torch.equal(getattr(st0, name), getattr(st1, name)), (label, name)
    assert all(0.0 < x < 1e5 for x in us), (label, us)
    log(f"[timed] {label}: kernel us per step {[round(x, 1) for x in us]}")


def test_empty_kernel_timed_both_ways():
    """A near-empty launch as the runtime brackets it, and between event
    commands recorded around it: both positive and finite."""
    stream = torch.cuda.current_stream()
    k_us = S.empty_kernel_us(torch, stream, reps=5)
    e_us = S.empty_launch_us(torch, stream, reps=5)
    log(f"[timed] empty launch: {k_us:.2f} us bracketed by the runtime, {e_us:.2f} us between event commands")
    assert 0.0 < k_us < 1e4 and 0.0 < e_us < 1e4
