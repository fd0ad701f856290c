"""The allocation-free split-replay entry point (gdn_decode_step_split_noalloc,
for callers that cannot allocate device memory) against the workspace entry
point (gdn_decode_step_split) and the FP64 oracle, called through the C ABI:
two calls in a row on the same GPU, the second with a smaller input (fewer
sequences and heads), so the second reuses the built-in scratch buffer that
still holds the first call's contents."""

import numpy as np
import pytest
import torch

import oracle.gdn_oracle as O
from gpu_util import TOL, log, rel_slices, rel_states
from linear_attention_beam_gdn_amd import binding as B
from linear_attention_beam_gdn_amd import synth

pytestmark = pytest.mark.gpu


def _run(kind, R, H, M, n_split, seed):
    channel, plain = kind != "scalar", kind == "plain"
    dk = dv = 128
    T = M + 2
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=T, s0_std=0.05, seed=seed, channel_decay=channel)
    ref = O.sequence_decode(seq["S0"], seq["tokens"], M, rule="plain" if plain else "delta")
    S0 = torch.from_numpy(seq["S0"]).cuda()
    na = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain, S=S0.clone())
    ws_store = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain, S=S0.clone())
    ws = torch.empty(B.split_workspace_bytes(ws_store) // 4, dtype=torch.float32, device="cuda")
    o_na = torch.empty(R, 1, H, dv, dtype=torch.float32, device="cuda")
    worst = 0.0
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        B.decode_step_split_noalloc(na, t, n_split, True, t == M - 1, *args, o_na)
        o_ws = B.decode_step_split(ws_store, t, n_split, True, t == M - 1, *args, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws), (kind, R, H, i)
        assert torch.equal(na.rec_delta, ws_store.rec_delta) and torch.equal(na.rec_k, ws_store.rec_k), (kind, i)
        e = rel_slices(o_na[:, 0].cpu().numpy().reshape(R * H, dv), ref["o"][i])
        worst = max(worst, e)
        assert e <= TOL, (kind, R, H, i, e)
        if t == M - 1:
            assert torch.equal(na.S, ws_store.S), (kind, i)
            e = rel_states(na.S.cpu().numpy().reshape(R * H, 1, dk, dv), ref["bases"][i // M][:, None])
            worst = max(worst, e)
            assert e <= TOL, (kind, R, H, i, e)
    return worst


@pytest.mark.parametrize("kind", ["scalar", "channel", "plain"])
def test_noalloc_split_matches_workspace_entry_point(kind):
    w1 = _run(kind, R=8, H=16, M=4, n_split=4, seed=950)   # first call: 128 (sequence, head) pairs
    w2 = _run(kind, R=3, H=5, M=8, n_split=2, seed=951)    # second, smaller: 15 pairs, stale scratch beyond
    log(f"[no-alloc] {kind}: equal to the workspace entry point, max rel err {max(w1, w2):.2e}")


def test_noalloc_split_refuses_what_does_not_fit():
    # 7,183 (sequence, head) pairs need more than the 8 MiB scratch buffer
    st = B.Store(7183, 1, 1, 128, 128, 2)
    d = {n: torch.zeros(7183, 1, 1, 128, dtype=torch.bfloat16, device="cuda") for n in ("q", "k", "v")}
    a = torch.zeros(7183, 1, 1, dtype=torch.float32, device="cuda")
    o = torch.empty(7183, 1, 1, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(B.GdnError) as e:
        B.decode_step_split_noalloc(st, 0, 2, True, False, d["q"], d["k"], d["v"], a, a, o)
    assert e.value.status == B.GDN_ESCRATCH
