"""Split-replay bounded-log decoding through the C ABI
(gdn_decode_step_split; DeltaLog Figure 5 caption: shared replay
preparation, parallel append decode across value tiles, single-writer
metadata commit; Figure 9: the split-replay ablation), against the FP64
oracle: every rule, log capacities 4 and 8, one, two and four value tiles,
the preparation shared through a workspace or repeated in every tile."""

import numpy as np
import pytest
import torch

import oracle.gdn_oracle as O
from gpu_util import TOL, log, rel_slices, rel_states
from linear_attention_beam_gdn_amd import binding as B
from linear_attention_beam_gdn_amd import synth

pytestmark = pytest.mark.gpu

ARMS = [(n, shared) for n in (1, 2, 4) for shared in (False, True)]


@pytest.mark.parametrize("Hk", [None, 2])
@pytest.mark.parametrize("M", [4, 8])
@pytest.mark.parametrize("kind", ["scalar", "channel", "plain"])
def test_split_arms(kind, M, Hk):
    """Two full merge cycles and a ragged third (the log left part full), all
    six arms side by side: each matches the oracle's o_t, update vectors and
    merged bases; the shared and repeated arms of one tiling give the same
    bits; the update vectors of the plain rule are v_t's own bits."""
    channel, plain = kind != "scalar", kind == "plain"
    R, H, dk, dv = 5, 4, 128, 128
    T = 2 * M + 3
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=T, s0_std=0.05, seed=900 + M + (Hk or 0),
                                     channel_decay=channel, Hk=Hk)
    ref = O.sequence_decode(seq["S0"], seq["tokens"], M, rule="plain" if plain else "delta")
    S0 = torch.from_numpy(seq["S0"]).cuda()
    stores = {arm: B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain, S=S0.clone(), Hk=Hk)
              for arm in ARMS}
    ws = torch.empty(B.split_workspace_bytes(stores[ARMS[0]]) // 4, dtype=torch.float32, device="cuda")
    worst = 0.0
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        outs = {}
        for (n, shared), st in stores.items():
            outs[(n, shared)] = B.decode_step_split(st, t, n, shared, t == M - 1, *args,
                                                    workspace=ws if shared else None)
        torch.cuda.synchronize()
        for (n, shared), st in stores.items():
            o = outs[(n, shared)]
            e = rel_slices(o[:, 0].cpu().numpy().reshape(R * H, dv), ref["o"][i])
            worst = max(worst, e)
            assert e <= TOL, (kind, M, n, shared, i, "o", e)
            if plain:
                bits = st.rec_delta[t, :, 0].view(torch.int16).cpu().numpy().view(np.uint16)
                assert np.array_equal(bits, seq["tokens"]["v"][i]), (n, shared, i)
            else:
                e = rel_slices(st.rec_delta[t, :, 0].cpu().numpy().reshape(R * H, dv), ref["delta"][i])
                worst = max(worst, e)
                assert e <= TOL, (kind, M, n, shared, i, "delta", e)
            assert np.array_equal(st.rec_k[t, :, 0].view(torch.int16).cpu().numpy().view(np.uint16),
                                  seq["tokens"]["k"][i]), (n, shared, i, "record key")
            if t == M - 1:
                e = rel_states(st.S.cpu().numpy().reshape(R * H, 1, dk, dv), ref["bases"][i // M][:, None])
                worst = max(worst, e)
                assert e <= TOL, (kind, M, n, shared, i, "base", e)
            if shared:  # the two arms of one tiling: the same arithmetic, the same bits
                other = stores[(n, False)]
                assert torch.equal(o, outs[(n, False)]), (n, i)
                assert torch.equal(st.rec_delta, other.rec_delta), (n, i)
                assert torch.equal(st.S, other.S), (n, i)
    log(f"[split] {kind} M={M} Hk={Hk}: six arms, max rel err {worst:.2e}")


def test_split_one_tile_equals_unsplit():
    """One tile with the preparation repeated is the unsplit kernel: the same
    bits as gdn_beam_decode_step and gdn_decode_merge_step."""
    R, H, dk, dv, M = 3, 2, 128, 128, 4
    T = 2 * M
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=T, s0_std=0.05, seed=931)
    S0 = torch.from_numpy(seq["S0"]).cuda()
    a = B.Store(R, 1, H, dk, dv, M, S=S0.clone())
    b = B.Store(R, 1, H, dk, dv, M, S=S0.clone())
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        o1 = B.decode_step_split(a, t, 1, False, t == M - 1, *args)
        o2 = B.decode_merge_step(b, t, *args) if t == M - 1 else B.decode_step(b, t, 1, zero, *args)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), i
        assert torch.equal(a.S, b.S) and torch.equal(a.rec_delta, b.rec_delta), i
