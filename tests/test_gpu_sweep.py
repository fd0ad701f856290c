"""Seeded sweep of beam-decode geometries through the C ABI against the FP64
oracle: head dims (square and the wide operator-suite pairs), decay kind,
value heads sharing key heads, request count, ragged beam widths with
W_t < W_max, chain lengths past every fused kernel's limit, and parent
patterns.  Each case also materialises a few beams at the last step.

The cases are drawn once from a fixed seed, so the sweep is the same on every
run; a failure names its case.
"""

import numpy as np
import pytest
import torch

import oracle.gdn_oracle as O
from gpu_util import TOL, log, rel_slices, rel_states, run_beam, step_records
from linear_attention_beam_gdn_amd import binding as B
from linear_attention_beam_gdn_amd import synth

pytestmark = pytest.mark.gpu

SCALAR_DIMS = [(16, 16), (32, 32), (64, 64), (128, 128), (128, 256), (128, 512), (256, 128), (256, 256),
               (256, 512)]
CHANNEL_DIMS = [(16, 16), (32, 32), (64, 64), (128, 128), (128, 256), (128, 512)]


def _cases(n=60, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        channel = bool(rng.random() < 0.35)
        dims = CHANNEL_DIMS if channel else SCALAR_DIMS
        dk, dv = dims[rng.integers(len(dims))]
        big = dk * dv >= 128 * 256
        H = int(rng.choice([1, 2, 3, 4, 6] if not big else [1, 2]))
        Hk = int(rng.choice([d for d in range(1, H + 1) if H % d == 0]))
        R = int(rng.integers(1, 4 if not big else 3))
        L = int(rng.integers(1, 8))
        W_max = int(rng.choice([1, 5, 16, 17, 40, 70] if not big else [1, 5, 17, 24]))
        widths = [int(rng.integers(max(1, W_max // 2), W_max + 1)) for _ in range(L)]
        parents = str(rng.choice(["topk", "uniform"]))
        out.append(dict(id=i, channel=channel, dk=dk, dv=dv, H=H, Hk=Hk, R=R, L=L, W_max=W_max, widths=widths,
                        parents=parents, seed=900 + i))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"c{c['id']}" for c in CASES])
def test_random_geometry(case):
    c = case
    label = (f"case {c['id']}: dk={c['dk']} dv={c['dv']} ch={c['channel']} R={c['R']} H={c['H']} Hk={c['Hk']} "
             f"L={c['L']} W_max={c['W_max']} widths={c['widths']} parents={c['parents']}")
    log(f"[sweep] {label}")
    inp = synth.make_inputs(R=c["R"], H=c["H"], dk=c["dk"], dv=c["dv"], W=c["W_max"], L=c["L"], s0_std=0.1,
                            seed=c["seed"], parents=c["parents"], channel_decay=c["channel"], widths=c["widths"],
                            Hk=c["Hk"])
    store, outs = run_beam(inp, c["channel"], W_max=c["W_max"])
    ref = O.beam_decode(inp["S0"], inp["steps"])
    worst = 0.0
    for t, st in enumerate(inp["steps"]):
        W_t = st["q"].shape[1]
        d, kbits, a, anc = step_records(store, t, W_t)
        assert np.array_equal(anc, ref["anc"][t]), f"{label}: ancestry differs at t={t}"
        assert np.array_equal(kbits, st["k"]), f"{label}: record keys differ at t={t}"
        assert np.array_equal(a.reshape(st["alpha"].shape), st["alpha"]), f"{label}: decays differ at t={t}"
        eo, ed = rel_slices(outs[t], ref["o"][t]), rel_slices(d, ref["delta"][t])
        worst = max(worst, eo, ed)
        assert eo <= TOL and ed <= TOL, (label, t, eo, ed)
    t = c["L"] - 1
    W_t = c["widths"][t]
    pairs = np.array([[r, b] for r in range(c["R"]) for b in {0, W_t - 1}], np.int32)
    S = B.materialize(store, t, torch.from_numpy(pairs).cuda()).cpu().numpy()
    es = rel_states(S, O.beam_states(inp["S0"], inp["steps"], t, [tuple(p) for p in pairs]))
    assert es <= TOL, (label, "materialise", es)
    log(f"[sweep] case {c['id']}: max rel err {max(worst, es):.2e}")
