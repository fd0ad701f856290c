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
    _check_geometry(case)


@pytest.mark.parametrize("case", CASES[:40], ids=[f"c{c['id']}" for c in CASES[:40]])
def test_random_geometry_one_chunk(case, monkeypatch):
    """The same cases with every (request, head) in one beam chunk
    (GDN_BEAM_CHUNK=512), so that the fused kernels order the beams
    depth-first with the counting sort instead of taking chunk order."""
    monkeypatch.setenv("GDN_BEAM_CHUNK", "512")
    _check_geometry(case)


def _wide_chain_cases(n=48, seed=77):
    """Cases weighted to the fused kernels' shape-dependent paths: channel
    decay at d_v 256 / 512 (256-row value slices up to three records, 128-row
    beyond), d_k 256 and d = 128 scalar chains up to six records (how many
    record depths' keys the tile buffers stage), ragged widths, and one or
    several beam chunks per (request, head)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = rng.integers(3)
        if kind == 0:
            channel, (dk, dv) = True, [(128, 256), (128, 512)][rng.integers(2)]
        elif kind == 1:
            channel, (dk, dv) = False, [(256, 128), (256, 256), (256, 512)][rng.integers(3)]
        else:
            channel, (dk, dv) = False, [(128, 128), (64, 64), (128, 512)][rng.integers(3)]
        H = int(rng.choice([1, 2, 3]))
        Hk = int(rng.choice([d for d in range(1, H + 1) if H % d == 0]))
        L = int(rng.integers(2, 8))
        W_max = int(rng.choice([5, 17, 40, 70, 130, 300]))
        widths = [int(rng.integers(max(1, W_max // 2), W_max + 1)) for _ in range(L)]
        out.append(dict(id=1000 + i, channel=channel, dk=dk, dv=dv, H=H, Hk=Hk, R=int(rng.integers(1, 3)), L=L,
                        W_max=W_max, widths=widths, parents=str(rng.choice(["topk", "uniform"])), seed=5000 + i,
                        one_chunk=bool(rng.random() < 0.5)))
    return out


WIDE_CHAIN_CASES = _wide_chain_cases()


@pytest.mark.parametrize("case", WIDE_CHAIN_CASES, ids=[f"w{c['id']}" for c in WIDE_CHAIN_CASES])
def test_random_wide_and_long_chains(case, monkeypatch):
    if case["one_chunk"]:
        monkeypatch.setenv("GDN_BEAM_CHUNK", "512")
    _check_geometry(case)


def _check_geometry(case):
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
        d, kbits, a, anc = step_records(store, t, W_t, [s_["q"].shape[1] for s_ in inp["steps"][:t + 1]])
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


def _seq_cases(n=30, seed=4048, m_range=(1, 9), long_logs=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = str(rng.choice(["scalar", "channel", "plain"]))
        square = [(16, 16), (32, 32), (64, 64), (128, 128)]
        wide = [(128, 256), (128, 512), (256, 256)] if kind == "scalar" else ([(128, 256)] if kind == "channel" else [])
        dims = square + wide
        dk, dv = dims[rng.integers(len(dims))]
        fused = (dk, dv) in square and bool(rng.random() < 0.6)  # the merge in the decode: square shapes
        H = int(rng.choice([1, 2, 3, 4, 6]))
        Hk = int(rng.choice([d for d in range(1, H + 1) if H % d == 0]))
        if not long_logs:
            out.append(dict(id=i, kind=kind, dk=dk, dv=dv, H=H, Hk=Hk, R=int(rng.integers(1, 6)),
                            T=int(rng.integers(1, 21)), M=int(rng.integers(*m_range)), fused=fused, seed=1900 + i))
        else:
            M = int(rng.integers(*m_range))
            out.append(dict(id=i, kind=kind, dk=dk, dv=dv, H=H, Hk=Hk, R=int(rng.integers(1, 4)),
                            T=int(rng.integers(M, 2 * M + 4)), M=M, fused=fused, seed=2900 + i))
    return out


SEQ_CASES = _seq_cases()
# long logs (capacity 9 .. 16, the largest a store holds): one or two merges
# per case, every log length up to M - 1
SEQ_LONG_CASES = _seq_cases(n=16, seed=5150, m_range=(9, 17), long_logs=True)


@pytest.mark.parametrize("case", SEQ_CASES, ids=[f"s{c['id']}" for c in SEQ_CASES])
def test_random_sequences(case):
    """Bounded-log decoding of independent sequences over a seeded sweep: log
    capacity M, token count, decay kind and update rule, key heads, and the
    merge either fused into the decode that fills the log or run separately."""
    _check_sequences(case)


@pytest.mark.parametrize("case", SEQ_LONG_CASES, ids=[f"l{c['id']}" for c in SEQ_LONG_CASES])
def test_random_sequences_long_logs(case):
    """The same sweep with long logs (capacity 9 .. 16)."""
    _check_sequences(case)


def _check_sequences(c):
    channel, plain = c["kind"] != "scalar", c["kind"] == "plain"
    R, H, dk, dv, T, M = c["R"], c["H"], c["dk"], c["dv"], c["T"], c["M"]
    label = f"seq case {c['id']}: {c['kind']} dk={dk} dv={dv} R={R} H={H} Hk={c['Hk']} T={T} M={M} fused={c['fused']}"
    log(f"[sweep] {label}")
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=T, s0_std=0.1, seed=c["seed"], channel_decay=channel,
                                     Hk=c["Hk"])
    ref = O.sequence_decode(seq["S0"], seq["tokens"], M, rule="plain" if plain else "delta")
    store = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain,
                    S=torch.from_numpy(seq["S0"]).cuda(), Hk=c["Hk"])
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    worst = 0.0
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        if t == M - 1 and c["fused"]:
            o = B.decode_merge_step(store, t, *args)
        else:
            o = B.decode_step(store, t, 1, zero, *args)
            if t == M - 1:
                B.log_merge(store, M, 0)
        e = rel_slices(o[:, 0].cpu().numpy().reshape(R * H, dv), ref["o"][i])
        worst = max(worst, e)
        assert e <= TOL, (label, i, e)
        if plain:  # the bf16 log keeps v_t's own bits
            bits = store.rec_delta[t, :, 0].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(bits, seq["tokens"]["v"][i]), (label, "log bits", i)
        else:
            e = rel_slices(store.rec_delta[t, :, 0].cpu().numpy().reshape(R * H, dv), ref["delta"][i])
            worst = max(worst, e)
            assert e <= TOL, (label, "delta", i, e)
        if t == M - 1:
            e = rel_states(store.S.cpu().numpy().reshape(R * H, 1, dk, dv), ref["bases"][i // M][:, None])
            worst = max(worst, e)
            assert e <= TOL, (label, "base after merge", i, e)
    log(f"[sweep] seq case {c['id']}: max rel err {worst:.2e}")
