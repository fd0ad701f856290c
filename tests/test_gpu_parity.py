"""Parity of the HIP path, called through the C ABI, with the FP64 oracle.

Bars: ancestry, record keys and decays bit-exact; o_t, delta_t, materialised
and merged states within 1e-4 max relative error per slice (infinity norm of
the difference over the infinity norm of the oracle's slice).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle.gdn_oracle as O
from gpu_util import TOL, log, rel_slices, rel_states, run_beam, step_records
from linear_attention_beam_gdn_amd import binding as B
from linear_attention_beam_gdn_amd import configs, synth

GDN_MAX = B.GDN_MAX_STEPS  # longest log a store holds

pytestmark = pytest.mark.gpu


def check_beam(inp, channel, requests=None, heads=None, label="", **run_kw):
    log(f"[parity] {label} R,H,dk,dv={inp['S0'].shape} W={[s['q'].shape[1] for s in inp['steps']]}")
    store, outs = run_beam(inp, channel, **run_kw)
    ref = O.beam_decode(inp["S0"], inp["steps"], requests=requests, heads=heads)
    worst = 0.0
    for t, st in enumerate(inp["steps"]):
        W_t = st["q"].shape[1]
        d, kbits, a, anc = step_records(store, t, W_t, [s_["q"].shape[1] for s_ in inp["steps"][:t + 1]])
        assert np.array_equal(anc, ref["anc"][t]), f"{label}: ancestry differs at t={t}"
        assert np.array_equal(kbits, st["k"]), f"{label}: record keys differ at t={t}"
        assert np.array_equal(a.reshape(st["alpha"].shape), st["alpha"]), f"{label}: decays t={t}"
        eo = rel_slices(outs[t], ref["o"][t])
        ed = rel_slices(d, ref["delta"][t])
        worst = max(worst, eo, ed)
        assert eo <= TOL and ed <= TOL, (label, t, eo, ed)
    log(f"[parity] {label}: max rel err {worst:.2e}")
    return store, outs, ref


# ----------------------------------------------------------- the five workloads

def test_tiny_workload():
    check_beam(configs.TINY.inputs(), False, label="tiny")


def test_single_request_workload():
    check_beam(configs.SINGLE.inputs(), False, label="single-request")


def _full_beam(w, channel, tmp_path, **over):
    """Workload ``w`` at full size: ancestry, record keys and decays bit-exact
    for every beam here, then o_t and delta_t of every (request, head) pair
    against the FP64 eager oracle in a child process (full_parity)."""
    import full_parity

    if over:
        w = dataclasses.replace(w, **over)
    inp = w.inputs()
    log(f"[parity] full size {w.name}: R={w.R} W={w.W} H={w.H} dk={w.dk} dv={w.dv} L={w.L}, every pair")
    store, outs = run_beam(inp, channel)
    steps = inp["steps"]
    anc = O.ancestry([st.get("parent") for st in steps], w.R, steps[0]["q"].shape[1])
    for t, st in enumerate(steps):
        d, kbits, a, anc_t = step_records(store, t, w.W)
        assert np.array_equal(anc_t, anc[t]), f"{w.name}: ancestry differs at t={t}"
        assert np.array_equal(kbits, st["k"]), f"{w.name}: record keys differ at t={t}"
        assert np.array_equal(a.reshape(st["alpha"].shape), st["alpha"]), f"{w.name}: decays differ at t={t}"
        np.save(tmp_path / f"o_{t}.npy", outs[t])
        np.save(tmp_path / f"d_{t}.npy", d)
    del store, outs
    res = full_parity.run("beam", w.name, str(tmp_path), over=over or None)
    log(f"[parity] full size {w.name}: {res['pairs']} pairs, worst {res['worst']}, {res['seconds']:.0f} s "
        f"on {res['workers']} host workers")
    for k, v in res["worst"].items():
        assert v["rel_err"] <= TOL, (w.name, k, v)


@pytest.mark.parametrize("wname,channel", [("LARGE", False), ("KDA", True), ("SHARED_KEYS", False)])
def test_full_size_workload_every_pair(wname, channel, tmp_path):
    """The large-beam (8 x 512 beams, 30 % hot parent) and channel-decay
    (16 x 256 beams) workloads, and the shared-key-head variant, compared in
    full: every beam, head and step."""
    _full_beam(getattr(configs, wname), channel, tmp_path)


def test_kda_two_heads_per_workgroup_same_bits(monkeypatch):
    """The channel-decay workload at full size (16 x 256 beams, H = 32: two
    rounds of workgroups, so the launch takes two heads per workgroup) gives
    the same bits as one head per workgroup (GDN_BEAM_PAIR=0): outputs,
    update vectors, keys, decays and ancestry of every step."""
    inp = configs.KDA.inputs()
    log("[parity] kda_channel_decay_beam: two heads per workgroup against one, every step")
    store2, outs2 = run_beam(inp, True)
    monkeypatch.setenv("GDN_BEAM_PAIR", "0")
    store1, outs1 = run_beam(inp, True)
    for t in range(len(outs1)):
        assert np.array_equal(outs1[t], outs2[t]), t
    for name in ("rec_delta", "rec_k", "rec_alpha", "anc"):
        assert torch.equal(getattr(store1, name), getattr(store2, name)), name


def test_large_beam_workload_sampled():
    # full size, eager oracle on a sample (kept beside the full comparison)
    check_beam(configs.LARGE.inputs(), False, requests=[0, 5], heads=[0, 13, 31],
               label="large-beam")


def test_shared_key_heads_workload_sampled():
    # full size, 32 value heads on 16 key heads; heads 0, 1 share key head 0
    check_beam(configs.SHARED_KEYS.inputs(), False, requests=[0, 7], heads=[0, 1, 17, 30],
               label="large-beam shared key heads")


def test_wide_state_workload_sampled():
    # full size, d_k = 256, d_v = 512 (four value slices per (request, head))
    check_beam(configs.WIDE.inputs(), False, requests=[3], heads=[0, 15], label="wide state")


def test_kda_wide_value_workload_sampled():
    # full size, channel decay with d_v = 512 (four value slices)
    check_beam(configs.KDA_WIDE.inputs(), True, requests=[2], heads=[0, 15], label="kda wide value")


@pytest.mark.parametrize("wname,requests,heads", [("QWEN_R4", [1], [0, 15]), ("QWEN_R16", [11], [7])])
def test_qwen_geometry_workloads_sampled(wname, requests, heads):
    # full size, six decode steps (chains of up to five records in the fused kernel)
    w = getattr(configs, wname)
    check_beam(w.inputs(), False, requests=requests, heads=heads, label=w.name)


@pytest.mark.parametrize("H,Hk,dv,R,W,channel", [(64, 4, 128, 4, 256, False), (64, 16, 256, 2, 128, False),
                                                 (64, 8, 128, 2, 256, True)])
def test_many_value_heads_sampled(H, Hk, dv, R, W, channel):
    # the OneLA operator suite's largest head counts: 64 value heads on 4 to 16
    # key heads (16 down to 4 value heads per key head), hot-parent lineage
    inp = synth.make_inputs(R=R, H=H, dk=128, dv=dv, W=W, L=4, s0_std=0.05, seed=31 + Hk, parents="topk_hot",
                            channel_decay=channel, Hk=Hk)
    g = H // Hk
    heads = [0, g - 1, g, H - 1]  # two value heads of key head 0, the first of key head 1, the last
    check_beam(inp, channel, requests=[R - 1], heads=heads, label=f"H = {H} on H_k = {Hk}, d_v = {dv}")


@pytest.mark.parametrize("dk,dv,pair", [(64, 64, "1"), (128, 256, "1"), (128, 256, "0")])
def test_channel_decay_two_rounds_of_heads(dk, dv, pair, monkeypatch):
    # 16 x 32 (request, head) pairs in one value slice: a grid of two rounds,
    # which the launch folds into two heads per workgroup at d_v = 64 (pair
    # "1"); at d_v = 256 (two row blocks per consumer wave) it keeps one head
    # per workgroup either way.  Both heads of a workgroup pair are checked.
    monkeypatch.setenv("GDN_BEAM_PAIR", pair)
    inp = synth.make_inputs(R=16, H=32, dk=dk, dv=dv, W=48, L=4, s0_std=0.05, seed=57, parents="topk",
                            channel_decay=True)
    check_beam(inp, True, requests=[0, 15], heads=[0, 1, 30, 31], label=f"channel decay {dk} x {dv}, pair={pair}")


@pytest.mark.parametrize("dk,dv,channel", [(128, 256, False), (256, 128, False), (256, 256, False),
                                            (128, 512, True)])
def test_grids_of_several_rounds(dk, dv, channel):
    # 16 x 32 (request, head) pairs: every value slice of every head in a grid
    # of two rounds or more on the 256 compute units (the XCD-grouped
    # workgroup order, slices and store windows at that size); the first and
    # last heads of the first and last requests are checked
    inp = synth.make_inputs(R=16, H=32, dk=dk, dv=dv, W=40, L=4, s0_std=0.05, seed=59 + dk + dv, parents="topk",
                            channel_decay=channel)
    check_beam(inp, channel, requests=[0, 15], heads=[0, 1, 30, 31], label=f"{dk} x {dv}, 16 x 32 heads")


@pytest.mark.parametrize("wname,channel,requests,heads", [("LARGE", False, [6], [0, 29]),
                                                           ("WIDE", False, [2], [11]),
                                                           ("KDA", True, [9], [4])])
def test_long_chain_workloads_sampled(wname, channel, requests, heads):
    # full size, seven decode steps (t = 0 .. 6), as the long-chain bench rows
    # time them: at t = 6 the d = 128 kernel stages five of the six record
    # depths' keys and its dot wave gathers the sixth; d_k = 256 stages two
    # at t = 3, 4 and three from t = 5; channel decay runs its ring at three
    # buffers from t = 5
    w = dataclasses.replace(getattr(configs, wname), L=7)
    check_beam(w.inputs(), channel, requests=requests, heads=heads, label=f"{w.name} L = 7")


def _full_sequences(w, fused, tmp_path, split=None):
    """Bounded-log decoding of workload ``w`` at full size, every token's o_t
    and appended update vector and every merged base, for every (sequence,
    head) pair against the FP64 eager oracle in a child process
    (full_parity).  ``split`` = (n_split, shared_prep) runs every token
    through gdn_decode_step_split instead (merge fused into the token that
    fills the log)."""
    import full_parity

    seq = w.inputs()
    log(f"[parity] {w.name} R={w.R} H={w.H} T={w.T} M={w.M} fused merge={fused} split={split}, every pair")
    store = B.Store(w.R, 1, w.H, w.dk, w.dv, w.M, channel_decay=w.channel_decay, plain_update=w.plain_update,
                    S=torch.from_numpy(seq["S0"]).cuda())
    ws = None
    if split is not None and split[1]:
        ws = torch.empty(B.split_workspace_bytes(store) // 4, dtype=torch.float32, device="cuda")
    zero = torch.zeros(w.R, 1, dtype=torch.int32, device="cuda")
    o_all = np.empty((w.T, w.R, w.H, w.dv), np.float32)
    d_all = np.empty_like(o_all)
    for i in range(w.T):
        t = i % w.M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        if split is not None:
            o = B.decode_step_split(store, t, split[0], split[1], t == w.M - 1, *args, workspace=ws)
        elif fused and t == w.M - 1:
            o = B.decode_merge_step(store, t, *args)
        else:
            o = B.decode_step(store, t, 1, zero, *args)
        o_all[i] = o[:, 0].cpu().numpy()
        d_all[i] = store.rec_delta[t, :, 0].float().cpu().numpy()
        if w.plain_update:  # the bf16 log holds v_t's own bits (DeltaLog Table 3, RWKV6 row)
            bits = store.rec_delta[t, :, 0].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(bits, seq["tokens"]["v"][i]), i
        if t == w.M - 1:
            if not fused and split is None:
                B.log_merge(store, w.M, 0)
            np.save(tmp_path / f"S_{i // w.M}.npy", store.S.cpu().numpy())
    np.save(tmp_path / "o.npy", o_all)
    np.save(tmp_path / "d.npy", d_all)
    del store, o_all, d_all
    res = full_parity.run("seq", w.name, str(tmp_path), over={"M": w.M})
    log(f"[parity] {w.name} fused={fused} split={split}: {res['pairs']} pairs, worst {res['worst']}, "
        f"{res['seconds']:.0f} s on {res['workers']} host workers")
    for k, v in res["worst"].items():
        assert v["rel_err"] <= TOL, (w.name, k, v)


@pytest.mark.parametrize("wname,fused", [("DELTALOG", False), ("DELTALOG", True), ("RWKV6", True),
                                         ("KDA_LOG", True)])
def test_deltalog_workload_every_pair(wname, fused, tmp_path):
    """Bounded-log decoding at full size (128 sequences x 32 heads, 64
    tokens), every pair: the GDN log (M = 8) with separate and fused merges,
    and the RWKV6 and KDA logs (M = 4, DeltaLog Table 3)."""
    _full_sequences(getattr(configs, wname), fused, tmp_path)


@pytest.mark.parametrize("wname,M,split", [("DELTALOG", 8, (4, True)), ("DELTALOG", 4, (2, False)),
                                           ("KDA_LOG", 4, (2, True)), ("KDA_LOG", 8, (4, False)),
                                           ("RWKV6", 4, (4, True)), ("RWKV6", 8, (2, False))])
def test_split_replay_workload_every_pair(wname, M, split, tmp_path):
    """The split-replay path (value tiles; preparation shared through the
    workspace or repeated per tile) at full size, every pair, for the three
    rules at log capacities 4 and 8 (DeltaLog Figure 9)."""
    _full_sequences(dataclasses.replace(getattr(configs, wname), M=M), True, tmp_path, split=split)


# ------------------------------------------------- shapes: tiles, ragged tails

@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("dims", [(16, 16), (32, 32), (64, 64), (128, 128)])
def test_ragged_widths(dims, channel):
    dk, dv = dims
    inp = synth.make_inputs(R=3, H=3, dk=dk, dv=dv, W=37, L=4, s0_std=0.1, seed=100 + dk,
                            parents="topk", channel_decay=channel, widths=[37, 29, 37, 20])
    check_beam(inp, channel, label=f"ragged dk={dk} ch={channel}")


@pytest.mark.parametrize("dims,channel", [((32, 32), False), ((64, 64), False), ((128, 128), False),
                                          ((64, 64), True), ((128, 128), True), ((128, 512), True)])
def test_chains_up_to_six_records(dims, channel):
    """Steps t = 5, 6 (the longest chains of the OneLA operator suite, T = 6)
    on the fused kernels (scalar and channel decay; at channel decay the
    chain of six records takes S0 from HBM, not LDS), with ragged widths."""
    dk, dv = dims
    inp = synth.make_inputs(R=2, H=2, dk=dk, dv=dv, W=37, L=7, s0_std=0.1, seed=200 + dk + dv // 64,
                            parents="topk", widths=[37, 29, 37, 20, 33, 37, 17], channel_decay=channel)
    check_beam(inp, channel, label=f"L=7 dk={dk} dv={dv} ch={channel}")


def test_channel_decay_long_chains_one_chunk(monkeypatch):
    monkeypatch.setenv("GDN_BEAM_CHUNK", "512")
    inp = synth.make_inputs(R=2, H=2, dk=128, dv=128, W=40, L=7, s0_std=0.1, seed=240, parents="topk_hot",
                            channel_decay=True)
    check_beam(inp, True, label="channel decay L=7 one chunk")


@pytest.mark.parametrize("channel", [False, True])
def test_beams_wider_than_one_workgroup(channel):
    """W = 1030 beams: each (request, head) is split over several workgroups
    (chunk order instead of the depth-first schedule, chunk offsets in every
    store window), with a ragged last chunk."""
    inp = synth.make_inputs(R=1, H=2, dk=64, dv=64, W=1030, L=3, s0_std=0.1, seed=300,
                            parents="topk", channel_decay=channel)
    check_beam(inp, channel, label=f"W=1030 ch={channel}")


@pytest.mark.parametrize("dims,channel,Hk", [((16, 16), False, 2), ((64, 64), False, 2), ((128, 128), False, 1),
                                             ((64, 64), True, 2), ((128, 128), True, 1), ((32, 32), True, 2)])
def test_value_heads_sharing_key_heads(dims, channel, Hk):
    """H = 4 value heads on Hk key heads (OneLA §4.1 geometries): the general
    (d = 16), scalar-decay and channel-decay kernels read each value head's
    key head, and the record keys are written once per key head."""
    dk, dv = dims
    inp = synth.make_inputs(R=2, H=4, dk=dk, dv=dv, W=37, L=4, s0_std=0.1, seed=400 + dk + Hk,
                            parents="topk", channel_decay=channel, widths=[37, 29, 37, 20], Hk=Hk)
    store, _, _ = check_beam(inp, channel, label=f"H=4 Hk={Hk} dk={dk} ch={channel}")
    assert store.rec_k.shape[3] == Hk
    pairs = np.array([[0, 3], [1, 19]], np.int32)
    S = B.materialize(store, 3, torch.from_numpy(pairs).cuda()).cpu().numpy()
    ref = O.beam_states(inp["S0"], inp["steps"], 3, [tuple(p) for p in pairs])
    assert rel_states(S, ref) <= TOL


@pytest.mark.parametrize("dk,dv,channel,Hk", [(128, 256, False, 2), (128, 512, False, 1), (256, 128, False, 2),
                                               (256, 256, False, 1), (256, 512, False, 1), (128, 256, True, 2),
                                               (128, 512, True, 1)])
def test_wider_geometries(dk, dv, channel, Hk):
    """Operator-suite head dims beyond 128 (OneLA §4.1: K up to 256, V up to
    512): d_v cut into value slices over workgroups, and the fold's row
    slices, for materialisation and the in-place merge."""
    H = 2
    inp = synth.make_inputs(R=2, H=H, dk=dk, dv=dv, W=37, L=5, s0_std=0.05, seed=500 + dk + dv // 8 + Hk,
                            parents="topk", channel_decay=channel, widths=[37, 29, 37, 20, 33], Hk=Hk)
    store, _, _ = check_beam(inp, channel, label=f"dk={dk} dv={dv} Hk={Hk} ch={channel}")
    pairs = np.array([[0, 3], [1, 19], [1, 32]], np.int32)
    S = B.materialize(store, 4, torch.from_numpy(pairs).cuda()).cpu().numpy()
    ref = O.beam_states(inp["S0"], inp["steps"], 4, [tuple(p) for p in pairs])
    assert rel_states(S, ref) <= TOL
    B.log_merge(store, 5, 7)  # every request's base folded with beam 7's chain
    merged = store.S.cpu().numpy()
    ref = O.beam_states(inp["S0"], inp["steps"], 4, [(0, 7), (1, 7)])
    assert rel_states(merged, ref) <= TOL


@pytest.mark.parametrize("dv", [128, 512])
def test_wide_state_long_chains(dv):
    """d_k = 256 with chains of up to six records: the keys of depths 3 .. 5
    come from the record store, not the tile buffer (depth-first schedule with
    one chunk per (request, head), and chunk order)."""
    inp = synth.make_inputs(R=2, H=2, dk=256, dv=dv, W=48, L=7, s0_std=0.05, seed=620 + dv // 128,
                            parents="topk", widths=[48, 41, 48, 37, 48, 45, 48], Hk=1)
    store, _, _ = check_beam(inp, False, label=f"dk=256 dv={dv} L=7")
    pairs = np.array([[0, 5], [1, 47]], np.int32)
    S = B.materialize(store, 6, torch.from_numpy(pairs).cuda()).cpu().numpy()
    assert rel_states(S, O.beam_states(inp["S0"], inp["steps"], 6, [tuple(p) for p in pairs])) <= TOL


def test_wide_state_long_chains_one_chunk(monkeypatch):
    monkeypatch.setenv("GDN_BEAM_CHUNK", "512")
    inp = synth.make_inputs(R=2, H=2, dk=256, dv=256, W=48, L=7, s0_std=0.05, seed=630, parents="topk_hot")
    check_beam(inp, False, label="dk=256 dv=256 L=7 one chunk")


def test_wide_state_beams_over_many_workgroups():
    """d_k = 256, d_v = 512 with one request: four value slices, each cut into
    16-beam chunks (chunk order, ragged last chunk), two value heads sharing
    one key head."""
    inp = synth.make_inputs(R=1, H=2, dk=256, dv=512, W=300, L=4, s0_std=0.05, seed=610,
                            parents="topk", widths=[300, 283, 300, 271], Hk=1)
    check_beam(inp, False, label="dk=256 dv=512 W=300 chunked")


def test_wide_state_sequences():
    """One beam per request with d_k = 256, d_v = 512: the step runs through
    the beam kernel at W = 1, the log merge through the fold."""
    R, H, dk, dv, T, M = 3, 2, 256, 512, 7, 3
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=T, s0_std=0.05, seed=19)
    ref = O.sequence_decode(seq["S0"], seq["tokens"], M)
    store = B.Store(R, 1, H, dk, dv, M, S=torch.from_numpy(seq["S0"]).cuda())
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        o = B.decode_step(store, t, 1, zero, d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        assert rel_slices(o[:, 0].cpu().numpy().reshape(R * H, dv), ref["o"][i]) <= TOL
        if t == M - 1:
            B.log_merge(store, M, 0)
            S = store.S.cpu().numpy().reshape(R * H, 1, dk, dv)
            assert rel_states(S, ref["bases"][i // M][:, None]) <= TOL


@pytest.mark.parametrize("kind", ["scalar", "channel", "plain"])
def test_sequences_with_shared_key_heads(kind):
    """Bounded-log decoding, fused merge path and fold with H = 6 value heads
    on 3 key heads."""
    channel, plain = kind != "scalar", kind == "plain"
    R, H, Hk, dk, dv, T, M = 3, 6, 3, 64, 64, 8, 4
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=T, s0_std=0.1, seed=17,
                                     channel_decay=channel, Hk=Hk)
    ref = O.sequence_decode(seq["S0"], seq["tokens"], M, rule="plain" if plain else "delta")
    S0 = torch.from_numpy(seq["S0"]).cuda()
    fused = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain, S=S0.clone(), Hk=Hk)
    split = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain, S=S0.clone(), Hk=Hk)
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        o_f = B.decode_merge_step(fused, t, *args) if t == M - 1 else B.decode_step(fused, t, 1, zero, *args)
        o_s = B.decode_step(split, t, 1, zero, *args)
        if t == M - 1:
            B.log_merge(split, M, 0)
        torch.cuda.synchronize()
        assert torch.equal(o_f, o_s), i
        assert rel_slices(o_f[:, 0].cpu().numpy().reshape(R * H, dv), ref["o"][i]) <= TOL
        if t == M - 1:
            assert torch.equal(fused.S, split.S), i
            assert rel_states(fused.S.cpu().numpy().reshape(R * H, 1, dk, dv), ref["bases"][i // M][:, None]) <= TOL


@pytest.mark.parametrize("kind", ["scalar", "channel", "plain"])
def test_sequences_small(kind):
    channel, plain = kind != "scalar", kind == "plain"
    R, H, dk, dv, T, M = 5, 3, 64, 64, 12, 4
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=T, s0_std=0.1, seed=7,
                                     channel_decay=channel)
    ref = O.sequence_decode(seq["S0"], seq["tokens"], M, rule="plain" if plain else "delta")
    store = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain,
                    S=torch.from_numpy(seq["S0"]).cuda())
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        o = B.decode_step(store, t, 1, zero, d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        assert rel_slices(o[:, 0].cpu().numpy().reshape(R * H, dv), ref["o"][i]) <= TOL
        if t == M - 1:
            B.log_merge(store, M, 0)
            S = store.S.cpu().numpy().reshape(R * H, 1, dk, dv)
            assert rel_states(S, ref["bases"][i // M][:, None]) <= TOL


@pytest.mark.parametrize("kind", ["scalar", "channel", "plain"])
def test_decode_merge_step(kind):
    """The merge path fused into the decode that fills the log: matches the
    oracle's merged bases and outputs, and equals decode-then-merge exactly."""
    channel, plain = kind != "scalar", kind == "plain"
    R, H, dk, dv, T, M = 5, 3, 64, 64, 12, 4
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=T, s0_std=0.1, seed=11,
                                     channel_decay=channel)
    ref = O.sequence_decode(seq["S0"], seq["tokens"], M, rule="plain" if plain else "delta")
    S0 = torch.from_numpy(seq["S0"]).cuda()
    fused = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain, S=S0.clone())
    split = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, plain_update=plain, S=S0.clone())
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        if t == M - 1:
            o_f = B.decode_merge_step(fused, t, *args)
        else:
            o_f = B.decode_step(fused, t, 1, zero, *args)
        o_s = B.decode_step(split, t, 1, zero, *args)
        if t == M - 1:
            B.log_merge(split, M, 0)
        torch.cuda.synchronize()
        assert torch.equal(o_f, o_s), i
        assert rel_slices(o_f[:, 0].cpu().numpy().reshape(R * H, dv), ref["o"][i]) <= TOL
        if t == M - 1:
            assert torch.equal(fused.S, split.S), i
            S = fused.S.cpu().numpy().reshape(R * H, 1, dk, dv)
            assert rel_states(S, ref["bases"][i // M][:, None]) <= TOL
    log(f"[parity] decode+merge fused {kind}: equal to decode-then-merge")



@pytest.mark.parametrize("dk", [16, 128])
@pytest.mark.parametrize("kind", ["scalar", "channel", "plain"])
def test_sequences_full_log_capacity(dk, kind):
    """Logs of the largest capacity (16 records): every log length 0 .. 15,
    so the sequence kernel stages up to 17 key rows, 15 update vectors and 16
    decay rows (at d = 128 a second staged load per thread; at d = 16 the
    64 threads are exactly filled).  Decode-then-merge and the fused merge
    path agree bit for bit, and both match the oracle, over two full cycles."""
    channel, plain = kind != "scalar", kind == "plain"
    R, H, M = 2, 3, GDN_MAX
    T = 2 * M
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dk, T=T, s0_std=0.1, seed=23,
                                     channel_decay=channel)
    ref = O.sequence_decode(seq["S0"], seq["tokens"], M, rule="plain" if plain else "delta")
    S0 = torch.from_numpy(seq["S0"]).cuda()
    fused = B.Store(R, 1, H, dk, dk, M, channel_decay=channel, plain_update=plain, S=S0.clone())
    split = B.Store(R, 1, H, dk, dk, M, channel_decay=channel, plain_update=plain, S=S0.clone())
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    worst = 0.0
    for i in range(T):
        t = i % M
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        o_f = B.decode_merge_step(fused, t, *args) if t == M - 1 else B.decode_step(fused, t, 1, zero, *args)
        o_s = B.decode_step(split, t, 1, zero, *args)
        if t == M - 1:
            B.log_merge(split, M, 0)
        torch.cuda.synchronize()
        assert torch.equal(o_f, o_s), i
        e = rel_slices(o_f[:, 0].cpu().numpy().reshape(R * H, dk), ref["o"][i])
        worst = max(worst, e)
        assert e <= TOL, (i, e)
        if t == M - 1:
            assert torch.equal(fused.S, split.S), i
            e = rel_states(fused.S.cpu().numpy().reshape(R * H, 1, dk, dk), ref["bases"][i // M][:, None])
            worst = max(worst, e)
            assert e <= TOL, (i, e)
    log(f"[parity] full log capacity d={dk} {kind}: max rel err {worst:.2e}")


# ---------------------------------------------------------------- edge cases

def test_single_beam_in_wide_store():
    inp = synth.make_inputs(R=2, H=2, dk=128, dv=128, W=1, L=3, s0_std=0.05, seed=8,
                            parents="uniform")
    check_beam(inp, False, W_max=16, label="W_t=1")


def test_longest_chain():
    inp = synth.make_inputs(R=2, H=2, dk=32, dv=32, W=6, L=B.GDN_MAX_STEPS, s0_std=0.1, seed=9,
                            parents="uniform")
    check_beam(inp, False, label="L=16")
    inp = synth.make_inputs(R=1, H=2, dk=32, dv=32, W=6, L=B.GDN_MAX_STEPS, s0_std=0.1, seed=9,
                            parents="uniform", channel_decay=True)
    check_beam(inp, True, label="L=16 channel")


@pytest.mark.parametrize("kind", ["identity", "fanout"])
def test_degenerate_lineages(kind):
    inp = synth.make_inputs(R=2, H=2, dk=128, dv=128, W=24, L=4, s0_std=0.05, seed=10,
                            parents="uniform")
    for st in inp["steps"][1:]:
        st["parent"][:] = np.arange(24) if kind == "identity" else 7
    _, outs, ref = check_beam(inp, False, label=kind)
    if kind == "identity":
        assert np.all(ref["anc"][3] == np.arange(24)[None, :, None])


@pytest.mark.parametrize("channel", [False, True])
def test_gates_at_extremes(channel):
    # beta = 0: o = (prod decay) S0^T q; alpha = 1: S0 enters at full weight
    inp = synth.make_inputs(R=2, H=2, dk=128, dv=128, W=20, L=4, s0_std=0.05, seed=11,
                            parents="topk", channel_decay=channel, beta_const=0.0)
    store, _, _ = check_beam(inp, channel, label="beta=0")
    assert torch.count_nonzero(store.rec_delta) == 0
    inp = synth.make_inputs(R=2, H=2, dk=128, dv=128, W=20, L=4, s0_std=0.05, seed=12,
                            parents="topk", channel_decay=channel, alpha_const=1.0)
    check_beam(inp, channel, label="alpha=1")


@pytest.mark.parametrize("dk,dv,channel", [(256, 512, False), (256, 128, False), (128, 512, False), (128, 512, True)])
def test_wide_gates_at_extremes(dk, dv, channel):
    """The S0 contraction of the wide geometries at full weight (two bf16
    planes at d_k = 256): beta = 0 gives o = (prod decay) S0^T q, alpha = 1
    keeps S0 undecayed through the chain."""
    inp = synth.make_inputs(R=2, H=2, dk=dk, dv=dv, W=20, L=4, s0_std=0.05, seed=700 + dk + dv // 8,
                            parents="topk", channel_decay=channel, beta_const=0.0)
    store, _, _ = check_beam(inp, channel, label=f"dk={dk} dv={dv} beta=0")
    assert torch.count_nonzero(store.rec_delta) == 0
    inp = synth.make_inputs(R=2, H=2, dk=dk, dv=dv, W=20, L=4, s0_std=0.05, seed=701 + dk + dv // 8,
                            parents="topk", channel_decay=channel, alpha_const=1.0)
    check_beam(inp, channel, label=f"dk={dk} dv={dv} alpha=1")


@pytest.mark.parametrize("wname,channel,requests,heads", [("LARGE", False, [3], [0, 31]), ("KDA", True, [9], [0, 31]),
                                                          ("WIDE", False, [5], [15]), ("KDA_WIDE", True, [1], [7]),
                                                          ("SHARED_KEYS", False, [6], [2, 3])])
def test_workloads_with_undecayed_context(wname, channel, requests, heads):
    """Each full-size beam workload with alpha = 1 (scalar or every channel),
    so that the shared-context term is not damped by the chain's decays."""
    w = getattr(configs, wname)
    check_beam(w.inputs(alpha_const=1.0), channel, requests=requests, heads=heads, label=f"{w.name} alpha=1")


def test_orthonormal_keys_retrieve_exactly():
    inp = synth.make_inputs(R=2, H=2, dk=32, dv=32, W=9, L=4, s0_std=0.05, seed=13,
                            parents="uniform", alpha_const=1.0, beta_const=1.0)
    sigma = [3, 30, 11, 17]
    one = synth.bf16_bits(np.float32(1.0))
    for t, st in enumerate(inp["steps"]):
        st["k"][:] = 0
        st["k"][..., sigma[t]] = one
        st["q"][:] = 0
        st["q"][..., sigma[t // 2]] = one
    inp["S0"][:] = 0
    store, outs = run_beam(inp)
    anc = O.ancestry([s.get("parent") for s in inp["steps"]], 2, 9)
    for t in range(4):
        j = t // 2
        for r in range(2):
            slot = anc[t][r, :, j] if j < t else np.arange(9)
            v = synth.bf16_bits_to_f32(inp["steps"][j]["v"][r, slot])
            assert np.array_equal(outs[t][r], v), (t, r)


# --------------------------------------------------------- materialise / merge

@pytest.mark.parametrize("channel", [False, True])
def test_materialize(channel):
    inp = synth.make_inputs(R=2, H=3, dk=128, dv=128, W=40, L=3, s0_std=0.05, seed=14,
                            parents="topk", channel_decay=channel)
    store, _ = run_beam(inp, channel)
    pairs = [(0, 0), (1, 39), (0, 17), (1, 5)]
    rb = torch.tensor(pairs, dtype=torch.int32, device="cuda")
    for t in range(3):
        S = B.materialize(store, t, rb).cpu().numpy()
        ref = O.beam_states(inp["S0"], inp["steps"], t, pairs)
        err = rel_states(S, ref)
        log(f"[parity] materialize t={t} ch={channel}: {err:.2e}")
        assert err <= TOL


@pytest.mark.parametrize("dims", [(128, 128), (64, 64)])
def test_kernels_mixed_on_one_store(dims, monkeypatch):
    """Scalar-decay beam steps alternate between the fused kernel (records at
    the beams' depth-first positions) and the general kernel (records at the
    beams' indices) on one store, with a hot parent so that the order is far
    from the index order: every step, the ancestry and the records still
    match the oracle, and so do states materialised from the store."""
    dk, dv = dims
    inp = synth.make_inputs(R=2, H=3, dk=dk, dv=dv, W=96, L=6, s0_std=0.05, seed=31, parents="topk_hot")
    S0 = inp["S0"]
    store = B.Store(2, 96, 3, dk, dv, 6, S=torch.from_numpy(S0).cuda())
    outs = []
    for t, st in enumerate(inp["steps"]):
        if t % 2:
            monkeypatch.setenv("GDN_BEAM_GENERIC", "1")
        else:
            monkeypatch.delenv("GDN_BEAM_GENERIC", raising=False)
        d = B.upload(st)
        outs.append(B.decode_step(store, t, 96, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"]))
    monkeypatch.delenv("GDN_BEAM_GENERIC", raising=False)
    torch.cuda.synchronize()
    ref = O.beam_decode(S0, inp["steps"])
    for t, st in enumerate(inp["steps"]):
        d, kbits, a, anc = step_records(store, t, 96)
        assert np.array_equal(anc, ref["anc"][t]), t
        assert np.array_equal(kbits, st["k"]), t
        eo, ed = rel_slices(outs[t].cpu().numpy(), ref["o"][t]), rel_slices(d, ref["delta"][t])
        assert eo <= TOL and ed <= TOL, (t, eo, ed)
    pairs = [(0, 0), (1, 95), (0, 41), (1, 7)]
    rb = torch.tensor(pairs, dtype=torch.int32, device="cuda")
    for t in range(6):
        err = rel_states(B.materialize(store, t, rb).cpu().numpy(), O.beam_states(S0, inp["steps"], t, pairs))
        assert err <= TOL, (t, err)
    log(f"[parity] fused and general kernels on one store, d = {dk}: ok")


def test_merge_of_beam_chain():
    inp = synth.make_inputs(R=3, H=2, dk=64, dv=64, W=12, L=3, s0_std=0.1, seed=15,
                            parents="topk")
    store, _ = run_beam(inp)
    B.log_merge(store, 3, beam=5)
    ref = O.beam_states(inp["S0"], inp["steps"], 2, [(r, 5) for r in range(3)])
    assert rel_states(store.S.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("channel", [False, True])
def test_merge_then_decode_equals_decode_with_log(channel):
    R, H, dk, dv, M = 4, 4, 128, 128, 4
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=M, s0_std=0.05, seed=16,
                                     channel_decay=channel)
    toks = [B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
            for i in range(M)]
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    S0 = torch.from_numpy(seq["S0"]).cuda()
    a = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, S=S0.clone())
    for i, d in enumerate(toks):
        o_log = B.decode_step(a, i, 1, zero, d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    b = B.Store(R, 1, H, dk, dv, M, channel_decay=channel, S=S0.clone())
    for i, d in enumerate(toks[:-1]):
        B.decode_step(b, i, 1, zero, d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    B.log_merge(b, M - 1, 0)
    d = toks[-1]
    o_merged = B.decode_step(b, 0, 1, zero, d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    assert rel_slices(o_merged.cpu().numpy(), o_log.cpu().numpy()) <= TOL


def test_identity_merge_is_bit_exact():
    R, H, dk, dv, M = 3, 2, 128, 128, 5
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=M, s0_std=0.05, seed=17)
    seq["tokens"]["alpha"][:] = 1.0
    seq["tokens"]["beta"][:] = 0.0
    S0 = torch.from_numpy(seq["S0"]).cuda()
    st = B.Store(R, 1, H, dk, dv, M, S=S0.clone())
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")
    for i in range(M):
        d = B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
        B.decode_step(st, i, 1, zero, d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    B.log_merge(st, M, 0)
    assert torch.equal(st.S, S0)


# ------------------------------------------ determinism, reordering, isolation

def test_deterministic_and_reorder_invariant():
    inp = synth.make_inputs(R=2, H=4, dk=128, dv=128, W=48, L=4, s0_std=0.05, seed=18,
                            parents="topk")
    _, o1 = run_beam(inp)
    _, o2 = run_beam(inp)
    for a, b in zip(o1, o2):
        assert np.array_equal(a, b)
    rng = np.random.default_rng(0)
    perms = [rng.permutation(48) for _ in inp["steps"]]
    inv = [np.argsort(p) for p in perms]
    pinp = {"S0": inp["S0"], "steps": []}
    for t, st in enumerate(inp["steps"]):
        ps = {n: np.ascontiguousarray(st[n][:, perms[t]]) for n in ("q", "k", "v", "alpha", "beta")}
        if t:
            ps["parent"] = inv[t - 1][st["parent"][:, perms[t]]].astype(np.int32)
        pinp["steps"].append(ps)
    _, op = run_beam(pinp)
    for t in range(4):
        assert np.array_equal(op[t], o1[t][:, perms[t]]), t


def test_duplicate_children_agree():
    inp = synth.make_inputs(R=1, H=2, dk=128, dv=128, W=32, L=3, s0_std=0.05, seed=19,
                            parents="uniform")
    for t in (1, 2):
        st = inp["steps"][t]
        st["parent"][0, 1] = st["parent"][0, 0]
        for n in ("q", "k", "v", "alpha", "beta"):
            st[n][0, 1] = st[n][0, 0]
        if t == 2:
            st["parent"][0, 0], st["parent"][0, 1] = 0, 1
    _, outs = run_beam(inp)
    assert np.array_equal(outs[1][0, 0], outs[1][0, 1])
    assert np.array_equal(outs[2][0, 0], outs[2][0, 1])


def test_append_only_and_guards():
    inp = synth.make_inputs(R=2, H=2, dk=128, dv=128, W=30, L=4, s0_std=0.05, seed=20,
                            parents="topk")
    W_max, W = 40, 30
    store = B.Store(2, W_max, 2, 128, 128, 4, S=torch.from_numpy(inp["S0"]).cuda())
    store.rec_delta.fill_(float("nan"))
    store.rec_alpha.fill_(float("nan"))
    n_o = 2 * W * 2 * 128
    guard = 64
    o_big = torch.full((n_o + 2 * guard,), -7.0, device="cuda")
    o = o_big[guard:guard + n_o].view(2, W, 2, 128)
    snaps = []
    for t, st in enumerate(inp["steps"]):
        d = B.upload(st)
        B.decode_step(store, t, W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"],
                      d["beta"], o=o)
        torch.cuda.synchronize()
        for j, (sd, sk, sa) in enumerate(snaps):  # earlier records are never rewritten
            assert torch.equal(store.rec_delta[j, :, :W], sd)
            assert torch.equal(store.rec_k[j, :, :W], sk)
            assert torch.equal(store.rec_alpha[j, :, :W], sa)
        snaps.append((store.rec_delta[t, :, :W].clone(), store.rec_k[t, :, :W].clone(),
                      store.rec_alpha[t, :, :W].clone()))
        assert torch.all(o_big[:guard] == -7.0) and torch.all(o_big[guard + n_o:] == -7.0)
        assert torch.isnan(store.rec_delta[t, :, W:]).all()  # slots >= W_t untouched
        assert torch.isnan(store.rec_alpha[t, :, W:]).all()
        assert not torch.isnan(store.rec_delta[t, :, :W]).any()
        assert not torch.isnan(o).any()


@pytest.mark.parametrize("dk,dv,channel", [(128, 128, False), (128, 128, True), (16, 16, False), (256, 512, False)])
def test_beam_decode_graph_replay(dk, dv, channel):
    """All L steps of a beam decode captured once in a HIP graph (the fused
    scalar and channel-decay kernels, the general kernel, the value-sliced
    d_k = 256 kernel): every replay, with eager work and synchronisation in
    between, equals an eager run bit for bit (outputs, records and ancestry;
    the schedule-order entry of each ancestry row may differ with tie order)."""
    R, H, W, L = 2, 2, 40, 4
    inp = synth.make_inputs(R=R, H=H, dk=dk, dv=dv, W=W, L=L, s0_std=0.05, seed=31 + dk, parents="topk",
                            channel_decay=channel)
    S0 = torch.from_numpy(inp["S0"]).cuda()
    steps = [B.upload(st) for st in inp["steps"]]

    def run(store, outs):
        for t in range(L):
            d = steps[t]
            B.decode_step(store, t, W, d.get("parent"), d["q"], d["k"], d["v"], d["alpha"], d["beta"], o=outs[t])

    mk = lambda: B.Store(R, W, H, dk, dv, L, channel_decay=channel, S=S0.clone())
    new_outs = lambda: [torch.empty(R, W, H, dv, device="cuda") for _ in range(L)]
    run(mk(), new_outs())  # warm-up outside the capture
    torch.cuda.synchronize()
    eager, graphed = mk(), mk()
    e_out, g_out = new_outs(), new_outs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(graphed, g_out)
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        run(eager, e_out)
        torch.cuda.synchronize()
        for t in range(L):
            assert torch.equal(g_out[t], e_out[t]), (rep, t)
            assert torch.equal(graphed.anc[t, :, :, :t], eager.anc[t, :, :, :t]), (rep, t)
        for name in ("rec_delta", "rec_k", "rec_alpha"):
            assert torch.equal(getattr(graphed, name), getattr(eager, name)), (rep, name)
    ref = O.beam_decode(inp["S0"], inp["steps"])
    assert max(rel_slices(g_out[t].cpu().numpy(), ref["o"][t]) for t in range(L)) <= TOL
    log(f"[parity] beam decode dk={dk} dv={dv} ch={channel}: 3 graph replays equal the eager run")


def test_merge_cycle_graph_replay():
    """A bounded-log merge cycle (M - 1 appends, then the decode that merges)
    captured once in a HIP graph: every replay, with eager work and
    synchronisation between replays, equals the same cycle run eagerly."""
    R, H, dk, dv, M = 4, 2, 64, 64, 4
    seq = synth.make_sequence_inputs(R=R, H=H, dk=dk, dv=dv, T=M, s0_std=0.1, seed=21)
    S0 = torch.from_numpy(seq["S0"]).cuda()
    toks = [B.upload({n: seq["tokens"][n][i][:, None] for n in ("q", "k", "v", "alpha", "beta")})
            for i in range(M)]
    zero = torch.zeros(R, 1, dtype=torch.int32, device="cuda")

    def cycle(store, outs):
        for i in range(M):
            a = (toks[i]["q"], toks[i]["k"], toks[i]["v"], toks[i]["alpha"], toks[i]["beta"])
            if i == M - 1:
                B.decode_merge_step(store, i, *a, o=outs[i])
            else:
                B.decode_step(store, i, 1, zero, *a, o=outs[i])

    warm = B.Store(R, 1, H, dk, dv, M, S=S0.clone())
    cycle(warm, [torch.empty(R, 1, H, dv, device="cuda") for _ in range(M)])
    torch.cuda.synchronize()
    eager = B.Store(R, 1, H, dk, dv, M, S=S0.clone())
    graphed = B.Store(R, 1, H, dk, dv, M, S=S0.clone())
    e_out = [torch.empty(R, 1, H, dv, device="cuda") for _ in range(M)]
    g_out = [torch.empty(R, 1, H, dv, device="cuda") for _ in range(M)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cycle(graphed, g_out)
    torch.cuda.synchronize()
    # capture records the launches without running them: the graphed store is untouched
    assert torch.equal(graphed.S, S0)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        cycle(eager, e_out)
        torch.cuda.synchronize()
        for i in range(M):
            assert torch.equal(g_out[i], e_out[i]), (rep, i)
        assert torch.equal(graphed.S, eager.S), rep
        assert torch.equal(graphed.rec_delta, eager.rec_delta), rep
    log("[parity] merge cycle: 3 graph replays equal the eager cycle")
