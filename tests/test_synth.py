"""The seeded input generator: determinism, formats and distributions."""

import numpy as np
import torch

from linear_attention_beam_gdn_amd import configs, synth


def test_bf16_encoding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 3
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_shaped():
    a = configs.TINY.inputs()
    b = configs.TINY.inputs()
    assert np.array_equal(a["S0"], b["S0"])
    for sa, sb in zip(a["steps"], b["steps"]):
        for n in sa:
            assert np.array_equal(sa[n], sb[n])
    w = configs.TINY
    assert a["S0"].shape == (w.R, w.H, w.dk, w.dv) and a["S0"].dtype == np.float32
    for t, st in enumerate(a["steps"]):
        assert st["q"].shape == (w.R, w.W, w.H, w.dk) and st["q"].dtype == np.uint16
        assert st["v"].shape == (w.R, w.W, w.H, w.dv)
        assert st["alpha"].shape == (w.R, w.W, w.H) and st["alpha"].dtype == np.float32
        assert ("parent" in st) == (t > 0)


def test_distributions():
    inp = synth.make_inputs(R=2, H=4, dk=128, dv=64, W=64, L=2, s0_std=0.05, seed=9,
                            parents="topk", channel_decay=True)
    st = inp["steps"][1]
    for n in ("q", "k"):
        norms = np.linalg.norm(synth.bf16_bits_to_f32(st[n]).astype(np.float64), axis=-1)
        assert np.all(np.abs(norms - 1) < 2 ** -7)
    assert st["alpha"].shape == (2, 64, 4, 128)
    assert np.all((st["alpha"] > 0) & (st["alpha"] < 1))
    assert np.all((st["beta"] > 0) & (st["beta"] < 1))
    assert abs(float(inp["S0"].std()) - 0.05) < 0.002
    assert np.all((st["parent"] >= 0) & (st["parent"] < 64))


def test_hot_parent_fanout():
    inp = synth.make_inputs(R=3, H=1, dk=16, dv=16, W=100, L=3, s0_std=0.05, seed=2,
                            parents="topk_hot", hot_frac=0.3)
    for st in inp["steps"][1:]:
        for r in range(3):
            counts = np.bincount(st["parent"][r], minlength=100)
            assert counts.max() >= 30


def test_topk_parents_from_expansion():
    inp = synth.make_inputs(R=1, H=1, dk=16, dv=16, W=32, L=4, s0_std=0.05, seed=4,
                            parents="topk", expand=8)
    for st in inp["steps"][1:]:
        p = st["parent"][0]
        assert np.all((p >= 0) & (p < 32))
        assert len(np.unique(p)) < 32  # reselection merges and prunes branches


def test_key_heads():
    """Hk = H draws exactly what the default draws; Hk < H gives q and k Hk
    heads (unit-norm) and leaves v, the gates and the parents per value head."""
    kw = dict(R=2, H=4, dk=16, dv=8, W=10, L=3, s0_std=0.1, seed=12, parents="topk")
    a, b = synth.make_inputs(**kw), synth.make_inputs(Hk=4, **kw)
    for sa, sb in zip(a["steps"], b["steps"]):
        for n in sa:
            assert np.array_equal(sa[n], sb[n])
    c = synth.make_inputs(Hk=2, **kw)
    for st in c["steps"]:
        assert st["q"].shape == (2, 10, 2, 16) and st["k"].shape == (2, 10, 2, 16)
        assert st["v"].shape == (2, 10, 4, 8) and st["alpha"].shape == (2, 10, 4)
        norms = np.linalg.norm(synth.bf16_bits_to_f32(st["k"]).astype(np.float64), axis=-1)
        assert np.all(np.abs(norms - 1) < 2 ** -7)
    seq = synth.make_sequence_inputs(R=2, H=6, dk=8, dv=8, T=3, s0_std=0.1, seed=3, Hk=3)
    assert seq["tokens"]["q"].shape == (3, 2, 3, 8) and seq["tokens"]["v"].shape == (3, 2, 6, 8)
