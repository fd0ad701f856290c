"""The full-size parity checker (full_parity.py) on the CPU: it must report
agreement for outputs equal to the oracle's, rounded to FP32, and must find a
single planted error in one (request, head) pair."""

import numpy as np

import full_parity
import oracle.gdn_oracle as O
from linear_attention_beam_gdn_amd import configs


def _beam_outputs(w, inp):
    ref = O.beam_decode(inp["S0"], inp["steps"])
    return [o.astype(np.float32) for o in ref["o"]], [d.astype(np.float32) for d in ref["delta"]]


def test_beam_checker_agrees_and_finds_a_planted_error(tmp_path):
    over = {"R": 2, "W": 24, "H": 3}
    w = configs.LARGE.__class__(**{**configs.LARGE.__dict__, **over})
    o, d = _beam_outputs(w, w.inputs())
    for t in range(w.L):
        np.save(tmp_path / f"o_{t}.npy", o[t])
        np.save(tmp_path / f"d_{t}.npy", d[t])
    res = full_parity.run("beam", "gdn_large_beam", str(tmp_path), over=over)
    assert res["pairs"] == 6
    assert res["worst"]["o"]["rel_err"] < 1e-6 and res["worst"]["delta"]["rel_err"] < 1e-6
    # one value of one beam of pair (1, 2) at the last step, off by 1e-3 relative
    d[3][1, 5, 2, 7] += 1e-3 * np.abs(d[3][1, 5, 2]).max()
    np.save(tmp_path / "d_3.npy", d[3])
    res = full_parity.run("beam", "gdn_large_beam", str(tmp_path), over=over)
    assert res["worst"]["delta"]["pair"] == [1, 2]
    assert 0.9e-3 < res["worst"]["delta"]["rel_err"] < 1.1e-3


def test_sequence_checker_agrees_and_finds_a_planted_error(tmp_path):
    over = {"R": 3, "H": 2, "T": 12, "M": 4}
    w = configs.DELTALOG.__class__(**{**configs.DELTALOG.__dict__, **over})
    seq = w.inputs()
    ref = O.sequence_decode(seq["S0"], seq["tokens"], w.M)
    # the oracle's pair order is (r, h) row-major: back to [T, R, H, ...]
    o = ref["o"].reshape(w.T, w.R, w.H, w.dv).astype(np.float32)
    d = ref["delta"].reshape(w.T, w.R, w.H, w.dv).astype(np.float32)
    bases = ref["bases"].reshape(-1, w.R, w.H, w.dk, w.dv).astype(np.float32)
    np.save(tmp_path / "o.npy", o)
    np.save(tmp_path / "d.npy", d)
    for m in range(bases.shape[0]):
        np.save(tmp_path / f"S_{m}.npy", bases[m])
    res = full_parity.run("seq", "deltalog_bounded_log", str(tmp_path), over=over)
    assert res["pairs"] == 6
    assert max(v["rel_err"] for v in res["worst"].values()) < 1e-6
    bases[2, 2, 1, 3, 4] += 2e-3 * np.abs(bases[2, 2, 1]).max()
    np.save(tmp_path / "S_2.npy", bases[2])
    res = full_parity.run("seq", "deltalog_bounded_log", str(tmp_path), over=over)
    assert 1.9e-3 < res["worst"]["base"]["rel_err"] < 2.1e-3
