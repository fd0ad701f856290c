"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one: a flipped sign, a transposed operand, a dropped or misplaced
decay or gate, a read-out before the write, a decay on the wrong side, and
ancestry indexed by the child instead of the parent."""

import numpy as np
import pytest

import oracle.gdn_oracle as O
import pins

_transition = O.transition  # the oracle's own, for the rule a mutant leaves alone


def _sign(S, k, v, alpha, beta, rule="delta"):
    if rule != "delta":
        return _transition(S, k, v, alpha, beta, rule)
    S_dec = O.decay(S, alpha)
    delta = beta[:, None] * (v + O.readout(S_dec, k))
    return S_dec + k[:, :, None] * delta[:, None, :], delta


def _transposed(S, k, v, alpha, beta, rule="delta"):
    if rule != "delta":
        return _transition(S, k, v, alpha, beta, rule)
    S_dec = O.decay(S, alpha)
    if S.shape[1] != S.shape[2]:
        raise ValueError("transposed read-out only type-checks for square states")
    delta = beta[:, None] * (v - np.matmul(S_dec, k[:, :, None])[:, :, 0])
    return S_dec + k[:, :, None] * delta[:, None, :], delta


def _undecayed_prediction(S, k, v, alpha, beta, rule="delta"):
    if rule != "delta":
        return _transition(S, k, v, alpha, beta, rule)
    delta = beta[:, None] * (v - O.readout(S, k))
    return O.decay(S, alpha) + k[:, :, None] * delta[:, None, :], delta


def _no_beta(S, k, v, alpha, beta, rule="delta"):
    if rule != "delta":
        return _transition(S, k, v, alpha, beta, rule)
    S_dec = O.decay(S, alpha)
    delta = v - O.readout(S_dec, k)
    return S_dec + k[:, :, None] * delta[:, None, :], delta


def _decay_after_write(S, k, v, alpha, beta, rule="delta"):
    if rule != "delta":
        return _transition(S, k, v, alpha, beta, rule)
    delta = beta[:, None] * (v - O.readout(S, k))
    return O.decay(S + k[:, :, None] * delta[:, None, :], alpha), delta


def _decay_value_side(S, alpha):
    if alpha.ndim == 1:
        return alpha[:, None, None] * S
    if S.shape[1] != S.shape[2]:
        raise ValueError("value-side decay only type-checks for square states")
    return alpha[:, None, :] * S


def _no_scalar_decay(S, alpha):
    if alpha.ndim == 1:
        return S
    return alpha[:, :, None] * S


def _readout_before_write(S0, steps, anc, t, r, h, beams, rule="delta"):
    beams = np.asarray(beams, dtype=np.int64)
    S = np.repeat(S0[r, h][None].astype(np.float64), len(beams), axis=0)
    for j in range(t):
        slot = anc[t][r, beams, j]
        _, k, v, alpha, beta = O._token(steps[j], r, slot, h)
        S, _ = O.transition(S, k, v, alpha, beta, rule)
    q, k, v, alpha, beta = O._token(steps[t], r, beams, h)
    S_new, delta = O.transition(S, k, v, alpha, beta, rule)
    return S, delta, q


def _plain_scaled_by_beta(S, k, v, alpha, beta, rule="delta"):
    if rule != "plain":
        return _transition(S, k, v, alpha, beta, rule)
    delta = beta[:, None] * v
    return O.decay(S, alpha) + k[:, :, None] * delta[:, None, :], delta


def _plain_decay_after_write(S, k, v, alpha, beta, rule="delta"):
    if rule != "plain":
        return _transition(S, k, v, alpha, beta, rule)
    return O.decay(S + k[:, :, None] * v[:, None, :], alpha), v


def _plain_with_delta_correction(S, k, v, alpha, beta, rule="delta"):
    return _transition(S, k, v, alpha, beta, "delta")


def _key_head_by_value_head(step, h):
    return min(h, step["q"].shape[2] - 1)


def _anc_child_index(parents, R, W0):
    anc = [np.zeros((R, W0, 0), dtype=np.int64)]
    for t in range(1, len(parents)):
        pi = np.asarray(parents[t], dtype=np.int64)
        prev = anc[t - 1]
        Wt = pi.shape[1]
        row = np.empty((R, Wt, t), dtype=np.int64)
        for r in range(R):
            own = np.minimum(np.arange(Wt), prev.shape[1] - 1)
            row[r, :, : t - 1] = prev[r, own, :]
            row[r, :, t - 1] = pi[r]
        anc.append(row)
    return anc


def _anc_depth_swapped(parents, R, W0):
    anc = [np.zeros((R, W0, 0), dtype=np.int64)]
    for t in range(1, len(parents)):
        pi = np.asarray(parents[t], dtype=np.int64)
        prev = anc[t - 1]
        row = np.empty((R, pi.shape[1], t), dtype=np.int64)
        for r in range(R):
            row[r, :, 1:] = prev[r, pi[r], :]
            row[r, :, 0] = pi[r]
        anc.append(row)
    return anc


MUTANTS = {
    "delta_sign": ("transition", _sign),
    "transposed_readout": ("transition", _transposed),
    "prediction_from_undecayed_state": ("transition", _undecayed_prediction),
    "beta_dropped": ("transition", _no_beta),
    "decay_after_write": ("transition", _decay_after_write),
    "channel_decay_on_value_side": ("decay", _decay_value_side),
    "scalar_decay_dropped": ("decay", _no_scalar_decay),
    "readout_before_write": ("_eager_chain", _readout_before_write),
    "ancestry_child_index": ("ancestry", _anc_child_index),
    "ancestry_depth_order": ("ancestry", _anc_depth_swapped),
    "plain_update_scaled_by_beta": ("transition", _plain_scaled_by_beta),
    "plain_decay_after_write": ("transition", _plain_decay_after_write),
    "plain_with_delta_correction": ("transition", _plain_with_delta_correction),
    "key_head_indexed_by_value_head": ("_key_head", _key_head_by_value_head),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pname, pin in pins.ALL_PINS.items():
        try:
            pin()
        except AssertionError:
            caught.append(pname)
        except (ValueError, IndexError):
            pass  # a shape error is not counted as a catch
    assert caught, f"no pin caught the planted mistake {name!r}"
