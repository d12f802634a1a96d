"""The oracle's pins catch plausible mistakes in the oracle.

Each case below plants one mistake in the oracle (on the CPU, through
monkeypatch; the oracle's source is untouched): a dropped term, a wrong
sign, swapped halves of [left | gate], a transposed or misindexed operand,
a wrong expert or layer.  Every pin in ``test_oracle.py`` then runs against
the planted oracle, and at least one of them must fail.  The control case
runs the same pins on the untouched oracle and all of them must pass, so a
failure under a mutant is the mutant's doing.
"""
import inspect
import warnings

import numpy as np
import pytest

import oracle
import oracle.swiglu as osw
import test_oracle as pins

# the untouched functions, for the mutants that wrap them
_sigmoid, _backward = osw.sigmoid, osw.backward
_bwd_elem, _fwd_elem = osw.swiglu_bwd_elementwise, osw.swiglu_fwd_elementwise
_moe_backward, _stack_backward = osw.moe_backward, osw.stack_backward
_backward_residual, _sampled = osw.backward_residual, osw.sampled_forward_backward
_bytes = osw.algorithmic_bytes


def _sigmoid_sign_flipped(g):
    return 1.0 / (1.0 + np.exp(np.asarray(g, dtype=np.float64)))


def _silu_without_sigma(g):
    return np.asarray(g, dtype=np.float64)


def _dsilu_drops_term(g):
    return _sigmoid(g)


def _dsilu_wrong_sign(g):
    g = np.asarray(g, dtype=np.float64)
    s = _sigmoid(g)
    return s * (1.0 - g * (1.0 - s))


def _bwd_dgate_drops_left(preact, dout):
    P = np.asarray(preact, dtype=np.float64)
    I = P.shape[1] // 2
    gp, h = _bwd_elem(preact, dout)
    gp[:, I:] = np.asarray(dout) * osw.dsilu(P[:, I:])
    return gp, h


def _bwd_halves_swapped(preact, dout):
    P = np.asarray(preact, dtype=np.float64)
    I = P.shape[1] // 2
    return _bwd_elem(np.concatenate([P[:, I:], P[:, :I]], axis=1), dout)


def _fwd_halves_swapped(preact):
    P = np.asarray(preact, dtype=np.float64)
    I = P.shape[1] // 2
    return _fwd_elem(np.concatenate([P[:, I:], P[:, :I]], axis=1))


def _backward_dx_drops_gate_half(x, W1, Wd, dy):
    r = _backward(x, W1, Wd, dy)
    I = np.asarray(Wd).shape[0]
    r["dx"] = r["grad_preact"][:, :I] @ np.asarray(W1, dtype=np.float64)[:, :I].T
    return r


def _backward_dW1_rows_shifted(x, W1, Wd, dy):
    r = _backward(x, W1, Wd, dy)
    r["dW1"] = np.roll(np.asarray(x, dtype=np.float64), 1, axis=0).T @ r["grad_preact"]
    return r


def _backward_dW_down_from_gate(x, W1, Wd, dy):
    r = _backward(x, W1, Wd, dy)
    I = np.asarray(Wd).shape[0]
    r["dW_down"] = r["preact"][:, I:].T @ np.asarray(dy, dtype=np.float64)
    return r


def _backward_dout_doubled(x, W1, Wd, dy):
    # dout counted twice (a doubled term), carried through to its products
    r = _backward(x, W1, Wd, dy)
    for k in ("dout", "grad_preact", "dx", "dW1"):
        r[k] = 2.0 * r[k]
    return r


def _residual_drops_identity_grad(x, W1, Wd, dy):
    r = _backward_residual(x, W1, Wd, dy)
    r["dx"] = r["dx"] - np.asarray(dy, dtype=np.float64)
    return r


def _stack_layers_reversed(x, layers, dy):
    r = _stack_backward(x, layers, dy)
    r["dW1"], r["dW_down"] = r["dW1"][::-1], r["dW_down"][::-1]
    return r


def _moe_wrong_expert(x, W1s, Wds, offsets, dy):
    r = _moe_backward(x, W1s, Wds, offsets, dy)
    r["dW1"] = np.roll(r["dW1"], 1, axis=0)
    return r


def _sampled_rows_reversed(x, W1, Wd, dy, rows, chans):
    r = _sampled(x, W1, Wd, dy, rows, chans)
    r["dW_down_rows"] = r["dW_down_rows"][::-1]
    return r


def _bytes_fused_without_h(M, D, I, Dout, elem=2):
    b = _bytes(M, D, I, Dout, elem)
    b["fused_dgrad"] -= elem * M * I
    b["unfused_dgrad"] -= elem * M * I
    return b


def _bytes_forward_h_once(M, D, I, Dout, elem=2):
    b = _bytes(M, D, I, Dout, elem)
    b["forward"] -= elem * M * I
    return b


MUTANTS = {
    "sigmoid with the exponent's sign flipped": {"sigmoid": _sigmoid_sign_flipped},
    "silu without its sigma factor": {"silu": _silu_without_sigma},
    "silu' dropping g(1-sigma)": {"dsilu": _dsilu_drops_term, "dsilu_form2": _dsilu_drops_term},
    "silu' with a wrong sign": {"dsilu": _dsilu_wrong_sign, "dsilu_form2": _dsilu_wrong_sign},
    "dgate without the left factor": {"swiglu_bwd_elementwise": _bwd_dgate_drops_left},
    "backward reading gate as left": {"swiglu_bwd_elementwise": _bwd_halves_swapped},
    "forward reading gate as left": {"swiglu_fwd_elementwise": _fwd_halves_swapped},
    "dx without the gate half's term": {"backward": _backward_dx_drops_gate_half},
    "dW1 with x's rows shifted by one": {"backward": _backward_dW1_rows_shifted},
    "dW_down from the gate instead of h": {"backward": _backward_dW_down_from_gate},
    "dout doubled": {"backward": _backward_dout_doubled},
    "residual dx without the identity path": {"backward_residual": _residual_drops_identity_grad},
    "stack gradients in reversed layer order": {"stack_backward": _stack_layers_reversed},
    "MoE dW1 given to the wrong expert": {"moe_backward": _moe_wrong_expert},
    "sampled dW_down rows misordered": {"sampled_forward_backward": _sampled_rows_reversed},
    "fused dgrad bytes without the h store": {"algorithmic_bytes": _bytes_fused_without_h},
    "forward bytes with h moved once": {"algorithmic_bytes": _bytes_forward_h_once},
}


def _pins():
    """Every test function of test_oracle.py with its arguments (the first
    value of each parametrized argument)."""
    out = []
    for name, fn in sorted(vars(pins).items()):
        if not (name.startswith("test_") and callable(fn)):
            continue
        kwargs = {}
        for mark in getattr(fn, "pytestmark", []):
            if mark.name == "parametrize":
                kwargs[mark.args[0]] = mark.args[1][0]
        assert set(kwargs) == set(inspect.signature(fn).parameters), name
        out.append((name, fn, kwargs))
    return out


def _failing_pins():
    failed = []
    for name, fn, kwargs in _pins():
        with warnings.catch_warnings(), np.errstate(all="ignore"):
            warnings.simplefilter("ignore")
            try:
                fn(**kwargs)
            except Exception:  # an assertion, or an error the mistake causes
                failed.append(name)
    return failed


def test_every_pin_passes_on_the_untouched_oracle():
    assert len(_pins()) >= 20
    assert _failing_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_a_pin_catches_the_planted_mistake(mutant, monkeypatch):
    for attr, fn in MUTANTS[mutant].items():
        monkeypatch.setattr(osw, attr, fn)     # the oracle's own callers
        monkeypatch.setattr(oracle, attr, fn)  # the pins' view of it
    assert _failing_pins(), f"no pin fails with the planted mistake: {mutant}"
