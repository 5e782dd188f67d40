"""CPU tests: the oracle against its pins, and planted mistakes that the pins must catch."""
import numpy as np
import pytest

import oracle.moe_oracle as orc
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(orc)


# ---------------------------------------------------------------- planted mistakes
# Each entry replaces one oracle function by a plausible wrong version; some pin
# must then fail. The mistakes live only here, in the CPU tests.

f64, _int = orc.f64, orc._int


def _gate_transposed(x, w_router, bias=None):
    L = f64(x) @ f64(w_router)  # wrong operand orientation
    return L if bias is None else L + f64(bias)


def _gate_transposed2(x, w_router, bias=None):
    return (f64(w_router) @ f64(x).T).T[:, ::-1] + (0 if bias is None else f64(bias))


def _gate_no_bias(x, w_router, bias=None):
    return f64(x) @ f64(w_router).T


def _softmax_no_shift(logits):
    z = np.exp(f64(logits))
    return z / z.sum(-1, keepdims=True)


def _softmax_sign(logits):
    L = f64(logits)
    z = np.exp(-(L - L.max(-1, keepdims=True)))
    return z / z.sum(-1, keepdims=True)


def _topk_high_id(logits, k):
    L = f64(logits)
    ids = np.broadcast_to(np.arange(L.shape[1]), L.shape)
    return np.lexsort((-ids, -L), axis=-1)[:, :k]


def _topk_ascending(logits, k):
    L = f64(logits)
    ids = np.broadcast_to(np.arange(L.shape[1]), L.shape)
    return np.lexsort((ids, L), axis=-1)[:, :k]


def _renorm_none(probs, idx):
    return np.take_along_axis(f64(probs), _int(idx), axis=-1)


def _permute_unstable(idx, E):
    I = _int(idx)
    T, k = I.shape
    flat = I.reshape(-1)
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.bincount(flat, minlength=E))
    order = np.lexsort((-np.arange(T * k), flat))
    row_of = np.empty(T * k, dtype=np.int64)
    row_of[order] = np.arange(T * k)
    return off, row_of.reshape(T, k), order // k


def _gather_shift(x, row_src):
    return f64(x)[(_int(row_src) + 1) % f64(x).shape[0]]


def _silu_sign(g):
    g = f64(g)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(g))


def _swiglu_swapped(X, wg, wu, wd):
    X = f64(X)
    G, U = X @ f64(wu).T, X @ f64(wg).T
    H = orc.silu(G) * U
    return H, H @ f64(wd).T


def _swiglu_no_act(X, wg, wu, wd):
    X = f64(X)
    H = (X @ f64(wg).T) * (X @ f64(wu).T)
    return H, H @ f64(wd).T


def _combine_slot_reversed(Y, row_of, w):
    Yv, R, W = f64(Y), _int(row_of), f64(w)
    T, k = R.shape
    out = np.zeros((T, Yv.shape[1]))
    for j in range(k):
        out += W[:, k - 1 - j:k - j] * Yv[R[:, j]]
    return out


def _combine_unweighted(Y, row_of, w):
    Yv, R = f64(Y), _int(row_of)
    return sum(Yv[R[:, j]] for j in range(R.shape[1])) / R.shape[1]


MUTANTS = {
    "gate_transposed": ("gate_logits", _gate_transposed),
    "gate_transposed_reordered": ("gate_logits", _gate_transposed2),
    "gate_no_bias": ("gate_logits", _gate_no_bias),
    "softmax_no_shift": ("softmax", _softmax_no_shift),
    "softmax_sign": ("softmax", _softmax_sign),
    "topk_ties_high_id": ("topk_indices", _topk_high_id),
    "topk_ascending": ("topk_indices", _topk_ascending),
    "renormalise_missing": ("renormalise", _renorm_none),
    "permute_unstable": ("permute", _permute_unstable),
    "gather_shifted": ("gather", _gather_shift),
    "silu_sign": ("silu", _silu_sign),
    "swiglu_gate_up_swapped": ("expert_swiglu", _swiglu_swapped),
    "swiglu_no_activation": ("expert_swiglu", _swiglu_no_act),
    "combine_slot_reversed": ("combine", _combine_slot_reversed),
    "combine_unweighted": ("combine", _combine_unweighted),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(orc)
        except Exception as exc:  # AssertionError, or a shape error from the wrong operand
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
