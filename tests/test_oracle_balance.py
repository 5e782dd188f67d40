"""CPU tests: the load-balancing oracle against its pins, and planted mistakes
that the pins must catch."""
import numpy as np
import pytest

import oracle.balance as bal
from tests import pins_balance as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_balance_pin(pin):
    pin(bal)


# ---------------------------------------------------------------- planted mistakes

def _aux_no_uniform(probs):
    m = bal.expert_prob_mean(probs)
    return float(np.sum(m ** 2)), m


def _aux_abs(probs):
    m = bal.expert_prob_mean(probs)
    return float(np.sum(np.abs(m - 1.0 / m.shape[0]))), m


def _prob_mean_over_experts(probs):
    P = bal._f64(probs)
    return P.mean(axis=1)[: P.shape[1]] if P.shape[0] >= P.shape[1] else P.mean(axis=1)


def _select_k_cutoff(logits, bias, k):
    idx, _ = _real_select(logits, bias, k)
    S = (bal._f32(logits) + bal._f32(bias)[None]).astype(np.float32)
    return idx, np.take_along_axis(S, idx[:, k - 1:k], axis=-1)[:, 0]


def _select_unbiased(logits, bias, k):
    return _real_select(logits, np.zeros_like(bal._f32(bias)), k)


def _select_float64(logits, bias, k):
    S = bal._f64(logits) + bal._f64(bias)[None]
    T, E = S.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -S), axis=-1)[:, :k + 1]
    return order[:, :k], np.take_along_axis(S, order[:, k:k + 1], axis=-1)[:, 0].astype(np.float32)


def _select_high_id(logits, bias, k):
    S = (bal._f32(logits) + bal._f32(bias)[None]).astype(np.float32)
    T, E = S.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((-ids, -S.astype(np.float64)), axis=-1)[:, :k + 1]
    return order[:, :k], np.take_along_axis(S, order[:, k:k + 1], axis=-1)[:, 0]


def _weights_plain(logits, idx):
    sel = np.take_along_axis(bal._f64(logits), bal._i64(idx), axis=-1)
    return sel / sel.sum(-1, keepdims=True)


def _margins_reversed(logits, alpha):
    return (bal._f32(alpha)[:, None] - bal._f32(logits)).astype(np.float32)


def _bin_round(margins, lo, width, n_bins):
    M = np.asarray(margins, np.float32)
    u = np.rint((M - np.float32(lo)) / np.float32(width))
    return np.clip(np.nan_to_num(u), 0, n_bins - 1).astype(np.int64)


def _quantile_lower_edge(hist, k, lo, width):
    Q = _real_quantile(hist, k, lo, width)
    return lo + width * np.floor((Q - lo) / width - 1e-12)


def _quantile_wrong_p(hist, k, lo, width):
    E = np.asarray(hist).shape[0]
    return _real_quantile(hist, E - k, lo, width)


def _quantile_from_top(hist, k, lo, width):
    H = bal._i64(hist)[:, ::-1]
    B = H.shape[1]
    return lo + width * B - (_real_quantile(H, k, 0.0, width))


def _update_plus(hist, k, lo, width, bias_in):
    Q = bal.qb_quantile(hist, k, lo, width)
    b = bal._f32(bias_in).astype(np.float64)
    return np.where(np.isnan(Q), b, Q).astype(np.float32)


def _update_reset(hist, k, lo, width, bias_in):
    Q = bal.qb_quantile(hist, k, lo, width)
    return np.where(np.isnan(Q), 0.0, -Q).astype(np.float32)


_real_select = bal.qb_select
_real_quantile = bal.qb_quantile

MUTANTS = {
    "aux_no_uniform_share": ("aux_loss", _aux_no_uniform),
    "aux_abs_not_square": ("aux_loss", _aux_abs),
    "prob_mean_over_experts": ("expert_prob_mean", _prob_mean_over_experts),
    "select_cutoff_is_kth": ("qb_select", _select_k_cutoff),
    "select_ignores_bias": ("qb_select", _select_unbiased),
    "select_sum_in_float64": ("qb_select", _select_float64),
    "select_ties_high_id": ("qb_select", _select_high_id),
    "weights_not_softmax": ("qb_weights", _weights_plain),
    "margins_reversed": ("qb_margins", _margins_reversed),
    "bin_rounds": ("qb_bin", _bin_round),
    "quantile_lower_edge": ("qb_quantile", _quantile_lower_edge),
    "quantile_wrong_p": ("qb_quantile", _quantile_wrong_p),
    "quantile_from_top": ("qb_quantile", _quantile_from_top),
    "update_plus_sign": ("qb_update", _update_plus),
    "update_resets_empty_rows": ("qb_update", _update_reset),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_balance_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(bal, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bal)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
