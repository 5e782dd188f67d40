"""Pins of the load-balancing oracle (aux loss and Quantile Balancing) against
facts that do not come from the oracle itself: closed forms, hand-worked
grouped-data quantiles, brute force over tiny inputs, a library quantile, and
the property QB exists for -- the bias it produces evens out the expert loads.

Each pin takes an oracle namespace `bal` (the real module, or a copy with a
planted mistake in the mutation tests) and raises AssertionError on failure.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max |diff| {err} > {tol}"


def _softmax64(L):
    return torch.softmax(torch.as_tensor(np.asarray(L, dtype=np.float64)), dim=-1).numpy()


# --------------------------------------------------------------------- aux loss

def pin_aux_closed_forms(bal):
    """Equal logits: every mean is 1/E and the loss is 0. Every token certain of
    expert 0: means (1, 0, ..., 0), loss (1 - 1/E)^2 + (E - 1)/E^2 = (E - 1)/E.
    Two experts: loss = 2 (mean p_0 - 1/2)^2 with p_0 = sigmoid(l_0 - l_1)."""
    loss, m = bal.aux_loss(_softmax64(np.full((5, 7), 0.3)))
    _close(m, np.full(7, 1.0 / 7), 1e-15, "uniform means")
    _close(loss, 0.0, 1e-15, "uniform loss")
    for E in (2, 5, 64):
        P = np.zeros((9, E))
        P[:, 0] = 1.0
        loss, m = bal.aux_loss(P)
        _close(loss, (E - 1) / E, 1e-14, f"one-hot loss E={E}")
    l = np.array([[0.4, -1.1], [2.0, 0.5], [-0.3, -0.3]])
    p0 = 1.0 / (1.0 + np.exp(-(l[:, 0] - l[:, 1])))
    loss, m = bal.aux_loss(_softmax64(l))
    _close(m, [p0.mean(), 1.0 - p0.mean()], 1e-15, "two-expert means")
    _close(loss, 2.0 * (p0.mean() - 0.5) ** 2, 1e-15, "two-expert loss")


def pin_aux_balanced_and_identity(bal):
    """T = E tokens, token t peaked on expert t: by symmetry every expert's mean
    is 1/E and the loss vanishes. In general, since the means sum to one, the
    loss equals sum_e mean_e^2 - 1/E, and the means are the batch averages."""
    E = 12
    loss, m = bal.aux_loss(_softmax64(3.0 * np.eye(E)))
    _close(m, np.full(E, 1.0 / E), 1e-15, "balanced means")
    _close(loss, 0.0, 1e-15, "balanced loss")
    P = _softmax64(_rng(11).standard_normal((37, E)) * 2)
    loss, m = bal.aux_loss(P)
    _close(m, [sum(P[t, e] for t in range(37)) / 37 for e in range(E)], 1e-15, "batch average")
    _close(loss, float(np.dot(m, m)) - 1.0 / E, 1e-15, "sum of squares identity")
    assert loss > 0


# ------------------------------------------------------------------ QB select

def _brute_select(L32, b32, k):
    T, E = L32.shape
    idx, alpha = [], []
    for t in range(T):
        score = [np.float32(L32[t, e]) + np.float32(b32[e]) for e in range(E)]  # float32 adds
        order = sorted(range(E), key=lambda e: (-float(score[e]), e))
        idx.append(order[:k])
        alpha.append(score[order[k]])
    return np.array(idx), np.array(alpha, dtype=np.float32)


def pin_qb_select_bruteforce(bal):
    """Zero bias: the plain top-k and the (k+1)-th largest logit; random biases
    and tied scores against a full sort of each token's biased scores."""
    r = _rng(12)
    for (T, E, k) in [(6, 5, 1), (9, 8, 3), (4, 16, 15)]:
        L = r.standard_normal((T, E)).astype(np.float32)
        idx, alpha = bal.qb_select(L, np.zeros(E, np.float32), k)
        order = np.argsort(-L.astype(np.float64), axis=-1, kind="stable")
        assert np.array_equal(idx, order[:, :k]), (T, E, k)
        _close(alpha, np.sort(L, axis=-1)[:, ::-1][:, k], 0.0, "alpha = (k+1)-th logit")
        b = (r.standard_normal(E) * 2).astype(np.float32)
        bi, ba = _brute_select(L, b, k)
        idx, alpha = bal.qb_select(L, b, k)
        assert np.array_equal(idx, bi), (T, E, k)
        _close(alpha, ba, 0.0, "alpha")
    # ties on the biased score go to the lower id
    L = np.array([[1.0, 0.5, 0.25, 0.5]], np.float32)
    b = np.array([-0.5, 0.0, 0.25, 0.0], np.float32)
    idx, alpha = bal.qb_select(L, b, 2)
    assert list(idx[0]) == [0, 1] and alpha[0] == np.float32(0.5), (idx, alpha)


def pin_qb_select_bias_moves_choice(bal):
    """A large bias forces an expert into every token's set; a large negative one
    keeps it out; the sum s + b is rounded to float32 before comparing
    (1 + 2^-24 rounds to 1, so expert 1 then only ties expert 0 and loses)."""
    r = _rng(13)
    L = r.standard_normal((20, 6)).astype(np.float32)
    b = np.zeros(6, np.float32)
    b[4] = 100.0
    idx, _ = bal.qb_select(L, b, 2)
    assert np.all(idx[:, 0] == 4)
    b[4] = -100.0
    idx, alpha = bal.qb_select(L, b, 5)
    assert not np.any(idx == 4)
    _close(alpha, L[:, 4] - 100.0, 1e-5, "excluded expert is the cutoff")
    L = np.array([[1.0, 1.0, 0.0]], np.float32)
    b = np.array([0.0, 2.0 ** -24, 0.0], np.float32)
    idx, alpha = bal.qb_select(L, b, 1)
    assert idx[0, 0] == 0 and alpha[0] == np.float32(1.0), (idx, alpha)


def pin_qb_weights_unbiased(bal):
    """The weights ignore the bias: k = 2 gives w = (sigmoid(s_a - s_b), ...) of the
    unbiased logits, whatever bias brought a and b in, and with zero bias they
    are the softmax probabilities of the chosen experts rescaled to sum to one."""
    L = np.array([[0.2, 1.7, -0.4, 0.9]], np.float32)
    w = bal.qb_weights(L, np.array([[2, 0]]))
    s = 1.0 / (1.0 + math.exp(-(float(L[0, 2]) - float(L[0, 0]))))
    _close(w, [[s, 1.0 - s]], 1e-15, "k=2 weights")
    r = _rng(14)
    L = r.standard_normal((30, 10)).astype(np.float32)
    idx, _ = bal.qb_select(L, np.zeros(10, np.float32), 4)
    P = _softmax64(L)
    sel = np.take_along_axis(P, idx, axis=-1)
    _close(bal.qb_weights(L, idx), sel / sel.sum(-1, keepdims=True), 1e-14, "zero-bias weights")


# ------------------------------------------------------------ margins and bins

def pin_qb_bins_edges(bal):
    """Bins [lo + b w, lo + (b+1) w): an exact edge opens its bin, a value w/1024
    below it falls in the bin before (a single ulp below may round back onto the
    edge in m - lo, which the float32 rule then counts in the upper bin), and
    values outside the range clamp."""
    lo, w, B = -4.0, 0.25, 32
    edges = np.array([lo + b * w for b in range(B)], np.float32)
    assert np.array_equal(bal.qb_bin(edges, lo, w, B), np.arange(B))
    below = (edges[1:] - np.float32(w / 1024)).astype(np.float32)
    assert np.array_equal(bal.qb_bin(below, lo, w, B), np.arange(B - 1))
    far = np.array([-1e30, -4.5, lo + B * w, 1e30, 3.99], np.float32)
    assert list(bal.qb_bin(far, lo, w, B)) == [0, 0, B - 1, B - 1, B - 1]


def pin_qb_histogram_bruteforce(bal):
    """Margins s - alpha counted one by one in pure Python, on a hand-made input,
    and row sums equal to the token count."""
    L = np.array([[0.5, -1.0, 2.0], [0.0, 0.25, -3.0]], np.float32)
    alpha = np.array([0.5, -0.5], np.float32)
    # margins: [[0, -1.5, 1.5], [0.5, 0.75, -2.5]]; lo = -2, w = 0.5, B = 8 -> bins
    # [[4, 1, 7], [5, 5, 0]] (-2.5 clamps to bin 0)
    H = bal.qb_histogram(L, alpha, -2.0, 0.5, 8)
    want = np.zeros((3, 8), np.int64)
    for (t, j, b) in [(0, 0, 4), (0, 1, 1), (0, 2, 7), (1, 0, 5), (1, 1, 5), (1, 2, 0)]:
        want[j, b] += 1
    assert np.array_equal(H, want), H
    r = _rng(15)
    L = r.standard_normal((50, 7)).astype(np.float32)
    _, alpha = bal.qb_select(L, np.zeros(7, np.float32), 2)
    H = bal.qb_histogram(L, alpha, -6.0, 0.05, 200)
    assert np.all(H.sum(axis=1) == 50)
    M = [[float(np.float32(L[t, j]) - np.float32(alpha[t])) for j in range(7)] for t in range(50)]
    for j in range(7):
        for b in (0, 90, 119, 120, 199):
            n = sum(1 for t in range(50) if -6.0 + b * 0.05 <= M[t][j] < -6.0 + (b + 1) * 0.05
                    or (b == 0 and M[t][j] < -6.0) or (b == 199 and M[t][j] >= 4.0))
            assert H[j, b] == n, (j, b, H[j, b], n)


# ------------------------------------------------------------------- quantile

def pin_qb_quantile_grouped_by_hand(bal):
    """Grouped-data quantiles worked by hand. Classes of width 10 from 0 with
    counts 5, 8, 12, 10, 5 (m = 40, cumulative 5, 13, 25, 35, 40):
      E = 2, k = 1 -> p = 1/2, p m = 20, reached in class 20-30 (C = 13, f = 12):
         Q = 20 + (20 - 13) / 12 * 10 = 25.8333...
      E = 4, k = 1 -> p = 3/4, p m = 30, class 30-40 (C = 25, f = 10): Q = 35
      E = 8, k = 7 -> p = 1/8, p m = 5, class 0-10 (C = 0, f = 5): Q = 10
    The update sets the bias to -Q."""
    counts = [5, 8, 12, 10, 5]
    for E, k, q in [(2, 1, 20.0 + 70.0 / 12.0), (4, 1, 35.0), (8, 7, 10.0)]:
        H = np.array([counts] * E)
        _close(bal.qb_quantile(H, k, 0.0, 10.0), np.full(E, q), 1e-12, f"quantile E={E} k={k}")
        _close(bal.qb_update(H, k, 0.0, 10.0, np.zeros(E, np.float32)),
               np.full(E, -q, np.float32), 0.0, "bias = -Q")


def pin_qb_quantile_uniform(bal):
    """One margin per bin spreads the mass evenly over [lo, lo + B w): the
    p-quantile is lo + p B w exactly."""
    lo, w, B = -3.0, 0.125, 64
    H = np.ones((16, B), np.int64)
    for k in (1, 4, 15):
        p = 1.0 - k / 16.0
        _close(bal.qb_quantile(H, k, lo, w), np.full(16, lo + p * B * w), 1e-12, f"uniform k={k}")


def pin_qb_quantile_vs_numpy(bal):
    """On fine bins the histogram quantile lies within one bin width of the exact
    inverted-CDF quantile of the margins (numpy), for several k."""
    r = _rng(16)
    T, E = 3000, 12
    L = (r.standard_normal((T, E)) * 1.5).astype(np.float32)
    lo, w, B = -15.0, 0.01, 3000
    for k in (1, 3, 8):
        _, alpha = bal.qb_select(L, np.zeros(E, np.float32), k)
        H = bal.qb_histogram(L, alpha, lo, w, B)
        M = L.astype(np.float64) - alpha.astype(np.float64)[:, None]
        exact = np.quantile(M, 1.0 - k / E, axis=0, method="inverted_cdf")
        _close(bal.qb_quantile(H, k, lo, w), exact, w * (1 + 1e-9), f"quantile k={k}")


def pin_qb_balances_load(bal):
    """The point of QB: from a Zipf-skewed router (one expert draws about seven
    times its share), a few bias updates bring every expert close to the load
    target T k / E; no update at all leaves it skewed."""
    r = _rng(17)
    T, E, k = 4000, 16, 2
    zipf = (1.5 * np.log(1.0 / np.arange(1, E + 1)))[r.permutation(E)]
    L = (r.standard_normal((T, E)) + zipf[None, :]).astype(np.float32)
    b = np.zeros(E, np.float32)
    target = T * k / E
    loads = []
    for _ in range(9):
        idx, alpha = bal.qb_select(L, b, k)
        loads.append(np.bincount(idx.ravel(), minlength=E) / target)
        b = bal.qb_update(bal.qb_histogram(L, alpha, -12.0, 0.01, 2400), k, -12.0, 0.01, b)
    assert loads[0].max() > 5.0, loads[0]
    assert loads[-1].max() < 1.05 and loads[-1].min() > 0.9, loads[-1]


def pin_qb_update_rules(bal):
    """An empty histogram row keeps its bias. Measuring the margins on the biased
    score and moving the old bias by minus their quantile gives the same bias
    (within one bin) as -Q of the unbiased margins."""
    H = np.zeros((3, 10), np.int64)
    H[1, 4] = 7
    b0 = np.array([0.5, -0.25, 2.0], np.float32)
    out = bal.qb_update(H, 1, 0.0, 1.0, b0)
    assert out[0] == np.float32(0.5) and out[2] == np.float32(2.0), out
    _close(out[1], -(4.0 + (7 * 2 / 3) / 7), 1e-6, "single-bin row")
    r = _rng(18)
    T, E, k = 2000, 8, 2
    L = r.standard_normal((T, E)).astype(np.float32)
    b = (r.standard_normal(E) * 0.7).astype(np.float32)
    lo, w, B = -12.0, 0.005, 4800
    _, alpha = bal.qb_select(L, b, k)
    direct = bal.qb_update(bal.qb_histogram(L, alpha, lo, w, B), k, lo, w, b)
    biased = (L + b[None, :]).astype(np.float32)
    moved = b - bal.qb_quantile(bal.qb_histogram(biased, alpha, lo, w, B), k, lo, w)
    _close(direct, moved, 2 * w, "two readings agree")


ALL_PINS = [
    pin_aux_closed_forms,
    pin_aux_balanced_and_identity,
    pin_qb_select_bruteforce,
    pin_qb_select_bias_moves_choice,
    pin_qb_weights_unbiased,
    pin_qb_bins_edges,
    pin_qb_histogram_bruteforce,
    pin_qb_quantile_grouped_by_hand,
    pin_qb_quantile_uniform,
    pin_qb_quantile_vs_numpy,
    pin_qb_balances_load,
    pin_qb_update_rules,
]
