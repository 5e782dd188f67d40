"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin takes an oracle namespace `orc` (the real module, or a copy with a
planted mistake in the mutation tests) and raises AssertionError on failure.
The expected values come from brute force over tiny inputs, closed forms,
special cases that reduce to an independent library routine (torch float64
on the CPU), invariants, and the hand-derived worked example in
tests/golden/worked_example.json.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, np.max(np.abs(b)) if b.size else 0.0)
    assert err <= tol * scale, f"{what}: max |diff| {err} > {tol * scale}"


# ------------------------------------------------------------------ gate logits

def pin_gate_onehot(orc):
    """One-hot tokens read out one input column of the gate: logits[t, e] = W[e, i_t].
    E != d so a transposed operand cannot pass."""
    r = _rng(1)
    E, d = 5, 7
    W = r.standard_normal((E, d))
    cols = [3, 0, 6, 2]
    x = np.zeros((len(cols), d))
    for t, i in enumerate(cols):
        x[t, i] = 1.0
    L = orc.gate_logits(x, W)
    _close(L, np.stack([W[:, i] for i in cols]), what="one-hot gate")


def pin_gate_bias_and_linearity(orc):
    """x = 0 gives the bias alone; the logits are linear in x (2x -> 2L - b)."""
    r = _rng(2)
    E, d, T = 6, 4, 3
    W = r.standard_normal((E, d))
    b = r.standard_normal(E)
    _close(orc.gate_logits(np.zeros((T, d)), W, b), np.broadcast_to(b, (T, E)), what="bias only")
    x = r.standard_normal((T, d))
    L1 = orc.gate_logits(x, W, b)
    L2 = orc.gate_logits(2 * x, W, b)
    _close(L2, 2 * L1 - b, tol=1e-12, what="linearity")
    # a single product by hand: one token, one expert, d = 2
    _close(orc.gate_logits(np.array([[2.0, -3.0]]), np.array([[0.5, 0.25]]), np.array([1.0])),
           [[2.0 * 0.5 - 3.0 * 0.25 + 1.0]], what="hand product")


# ----------------------------------------------------------------------- softmax

def pin_softmax_closed_forms(orc):
    """Two experts: p = (sigmoid(a-b), sigmoid(b-a)); equal logits: 1/E; softmax(ln n_e) = n_e / sum n."""
    for a, b in [(0.3, -1.2), (5.0, 5.0), (-2.0, 7.5)]:
        p = orc.softmax(np.array([[a, b]]))
        s = 1.0 / (1.0 + math.exp(-(a - b)))
        _close(p, [[s, 1.0 - s]], tol=1e-14, what="two-expert softmax")
    _close(orc.softmax(np.full((2, 7), 0.7)), np.full((2, 7), 1.0 / 7), tol=1e-14, what="uniform")
    n = np.array([3.0, 1.0, 2.0, 6.0])
    _close(orc.softmax(np.log(n)[None]), (n / n.sum())[None], tol=1e-14, what="log counts")


def pin_softmax_large_logits(orc):
    """Shift invariance, and no overflow for logits near the float64 exp limit."""
    L = np.array([[1000.0, 999.0, 998.0]])
    p = orc.softmax(L)
    assert np.all(np.isfinite(p)), "softmax overflowed"
    _close(p, orc.softmax(L - 1000.0), tol=1e-14, what="shift")


# ------------------------------------------------------------------------ top-k

def _brute_topk(L, k):
    T, E = L.shape
    return np.array([sorted(range(E), key=lambda e: (-L[t, e], e))[:k] for t in range(T)], dtype=np.int64)


def pin_topk_bruteforce(orc):
    r = _rng(3)
    for (T, E, k) in [(9, 8, 2), (5, 13, 5), (4, 6, 6), (7, 1, 1)]:
        L = r.standard_normal((T, E))
        assert np.array_equal(orc.topk_indices(L, k), _brute_topk(L, k)), (T, E, k)
    # planted ties: few distinct values, +-0.0, all equal
    L = r.integers(-2, 3, size=(40, 10)).astype(np.float64)
    L[0] = 0.0
    L[1, ::2] = -0.0
    L[2] = np.array([1, -0.0, 0.0, -0.0, 1, 2, 2, -1, 0.0, 2])
    for k in (1, 3, 10):
        got = orc.topk_indices(L, k)
        assert np.array_equal(got, _brute_topk(L, k)), k
    assert list(orc.topk_indices(L, 10)[0]) == list(range(10))
    assert list(orc.topk_indices(L[2:3], 6)[0]) == [5, 6, 9, 0, 4, 1]  # -0.0 ties +0.0 -> lower id


def pin_topk_exhaustive_tiny(orc):
    """Every logit vector over {-1, 0, 1}^4: the chosen set is the k largest, lower id first."""
    vals = [-1.0, 0.0, 1.0]
    rows = np.array(list(itertools.product(vals, repeat=4)))
    for k in (1, 2, 3):
        assert np.array_equal(orc.topk_indices(rows, k), _brute_topk(rows, k)), k


# ---------------------------------------------------------------- route weights

def pin_route_closed_forms(orc):
    """Zero logits -> experts 0..k-1 with weight 1/k; k = 2 -> w0 = sigmoid(l_top1 - l_top2);
    weights sum to one and do not increase with the slot."""
    idx, w, _ = orc.route(np.zeros((3, 9)), 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (3, 1)))
    _close(w, np.full((3, 4), 0.25), tol=1e-15, what="zero router")
    L = np.array([[0.1, 2.0, -1.0, 1.5]])
    idx, w, _ = orc.route(L, 2)
    assert list(idx[0]) == [1, 3]
    s = 1.0 / (1.0 + math.exp(-(2.0 - 1.5)))
    _close(w, [[s, 1.0 - s]], tol=1e-14, what="k=2 weights")
    r = _rng(4)
    L = r.standard_normal((50, 16)) * 3
    idx, w, p = orc.route(L, 5)
    _close(w.sum(-1), np.ones(50), tol=1e-14, what="sum to one")
    assert np.all(np.diff(w, axis=-1) <= 1e-15), "weights increase with slot"
    # renormalised weights are proportional to the selected probabilities
    sel = np.take_along_axis(p, idx, axis=-1)
    _close(w / w[:, :1], sel / sel[:, :1], tol=1e-12, what="proportional")


# ------------------------------------------------------------------ permutation

def _brute_perm(idx, E):
    T, k = idx.shape
    flat = idx.reshape(-1)
    order = sorted(range(T * k), key=lambda a: (flat[a], a))
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + int(np.sum(flat == e)))
    row_src = [a // k for a in order]
    row_of = [0] * (T * k)
    for r, a in enumerate(order):
        row_of[a] = r
    return np.array(offsets), np.array(row_of).reshape(T, k), np.array(row_src)


def pin_permute_bruteforce(orc):
    r = _rng(5)
    for (T, E, k) in [(13, 6, 3), (1, 4, 4), (30, 17, 2), (8, 3, 1)]:
        idx = np.stack([r.permutation(E)[:k] for _ in range(T)])
        off, row_of, row_src = orc.permute(idx, E)
        boff, brow_of, brow_src = _brute_perm(idx, E)
        assert np.array_equal(off, boff) and np.array_equal(row_of, brow_of) and np.array_equal(row_src, brow_src)
        # invariants
        assert off[-1] == T * k
        for t in range(T):
            for j in range(k):
                rr = row_of[t, j]
                assert row_src[rr] == t and off[idx[t, j]] <= rr < off[idx[t, j] + 1]
        for e in range(E):
            seg = row_src[off[e]:off[e + 1]]
            assert np.all(np.diff(seg) > 0), "rows of an expert not in token order"
    # an expert nobody picked has an empty segment
    off, _, _ = orc.permute(np.array([[2, 0], [0, 2]]), 4)
    assert list(off) == [0, 2, 2, 4, 4]


def pin_gather(orc):
    r = _rng(6)
    x = r.standard_normal((5, 3))
    row_src = np.array([4, 0, 0, 2, 1, 4])
    xp = orc.gather(x, row_src)
    for rr, t in enumerate(row_src):
        assert np.array_equal(xp[rr], x[t])


# ------------------------------------------------------------------------ SwiGLU

def pin_silu_closed_forms(orc):
    ln3 = math.log(3.0)
    _close(orc.silu(np.array([0.0, ln3, -ln3])), [0.0, 0.75 * ln3, -0.25 * ln3], tol=1e-15, what="silu")
    big = orc.silu(np.array([800.0, -800.0, 40.0]))
    assert np.all(np.isfinite(big))
    _close(big, [800.0, 0.0, 40.0], tol=1e-15, what="silu tails")


def _torch_ffn(X, wg, wu, wd):
    X, wg, wu, wd = (torch.as_tensor(np.asarray(a, dtype=np.float64)) for a in (X, wg, wu, wd))
    return torch.matmul(torch.nn.functional.silu(torch.matmul(X, wg.t())) * torch.matmul(X, wu.t()), wd.t()).numpy()


def pin_expert_swiglu_vs_torch(orc):
    """One expert against torch's float64 silu and matmul (h != d catches a transposed operand)."""
    r = _rng(7)
    M, d, h = 6, 5, 9
    X, wg, wu, wd = r.standard_normal((M, d)), r.standard_normal((h, d)), r.standard_normal((h, d)), r.standard_normal((d, h))
    H, Y = orc.expert_swiglu(X, wg, wu, wd)
    _close(Y, _torch_ffn(X, wg, wu, wd), tol=1e-12, what="swiglu vs torch")
    Ht = (torch.nn.functional.silu(torch.as_tensor(X @ wg.T)) * torch.as_tensor(X @ wu.T)).numpy()
    _close(H, Ht, tol=1e-12, what="H vs torch")


# -------------------------------------------------------------- whole-layer cases

def _layer(r, T, d, E, k, h, scale=1.0):
    x = r.standard_normal((T, d))
    wr = r.standard_normal((E, d)) * scale / math.sqrt(d)
    wg = r.standard_normal((E, h, d)) / math.sqrt(d)
    wu = r.standard_normal((E, h, d)) / math.sqrt(d)
    wd = r.standard_normal((E, d, h)) / math.sqrt(h)
    return x, wr, wg, wu, wd


def pin_identical_experts_dense(orc):
    """All experts equal -> the layer is one dense SwiGLU FFN (weights sum to one)."""
    r = _rng(8)
    T, d, E, k, h = 11, 6, 7, 3, 10
    x, wr, wg, wu, wd = _layer(r, T, d, E, k, h, scale=3.0)
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    res = orc.forward(x, wr, None, wg, wu, wd, k)
    _close(res["out"], _torch_ffn(x, wg[0], wu[0], wd[0]), tol=1e-12, what="identical experts")


def pin_k_equals_E_mixture(orc):
    """k = E -> out[t] = sum_e softmax(x W_r^T)[t, e] * FFN_e(x[t]), brute force over every expert."""
    r = _rng(9)
    T, d, E, h = 7, 5, 4, 6
    x, wr, wg, wu, wd = _layer(r, T, d, E, E, h, scale=2.0)
    b = r.standard_normal(E)
    res = orc.forward(x, wr, b, wg, wu, wd, E)
    xt = torch.as_tensor(x)
    p = torch.softmax(xt @ torch.as_tensor(wr).t() + torch.as_tensor(b), dim=-1).numpy()
    ref = np.zeros((T, d))
    for e in range(E):
        ref += p[:, e:e + 1] * _torch_ffn(x, wg[e], wu[e], wd[e])
    _close(res["out"], ref, tol=1e-12, what="k = E mixture")


def pin_single_expert_dense(orc):
    """E = k = 1 -> dense FFN with weight exactly 1."""
    r = _rng(10)
    x, wr, wg, wu, wd = _layer(r, 5, 4, 1, 1, 8)
    res = orc.forward(x, wr, None, wg, wu, wd, 1)
    assert np.all(res["w"] == 1.0)
    _close(res["out"], _torch_ffn(x, wg[0], wu[0], wd[0]), tol=1e-12, what="E = k = 1")


def pin_zero_down_and_equivariance(orc):
    """W_down = 0 -> out = 0 exactly; permuting tokens permutes the output rows."""
    r = _rng(11)
    T, d, E, k, h = 9, 4, 6, 2, 5
    x, wr, wg, wu, wd = _layer(r, T, d, E, k, h)
    res0 = orc.forward(x, wr, None, wg, wu, np.zeros_like(wd), k)
    assert np.all(res0["out"] == 0.0)
    perm = r.permutation(T)
    a = orc.forward(x, wr, None, wg, wu, wd, k)["out"]
    b = orc.forward(x[perm], wr, None, wg, wu, wd, k)["out"]
    _close(b, a[perm], tol=1e-12, what="token equivariance")


def _expr(v):
    if isinstance(v, str):
        neg = v.startswith("-")
        s = v.lstrip("-")
        val = {"ln3": math.log(3.0), "ln2": math.log(2.0)}.get(s)
        if val is None:
            val = float(s)
        return -val if neg else val
    return float(v)


def load_worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        j = json.load(f)
    conv = lambda a: np.vectorize(_expr, otypes=[np.float64])(np.array(a, dtype=object))  # noqa: E731
    return j, conv(j["logits"]), conv(j["x"]), conv(j["w_gate"]), conv(j["w_up"]), conv(j["w_down"])


def pin_worked_example(orc):
    j, L, x, wg, wu, wd = load_worked_example()
    ex = j["expected"]
    ln3 = math.log(3.0)
    E = j["shape"]["E"]
    res = orc.forward(x, np.zeros((E, x.shape[1])), None, wg, wu, wd, j["shape"]["k"], logits=L)
    _close(res["probs"][0], ex["probs_token0"], tol=1e-15, what="probs")
    assert np.array_equal(res["idx"], ex["idx"])
    _close(res["w"], ex["w"], tol=1e-15, what="w")
    assert np.array_equal(res["offsets"], ex["offsets"])
    assert np.array_equal(res["row_src"], ex["row_src"])
    assert np.array_equal(res["row_of"], ex["row_of"])
    _close(res["H"], np.array(ex["H_in_ln3"]) * ln3, tol=1e-15, what="H")
    _close(res["Y"], np.array(ex["Y_in_ln3"]) * ln3, tol=1e-15, what="Y")
    _close(res["out"], np.array(ex["out_in_ln3"]) * ln3, tol=1e-15, what="out")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
