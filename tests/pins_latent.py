"""Pins of the LatentMoE oracle against facts that do not come from it: bf16
rounding at known ties, RMSNorm closed forms, a hand-worked scalar layer,
reduction to the (separately pinned) plain routed layer, and shared experts
checked against torch float64.

Each pin takes the oracle module `lat` (or a copy with a planted mistake) and
raises AssertionError on failure.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.moe_oracle as orc


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max |diff| {err} > {tol}"


def _torch_swiglu(X, wg, wu, wd):
    X, wg, wu, wd = (torch.as_tensor(np.asarray(v, dtype=np.float64)) for v in (X, wg, wu, wd))
    return (torch.nn.functional.silu(X @ wg.T) * (X @ wu.T)) @ wd.T


def pin_bf16_round_ties(lat):
    """bf16 keeps 8 significant bits: at 1 the spacing is 2^-7. 1 + 2^-8 is a tie
    and goes to the even neighbour 1; 1 + 3*2^-8 ties between 1 + 2^-7 (odd) and
    1 + 2^-6 (even); just above a tie rounds up; signs are symmetric."""
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 3 * 2 ** -8), 3.0, 0.0])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -(1 + 2 ** -6), 3.0, 0.0])
    _close(lat.bf16_round(v), want, 0.0, "bf16 ties")


def pin_rmsnorm_closed_forms(lat):
    """Constant rows normalise to sign(c) * g (eps = 0); [3, 4] has mean square 12.5;
    the output has unit RMS for g = 1, eps = 0; scaling u by a > 0 changes nothing
    (eps = 0); u = 0 stays 0 for eps > 0; eps sits inside the square root."""
    g = np.array([2.0, -1.0, 0.5])
    _close(lat.rmsnorm(np.array([[-4.0, -4.0, -4.0]]), g, 0.0), [[-2.0, 1.0, -0.5]], 1e-15, "constant row")
    _close(lat.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.0), [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]],
           1e-15, "3-4 row")
    u = _rng(1).standard_normal((5, 16))
    r = lat.rmsnorm(u, np.ones(16), 0.0)
    _close(np.sqrt(np.mean(r * r, axis=-1)), np.ones(5), 1e-14, "unit RMS")
    _close(lat.rmsnorm(7.5 * u, np.ones(16), 0.0), r, 1e-14, "scale invariance")
    _close(lat.rmsnorm(np.zeros((2, 4)), np.ones(4), 1e-6), np.zeros((2, 4)), 0.0, "zero row")
    _close(lat.rmsnorm(np.array([[1.0, 1.0]]), np.ones(2), 3.0), [[0.5, 0.5]], 1e-15, "eps inside the root")


def pin_latent_scalar_by_hand(lat):
    """d = 2, l = 1, E = k = 1, h = 1, no shared experts: x = (1, 2), W_down_proj = (1, 1)
    gives z = 3; the expert gives u = silu(3) * 2 * 3 * 1 > 0; RMSNorm of a positive
    scalar with gain 2 and eps = 0 is exactly 2 whatever u is; W_up_proj = (0.5, -1)^T
    then gives out = (1, -2). With eps = u^2 * 3 the norm halves: out = (0.5, -1)."""
    x = np.array([[1.0, 2.0]])
    wr = np.array([[0.3, -0.2]])
    wpd = np.array([[1.0, 1.0]])
    wg, wu, wd = np.array([[[1.0]]]), np.array([[[2.0]]]), np.array([[[1.0]]])
    wpu = np.array([[0.5], [-1.0]])
    none = np.zeros((0, 1, 2)), np.zeros((0, 1, 2)), np.zeros((0, 2, 1))
    res = lat.latent_forward(x, wr, None, wpd, wg, wu, wd, np.array([2.0]), 0.0, wpu, *none, k=1,
                             bf16_operands=False)
    u = 3.0 / (1.0 + math.exp(-3.0)) * 6.0
    _close(res["z"], [[3.0]], 1e-15, "z")
    _close(res["u"], [[u]], 1e-12, "u")
    _close(res["out"], [[1.0, -2.0]], 1e-15, "out")
    res = lat.latent_forward(x, wr, None, wpd, wg, wu, wd, np.array([2.0]), 3.0 * u * u, wpu, *none, k=1,
                             bf16_operands=False)
    _close(res["out"], [[0.5, -1.0]], 1e-12, "out with eps")


def _plain_layer(r, T, d, E, k, h):
    x = r.standard_normal((T, d))
    wr = r.standard_normal((E, d)) / math.sqrt(d)
    wg = r.standard_normal((E, h, d)) / math.sqrt(d)
    wu = r.standard_normal((E, h, d)) / math.sqrt(d)
    wd = r.standard_normal((E, d, h)) / math.sqrt(h)
    return x, wr, wg, wu, wd


def pin_latent_identity_projections(lat):
    """l = d, W_down_proj = W_up_proj = I, g = 1, eps = 0, no shared experts, no
    rounding: the layer is RMSNorm of the plain routed layer's output."""
    r = _rng(2)
    T, d, E, k, h = 11, 6, 5, 2, 4
    x, wr, wg, wu, wd = _plain_layer(r, T, d, E, k, h)
    I = np.eye(d)
    none = np.zeros((0, h, d)), np.zeros((0, h, d)), np.zeros((0, d, h))
    res = lat.latent_forward(x, wr, None, I, wg, wu, wd, np.ones(d), 0.0, I, *none, k=k, bf16_operands=False)
    plain = orc.forward(x, wr, None, wg, wu, wd, k)["out"]
    ms = np.mean(plain * plain, axis=-1, keepdims=True)
    _close(res["out"], plain / np.sqrt(ms), 1e-12, "identity projections")


def pin_latent_shared_experts(lat):
    """Routed down weights of zero make u = 0 and (eps > 0) the routed branch 0: the
    output is the sum of the shared SwiGLU experts on x (torch float64); the router
    reads x, so its choice ignores W_down_proj."""
    r = _rng(3)
    T, d, l, E, k, h, S, hs = 9, 8, 4, 6, 2, 5, 2, 7
    x = r.standard_normal((T, d))
    wr = r.standard_normal((E, d))
    wpd = r.standard_normal((l, d))
    wg, wu = r.standard_normal((E, h, l)), r.standard_normal((E, h, l))
    wd = np.zeros((E, l, h))
    sg, su, sd = r.standard_normal((S, hs, d)), r.standard_normal((S, hs, d)), r.standard_normal((S, d, hs))
    wpu = r.standard_normal((d, l))
    res = lat.latent_forward(x, wr, None, wpd, wg, wu, wd, np.ones(l), 1e-6, wpu, sg, su, sd, k=k,
                             bf16_operands=False)
    want = sum(_torch_swiglu(x, sg[s], su[s], sd[s]).numpy() for s in range(S))
    _close(res["out"], want, 1e-12, "shared experts only")
    res2 = lat.latent_forward(x, wr, None, 3.0 * wpd, wg, wu, wd, np.ones(l), 1e-6, wpu, sg, su, sd, k=k,
                              bf16_operands=False)
    assert np.array_equal(res["idx"], res2["idx"]), "the router must read x, not z"
    assert np.array_equal(res["idx"], orc.topk_indices(x @ wr.T, k))


def pin_latent_up_projection_linear(lat):
    """The routed branch enters linearly through W_up_proj (2 W_up_proj doubles
    out - shared) and the shared experts add on top."""
    r = _rng(4)
    T, d, l, E, k, h, S, hs = 7, 8, 6, 4, 2, 3, 1, 5
    x = r.standard_normal((T, d))
    args = [r.standard_normal((E, d)), None, r.standard_normal((l, d)), r.standard_normal((E, h, l)),
            r.standard_normal((E, h, l)), r.standard_normal((E, l, h)), 1.0 + 0.1 * r.standard_normal(l), 1e-5]
    wpu = r.standard_normal((d, l))
    sh = r.standard_normal((S, hs, d)), r.standard_normal((S, hs, d)), r.standard_normal((S, d, hs))
    a = lat.latent_forward(x, *args, wpu, *sh, k=k, bf16_operands=False)
    b = lat.latent_forward(x, *args, 2.0 * wpu, *sh, k=k, bf16_operands=False)
    shared = _torch_swiglu(x, sh[0][0], sh[1][0], sh[2][0]).numpy()
    _close(b["out"] - shared, 2.0 * (a["out"] - shared), 1e-11, "linear in W_up_proj")
    _close(a["out"] - a["up"], shared, 1e-12, "shared added at full width")


def pin_latent_rounding_points(lat):
    """With bf16 operands, z, the experts' H and RMSNorm(u) are bf16 values (fixed by
    rounding), the routed experts' rows equal the plain layer's expert FFN on bf16
    H by torch float64, and the result stays near the unrounded layer."""
    r = _rng(5)
    T, d, l, E, k, h = 10, 8, 4, 5, 2, 6
    x = r.standard_normal((T, d))
    args = [r.standard_normal((E, d)), None, r.standard_normal((l, d)) / math.sqrt(d),
            r.standard_normal((E, h, l)) / 2, r.standard_normal((E, h, l)) / 2, r.standard_normal((E, l, h)) / 2,
            np.ones(l), 1e-6, r.standard_normal((d, l)) / 2]
    none = np.zeros((0, 2, d)), np.zeros((0, 2, d)), np.zeros((0, d, 2))
    a = lat.latent_forward(x, *args, *none, k=k, bf16_operands=True)
    b = lat.latent_forward(x, *args, *none, k=k, bf16_operands=False)
    for name in ("z", "r", "H"):
        v = a[name][~np.isnan(a[name])]
        _close(lat.bf16_round(v), v, 0.0, f"{name} is bf16")
    _close(a["z"], b["z"], 2.0 ** -8 * np.abs(b["z"]).max(), "z rounding")
    # one routed expert by torch: H = bf16(silu(z Wg^T) * z Wu^T), Y = H Wd^T
    off, row_src = a["offsets"], a["row_src"]
    e = int(np.argmax(np.diff(off)))
    Z = torch.as_tensor(a["z"][row_src[off[e]:off[e + 1]]])
    wg, wu, wd = (torch.as_tensor(np.asarray(v[e], dtype=np.float64)) for v in args[3:6])
    Ht = (torch.nn.functional.silu(Z @ wg.T) * (Z @ wu.T)).float().to(torch.bfloat16).double()
    _close(a["H"][off[e]:off[e + 1]], Ht.numpy(), 0.0, "routed H")
    _close(a["Y"][off[e]:off[e + 1]], (Ht @ wd.T).numpy(), 1e-12, "routed Y")
    assert np.abs(a["out"] - b["out"]).max() < 0.05 * np.abs(b["out"]).max()
    assert not np.array_equal(a["out"], b["out"])


ALL_PINS = [
    pin_bf16_round_ties,
    pin_rmsnorm_closed_forms,
    pin_latent_scalar_by_hand,
    pin_latent_identity_projections,
    pin_latent_shared_experts,
    pin_latent_up_projection_linear,
    pin_latent_rounding_points,
]
