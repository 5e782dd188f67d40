"""How far the device's Stable LatentMoE output may lie from the float64 layer.

The layer ("Kimi K3: Open Frontier Intelligence", section "Operational
Execution Flow"): z = W_down_proj x, routed SwiGLU experts on z, u = the
gate-weighted sum of their outputs, r = RMSNorm(u), out = W_up_proj r plus the
shared SwiGLU experts on x. The oracle computes it in float64 with no rounding.
The device computes in float32 and rounds three kinds of activation to
bfloat16 before they enter a matrix product: z, every expert's SwiGLU
activation H (routed and shared), and r. Each rounding moves a value by at
most 2^-8 of its magnitude; the question is what that does to the output.

A worst-case answer (absolute values carried through every product) grows by
about sqrt(K) at each K-term product and, after two products, exceeds the
values themselves, so it cannot serve as a tolerance. This module uses the
usual probabilistic model of round to nearest instead: each rounding error is
uniform on +-half a bfloat16 ulp (variance ulp^2 / 12) and independent of the
others. To first order the output error is then a sum of many independent
terms, close to normal, with a standard deviation sigma that follows from the
float64 intermediates:
  * a rounding adds ulp(v)^2 / 12 of variance to v;
  * a linear step y = A v maps variances by A^2 (elementwise square);
  * the SwiGLU step by its Jacobian, dH = silu'(G) U dG + silu(G) dU;
  * the weighted sum by the squared top-k weights;
  * the RMSNorm r = g u / s by its Jacobian g (du / s - u (u . du) / (l s^3)).
Errors of one token's z reach its k experts alike; the model treats the k
expert outputs as independent, which holds on average over weights with
independent entries. float32 summation (2^-24 against 2^-8) is left out.

The test then asks for |out - ref| <= 8 sigma + 1e-6 max|ref| elementwise and
||out - ref||_2 <= 2 ||sigma||_2: a mistake bigger than the rounding noise,
anywhere in the layer, fails one of the two. (All d outputs of a token share
that token's rounding of r, so the elementwise errors are a mixture of
normals whose scale varies by token, 0.7 to 1.5 times sigma, and their tail is
a little heavier than one normal's: 8 sigma rather than 6.) The model itself
is checked on the CPU against the float64 layer with the same three roundings
applied.
"""
from __future__ import annotations

import numpy as np

import oracle.moe_oracle as orc


def ulp_bf16(v) -> np.ndarray:
    """Spacing of bfloat16 numbers at |v| (2^(e - 7) for 2^e <= |v| < 2^(e+1)); 0 at v = 0."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    out = np.zeros_like(a)
    nz = a > 0
    out[nz] = np.exp2(np.floor(np.log2(a[nz])) - 7)
    return out


def _rounding_var(v):
    return ulp_bf16(v) ** 2 / 12


def _silu_grad(g):
    s = 0.5 * (1.0 + np.tanh(0.5 * g))
    return s * (1.0 + g * (1.0 - s))


def swiglu_output_var(X, vX, wg, wu, wd):
    """Variance of a SwiGLU expert's output rows Y = (silu(X Wg^T) * X Wu^T) Wd^T when its
    input rows X carry independent errors of variance vX and H is rounded to bf16."""
    Wg, Wu, Wd = orc.f64(wg), orc.f64(wu), orc.f64(wd)
    G, U = X @ Wg.T, X @ Wu.T
    S = orc.silu(G)
    a, b = _silu_grad(G) * U, S
    vH = _rounding_var(S * U)
    if np.any(vX):
        vH = vH + (a * a) * (vX @ (Wg * Wg).T) + (b * b) * (vX @ (Wu * Wu).T) + 2 * a * b * (vX @ (Wg * Wu).T)
    return vH @ (Wd * Wd).T


def latent_output_sigma(x, w_proj_down, w_gate, w_up, w_down, gain, eps, w_proj_up, shared_gate, shared_up,
                        shared_down, ref):
    """Per-element standard deviation [T, d] of (device out - float64 out) under the model above.

    `ref` is the oracle's latent_forward(..., bf16_operands=False) on the same x (its
    routing, z, u and r are used); weights as latent_forward takes them (expert tensors
    may be lazy per-expert views)."""
    X = orc.f64(x)
    T = X.shape[0]
    z, u, r = ref["z"], ref["u"], ref["r"]
    idx, w = np.asarray(ref["idx"]), np.asarray(ref["w"])
    k = idx.shape[1]
    l = z.shape[1]
    vz = _rounding_var(z)
    flat_e = idx.reshape(-1)
    vY = np.zeros((T * k, l))
    for e in np.unique(flat_e):
        rows = np.nonzero(flat_e == e)[0]
        toks = rows // k
        vY[rows] = swiglu_output_var(z[toks], vz[toks], w_gate[e], w_up[e], w_down[e])
    vY = vY.reshape(T, k, l)
    vu = np.sum((w * w)[:, :, None] * vY, axis=1)
    g = orc.f64(gain)
    s = np.sqrt(np.mean(u * u, axis=1, keepdims=True) + eps)
    vr = (g * g) * (vu / s ** 2 - 2 * u * u * vu / (l * s ** 4)
                    + u * u * np.sum(u * u * vu, axis=1, keepdims=True) / (l * l * s ** 6))
    vr = vr + _rounding_var(r)
    Wpu = orc.f64(w_proj_up)
    v_out = vr @ (Wpu * Wpu).T
    n_shared = 0 if shared_gate is None else len(shared_gate)
    zeros = np.zeros_like(X)
    for si in range(n_shared):
        v_out = v_out + swiglu_output_var(X, zeros, shared_gate[si], shared_up[si], shared_down[si])
    return np.sqrt(v_out)


def check_latent_out(out_dev, out_ref, sigma, what="latent out", n_sigma: float = 8.0, factor: float = 2.0):
    """|out - ref| <= n_sigma sigma + 1e-6 max|ref| elementwise and ||out - ref||_2 <= factor ||sigma||_2.
    Returns (error norm / ||sigma||_2, largest |out - ref| / sigma, max rel, mean abs)."""
    g = orc.f64(out_dev)
    r = np.asarray(out_ref, dtype=np.float64)
    err = np.abs(g - r)
    floor = 1e-6 * np.abs(r).max()
    bound = n_sigma * sigma + floor
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} entries beyond {n_sigma} sigma of the rounding "
                           f"model, worst {(err / np.maximum(sigma, floor)).max():.1f} sigma")
    s_norm = float(np.sqrt(np.sum(sigma * sigma)))
    e_norm = float(np.sqrt(np.sum(err * err)))
    ratio = e_norm / max(s_norm, 1e-300)
    assert ratio <= factor, f"{what}: error norm {e_norm:.3e} is {ratio:.2f} x the rounding model's {s_norm:.3e}"
    worst = float((err / np.maximum(sigma, floor)).max())
    return ratio, worst, err.max() / max(np.abs(r).max(), 1e-300), err.mean()
