"""Plain CPU oracle of the Stable LatentMoE layer (forward).

TEST INFRASTRUCTURE. Only tests/, the smoke check and the benchmark's CPU
baseline may import or call this module; the HIP library never does, and the
two share no code (kernels, headers, helpers, tables or constants).

Source: "Kimi K3: Open Frontier Intelligence", section "Operational Execution
Flow: From Native Multimodal Inputs to Sparse Channel Activations". For a token
x in R^d, two full-width shared experts read x itself; the routed path first
projects x down to a latent z = W_down_proj x in R^l (l = 3584 on the page),
sends z to the k experts the router picks out of E, sums their outputs
weighted by the gate probabilities into u, applies an explicit RMSNorm to u
and projects the result back up to R^d with W_up_proj. The formula that joins
the pieces is lost from the page.

Readings (also listed in the design notes):
  * y = W_up_proj RMSNorm(u) + sum_s SharedExpert_s(x): the order of the
    sentence, the shared experts added at full width;
  * the router scores x (the top-k set is written as a function of x), with the
    same gate, softmax, top-k and renormalisation as the plain routed layer;
  * RMSNorm(u) = g * u / sqrt(mean_j u_j^2 + eps), with a gain g in R^l;
  * every expert (routed in R^l, shared in R^d) is SwiGLU without biases.

The layer is computed in float64 with no intermediate rounding: that is the
definition the device is compared with. `bf16_operands=True` is a diagnostic
only: it rounds z, every expert's SwiGLU activation H and RMSNorm(u) to
bfloat16 (round to nearest even, through float32) before their products,
where the device rounds them, so that a test can look at the rounding points
one at a time. The tests bound the effect of those roundings on the output by
propagating them through the float64 layer.
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as _m

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def bf16_round(a) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float64 (library rounding)."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def rmsnorm(u, gain, eps: float) -> np.ndarray:
    """g * u / sqrt(mean_j u_j^2 + eps), row by row (float64)."""
    U = _m.f64(u)
    g = _m.f64(gain)
    ms = np.mean(U * U, axis=-1, keepdims=True)
    return U / np.sqrt(ms + eps) * g


def swiglu_rows(X, w_gate, w_up, w_down, bf16_operands: bool):
    """One SwiGLU FFN on the rows of X (weights [h, d], [h, d], [d, h]):
    H = silu(X Wg^T) * (X Wu^T), bf16-rounded when bf16_operands; Y = H Wd^T. Returns (H, Y)."""
    X = _m.f64(X)
    H = _m.silu(X @ _m.f64(w_gate).T) * (X @ _m.f64(w_up).T)
    if bf16_operands:
        H = bf16_round(H)
    return H, H @ _m.f64(w_down).T


def dense_swiglu(X, w_gate, w_up, w_down, bf16_operands: bool = False):
    """One SwiGLU FFN applied to every row of X (weights [h, d], [h, d], [d, h])."""
    return swiglu_rows(X, w_gate, w_up, w_down, bf16_operands)[1]


def routed_experts(z_rows, offsets, w_gate, w_up, w_down, bf16_operands: bool):
    """Expert e on its rows offsets[e] .. offsets[e+1]-1 of z_rows (rows of experts with no
    rows are skipped). Returns (H, Y) with NaN in rows no expert computed."""
    Z = _m.f64(z_rows)
    off = _m._int(offsets)
    H = Y = None
    for e in range(off.shape[0] - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        He, Ye = swiglu_rows(Z[lo:hi], w_gate[e], w_up[e], w_down[e], bf16_operands)
        if H is None:
            H = np.full((Z.shape[0], He.shape[1]), np.nan)
            Y = np.full((Z.shape[0], Ye.shape[1]), np.nan)
        H[lo:hi] = He
        Y[lo:hi] = Ye
    return H, Y


def latent_forward(x, w_router, bias, w_proj_down, w_gate, w_up, w_down, gain, eps, w_proj_up,
                   shared_gate, shared_up, shared_down, k: int, logits=None, bf16_operands: bool = False):
    """The layer: returns a dict with every intermediate.

    x [T, d]; w_router [E, d]; bias [E] or None; w_proj_down [l, d];
    w_gate, w_up [E, h, l]; w_down [E, l, h]; gain [l]; w_proj_up [d, l];
    shared_gate, shared_up [S, hs, d]; shared_down [S, d, hs] (S may be 0, or the three None).
    `logits` replaces the oracle's own gate logits (e.g. the device's).
    """
    X = _m.f64(x)
    E = _m.f64(w_router).shape[0]
    L = _m.gate_logits(X, w_router, bias) if logits is None else _m.f64(logits)
    idx, w, probs = _m.route(L, k)
    offsets, row_of, row_src = _m.permute(idx, E)
    z = X @ _m.f64(w_proj_down).T
    if bf16_operands:
        z = bf16_round(z)
    H, Y = routed_experts(z[row_src], offsets, w_gate, w_up, w_down, bf16_operands)
    u = _m.combine(Y, row_of, w)
    r = rmsnorm(u, gain, eps)
    if bf16_operands:
        r = bf16_round(r)
    up = r @ _m.f64(w_proj_up).T
    n_shared = 0 if shared_gate is None else len(shared_gate)
    shared = [dense_swiglu(X, shared_gate[s], shared_up[s], shared_down[s], bf16_operands) for s in range(n_shared)]
    out = up.copy()
    for y in shared:
        out = out + y
    return dict(logits=L, idx=idx, w=w, offsets=offsets, row_of=row_of, row_src=row_src, z=z, H=H, Y=Y, u=u,
                r=r, up=up, shared=shared, out=out)
