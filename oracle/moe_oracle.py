"""Plain, slow float64 oracle of one routed Mixture-of-Experts FFN layer (forward).

TEST INFRASTRUCTURE. Only tests/, the smoke check and the benchmark's CPU
baseline may import or call this module; the HIP library never does, and the
two share no code (kernels, headers, helpers, tables or constants).

Sources (the Kimi K3 pages):
  [NC]  "Kimi K3: The Open Model That Just Cornered the AI Frontier",
        section "Mixture-of-Experts with Dynamic Load Balancing": the gating
        forward pass -- a linear projection of each token to one logit per
        expert, a softmax over the experts, then a top-k that returns the
        selected values and indices.
  [AQ]  "Kimi K3: Open Frontier Intelligence", section "Operational Execution
        Flow: From Native Multimodal Inputs to Sparse Channel Activations":
        the routed output of a token is the sum over its selected experts of
        the gate probability times that expert's output; the expert FFNs keep
        SwiGLU's form (the SiTU-GLU sentence names SwiGLU as the regime it
        preserves).
  [FC]  "Kimi K3: What Open-Source Frontier Models Reveal About RL Scaling for
        Reasoning", section "The Architecture": the router picks a fixed
        number of experts per token out of a large pool.

Readings where the pages are silent (each is also listed in the design notes):
  * selection is made on the float logits, not on the rounded probabilities
    (softmax is strictly increasing, so the chosen set is the same);
  * ties go to the lower expert id; -0.0 and +0.0 tie;
  * slot j of a token holds its j-th largest logit (the top-k returns its
    values sorted, largest first);
  * the k selected probabilities are renormalised to sum to one;
  * no capacity limit: every (token, slot) assignment is computed;
  * the expert FFN is SwiGLU without biases: y = (silu(x Wg^T) * (x Wu^T)) Wd^T
    with silu(g) = g * sigmoid(g);
  * rows are grouped by expert in ascending expert id; within one expert they
    keep the order of the flattened assignment index a = t * k + j.

Everything is float64 with no intermediate rounding. Inputs that are bfloat16
on the device are widened exactly. Every function is pinned by tests that do
not reuse its code (brute force, closed forms, invariants, special cases).
"""
from __future__ import annotations

import numpy as np

try:  # torch is only used to widen bfloat16 tensors exactly
    import torch
except ImportError:  # pragma: no cover
    torch = None


def f64(a) -> np.ndarray:
    """Exact widening of a torch tensor (any float dtype, any device) or array to float64."""
    if torch is not None and isinstance(a, torch.Tensor):
        return a.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def _int(a) -> np.ndarray:
    if torch is not None and isinstance(a, torch.Tensor):
        return a.detach().to("cpu").to(torch.int64).numpy()
    return np.asarray(a, dtype=np.int64)


# ---------------------------------------------------------------- routing [NC]

def gate_logits(x, w_router, bias=None) -> np.ndarray:
    """[NC] gate projection: one score per (token, expert).

    logits[t, e] = sum_i x[t, i] * w_router[e, i]  (+ bias[e])
    x: [T, d]; w_router: [E, d] (output-major storage); bias: [E] or None.
    """
    L = f64(x) @ f64(w_router).T
    if bias is not None:
        L = L + f64(bias)[None, :]
    return L


def softmax(logits) -> np.ndarray:
    """[NC] softmax over the expert axis: p[t,e] = exp(l[t,e] - m_t) / sum_e' exp(l[t,e'] - m_t)."""
    L = f64(logits)
    m = L.max(axis=-1, keepdims=True)
    z = np.exp(L - m)
    return z / z.sum(axis=-1, keepdims=True)


def topk_indices(logits, k: int) -> np.ndarray:
    """[NC] top-k selection, largest first, ties to the lower expert id.

    Sorts each token's experts by the key (-logit, expert id) and keeps the
    first k. -0.0 and +0.0 compare equal, so they tie.
    """
    L = f64(logits)
    T, E = L.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -L), axis=-1)  # last key is primary
    return order[:, :k].astype(np.int64)


def renormalise(probs, idx) -> np.ndarray:
    """Weights of the selected experts, rescaled to sum to one per token.

    w[t, j] = p[t, idx[t, j]] / sum_i p[t, idx[t, i]]
    """
    P = f64(probs)
    sel = np.take_along_axis(P, _int(idx), axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


def route(logits, k: int):
    """[NC] softmax -> top-k -> renormalised weights. Returns (idx [T,k], w [T,k], probs [T,E])."""
    probs = softmax(logits)
    idx = topk_indices(logits, k)
    return idx, renormalise(probs, idx), probs


# ----------------------------------------------------------- grouping by expert

def permute(idx, E: int):
    """Group the (token, slot) assignments by expert, stably.

    count[e]      = number of assignments with idx == e
    offsets[e+1]  = offsets[e] + count[e], offsets[0] = 0
    rows of expert e are offsets[e] .. offsets[e+1]-1, holding its assignments
    in increasing flattened index a = t*k + j.
    row_src[r] = token of row r; row_of[t, j] = row of assignment (t, j).
    """
    I = _int(idx)
    T, k = I.shape
    flat = I.reshape(-1)
    counts = np.bincount(flat, minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.lexsort((np.arange(T * k), flat))  # primary: expert id, then a
    row_src = order // k
    row_of = np.empty(T * k, dtype=np.int64)
    row_of[order] = np.arange(T * k)
    return offsets, row_of.reshape(T, k), row_src


def gather(x, row_src) -> np.ndarray:
    """Dispatch: x_perm[r] = x[row_src[r]]."""
    return f64(x)[_int(row_src)]


# ------------------------------------------------------------ expert FFN [AQ]

def silu(g) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    g = f64(g)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_swiglu(X, w_gate_e, w_up_e, w_down_e):
    """[AQ] one SwiGLU expert on its rows X [M, d]; weights stored [h, d], [h, d], [d, h].

    H = silu(X Wg^T) * (X Wu^T)   [M, h]
    Y = H Wd^T                     [M, d]
    """
    X = f64(X)
    G = X @ f64(w_gate_e).T
    U = X @ f64(w_up_e).T
    H = silu(G) * U
    Y = H @ f64(w_down_e).T
    return H, Y


def expert_ffn(x_perm, offsets, w_gate, w_up, w_down, experts=None):
    """Apply expert e to its rows offsets[e]..offsets[e+1]-1 of x_perm.

    w_gate, w_up, w_down are indexable by expert id (w[e] -> that expert's
    matrix). Experts with no rows are skipped. `experts` restricts the work to
    a subset of expert ids (rows of other experts are left as NaN).
    Returns (H [R, h], Y [R, d]).
    """
    Xp = f64(x_perm)
    off = _int(offsets)
    R = Xp.shape[0]
    E = off.shape[0] - 1
    H = Y = None
    for e in (range(E) if experts is None else experts):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        He, Ye = expert_swiglu(Xp[lo:hi], w_gate[e], w_up[e], w_down[e])
        if H is None:
            H = np.full((R, He.shape[1]), np.nan)
            Y = np.full((R, Ye.shape[1]), np.nan)
        H[lo:hi] = He
        Y[lo:hi] = Ye
    if H is None:
        h = f64(w_gate[0]).shape[0] if E > 0 else 0
        H = np.full((R, h), np.nan)
        Y = np.full((R, Xp.shape[1]), np.nan)
    return H, Y


def combine(Y, row_of, w) -> np.ndarray:
    """[AQ] out[t] = sum_j w[t, j] * Y[row_of[t, j]], summed in slot order j = 0..k-1."""
    Yv = f64(Y)
    R = _int(row_of)
    W = f64(w)
    T, k = R.shape
    out = np.zeros((T, Yv.shape[1]))
    for j in range(k):
        out += W[:, j:j + 1] * Yv[R[:, j]]
    return out


# ------------------------------------------------------------- whole layer

def forward(x, w_router, bias, w_gate, w_up, w_down, k: int, logits=None):
    """The whole layer. When `logits` is given (e.g. the device's float32
    logits), routing runs on those values; otherwise on the oracle's own.

    Returns a dict with every intermediate.
    """
    E = f64(w_router).shape[0]
    L = gate_logits(x, w_router, bias) if logits is None else f64(logits)
    idx, w, probs = route(L, k)
    offsets, row_of, row_src = permute(idx, E)
    x_perm = gather(x, row_src)
    H, Y = expert_ffn(x_perm, offsets, w_gate, w_up, w_down)
    out = combine(Y, row_of, w)
    return dict(logits=L, probs=probs, idx=idx, w=w, offsets=offsets, row_of=row_of,
                row_src=row_src, x_perm=x_perm, H=H, Y=Y, out=out)
