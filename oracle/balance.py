"""Plain CPU oracle of the two load-balancing statistics on the Kimi K3 pages.

TEST INFRASTRUCTURE. Only tests/, the smoke check and the benchmark's CPU
baseline may import or call this module; the HIP library never does, and the
two share no code (kernels, headers, helpers, tables or constants).

Sources (the Kimi K3 pages):
  [NC]  "Kimi K3: The Open Model That Just Cornered the AI Frontier",
        section "Mixture-of-Experts with Dynamic Load Balancing": the gating
        forward pass also returns an auxiliary loss, the squared distance of
        each expert's batch-mean softmax probability from the uniform share
        1/E, summed over the experts.
  [AQ]  "Kimi K3: Open Frontier Intelligence", section "Systems Optimization,
        Load Balancing, and Post-Training Alignment": Quantile Balancing (QB).
        Balancing is posed as the dual of a linear program. Each token's
        cutoff alpha_i comes from routing it to its top k+1 experts; the
        margin of token i for expert j is its router score minus that cutoff;
        expert j's bias is set from the (1 - k/E)-quantile of its margins over
        the batch, and that quantile is read off a per-expert histogram of
        B = 1000 bins whose counts are summed over the data-parallel ranks.

Readings where the pages are silent or garbled (also listed in the design notes):
  * aux loss: the listing averages over its first axis; for a flat batch of T
    tokens that is the mean over tokens. The loss weight (0.01 on the page) is
    the caller's business: the raw sum is returned.
  * QB score s_ij: the router logit (the gate output before the softmax). The
    bias moves only the selection; the weights of the chosen experts are the
    renormalised softmax of the unbiased logits.
  * alpha_i: the (k+1)-th largest biased score s_ij + b_j of token i (ties to
    the lower expert id, as in the plain top-k). With it, token i picks expert
    j when s_ij + b_j is above alpha_i, i.e. when its margin s_ij - alpha_i is
    above -b_j; so the new bias is b_j = -Q_j, Q_j the (1 - k/E)-quantile of
    the margins of expert j: then a share k/E of the tokens, the load target
    T*k/E, lies above it (-b_j is the dual price of expert j's capacity).
    Measuring margins on the biased score and moving the old bias by minus
    their quantile gives the same new bias.
  * the biased score, the margin and the bin index are float32 operations
    (they decide integers, so the oracle takes them in the precision of the
    float32 logits): score = fl(s + b), margin = fl(s - alpha),
    bin = floor(fl(fl(margin - lo) / width)), clamped to [0, B - 1]; so
    margins below lo count in bin 0 and those at or above lo + B*width in
    bin B - 1. The bin range (lo, width) is lost on the page and is a
    parameter: two float32 values, used as such in the quantile as well.
  * the quantile is read from the histogram with the grouped-data formula:
    the first bin b whose cumulative count C_b reaches p*m (m = the row's
    total, p = 1 - k/E), then Q = lo + width * (b + (p*m - C_{b-1}) / H_b),
    i.e. the margins of that bin are taken as spread evenly over it. An empty
    histogram row (m = 0) leaves that expert's bias unchanged.

Float64 wherever no integer is decided.
"""
from __future__ import annotations

import numpy as np

try:  # torch is only used to widen tensors exactly
    import torch
except ImportError:  # pragma: no cover
    torch = None


def _f64(a) -> np.ndarray:
    if torch is not None and isinstance(a, torch.Tensor):
        return a.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def _f32(a) -> np.ndarray:
    """Exact float32 view of float32 data (the logits, the bias, alpha)."""
    if torch is not None and isinstance(a, torch.Tensor):
        a = a.detach().to("cpu")
        assert a.dtype == torch.float32, a.dtype
        return a.numpy().copy()
    a = np.asarray(a)
    if a.dtype != np.float32:
        b = a.astype(np.float32)
        assert np.array_equal(b.astype(np.float64), a.astype(np.float64), equal_nan=True), \
            "value not representable in float32"
        a = b
    return a


def _i64(a) -> np.ndarray:
    if torch is not None and isinstance(a, torch.Tensor):
        return a.detach().to("cpu").to(torch.int64).numpy()
    return np.asarray(a, dtype=np.int64)


# ----------------------------------------------------------------- aux loss [NC]

def expert_prob_mean(probs) -> np.ndarray:
    """[NC] mean over the T tokens of each expert's softmax probability: [E]."""
    P = _f64(probs)
    T = P.shape[0]
    assert T > 0, "the mean over an empty batch is undefined"
    return P.sum(axis=0) / T


def aux_loss(probs):
    """[NC] auxiliary balance loss sum_e (mean_t p[t, e] - 1/E)^2.

    Returns (loss, mean [E])."""
    m = expert_prob_mean(probs)
    E = m.shape[0]
    return float(np.sum((m - 1.0 / E) ** 2)), m


# ----------------------------------------------------- Quantile Balancing [AQ]

def qb_select(logits, bias, k: int):
    """[AQ] top-(k+1) routing on the biased scores fl32(s + b).

    Returns (idx [T, k] int64, alpha [T] float32): the k selected experts,
    largest biased score first (ties to the lower id), and the (k+1)-th
    largest biased score as the token's cutoff.
    """
    S = _f32(logits)
    b = _f32(bias)
    T, E = S.shape
    assert 0 < k < E, "top-(k+1) needs k + 1 <= E"
    score = (S + b[None, :]).astype(np.float32)  # float32 sum, rounded once
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -score.astype(np.float64)), axis=-1)[:, :k + 1]
    alpha = np.take_along_axis(score, order[:, k:k + 1], axis=-1)[:, 0]
    return order[:, :k].astype(np.int64), alpha.astype(np.float32)


def qb_weights(logits, idx) -> np.ndarray:
    """Weights of the selected experts: the softmax of the unbiased logits,
    renormalised over the chosen set (so only the selected logits matter):
    w[t, j] = exp(s[t, idx[t, j]]) / sum_i exp(s[t, idx[t, i]])."""
    S = _f64(logits)
    sel = np.take_along_axis(S, _i64(idx), axis=-1)
    z = np.exp(sel - sel.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def qb_margins(logits, alpha) -> np.ndarray:
    """[AQ] margin[t, j] = fl32(s[t, j] - alpha[t]) (float32 [T, E])."""
    S = _f32(logits)
    a = _f32(alpha)
    return (S - a[:, None]).astype(np.float32)


def qb_bin(margins, lo: float, width: float, n_bins: int) -> np.ndarray:
    """Bin of each margin: floor(fl32(fl32(m - lo) / width)) clamped to [0, n_bins - 1]."""
    M = np.asarray(margins, dtype=np.float32)
    lo32, w32 = np.float32(lo), np.float32(width)
    u = ((M - lo32).astype(np.float32) / w32).astype(np.float32)
    out = np.empty(M.shape, dtype=np.int64)
    below = ~(u >= 0)  # also NaN
    above = u >= np.float32(n_bins)
    mid = ~below & ~above
    out[below] = 0
    out[above] = n_bins - 1
    out[mid] = np.floor(u[mid]).astype(np.int64)
    return np.minimum(out, n_bins - 1)


def qb_histogram(logits, alpha, lo: float, width: float, n_bins: int) -> np.ndarray:
    """[AQ] H[j, b] = number of tokens whose margin for expert j falls in bin b: int64 [E, n_bins]."""
    bins = qb_bin(qb_margins(logits, alpha), lo, width, n_bins)
    T, E = bins.shape
    H = np.zeros((E, n_bins), dtype=np.int64)
    for j in range(E):
        H[j] = np.bincount(bins[:, j], minlength=n_bins)
    return H


def qb_quantile(hist, k: int, lo: float, width: float) -> np.ndarray:
    """[AQ] (1 - k/E)-quantile of each histogram row by the grouped-data formula
    (float64 [E]; NaN for an empty row). The bin is chosen in exact integer
    arithmetic: the first b with C_b * E >= m * (E - k). lo and width are the
    float32 values that define the bins (as in qb_bin)."""
    lo, width = float(np.float32(lo)), float(np.float32(width))
    H = _i64(hist)
    E, B = H.shape
    Q = np.full(E, np.nan)
    for j in range(E):
        m = int(H[j].sum())
        if m == 0:
            continue
        need = m * (E - k)  # p * m, scaled by E
        below = 0  # C_{b-1}
        for b in range(B):
            if (below + int(H[j, b])) * E >= need:
                frac = (need - below * E) / (E * int(H[j, b]))
                Q[j] = lo + width * (b + frac)
                break
            below += int(H[j, b])
    return Q


def qb_update(hist, k: int, lo: float, width: float, bias_in) -> np.ndarray:
    """[AQ] new bias b_j = -Q_j (rounded to float32); rows with no counts keep bias_in."""
    Q = qb_quantile(hist, k, lo, width)
    b = _f32(bias_in).astype(np.float64)
    out = np.where(np.isnan(Q), b, -Q)
    return out.astype(np.float32)
