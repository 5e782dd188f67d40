"""Helpers of the GPU parity tests: tolerances and oracle comparisons.

Tolerances (floating point):
  * gate logits: |l_gpu - l_ref| <= 1e-4 * max(1, |l_ref|). The device sums
    exact bf16 x float32 products in float32; float32 rounding of a d-term sum
    stays orders of magnitude below this.
  * top-k weights: |w_gpu - w_ref| <= 1e-5, both computed from the same
    (device) logits.
  * H rows (bf16): the device rounds silu(g) * u once to bf16 (relative error
    <= 2^-8) after float32 accumulation, so
    |h_gpu - h_ref| <= 2^-8 |h_ref| + 1e-4 * max|h_ref| + 1e-6.
  * Y rows (float32): Y = sum_j bf16(h_j) w_j in float32; each rounded h_j
    carries at most 2^-8 |h_j| of error, so
    |y_gpu - y_ref| <= 2^-8 * sum_j |h_j| |w_j| * 1.01 + 1e-4 * max|y_ref|.
  * layer output: max|out - ref| / max|ref| <= 2e-2 and mean|out - ref| <= 1e-3
    (the layer's stated tolerance for bf16 inputs with float32 accumulation).
Integers (ids, offsets, permutation) and copies (x_perm) must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.moe_oracle as orc

U = 2.0 ** -8  # bf16 relative rounding bound (round to nearest)


def host(t):
    return t.detach().to("cpu")


def f64(t):
    return orc.f64(t)


def check_logits(gpu_logits, ref_logits, what="logits"):
    g = f64(gpu_logits)
    r = np.asarray(ref_logits, dtype=np.float64)
    err = np.abs(g - r)
    bound = 1e-4 * np.maximum(1.0, np.abs(r))
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} entries off, worst {err.max():.3e}"


def check_route(gpu_logits, gpu_idx, gpu_w, k):
    """Indices bit-exact and weights within 1e-5 of the oracle run on the device's own logits."""
    idx_ref, w_ref, _ = orc.route(f64(gpu_logits), k)
    gi = host(gpu_idx).to(torch.int64).numpy()
    mism = np.argwhere(gi != idx_ref)
    assert mism.size == 0, f"top-k ids differ at {mism[:5].tolist()} (of {len(mism)})"
    err = np.abs(f64(gpu_w) - w_ref)
    assert err.max() <= 1e-5, f"top-k weights off by {err.max():.3e}"
    return idx_ref, w_ref


def check_permutation(gpu_offsets, gpu_row_of, gpu_row_src, idx_ref, E):
    off, row_of, row_src = orc.permute(idx_ref, E)
    assert np.array_equal(host(gpu_offsets).numpy().astype(np.int64), off), "expert_offsets differ"
    assert np.array_equal(host(gpu_row_of).numpy().astype(np.int64), row_of), "row_of differs"
    assert np.array_equal(host(gpu_row_src).numpy().astype(np.int64), row_src), "row_src differs"
    return off, row_of, row_src


def check_h_rows(h_gpu, h_ref, what="H"):
    g = f64(h_gpu)
    r = np.asarray(h_ref, dtype=np.float64)
    bound = U * np.abs(r) + 1e-4 * np.abs(r).max() + 1e-6
    err = np.abs(g - r)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} entries off, worst excess {(err - bound).max():.3e}"


def check_y_rows(y_gpu, y_ref, h_ref, w_down_e, what="Y"):
    g = f64(y_gpu)
    r = np.asarray(y_ref, dtype=np.float64)
    absprod = np.abs(np.asarray(h_ref, dtype=np.float64)) @ np.abs(f64(w_down_e)).T
    bound = 1.01 * U * absprod + 1e-4 * np.abs(r).max() + 1e-6
    err = np.abs(g - r)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} entries off, worst excess {(err - bound).max():.3e}"


def layer_errors(out_gpu, out_ref):
    g = f64(out_gpu)
    r = np.asarray(out_ref, dtype=np.float64)
    d = np.abs(g - r)
    return d.max() / max(np.abs(r).max(), 1e-30), d.mean()


def check_layer(out_gpu, out_ref, what="out"):
    max_rel, mean_abs = layer_errors(out_gpu, out_ref)
    assert max_rel <= 2e-2 and mean_abs <= 1e-3, f"{what}: max rel {max_rel:.3e}, mean abs {mean_abs:.3e}"
    return max_rel, mean_abs


def packed(*ws):
    """Row-major bf16 weight tensors converted once to the library's packed layout (moe_pack_weights,
    on their device): the form every layer call takes."""
    from sparse_mixture_experts_fp32_amd import moe_pack_weights
    out = tuple(moe_pack_weights(w) for w in ws)
    return out if len(out) > 1 else out[0]


class LazyExperts:
    """Indexable view of one device weight tensor that copies expert e to the host on demand."""

    def __init__(self, t):
        self.t = t
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = host(self.t[e])
        return self.cache[e]
