"""Torch-tensor front end of libmoe.so.

PyTorch provides device memory and the current stream; every computation
happens in the library's kernels, reached through the C ABI with the same
call names (moe_route, moe_permute, moe_expert_ffn, moe_combine, moe_forward).
Tensors must be contiguous, on one GPU, in the dtypes include/moe.h states.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != _DT[dtype]:
        raise TypeError(f"{name} must be {_DT[dtype]}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need_packed(t, name, shape, device):
    """A bf16 weight tensor in the library's packed layout (made by moe_pack_weights)."""
    _need(t, name, "bf16", shape, device)
    if not getattr(t, "moe_packed", False):
        raise TypeError(f"{name} must be in the packed weight layout: convert the row-major tensor once with "
                        f"moe_pack_weights")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape_of(x, w_router, k, h):
    T, d = x.shape
    E = w_router.shape[0]
    return _lib.shape(T, d, E, k, h)


def workspace(s: _lib.MoeShape, call: int, device) -> torch.Tensor:
    n = _lib.workspace_bytes(s, call)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def moe_route(x, w_router, router_bias, k: int, *, out=None):
    """Gate logits [T,E] f32, top-k ids [T,k] i32, renormalised weights [T,k] f32."""
    _need(x, "x", "bf16")
    dev = x.device
    T, d = x.shape
    E = w_router.shape[0]
    _need(w_router, "w_router", "f32", (E, d), dev)
    if router_bias is not None:
        _need(router_bias, "router_bias", "f32", (E,), dev)
    s = _lib.shape(T, d, E, k, 128)
    if out is None:
        out = (torch.empty((T, E), dtype=torch.float32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.float32, device=dev))
    logits, idx, w = out
    _need(logits, "logits", "f32", (T, E), dev)
    _need(idx, "topk_idx", "i32", (T, k), dev)
    _need(w, "topk_w", "f32", (T, k), dev)
    ws = workspace(s, _lib.MOE_CALL_ROUTE, dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_route(ctypes.byref(s), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                      _ptr(logits), _ptr(idx), _ptr(w), _ptr(ws), ws.numel(), _stream(dev)))
    return logits, idx, w


def moe_topk_softmax(logits, k: int):
    """Top-k ids [T,k] i32 and renormalised weights [T,k] f32 from given f32 logits [T,E]."""
    _need(logits, "logits", "f32")
    dev = logits.device
    T, E = logits.shape
    s = _lib.shape(T, 128, E, k, 128)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_topk_softmax(ctypes.byref(s), _ptr(logits), _ptr(idx), _ptr(w), _stream(dev)))
    return idx, w


def moe_permute(x, topk_idx, E: int, gather: bool = True):
    """expert_offsets [E+1], row_of [T,k], row_src [T*k] (int32) and x_perm [T*k, d] bf16
    (x_perm is None when gather=False: moe_expert_ffn can read x through row_src instead)."""
    _need(x, "x", "bf16")
    dev = x.device
    T, d = x.shape
    k = topk_idx.shape[1] if topk_idx.dim() == 2 else 1
    _need(topk_idx, "topk_idx", "i32", (T, k), dev)
    s = _lib.shape(T, d, E, k, 128)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_of = torch.empty((T, k), dtype=torch.int32, device=dev)
    row_src = torch.empty(T * k, dtype=torch.int32, device=dev)
    x_perm = torch.empty((T * k, d), dtype=torch.bfloat16, device=dev) if gather else None
    ws = workspace(s, _lib.MOE_CALL_PERMUTE, dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_permute(ctypes.byref(s), _ptr(x), _ptr(topk_idx), _ptr(offsets), _ptr(row_of),
                                        _ptr(row_src), _ptr(x_perm), _ptr(ws), ws.numel(), _stream(dev)))
    return offsets, row_of, row_src, x_perm


def moe_permute_noalloc(x, topk_idx, E: int, gather: bool = True, out=None):
    """moe_permute through the entry point that allocates nothing: its scratch is a fixed
    array inside the library. `out` may hold preallocated (expert_offsets, row_of, row_src,
    x_perm) to write into; otherwise they are allocated here, by the caller's side."""
    _need(x, "x", "bf16")
    dev = x.device
    T, d = x.shape
    k = topk_idx.shape[1] if topk_idx.dim() == 2 else 1
    _need(topk_idx, "topk_idx", "i32", (T, k), dev)
    s = _lib.shape(T, d, E, k, 128)
    if out is None:
        out = (torch.empty(E + 1, dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev),
               torch.empty((T * k, d), dtype=torch.bfloat16, device=dev) if gather else None)
    offsets, row_of, row_src, x_perm = out
    _need(offsets, "expert_offsets", "i32", (E + 1,), dev)
    _need(row_of, "row_of", "i32", (T, k), dev)
    _need(row_src, "row_src", "i32", (T * k,), dev)
    if x_perm is not None:
        _need(x_perm, "x_perm", "bf16", (T * k, d), dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_permute_noalloc(ctypes.byref(s), _ptr(x), _ptr(topk_idx), _ptr(offsets), _ptr(row_of),
                                                _ptr(row_src), _ptr(x_perm), _stream(dev)))
    return offsets, row_of, row_src, x_perm


def _rows_operand(a, a_rows, T, k):
    """Validate the A operand of the grouped GEMM: x_perm [T*k, d], or x [T, d] with row_src [T*k]."""
    _need(a, "a", "bf16")
    dev = a.device
    n, d = a.shape
    if a_rows is None:
        if n != T * k:
            raise ValueError(f"x_perm has {n} rows, expected T*k = {T * k}")
    else:
        if n != T:
            raise ValueError(f"x has {n} rows, expected T = {T}")
        _need(a_rows, "a_rows", "i32", (T * k,), dev)
    return dev, d


def moe_expert_ffn(a, expert_offsets, w_gate, w_up, w_down, T: int, k: int, a_rows=None):
    """h_act [T*k, h] bf16 and y_rows [T*k, d] f32 for rows grouped by expert.

    The rows are a = x_perm [T*k, d] (a_rows None), or a = x [T, d] read through a_rows = row_src [T*k].
    The expert weights are packed (moe_pack_weights)."""
    dev, d = _rows_operand(a, a_rows, T, k)
    n = T * k
    E, h, _ = w_gate.shape
    _need(expert_offsets, "expert_offsets", "i32", (E + 1,), dev)
    _need_packed(w_gate, "w_gate", (E, h, d), dev)
    _need_packed(w_up, "w_up", (E, h, d), dev)
    _need_packed(w_down, "w_down", (E, d, h), dev)
    s = _lib.shape(T, d, E, k, h)
    h_act = torch.empty((n, h), dtype=torch.bfloat16, device=dev)
    y_rows = torch.empty((n, d), dtype=torch.float32, device=dev)
    ws = workspace(s, _lib.MOE_CALL_EXPERT_FFN, dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_expert_ffn(ctypes.byref(s), _ptr(a), _ptr(a_rows), _ptr(expert_offsets),
                                           _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(h_act), _ptr(y_rows),
                                           _ptr(ws), ws.numel(), _stream(dev)))
    return h_act, y_rows


def moe_combine(y_rows, row_of, topk_w):
    """out [T, d] f32 = sum_j topk_w[t, j] * y_rows[row_of[t, j]]."""
    _need(y_rows, "y_rows", "f32")
    dev = y_rows.device
    n, d = y_rows.shape
    T, k = row_of.shape
    if n != T * k:
        raise ValueError(f"y_rows has {n} rows, expected T*k = {T * k}")
    _need(row_of, "row_of", "i32", (T, k), dev)
    _need(topk_w, "topk_w", "f32", (T, k), dev)
    s = _lib.shape(T, d, max(k, 1), k, 128)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_combine(ctypes.byref(s), _ptr(y_rows), _ptr(row_of), _ptr(topk_w), _ptr(out),
                                        _stream(dev)))
    return out


def moe_pack_weights(w):
    """Row-major bf16 weights w ([G, N, K] expert tensors, or one [N, K] matrix) in the library's
    packed layout (16-row x 32-column tiles of 512 contiguous elements, each one MFMA operand in
    lane order): a new tensor of the same shape and values whose memory is in packed order, the
    form every layer call takes. A one-time conversion, like loading a checkpoint."""
    _need(w, "w", "bf16")
    dev = w.device
    G, N, K = (1, *w.shape) if w.dim() == 2 else w.shape
    out = torch.empty_like(w)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_pack_weights(G, N, K, _ptr(w), _ptr(out), _stream(dev)))
    out.moe_packed = True
    return out


class MoEForward:
    """moe_forward with a reusable workspace; expert weights packed (moe_pack_weights)."""

    def __init__(self, T: int, d: int, E: int, k: int, h: int, device):
        self.shape = _lib.shape(T, d, E, k, h)
        self.T, self.d, self.E, self.k, self.h = T, d, E, k, h
        self.device = torch.device(device)
        self.ws = workspace(self.shape, _lib.MOE_CALL_FORWARD, self.device)

    def __call__(self, x, w_router, router_bias, w_gate, w_up, w_down, out=None):
        T, d, E, k, h, dev = self.T, self.d, self.E, self.k, self.h, self.device
        _need(x, "x", "bf16", (T, d), dev)
        _need(w_router, "w_router", "f32", (E, d), dev)
        if router_bias is not None:
            _need(router_bias, "router_bias", "f32", (E,), dev)
        _need_packed(w_gate, "w_gate", (E, h, d), dev)
        _need_packed(w_up, "w_up", (E, h, d), dev)
        _need_packed(w_down, "w_down", (E, d, h), dev)
        if out is None:
            out = torch.empty((T, d), dtype=torch.float32, device=dev)
        _need(out, "out", "f32", (T, d), dev)
        with torch.cuda.device(dev):
            _lib.check(_lib.lib.moe_forward(ctypes.byref(self.shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_gate),
                          _ptr(w_up), _ptr(w_down), _ptr(out), _ptr(self.ws), self.ws.numel(), _stream(dev)))
        return out

    def intermediate(self, name: str) -> torch.Tensor:
        """A view of one intermediate that the last call left in the workspace."""
        T, d, E, k, h = self.T, self.d, self.E, self.k, self.h
        spec = {
            "logits": (torch.float32, (T, E)), "topk_idx": (torch.int32, (T, k)),
            "topk_w": (torch.float32, (T, k)), "expert_offsets": (torch.int32, (E + 1,)),
            "row_of": (torch.int32, (T, k)), "row_src": (torch.int32, (T * k,)),
            "h_act": (torch.bfloat16, (T * k, h)),
            "y_rows": (torch.float32, (T * k, d)),
        }
        dtype, shp = spec[name]
        off = _lib.forward_ws_offset(self.shape, _lib.FWD_SLOTS.index(name))
        n = 1
        for v in shp:
            n *= v
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype).view(shp)


def moe_forward(x, w_router, router_bias, w_gate, w_up, w_down, k: int):
    """One-shot forward on packed expert weights (allocates a workspace per call; use MoEForward
    to reuse one)."""
    T, d = x.shape
    E, h, _ = w_gate.shape
    return MoEForward(T, d, E, k, h, x.device)(x, w_router, router_bias, w_gate, w_up, w_down)


# ------------------------------------------------------------ load balancing

def moe_aux_loss(logits):
    """(prob_mean [E] f32, aux_loss [1] f32) from f32 logits [T, E]: each expert's
    batch-mean softmax probability and sum_e (prob_mean[e] - 1/E)^2."""
    _need(logits, "logits", "f32")
    dev = logits.device
    T, E = logits.shape
    if T == 0:
        raise ValueError("the aux loss of an empty batch is undefined")
    s = _lib.shape(T, 128, E, 1, 128)
    prob_mean = torch.empty(E, dtype=torch.float32, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    ws = workspace(s, _lib.MOE_CALL_AUX_LOSS, dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_aux_loss(ctypes.byref(s), _ptr(logits), _ptr(prob_mean), _ptr(aux), _ptr(ws),
                                         ws.numel(), _stream(dev)))
    return prob_mean, aux


def moe_qb_route(logits, qb_bias, k: int):
    """Quantile Balancing selection: top-k ids [T,k] i32 of logits + qb_bias, weights [T,k] f32
    from the unbiased logits, and the cutoff alpha [T] f32 (the (k+1)-th biased score)."""
    _need(logits, "logits", "f32")
    dev = logits.device
    T, E = logits.shape
    _need(qb_bias, "qb_bias", "f32", (E,), dev)
    s = _lib.shape(T, 128, E, k, 128)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    alpha = torch.empty(T, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_qb_route(ctypes.byref(s), _ptr(logits), _ptr(qb_bias), _ptr(idx), _ptr(w),
                                         _ptr(alpha), _stream(dev)))
    return idx, w, alpha


def moe_qb_histogram(logits, alpha, k: int, lo: float, width: float, n_bins: int, out=None):
    """Per-expert histogram [E, n_bins] i32 of the margins logits - alpha[:, None]."""
    _need(logits, "logits", "f32")
    dev = logits.device
    T, E = logits.shape
    _need(alpha, "alpha", "f32", (T,), dev)
    s = _lib.shape(T, 128, E, k, 128)
    hist = torch.empty((E, n_bins), dtype=torch.int32, device=dev) if out is None else out
    _need(hist, "hist", "i32", (E, n_bins), dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_qb_histogram(ctypes.byref(s), _ptr(logits), _ptr(alpha), lo, width, n_bins,
                                             _ptr(hist), _stream(dev)))
    return hist


def moe_qb_update(hist, k: int, lo: float, width: float, bias_in, out=None):
    """New Quantile Balancing bias [E] f32: minus the (1 - k/E)-quantile of each histogram row
    (rows with no counts keep bias_in). `out` may be bias_in itself."""
    _need(hist, "hist", "i32")
    dev = hist.device
    E, n_bins = hist.shape
    _need(bias_in, "bias_in", "f32", (E,), dev)
    bias_out = torch.empty(E, dtype=torch.float32, device=dev) if out is None else out
    _need(bias_out, "bias_out", "f32", (E,), dev)
    s = _lib.shape(0, 128, E, k, 128)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_qb_update(ctypes.byref(s), _ptr(hist), lo, width, n_bins, _ptr(bias_in),
                                          _ptr(bias_out), _stream(dev)))
    return bias_out


# ------------------------------------------------------------------ LatentMoE

def moe_combine_rmsnorm(y_rows, row_of, topk_w, gain, eps: float, want_u: bool = False):
    """r [T, l] bf16 = RMSNorm(u) with gain, u = sum_j topk_w[t, j] y_rows[row_of[t, j]]
    (and u [T, l] f32 when want_u)."""
    _need(y_rows, "y_rows", "f32")
    dev = y_rows.device
    n, l = y_rows.shape
    T, k = row_of.shape
    if n != T * k:
        raise ValueError(f"y_rows has {n} rows, expected T*k = {T * k}")
    _need(row_of, "row_of", "i32", (T, k), dev)
    _need(topk_w, "topk_w", "f32", (T, k), dev)
    _need(gain, "gain", "f32", (l,), dev)
    s = _lib.shape(T, l, max(k, 1), k, 128)
    r = torch.empty((T, l), dtype=torch.bfloat16, device=dev)
    u = torch.empty((T, l), dtype=torch.float32, device=dev) if want_u else None
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_combine_rmsnorm(ctypes.byref(s), _ptr(y_rows), _ptr(row_of), _ptr(topk_w), _ptr(gain),
                                                eps, _ptr(u), _ptr(r), _stream(dev)))
    return (r, u) if want_u else r


class LatentMoEForward:
    """moe_latent_forward with a reusable workspace (allocated once per shape); every bf16 weight
    packed (moe_pack_weights)."""

    def __init__(self, T: int, d: int, l: int, E: int, k: int, h: int, n_shared: int, h_shared: int, device):
        self.shape = _lib.latent_shape(T, d, l, E, k, h, n_shared, h_shared)
        self.T, self.d, self.l, self.E, self.k, self.h = T, d, l, E, k, h
        self.S, self.hs = n_shared, h_shared
        self.device = torch.device(device)
        n = _lib.latent_workspace_bytes(self.shape)
        self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)

    def __call__(self, x, w_router, router_bias, w_proj_down, w_gate, w_up, w_down, rms_gain, rms_eps, w_proj_up,
                 shared_gate=None, shared_up=None, shared_down=None, out=None):
        T, d, l, E, k, h, S, hs, dev = self.T, self.d, self.l, self.E, self.k, self.h, self.S, self.hs, self.device
        _need(x, "x", "bf16", (T, d), dev)
        _need(w_router, "w_router", "f32", (E, d), dev)
        if router_bias is not None:
            _need(router_bias, "router_bias", "f32", (E,), dev)
        _need_packed(w_proj_down, "w_proj_down", (l, d), dev)
        _need_packed(w_gate, "w_gate", (E, h, l), dev)
        _need_packed(w_up, "w_up", (E, h, l), dev)
        _need_packed(w_down, "w_down", (E, l, h), dev)
        _need(rms_gain, "rms_gain", "f32", (l,), dev)
        _need_packed(w_proj_up, "w_proj_up", (d, l), dev)
        if S > 0:
            _need_packed(shared_gate, "shared_gate", (S, hs, d), dev)
            _need_packed(shared_up, "shared_up", (S, hs, d), dev)
            _need_packed(shared_down, "shared_down", (S, d, hs), dev)
        if out is None:
            out = torch.empty((T, d), dtype=torch.float32, device=dev)
        _need(out, "out", "f32", (T, d), dev)
        with torch.cuda.device(dev):
            _lib.check(_lib.lib.moe_latent_forward(
                ctypes.byref(self.shape), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_proj_down),
                _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(rms_gain), rms_eps, _ptr(w_proj_up),
                _ptr(shared_gate if S > 0 else None), _ptr(shared_up if S > 0 else None),
                _ptr(shared_down if S > 0 else None), _ptr(out), _ptr(self.ws), self.ws.numel(), _stream(dev)))
        return out

    def intermediate(self, name: str) -> torch.Tensor:
        """A view of one intermediate that the last call left in the workspace."""
        T, d, l, E, k, h, S, hs = self.T, self.d, self.l, self.E, self.k, self.h, self.S, self.hs
        spec = {
            "logits": (torch.float32, (T, E)), "topk_idx": (torch.int32, (T, k)),
            "topk_w": (torch.float32, (T, k)), "expert_offsets": (torch.int32, (E + 1,)),
            "row_of": (torch.int32, (T, k)), "row_src": (torch.int32, (T * k,)),
            "z": (torch.bfloat16, (T, l)), "h_act": (torch.bfloat16, (T * k, h)),
            "y_rows": (torch.float32, (T * k, l)), "r": (torch.bfloat16, (T, l)),
            "shared_h": (torch.bfloat16, (S * T, hs)), "shared_y": (torch.float32, (S * T, d)),
        }
        dtype, shp = spec[name]
        off = _lib.latent_ws_offset(self.shape, _lib.LAT_SLOTS.index(name))
        n = 1
        for v in shp:
            n *= v
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype).view(shp)


# ------------------------------------------------------------------ MX experts

_U8 = torch.uint8


def moe_mx_quantize_weights(w):
    """MXFP4 codes [G, N, K/2] u8 (two per byte, low nibble first) and E8M0 scales [G, N, K/32] u8
    (matrix-core order) of bf16 weights w [G, N, K]."""
    _need(w, "w", "bf16")
    dev = w.device
    G, N, K = w.shape
    q = torch.empty((G, N, K // 2), dtype=_U8, device=dev)
    sc = torch.empty((G, N, K // 32), dtype=_U8, device=dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_mx_quantize_weights(G, N, K, _ptr(w), _ptr(q), _ptr(sc), _stream(dev)))
    return q, sc


def moe_mx_quantize_rows(x):
    """MXFP8 codes [R, K] u8 and E8M0 scales [R, K/32] u8 (row order) of rows x [R, K] (bf16 or f32)."""
    if not isinstance(x, torch.Tensor) or x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be a bf16 or float32 tensor")
    _need(x, "x", "bf16" if x.dtype == torch.bfloat16 else "f32")
    dev = x.device
    R, K = x.shape
    q = torch.empty((R, K), dtype=_U8, device=dev)
    sc = torch.empty((R, K // 32), dtype=_U8, device=dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_mx_quantize_rows(R, K, _ptr(x), int(x.dtype == torch.float32), _ptr(q), _ptr(sc),
                                                 _stream(dev)))
    return q, sc


def _need_u8(t, name, shape, dev):
    if not isinstance(t, torch.Tensor) or t.dtype != _U8 or t.device != dev or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous uint8 tensor on {dev}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def moe_mx_expert_ffn(a_q, a_s, expert_offsets, gate, up, down, T: int, k: int, h: int, a_rows=None):
    """MX expert FFN. gate, up, down are (codes, scales) pairs from moe_mx_quantize_weights of
    [E, h, d], [E, h, d], [E, d, h]; a_q/a_s are MXFP8 rows ([T*k, d], or [T, d] read through a_rows).
    Returns h_act [T*k, h] f32, h_q [T*k, h] u8, h_s [T*k, h/32] u8, y_rows [T*k, d] f32."""
    dev = a_q.device
    n = T * k
    d = a_q.shape[1]
    E = expert_offsets.shape[0] - 1
    _need_u8(a_q, "a_q", (n if a_rows is None else T, d), dev)
    _need_u8(a_s, "a_s", (n if a_rows is None else T, d // 32), dev)
    if a_rows is not None:
        _need(a_rows, "a_rows", "i32", (n,), dev)
    _need(expert_offsets, "expert_offsets", "i32", (E + 1,), dev)
    for name, (q, sc), (N, K) in (("gate", gate, (h, d)), ("up", up, (h, d)), ("down", down, (d, h))):
        _need_u8(q, f"{name} codes", (E, N, K // 2), dev)
        _need_u8(sc, f"{name} scales", (E, N, K // 32), dev)
    s = _lib.shape(T, d, E, k, h)
    h_act = torch.empty((n, h), dtype=torch.float32, device=dev)
    h_q = torch.empty((n, h), dtype=_U8, device=dev)
    h_s = torch.empty((n, h // 32), dtype=_U8, device=dev)
    y = torch.empty((n, d), dtype=torch.float32, device=dev)
    ws = workspace(s, _lib.MOE_CALL_EXPERT_FFN, dev)
    with torch.cuda.device(dev):
        _lib.check(_lib.lib.moe_mx_expert_ffn(ctypes.byref(s), _ptr(a_q), _ptr(a_s), _ptr(a_rows),
                                              _ptr(expert_offsets), _ptr(gate[0]), _ptr(gate[1]), _ptr(up[0]),
                                              _ptr(up[1]), _ptr(down[0]), _ptr(down[1]), _ptr(h_act), _ptr(h_q),
                                              _ptr(h_s), _ptr(y), _ptr(ws), ws.numel(), _stream(dev)))
    return h_act, h_q, h_s, y


class MXForward:
    """moe_mx_forward with a reusable workspace; expert weights are (codes, scales) pairs."""

    def __init__(self, T: int, d: int, E: int, k: int, h: int, device):
        self.shape = _lib.shape(T, d, E, k, h)
        self.T, self.d, self.E, self.k, self.h = T, d, E, k, h
        self.device = torch.device(device)
        self.ws = workspace(self.shape, _lib.MOE_CALL_MX_FORWARD, self.device)

    def __call__(self, x, w_router, router_bias, gate, up, down, out=None):
        T, d, E, k, h, dev = self.T, self.d, self.E, self.k, self.h, self.device
        _need(x, "x", "bf16", (T, d), dev)
        _need(w_router, "w_router", "f32", (E, d), dev)
        if router_bias is not None:
            _need(router_bias, "router_bias", "f32", (E,), dev)
        for name, (q, sc), (N, K) in (("gate", gate, (h, d)), ("up", up, (h, d)), ("down", down, (d, h))):
            _need_u8(q, f"{name} codes", (E, N, K // 2), dev)
            _need_u8(sc, f"{name} scales", (E, N, K // 32), dev)
        if out is None:
            out = torch.empty((T, d), dtype=torch.float32, device=dev)
        _need(out, "out", "f32", (T, d), dev)
        with torch.cuda.device(dev):
            _lib.check(_lib.lib.moe_mx_forward(ctypes.byref(self.shape), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                               _ptr(gate[0]), _ptr(gate[1]), _ptr(up[0]), _ptr(up[1]),
                                               _ptr(down[0]), _ptr(down[1]), _ptr(out), _ptr(self.ws),
                                               self.ws.numel(), _stream(dev)))
        return out

    def intermediate(self, name: str) -> torch.Tensor:
        T, d, E, k, h = self.T, self.d, self.E, self.k, self.h
        n = T * k
        spec = {
            "logits": (torch.float32, (T, E)), "topk_idx": (torch.int32, (T, k)),
            "topk_w": (torch.float32, (T, k)), "expert_offsets": (torch.int32, (E + 1,)),
            "row_of": (torch.int32, (T, k)), "row_src": (torch.int32, (n,)),
            "x_q": (_U8, (T, d)), "x_s": (_U8, (T, d // 32)), "h_act": (torch.float32, (n, h)),
            "h_q": (_U8, (n, h)), "h_s": (_U8, (n, h // 32)), "y_rows": (torch.float32, (n, d)),
        }
        dtype, shp = spec[name]
        off = _lib.mx_forward_ws_offset(self.shape, _lib.MX_SLOTS.index(name))
        cnt = 1
        for v in shp:
            cnt *= v
        nbytes = cnt * torch.tensor([], dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype).view(shp)
