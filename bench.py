#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one pass of the whole layer over one batch: gate logits + top-k
(moe_route), grouping by expert (moe_permute), the grouped SwiGLU GEMM
(moe_expert_gate_up reading x through row_src -- the dispatch gather fused
into the GEMM -- and moe_expert_down) and the weighted combine (moe_combine),
enqueued through the C ABI on one stream with buffers allocated beforehand --
exactly the kernels moe_forward launches, checked bitwise against it below.
HIP events on that stream time each GEMM pass inside every timed step.

Prints one JSON line: whole-layer tokens/s, the grouped GEMM's TFLOP/s and
MFMA fraction, the roofline of the dominant kernel (the gate/up pass) and the
CPU oracle's rate on a bounded sample of the same workload. The "hbm_kernels"
object times the top-k, the permute (with and without the x_perm gather) and
the combine calls on their own, each against HBM bandwidth, warm (back to back
on the same buffers, whose smaller inputs then sit in the 256 MB last-level
cache) and cold (a 512 MiB scratch buffer written between calls). The
"balance" object times the router's load-balancing calls on the step's own
logits: one Quantile Balancing step (moe_qb_route, moe_qb_histogram with 1000
bins, moe_qb_update) and moe_aux_loss, each against HBM bandwidth. The
"ceilings" object holds what this chip measurably reaches (libmoe_probe.so: a
plain read, the direct-to-LDS read the expert GEMM uses, a copy, and
back-to-back bf16 matrix-core products) beside the published peaks;
`--ceilings` prints only that object.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + grouped-GEMM TFLOP/s (% MFMA peak), d=7168 E=256 top-4"
# HBM bytes per launch of the dominant kernel, from two rocprofv3 counter runs
# (FETCH_SIZE, WRITE_SIZE scaled by a copy kernel of known size), recorded with
# a hash of the kernel's sources: reported only while those sources are unchanged.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_{workload}.json")
PROBE_LIB = os.path.join(ROOT, "sparse_mixture_experts_fp32_amd", "libmoe_probe.so")
FLUSH_BYTES = 512 << 20  # read between cold-cache calls: twice the last-level cache
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill",
                    help="named workload (prefill is the headline: T=8192 d=7168 E=256 k=4 h=2048; "
                         "'latent' times the Stable LatentMoE layer instead)")
    ap.add_argument("--cpu-experts", type=int, default=128,
                    help="experts the CPU oracle runs in its bounded sample (0 = skip the CPU baseline)")
    ap.add_argument("--experts", choices=["bf16", "mxfp4"], default="bf16",
                    help="expert weight format: bf16, or MXFP4 weights with MXFP8 activations (weights quantised "
                         "once before the timed steps)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure this chip's read, direct-to-LDS read, copy and bf16 matrix-core ceilings and "
                         "print them as one JSON line")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, run a plain float32 copy kernel (out = -in) over this many MiB three "
                         "times, so that a counter run can scale FETCH_SIZE / WRITE_SIZE by a known byte count")
    return ap.parse_args()


class Layer:
    """Preallocated buffers and C-ABI calls for one workload."""

    def __init__(self, lib, inp, cfg, dev, weights):
        """weights: the packed (w_gate, w_up, w_down) of the workload."""
        import torch
        self.lib, self.inp, self.cfg, self.dev = lib, inp, cfg, dev
        self.weights = weights
        T, d, E, k, h = cfg.T, cfg.d, cfg.E, cfg.k, cfg.h
        n = T * k
        e = lambda *s, dt: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        self.logits = e(T, E, dt=torch.float32)
        self.idx = e(T, k, dt=torch.int32)
        self.w = e(T, k, dt=torch.float32)
        self.offsets = e(E + 1, dt=torch.int32)
        self.row_of = e(T, k, dt=torch.int32)
        self.row_src = e(n, dt=torch.int32)
        self.h_act = e(n, h, dt=torch.bfloat16)
        self.y_rows = e(n, d, dt=torch.float32)
        self.out = e(T, d, dt=torch.float32)
        self.shape = lib.shape(T, d, E, k, h)
        self.ws_route = e(max(1, lib.workspace_bytes(self.shape, lib.MOE_CALL_ROUTE)), dt=torch.uint8)
        self.ws_perm = e(max(1, lib.workspace_bytes(self.shape, lib.MOE_CALL_PERMUTE)), dt=torch.uint8)
        self.ws_ffn = e(max(1, lib.workspace_bytes(self.shape, lib.MOE_CALL_EXPERT_FFN)), dt=torch.uint8)
        self.stream = torch.cuda.current_stream(dev)
        P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.P = P
        self.sh = ctypes.byref(self.shape)
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)

    def step(self, ev=None):
        L, P, sh, sp, i = self.lib.lib, self.P, self.sh, self.sp, self.inp
        c = self.lib.check
        c(L.moe_route(sh, P(i.x), P(i.w_router), P(i.router_bias), P(self.logits), P(self.idx), P(self.w),
                      P(self.ws_route), self.ws_route.numel(), sp))
        c(L.moe_permute(sh, None, P(self.idx), P(self.offsets), P(self.row_of), P(self.row_src), None,
                        P(self.ws_perm), self.ws_perm.numel(), sp))
        if ev is not None:
            ev[0].record(self.stream)
        wg, wu, wd = self.weights
        c(L.moe_expert_gate_up(sh, P(i.x), P(self.row_src), P(self.offsets), P(wg), P(wu), P(self.h_act),
                               P(self.ws_ffn), self.ws_ffn.numel(), sp))
        if ev is not None:
            ev[1].record(self.stream)
        c(L.moe_expert_down(sh, P(self.h_act), P(self.offsets), P(wd), P(self.y_rows), P(self.ws_ffn),
                            self.ws_ffn.numel(), sp))
        if ev is not None:
            ev[2].record(self.stream)
        c(L.moe_combine(sh, P(self.y_rows), P(self.row_of), P(self.w), P(self.out), sp))


def time_hbm_kernels(layer, reps):
    """Mean time of the routing top-k, permute (with and without the x_perm gather) and combine
    calls, each on its own, on the step's buffers (HIP events on the layer's stream; each rewrites
    the values the step wrote), and the rate of each in algorithmic bytes: every input read once,
    every output written once."""
    import torch
    L, P, sh, sp, c = layer.lib.lib, layer.P, layer.sh, layer.sp, layer.lib.check
    cfg = layer.cfg
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    calls = {
        "topk_softmax": (lambda: c(L.moe_topk_softmax(sh, P(layer.logits), P(layer.idx), P(layer.w), sp)),
                         4.0 * T * E + 8.0 * T * k, "hbm"),
        "permute": (lambda: c(L.moe_permute(sh, None, P(layer.idx), P(layer.offsets), P(layer.row_of),
                                            P(layer.row_src), None, P(layer.ws_perm), layer.ws_perm.numel(), sp)),
                    4.0 * T * k + 4.0 * (E + 1) + 8.0 * T * k, "latency"),
        "combine": (lambda: c(L.moe_combine(sh, P(layer.y_rows), P(layer.row_of), P(layer.w), P(layer.out), sp)),
                    4.0 * T * k * d + 8.0 * T * k + 4.0 * T * d, "hbm"),
    }
    # the dispatch gather as moe_permute's optional x_perm output (the layer fuses it into the gate/up pass):
    # the permute's bytes plus x read once and x_perm written once
    x_perm = torch.empty(T * k, d, dtype=torch.bfloat16, device=layer.dev)
    calls["permute_gather"] = (
        lambda: c(L.moe_permute(sh, P(layer.inp.x), P(layer.idx), P(layer.offsets), P(layer.row_of),
                                P(layer.row_src), P(x_perm), P(layer.ws_perm), layer.ws_perm.numel(), sp)),
        4.0 * T * k + 4.0 * (E + 1) + 8.0 * T * k + 2.0 * T * d + 2.0 * T * k * d, "hbm")
    out = {"reps": reps, "cold": f"{FLUSH_BYTES >> 20} MiB of scratch read before each cold call (a read evicts the "
                                  "caches with clean lines; a written flush leaves dirty lines whose write-back "
                                  "would be timed with the call)"}
    probe = ctypes.CDLL(PROBE_LIB)
    probe.moe_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=layer.dev)
    tiles_out = torch.empty(FLUSH_BYTES // 32768 + 1, dtype=torch.int32, device=layer.dev)

    def timed(fn, cold):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            if cold:
                probe.moe_probe_read_tiles(P(flush), FLUSH_BYTES, P(tiles_out), sp)
            a.record(layer.stream)
            fn()
            b.record(layer.stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3

    # a size-matched reference: the one-pass read probe (libmoe_probe.so) over as many bytes as
    # the call moves, timed the same way, shows what one launch of that size reaches on this chip
    for name, (call, nbytes, bound) in calls.items():
        for _ in range(3):
            call()
        us, us_cold = timed(call, False), timed(call, True)
        gbs, gbs_cold = nbytes / (us * 1e-6) / 1e9, nbytes / (us_cold * 1e-6) / 1e9
        rec = {"us": us, "us_cold": us_cold, "bytes": nbytes, "gbs": gbs, "gbs_cold": gbs_cold,
               "hbm_frac": gbs / HBM_PEAK_GBS, "hbm_frac_cold": gbs_cold / HBM_PEAK_GBS, "bound": bound}
        if bound == "hbm":  # the >= 70 % of HBM target, judged on the cold rate
            rec["target_70pct_met"] = gbs_cold / HBM_PEAK_GBS >= 0.70
            nb = int(nbytes) // 16 * 16
            buf = torch.ones(nb // 4, dtype=torch.float32, device=layer.dev)
            rout = torch.empty(nb // 32768 + 1, dtype=torch.int32, device=layer.dev)
            read = lambda: probe.moe_probe_read_tiles(P(buf), nb, P(rout), sp)  # noqa: E731
            for _ in range(3):
                read()
            r_us, r_us_cold = timed(read, False), timed(read, True)
            del buf, rout
            rec["plain_read_same_bytes"] = {"us": r_us, "us_cold": r_us_cold, "gbs": nb / (r_us * 1e-6) / 1e9,
                                            "gbs_cold": nb / (r_us_cold * 1e-6) / 1e9,
                                            "hbm_frac_cold": nb / (r_us_cold * 1e-6) / 1e9 / HBM_PEAK_GBS}
            rec["frac_of_plain_read_cold"] = r_us_cold / us_cold
        out[name] = rec
    del flush, tiles_out
    return out


def measure_ceilings(dev, note, nbytes=4 << 30, reps=5):
    """What this chip reaches: GB/s of a plain read, of the direct-to-LDS read the expert GEMM
    uses and of a copy (bytes read + written) over buffers far larger than the last-level
    cache, and TFLOP/s of back-to-back 16x16x32 bf16 matrix-core products (libmoe_probe.so;
    each probe's result is checked)."""
    import numpy as np
    import torch
    L = ctypes.CDLL(PROBE_LIB)
    for n in ("moe_probe_read", "moe_probe_dma_read"):
        getattr(L, n).argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.moe_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.moe_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def timed(fn):
        for _ in range(2):
            assert fn() == 0
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            assert fn() == 0
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3  # seconds per call

    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
    want = int(buf.to(torch.int64).sum().item()) % (1 << 32)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {"bytes": nbytes, "reps": reps}
    for key, fn in (("read_gbs", L.moe_probe_read), ("dma_read_gbs", L.moe_probe_dma_read)):
        t = timed(lambda: fn(P(buf), nbytes, P(sink), st))
        sink.zero_()
        assert fn(P(buf), nbytes, P(sink), st) == 0
        torch.cuda.synchronize()
        assert int(sink.cpu().numpy().astype(np.uint32)[0]) == want, f"{key}: probe checksum differs"
        out[key] = nbytes / t / 1e9
    dst = torch.empty_like(buf)
    half = nbytes // 2
    src_h, dst_h = buf[: half // 4], dst[: half // 4]
    t = timed(lambda: L.moe_probe_copy(P(src_h), P(dst_h), half, st))
    assert torch.equal(src_h, dst_h), "copy probe did not copy"
    out["copy_gbs"] = 2 * half / t / 1e9
    del buf, dst, src_h, dst_h
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    waves, iters = cus * 8, 4096
    msink = torch.empty(waves, dtype=torch.float32, device=dev)
    t = timed(lambda: L.moe_probe_mfma(waves, iters, P(msink), st))
    assert torch.all(msink == 16 * 32 * iters), "matrix-core probe sums differ"
    out["mfma_bf16_tflops"] = waves * iters * 16 * 16384.0 / t / 1e12
    out["mfma_bf16_frac_of_peak"] = out["mfma_bf16_tflops"] / MFMA_BF16_PEAK_TFLOPS
    for key in ("read_gbs", "dma_read_gbs", "copy_gbs"):
        out[key.replace("_gbs", "_frac_of_peak")] = out[key] / HBM_PEAK_GBS
    out["compute_units"] = cus
    note(f"ceilings: read {out['read_gbs']:.0f} GB/s, direct-to-LDS read {out['dma_read_gbs']:.0f} GB/s, "
         f"copy {out['copy_gbs']:.0f} GB/s, bf16 matrix cores {out['mfma_bf16_tflops']:.0f} TFLOP/s")
    return out


class Balance:
    """Buffers and C-ABI calls of the load-balancing step on a layer's logits."""

    BINS, LO, WIDTH = 1000, -16.0, 0.03125

    def __init__(self, layer):
        import torch
        lib, cfg, dev = layer.lib, layer.cfg, layer.dev
        self.layer, self.lib = layer, lib
        T, E, k = cfg.T, cfg.E, cfg.k
        e = lambda *s, dt: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        self.bias = torch.zeros(E, dtype=torch.float32, device=dev)
        self.idx = e(T, k, dt=torch.int32)
        self.w = e(T, k, dt=torch.float32)
        self.alpha = e(T, dt=torch.float32)
        self.hist = e(E, self.BINS, dt=torch.int32)
        self.prob_mean = e(E, dt=torch.float32)
        self.aux = e(1, dt=torch.float32)
        self.ws_aux = e(max(1, lib.workspace_bytes(layer.shape, lib.MOE_CALL_AUX_LOSS)), dt=torch.uint8)
        self.ok = k < E and k <= 63  # Quantile Balancing selects k + 1 experts

    def step(self, ev=None):
        """QB route, histogram, update (bias updated in place), then the aux loss."""
        L, P, sh, sp, c = self.lib.lib, self.layer.P, self.layer.sh, self.layer.sp, self.lib.check
        st = self.layer.stream
        rec = (lambda i: ev[i].record(st)) if ev is not None else (lambda i: None)
        f = ctypes.c_float
        rec(0)
        if self.ok:
            c(L.moe_qb_route(sh, P(self.layer.logits), P(self.bias), P(self.idx), P(self.w), P(self.alpha), sp))
            rec(1)
            c(L.moe_qb_histogram(sh, P(self.layer.logits), P(self.alpha), f(self.LO), f(self.WIDTH), self.BINS,
                                 P(self.hist), sp))
            rec(2)
            c(L.moe_qb_update(sh, P(self.hist), f(self.LO), f(self.WIDTH), self.BINS, P(self.bias), P(self.bias), sp))
        else:
            rec(1)
            rec(2)
        rec(3)
        c(L.moe_aux_loss(sh, P(self.layer.logits), P(self.prob_mean), P(self.aux), P(self.ws_aux),
                         self.ws_aux.numel(), sp))
        rec(4)

    def measure(self, reps):
        """Mean time of each call over `reps` steps (HIP events on the layer's stream) and its rate."""
        import torch
        cfg = self.layer.cfg
        T, E, k, B = cfg.T, cfg.E, cfg.k, self.BINS
        for _ in range(3):
            self.step()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
        for r in range(reps):
            self.step(evs[r])
        torch.cuda.synchronize()
        us = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / reps * 1e3 for i in range(4)]
        # algorithmic bytes: each input read once, each output written once
        nbytes = {"qb_route": 4.0 * T * E + 4.0 * E + 8.0 * T * k + 4.0 * T,
                  "qb_histogram": 4.0 * T * E + 4.0 * T + 4.0 * E * B,
                  "qb_update": 4.0 * E * B + 8.0 * E,
                  "aux_loss": 4.0 * T * E + 4.0 * E + 4.0}
        out = {"bins": B, "reps": reps}
        for name, t in zip(["qb_route", "qb_histogram", "qb_update", "aux_loss"], us):
            if not self.ok and name.startswith("qb_"):
                continue
            gbs = nbytes[name] / (t * 1e-6) / 1e9
            out[name] = {"us": t, "bytes": nbytes[name], "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
        return out


class MXLayer:
    """The routed layer with MXFP4 experts: preallocated buffers and C-ABI calls."""

    def __init__(self, lib, inp, cfg, dev):
        import torch

        from sparse_mixture_experts_fp32_amd import ops
        self.lib, self.inp, self.cfg, self.dev = lib, inp, cfg, dev
        T, d, E, k, h = cfg.T, cfg.d, cfg.E, cfg.k, cfg.h
        n = T * k
        e = lambda *s, dt: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        u8 = torch.uint8
        self.gate = ops.moe_mx_quantize_weights(inp.w_gate)
        self.up = ops.moe_mx_quantize_weights(inp.w_up)
        self.down = ops.moe_mx_quantize_weights(inp.w_down)
        self.logits, self.idx, self.w = e(T, E, dt=torch.float32), e(T, k, dt=torch.int32), e(T, k, dt=torch.float32)
        self.offsets, self.row_of, self.row_src = e(E + 1, dt=torch.int32), e(T, k, dt=torch.int32), e(n, dt=torch.int32)
        self.x_q, self.x_s = e(T, d, dt=u8), e(T, d // 32, dt=u8)
        self.h_act, self.h_q, self.h_s = e(n, h, dt=torch.float32), e(n, h, dt=u8), e(n, h // 32, dt=u8)
        self.y_rows, self.out = e(n, d, dt=torch.float32), e(T, d, dt=torch.float32)
        self.shape = lib.shape(T, d, E, k, h)
        self.ws_route = e(max(1, lib.workspace_bytes(self.shape, lib.MOE_CALL_ROUTE)), dt=u8)
        self.ws_perm = e(max(1, lib.workspace_bytes(self.shape, lib.MOE_CALL_PERMUTE)), dt=u8)
        self.ws_ffn = e(max(1, lib.workspace_bytes(self.shape, lib.MOE_CALL_EXPERT_FFN)), dt=u8)
        self.stream = torch.cuda.current_stream(dev)
        self.P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.sh = ctypes.byref(self.shape)
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)

    def step(self, ev=None):
        L, P, sh, sp, i, c = self.lib.lib, self.P, self.sh, self.sp, self.inp, self.lib.check
        T, d, h, n = self.cfg.T, self.cfg.d, self.cfg.h, self.cfg.T * self.cfg.k
        c(L.moe_route(sh, P(i.x), P(i.w_router), P(i.router_bias), P(self.logits), P(self.idx), P(self.w),
                      P(self.ws_route), self.ws_route.numel(), sp))
        c(L.moe_permute(sh, None, P(self.idx), P(self.offsets), P(self.row_of), P(self.row_src), None,
                        P(self.ws_perm), self.ws_perm.numel(), sp))
        c(L.moe_mx_quantize_rows(T, d, P(i.x), 0, P(self.x_q), P(self.x_s), sp))
        if ev is not None:
            ev[0].record(self.stream)
        c(L.moe_mx_expert_gate_up(sh, P(self.x_q), P(self.x_s), P(self.row_src), P(self.offsets), P(self.gate[0]),
                                  P(self.gate[1]), P(self.up[0]), P(self.up[1]), P(self.h_act), P(self.ws_ffn),
                                  self.ws_ffn.numel(), sp))
        if ev is not None:
            ev[1].record(self.stream)
        c(L.moe_mx_quantize_rows(n, h, P(self.h_act), 1, P(self.h_q), P(self.h_s), sp))
        if ev is not None:
            ev[2].record(self.stream)
        c(L.moe_mx_expert_down(sh, P(self.h_q), P(self.h_s), P(self.offsets), P(self.down[0]), P(self.down[1]),
                               P(self.y_rows), P(self.ws_ffn), self.ws_ffn.numel(), sp))
        if ev is not None:
            ev[3].record(self.stream)
        c(L.moe_combine(sh, P(self.y_rows), P(self.row_of), P(self.w), P(self.out), sp))


def mx_bench(args, lib, inp, cfg, dev, note):
    """Timed steps of the MXFP4-expert layer; returns the JSON result."""
    import torch

    from sparse_mixture_experts_fp32_amd import MXForward
    layer = MXLayer(lib, inp, cfg, dev)
    torch.cuda.synchronize()
    note("expert weights quantised to MXFP4")
    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    note(f"{args.warmup} warmup steps done")
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        layer.step(evs[s])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    note(f"{K} timed steps done")
    gate_up_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / K
    hq_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / K
    down_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / K
    fwd = MXForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev)
    ref = fwd(inp.x, inp.w_router, inp.router_bias, layer.gate, layer.up, layer.down)
    torch.cuda.synchronize()
    assert torch.equal(ref, layer.out), "bench step and moe_mx_forward disagree"
    del fwd, ref
    note("bench step equals moe_mx_forward bit for bit")
    T, d, E, k, h = cfg.T, cfg.d, cfg.E, cfg.k, cfg.h
    n = T * k
    counts = (layer.offsets[1:] - layer.offsets[:-1]).cpu()
    touched = int((counts > 0).sum())
    # algorithmic bytes of the MX gate/up pass: one E4M3 row (+ scales) per assignment,
    # the touched experts' E2M1 gate and up weights (+ scales) once, H written in float32
    w_bytes = lambda N, Kd: N * (Kd / 2 + Kd / 32)  # noqa: E731
    gu_bytes = n * (d + d / 32) + 2.0 * touched * w_bytes(h, d) + 4.0 * n * h
    gu_gbs = gu_bytes / (gate_up_ms * 1e-3) / 1e9
    dn_bytes = n * (h + h / 32) + touched * w_bytes(d, h) + 4.0 * n * d
    flops = 6.0 * n * d * h
    return {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8xfp4", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} d={d} E={E} top-{k} h={h}, SwiGLU experts in MXFP4 with MXFP8 "
                               f"activations, fp32 gate", "T": T, "d": d, "E": E, "k": k, "h": h, "seed": cfg.seed,
                   "experts_touched": touched},
        "grouped_gemm": {"ms": gate_up_ms + down_ms, "tflops": flops / ((gate_up_ms + down_ms) * 1e-3) / 1e12,
                         "mfma_frac_fp8": flops / ((gate_up_ms + down_ms) * 1e-3) / 1e12 / 5000.0,
                         "gate_up_ms": gate_up_ms, "h_quantise_ms": hq_ms, "down_ms": down_ms,
                         "down_gbs": dn_bytes / (down_ms * 1e-3) / 1e9},
        "roofline": {"kernel": "mx_ring_kernel<gated> (MX gate/up pass + SwiGLU)", "bound": "hbm",
                     "achieved": gu_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gu_gbs / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes": gu_bytes},
    }


def cpu_baseline(inp, cfg, n_experts):
    """The oracle, as it is, on the host cores over a bounded sample of the same workload.

    Timed: gate logits, softmax/top-k, permutation, gather and combine over every
    token, and the SwiGLU FFN of `n_experts` evenly spaced experts with all their
    rows. The layer time is the measured steps plus the sampled FFN time scaled by
    (rows of all experts) / (rows of the sampled experts). Copying inputs from the
    GPU to host memory is input preparation and is not timed.
    """
    import numpy as np
    import torch

    import oracle.moe_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count()
    E, k = cfg.E, cfg.k
    x_h = inp.x.cpu()
    wr_h = inp.w_router.cpu()
    b_h = None if inp.router_bias is None else inp.router_bias.cpu()
    sample = sorted({int(round(i * E / n_experts)) % E for i in range(n_experts)})
    wg = {e: inp.w_gate[e].cpu() for e in sample}
    wu = {e: inp.w_up[e].cpu() for e in sample}
    wd = {e: inp.w_down[e].cpu() for e in sample}
    t = {}
    t0 = time.perf_counter()
    L = orc.gate_logits(x_h, wr_h, b_h)
    t["gate"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    idx, w, _ = orc.route(L, k)
    t["route"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    off, row_of, row_src = orc.permute(idx, E)
    t["permute"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    x_perm = orc.gather(x_h, row_src)
    t["gather"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    H, Y = orc.expert_ffn(x_perm, off, wg, wu, wd, experts=sample)
    t["ffn_sample"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.combine(np.nan_to_num(Y), row_of, w)
    t["combine"] = time.perf_counter() - t0
    rows_all = int(off[-1])
    rows_sample = int(sum(off[e + 1] - off[e] for e in sample))
    scale = rows_all / max(rows_sample, 1)
    layer_s = t["gate"] + t["route"] + t["permute"] + t["gather"] + t["combine"] + t["ffn_sample"] * scale
    measured = sum(t.values())
    return {
        "value": cfg.T / layer_s, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": (f"{cfg.name} workload, float64 numpy oracle: gate logits, softmax/top-k, permutation, gather and "
                   f"combine over all {cfg.T} tokens; SwiGLU experts for {len(sample)} of {E} experts "
                   f"({rows_sample} of {rows_all} rows), that time scaled by {scale:.2f}; "
                   f"{measured:.1f} s of CPU work measured, {layer_s:.1f} s estimated per layer"),
        "torch_threads": torch.get_num_threads(),
        "seconds": {kk: round(v, 3) for kk, v in t.items()},
    }


def latent_bench(args, dev, note):
    """The Stable LatentMoE layer: K calls of moe_latent_forward on one stream."""
    import torch

    from synthetic import LATENT_CONFIGS, make_latent_inputs
    from sparse_mixture_experts_fp32_amd import _lib as lib

    cfg = LATENT_CONFIGS[args.workload]
    T, d, l, E, k, h, S, hs = cfg.T, cfg.d, cfg.l, cfg.E, cfg.k, cfg.h, cfg.n_shared, cfg.h_shared
    def progress(n):
        torch.cuda.synchronize()  # the line reports finished draws
        note(f"drew {n} of {E} experts' weights")

    inp = make_latent_inputs(cfg, device=dev, progress=progress)
    torch.cuda.synchronize()
    note("inputs ready")
    shape = lib.latent_shape(T, d, l, E, k, h, S, hs)
    ws = torch.empty(lib.latent_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    # every bf16 weight converted once, before timing, to the library's packed layout (the
    # row-major tensors stay for the CPU baseline)
    from sparse_mixture_experts_fp32_amd import moe_pack_weights
    wts = {}
    for key in ("w_proj_down", "w_gate", "w_up", "w_down", "w_proj_up", "shared_gate", "shared_up", "shared_down"):
        w = getattr(inp, key)
        wts[key] = None if w is None else moe_pack_weights(w)
    torch.cuda.synchronize()
    note("weights packed into matrix-core tiles")
    args_c = [ctypes.byref(shape), P(inp.x), P(inp.w_router), None, P(wts["w_proj_down"]), P(wts["w_gate"]),
              P(wts["w_up"]), P(wts["w_down"]), P(inp.rms_gain), ctypes.c_float(inp.rms_eps), P(wts["w_proj_up"]),
              P(wts["shared_gate"]), P(wts["shared_up"]), P(wts["shared_down"]), P(out), P(ws), ws.numel(),
              ctypes.c_void_p(stream.cuda_stream)]

    def step():
        lib.check(lib.lib.moe_latent_forward(*args_c))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    note(f"{args.warmup} warmup steps done")
    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(K):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    gpu_ms = start.elapsed_time(stop) / K
    note(f"{K} timed steps done")
    n = T * k
    flops = {"router": 2.0 * T * d * E, "down_projection": 2.0 * T * d * l, "routed_gate_up": 4.0 * n * l * h,
             "routed_down": 2.0 * n * l * h, "up_projection": 2.0 * T * l * d, "shared": 6.0 * S * T * d * hs}
    total = sum(flops.values())
    tflops = total / (gpu_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Stable LatentMoE, T={T} d={d} l={l} E={E} top-{k} h={h}, "
                               f"{S} shared experts of width {hs}, fp32 gate",
                   "T": T, "d": d, "l": l, "E": E, "k": k, "h": h, "n_shared": S, "h_shared": hs, "seed": cfg.seed},
        "gpu_ms_per_step": gpu_ms,
        "flops": flops,
        "roofline": {"kernel": "whole LatentMoE step (every kernel of moe_latent_forward)", "bound": "mfma",
                     "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None, "algorithmic_flops": total},
    }
    if args.cpu_experts > 0:
        note("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = latent_cpu_baseline(inp, cfg, n_tokens=16)
    return result


def latent_cpu_baseline(inp, cfg, n_tokens):
    """The LatentMoE oracle on the host cores for n_tokens evenly spaced tokens (every
    step of the layer for those tokens, the experts they route to copied to host
    memory first), scaled to the whole batch."""
    import numpy as np

    import oracle.latent as lat
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count()
    sample = np.linspace(0, cfg.T - 1, n_tokens).astype(np.int64)
    x = inp.x[sample].cpu()
    host = {name: getattr(inp, name).cpu() for name in ("w_router", "w_proj_down", "rms_gain", "w_proj_up",
                                                        "shared_gate", "shared_up", "shared_down")
            if getattr(inp, name) is not None}
    logits = (x.double() @ host["w_router"].double().T).numpy()
    need = sorted({int(e) for e in np.argsort(-logits, axis=1)[:, :cfg.k + 2].ravel()})

    class Experts(dict):
        def __init__(self, t):
            super().__init__({e: t[e].cpu() for e in need})
            self.t = t

        def __missing__(self, e):
            self[e] = self.t[e].cpu()
            return self[e]

    wg, wu, wd = Experts(inp.w_gate), Experts(inp.w_up), Experts(inp.w_down)
    t0 = time.perf_counter()
    lat.latent_forward(x, host["w_router"], None, host["w_proj_down"], wg, wu, wd, host["rms_gain"], inp.rms_eps,
                       host["w_proj_up"], host.get("shared_gate"), host.get("shared_up"), host.get("shared_down"),
                       k=cfg.k)
    sec = time.perf_counter() - t0
    layer_s = sec * cfg.T / n_tokens
    return {"value": cfg.T / layer_s, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": (f"{cfg.name} workload, float64 numpy oracle of the whole LatentMoE layer for {n_tokens} of "
                       f"{cfg.T} tokens (their experts copied to host memory beforehand); {sec:.1f} s measured, "
                       f"scaled by {cfg.T / n_tokens:.0f} to {layer_s:.0f} s per layer")}


def mx_cpu_baseline(inp, cfg, n_experts):
    """The MX oracle on the host cores: gate logits, routing, permutation and the MXFP8
    quantisation of x over every token, then n_experts evenly spaced experts (their
    weights quantised to MXFP4, their rows through the MX SwiGLU FFN), that time scaled
    by rows; the combine over every token."""
    import numpy as np

    import oracle.moe_oracle as orc
    import oracle.mx as mx
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count()
    E, k = cfg.E, cfg.k
    x_h, wr_h = inp.x.cpu(), inp.w_router.cpu()
    b_h = None if inp.router_bias is None else inp.router_bias.cpu()
    sample = sorted({int(round(i * E / n_experts)) % E for i in range(n_experts)})
    wts = {e: (inp.w_gate[e].cpu(), inp.w_up[e].cpu(), inp.w_down[e].cpu()) for e in sample}
    t = {}
    t0 = time.perf_counter()
    L = orc.gate_logits(x_h, wr_h, b_h)
    idx, w, _ = orc.route(L, k)
    off, row_of, row_src = orc.permute(idx, E)
    xq, xs = mx.quantize(x_h, mx.E4M3)
    t["routing_and_x"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    Y = np.zeros((cfg.T * k, cfg.d))
    for e in sample:
        gq, gs = mx.quantize(wts[e][0], mx.E2M1)
        uq, us = mx.quantize(wts[e][1], mx.E2M1)
        dq, ds = mx.quantize(wts[e][2], mx.E2M1)
        lo, hi = int(off[e]), int(off[e + 1])
        rows = row_src[lo:hi]
        H = mx.mx_expert_gate_up(xq[rows], xs[rows], gq, gs, uq, us)
        hq, hs = mx.quantize(H, mx.E4M3)
        Y[lo:hi] = mx.mx_expert_down(hq, hs, dq, ds)
    t["ffn_sample"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.combine(Y, row_of, w)
    t["combine"] = time.perf_counter() - t0
    rows_all = int(off[-1])
    rows_sample = int(sum(off[e + 1] - off[e] for e in sample))
    scale = E / len(sample)  # each expert's weights are quantised whatever its row count
    layer_s = t["routing_and_x"] + t["combine"] + t["ffn_sample"] * scale
    return {"value": cfg.T / layer_s, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": (f"{cfg.name} workload with MXFP4 experts, float64 numpy oracle: gate logits, routing, "
                       f"permutation, MXFP8 quantisation of x and combine over all {cfg.T} tokens; {len(sample)} of "
                       f"{E} experts quantised and run ({rows_sample} of {rows_all} rows), that time scaled by "
                       f"{scale:.0f}; {sum(t.values()):.1f} s measured, {layer_s:.0f} s estimated per layer")}


def _current_record(path, kernel):
    """A committed profile record (JSON) if it is for this kernel and the kernel's sources are
    unchanged since it was taken (their SHA-256 is in the record), else None."""
    import hashlib
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if kernel not in rec["kernel"]:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        p = os.path.join(ROOT, src)
        if not os.path.exists(p):
            return None
        with open(p, "rb") as g:
            h.update(g.read())
    return rec if h.hexdigest() == rec["sources_sha256"] else None


def measured_traffic(workload, kernel):
    """HBM bytes per gate/up launch from the committed counter record, or None if the record is for
    another kernel or the kernel's sources changed since."""
    rec = _current_record(TRAFFIC_RECORD.format(workload=workload), kernel)
    return None if rec is None else rec["traffic_bytes"]


def traced_duration(workload, kernel):
    """The kernel's average duration (us) over the timed steps of the default bench command run under
    rocprofv3 --kernel-trace (committed record), or None if the record is stale or missing."""
    rec = _current_record(os.path.join(ROOT, "profiles", f"trace_{workload}.json"), kernel)
    return None if rec is None else rec["avg_us_timed_steps"]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): the layer "
              "runs on a single GPU and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    from synthetic import CONFIGS, LATENT_CONFIGS, make_inputs
    from sparse_mixture_experts_fp32_amd import _lib as lib
    from sparse_mixture_experts_fp32_amd import MoEForward, moe_pack_weights

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.ceilings:
        note = lambda msg: print(f"[bench] {msg}", file=sys.stderr, flush=True)  # noqa: E731
        print(json.dumps({"ceilings": measure_ceilings(dev, note),
                          "peaks": {"hbm_gbs": HBM_PEAK_GBS, "mfma_bf16_tflops": MFMA_BF16_PEAK_TFLOPS}}), flush=True)
        return
    if args.copy_probe_mib > 0:
        # a plain float32 copy (out = -in) of known size, whose L2-to-fabric counters
        # calibrate those of the layer's kernels in the same profiled run
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
        print("[bench] copy probe done", file=sys.stderr, flush=True)
    if args.workload in LATENT_CONFIGS:
        note = lambda msg: print(f"[bench] {args.workload}: {msg}", file=sys.stderr, flush=True)  # noqa: E731
        print(json.dumps(latent_bench(args, dev, note)), flush=True)
        return
    cfg = CONFIGS[args.workload]
    def progress(n):
        # wait for the draws so that the line reports finished work (under a
        # counter-collecting profiler every one of the draw's thousands of small
        # kernels is serialised, and the draw can take minutes)
        torch.cuda.synchronize()
        print(f"[bench] {cfg.name}: drew {n} of {cfg.E} experts' weights", file=sys.stderr, flush=True)

    inp = make_inputs(cfg, device=dev, progress=progress)
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: inputs ready", file=sys.stderr, flush=True)
    note = lambda msg: print(f"[bench] {cfg.name}: {msg}", file=sys.stderr, flush=True)  # noqa: E731
    if args.experts == "mxfp4":
        result = mx_bench(args, lib, inp, cfg, dev, note)
        if args.cpu_experts > 0:
            note("timing the CPU oracle on a bounded sample")
            result["cpu_baseline"] = mx_cpu_baseline(inp, cfg, min(args.cpu_experts, 4))
        print(json.dumps(result), flush=True)
        return
    # once, before timing, the expert weights go into the library's packed layout (as a checkpoint
    # would be converted on loading); the row-major tensors stay for the CPU baseline
    weights = tuple(moe_pack_weights(w) for w in (inp.w_gate, inp.w_up, inp.w_down))
    torch.cuda.synchronize()
    note("expert weights packed into matrix-core tiles")
    layer = Layer(lib, inp, cfg, dev, weights)
    note("buffers allocated")

    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    note(f"{args.warmup} warmup steps done")

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(layer.stream)
    for s in range(K):
        layer.step(evs[s])
    stop.record(layer.stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / K
    note(f"{K} timed steps done")
    gpu_ms = start.elapsed_time(stop) / K
    gate_up_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / K
    down_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / K

    # the step is moe_forward's kernel sequence: the one boundary call gives the same output, bit
    # for bit, and is timed over a few calls of its own
    fwd = MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev)
    ref_out = fwd(inp.x, inp.w_router, inp.router_bias, *weights)
    torch.cuda.synchronize()
    assert torch.equal(ref_out, layer.out), "bench step and moe_forward disagree"
    note("bench step equals moe_forward bit for bit")
    reps = min(K, 10)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(layer.stream)
    for _ in range(reps):
        fwd(inp.x, inp.w_router, inp.router_bias, *weights, out=ref_out)
    b.record(layer.stream)
    torch.cuda.synchronize()
    assert torch.equal(ref_out, layer.out), "moe_forward output differs from the bench step"
    forward_calls = {"moe_forward_ms": a.elapsed_time(b) / reps, "reps": reps}
    del fwd, ref_out
    note("moe_forward calls timed")

    T, d, E, k, h = cfg.T, cfg.d, cfg.E, cfg.k, cfg.h
    n = T * k
    counts = (layer.offsets[1:] - layer.offsets[:-1]).cpu()
    touched = int((counts > 0).sum())
    gemm_flops = 6.0 * n * d * h
    gemm_tflops = gemm_flops / ((gate_up_ms + down_ms) * 1e-3) / 1e12
    # algorithmic bytes of one gate/up launch: one bf16 row of x per assignment
    # (gathered through row_src), touched experts' gate and up weights read once,
    # H written
    gu_bytes = 2.0 * n * d + 2.0 * 2 * d * h * touched + 2.0 * n * h
    gu_gbs = gu_bytes / (gate_up_ms * 1e-3) / 1e9
    down_bytes = 2.0 * n * h + 2.0 * d * h * touched + 4.0 * n * d
    down_gbs = down_bytes / (down_ms * 1e-3) / 1e9
    ms = wall_ms
    gu_name = "ffn_ring_kernel<true, false>"
    gu_kernel = gu_name + " (gate/up pass + SwiGLU)"
    result = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} d={d} E={E} top-{k} h={h}, SwiGLU experts, fp32 gate",
                   "T": T, "d": d, "E": E, "k": k, "h": h, "seed": cfg.seed,
                   "experts_touched": touched, "max_rows_per_expert": int(counts.max())},
        "gpu_ms_per_step": gpu_ms,
        "forward_calls": forward_calls,
        "grouped_gemm": {"ms": gate_up_ms + down_ms, "tflops": gemm_tflops,
                         "mfma_frac": gemm_tflops / MFMA_BF16_PEAK_TFLOPS,
                         "gate_up_ms": gate_up_ms, "down_ms": down_ms,
                         "down_gbs": down_gbs, "down_hbm_frac": down_gbs / HBM_PEAK_GBS},
        "roofline": {"kernel": gu_kernel, "bound": "hbm",
                     "achieved": gu_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gu_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(cfg.name, gu_name), "algorithmic_bytes": gu_bytes,
                     "event_us": gate_up_ms * 1e3},
    }
    trace_us = traced_duration(cfg.name, gu_name)
    if trace_us is not None:  # the same kernel's duration in the committed kernel trace
        result["roofline"]["trace_us"] = trace_us
        result["roofline"]["frac_trace"] = gu_bytes / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS
    result["ceilings"] = measure_ceilings(dev, note)
    result["roofline"]["frac_of_measured"] = gu_gbs / result["ceilings"]["dma_read_gbs"]
    out_before = layer.out.clone()
    result["hbm_kernels"] = time_hbm_kernels(layer, max(K, 10))
    torch.cuda.synchronize()
    assert torch.equal(out_before, layer.out), "re-running route / permute / combine changed the output"
    del out_before
    note("top-k, permute and combine timed on their own")
    result["balance"] = Balance(layer).measure(max(K, 10))
    note("load-balancing calls timed")
    if args.cpu_experts > 0:
        note("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_experts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
