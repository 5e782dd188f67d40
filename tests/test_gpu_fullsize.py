"""GPU parity at the full workload sizes (one moe_forward call). The oracle
checks what it can compute in seconds: gate logits of sampled tokens, every
routing id and weight, the whole permutation, sampled x_perm rows, every H and
Y row of two experts (a sample of rows for a very large expert), and the layer
output of sampled tokens computed one by one through their own experts. The
forward on packed expert weights, the configuration the benchmark times, must
then give the same output bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as orc
from synthetic import CONFIGS, make_inputs
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_fp32_amd as m
    return m


@pytest.mark.parametrize("name", ["decode", "prefill", "many_expert", "skewed"])
def test_full_size_layer(moe, name):
    cfg = CONFIGS[name]
    dev = torch.device("cuda:0")
    print(f"\n[full-size] {cfg}", flush=True)
    inp = make_inputs(cfg, device=dev)
    fwd = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev)
    out = fwd(inp.x, inp.w_router, inp.router_bias, inp.w_gate, inp.w_up, inp.w_down)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg.seed)
    x_h = inp.x.cpu()
    wr_h = inp.w_router.cpu()
    b_h = None if inp.router_bias is None else inp.router_bias.cpu()

    logits = fwd.intermediate("logits").cpu()
    rows = rng.choice(cfg.T, size=min(64, cfg.T), replace=False)
    gu.check_logits(logits[rows], orc.gate_logits(x_h[rows], wr_h, b_h))
    idx_ref, w_ref = gu.check_route(logits, fwd.intermediate("topk_idx"), fwd.intermediate("topk_w"), cfg.k)
    off, row_of, row_src = gu.check_permutation(fwd.intermediate("expert_offsets"), fwd.intermediate("row_of"),
                                                fwd.intermediate("row_src"), idx_ref, cfg.E)
    counts = np.diff(off)
    print(f"[full-size] rows per expert: max {counts.max()}, mean {counts.mean():.1f}, "
          f"empty {(counts == 0).sum()} of {cfg.E}", flush=True)
    # the standalone dispatch gather on the forward pass's routing: sampled rows of x_perm
    n = cfg.T * cfg.k
    xr = rng.choice(n, size=min(512, n), replace=False)
    _, _, rs2, xp = moe.moe_permute(inp.x, fwd.intermediate("topk_idx"), cfg.E)
    torch.cuda.synchronize()
    assert torch.equal(rs2.cpu(), torch.from_numpy(row_src.astype(np.int32)))
    assert torch.equal(xp[torch.from_numpy(xr).to(dev)].cpu(), x_h[torch.from_numpy(row_src[xr])])
    del xp, rs2

    # every H / Y row of two experts (at most 512 sampled rows of a very large one)
    nonempty = np.flatnonzero(counts)
    for e in {int(np.argmax(counts)), int(rng.choice(nonempty))}:
        lo, hi = int(off[e]), int(off[e + 1])
        sel = np.arange(lo, hi)
        if sel.size > 512:
            sel = np.sort(rng.choice(sel, size=512, replace=False))
        X = x_h[torch.from_numpy(row_src[sel])]
        wg, wu, wd = inp.w_gate[e].cpu(), inp.w_up[e].cpu(), inp.w_down[e].cpu()
        H_ref, Y_ref = orc.expert_swiglu(X, wg, wu, wd)
        st = torch.from_numpy(sel).to(dev)
        gu.check_h_rows(fwd.intermediate("h_act")[st].cpu(), H_ref, what=f"H expert {e}")
        gu.check_y_rows(fwd.intermediate("y_rows")[st].cpu(), Y_ref, H_ref, wd, what=f"Y expert {e}")

    # layer output of sampled tokens, each through its own experts
    toks = np.sort(rng.choice(cfg.T, size=min(4, cfg.T), replace=False))
    ref = orc.forward(x_h[toks], wr_h, b_h, gu.LazyExperts(inp.w_gate), gu.LazyExperts(inp.w_up),
                      gu.LazyExperts(inp.w_down), cfg.k, logits=logits[toks])
    max_rel, mean_abs = gu.check_layer(out[torch.from_numpy(toks).to(dev)].cpu(), ref["out"])
    print(f"[full-size] {name}: sampled out max rel {max_rel:.2e}, mean abs {mean_abs:.2e}", flush=True)
    del fwd
    # the benchmarked configuration: packed expert weights, the same output bit for bit
    packed = [moe.moe_pack_weights(w) for w in (inp.w_gate, inp.w_up, inp.w_down)]
    out_p = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev, packed=True)(inp.x, inp.w_router,
                                                                                inp.router_bias, *packed)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out), "packed-weight forward differs from the row-major forward"
    print(f"[full-size] {name}: packed-weight forward equal bit for bit", flush=True)
    del packed, out_p, out, inp
    torch.cuda.empty_cache()
