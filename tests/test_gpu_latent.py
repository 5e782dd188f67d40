"""GPU parity of the Stable LatentMoE layer (moe_latent_forward, moe_combine_rmsnorm)
against the CPU oracle, through the C ABI.

Stage by stage, each against the oracle run on the device's own inputs to that
stage, with the bounds of tests/gpu_util.py:
  * routing ids and the permutation: bit for bit (device logits);
  * z = x W_down_proj^T and RMSNorm(u), both bf16: one round-to-nearest-even
    after float32 arithmetic, |dz| <= 2^-8 |z| + 1e-4 max|z| + 1e-6;
  * routed and shared H (bf16) and Y (float32) rows: the expert FFN bounds;
  * out = (W_up_proj r) + shared_0 + shared_1 from the device's r and shared Y:
    float32 sums, |dout| <= 1e-4 max|out| + 1e-6;
and end to end against the float64 layer with no rounding (device logits for
the routing): the device's three bf16 roundings (z, H, r) carried to the
output by the first-order model of tests/latent_bounds.py give a standard
deviation sigma per element, and the test asks for |dout| <= 8 sigma and
||dout||_2 <= 2 ||sigma||_2. Beside it, the oracle with the device's rounding
points applied (bf16_operands) must come closer still: ||dout||_2 <= ||sigma||_2.
"""
import numpy as np
import pytest
import torch

import oracle.latent as lat
import oracle.moe_oracle as orc
from synthetic import LATENT_CONFIGS, make_latent_inputs, scaled_latent
from tests import gpu_util as gu
from tests import latent_bounds as lb

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_fp32_amd  # noqa: F401  (fails loudly if libmoe.so is missing)
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def moe(dev):
    import sparse_mixture_experts_fp32_amd as m
    return m


def _packed_args(inp):
    """The layer's arguments after x with every bf16 weight matrix in the packed layout."""
    wr, b, wpd, wg, wu, wd, gain, eps, wpu, sg, su, sd = inp.args()
    pk = lambda w: None if w is None else gu.packed(w)  # noqa: E731
    return wr, b, pk(wpd), pk(wg), pk(wu), pk(wd), gain, eps, pk(wpu), pk(sg), pk(su), pk(sd)


def _run(moe, dev, inp):
    c = inp.cfg
    fwd = moe.LatentMoEForward(c.T, c.d, c.l, c.E, c.k, c.h, c.n_shared, c.h_shared, dev)
    args = _packed_args(inp)
    out = fwd(inp.x, *args)
    torch.cuda.synchronize()
    fwd.args = args
    return fwd, out


def _check_out_close(got, ref, what):
    g = gu.f64(got)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(g - r)
    bound = 1e-4 * np.abs(r).max() + 1e-6
    assert err.max() <= bound, f"{what}: max |diff| {err.max():.3e} > {bound:.3e}"


def _check_stages(moe, dev, inp, fwd, out, full=True):
    c = inp.cfg
    T, E, k = c.T, c.E, c.k
    it = fwd.intermediate
    logits = it("logits")
    gu.check_logits(logits, orc.gate_logits(inp.x, inp.w_router, inp.router_bias))
    idx_ref, _ = gu.check_route(logits, it("topk_idx"), it("topk_w"), k)
    off, row_of, row_src = gu.check_permutation(it("expert_offsets"), it("row_of"), it("row_src"), idx_ref, E)
    # z = x W_down_proj^T, bf16
    z_ref = gu.f64(inp.x) @ gu.f64(inp.w_proj_down).T
    gu.check_h_rows(it("z"), z_ref, "z")
    # routed experts on the device's z
    z_dev = gu.f64(it("z"))
    H_dev, Y_dev = it("h_act"), it("y_rows")
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        He, Ye = orc.expert_swiglu(z_dev[row_src[lo:hi]], inp.w_gate[e], inp.w_up[e], inp.w_down[e])
        gu.check_h_rows(H_dev[lo:hi], He, f"routed H of expert {e}")
        gu.check_y_rows(Y_dev[lo:hi], Ye, He, inp.w_down[e], f"routed Y of expert {e}")
    # RMSNorm of u = sum_j w_j Y_j, from the device's Y and weights
    u_ref = orc.combine(gu.f64(Y_dev), gu.host(it("row_of")).to(torch.int64).numpy(), gu.f64(it("topk_w")))
    r_ref = lat.rmsnorm(u_ref, gu.f64(inp.rms_gain), inp.rms_eps)
    gu.check_h_rows(it("r"), r_ref, "RMSNorm(u)")
    # shared experts on x
    up = gu.f64(it("r")) @ gu.f64(inp.w_proj_up).T
    for s in range(c.n_shared):
        Hs, Ys = orc.expert_swiglu(gu.f64(inp.x), inp.shared_gate[s], inp.shared_up[s], inp.shared_down[s])
        gu.check_h_rows(it("shared_h")[s * T:(s + 1) * T], Hs, f"shared H {s}")
        gu.check_y_rows(it("shared_y")[s * T:(s + 1) * T], Ys, Hs, inp.shared_down[s], f"shared Y {s}")
        up = up + gu.f64(it("shared_y")[s * T:(s + 1) * T])
    _check_out_close(out, up, "out from the device's r and shared rows")
    if full:  # end to end, the oracle's own z, H, u, r (device logits for the routing)
        return _check_end_to_end(inp, out, gu.f64(logits), k)


def _check_end_to_end(inp, out, logits, k, x=None, w_gate=None, w_up=None, w_down=None):
    """The device's out against the float64 layer under the rounding model, then against the
    oracle with the device's rounding points applied (a closer match). `x` and the expert
    tensors default to the input's (the full-size test passes sampled tokens and lazy views)."""
    x = inp.x if x is None else x
    wts = [inp.w_gate if w_gate is None else w_gate, inp.w_up if w_up is None else w_up,
           inp.w_down if w_down is None else w_down]
    args = (inp.w_router, inp.router_bias, inp.w_proj_down, *wts, inp.rms_gain, inp.rms_eps, inp.w_proj_up,
            inp.shared_gate, inp.shared_up, inp.shared_down)
    ref = lat.latent_forward(x, *args, k=k, logits=logits, bf16_operands=False)
    sigma = lb.latent_output_sigma(x, inp.w_proj_down, *wts, inp.rms_gain, inp.rms_eps, inp.w_proj_up,
                                   inp.shared_gate, inp.shared_up, inp.shared_down, ref)
    ratio, worst, max_rel, mean_abs = lb.check_latent_out(out, ref["out"], sigma, "latent out")
    rounded = lat.latent_forward(x, *args, k=k, logits=logits, bf16_operands=True)
    ratio_r, _, _, _ = lb.check_latent_out(out, rounded["out"], sigma, "latent out (bf16 operands)", factor=1.0)
    print(f"  end to end: error norm {ratio:.2f} sigma (worst element {worst:.1f} sigma), max rel {max_rel:.2e}, "
          f"mean abs {mean_abs:.2e}; against the rounded oracle {ratio_r:.2f} sigma", flush=True)
    return ratio, ratio_r


CASES = {
    "tiny": dict(),
    "no_shared": dict(n_shared=0, h_shared=0),
    "ragged": dict(T=77, d=128, l=256, E=12, k=3, h=256, n_shared=1, h_shared=256),
    "one_token": dict(T=1, E=5, k=2),
    "k_equals_E": dict(T=40, E=4, k=4),
    "many_tiles": dict(T=1000, d=512, l=384, E=70, k=4, h=128, n_shared=2, h_shared=256),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_latent_forward_matches_oracle(dev, moe, case):
    cfg = scaled_latent("latent_tiny", name=f"latent_{case}", **CASES[case])
    print(f"latent case {case}: {cfg}", flush=True)
    inp = make_latent_inputs(cfg)
    inp_d = make_latent_inputs(cfg, device=dev, gen_device="cpu")
    fwd, out = _run(moe, dev, inp_d)
    _check_stages(moe, dev, inp, fwd, out)


@pytest.mark.parametrize("seed", range(6))
def test_latent_forward_random_shapes(dev, moe, seed):
    """Seeded LatentMoE shapes: ragged token counts, latent widths below and above d, zero to three
    shared experts."""
    r = np.random.default_rng(3000 + seed)
    E = int(r.integers(1, 65))
    S = int(r.integers(0, 4))
    over = dict(T=int(r.integers(1, 301)), d=int(r.choice([128, 256, 512])), l=int(r.choice([128, 256, 384])),
                E=E, k=int(r.integers(1, min(E, 8) + 1)), h=int(r.choice([128, 256])), n_shared=S,
                h_shared=int(r.choice([128, 256])) if S else 0)
    cfg = scaled_latent("latent_tiny", name=f"latent_random_{seed}", seed=400 + seed, **over)
    print(f"latent random {seed}: {cfg}", flush=True)
    inp = make_latent_inputs(cfg)
    inp_d = make_latent_inputs(cfg, device=dev, gen_device="cpu")
    fwd, out = _run(moe, dev, inp_d)
    _check_stages(moe, dev, inp, fwd, out)


def test_latent_forward_deterministic(dev, moe):
    cfg = scaled_latent("latent_tiny", T=300, E=16, k=4)
    inp = make_latent_inputs(cfg, device=dev, gen_device="cpu")
    fwd, a = _run(moe, dev, inp)
    a = a.clone()
    b = fwd(inp.x, *fwd.args)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("T,l,k", [(50, 128, 2), (33, 3584, 16), (9, 8192, 4), (130, 384, 1)])
def test_combine_rmsnorm_host_rows(dev, moe, T, l, k):
    """Host-made expert rows, weights and gain (some row_of entries -1): u in slot
    order as moe_combine, r within one bf16 rounding of the oracle's RMSNorm(u)."""
    r = np.random.default_rng(T + l)
    n = T * k
    Y = r.standard_normal((n, l)).astype(np.float32)
    row_of = r.permutation(n).reshape(T, k).astype(np.int32)
    row_of[0, 0] = -1
    w = r.random((T, k)).astype(np.float32)
    gain = (1 + 0.1 * r.standard_normal(l)).astype(np.float32)
    eps = 1e-5
    td = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    rr, uu = moe.moe_combine_rmsnorm(td(Y), td(row_of), td(w), td(gain), eps, want_u=True)
    u_plain = moe.moe_combine(td(Y), td(row_of), td(w))
    torch.cuda.synchronize()
    assert torch.equal(uu, u_plain), "u must equal moe_combine's sum bit for bit"
    ro = row_of.astype(np.int64)
    u_ref = np.zeros((T, l))
    for j in range(k):
        ok = ro[:, j] >= 0
        u_ref[ok] += w[ok, j:j + 1].astype(np.float64) * Y[ro[ok, j]].astype(np.float64)
    gu.check_h_rows(rr, lat.rmsnorm(u_ref, gain, eps), "RMSNorm(u)")


@pytest.mark.slow
def test_latent_full_size_sampled(dev, moe):
    """The page's layer (T = 16384, d = 7168, l = 3584, E = 896, k = 16, two shared
    experts): every routing id and the whole permutation bit for bit; z, r and
    out of sampled tokens against the oracle computed for those tokens alone."""
    cfg = LATENT_CONFIGS["latent"]
    print("latent full size: drawing inputs", flush=True)
    inp = make_latent_inputs(cfg, device=dev)
    fwd, out = _run(moe, dev, inp)
    print("latent full size: forward done", flush=True)
    it = fwd.intermediate
    logits = it("logits")
    idx_ref, _ = gu.check_route(logits, it("topk_idx"), it("topk_w"), cfg.k)
    gu.check_permutation(it("expert_offsets"), it("row_of"), it("row_src"), idx_ref, cfg.E)
    sample = np.array([0, 1, 4097, 9000, 12345, cfg.T - 1])
    lazy = gu.LazyExperts
    xs = inp.x[sample]
    gu.check_h_rows(it("z")[sample], gu.f64(xs) @ gu.f64(inp.w_proj_down).T, "z (sampled)")
    # r of the sampled tokens from the device's own expert rows
    ro = gu.host(it("row_of")).to(torch.int64).numpy()[sample]
    wv = gu.f64(it("topk_w"))[sample]
    Y = it("y_rows")
    u_ref = np.zeros((len(sample), cfg.l))
    for j in range(cfg.k):
        u_ref += wv[:, j:j + 1] * gu.f64(Y[torch.from_numpy(ro[:, j]).to(dev)])
    gu.check_h_rows(it("r")[sample], lat.rmsnorm(u_ref, gu.f64(inp.rms_gain), inp.rms_eps), "r (sampled)")
    _check_end_to_end(inp, out[sample], gu.f64(logits)[sample], cfg.k, x=xs, w_gate=lazy(inp.w_gate),
                      w_up=lazy(inp.w_up), w_down=lazy(inp.w_down))
