"""GPU tests of the packed expert-weight layout: packing moves every element to
the place include/moe.h states (bit for bit), and every *_packed call gives
bitwise the result of its row-major counterpart (the same products in the same
order), from tiny layers to the full prefill layer."""
import numpy as np
import pytest
import torch

from synthetic import CONFIGS, make_inputs, scaled_config

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


def _unpack(p):
    """Packed [G, N, K] -> row-major: tile (n // 16, k // 32) is 512 contiguous elements,
    element (r, c) of it at (r + 16 * (c // 8)) * 8 + c % 8."""
    G, N, K = p.shape
    t = p.reshape(G, N // 16, K // 32, 4, 16, 8)  # (.., column group c // 8, row r, c % 8)
    return t.permute(0, 1, 4, 2, 3, 5).reshape(G, N, K)


@pytest.mark.parametrize("G,N,K", [(3, 32, 128), (2, 48, 96), (1, 2048, 7168)])
def test_pack_weights_layout(dev, moe, G, N, K):
    g = torch.Generator(device="cpu").manual_seed(G * N + K)
    w = torch.randn((G, N, K), generator=g).to(torch.bfloat16).to(dev)
    p = moe.moe_pack_weights(w)
    torch.cuda.synchronize()
    assert torch.equal(_unpack(p.view(torch.int16)).view(torch.bfloat16), w)


CASES = {
    "tiny": dict(),
    "ragged": dict(T=77, d=256, E=12, k=3, h=384),
    "many_tiles": dict(T=1000, d=128, E=3, k=2, h=256),
    "one_token": dict(T=1, E=5, k=2),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_packed_equals_rowmajor(dev, moe, case):
    cfg = scaled_config("tiny", name=f"packed_{case}", **CASES[case])
    di = make_inputs(cfg).to(dev)
    ref = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev)(di.x, di.w_router, di.router_bias, di.w_gate,
                                                                di.w_up, di.w_down)
    pw = [moe.moe_pack_weights(w) for w in (di.w_gate, di.w_up, di.w_down)]
    fwd = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev, packed=True)
    out = fwd(di.x, di.w_router, di.router_bias, *pw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.slow
def test_forward_packed_equals_rowmajor_prefill(dev, moe):
    cfg = CONFIGS["prefill"]
    print("packed prefill: drawing inputs", flush=True)
    inp = make_inputs(cfg, device=dev)
    ref = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev)(inp.x, inp.w_router, None, inp.w_gate, inp.w_up,
                                                                inp.w_down)
    torch.cuda.synchronize()
    ref = ref.clone()
    packed = []
    for name in ("w_gate", "w_up", "w_down"):  # one tensor at a time, freeing the row-major one
        w = getattr(inp, name)
        packed.append(moe.moe_pack_weights(w))
        setattr(inp, name, None)
        del w
    out = moe.MoEForward(cfg.T, cfg.d, cfg.E, cfg.k, cfg.h, dev, packed=True)(inp.x, inp.w_router, None, *packed)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def _pack_latent(moe, inp):
    """The LatentMoE layer's bf16 weights in packed order (2-D projections as one group each)."""
    one = lambda w: moe.moe_pack_weights(w.unsqueeze(0)).squeeze(0)  # noqa: E731
    S = inp.cfg.n_shared
    return dict(w_proj_down=one(inp.w_proj_down), w_gate=moe.moe_pack_weights(inp.w_gate),
                w_up=moe.moe_pack_weights(inp.w_up), w_down=moe.moe_pack_weights(inp.w_down),
                w_proj_up=one(inp.w_proj_up),
                shared_gate=moe.moe_pack_weights(inp.shared_gate) if S > 0 else None,
                shared_up=moe.moe_pack_weights(inp.shared_up) if S > 0 else None,
                shared_down=moe.moe_pack_weights(inp.shared_down) if S > 0 else None)


def _latent_pair(moe, dev, inp):
    c = inp.cfg
    ref = moe.LatentMoEForward(c.T, c.d, c.l, c.E, c.k, c.h, c.n_shared, c.h_shared, dev)(inp.x, *inp.args())
    torch.cuda.synchronize()
    ref = ref.clone()
    p = _pack_latent(moe, inp)
    fwd = moe.LatentMoEForward(c.T, c.d, c.l, c.E, c.k, c.h, c.n_shared, c.h_shared, dev, packed=True)
    out = fwd(inp.x, inp.w_router, inp.router_bias, p["w_proj_down"], p["w_gate"], p["w_up"], p["w_down"],
              inp.rms_gain, inp.rms_eps, p["w_proj_up"], p["shared_gate"], p["shared_up"], p["shared_down"])
    torch.cuda.synchronize()
    return ref, out


LATENT_CASES = {
    "tiny": dict(),
    "ragged": dict(T=77, d=384, l=256, E=12, k=3, h=384, n_shared=1, h_shared=128),
    "no_shared": dict(T=40, n_shared=0),
    "many_tiles": dict(T=1000, d=512, l=384, E=70, k=4, h=128, n_shared=2, h_shared=256),
}


@pytest.mark.parametrize("case", sorted(LATENT_CASES))
def test_latent_packed_equals_rowmajor(dev, moe, case):
    from synthetic import make_latent_inputs, scaled_latent
    cfg = scaled_latent("latent_tiny", name=f"latent_packed_{case}", **LATENT_CASES[case])
    print(f"latent packed case {case}: {cfg}", flush=True)
    inp = make_latent_inputs(cfg, device=dev, gen_device="cpu")
    ref, out = _latent_pair(moe, dev, inp)
    assert torch.equal(out, ref)


@pytest.mark.slow
def test_latent_packed_equals_rowmajor_full_size(dev, moe):
    from synthetic import LATENT_CONFIGS, make_latent_inputs
    cfg = LATENT_CONFIGS["latent"]
    print("latent packed full size: drawing inputs", flush=True)
    inp = make_latent_inputs(cfg, device=dev)
    ref, out = _latent_pair(moe, dev, inp)
    assert torch.equal(out, ref)
