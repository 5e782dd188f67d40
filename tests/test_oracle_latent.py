"""CPU tests: the LatentMoE oracle against its pins, and planted mistakes that
the pins must catch."""
import numpy as np
import pytest

import oracle.latent as lat
import oracle.moe_oracle as orc
from tests import pins_latent as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_latent_pin(pin):
    pin(lat)


# ---------------------------------------------------------------- planted mistakes

f64 = orc.f64
_real_forward = lat.latent_forward


def _rms_no_sqrt(u, gain, eps):
    U = f64(u)
    return U / (np.mean(U * U, axis=-1, keepdims=True) + eps) * f64(gain)


def _rms_sum(u, gain, eps):
    U = f64(u)
    return U / np.sqrt(np.sum(U * U, axis=-1, keepdims=True) + eps) * f64(gain)


def _rms_no_gain(u, gain, eps):
    U = f64(u)
    return U / np.sqrt(np.mean(U * U, axis=-1, keepdims=True) + eps)


def _rms_eps_outside(u, gain, eps):
    U = f64(u)
    return U / (np.sqrt(np.mean(U * U, axis=-1, keepdims=True)) + eps) * f64(gain)


def _bf16_truncate(a):
    import torch
    t = torch.as_tensor(np.asarray(a, dtype=np.float32)).view(torch.int32)
    return (t & ~0xFFFF).view(torch.float32).to(torch.float64).numpy()


def _forward_norm_after_up(x, w_router, bias, w_proj_down, w_gate, w_up, w_down, gain, eps, w_proj_up,
                           shared_gate, shared_up, shared_down, k, logits=None, bf16_operands=False):
    X = f64(x)
    E = f64(w_router).shape[0]
    L = orc.gate_logits(X, w_router, bias) if logits is None else f64(logits)
    idx, w, _ = orc.route(L, k)
    off, row_of, row_src = orc.permute(idx, E)
    z = X @ f64(w_proj_down).T
    _, Y = orc.expert_ffn(z[row_src], off, w_gate, w_up, w_down)
    u = orc.combine(Y, row_of, w)
    up = u @ f64(w_proj_up).T
    up = up / np.sqrt(np.mean(up * up, axis=-1, keepdims=True) + eps)
    shared = [lat.dense_swiglu(X, shared_gate[s], shared_up[s], shared_down[s]) for s in range(len(shared_gate))]
    out = up + sum(shared) if shared else up
    return dict(idx=idx, z=z, u=u, r=u, up=up, shared=shared, out=out)


def _forward_shared_inside_norm(x, w_router, bias, w_proj_down, w_gate, w_up, w_down, gain, eps, w_proj_up,
                                shared_gate, shared_up, shared_down, k, logits=None, bf16_operands=False):
    res = _real_forward(x, w_router, bias, w_proj_down, w_gate, w_up, w_down, gain, eps, w_proj_up,
                        shared_gate, shared_up, shared_down, k, logits=logits, bf16_operands=bf16_operands)
    tot = res["up"]
    for y in res["shared"]:
        tot = tot + y
    ms = np.mean(tot * tot, axis=-1, keepdims=True)
    res["out"] = tot / np.sqrt(ms + eps)
    return res


MUTANTS = {
    "rmsnorm_no_sqrt": ("rmsnorm", _rms_no_sqrt),
    "rmsnorm_sum_not_mean": ("rmsnorm", _rms_sum),
    "rmsnorm_no_gain": ("rmsnorm", _rms_no_gain),
    "rmsnorm_eps_outside_root": ("rmsnorm", _rms_eps_outside),
    "bf16_truncates": ("bf16_round", _bf16_truncate),
    "rmsnorm_skipped": ("rmsnorm", lambda u, gain, eps: f64(u)),
    "norm_after_up_projection": ("latent_forward", _forward_norm_after_up),
    "shared_inside_norm": ("latent_forward", _forward_shared_inside_norm),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_latent_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(lat, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lat)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake {name}"


# ------------------------------------------------ the end-to-end rounding tolerance

@pytest.mark.parametrize("case", [dict(), dict(T=77, d=128, l=256, E=12, k=3, h=256, n_shared=1, h_shared=256),
                                  dict(T=1, E=5, k=2), dict(T=200, d=512, l=384, E=10, k=4, h=128),
                                  dict(T=64, d=1024, l=1024, E=16, k=8, h=256, n_shared=2, h_shared=512)])
def test_latent_error_model_covers_the_rounding_points(case):
    """The tolerance the GPU test applies to the LatentMoE output, checked on the CPU
    against the same three bf16 rounding points (z, H, r) applied inside the float64
    layer: the rounded layer stays within 8 sigma of the unrounded one everywhere, and
    the norm of the difference is what the first-order model predicts (within 30 %)."""
    from synthetic import make_latent_inputs, scaled_latent
    from tests import latent_bounds as lb
    cfg = scaled_latent("latent_tiny", name="bounds", **case)
    inp = make_latent_inputs(cfg)
    exact = lat.latent_forward(inp.x, *inp.args(), k=cfg.k, bf16_operands=False)
    rounded = lat.latent_forward(inp.x, *inp.args(), k=cfg.k, logits=exact["logits"], bf16_operands=True)
    sigma = lb.latent_output_sigma(inp.x, inp.w_proj_down, inp.w_gate, inp.w_up, inp.w_down, inp.rms_gain,
                                   inp.rms_eps, inp.w_proj_up, inp.shared_gate, inp.shared_up, inp.shared_down,
                                   exact)
    ratio, worst, _, _ = lb.check_latent_out(rounded["out"], exact["out"], sigma, factor=1.3)
    assert ratio >= 0.7, f"the rounding model overstates the error {1 / ratio:.2f} times"
    # a systematic mistake of a few bf16 ulps (a gain off by 3 %) fails the check
    with pytest.raises(AssertionError):
        lb.check_latent_out(exact["out"] + 0.03 * exact["up"], exact["out"], sigma)
    # so does dropping one token's routed branch
    broken = exact["out"].copy()
    broken[0] -= exact["up"][0]
    with pytest.raises(AssertionError):
        lb.check_latent_out(broken, exact["out"], sigma)


def test_ulp_bf16_values():
    """bf16 spacing: 2^-7 in [1, 2), 2^-6 in [2, 4), 2^-8 in [0.5, 1); zero at 0."""
    from tests import latent_bounds as lb
    got = lb.ulp_bf16(np.array([1.0, 1.99, 2.0, -3.5, 0.75, 0.0]))
    assert np.array_equal(got, [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -8, 0.0])
