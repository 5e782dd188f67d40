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
                           shared_gate, shared_up, shared_down, k, logits=None, bf16_operands=True):
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
                                shared_gate, shared_up, shared_down, k, logits=None, bf16_operands=True):
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
