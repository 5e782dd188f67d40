"""Seeded synthetic workloads for the Stable LatentMoE layer (forward pass).

Sizes from "Kimi K3: Open Frontier Intelligence" (section "Operational
Execution Flow"): hidden width d = 7168, latent width l = 3584, 896 routed
experts with 16 active, two shared experts. The routed experts' hidden width
(1024, as the many-expert workload) and the shared experts' hidden width
(2048) are not on the page and are synthetic choices. Every value is synthetic.

Recipe (the same scheme as the routed-layer inputs): one torch.Generator per
(seed, tag, index), seeded with seed * 2**20 + tag * 2**12 + index; float32
standard normals times the stated standard deviation, rounded to bfloat16
for activations and matrix weights:
  x ~ N(0, 1) [T, d] bf16;  w_router ~ N(0, 1/d) [E, d] f32 (no bias);
  w_proj_down ~ N(0, 1/d) [l, d] bf16;  w_proj_up ~ N(0, 1/l) [d, l] bf16;
  routed w_gate, w_up ~ N(0, 1/l) [E, h, l], w_down ~ N(0, 1/h) [E, l, h] bf16;
  rms_gain = 1 + 0.1 N(0, 1) [l] f32 (a trained gain near its initial 1);
  rms_eps = 1e-6;
  shared gate, up ~ N(0, 1/d) [S, hs, d], down ~ N(0, 1/hs) [S, d, hs] bf16.

This module holds no arithmetic of the layer itself; it only draws inputs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

from .moe_inputs import TAG_DOWN, TAG_GATE, TAG_ROUTER, TAG_UP, TAG_X, _gen, _normal

TAG_PROJ_DOWN, TAG_PROJ_UP, TAG_GAIN, TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN = range(6, 12)


@dataclasses.dataclass(frozen=True)
class LatentConfig:
    name: str
    T: int         # tokens
    d: int         # model width
    l: int         # latent width of the routed path
    E: int         # routed experts
    k: int         # experts per token
    h: int         # routed expert hidden width
    n_shared: int  # shared experts
    h_shared: int  # shared expert hidden width
    seed: int
    rms_eps: float = 1e-6

    def weight_bytes(self) -> int:
        return 2 * (3 * self.E * self.l * self.h + 2 * self.l * self.d + 3 * self.n_shared * self.h_shared * self.d)


LATENT_CONFIGS = {
    "latent_tiny": LatentConfig("latent_tiny", T=64, d=256, l=128, E=8, k=2, h=128, n_shared=2, h_shared=128,
                                seed=10),
    # the page's layer: d = 7168, l = 3584, 896 experts, 16 active, 2 shared
    "latent": LatentConfig("latent", T=16384, d=7168, l=3584, E=896, k=16, h=1024, n_shared=2, h_shared=2048,
                           seed=11),
}


def scaled_latent(base: str, **overrides) -> LatentConfig:
    fields = dataclasses.asdict(LATENT_CONFIGS[base])
    fields.update(overrides)
    if "name" not in overrides:
        fields["name"] = base + "_scaled"
    return LatentConfig(**fields)


@dataclasses.dataclass
class LatentInputs:
    cfg: LatentConfig
    x: torch.Tensor
    w_router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    w_proj_down: torch.Tensor
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    rms_gain: torch.Tensor
    rms_eps: float
    w_proj_up: torch.Tensor
    shared_gate: Optional[torch.Tensor]
    shared_up: Optional[torch.Tensor]
    shared_down: Optional[torch.Tensor]

    def args(self):
        """The layer's arguments in call order (after x)."""
        return (self.w_router, self.router_bias, self.w_proj_down, self.w_gate, self.w_up, self.w_down,
                self.rms_gain, self.rms_eps, self.w_proj_up, self.shared_gate, self.shared_up, self.shared_down)


def make_latent_inputs(cfg: LatentConfig, device: str = "cpu", gen_device: Optional[str] = None,
                       progress=None) -> LatentInputs:
    """Draw every input of one LatentMoE layer call (small ones on the CPU, large on the device)."""
    if gen_device is None:
        gen_device = "cpu" if cfg.weight_bytes() <= (256 << 20) else str(device)
    if str(gen_device).startswith("cuda"):
        gen_device = "cuda"
    T, d, l, E, h, S, hs, sd = cfg.T, cfg.d, cfg.l, cfg.E, cfg.h, cfg.n_shared, cfg.h_shared, cfg.seed
    bf = lambda t: t.to(torch.bfloat16).to(device)  # noqa: E731
    x = bf(_normal((T, d), 1.0, _gen(gen_device, sd, TAG_X), gen_device))
    w_router = _normal((E, d), 1.0 / math.sqrt(d), _gen(gen_device, sd, TAG_ROUTER), gen_device).to(device)
    w_proj_down = bf(_normal((l, d), 1.0 / math.sqrt(d), _gen(gen_device, sd, TAG_PROJ_DOWN), gen_device))
    w_proj_up = bf(_normal((d, l), 1.0 / math.sqrt(l), _gen(gen_device, sd, TAG_PROJ_UP), gen_device))
    gain = (1.0 + 0.1 * _normal((l,), 1.0, _gen(gen_device, sd, TAG_GAIN), gen_device)).to(device)
    w_gate = torch.empty((E, h, l), dtype=torch.bfloat16, device=device)
    w_up = torch.empty((E, h, l), dtype=torch.bfloat16, device=device)
    w_down = torch.empty((E, l, h), dtype=torch.bfloat16, device=device)
    for e in range(E):
        w_gate[e].copy_(_normal((h, l), 1.0 / math.sqrt(l), _gen(gen_device, sd, TAG_GATE, e), gen_device).to(torch.bfloat16))
        w_up[e].copy_(_normal((h, l), 1.0 / math.sqrt(l), _gen(gen_device, sd, TAG_UP, e), gen_device).to(torch.bfloat16))
        w_down[e].copy_(_normal((l, h), 1.0 / math.sqrt(h), _gen(gen_device, sd, TAG_DOWN, e), gen_device).to(torch.bfloat16))
        if progress is not None and (e + 1) % 64 == 0:
            progress(e + 1)
    if S > 0:
        sg = torch.stack([_normal((hs, d), 1.0 / math.sqrt(d), _gen(gen_device, sd, TAG_SH_GATE, s), gen_device)
                          for s in range(S)])
        su = torch.stack([_normal((hs, d), 1.0 / math.sqrt(d), _gen(gen_device, sd, TAG_SH_UP, s), gen_device)
                          for s in range(S)])
        sdn = torch.stack([_normal((d, hs), 1.0 / math.sqrt(hs), _gen(gen_device, sd, TAG_SH_DOWN, s), gen_device)
                           for s in range(S)])
        sg, su, sdn = bf(sg), bf(su), bf(sdn)
    else:
        sg = su = sdn = None
    return LatentInputs(cfg, x, w_router, None, w_proj_down, w_gate, w_up, w_down, gain, cfg.rms_eps, w_proj_up,
                        sg, su, sdn)
