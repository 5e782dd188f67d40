"""Seeded synthetic workloads for one routed-MoE FFN layer (forward pass).

The workload shapes follow the sizes the Kimi K3 pages quote for the sparse
layer: hidden width d = 7168 (arxiviq summary, "Mathematical Foundational
Substrates"); 384 experts with 8 selected (fde-coach, "The Architecture");
256 experts with top-4 (namoclaw, "Model Card at a Glance"); 896 routed
experts with 16 active (arxiviq summary, "Operational Execution Flow").
The pages publish no tensors, so every value here is synthetic.

Recipe (one choice for the whole repository):
  * one torch.Generator per (config seed, tensor tag, expert id), seeded with
    seed * 2**20 + tag * 2**12 + e; tags x=0, router=1, rank=2, gate=3,
    up=4, down=5;
  * values are float32 standard normals times the stated standard deviation,
    rounded to bfloat16 (round-to-nearest-even) for x and the expert weights;
    the router weight stays float32;
  * x ~ N(0, 1); router W_r ~ N(0, 1/d); W_gate, W_up ~ N(0, 1/d);
    W_down ~ N(0, 1/h);
  * the skewed workload adds a router bias b_e = 1.5 * ln(1 / rank_e) where
    rank is a seeded permutation of 1..E, so the favoured experts are not
    simply the lowest ids.

Storage layout (row-major, the "output-major, input-contiguous" convention of
a linear layer's weight):
  x          [T, d]     bfloat16
  w_router   [E, d]     float32   (logits = x @ w_router.T (+ bias))
  router_bias[E]        float32 or None
  w_gate     [E, h, d]  bfloat16  (gate = x_e @ w_gate[e].T)
  w_up       [E, h, d]  bfloat16  (up   = x_e @ w_up[e].T)
  w_down     [E, d, h]  bfloat16  (y    = h_e @ w_down[e].T)

This module holds no arithmetic of the layer itself; it only draws inputs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

TAG_X, TAG_ROUTER, TAG_RANK, TAG_GATE, TAG_UP, TAG_DOWN = range(6)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int  # tokens
    d: int  # hidden width
    E: int  # routed experts
    k: int  # experts selected per token
    h: int  # SwiGLU hidden width of one expert
    seed: int
    skewed: bool = False  # adds the Zipf-like router bias

    @property
    def assignments(self) -> int:
        return self.T * self.k

    def expert_weight_bytes(self) -> int:
        return 3 * self.E * self.d * self.h * 2


CONFIGS = {
    # tiny layer that the oracle finishes instantly
    "tiny": MoEConfig("tiny", T=64, d=128, E=8, k=2, h=256, seed=0),
    # decode-like small batch: weight-streaming bound, most experts see 0-3 rows
    "decode": MoEConfig("decode", T=128, d=7168, E=384, k=8, h=2048, seed=1),
    # prefill batch, near-uniform expert load (the headline workload)
    "prefill": MoEConfig("prefill", T=8192, d=7168, E=256, k=4, h=2048, seed=2),
    # fine-grained many-expert layer
    "many_expert": MoEConfig("many_expert", T=16384, d=7168, E=896, k=16, h=1024, seed=3),
    # as many_expert, with a Zipf-like router bias that skews the load
    "skewed": MoEConfig("skewed", T=16384, d=7168, E=896, k=16, h=1024, seed=4, skewed=True),
}


def scaled_config(base: str, **overrides) -> MoEConfig:
    """A copy of a named workload with some sizes replaced (for small tests)."""
    cfg = CONFIGS[base]
    fields = dataclasses.asdict(cfg)
    fields.update(overrides)
    if "name" not in overrides:
        fields["name"] = base + "_scaled"
    return MoEConfig(**fields)


@dataclasses.dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor
    w_router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor

    def to(self, device) -> "MoEInputs":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return MoEInputs(self.cfg, mv(self.x), mv(self.w_router), mv(self.router_bias),
                         mv(self.w_gate), mv(self.w_up), mv(self.w_down))


def _gen(device: str, seed: int, tag: int, e: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 2**20 + tag * 2**12 + e)
    return g


def _normal(shape, std: float, g: torch.Generator, device: str) -> torch.Tensor:
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std


def router_bias_for(cfg: MoEConfig, device: str = "cpu") -> Optional[torch.Tensor]:
    """Zipf-like bias b_e = 1.5 * ln(1 / rank_e), ranks a seeded permutation of 1..E."""
    if not cfg.skewed:
        return None
    g = _gen("cpu", cfg.seed, TAG_RANK)
    rank = torch.randperm(cfg.E, generator=g).to(torch.float64) + 1.0
    return (-1.5 * torch.log(rank)).to(torch.float32).to(device)


def make_inputs(cfg: MoEConfig, device: str = "cpu", gen_device: Optional[str] = None,
                experts: bool = True, progress=None) -> MoEInputs:
    """Draw every input of one layer invocation.

    gen_device is where the random numbers are drawn ("cpu" or "cuda"); the
    two devices' generators give different (equally valid) streams, so a test
    must draw a workload once and hand the same tensors to both sides. By
    default small workloads are drawn on the CPU (reproducible everywhere)
    and large ones on the target device (drawing tens of GB of normals on the
    host would take minutes). `progress`, if given, is called with the number
    of experts drawn so far, every 64 experts.
    """
    if gen_device is None:
        gen_device = "cpu" if cfg.expert_weight_bytes() <= (256 << 20) else str(device)
    if str(gen_device).startswith("cuda"):
        gen_device = "cuda"
    T, d, E, h = cfg.T, cfg.d, cfg.E, cfg.h
    x = _normal((T, d), 1.0, _gen(gen_device, cfg.seed, TAG_X), gen_device)
    x = x.to(torch.bfloat16).to(device)
    w_router = _normal((E, d), 1.0 / math.sqrt(d), _gen(gen_device, cfg.seed, TAG_ROUTER), gen_device)
    w_router = w_router.to(device)
    bias = router_bias_for(cfg, device)
    if experts:
        w_gate = torch.empty((E, h, d), dtype=torch.bfloat16, device=device)
        w_up = torch.empty((E, h, d), dtype=torch.bfloat16, device=device)
        w_down = torch.empty((E, d, h), dtype=torch.bfloat16, device=device)
        for e in range(E):
            w_gate[e].copy_(_normal((h, d), 1.0 / math.sqrt(d), _gen(gen_device, cfg.seed, TAG_GATE, e), gen_device).to(torch.bfloat16))
            w_up[e].copy_(_normal((h, d), 1.0 / math.sqrt(d), _gen(gen_device, cfg.seed, TAG_UP, e), gen_device).to(torch.bfloat16))
            w_down[e].copy_(_normal((d, h), 1.0 / math.sqrt(h), _gen(gen_device, cfg.seed, TAG_DOWN, e), gen_device).to(torch.bfloat16))
            if progress is not None and (e + 1) % 64 == 0:
                progress(e + 1)
    else:
        w_gate = w_up = w_down = None
    return MoEInputs(cfg, x, w_router, bias, w_gate, w_up, w_down)
