"""MI355X (gfx950) routed Mixture-of-Experts FFN forward pass.

The layer -- linear gate, softmax and top-k routing, grouping by expert,
per-expert SwiGLU FFN, weighted combine -- and the router's load-balancing
statistics (auxiliary loss, Quantile Balancing) run in hand-written HIP kernels in
libmoe.so (C ABI: include/moe.h). This package is its thin Python binding.
Using any op fails loudly if libmoe.so has not been built; the build module
itself (`python -m sparse_mixture_experts_fp32_amd.build`) does not load it.
"""
_OPS = ("LatentMoEForward", "MXForward", "MoEForward", "moe_mx_expert_ffn", "moe_mx_quantize_rows",
        "moe_mx_quantize_weights", "moe_pack_weights", "moe_aux_loss", "moe_combine_rmsnorm", "moe_combine", "moe_expert_ffn", "moe_forward", "moe_permute", "moe_permute_noalloc",
        "moe_qb_histogram", "moe_qb_route", "moe_qb_update", "moe_route", "moe_topk_softmax")

__all__ = list(_OPS)


def __getattr__(name):
    if name in _OPS:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
