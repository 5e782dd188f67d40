"""ctypes binding of libmoe.so: the C ABI declared in include/moe.h, same names.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. If libmoe.so is missing or does not load, importing this module
raises; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY may name another build of the same library (the sanitizer build, libmoe_san.so)
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

MOE_CALL_PERMUTE = 0
MOE_CALL_EXPERT_FFN = 1
MOE_CALL_FORWARD = 2
MOE_CALL_ROUTE = 3
MOE_CALL_AUX_LOSS = 4
MOE_CALL_MX_FORWARD = 5

MX_SLOTS = ["logits", "topk_idx", "topk_w", "expert_offsets", "row_of", "row_src", "x_q", "x_s", "h_act", "h_q",
            "h_s", "y_rows"]
LAT_SLOTS = ["logits", "topk_idx", "topk_w", "expert_offsets", "row_of", "row_src", "z", "h_act", "y_rows", "r",
             "shared_h", "shared_y"]
FWD_SLOTS = ["logits", "topk_idx", "topk_w", "expert_offsets", "row_of", "row_src", "h_act", "y_rows"]
ABI_VERSION = 10


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("h", ctypes.c_int32)]


class MoeLatentShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("l", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("h", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("h_shared", ctypes.c_int32)]


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_mixture_experts_fp32_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    S = ctypes.POINTER(MoeShape)
    LS = ctypes.POINTER(MoeLatentShape)
    sig = {
        "moe_abi_version": (ctypes.c_int, []),
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_workspace_bytes": (ctypes.c_size_t, [S, ctypes.c_int]),
        "moe_forward_ws_offset": (ctypes.c_int, [S, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_route": (ctypes.c_int, [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_topk_softmax": (ctypes.c_int, [S, P, P, P, P]),
        "moe_permute": (ctypes.c_int, [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_permute_noalloc": (ctypes.c_int, [S, P, P, P, P, P, P, P]),
        "moe_expert_ffn": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_expert_gate_up": (ctypes.c_int, [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_expert_down": (ctypes.c_int, [S, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_combine": (ctypes.c_int, [S, P, P, P, P, P]),
        "moe_forward": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_aux_loss": (ctypes.c_int, [S, P, P, P, P, ctypes.c_size_t, P]),
        "moe_pack_weights": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P]),
        "moe_qb_route": (ctypes.c_int, [S, P, P, P, P, P, P]),
        "moe_qb_histogram": (ctypes.c_int, [S, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_int32, P, P]),
        "moe_qb_update": (ctypes.c_int, [S, P, ctypes.c_float, ctypes.c_float, ctypes.c_int32, P, P, P]),
        "moe_latent_workspace_bytes": (ctypes.c_size_t, [LS]),
        "moe_latent_ws_offset": (ctypes.c_int, [LS, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_latent_forward": (ctypes.c_int, [LS, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P,
                                              ctypes.c_size_t, P]),
        "moe_combine_rmsnorm": (ctypes.c_int, [S, P, P, P, P, ctypes.c_float, P, P, P]),
        "moe_mx_quantize_weights": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, P]),
        "moe_mx_quantize_rows": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, P, ctypes.c_int32, P, P, P]),
        "moe_mx_expert_ffn": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_mx_expert_gate_up": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_mx_expert_down": (ctypes.c_int, [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "moe_mx_forward_ws_offset": (ctypes.c_int, [S, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
        "moe_mx_forward": (ctypes.c_int, [S, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.moe_abi_version()}, this binding needs {ABI_VERSION}")
    return lib


lib = _load()


def check(status: int) -> None:
    if status != MOE_OK:
        msg = lib.moe_last_error().decode() or lib.moe_status_str(status).decode()
        raise MoEError(status, msg)


def shape(T: int, d: int, E: int, k: int, h: int) -> MoeShape:
    return MoeShape(T, d, E, k, h)


def workspace_bytes(s: MoeShape, call: int) -> int:
    n = lib.moe_workspace_bytes(ctypes.byref(s), call)
    err = lib.moe_last_error().decode()
    if n == 0 and err:
        raise MoEError(MOE_ERR_INVALID_ARG, err)
    return n


def forward_ws_offset(s: MoeShape, slot: int) -> int:
    off = ctypes.c_size_t(0)
    check(lib.moe_forward_ws_offset(ctypes.byref(s), slot, ctypes.byref(off)))
    return off.value


def latent_shape(T: int, d: int, l: int, E: int, k: int, h: int, n_shared: int, h_shared: int) -> MoeLatentShape:
    return MoeLatentShape(T, d, l, E, k, h, n_shared, h_shared)


def latent_workspace_bytes(s: MoeLatentShape) -> int:
    n = lib.moe_latent_workspace_bytes(ctypes.byref(s))
    err = lib.moe_last_error().decode()
    if n == 0 and err:
        raise MoEError(MOE_ERR_INVALID_ARG, err)
    return n


def latent_ws_offset(s: MoeLatentShape, slot: int) -> int:
    off = ctypes.c_size_t(0)
    check(lib.moe_latent_ws_offset(ctypes.byref(s), slot, ctypes.byref(off)))
    return off.value


def mx_forward_ws_offset(s: MoeShape, slot: int) -> int:
    off = ctypes.c_size_t(0)
    check(lib.moe_mx_forward_ws_offset(ctypes.byref(s), slot, ctypes.byref(off)))
    return off.value
