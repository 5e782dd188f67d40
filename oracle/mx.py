"""Plain CPU oracle of the MX-format expert FFN (MXFP4 weights, MXFP8 activations).

TEST INFRASTRUCTURE. Only tests/, the smoke check and the benchmark's CPU
baseline may import or call this module; the HIP library never does, and the
two share no code (kernels, headers, helpers, tables or constants).

Source: "Kimi K3: Open Frontier Intelligence", section "Systems Optimization,
Load Balancing, and Post-Training Alignment": for serving, the MoE weights are
MXFP4 (quantisation-aware post-training) and the activations MXFP8. The pages
do not define the formats; they are the OCP Microscaling (MX) formats, v1.0:
  * a block of 32 consecutive elements shares one scale X = 2^s, stored as an
    E8M0 byte s + 127 (s in [-127, 127]);
  * FP4 E2M1 elements: sign, 2 exponent bits (bias 1), 1 mantissa bit; values
    0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives;
  * FP8 E4M3 elements: sign, 4 exponent bits (bias 7), 3 mantissa bits,
    subnormals below 2^-6 in steps of 2^-9, largest finite 448, no infinity
    (S.1111.111 is NaN);
  * conversion of a block V: s = floor(log2(max_i |V_i|)) - emax, emax the
    exponent of the element format's largest normal (2 for E2M1, 8 for E4M3);
    each V_i / 2^s is rounded to the nearest element value, ties to the even
    code, and values beyond the largest one are clamped to it.

Readings (also listed in the design notes):
  * blocks run along the contraction dimension K (a weight row [n, :] and an
    activation row [r, :] split into K/32 blocks);
  * an all-zero block gets s = -127 (scale byte 0) and zero elements; s is
    clamped to [-127, 127];
  * the sign of a value that rounds to zero is kept (negative zero code);
  * the expert FFN runs on the dequantised values: x rows and H rows are
    quantised to MXFP8, weights to MXFP4; the products of dequantised values
    are exact and summed in float64; SwiGLU in float64. H is quantised from
    the values given (the device passes its own float32 H, so that both sides
    decide the codes on the same numbers).
"""
from __future__ import annotations

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

from . import moe_oracle as _m

BLOCK = 32


def _code_table(exp_bits: int, man_bits: int, bias: int, nan_codes=()):
    """All non-negative finite values of a sign/exponent/mantissa format, by code."""
    vals = {}
    for code in range(1 << (exp_bits + man_bits)):
        if code in nan_codes:
            continue
        e, m = code >> man_bits, code & ((1 << man_bits) - 1)
        if e == 0:
            v = m / (1 << man_bits) * 2.0 ** (1 - bias)
        else:
            v = (1 + m / (1 << man_bits)) * 2.0 ** (e - bias)
        vals[code] = v
    return vals


E2M1 = dict(bits=4, table=_code_table(2, 1, 1), emax=2)
E4M3 = dict(bits=8, table=_code_table(4, 3, 7, nan_codes=(0x7F,)), emax=8)


def element_value(codes, fmt) -> np.ndarray:
    """Value of each element code (sign bit on top), looked up in the format's table."""
    c = np.asarray(codes, dtype=np.int64)
    sign_bit = 1 << (fmt["bits"] - 1)
    lut = np.full(sign_bit, np.nan)
    for code, v in fmt["table"].items():
        lut[code] = v
    mag = lut[c & (sign_bit - 1)]
    return np.where(c & sign_bit, -mag, mag)


def round_to_element(v, fmt) -> np.ndarray:
    """Nearest element code of each value (ties to the code with an even mantissa,
    i.e. an even magnitude code; beyond the largest value: the largest). The sign
    is kept, also for values that round to zero. A table search: the two table
    values around |v| are compared."""
    v = np.asarray(v, dtype=np.float64)
    codes = np.array(sorted(fmt["table"]), dtype=np.int64)
    vals = np.array([fmt["table"][c] for c in codes])  # increasing with the code
    a = np.abs(v).reshape(-1)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)  # first value >= |v|
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    idx = np.where(a <= vals[0], 0, np.where(pick_hi, hi, lo))
    idx = np.where(a >= vals[-1], len(vals) - 1, idx)
    out = codes[idx]
    sign_bit = 1 << (fmt["bits"] - 1)
    out = np.where(np.signbit(v.reshape(-1)), out | sign_bit, out)
    return out.reshape(v.shape)


def block_exponent(block_amax, fmt) -> np.ndarray:
    """Shared exponent s = floor(log2(amax)) - emax, clamped to [-127, 127]; -127 for amax = 0."""
    a = np.asarray(block_amax, dtype=np.float64)
    s = np.full(a.shape, -127, dtype=np.int64)
    nz = a > 0
    s[nz] = np.floor(np.log2(a[nz])).astype(np.int64) - fmt["emax"]
    return np.clip(s, -127, 127)


def quantize(v, fmt):
    """MX conversion of rows along the last axis (a multiple of 32).

    Returns (codes [..., K] int64, scale_bytes [..., K/32] int64 = s + 127)."""
    V = np.asarray(_m.f64(v), dtype=np.float64)
    K = V.shape[-1]
    assert K % BLOCK == 0
    blocks = V.reshape(V.shape[:-1] + (K // BLOCK, BLOCK))
    s = block_exponent(np.abs(blocks).max(axis=-1), fmt)
    codes = round_to_element(blocks / np.exp2(s)[..., None], fmt)
    return codes.reshape(V.shape), s + 127


def dequantize(codes, scale_bytes, fmt) -> np.ndarray:
    """codes [..., K], scale bytes [..., K/32] -> float64 values."""
    c = np.asarray(codes)
    K = c.shape[-1]
    vals = element_value(c, fmt).reshape(c.shape[:-1] + (K // BLOCK, BLOCK))
    s = np.asarray(scale_bytes, dtype=np.int64) - 127
    return (vals * np.exp2(s)[..., None]).reshape(c.shape)


def mx_expert_gate_up(x_rows_q, x_scales, wg_q, wg_s, wu_q, wu_s):
    """H = silu(x Wg^T) * (x Wu^T) on dequantised MXFP8 rows and MXFP4 weights (float64)."""
    X = dequantize(x_rows_q, x_scales, E4M3)
    G = X @ dequantize(wg_q, wg_s, E2M1).T
    U = X @ dequantize(wu_q, wu_s, E2M1).T
    return _m.silu(G) * U


def mx_expert_down(h_rows_q, h_scales, wd_q, wd_s):
    """Y = H Wd^T on dequantised MXFP8 H rows and MXFP4 weights (float64)."""
    return dequantize(h_rows_q, h_scales, E4M3) @ dequantize(wd_q, wd_s, E2M1).T
