"""Pins of the MX-format oracle against facts that do not come from it: the
E2M1 value list of the OCP MX specification, torch's float8_e4m3fn decoding and
rounding (an independent library implementation), hand-worked ties and
saturation, shared exponents worked by hand, exact round trips of representable
blocks, the per-element error bound, and the MX expert FFN against torch on
exactly representable operands.

Each pin takes the oracle module `mx` (or a copy with a planted mistake) and
raises AssertionError on failure.
"""
from __future__ import annotations

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


def pin_e2m1_values(mx):
    """The sixteen E2M1 codes: 0, 0.5, 1, 1.5, 2, 3, 4, 6, then the same negated."""
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    got = mx.element_value(np.arange(16), mx.E2M1)
    assert np.array_equal(got, np.array(want)), got
    assert np.signbit(got[8])


def pin_e4m3_values_vs_torch(mx):
    """Every non-NaN E4M3 code decodes as torch's float8_e4m3fn does (0x7F and 0xFF are NaN)."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mx.element_value(codes, mx.E4M3)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    assert got.max() == 448.0 and np.min(np.abs(got[got != 0])) == 2.0 ** -9


def pin_rounding_hand_cases(mx):
    """Ties go to the even code, values beyond the largest saturate, signs are kept."""
    e2 = [(0.24, 0.0), (0.25, 0.0), (0.26, 0.5), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0),
          (3.5, 4.0), (5.0, 4.0), (5.01, 6.0), (7.0, 6.0), (1e9, 6.0), (-2.5, -2.0), (-0.1, -0.0)]
    v = np.array([a for a, _ in e2])
    got = mx.element_value(mx.round_to_element(v, mx.E2M1), mx.E2M1)
    assert np.array_equal(got, np.array([b for _, b in e2])), got
    assert np.signbit(got[-1])
    e4 = [(2.0 ** -10, 0.0), (3 * 2.0 ** -10, 2.0 ** -8), (1.0625, 1.0), (1.1875, 1.25), (248.0, 256.0),
          (449.0, 448.0), (1e6, 448.0), (-464.0, -448.0)]
    v = np.array([a for a, _ in e4])
    got = mx.element_value(mx.round_to_element(v, mx.E4M3), mx.E4M3)
    assert np.array_equal(got, np.array([b for _, b in e4])), got


def pin_rounding_vs_torch(mx):
    """Round to nearest even on E4M3 agrees with torch's float32 -> float8_e4m3fn cast
    for values in range, subnormals included."""
    r = _rng(1)
    v = np.concatenate([r.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 150)]).astype(np.float32)
    v = v[np.abs(v) < 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    got = mx.round_to_element(v, mx.E4M3)
    assert np.array_equal(got, ref), (v[got != ref][:5], got[got != ref][:5], ref[got != ref][:5])


def pin_block_exponent(mx):
    """s = floor(log2 amax) - emax: amax 6 -> 0 and 1 -> -2 for E2M1 (1.0 is then the element 4);
    amax 448 -> 0 and 1 -> -8 for E4M3; 0 -> -127; clamped to [-127, 127]."""
    got = mx.block_exponent(np.array([6.0, 7.99, 8.0, 1.0, 0.0, 2.0 ** -200, 2.0 ** 200]), mx.E2M1)
    assert list(got) == [0, 0, 1, -2, -127, -127, 127], got
    got = mx.block_exponent(np.array([448.0, 1.0, 2.0 ** -9]), mx.E4M3)
    assert list(got) == [0, -8, -17], got


def pin_quantize_round_trip(mx):
    """A block made of table values times 2^s, with its largest magnitude in [4, 8) * 2^s
    (E2M1) or [256, 512) * 2^s (E4M3), comes back exactly; the scale byte is s + 127."""
    r = _rng(2)
    for fmt, top in ((mx.E2M1, 6.0), (mx.E4M3, 448.0)):
        table = np.array(sorted(fmt["table"].values()))
        for s in (-5, 0, 3):
            blk = r.choice(table, size=(3, 64)) * r.choice([-1.0, 1.0], size=(3, 64))
            blk[:, 0] = top
            blk[:, 40] = -top
            v = blk * 2.0 ** s
            codes, sc = mx.quantize(v, fmt)
            assert np.all(sc == s + 127), sc
            assert np.array_equal(mx.dequantize(codes, sc, fmt), v)


def pin_quantize_error_bound(mx):
    """Random rows: every element lies within half a spacing of its value, or is clamped
    from below 2^(emax+1) * 2^s: |v - q| <= 2^(s+1) for E2M1 (spacing 2 at the top, clamping
    from < 8 to 6) and 2^(s+6) for E4M3 (spacing 32 at the top, clamping from < 512 to 448);
    an all-zero block quantises to zeros with scale byte 0."""
    r = _rng(3)
    v = r.standard_normal((40, 128)) * np.exp(r.uniform(-8, 8, size=(40, 1)))
    v[5, 32:64] = 0.0
    for fmt, slack in ((mx.E2M1, 1), (mx.E4M3, 6)):
        codes, sc = mx.quantize(v, fmt)
        q = mx.dequantize(codes, sc, fmt)
        s = np.repeat(sc - 127, 32, axis=-1)
        assert np.all(np.abs(q - v) <= 2.0 ** (s + slack)), np.max(np.abs(q - v) / 2.0 ** (s + slack))
        assert sc[5, 1] == 0 and np.all(q[5, 32:64] == 0)


def pin_mx_ffn_exact_operands(mx):
    """With operands the MX formats hold exactly, the MX expert FFN is the float64 SwiGLU
    FFN of those values (torch)."""
    r = _rng(4)
    M, d, h = 7, 64, 32
    t2, t4 = np.array(sorted(mx.E2M1["table"].values())), np.array(sorted(mx.E4M3["table"].values()))

    def exact(table, top, shape, s):
        v = r.choice(table, size=shape) * r.choice([-1.0, 1.0], size=shape)
        v[..., ::32] = top
        return v * 2.0 ** s

    x = exact(t4, 448.0, (M, d), -9)
    wg, wu, wd = exact(t2, 6.0, (h, d), -4), exact(t2, 6.0, (h, d), -5), exact(t2, 6.0, (d, h), -3)
    xq, xs = mx.quantize(x, mx.E4M3)
    gq, gs = mx.quantize(wg, mx.E2M1)
    uq, us = mx.quantize(wu, mx.E2M1)
    H = mx.mx_expert_gate_up(xq, xs, gq, gs, uq, us)
    X, G, U = (torch.from_numpy(a) for a in (x, wg, wu))
    Ht = (torch.nn.functional.silu(X @ G.T) * (X @ U.T)).numpy()
    assert np.allclose(H, Ht, rtol=1e-13, atol=1e-300), np.max(np.abs(H - Ht))
    hq, hs = mx.quantize(H, mx.E4M3)
    dq, ds = mx.quantize(wd, mx.E2M1)
    Y = mx.mx_expert_down(hq, hs, dq, ds)
    Yt = mx.dequantize(hq, hs, mx.E4M3) @ wd.T
    assert np.allclose(Y, Yt, rtol=1e-13, atol=1e-300)


ALL_PINS = [
    pin_e2m1_values,
    pin_e4m3_values_vs_torch,
    pin_rounding_hand_cases,
    pin_rounding_vs_torch,
    pin_block_exponent,
    pin_quantize_round_trip,
    pin_quantize_error_bound,
    pin_mx_ffn_exact_operands,
]
