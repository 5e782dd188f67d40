"""CPU tests: the MX-format oracle against its pins, and planted mistakes that
the pins must catch."""
import numpy as np
import pytest

import oracle.mx as mx
from tests import pins_mx as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_mx_pin(pin):
    pin(mx)


# ---------------------------------------------------------------- planted mistakes

_real_round = mx.round_to_element
_real_exp = mx.block_exponent


def _round_half_up(v, fmt):
    """Ties away from zero instead of to the even code."""
    v = np.asarray(v, dtype=np.float64)
    codes = np.array(sorted(fmt["table"]))
    vals = np.array([fmt["table"][c] for c in codes])
    a = np.abs(v).reshape(-1)
    hi = np.clip(np.searchsorted(vals, a), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    idx = np.where(vals[hi] - a <= a - vals[lo], hi, lo)
    out = codes[np.where(a >= vals[-1], len(vals) - 1, idx)]
    sign_bit = 1 << (fmt["bits"] - 1)
    return np.where(np.signbit(v.reshape(-1)), out | sign_bit, out).reshape(v.shape)


def _round_drop_negative_zero(v, fmt):
    out = _real_round(v, fmt)
    sign_bit = 1 << (fmt["bits"] - 1)
    return np.where((out & (sign_bit - 1)) == 0, 0, out)


def _exp_ceil(amax, fmt):
    a = np.asarray(amax, dtype=np.float64)
    s = np.full(a.shape, -127, dtype=np.int64)
    nz = a > 0
    s[nz] = np.ceil(np.log2(a[nz])).astype(np.int64) - fmt["emax"]
    return np.clip(s, -127, 127)


def _exp_emax_off(amax, fmt):
    return np.clip(_real_exp(amax, fmt) - 1, -127, 127)


_real_value = mx.element_value


def _value_bias_off(codes, fmt):
    """Normal values twice too large (an exponent bias off by one)."""
    v = _real_value(codes, fmt)
    return v * np.where(np.abs(v) >= 1, 2.0, 1.0)


def _dequant_scale_off(codes, scale_bytes, fmt):
    c = np.asarray(codes)
    K = c.shape[-1]
    vals = _real_value(c, fmt).reshape(c.shape[:-1] + (K // 32, 32))
    s = np.asarray(scale_bytes, dtype=np.int64) - 128
    return (vals * np.exp2(s)[..., None]).reshape(c.shape)


MUTANTS = {
    "ties_away_from_zero": ("round_to_element", _round_half_up),
    "negative_zero_dropped": ("round_to_element", _round_drop_negative_zero),
    "shared_exponent_ceil": ("block_exponent", _exp_ceil),
    "shared_exponent_emax_off": ("block_exponent", _exp_emax_off),
    "element_values_wrong_above_one": ("element_value", _value_bias_off),
    "scale_bias_128": ("dequantize", _dequant_scale_off),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mx_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(mx, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mx)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
