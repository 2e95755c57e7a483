"""Pins of the projection oracle (oracle/proj_oracle.py): the MXFP4 element
and scale values of the OCP MX specification, decoding against an
independent per-element loop, the projection against explicit sums, the
[q | k | v] x heads x features split on a hand-placed case, and planted
mistakes that must fail at least one pin."""
import json
import math
import os

import numpy as np
import pytest

from oracle import proj_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_e2m1.json")


def _check_element_values():
    g = json.load(open(GOLDEN))
    for code, val in g["e2m1_code_value"]:
        got = float(orc.e2m1_value(code))
        if got != val or math.copysign(1.0, got) != math.copysign(1.0, val):
            return False
    for byte, val in g["e8m0_byte_value"]:
        if float(orc.e8m0_value(byte)) != val:
            return False
    return bool(np.isnan(orc.e8m0_value(255)))


def _check_decode_by_loop():
    """Element (n, k) = value(code[n, k]) * 2^(scale[n, k // 32] - 127),
    evaluated one element at a time from the golden table."""
    table = {c: v for c, v in json.load(open(GOLDEN))["e2m1_code_value"]}
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, (5, 64))
    scales = rng.integers(110, 140, (5, 2))
    w = orc.mxfp4_decode(codes, scales)
    for n in range(5):
        for k in range(64):
            if w[n, k] != math.ldexp(table[int(codes[n, k])], int(scales[n, k // 32]) - 127):
                return False
    return True


def _check_projection_by_sums():
    rng = np.random.default_rng(1)
    B, N, C, H, d = 2, 3, 64, 2, 4
    x = rng.standard_normal((B, N, C))
    codes = rng.integers(0, 16, (3 * H * d, C))
    scales = rng.integers(120, 132, (3 * H * d, C // 32))
    bias = rng.standard_normal(3 * H * d)
    q, k, v = orc.qkv_project(x, codes, scales, bias, H, d)
    table = {c: v for c, v in json.load(open(GOLDEN))["e2m1_code_value"]}
    outs = (q, k, v)
    for b in range(B):
        for t in range(N):
            for which in range(3):
                for h in range(H):
                    for f in range(d):
                        col = which * H * d + h * d + f
                        ref = bias[col] + sum(x[b, t, c] * math.ldexp(table[int(codes[col, c])],
                                                                     int(scales[col, c // 32]) - 127)
                                              for c in range(C))
                        if abs(outs[which][b, h, t, f] - ref) > 1e-12 * max(1.0, abs(ref)):
                            return False
    return True


def _check_split_by_hand():
    """One non-zero weight per output column: column n holds code 2 (value 1)
    at input channel n, scale 127 -- so output column n copies x[..., n].
    With C = 3 H d, q[b, h, t, f] = x[b, t, h d + f], k takes the next H d
    channels, v the last."""
    H, d = 2, 3
    C = 3 * H * d + 14  # pad C to a multiple of 32
    codes = np.zeros((3 * H * d, C), dtype=np.int64)
    for n in range(3 * H * d):
        codes[n, n] = 2
    scales = np.full((3 * H * d, C // 32), 127)
    x = np.arange(2 * 5 * C, dtype=np.float64).reshape(2, 5, C)
    q, k, v = orc.qkv_project(x, codes, scales, None, H, d)
    for which, out in enumerate((q, k, v)):
        for h in range(H):
            for f in range(d):
                if not np.array_equal(out[:, h, :, f], x[:, :, which * H * d + h * d + f]):
                    return False
    return True


PINS = [_check_element_values, _check_decode_by_loop, _check_projection_by_sums, _check_split_by_hand]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__[7:] for p in PINS])
def test_pin(pin):
    assert pin()


_e2m1_ok = orc.e2m1_value
_decode_ok = orc.mxfp4_decode
_project_ok = orc.qkv_project


def _no_sign(code):
    return np.abs(_e2m1_ok(code))


def _bias_zero_exponent(code):
    code = np.asarray(code, dtype=np.int64)
    e, m = (code >> 1) & 3, code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e))
    return np.where(code & 8, -1.0, 1.0) * mag


def _scale_along_outputs(codes, scales):
    codes = np.asarray(codes)
    w = _e2m1_ok(codes)
    sc = orc.e8m0_value(np.asarray(scales))
    return w * sc[np.arange(codes.shape[0]) // 32 % sc.shape[0], :1]


def _qk_swapped(x, codes, scales, bias, H, d):
    q, k, v = _project_ok(x, codes, scales, bias, H, d)
    return k, q, v


def _heads_features_swapped(x, codes, scales, bias, H, d):
    x = np.asarray(x, dtype=np.float64)
    B, N, C = x.shape
    y = x @ orc.mxfp4_decode(codes, scales).T
    if bias is not None:
        y = y + bias
    y = y.reshape(B, N, 3, d, H).transpose(2, 0, 4, 1, 3)
    return y[0], y[1], y[2]


MUTANTS = {
    "no_sign": ("e2m1_value", _no_sign),
    "exponent_bias_0": ("e2m1_value", _bias_zero_exponent),
    "scale_blocks_along_outputs": ("mxfp4_decode", _scale_along_outputs),
    "q_k_swapped": ("qkv_project", _qk_swapped),
    "heads_features_swapped": ("qkv_project", _heads_features_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert not all(p() for p in PINS), f"planted mistake {name!r} went unnoticed"
