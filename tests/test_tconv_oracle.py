"""Pins of the temporal-convolution oracle (oracle/tconv_oracle.py) against
things other than itself: a hand-worked example, numpy's convolution for the
two cases that reduce to a textbook convolution, the brute-force visibility
stencil, streaming against one-shot, block causality, and planted mistakes
that must fail at least one pin."""
import json
import os

import numpy as np
import pytest

from brute_tconv import brute_tconv
from oracle import tconv_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tconv_hand.json")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _check_golden():
    g = json.load(open(GOLDEN))
    x = np.asarray(g["x_t_c"], np.float64)[None, :, None, None, :]
    w = np.asarray(g["w_c_tap"], np.float64)
    b = np.asarray(g["bias_c"], np.float64)
    for case in g["cases"]:
        cache = None if case["cache_c"] is None else np.asarray(case["cache_c"], np.float64)[None, None, None, :]
        y, last = orc.tconv_fwd(x, w, b, case["F"], cache=cache)
        if not np.array_equal(y[0, :, 0, 0], np.asarray(case["y_t_c"], np.float64)):
            return False
        if not np.array_equal(last[0, 0, 0], np.asarray(case["cache_out_c"], np.float64)):
            return False
    return True


def _check_single_block_is_same_conv():
    """One block, no cache: zero on both sides, i.e. numpy's 'same'
    convolution with the taps reversed (convolution flips the kernel)."""
    x = _rand((1, 7, 2, 3, 4), 1)
    w = _rand((4, 3), 2)
    b = _rand((4,), 3)
    y, _ = orc.tconv_fwd(x, w, b, 7)
    for hh in range(2):
        for ww in range(3):
            for c in range(4):
                ref = np.convolve(x[0, :, hh, ww, c], w[c, ::-1], mode="same") + b[c]
                if not np.allclose(y[0, :, hh, ww, c], ref, rtol=1e-13, atol=1e-13):
                    return False
    return True


def _check_one_frame_blocks_are_causal_two_tap():
    """F = 1: the next frame is always a separator, so the op is the
    strictly causal convolution with taps (w0, w1): numpy's 'full'
    convolution truncated to T."""
    x = _rand((2, 6, 1, 2, 3), 4)
    w = _rand((3, 3), 5)
    y, _ = orc.tconv_fwd(x, w, None, 1)
    for bb in range(2):
        for ww in range(2):
            for c in range(3):
                ref = np.convolve(x[bb, :, 0, ww, c], [w[c, 1], w[c, 0]], mode="full")[:6]
                if not np.allclose(y[bb, :, 0, ww, c], ref, rtol=1e-13, atol=1e-13):
                    return False
    return True


BRUTE_CASES = [((1, 6, 2, 3, 4), 2, False), ((2, 9, 1, 2, 3), 3, True), ((1, 4, 3, 1, 2), 1, True),
               ((1, 5, 2, 2, 5), 5, True)]


def _check_brute_force():
    for i, (shape, F, with_cache) in enumerate(BRUTE_CASES):
        x = _rand(shape, 10 + i)
        w = _rand((shape[-1], 3), 20 + i)
        b = _rand((shape[-1],), 30 + i)
        cache = _rand((shape[0],) + shape[2:], 40 + i) if with_cache else None
        y, last = orc.tconv_fwd(x, w, b, F, cache=cache)
        if not np.allclose(y, brute_tconv(x, w, b, F, cache=cache), rtol=1e-13, atol=1e-13):
            return False
        if not np.array_equal(last, x[:, -1]):
            return False
    return True


def _check_streaming():
    """apply block c against the cache committed from blocks < c equals the
    one-shot output of block c; apply leaves the cache untouched."""
    F, nb = 3, 4
    x = _rand((1, F * nb, 2, 2, 3), 50)
    w = _rand((3, 3), 51)
    b = _rand((3,), 52)
    cache0 = _rand((1, 2, 2, 3), 53)
    y_full, last = orc.tconv_fwd(x, w, b, F, cache=cache0)
    cache = cache0.copy()
    for c in range(nb):
        blk = x[:, c * F:(c + 1) * F]
        before = cache.copy()
        yc = orc.tconv_apply(cache, blk, w, b)
        if not np.array_equal(cache, before):
            return False
        if not np.allclose(yc, y_full[:, c * F:(c + 1) * F], rtol=1e-14, atol=1e-14):
            return False
        cache = orc.tconv_commit(cache, blk)
    return np.array_equal(cache, last)


def _check_causality():
    """Changing any frame of block c' > c leaves blocks <= c bit-identical;
    changing the last frame of block c changes the first output of c + 1."""
    F, nb = 2, 4
    x = _rand((1, F * nb, 1, 2, 3), 60)
    w = _rand((3, 3), 61)
    b = _rand((3,), 62)
    y, _ = orc.tconv_fwd(x, w, b, F)
    for c in range(nb - 1):
        x2 = x.copy()
        x2[:, (c + 1) * F:] += 1.0
        y2, _ = orc.tconv_fwd(x2, w, b, F)
        if not np.array_equal(y2[:, :(c + 1) * F], y[:, :(c + 1) * F]):
            return False
        x3 = x.copy()
        x3[:, (c + 1) * F - 1] += 1.0
        y3, _ = orc.tconv_fwd(x3, w, b, F)
        if np.allclose(y3[:, (c + 1) * F], y[:, (c + 1) * F]):
            return False
    return True


PINS = [_check_golden, _check_single_block_is_same_conv, _check_one_frame_blocks_are_causal_two_tap,
        _check_brute_force, _check_streaming, _check_causality]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__[7:] for p in PINS])
def test_pin(pin):
    assert pin()


def test_cache_size_is_constant_in_the_number_of_blocks():
    for nb in (1, 5, 40):
        x = _rand((1, 2 * nb, 3, 4, 8), nb)
        _, last = orc.tconv_fwd(x, _rand((8, 3), 0), None, 2)
        assert last.shape == (1, 3, 4, 8)


def test_linear_in_x():
    x1, x2 = _rand((1, 6, 2, 2, 3), 70), _rand((1, 6, 2, 2, 3), 71)
    w = _rand((3, 3), 72)
    y1, _ = orc.tconv_fwd(x1, w, None, 3)
    y2, _ = orc.tconv_fwd(x2, w, None, 3)
    y12, _ = orc.tconv_fwd(2 * x1 - 3 * x2, w, None, 3)
    assert np.allclose(y12, 2 * y1 - 3 * y2, rtol=1e-13, atol=1e-13)


# Planted mistakes.  Each replaces one oracle function on the CPU; the pins
# above must fail for every one.
_block_ok = orc.tconv_block
_fwd_ok = orc.tconv_fwd


def _reversed_taps(x_blk, carried, w, b):
    return _block_ok(x_blk, carried, np.asarray(w)[:, ::-1], b)


def _no_carry(x_blk, carried, w, b):
    return _block_ok(x_blk, np.zeros_like(np.asarray(carried, np.float64)), w, b)


def _edge_instead_of_separator(x_blk, carried, w, b):
    """Replicates the block's last frame where the zero token belongs."""
    y = _block_ok(x_blk, carried, w, b)
    y[:, -1] += np.asarray(w)[:, 2] * np.asarray(x_blk)[:, -1]
    return y


def _no_separator(x, w, b, F, cache=None):
    """Ignores the blocks: one 'same' convolution over the whole sequence."""
    y, last = _fwd_ok(x, w, b, x.shape[1], cache=cache)
    return y, last


def _carries_first_frame(x, w, b, F, cache=None):
    x = np.asarray(x, np.float64)
    B, T, Hs, Ws, C = x.shape
    carried = np.zeros((B, Hs, Ws, C)) if cache is None else np.asarray(cache, np.float64)
    y = np.empty_like(x)
    for c in range(T // F):
        blk = x[:, c * F:(c + 1) * F]
        y[:, c * F:(c + 1) * F] = orc.tconv_block(blk, carried, w, b)
        carried = blk[:, 0]
    return y, x[:, -1].copy()


MUTANTS = {
    "reversed_taps": ("tconv_block", _reversed_taps),
    "no_carry": ("tconv_block", _no_carry),
    "edge_instead_of_separator": ("tconv_block", _edge_instead_of_separator),
    "no_separator": ("tconv_fwd", _no_separator),
    "carries_first_frame": ("tconv_fwd", _carries_first_frame),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert not all(p() for p in PINS), f"planted mistake {name!r} went unnoticed"
