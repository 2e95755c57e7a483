"""Planted mistakes in the oracle (on the CPU, by monkeypatching) must be
caught by the pins: each mutant makes the oracle disagree with the brute
force or with the hand-worked closed forms.  This shows the pins are strong
enough to catch a dropped term, a wrong sign, a wrong index or a transposed
operand."""
import json
import math
import os

import numpy as np
import pytest

from oracle import sva_oracle as orc
from brute_force import brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
_rope_ok = orc.rope_rotate
_states_ok = orc.block_states
_coords_ok = orc.token_coords
_prep_ok = orc._prep


def _rope_sign_flipped(x, t, h, w, split, base):
    return _rope_ok(x, -np.asarray(t), -np.asarray(h), -np.asarray(w), split, base)


def _rope_axes_swapped(x, t, h, w, split, base):
    return _rope_ok(x, t, w, h, split, base)


def _states_exclusive(kt, pk, v, block_len):
    A, Z = _states_ok(kt, pk, v, block_len)
    A2, Z2 = np.zeros_like(A), np.zeros_like(Z)
    A2[1:], Z2[1:] = A[:-1], Z[:-1]           # a block no longer sees itself
    return A2, Z2


def _states_transposed(kt, pk, v, block_len):
    A, Z = _states_ok(kt, pk, v, block_len)
    return np.transpose(A, (0, 2, 1)).copy(), Z


def _states_dropped_z(kt, pk, v, block_len):
    A, Z = _states_ok(kt, pk, v, block_len)
    return A, Z * 0.0


def _prep_rope_in_denominator(q, k, grid, t0, rope, split, base):
    pq, pk, qt, kt = _prep_ok(q, k, grid, t0, rope, split, base)
    return qt, kt, qt, kt


def _coords_swapped_divisors(T, Hs, Ws, t0=0):
    n = np.arange(T * Hs * Ws)
    return t0 + n // (Hs * Ws), (n // Hs) % Ws, n % Hs    # Hs and Ws mixed up


MUTANTS = {
    "rope_sign": ("rope_rotate", _rope_sign_flipped),
    "rope_axes_swapped": ("rope_rotate", _rope_axes_swapped),
    "exclusive_prefix": ("block_states", _states_exclusive),
    "transposed_state": ("block_states", _states_transposed),
    "dropped_normaliser": ("block_states", _states_dropped_z),
    "rope_in_denominator": ("_prep", _prep_rope_in_denominator),
    "hw_decode_mixed_up": ("token_coords", _coords_swapped_divisors),
}


def _pins_hold():
    """The brute-force pin (two grids) and the hand-worked pin; True iff all pass."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    eps = inp["eps"]
    env = {"eps": eps, "cos": math.cos, "sin": math.sin}
    for case in g["cases"]:
        out, _, _ = orc.lin_attn_fwd(np.array(inp["q"])[None, None], np.array(inp["k"])[None, None],
                                     np.array(inp["v"])[None, None], tuple(case["grid"]),
                                     case["frames_per_block"], t0=case["t0"], rope=True,
                                     split=tuple(case["split"]), eps=eps)
        exp = np.array([[eval(e, {"__builtins__": {}}, env) for e in r] for r in case["expected"]])
        if not np.allclose(out[0, 0], exp, rtol=0, atol=1e-12):
            return False
    for (T, Hs, Ws, F, d, split, t0) in ((4, 2, 3, 2, 16, (4, 6, 6), 3), (4, 3, 2, 2, 8, (2, 2, 4), 0)):
        N = T * Hs * Ws
        rng = np.random.default_rng(7)
        q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
        out, _, _ = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, t0=t0, rope=True, split=split)
        ref = brute_force(q[0, 0], k[0, 0], v[0, 0], (T, Hs, Ws), F, t0=t0, rope=True, split=split)
        if np.max(np.abs(out[0, 0] - ref)) > 1e-10 * np.max(np.abs(ref)):
            return False
    return True


def test_unmutated_oracle_passes_pins():
    assert _pins_hold()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert not _pins_hold(), f"planted mistake {name!r} went unnoticed"
