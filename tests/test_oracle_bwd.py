"""Pins of the oracle's backward against something other than itself: central
finite differences of the forward oracle.

For L = sum(out * dout) + sum(S_final * dS_final) + sum(z_final * dz_final),
the directional derivative of L along a random direction U of one input,
(L(X + hU) - L(X - hU)) / 2h, must equal <dL/dX, U> from lin_attn_bwd.  The
forward oracle is itself pinned to the brute-force quadratic form, so this
checks the gradient formulas independently of how they were derived.
Inputs keep |q|, |k| >= 0.05 so that no step of size h crosses the ReLU kink.

Planted mistakes in the backward (monkeypatched on the CPU) must fail the
same pin: a missing ReLU mask, the forward rotation in place of its
transpose, a prefix in place of the suffix, a dropped denominator term, an
untransposed state.
"""
import numpy as np
import pytest

from oracle import sva_oracle as orc

# (grid, F, d, split or None, t0, with initial cache, with final-state gradient)
CASES = [
    ((4, 2, 3), 2, 8, (2, 2, 4), 1, False, False),
    ((6, 2, 2), 3, 6, (2, 2, 2), 0, True, True),
    ((3, 3, 2), 1, 8, None, 0, True, False),
    ((2, 2, 5), 2, 4, (0, 2, 2), 5, False, True),
    ((4, 1, 4), 1, 6, (4, 0, 2), 2, True, True),
]


def _away_from_zero(rng, shape):
    x = rng.standard_normal(shape)
    return np.sign(x) * (0.05 + np.abs(x))


def _inputs(case, seed):
    grid, F, d, split, t0, with_cache, with_final = case
    rng = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    x = {"q": _away_from_zero(rng, (1, 2, N, d)), "k": _away_from_zero(rng, (1, 2, N, d)),
         "v": rng.standard_normal((1, 2, N, d))}
    x["S0"] = rng.standard_normal((1, 2, d, d)) if with_cache else None
    x["z0"] = np.abs(rng.standard_normal((1, 2, d))) if with_cache else None
    g = {"dout": rng.standard_normal((1, 2, N, d)),
         "dS_final": rng.standard_normal((1, 2, d, d)) if with_final else None,
         "dz_final": rng.standard_normal((1, 2, d)) if with_final else None}
    kw = dict(t0=t0, rope=split is not None, split=split, eps=1e-3)
    return x, g, kw


def _loss(x, g, case, kw):
    grid, F = case[0], case[1]
    out, S_f, z_f = orc.lin_attn_fwd(x["q"], x["k"], x["v"], grid, F, S0=x["S0"], z0=x["z0"], **kw)
    L = np.sum(out * g["dout"])
    if g["dS_final"] is not None:
        L += np.sum(S_f * g["dS_final"]) + np.sum(z_f * g["dz_final"])
    return L


def _fd_holds(case, seed=0, h=1e-6, rtol=1e-6):
    """True iff every input's directional derivative matches the backward."""
    x, g, kw = _inputs(case, seed)
    grid, F = case[0], case[1]
    dq, dk, dv, dS0, dz0 = orc.lin_attn_bwd(x["q"], x["k"], x["v"], g["dout"], grid, F, S0=x["S0"],
                                            z0=x["z0"], dS_final=g["dS_final"], dz_final=g["dz_final"], **kw)
    grads = {"q": dq, "k": dk, "v": dv, "S0": dS0, "z0": dz0}
    rng = np.random.default_rng(seed + 100)
    for name in ("q", "k", "v", "S0", "z0"):
        if x[name] is None:
            continue
        U = rng.standard_normal(x[name].shape)
        xp = dict(x); xp[name] = x[name] + h * U
        xm = dict(x); xm[name] = x[name] - h * U
        fd = (_loss(xp, g, case, kw) - _loss(xm, g, case, kw)) / (2 * h)
        an = np.sum(grads[name] * U)
        if not abs(fd - an) <= rtol * max(1.0, abs(an)):
            return False
    return True


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_backward_matches_finite_differences(case):
    assert _fd_holds(case)


def test_zero_initial_cache_gradient_equals_suffix_of_everything():
    """dS0 is the gradient reaching every block's state: with no RoPE, one
    block and eps -> 0 dropped, it equals phi(q)^T (dout / den)."""
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal((1, 1, 12, 4)) for _ in range(4))
    _, _, _, dS0, _ = orc.lin_attn_bwd(q, k, v, do, (1, 3, 4), 1, eps=1e-6)
    pq, pk = np.maximum(q[0, 0], 0), np.maximum(k[0, 0], 0)
    den = pq @ pk.sum(axis=0) + 1e-6
    assert np.allclose(dS0[0, 0], pq.T @ (do[0, 0] / den[:, None]), rtol=1e-12, atol=1e-12)


def test_dv_is_linear_in_dout_and_independent_of_v():
    rng = np.random.default_rng(4)
    q, k, v, d1, d2 = (rng.standard_normal((1, 1, 18, 6)) for _ in range(5))
    kw = dict(rope=True, split=(2, 2, 2), t0=1)
    a = orc.lin_attn_bwd(q, k, v, d1, (3, 2, 3), 1, **kw)[2]
    b = orc.lin_attn_bwd(q, k, v, d2, (3, 2, 3), 1, **kw)[2]
    ab = orc.lin_attn_bwd(q, k, v, 2 * d1 - d2, (3, 2, 3), 1, **kw)[2]
    assert np.allclose(ab, 2 * a - b, rtol=1e-12, atol=1e-12)
    c = orc.lin_attn_bwd(q, k, 3 * v, d1, (3, 2, 3), 1, **kw)[2]
    assert np.allclose(c, a, rtol=1e-12, atol=1e-12)


_relu_grad_ok = orc._relu_grad
_suffix_ok = orc._suffix_sum
_out_grads_ok = orc._out_grads
_state_grads_ok = orc._state_grads


def _rope_t_forward(x, t, h, w, split, base):
    return orc.rope_rotate(x, t, h, w, split, base)


def _no_mask(x):
    return np.ones_like(np.asarray(x, dtype=np.float64))


def _prefix(x):
    return np.cumsum(x, axis=0)


def _dropped_den(qt_c, pq_c, S_c, Z_c, dout_c, eps):
    dqt, dpq, dS, dZ = _out_grads_ok(qt_c, pq_c, S_c, Z_c, dout_c, eps)
    return dqt, dpq * 0.0, dS, dZ * 0.0


def _untransposed_S(qt_c, pq_c, S_c, Z_c, dout_c, eps):
    dqt, dpq, dS, dZ = _out_grads_ok(qt_c, pq_c, S_c, Z_c, dout_c, eps)
    den = pq_c @ Z_c + eps
    return (dout_c / den[:, None]) @ S_c, dpq, dS, dZ


def _untransposed_G(kt_c, v_c, G_c, g_c):
    dkt, dv, dpk = _state_grads_ok(kt_c, v_c, G_c, g_c)
    return v_c @ G_c, dv, dpk


BWD_MUTANTS = {
    "no_relu_mask": ("_relu_grad", _no_mask),
    "rope_not_transposed": ("_rope_transpose", _rope_t_forward),
    "prefix_not_suffix": ("_suffix_sum", _prefix),
    "dropped_denominator_term": ("_out_grads", _dropped_den),
    "untransposed_state": ("_out_grads", _untransposed_S),
    "untransposed_state_gradient": ("_state_grads", _untransposed_G),
}


def _all_cases_hold():
    return all(_fd_holds(c) for c in CASES)


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name, monkeypatch):
    attr, fn = BWD_MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert not _all_cases_hold(), f"planted mistake {name!r} went unnoticed"
