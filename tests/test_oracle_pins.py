"""Pins of the fp64 oracle against things other than itself: a hand-worked
closed form, the brute-force masked quadratic form, a textbook special case,
and invariants the method must satisfy.  CPU only.

Pages: [talk] SANA-Video ICLR 2026 Oral talk transcript (shadowingenglish.com);
[news] cstia.com SANA-Video article.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import sva_oracle as orc
from brute_force import brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _relerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# (T, Hs, Ws, F, d, rope, split, t0)
BRUTE_CASES = [
    (4, 8, 8, 1, 32, False, None, 0),          # tiny-config shape, 4 blocks x 64 tokens
    (4, 2, 3, 2, 16, True, (4, 6, 6), 0),      # tiny RoPE grid, 2 blocks
    (6, 3, 2, 2, 8, True, (2, 2, 4), 5),       # global t0 != 0, 3 blocks
    (3, 2, 5, 3, 12, True, (4, 0, 8), 2),      # single block, one axis unused
    (5, 1, 4, 1, 6, True, (2, 2, 2), 0),       # block per frame, Hs = 1
]


def _golden_eval(expr, eps):
    return eval(expr, {"__builtins__": {}}, {"eps": eps, "cos": math.cos, "sin": math.sin})


def test_hand_worked_golden():
    """Hand-derived closed forms (tests/golden/hand_worked.json) pin the
    rotation direction, the axis a pair follows, the block-causal rule and the
    RoPE-free denominator."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    q = np.array(inp["q"])[None, None]
    k = np.array(inp["k"])[None, None]
    v = np.array(inp["v"])[None, None]
    eps = inp["eps"]
    for case in g["cases"]:
        out, _, _ = orc.lin_attn_fwd(q, k, v, tuple(case["grid"]), case["frames_per_block"],
                                     t0=case["t0"], rope=True, split=tuple(case["split"]),
                                     base=10000.0, eps=eps)
        exp = np.array([[_golden_eval(e, eps) for e in row] for row in case["expected"]])
        np.testing.assert_allclose(out[0, 0], exp, rtol=0, atol=1e-14, err_msg=case["name"])


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_factored_equals_brute_force(case):
    T, Hs, Ws, F, d, rope, split, t0 = case
    N = T * Hs * Ws
    B, H = 1, 2
    q = _rand(1, (B, H, N, d))
    k = _rand(2, (B, H, N, d))
    v = _rand(3, (B, H, N, d))
    out, _, _ = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, t0=t0, rope=rope, split=split, eps=1e-6)
    for h in range(H):
        ref = brute_force(q[0, h], k[0, h], v[0, h], (T, Hs, Ws), F, t0=t0, rope=rope,
                          split=split, eps=1e-6)
        assert _relerr(out[0, h], ref) <= 1e-12


def test_factored_equals_brute_force_with_initial_cache():
    T, Hs, Ws, F, d, split = 4, 2, 3, 2, 16, (4, 6, 6)
    N = T * Hs * Ws
    q, k, v = (_rand(s, (1, 1, N, d)) for s in (4, 5, 6))
    S0 = _rand(7, (1, 1, d, d))
    z0 = np.abs(_rand(8, (1, 1, d))) * 3
    out, S_f, z_f = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, t0=6, rope=True, split=split,
                                     S0=S0, z0=z0)
    ref = brute_force(q[0, 0], k[0, 0], v[0, 0], (T, Hs, Ws), F, t0=6, rope=True, split=split,
                      S0=S0[0, 0], z0=z0[0, 0])
    assert _relerr(out[0, 0], ref) <= 1e-12


def test_single_block_is_noncausal_relu_linear_attention():
    """One block, no RoPE: every token sees every token, so the result is
    textbook non-causal linear attention phiQ (phiK^T V) / (phiQ phiK^T 1 + eps)."""
    N, d = 200, 32
    q, k, v = (_rand(s, (N, d)) for s in (10, 11, 12))
    fq, fk = np.clip(q, 0, None), np.clip(k, 0, None)
    ref = (fq @ (fk.T @ v)) / ((fq @ fk.T.sum(axis=1)) + 1e-6)[:, None]
    out, _, _ = orc.lin_attn_fwd(q[None, None], k[None, None], v[None, None], (1, 10, 20), 1)
    assert _relerr(out[0, 0], ref) <= 1e-12


def test_all_zero_positions_equal_no_rope():
    """With dt = 0 and a 1 x 1 frame, every RoPE angle is zero: the RoPE
    result must equal the no-RoPE result exactly."""
    T, d = 6, 16
    q, k, v = (_rand(s, (1, 2, T, d)) for s in (20, 21, 22))
    a, Sa, za = orc.lin_attn_fwd(q, k, v, (T, 1, 1), 2, rope=True, split=(0, 8, 8))
    b, Sb, zb = orc.lin_attn_fwd(q, k, v, (T, 1, 1), 2, rope=False)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(Sa, Sb)


def test_rotation_preserves_pair_norms():
    N, d, split = 500, 64, (16, 24, 24)
    x = _rand(30, (N, d))
    rng = np.random.default_rng(31)
    t, h, w = (rng.integers(0, 300, N) for _ in range(3))
    y = orc.rope_rotate(x, t, h, w, split, 10000.0)
    nx = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    ny = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13, atol=0)


def test_rope_dot_depends_only_on_relative_position():
    """(R(p+c) x) . (R(p'+c) y) = (R(p) x) . (R(p') y) on every axis."""
    N, d, split = 300, 64, (16, 24, 24)
    x, y = _rand(40, (N, d)), _rand(41, (N, d))
    rng = np.random.default_rng(42)
    p1 = [rng.integers(0, 50, N) for _ in range(3)]
    p2 = [rng.integers(0, 50, N) for _ in range(3)]
    base = np.sum(orc.rope_rotate(x, *p1, split, 1e4) * orc.rope_rotate(y, *p2, split, 1e4), axis=1)
    for axis in range(3):
        s1 = [p + (17 if a == axis else 0) for a, p in enumerate(p1)]
        s2 = [p + (17 if a == axis else 0) for a, p in enumerate(p2)]
        shifted = np.sum(orc.rope_rotate(x, *s1, split, 1e4) * orc.rope_rotate(y, *s2, split, 1e4), axis=1)
        np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-10)


def test_global_frame_shift_leaves_output_unchanged():
    """Shifting every t by a constant (t0) changes no one-shot output: the
    numerator depends on relative positions only, the denominator has no RoPE."""
    T, Hs, Ws, F, d, split = 6, 3, 4, 2, 16, (4, 6, 6)
    N = T * Hs * Ws
    q, k, v = (_rand(s, (1, 1, N, d)) for s in (50, 51, 52))
    a, _, _ = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, t0=0, rope=True, split=split)
    b, _, _ = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, t0=37, rope=True, split=split)
    assert _relerr(b, a) <= 1e-12


def test_v_ones_gives_one_without_rope_and_not_with_rope():
    """[news] positional-encoding paragraph: RoPE only in the numerator.
    Without RoPE, V = 1 gives o = den / (den + eps), i.e. 1 up to eps/den.
    With RoPE the numerator and denominator differ, so o != 1."""
    T, Hs, Ws, F, d = 4, 4, 4, 2, 16
    N = T * Hs * Ws
    q, k = _rand(60, (1, 1, N, d)), _rand(61, (1, 1, N, d))
    ones = np.ones((1, 1, N, d))
    o, _, _ = orc.lin_attn_fwd(q, k, ones, (T, Hs, Ws), F, rope=False, eps=1e-6)
    assert np.max(np.abs(o - 1.0)) < 1e-5
    o2, _, _ = orc.lin_attn_fwd(q, k, ones, (T, Hs, Ws), F, rope=True, split=(4, 6, 6), eps=1e-6)
    assert np.max(np.abs(o2 - 1.0)) > 1e-2


def test_output_is_linear_in_v():
    T, Hs, Ws, F, d, split = 4, 3, 3, 2, 16, (4, 6, 6)
    N = T * Hs * Ws
    q, k, v1, v2 = (_rand(s, (1, 1, N, d)) for s in (70, 71, 72, 73))
    f = lambda v: orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, rope=True, split=split)[0]
    lhs = f(2.5 * v1 - 0.75 * v2)
    rhs = 2.5 * f(v1) - 0.75 * f(v2)
    assert _relerr(lhs, rhs) <= 1e-12


def test_streaming_apply_commit_equals_one_shot():
    """[talk] block KV cache segment: the state of block i is the cache of
    blocks < i plus block i's own KV.  Streaming one block at a time against
    a committed cache must give the one-shot forward's outputs and final
    cache; apply must leave the cache untouched; a snapshot of the cache
    restores the stream exactly."""
    T, Hs, Ws, F, d, split = 8, 3, 4, 2, 16, (4, 6, 6)
    HW = Hs * Ws
    N = T * HW
    B, H = 2, 2
    q, k, v = (_rand(s, (B, H, N, d)) for s in (80, 81, 82))
    ref, S_ref, z_ref = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, rope=True, split=split)
    S = np.zeros((B, H, d, d))
    z = np.zeros((B, H, d))
    snap = None
    for c in range(T // F):
        sl = slice(c * F * HW, (c + 1) * F * HW)
        S_before, z_before = S.copy(), z.copy()
        out = orc.block_cache_apply(S, z, q[:, :, sl], k[:, :, sl], v[:, :, sl], (F, Hs, Ws),
                                    t0=c * F, rope=True, split=split)
        np.testing.assert_array_equal(S, S_before)
        np.testing.assert_array_equal(z, z_before)
        assert _relerr(out, ref[:, :, sl]) <= 1e-12
        S, z = orc.block_cache_commit(S, z, k[:, :, sl], v[:, :, sl], (F, Hs, Ws),
                                      t0=c * F, rope=True, split=split)
        if c == 1:
            snap = (S.copy(), z.copy())
    assert _relerr(S, S_ref) <= 1e-12 and _relerr(z, z_ref) <= 1e-12
    # resume from the snapshot taken after block 1
    S2, z2 = snap
    for c in range(2, T // F):
        sl = slice(c * F * HW, (c + 1) * F * HW)
        S2, z2 = orc.block_cache_commit(S2, z2, k[:, :, sl], v[:, :, sl], (F, Hs, Ws),
                                        t0=c * F, rope=True, split=split)
    np.testing.assert_array_equal(S2, S)
    np.testing.assert_array_equal(z2, z)


def test_cache_size_is_constant_in_block_count():
    """[talk]: constant memory usage regardless of the sequence length."""
    d, Hs, Ws, F = 8, 2, 2, 1
    sizes = set()
    for T in (1, 2, 5, 13):
        N = T * Hs * Ws
        q, k, v = (_rand(s, (1, 1, N, d)) for s in (90, 91, 92))
        _, S, z = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, rope=True, split=(2, 2, 4))
        sizes.add((S.shape, z.shape))
    assert sizes == {((1, 1, d, d), (1, 1, d))}


def test_scaling_k_changes_output_only_through_eps():
    T, Hs, Ws, F, d, split = 4, 3, 3, 2, 16, (4, 6, 6)
    N = T * Hs * Ws
    q, k, v = (_rand(s, (1, 1, N, d)) for s in (100, 101, 102))
    a, _, _ = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, rope=True, split=split, eps=1e-6)
    b, _, _ = orc.lin_attn_fwd(q, 0.5 * k, v, (T, Hs, Ws), F, rope=True, split=split, eps=1e-6)
    c, _, _ = orc.lin_attn_fwd(q, 0.5 * k, v, (T, Hs, Ws), F, rope=True, split=split, eps=0.0)
    d0, _, _ = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, rope=True, split=split, eps=0.0)
    assert _relerr(c, d0) <= 1e-12          # exactly invariant at eps = 0
    assert _relerr(b, a) <= 1e-5            # only an eps-sized change otherwise
    assert _relerr(b, a) > 0


def test_block_causality():
    """[talk] block causal segment: block 1 cannot see block 2, block 2 sees
    block 1.  Changing block c' leaves every block before c' bit-identical and
    changes later blocks (global history)."""
    T, Hs, Ws, F, d, split = 8, 2, 3, 2, 16, (4, 6, 6)
    HW = Hs * Ws
    N = T * HW
    q, k, v = (_rand(s, (1, 1, N, d)) for s in (110, 111, 112))
    base, _, _ = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, rope=True, split=split)
    for cp in range(T // F):
        sl = slice(cp * F * HW, (cp + 1) * F * HW)
        k2, v2 = k.copy(), v.copy()
        k2[:, :, sl] += _rand(113 + cp, k2[:, :, sl].shape)
        v2[:, :, sl] += 1.0
        out, _, _ = orc.lin_attn_fwd(q, k2, v2, (T, Hs, Ws), F, rope=True, split=split)
        np.testing.assert_array_equal(out[:, :, :cp * F * HW], base[:, :, :cp * F * HW])
        assert np.max(np.abs(out[:, :, cp * F * HW:] - base[:, :, cp * F * HW:])) > 1e-3


def test_relu_of_negative_zero_and_dead_queries():
    """phi(q) = 0 gives an output of exactly 0 (numerator 0, den = eps)."""
    T, Hs, Ws, F, d = 2, 2, 2, 1, 8
    N = T * Hs * Ws
    q = -np.abs(_rand(120, (1, 1, N, d)))
    q[0, 0, 0] = -0.0
    k, v = _rand(121, (1, 1, N, d)), _rand(122, (1, 1, N, d))
    out, _, _ = orc.lin_attn_fwd(q, k, v, (T, Hs, Ws), F, rope=True, split=(2, 2, 4))
    np.testing.assert_array_equal(out, np.zeros_like(out))
