"""Plain fp64 CPU oracle for block-causal ReLU linear attention with a
numerator-only 3D RoPE and a constant-size block KV cache (SANA-Video).

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
statement of what the HIP library computes.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path (the C-ABI library and its Python binding) never does, and this module
imports nothing from the product.

Sources (the pages this follows):
  [talk]  "SANA-Video: Efficient Video Generation with Block Linear Diffusion
          Transformer, [ICLR 2026, Oral]" -- talk transcript
          (shadowingenglish.com).  Segments used: "linear attention ... the
          state ... a fixed shape of D times D"; "the block KV cache" (state of
          block 1 cached, each later block's KV added to the cache); "block
          causal linear attention" (block 1 cannot see block 2, block 2 sees
          block 1; constant memory, global history); "3D rope for the linear
          attention".
  [news]  cstia.com article "NVIDIA团队重磅突破：只用一张RTX 5090就能高速生成
          分钟级视频", paragraph on positional encoding: RoPE kept in the
          numerator, removed from the denominator for numerical stability.

Readings taken where the pages are silent (each is a choice, not a quote):
  * feature map phi = ReLU, applied elementwise to q and k;
  * output o = numerator / (denominator + eps) with
        numerator   = RoPE(phi q)^T S,      S = sum RoPE(phi k) v^T
        denominator = phi q . z,            z = sum phi k      (no RoPE);
  * ReLU first, then rotate; both q and k are rotated in the numerator;
  * 3D RoPE: head dims split into consecutive slices [t | h | w] of even
    widths (dt, dh, dw); inside the slice of axis a (width d_a), the pair of
    adjacent dims (2i, 2i+1) turns by angle pos_a * base**(-2i/d_a);
  * positions are integer latent coordinates; t is the global latent frame
    index (t0 + local frame), h and w start at 0 in every frame;
  * tokens are in row-major (t, h, w) order; a block is F whole latent
    frames; a token sees its own block (bidirectionally) and every earlier
    block; the initial cache is zero unless one is given.

The backward (lin_attn_bwd) is reverse-mode differentiation of the same
steps, for the training the pages run block-causally ([talk], block causal
segment); it is pinned by finite differences of lin_attn_fwd.

Parity unpinned: the RoPE pair convention (interleaved adjacent pairs) and
frequency schedule cannot be checked against the authors' code, which the
pages do not hold.  Everything else here is pinned by the CPU tests against
the brute-force masked quadratic form, closed forms and invariants.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "token_coords",
    "phi",
    "rope_rotate",
    "block_states",
    "lin_attn_fwd",
    "block_cache_apply",
    "block_cache_commit",
    "lin_attn_bwd",
]


def token_coords(T: int, Hs: int, Ws: int, t0: int = 0):
    """(t, h, w) of every token of a T x Hs x Ws latent grid in row-major
    order; t is global (t0 + local frame).  [talk], "3D rope" segment: the
    positions RoPE uses are the latent video coordinates."""
    n = np.arange(T * Hs * Ws, dtype=np.int64)
    t = t0 + n // (Hs * Ws)
    h = (n // Ws) % Hs
    w = n % Ws
    return t, h, w


def phi(x: np.ndarray) -> np.ndarray:
    """Kernel feature map of the linear attention.  The pages do not name it;
    the reading taken is ReLU."""
    return np.maximum(x, 0.0)


def rope_rotate(x: np.ndarray, t, h, w, split, base: float) -> np.ndarray:
    """3D RoPE of the rows of x ([N, d], fp64) at positions (t, h, w).

    [talk], "3D rope for the linear attention": position enters through a
    rotation per axis.  Head dims [0, dt) follow t, [dt, dt+dh) follow h and
    [dt+dh, d) follow w.  Inside an axis slice of width d_a the pair
    (2i, 2i+1) is turned by theta = pos * base**(-2i/d_a):
        (x, y) -> (x cos theta - y sin theta, x sin theta + y cos theta).
    """
    N, d = x.shape
    dt, dh, dw = split
    if dt + dh + dw != d or dt % 2 or dh % 2 or dw % 2:
        raise ValueError("RoPE split must be even widths summing to d")
    out = np.array(x, dtype=np.float64, copy=True)
    off = 0
    for pos, da in ((t, dt), (h, dh), (w, dw)):
        if da == 0:
            continue
        i = np.arange(da // 2, dtype=np.float64)
        inv_freq = float(base) ** (-2.0 * i / da)
        theta = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
        c = np.cos(theta)
        s = np.sin(theta)
        xe = x[:, off:off + da:2]
        xo = x[:, off + 1:off + da:2]
        out[:, off:off + da:2] = xe * c - xo * s
        out[:, off + 1:off + da:2] = xe * s + xo * c
        off += da
    return out


def _prep(q, k, grid, t0, rope, split, base):
    """phi on q and k, plus the rotated numerator copies (RoPE only on the
    numerator side, [news] paragraph on positional encoding)."""
    T, Hs, Ws = grid
    pq = phi(np.asarray(q, dtype=np.float64))
    pk = phi(np.asarray(k, dtype=np.float64))
    if rope:
        t, h, w = token_coords(T, Hs, Ws, t0)
        qt = rope_rotate(pq, t, h, w, split, base)
        kt = rope_rotate(pk, t, h, w, split, base)
    else:
        qt, kt = pq, pk
    return pq, pk, qt, kt


def block_states(kt: np.ndarray, pk: np.ndarray, v: np.ndarray, block_len: int):
    """Per-block state A_c = sum_{n in c} kt_n v_n^T (d x d) and normaliser
    zeta_c = sum_{n in c} phi(k)_n.  [talk], linear-attention segment: the
    state has a fixed d x d shape whatever the sequence length; block KV
    cache segment: a block's contribution is its own KV sum."""
    N, d = kt.shape
    nb = N // block_len
    A = np.zeros((nb, d, d), dtype=np.float64)
    Z = np.zeros((nb, d), dtype=np.float64)
    for c in range(nb):
        sl = slice(c * block_len, (c + 1) * block_len)
        A[c] = kt[sl].T @ np.asarray(v[sl], dtype=np.float64)
        Z[c] = pk[sl].sum(axis=0)
    return A, Z


def _fwd_slice(q, k, v, grid, F, t0, rope, split, base, eps, S0, z0):
    T, Hs, Ws = grid
    N, d = q.shape
    block_len = F * Hs * Ws
    nb = T // F
    pq, pk, qt, kt = _prep(q, k, grid, t0, rope, split, base)
    A, Z = block_states(kt, pk, v, block_len)
    # Block-causal prefix ([talk], block KV cache segment): the state a block
    # sees is the cache plus every block up to and including itself.
    S = np.asarray(S0, dtype=np.float64)[None] + np.cumsum(A, axis=0)
    Zc = np.asarray(z0, dtype=np.float64)[None] + np.cumsum(Z, axis=0)
    out = np.empty((N, v.shape[1]), dtype=np.float64)
    for c in range(nb):
        sl = slice(c * block_len, (c + 1) * block_len)
        num = qt[sl] @ S[c]                 # RoPE'd numerator
        den = pq[sl] @ Zc[c] + eps          # RoPE-free denominator
        out[sl] = num / den[:, None]
    return out, S[-1], Zc[-1]


def _check(q, k, v, grid, F):
    T, Hs, Ws = grid
    if q.ndim != 4 or q.shape != k.shape or q.shape[:3] != v.shape[:3]:
        raise ValueError("q, k, v must be [B, H, N, d] with equal B, H, N")
    if q.shape[2] != T * Hs * Ws:
        raise ValueError("N must equal T*Hs*Ws")
    if T % F:
        raise ValueError("T must be a multiple of frames_per_block")


def lin_attn_fwd(q, k, v, grid, F, *, t0=0, rope=False, split=None,
                 base=10000.0, eps=1e-6, S0=None, z0=None):
    """One-shot block-causal forward over all T/F blocks.

    q, k, v: [B, H, N, d] (any float dtype; upcast to fp64).  grid=(T, Hs, Ws).
    S0: [B, H, d, d], z0: [B, H, d] initial cache (zeros if None).
    Returns (out [B,H,N,d] fp64, S_final [B,H,d,d], z_final [B,H,d]).
    """
    _check(q, k, v, grid, F)
    B, H, N, d = q.shape
    dv = v.shape[3]
    out = np.empty((B, H, N, dv), dtype=np.float64)
    S_f = np.empty((B, H, d, dv), dtype=np.float64)
    z_f = np.empty((B, H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s0 = np.zeros((d, dv)) if S0 is None else S0[b, h]
            zz = np.zeros(d) if z0 is None else z0[b, h]
            out[b, h], S_f[b, h], z_f[b, h] = _fwd_slice(
                q[b, h], k[b, h], v[b, h], grid, F, t0, rope, split, base,
                eps, s0, zz)
    return out, S_f, z_f


def block_cache_apply(S, z, q, k, v, frame_grid, *, t0, rope=False, split=None,
                      base=10000.0, eps=1e-6):
    """Output of one block (frame_grid = (F, Hs, Ws), first frame at global
    index t0) against a committed cache (S, z), which is left unchanged.

    [talk] opening ("generate video block by block causally and diffuse
    within the block") and block KV cache segment (the current block uses
    the cached state plus its own contribution).
    """
    F = frame_grid[0]
    out, _, _ = lin_attn_fwd(q, k, v, frame_grid, F, t0=t0, rope=rope,
                             split=split, base=base, eps=eps, S0=S, z0=z)
    return out


def block_cache_commit(S, z, k, v, frame_grid, *, t0, rope=False, split=None,
                       base=10000.0):
    """Cache after adding one block: S + sum RoPE(phi k) v^T, z + sum phi k.
    [talk], block KV cache segment: the state is updated additively, only
    the current block's contribution is added to the previous cache.
    Returns new arrays; the inputs are not modified."""
    F, Hs, Ws = frame_grid
    B, H, N, d = k.shape
    if N != F * Hs * Ws:
        raise ValueError("commit takes exactly one block")
    S_new = np.array(S, dtype=np.float64, copy=True)
    z_new = np.array(z, dtype=np.float64, copy=True)
    for b in range(B):
        for h in range(H):
            _, pk, _, kt = _prep(k[b, h], k[b, h], frame_grid, t0, rope,
                                 split, base)
            A, Zb = block_states(kt, pk, v[b, h], N)
            S_new[b, h] += A[0]
            z_new[b, h] += Zb[0]
    return S_new, z_new


def _rope_transpose(x, t, h, w, split, base):
    """Transpose of rope_rotate at (t, h, w): every pair turns by the opposite
    angle, i.e. the same rotation at negated positions."""
    return rope_rotate(x, -np.asarray(t), -np.asarray(h), -np.asarray(w), split, base)


def _relu_grad(x):
    """d/dx ReLU(x): 1 where x > 0, 0 elsewhere (0 taken at the kink)."""
    return (np.asarray(x) > 0).astype(np.float64)


def _suffix_sum(x):
    """Inclusive suffix sums along axis 0: the transpose of the block prefix."""
    return np.cumsum(x[::-1], axis=0)[::-1]


def _out_grads(qt_c, pq_c, S_c, Z_c, dout_c, eps):
    """Gradients through one block's outputs o = (qt S_c) / (pq . Z_c + eps):
    returns (dqt, dpq from the denominator, dS_c, dZ_c)."""
    num = qt_c @ S_c
    den = pq_c @ Z_c + eps
    dnum = dout_c / den[:, None]
    dden = -(dout_c * num).sum(axis=1) / den ** 2
    return dnum @ S_c.T, dden[:, None] * Z_c[None, :], qt_c.T @ dnum, pq_c.T @ dden


def _state_grads(kt_c, v_c, G_c, g_c):
    """Gradients through one block's state A_c = kt^T v, zeta_c = sum pk when
    G_c, g_c reach A_c, zeta_c: returns (dkt, dv, dpk)."""
    return v_c @ G_c.T, kt_c @ G_c, np.broadcast_to(g_c[None, :], kt_c.shape)


def _bwd_slice(q, k, v, dout, grid, F, t0, rope, split, base, eps, S0, z0, dS_fin, dz_fin):
    """Reverse mode through _fwd_slice, step by step in the opposite order.

    Forward (per block c):  num = qt S_c,  den = pq . Z_c + eps,  o = num/den,
    with S_c = S0 + sum_{c'<=c} A_c', Z_c = z0 + sum_{c'<=c} zeta_c',
    A_c = sum kt v^T, zeta_c = sum pk.  Given dout (and optionally the
    gradient of the final state S_{nb-1}, Z_{nb-1}):
      dnum = dout / den,  dden = -(dout . num) / den^2
      dqt = dnum S_c^T,   dS_c = qt^T dnum,   dZ_c = pq^T dden,  dpq += dden Z_c
    The prefix turns into a suffix: the gradient reaching A_c (and S0) is
    G_c = sum_{c'>=c} dS_c' (+ dS_final), likewise g_c for zeta_c, so
      dkt = v G_c^T,  dv = kt G_c,  dpk = g_c.
    RoPE is a rotation per token, so its transpose is the rotation by the
    opposite angle, and d/dx ReLU(x) = 1 for x > 0, else 0."""
    T, Hs, Ws = grid
    N, d = q.shape
    block_len = F * Hs * Ws
    nb = T // F
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    pq, pk, qt, kt = _prep(q, k, grid, t0, rope, split, base)
    A, Z = block_states(kt, pk, v, block_len)
    S = np.asarray(S0, dtype=np.float64)[None] + np.cumsum(A, axis=0)
    Zc = np.asarray(z0, dtype=np.float64)[None] + np.cumsum(Z, axis=0)
    dqt = np.empty_like(qt)
    dpq = np.empty_like(pq)
    dS = np.empty_like(S)
    dZ = np.empty_like(Zc)
    for c in range(nb):
        sl = slice(c * block_len, (c + 1) * block_len)
        dqt[sl], dpq[sl], dS[c], dZ[c] = _out_grads(qt[sl], pq[sl], S[c], Zc[c], dout[sl], eps)
    # everything from block c on sees A_c: the prefix becomes a suffix
    G = _suffix_sum(dS) + np.asarray(dS_fin, dtype=np.float64)[None]
    g = _suffix_sum(dZ) + np.asarray(dz_fin, dtype=np.float64)[None]
    dkt = np.empty_like(kt)
    dv = np.empty_like(v)
    dpk = np.empty_like(pk)
    for c in range(nb):
        sl = slice(c * block_len, (c + 1) * block_len)
        dkt[sl], dv[sl], dpk[sl] = _state_grads(kt[sl], v[sl], G[c], g[c])
    if rope:
        t, h, w = token_coords(T, Hs, Ws, t0)
        dpq = dpq + _rope_transpose(dqt, t, h, w, split, base)
        dpk = dpk + _rope_transpose(dkt, t, h, w, split, base)
    else:
        dpq = dpq + dqt
        dpk = dpk + dkt
    return dpq * _relu_grad(q), dpk * _relu_grad(k), dv, G[0], g[0]


def lin_attn_bwd(q, k, v, dout, grid, F, *, t0=0, rope=False, split=None,
                 base=10000.0, eps=1e-6, S0=None, z0=None, dS_final=None, dz_final=None):
    """Gradients of lin_attn_fwd: for the scalar
        L = sum(out * dout) + sum(S_final * dS_final) + sum(z_final * dz_final)
    returns (dq, dk, dv, dS0, dz0), fp64, shaped like q, k, v, S0, z0.
    dS_final / dz_final default to zero (the final cache unused)."""
    _check(q, k, v, grid, F)
    B, H, N, d = q.shape
    dvv = v.shape[3]
    dq = np.empty((B, H, N, d))
    dk = np.empty((B, H, N, d))
    dv = np.empty((B, H, N, dvv))
    dS0 = np.empty((B, H, d, dvv))
    dz0 = np.empty((B, H, d))
    for b in range(B):
        for h in range(H):
            s0 = np.zeros((d, dvv)) if S0 is None else S0[b, h]
            zz = np.zeros(d) if z0 is None else z0[b, h]
            dsf = np.zeros((d, dvv)) if dS_final is None else dS_final[b, h]
            dzf = np.zeros(d) if dz_final is None else dz_final[b, h]
            dq[b, h], dk[b, h], dv[b, h], dS0[b, h], dz0[b, h] = _bwd_slice(
                q[b, h], k[b, h], v[b, h], dout[b, h], grid, F, t0, rope, split,
                base, eps, s0, zz, dsf, dzf)
    return dq, dk, dv, dS0, dz0
