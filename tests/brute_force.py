"""Brute-force statement of block-causal linear attention: the O(N^2)
masked quadratic form, used to pin the factored oracle on tiny inputs.

It is written independently of oracle/: positions come from numpy's
unravel_index, RoPE is a complex multiply (x_{2i} + i x_{2i+1}) e^{i theta},
and the block-causal rule is an explicit N x N mask blk(m) <= blk(n)
([talk] "SANA-Video ... ICLR 2026 Oral" transcript, block causal linear
attention segment: block 1 cannot see block 2, block 2 sees block 1).
The numerator carries RoPE and the denominator does not ([news] cstia.com
SANA-Video article, positional-encoding paragraph).
"""
import numpy as np


def _rope_complex(x, pos_by_axis, split, base):
    out = np.zeros_like(x)
    start = 0
    for pos, width in zip(pos_by_axis, split):
        for i in range(width // 2):
            ang = pos * base ** (-(2.0 * i) / width)
            zc = (x[:, start + 2 * i] + 1j * x[:, start + 2 * i + 1]) * np.exp(1j * ang)
            out[:, start + 2 * i] = zc.real
            out[:, start + 2 * i + 1] = zc.imag
        start += width
    return out


def brute_force(q, k, v, grid, F, t0=0, rope=False, split=None, base=10000.0,
                eps=1e-6, S0=None, z0=None):
    """q, k, v: [N, d] for ONE (batch, head) slice; returns [N, dv] fp64."""
    T, Hs, Ws = grid
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N = q.shape[0]
    tt, hh, ww = np.unravel_index(np.arange(N), (T, Hs, Ws))
    frame = tt
    tt = tt + t0
    fq = np.where(q > 0, q, 0.0)
    fk = np.where(k > 0, k, 0.0)
    if rope:
        pos = (tt.astype(np.float64), hh.astype(np.float64), ww.astype(np.float64))
        rq = _rope_complex(fq, pos, split, base)
        rk = _rope_complex(fk, pos, split, base)
    else:
        rq, rk = fq, fk
    blk = frame // F
    mask = (blk[None, :] <= blk[:, None]).astype(np.float64)   # [n, m]
    num = (mask * (rq @ rk.T)) @ v
    den = (mask * (fq @ fk.T)).sum(axis=1)
    if S0 is not None:
        num = num + rq @ np.asarray(S0, np.float64)
        den = den + fq @ np.asarray(z0, np.float64)
    return num / (den + eps)[:, None]
