"""Brute-force statement of the causal temporal convolution with a block
cache, used to pin oracle/tconv_oracle.py on tiny inputs.

Written independently of the oracle, from the visibility rule rather than
the padded-block construction: output frame t takes input frame s through
tap s - t + 1 when |s - t| <= 1 and s's block is not later than t's
([talk] "SANA-Video ... ICLR 2026 Oral" transcript, causal FFN with a
temporal convolution segment: block 1 cannot see block 2, block 2 sees block
1's last token).  Frame -1 is the cache (zero when absent).
"""
import numpy as np


def brute_tconv(x, w, b, F, cache=None):
    """x [B, T, Hs, Ws, C]; returns y fp64 of the same shape."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    B, T, Hs, Ws, C = x.shape
    ext = np.zeros((B, T + 1, Hs, Ws, C))  # ext[s + 1] = frame s, ext[0] = frame -1
    ext[:, 1:] = x
    if cache is not None:
        ext[:, 0] = np.asarray(cache, np.float64)
    y = np.zeros_like(x)
    for t in range(T):
        for s in range(-1, T):
            if abs(s - t) > 1:
                continue
            blk_s = -1 if s < 0 else s // F
            if blk_s > t // F:
                continue
            y[:, t] += w[:, s - t + 1] * ext[:, s + 1]
    if b is not None:
        y += np.asarray(b, np.float64)
    return y
