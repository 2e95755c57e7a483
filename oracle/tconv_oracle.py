"""Plain fp64 CPU oracle for the causal temporal convolution of SANA-Video's
Mix-FFN and its constant-size block cache.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
statement of what the HIP library computes.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path (the C-ABI library and its Python binding) never does, and this module
imports nothing from the product.

Sources (the pages this follows):
  [talk]  "SANA-Video: Efficient Video Generation with Block Linear Diffusion
          Transformer, [ICLR 2026, Oral]" -- talk transcript
          (shadowingenglish.com), segment on the causal FFN with a temporal
          convolution.  With two blocks: in causal training block 1 must not
          see block 2, so one zero token is placed between them; block 2 must
          see block 1, so block 1's last token is carried in front of block 2;
          the padding's outputs are dropped.
  [study] the ICLR 2026 writing study of the paper (Computational Pathology
          pages), whose boundary note calls the attention state and the
          convolution history constant-size caches.

Readings taken where the pages are silent (each is a choice, not a quote):
  * the convolution runs along latent frames t, separately for every spatial
    position (h, w) and channel c (depthwise), with three taps w[c, 0..2] and
    a bias b[c]: three, because exactly one token of history is carried and
    one zero token closes a block;
  * cross-correlation order: w[c, 0] weighs the previous frame, w[c, 1] the
    frame itself, w[c, 2] the next frame;
  * activations are [B, T, Hs, Ws, C] (tokens in row-major (t, h, w) order,
    channels contiguous); a block is F whole latent frames;
  * the carried token of the first block is zero unless a cache is given;
    the cache is the last latent frame of the last committed block,
    [B, Hs, Ws, C], in the activation dtype (a copy of an input is exact).

Every function here is pinned by the CPU tests: a hand-worked example, the
textbook zero-padded convolution (single block), the strictly causal two-tap
convolution (one-frame blocks), a brute-force masked stencil, streaming
against one-shot, and planted mistakes.
"""

from __future__ import annotations

import numpy as np

__all__ = ["tconv_block", "tconv_fwd", "tconv_apply", "tconv_commit"]


def tconv_block(x_blk, carried, w, b):
    """One block as the talk builds it: the sequence [carried token, the
    block's F frames, one zero token] goes through a 'valid' three-tap
    correlation along t, which leaves exactly the block's F outputs.

    x_blk [B, F, Hs, Ws, C], carried [B, Hs, Ws, C], w [C, 3], b [C] or None.
    """
    x_blk = np.asarray(x_blk, dtype=np.float64)
    carried = np.asarray(carried, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, F, Hs, Ws, C = x_blk.shape
    seq = np.concatenate([carried[:, None], x_blk, np.zeros((B, 1, Hs, Ws, C))], axis=1)
    y = np.zeros_like(x_blk)
    for j in range(F):  # output j reads padded frames j, j+1, j+2
        for tap in range(3):
            y[:, j] += w[None, None, None, :, tap] * seq[:, j + tap]
    if b is not None:
        y += np.asarray(b, dtype=np.float64)[None, None, None, None, :]
    return y


def tconv_fwd(x, w, b, F, cache=None):
    """One-shot block-causal form over all T / F blocks (the training form):
    block c carries the last frame of block c-1 (block 0 carries `cache`, or
    zero).  Returns (y [B, T, Hs, Ws, C], last frame [B, Hs, Ws, C]), fp64."""
    x = np.asarray(x, dtype=np.float64)
    B, T, Hs, Ws, C = x.shape
    if T % F != 0:
        raise ValueError("T must be a whole number of blocks")
    carried = np.zeros((B, Hs, Ws, C)) if cache is None else np.asarray(cache, dtype=np.float64)
    y = np.empty_like(x)
    for c in range(T // F):
        blk = x[:, c * F:(c + 1) * F]
        y[:, c * F:(c + 1) * F] = tconv_block(blk, carried, w, b)
        carried = blk[:, -1]
    return y, x[:, -1].copy()


def tconv_apply(cache, x, w, b):
    """Output of one block (x holds exactly one block) against the cache;
    the cache is not modified."""
    return tconv_block(x, cache, w, b)


def tconv_commit(cache, x):
    """Cache after committing one block: its last frame.  Returns a new array
    (the previous cache is not needed: only one token of history is kept)."""
    del cache
    return np.array(np.asarray(x, dtype=np.float64)[:, -1], copy=True)
