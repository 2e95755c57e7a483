"""Plain fp64 CPU oracle for the QKV projection with 4-bit block-scaled
weights that feeds the attention.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
statement of what the HIP library computes.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path never does, and this module imports nothing from the product.

Sources:
  [news]  cstia.com SANA-Video article: the 4-bit quantization paragraph
          (SVDQuant puts the self-attention QKV and output projections, the
          cross-attention query and output projections and the FFN 1x1
          convolutions in 4 bits; norms, the temporal convolution and the
          cross-attention KV projections stay in higher precision) and the
          performance paragraph (NVFP4 deployment on an RTX 5090).
  OCP Microscaling Formats (MX) Specification v1.0: the MXFP4 format used
          here -- blocks of 32 elements share one E8M0 scale (2^(e-127),
          e = 255 is NaN); each element is FP4 E2M1 (1 sign, 2 exponent bits
          with bias 1, 1 mantissa bit; exponent 0 is subnormal: 0 or 0.5).

  OCP MX Specification v1.0, conversion to an MX format (its section 6.3):
          a block's shared scale is 2^(floor(log2(max |V_i|)) - emax_elem),
          emax_elem being the largest exponent of the element format (2 for
          E2M1, whose largest value is 6 = 1.5 * 2^2); each element is
          V_i / scale rounded to the element format, ties to even, values
          past the largest normal clamped to it.

Readings taken (each is a choice, not a quote):
  * the 4-bit format is MXFP4 (the block-scaled FP4 that gfx950 implements),
    not NVFP4; the blocks run along the input channels;
  * two activation precisions: bf16 activations (W4A16: 4-bit weights,
    16-bit activations), and MXFP4 activations (W4A4, as SVDQuant's NVFP4
    deployment quantizes both operands of the projection to 4 bits), each
    token row quantized per 32 input channels as the MX conversion above
    states, the shared exponent clamped to E8M0's range [-127, 127] and an
    all-zero block given scale byte 0; weights are decoded exactly and the
    products accumulate in fp32 on the GPU;
  * the fused weight's output columns are [q | k | v], each H heads of d
    features: column n = which * H * d + h * d + f;
  * the outputs are q, k, v in the attention's [B, H, N, d] layout, rounded
    to bf16; the bias, if any, is fp32.
"""

from __future__ import annotations

import numpy as np

__all__ = ["e2m1_value", "e8m0_value", "mxfp4_decode", "mxfp4_quantize", "qkv_project", "qkv_project_w4a4"]


def e2m1_value(code):
    """Value of a 4-bit E2M1 code (0..15): bit 3 sign, bits 2..1 exponent
    (bias 1), bit 0 mantissa; exponent 0 holds the subnormals 0 and 0.5."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 8, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return sign * mag


def e8m0_value(s):
    """Value of an E8M0 scale byte: 2^(s - 127); 255 is NaN."""
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def mxfp4_decode(codes, scales):
    """codes [N_out, K] (4-bit values), scales [N_out, K / 32] (bytes) ->
    W^T [N_out, K] fp64: element (n, k) is e2m1(code) * 2^(scale[n, k//32] - 127)."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    n_out, k = codes.shape
    if k % 32 != 0 or scales.shape != (n_out, k // 32):
        raise ValueError("scales must be [N_out, K / 32]")
    return e2m1_value(codes) * np.repeat(e8m0_value(scales), 32, axis=1)


def qkv_project(x, codes, scales, bias, H, d):
    """x [B, N, C] -> (q, k, v), each [B, H, N, d] fp64:
    y = x W + bias with W = mxfp4_decode(codes, scales)^T, columns split as
    [q | k | v] x H heads x d features."""
    x = np.asarray(x, dtype=np.float64)
    B, N, C = x.shape
    wt = mxfp4_decode(codes, scales)  # [3 H d, C]
    if wt.shape != (3 * H * d, C):
        raise ValueError("weights must be [3 * H * d, C]")
    y = x @ wt.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, None, :]
    y = y.reshape(B, N, 3, H, d).transpose(2, 0, 3, 1, 4)  # [3, B, H, N, d]
    return y[0].copy(), y[1].copy(), y[2].copy()


_E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # codes 0..7


def mxfp4_quantize(x):
    """x [..., K] (K a multiple of 32) -> (codes [..., K] in 0..15, scales
    [..., K / 32] bytes), by the MX conversion: per block of 32 consecutive
    elements, E = floor(log2(max |x_i|)) - 2 clamped to [-127, 127] (an
    all-zero block takes E = -127), scale byte E + 127, and element i the
    E2M1 code whose magnitude is nearest to |x_i| / 2^E -- at equal distance
    the even code -- with the sign of x_i (so -0.0 and negatives that round to
    zero keep the sign bit).  The largest magnitude, 6, is the nearest value
    for everything above 5, which is the clamping of the specification."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % 32 != 0:
        raise ValueError("the last axis must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (K // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(amax)  # amax = m 2^e, m in [0.5, 1): floor(log2 amax) = e - 1
    E = np.where(amax > 0, e - 1 - 2, -127)
    E = np.clip(E, -127, 127)
    v = np.abs(blocks) / np.ldexp(1.0, E)[..., None]
    dist = np.abs(v[..., None] - _E2M1_MAGNITUDES)  # [..., 32, 8]
    best = dist.min(axis=-1, keepdims=True)
    # the nearest magnitudes; among two at equal distance, the even code
    cand = np.where(dist == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    code = np.where(even < 99, even, cand.min(axis=-1))
    code = code + 8 * np.signbit(blocks)
    return code.reshape(x.shape).astype(np.int64), (E + 127).astype(np.int64)


def qkv_project_w4a4(x, codes, scales, bias, H, d):
    """As qkv_project, with the activations taken through mxfp4_quantize first
    (per token row, blocks along the input channels): y = X W + bias with
    X = mxfp4_decode(mxfp4_quantize(x)) and W = mxfp4_decode(codes, scales)^T."""
    x = np.asarray(x, dtype=np.float64)
    B, N, C = x.shape
    xc, xs = mxfp4_quantize(x.reshape(B * N, C))
    xq = mxfp4_decode(xc, xs).reshape(B, N, C)
    return qkv_project(xq, codes, scales, bias, H, d)
