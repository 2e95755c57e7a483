/*
 * sva_proj.h -- C ABI of the QKV projection with 4-bit block-scaled weights
 * that feeds libsva's attention, for AMD MI355X (gfx950).  Part of libsva.
 *
 * Pages this interface follows:
 *   [news] cstia.com SANA-Video article: its 4-bit quantization paragraph
 *          puts the self-attention QKV projections (among others) in 4-bit
 *          weights with SVDQuant, and its performance paragraph deploys
 *          them in NVFP4 on an RTX 5090.
 *   OCP Microscaling Formats (MX) Specification v1.0: the MXFP4 format used
 *          here (gfx950 implements the MX formats; NVFP4 is NVIDIA's).
 *
 * What is computed (readings: MXFP4 weights, bf16 activations, fp32
 * accumulation; output columns ordered [q | k | v] x H heads x d features):
 *   W[c][n]  = e2m1(code[n][c]) * 2^(scale[n][c / 32] - 127)
 *   y[m][n]  = sum_c x[m][c] W[c][n] + bias[n]        (m = b * N + token)
 *   q[b][h][t][f] = y[b*N + t][0*H*d + h*d + f], k: 1*H*d + ..., v: 2*H*d + ...
 * E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa; exponent 0
 * holds 0 and 0.5.  E8M0: 2^(e - 127), e = 255 is NaN.  Every weight is
 * decoded exactly to bf16; the products accumulate in fp32 and the outputs
 * are rounded to bf16 (nearest even).  A weight whose value exceeds the
 * bf16 range (e8m0 253 with |e2m1| >= 4, or 254 with |e2m1| >= 2: above
 * 2^128, out of fp32's range too) decodes to an infinity, and sums beyond
 * the range become infinities as the rounding dictates.
 *
 * Layouts:
 *   x       [B, N, C] bf16, contiguous (tokens of a sample in order)
 *   codes   [3*H*d, C/2] bytes: output row n holds the codes of input
 *           channels 2j (low nibble) and 2j+1 (high nibble) in byte j
 *   scales  [3*H*d, C/32] bytes (E8M0), one per 32 input channels
 *   bias    [3*H*d] fp32, or NULL
 *   q, k, v [B, H, N, d] bf16, the layout sva_lin_attn_* take
 * Limits: C a multiple of 128; H*d a multiple of 128; d a multiple of 8.
 *
 * Ownership and errors as in sva.h: caller-owned device pointers (x, q, k,
 * v 16-byte aligned; codes 8-byte and scales 4-byte aligned), nothing
 * allocated or kept, synchronous validation before any launch (nothing
 * written on error), work queued on `stream`.  No workspace is needed.
 */
#ifndef SVA_PROJ_H
#define SVA_PROJ_H

#include "sva.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sva_proj_desc {
  int B;  /* samples */
  int N;  /* tokens per sample */
  int C;  /* input channels */
  int H;  /* heads */
  int d;  /* head dimension */
} sva_proj_desc;

/* q, k, v = split(x W + bias) as above.  q, k, v must not overlap each
 * other or any input.  SVA_ERR_UNSUPPORTED for C, H*d or d outside the
 * limits; SVA_ERR_INVALID_ARG for a bad shape, pointer or overlap. */
sva_status sva_qkv_proj_mxfp4(const sva_proj_desc* desc, const void* x, const void* codes,
                              const void* scales, const float* bias, void* q, void* k, void* v,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVA_PROJ_H */
