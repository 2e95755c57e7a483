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
 * What is computed (readings: MXFP4 weights, bf16 activations -- or MXFP4
 * activations, see sva_qkv_proj_w4a4 -- fp32 accumulation; output columns
 * ordered [q | k | v] x H heads x d features):
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
 *   wpack   the same codes and scales reordered by sva_mxfp4_pack_weights
 *           for the projection's loads; 3*H*d*C/2 + 3*H*d*C/32 bytes (the
 *           size of codes plus scales).  With P = 3*H*d/64 blocks of 64
 *           output rows and S = C/128 stages of 128 channels:
 *             codes part, [P][S][4][64] x 16 bytes: entry (p, s, t, l) holds
 *               channels 128 s + 32 (l / 16) .. + 31 of row 64 p + r(t, l % 16);
 *             scales part (after it), [P][S][64] words: byte t of word
 *               (p, s, l) is the scale of the same block;
 *             r(t, i) = 32 (t / 2) + 8 (i / 4) + 4 (t % 2) + i % 4.
 *   bias    [3*H*d] fp32, or NULL
 *   q, k, v [B, H, N, d] bf16, the layout sva_lin_attn_* take
 * Limits: C a multiple of 128; H*d a multiple of 64; d a multiple of 8.
 *
 * Ownership and errors as in sva.h: caller-owned device pointers (x, q, k,
 * v, codes and wpack 16-byte aligned), nothing allocated or kept,
 * synchronous validation before any launch (nothing written on error), work
 * queued on `stream`.  No workspace is needed.
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
  int range_tokens; /* sva_proj_lin_attn_fwd only: tokens per reduction
                       range, 0 = chosen by the library (see there);
                       ignored by the pack and projection calls */
} sva_proj_desc;

/* wpack = the packed form of (codes, scales), as above.  Weights are
 * constant across calls: pack them once.  wpack must not overlap codes or
 * scales.  SVA_ERR_UNSUPPORTED / SVA_ERR_INVALID_ARG as for the projection. */
sva_status sva_mxfp4_pack_weights(const sva_proj_desc* desc, const void* codes, const void* scales, void* wpack,
                                  void* stream);

/* q, k, v = split(x W + bias) as above, W given packed.  q, k, v must not
 * overlap each other or any input.  SVA_ERR_UNSUPPORTED for C, H*d or d
 * outside the limits; SVA_ERR_INVALID_ARG for a bad shape, pointer or
 * overlap. */
sva_status sva_qkv_proj_mxfp4(const sva_proj_desc* desc, const void* x, const void* wpack, const float* bias,
                              void* q, void* k, void* v, void* stream);

/* W4A4: the activations in MXFP4 as well.  SVDQuant's NVFP4 deployment
 * ([news], 4-bit quantization and performance paragraphs) quantizes both
 * operands of the projection to 4 bits; here the activations go through
 * the OCP MX conversion (specification section 6.3), per token row and 32
 * input channels:
 *   E      = floor(log2(max |x_i|)) - 2, clamped to >= -127 (an all-zero
 *            block: -127); scale byte E + 127
 *   code_i = the E2M1 code nearest to x_i / 2^E, ties to the even code,
 *            magnitudes above 6 clamped to 6, sign bit = x_i's (so values
 *            that round to zero keep it)
 * and the projection multiplies the 4-bit x by the 4-bit weights on the
 * scaled MFMA (exact products, fp32 sums), then adds the bias and rounds to
 * bf16 as sva_qkv_proj_mxfp4 does:
 *   y[m][n] = sum_c X[m][c] W[c][n] + bias[n],  X = decode(codes_x, scales_x).
 * x must be finite (a block holding an infinity or NaN gets unspecified
 * codes); weight scale byte 255 (NaN) is outside the contract here.
 *
 * Quantized activations (xq): codes [B*N, C/2] (channels 2j low nibble,
 * 2j+1 high nibble of byte j), then scales [B*N, C/32] (E8M0 bytes):
 * sva_mxfp4_acts_bytes bytes, 16-byte aligned, caller-owned. */
sva_status sva_mxfp4_acts_bytes(const sva_proj_desc* desc, size_t* bytes);

/* xq = the MX conversion of x [B, N, C] bf16, as above.  xq must not overlap
 * x.  Errors as for the projection. */
sva_status sva_mxfp4_quant_acts(const sva_proj_desc* desc, const void* x, void* xq, void* stream);

/* q, k, v = split(X W + bias) with X the 4-bit activations in xq (from
 * sva_mxfp4_quant_acts with the same descriptor) and W packed by
 * sva_mxfp4_pack_weights; layouts, limits and errors as for
 * sva_qkv_proj_mxfp4. */
sva_status sva_qkv_proj_w4a4(const sva_proj_desc* desc, const void* xq, const void* wpack, const float* bias,
                             void* q, void* k, void* v, void* stream);

/* Projection and attention without q, k or v in memory:
 *   out = sva_lin_attn_fwd(attn, q, k, v, ...) with (q, k, v) =
 *         sva_qkv_proj_mxfp4(proj, x, wpack, bias) rounded to bf16.
 * The k, v projection's epilogue applies phi and the numerator-only RoPE to
 * k (the [talk] 3D RoPE segment and the [news] positional-encoding
 * paragraph) and adds each 64-token tile's RoPE(phi k)^T v and phi k to the
 * block states ([talk] linear-attention and block KV cache segments); once
 * the block prefix is formed, q is projected a second pass over x inside
 * the output pass, per 64-token tile and head.  The SANA-Video article's
 * 4-bit quantization paragraph motivates fusing the projection into the
 * attention.
 *   attn: bf16, d = 64, H even; proj: the same B, H, d, N = T*Hs*Ws, and
 *   C a multiple of 256 (an even number of 128-channel stages);
 *   S0, z0, S_out, z_out, eps and RoPE as in sva_lin_attn_fwd.
 * SVA_ERR_UNSUPPORTED outside those limits or the projection's; the
 * workspace is sva_proj_lin_attn_fwd_workspace bytes.
 * The tokens are reduced in ranges of L tokens that divide the block
 * length, one workgroup per (range, head pair); L is chosen for occupancy
 * when proj->range_tokens is 0, else L = proj->range_tokens (a divisor of
 * the block length, else SVA_ERR_INVALID_ARG).  L fixes the order of the
 * fp32 sums, and the workspace size depends on it: query the workspace with
 * the same descriptor. */
sva_status sva_proj_lin_attn_fwd_workspace(const sva_desc* attn, const sva_proj_desc* proj, size_t* bytes);
sva_status sva_proj_lin_attn_fwd(const sva_desc* attn, const sva_proj_desc* proj, const void* x,
                                 const void* wpack, const float* bias, void* out, const float* S0,
                                 const float* z0, float* S_out, float* z_out, void* ws, size_t ws_bytes,
                                 void* stream);

/* The same pass on 4-bit activations (W4A4, as SVDQuant deploys it: [news],
 * 4-bit quantization paragraph):
 *   out = sva_lin_attn_fwd(attn, q, k, v, ...) with (q, k, v) =
 *         sva_qkv_proj_w4a4(proj, xq, wpack, bias) rounded to bf16,
 * xq being sva_mxfp4_quant_acts' output for the same proj descriptor
 * (sva_mxfp4_acts_bytes bytes; xq must not overlap out or the workspace).
 * q, k and v never reach memory, as above.  Limits, range length, workspace
 * (sva_proj_lin_attn_fwd_workspace with the same descriptors: the block
 * partials and prefix operands) and errors as for sva_proj_lin_attn_fwd. */
sva_status sva_proj_lin_attn_fwd_w4a4(const sva_desc* attn, const sva_proj_desc* proj, const void* xq,
                                      const void* wpack, const float* bias, void* out, const float* S0,
                                      const float* z0, float* S_out, float* z_out, void* ws, size_t ws_bytes,
                                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVA_PROJ_H */
