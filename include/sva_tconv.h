/*
 * sva_tconv.h -- C ABI of the causal temporal convolution that SANA-Video
 * puts in its Mix-FFN, with the one-token block cache that makes it
 * streamable, for AMD MI355X (gfx950).  Part of libsva.
 *
 * Pages this interface follows:
 *   [talk]  "SANA-Video: Efficient Video Generation with Block Linear
 *           Diffusion Transformer, [ICLR 2026, Oral]" talk transcript
 *           (shadowingenglish.com), segment on the causal FFN with a temporal
 *           convolution: one zero token between consecutive blocks keeps a
 *           block from seeing the next one; the previous block's last token
 *           is carried in front of the block so that it sees its past; the
 *           padding outputs are dropped.
 *   [study] the ICLR 2026 writing study of the paper: the attention state
 *           and the convolution history are both constant-size caches.
 *
 * What is computed (readings taken where the pages are silent: a depthwise
 * convolution along latent frames with three taps per channel, taps in
 * correlation order).  Activations x, y are [B, T, Hs, Ws, C] (tokens in
 * row-major (t, h, w) order, channels contiguous); a block is F whole
 * frames.  For frame t of block c = t / F, position (h, w), channel ch:
 *   prev = x[t-1]  (for the first frame of a block: the last frame of the
 *                   previous block; for block 0: the cache, or zero)
 *   next = x[t+1] if t+1 is in the same block, else 0 (the separator)
 *   y[t] = w[ch][0] * prev + w[ch][1] * x[t] + w[ch][2] * next + bias[ch]
 * The cache is one latent frame, [B, Hs, Ws, C] in the activation dtype:
 * its size does not depend on how many blocks came before.
 *
 * Numerics: fp32 arithmetic (fused multiply-adds, taps in a fixed order),
 * output rounded to the activation dtype (bf16: round to nearest even).
 *
 * Ownership and errors as in sva.h: every pointer is a caller-owned device
 * pointer, 16-byte aligned; the library allocates nothing and keeps nothing;
 * validation is synchronous and happens before any launch, and on error
 * nothing is written; work is queued on `stream` (a hipStream_t).  No
 * workspace is needed.
 */
#ifndef SVA_TCONV_H
#define SVA_TCONV_H

#include "sva.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sva_tconv_desc {
  int B;                 /* samples */
  int T, Hs, Ws;         /* latent frames and spatial grid */
  int C;                 /* channels: a multiple of 8 (bf16) or 4 (fp32) */
  int frames_per_block;  /* F >= 1, T % F == 0 */
  sva_dtype dtype;       /* SVA_BF16 or SVA_F32, for x, y and the cache */
} sva_tconv_desc;

/* One-shot block-causal form over all T / F blocks (the training form):
 *   x         in:  [B, T, Hs, Ws, C]
 *   w         in:  [C, 3] fp32 taps (previous, current, next frame)
 *   bias      in:  [C] fp32, or NULL (no bias)
 *   cache_in  in:  [B, Hs, Ws, C], the frame carried into block 0, or NULL
 *                  (zero)
 *   y         out: [B, T, Hs, Ws, C]; must not overlap x or either cache
 *   cache_out out: [B, Hs, Ws, C], the last frame of x (the cache after
 *                  committing every block), or NULL; may be cache_in itself
 *                  (each element is read before it is written) but must not
 *                  overlap it otherwise, nor x or y
 * SVA_ERR_UNSUPPORTED for another dtype or a C that is not a whole number of
 * 16-byte vectors; SVA_ERR_INVALID_ARG for a bad shape, pointer or overlap. */
sva_status sva_tconv_fwd(const sva_tconv_desc* desc, const void* x, const float* w,
                         const float* bias, const void* cache_in, void* y, void* cache_out,
                         void* stream);

/* Output of one block against the cache (desc->T == desc->frames_per_block):
 * the block's first frame sees the cached frame, its last frame sees the
 * separator.  The cache is read only, so a denoising loop may call this any
 * number of times.  Arguments as in sva_tconv_fwd; cache must not be NULL. */
sva_status sva_tconv_apply(const sva_tconv_desc* desc, const void* cache, const void* x,
                           const float* w, const float* bias, void* y, void* stream);

/* Commit one block (desc->T == desc->frames_per_block): cache <- its last
 * frame x[:, T-1].  cache [B, Hs, Ws, C] must not overlap x. */
sva_status sva_tconv_commit(const sva_tconv_desc* desc, void* cache, const void* x, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVA_TCONV_H */
