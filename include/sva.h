/*
 * sva.h -- C ABI of libsva: block-causal ReLU linear attention with a
 * numerator-only 3D RoPE and a constant-size block KV cache, as used by
 * SANA-Video, for AMD MI355X (gfx950).
 *
 * Pages this interface follows:
 *   [talk] "SANA-Video: Efficient Video Generation with Block Linear Diffusion
 *          Transformer, [ICLR 2026, Oral]" talk transcript (shadowingenglish.com):
 *          - linear-attention segment: the state is d x d whatever the length;
 *          - block KV cache segment: the state of a block is cached and each
 *            later block adds only its own KV contribution to the cache;
 *          - block causal segment: block 1 cannot see block 2, block 2 sees
 *            block 1; constant memory with global history;
 *          - opening: generate block by block causally, diffuse within a block;
 *          - 3D RoPE segment: RoPE over (t, h, w) for the linear attention.
 *   [news] cstia.com SANA-Video article, positional-encoding paragraph: RoPE is
 *          kept in the numerator and removed from the denominator.
 *
 * What is computed, per batch b and head h (tokens n in row-major (t, h, w)
 * order on a T x Hs x Ws latent grid, blocks of F whole frames):
 *   phi(x)   = max(x, 0)                     (reading taken: ReLU)
 *   qr, kr   = RoPE(phi q), RoPE(phi k)      (numerator copies only)
 *   A_c      = sum_{n in block c} kr_n v_n^T      (d x d)
 *   zeta_c   = sum_{n in block c} phi(k)_n        (d)
 *   S_c      = S0 + sum_{c' <= c} A_c',  Z_c = z0 + sum_{c' <= c} zeta_c'
 *   out_n    = (qr_n^T S_c) / (phi(q)_n . Z_c + eps),  c = block of n.
 * RoPE: head dims [0, dt) follow the global latent frame t = t0 + local frame,
 * [dt, dt+dh) follow h, [dt+dh, d) follow w.  In an axis slice of width d_a
 * the adjacent pair (2i, 2i+1) turns by pos * rope_base^(-2i/d_a) radians:
 * (x, y) -> (x cos - y sin, x sin + y cos).
 *
 * Layouts: q, k, v, out are contiguous [B, H, N, d], N = T*Hs*Ws, in the
 * descriptor's dtype (fp32 or bf16).  S is fp32 [B, H, d, d] row-major with
 * S[i][j] = sum kr_i v_j; z is fp32 [B, H, d].  Every pointer is a device
 * pointer and must be 16-byte aligned.
 *
 * Ownership: the caller allocates and frees every buffer, including the
 * workspace.  The library allocates nothing and keeps no pointer after a
 * call returns.  Its only process-wide state is a per-device memo of the
 * occupancy and compute-unit queries that size its grids (filled on first
 * use, under a mutex, and never changed after), so calls on disjoint buffers may run
 * concurrently from several threads.  `out` must not overlap q, k or v.
 *
 * Errors: validation is synchronous, happens before anything is launched,
 * and on error nothing is written.  Work is queued on `stream` (a
 * hipStream_t; NULL = the default stream) and runs asynchronously; a kernel
 * fault surfaces at the caller's next synchronisation.  A failed launch
 * returns SVA_ERR_HIP.  NaN/Inf inputs are not checked.  phi is a max with
 * zero on the bit pattern: every value with the sign bit set (negative
 * numbers, -0, -Inf and a NaN with its sign bit set) becomes +0, every
 * other value (+Inf and a NaN with its sign bit clear included) passes
 * unchanged and propagates into the sums.
 * Sums are taken in a fixed order: two calls on equal inputs give equal bits.
 */
#ifndef SVA_H
#define SVA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sva_dtype { SVA_F32 = 0, SVA_BF16 = 1 } sva_dtype;

typedef enum sva_status {
  SVA_OK = 0,
  SVA_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad shape, overlap */
  SVA_ERR_UNSUPPORTED = -2,  /* d not 32/64, bad RoPE split, grid too large
                                (with RoPE: F, Hs, Ws <= 1024 and at most 3584
                                cos/sin table entries, F*dt/2 + Hs*dh/2 +
                                Ws*dw/2) */
  SVA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
  SVA_ERR_HIP = -4           /* a HIP launch failed */
} sva_status;

/* Problem descriptor.  All fields are read; none is kept after the call. */
typedef struct sva_desc {
  int B, H, d;               /* batch, heads, head dim (32 or 64) */
  int T, Hs, Ws;             /* latent grid of this call: frames x height x width */
  int frames_per_block;      /* F; T % F == 0.  apply/commit need T == F */
  int t0;                    /* global latent frame index of this call's frame 0 */
  int rope;                  /* 0: no RoPE, 1: 3D RoPE on the numerator */
  int rope_dt, rope_dh, rope_dw; /* even widths with dt + dh + dw == d */
  float rope_base;           /* frequency base, > 0 (10000 is customary) */
  float eps;                 /* added to the denominator, >= 0 */
  int dtype;                 /* sva_dtype of q, k, v and out */
} sva_desc;

/* Human-readable text for a status code (static storage). */
const char* sva_status_string(int status);

/* ABI version of this header: 1. */
int sva_version(void);

/* Workspace bytes sva_lin_attn_fwd needs for this descriptor (arrival
 * counters, per-block partial states and the prefix states; about
 * nb*B*H*d*d*8 bytes).
 * Every workspace (this one, the backward's and the block cache's) must be
 * zero-filled once before its first use: it starts with B*H arrival
 * counters that the reduction's workgroups count on, and every call leaves
 * them zero again, so a workspace that is reused needs no further clearing.
 * Calls that share a workspace must not run concurrently. */
sva_status sva_lin_attn_fwd_workspace(const sva_desc* desc, size_t* bytes);

/* One-shot block-causal forward over all T/F blocks ([talk], block causal
 * segment: the whole sequence in one pass, as in block-causal training).
 *   q, k, v  in:  [B, H, N, d] dtype
 *   out      out: [B, H, N, d] dtype (round-to-nearest-even for bf16)
 *   S0, z0   in:  initial cache [B,H,d,d], [B,H,d] fp32, or both NULL (zeros)
 *   S_out, z_out out: final cache (S_{nb-1}, Z_{nb-1}) fp32, or both NULL;
 *            may be the same buffers as S0, z0 (updated in place)
 *   ws, ws_bytes: caller-owned scratch of at least sva_lin_attn_fwd_workspace
 * With one block (T == frames_per_block, t0 = its first frame) and the cache
 * as both S0/z0 and S_out/z_out, one call gives the block's output and
 * commits the block: sva_block_cache_apply then sva_block_cache_commit in a
 * single pass over q, k, v (a block's last denoising step).
 */
sva_status sva_lin_attn_fwd(const sva_desc* desc, const void* q, const void* k,
                            const void* v, void* out, const float* S0,
                            const float* z0, float* S_out, float* z_out,
                            void* ws, size_t ws_bytes, void* stream);

/* Kernels of sva_lin_attn_fwd, selectable for profiling one at a time. */
typedef enum sva_stage {
  SVA_STAGE_REDUCE = 1, /* per-block state reduction (with the prefix, where it is folded in) */
  SVA_STAGE_SCAN = 2,   /* separate prefix scan (a no-op where the reduction forms the prefix) */
  SVA_STAGE_APPLY = 4,  /* output pass */
  SVA_STAGE_ALL = 7
} sva_stage;

/* sva_lin_attn_fwd restricted to the kernels in `stages` (a mask of
 * sva_stage), launched back to back on `stream`, so that a caller can time
 * each kernel alone.  A stage reads what the earlier stages of a complete
 * call left in the workspace: the output pass alone repeats the output of
 * the last full call made with this workspace, descriptor and inputs.
 * SVA_STAGE_ALL is sva_lin_attn_fwd.  stages outside 1..7:
 * SVA_ERR_INVALID_ARG. */
sva_status sva_lin_attn_fwd_stages(const sva_desc* desc, const void* q, const void* k,
                                   const void* v, void* out, const float* S0,
                                   const float* z0, float* S_out, float* z_out,
                                   void* ws, size_t ws_bytes, void* stream,
                                   int stages);
/* Workspace bytes sva_lin_attn_bwd needs (the same as the forward's).
 * SVA_ERR_UNSUPPORTED unless desc->dtype == SVA_BF16. */
sva_status sva_lin_attn_bwd_workspace(const sva_desc* desc, size_t* bytes);

/* Gradients of sva_lin_attn_fwd, for the block-causal training the pages
 * run ([talk], block causal segment), by the chain rule through the same
 * steps.  For L = <out, dout> + <S_final, dS_out> + <z_final, dz_out>:
 *   q, k, v   in:  the forward's inputs [B, H, N, d] bf16
 *   dout      in:  dL/dout [B, H, N, d] bf16
 * The forward's output is not an input: the denominator's term needs
 * dout . out, and out is formed again from q and the prefix states (bf16
 * operands, fp32 sums, not rounded to bf16).
 *   S0, z0    in:  the forward's initial cache fp32, or both NULL (zeros)
 *   dS_out, dz_out in: dL/d(final cache) [B,H,d,d], [B,H,d] fp32, or both
 *                  NULL (zero)
 *   dq, dk, dv out: [B, H, N, d] bf16 (round-to-nearest-even); none of
 *                  them may overlap another or any input
 *   states    in:  the prefix states the forward saved
 *                  (sva_lin_attn_fwd_save with the same descriptor, inputs
 *                  and initial cache), or NULL to recompute them (one more
 *                  pass over k and v)
 *   dS0, dz0  out: dL/d(initial cache) fp32, or both NULL
 *   ws, ws_bytes: caller-owned scratch of at least
 *                  sva_lin_attn_bwd_workspace bytes
 * The derivative of ReLU is taken as 0 at 0.  bf16 only: other dtypes return
 * SVA_ERR_UNSUPPORTED before any work. */
sva_status sva_lin_attn_bwd(const sva_desc* desc, const void* q, const void* k,
                            const void* v, const void* dout,
                            const float* S0, const float* z0,
                            const float* dS_out, const float* dz_out,
                            const void* states, void* dq, void* dk, void* dv,
                            float* dS0, float* dz0, void* ws, size_t ws_bytes,
                            void* stream);

/* Bytes of the prefix states one forward call can keep for the backward:
 * every block's S_c (in the input dtype; for bf16 also its remainder S_c -
 * bf16(S_c) in bf16, which the backward adds back) and Z_c (fp32):
 * B*H*nb*(d*d*esize*(bf16 ? 2 : 1) + d*4) plus alignment; about 1.9 MB for
 * 16 heads of d = 64 in 7 blocks. */
sva_status sva_lin_attn_states_bytes(const sva_desc* desc, size_t* bytes);

/* sva_lin_attn_fwd that also keeps its prefix states in `states`
 * (caller-owned, sva_lin_attn_states_bytes long, 16-byte aligned) for
 * sva_lin_attn_bwd.  The states are written instead of a workspace copy
 * (plus, for bf16, the remainders: d*d*2 bytes per block and head), and the
 * prefix always runs in the scan kernel, which forms the remainders. */
sva_status sva_lin_attn_fwd_save(const sva_desc* desc, const void* q,
                                 const void* k, const void* v, void* out,
                                 const float* S0, const float* z0,
                                 float* S_out, float* z_out, void* states,
                                 void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes sva_block_cache_apply / sva_block_cache_commit need for a
 * one-block descriptor; independent of how many blocks were committed. */
sva_status sva_block_cache_workspace(const sva_desc* desc, size_t* bytes);

/* Output of ONE block (desc->T == desc->frames_per_block, first frame at
 * global index desc->t0) against a committed cache (S, z): the block sees
 * the cache and itself ([talk] opening: diffuse within the current block;
 * block KV cache segment: cached state plus the current block's KV).
 * The cache is read only and left unchanged, so this may be called for
 * every denoising step of the block.
 *   S, z     in:  cache [B,H,d,d], [B,H,d] fp32
 *   q, k, v  in:  [B, H, F*Hs*Ws, d];  out: same shape and dtype */
sva_status sva_block_cache_apply(const sva_desc* desc, const float* S,
                                 const float* z, const void* q, const void* k,
                                 const void* v, void* out, void* ws,
                                 size_t ws_bytes, void* stream);

/* sva_block_cache_apply without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: its scratch is a
 * static array of 16 MiB in the library's device code, one copy per GPU,
 * held until the process ends.  The result equals sva_block_cache_apply's.
 * The scratch a call needs is (R + B*H) * (d*d + d) * 4 bytes for the
 * reduction's per-workgroup pieces (R: the device's resident reduction
 * workgroups, 256 on MI355X) plus B*H*d*d*esize + B*H*d*4 for the prefix
 * operands, with 256-byte alignment: up to about 480 heads x samples of
 * d = 64 in bf16; beyond the array's size it returns SVA_ERR_WORKSPACE
 * before any launch.  Every call on one GPU shares that GPU's copy: calls
 * that overlap on one GPU (other streams or threads) race and must be
 * serialised by the caller. */
sva_status sva_block_cache_apply_noalloc(const sva_desc* desc, const float* S,
                                         const float* z, const void* q,
                                         const void* k, const void* v,
                                         void* out, void* stream);

/* Adds ONE block to the cache in place ([talk], block KV cache segment: the
 * state is updated additively): S += sum RoPE(phi k) v^T, z += sum phi k over
 * the block's tokens at global frames t0 .. t0+F-1.  The caller chooses which
 * step's k, v to commit and zero-fills a fresh cache.  The cache size,
 * B*H*(d*d+d)*4 bytes, does not depend on the number of committed blocks. */
sva_status sva_block_cache_commit(const sva_desc* desc, float* S, float* z,
                                  const void* k, const void* v, void* ws,
                                  size_t ws_bytes, void* stream);

/* The phi + 3D-RoPE stage on its own, for testing it in isolation:
 *   x      in:  [B, H, N, d] dtype
 *   x_rot  out: [B, H, N, d] fp32 = RoPE(phi x)   (phi x when desc->rope == 0)
 *   x_phi  out: [B, H, N, d] fp32 = phi x  (may be NULL)
 * The fused kernels run exactly this stage in registers. */
sva_status sva_phi_rope_prep(const sva_desc* desc, const void* x, float* x_rot,
                             float* x_phi, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVA_H */
