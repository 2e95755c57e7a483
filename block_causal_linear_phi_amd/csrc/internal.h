// Internal interfaces between the library's source files (not part of the
// C ABI): division by run-time constants, and the projection file's
// launchers that the fused projection + attention entry point in sva.hip
// drives.
#ifndef SVA_INTERNAL_H
#define SVA_INTERNAL_H

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "sva.h"
#include "sva_proj.h"

// n / d for 0 <= n < 2^31 as (umulhi(n, mul) + n) >> shift, constants from
// the round-up method (Granlund & Montgomery, "Division by invariant
// integers using multiplication", 1994).
struct FastDiv {
  uint32_t mul, shift, div;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  f.mul = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  f.div = d;
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.mul) + n) >> f.shift;
}

// Geometry of the fused k, v projection + per-block state reduction (head
// dimension 64; H even; L divides Nb, Nb divides N).
struct SvaKvReduceArgs {
  int B, N, C, H;      // samples, tokens per sample, input channels, heads
  int Nb, nb, L;       // tokens per block, blocks, tokens per range
  int Hs, Ws, t0;      // latent rows, columns, first frame
  int rope, dt, dh;    // RoPE on; t and h axis widths
  float rope_base;
};

// Partials of every (range, block) piece at slot g + bhc (g: the range's
// index along the flattened (b, h, token) axis in units of L; bhc: the
// block's flattened index), each S^T (64 x 64) then z (64), fp32.
hipError_t sva_internal_kv_proj_reduce(const SvaKvReduceArgs& a, const void* x, const void* wpack,
                                       const float* bias, float* partials, hipStream_t stream);

// The same from the 4-bit activations xq (sva_mxfp4_quant_acts' layout).
hipError_t sva_internal_kv_proj_reduce_w4a4(const SvaKvReduceArgs& a, const void* xq, const void* wpack,
                                            const float* bias, float* partials, hipStream_t stream);

// sva_qkv_proj_mxfp4 restricted to output features [0, f_end) (q alone:
// f_end = H * d); validation as for the full projection.
sva_status sva_internal_proj_features(const sva_proj_desc* desc, const void* x, const void* wpack,
                                      const float* bias, int f_end, void* q, void* k, void* v, void* stream);

// q projected from the activations (w4a4: the 4-bit xq; else x [B, N, C]
// bf16) and applied in the same pass: out [B, H, N, 64] bf16 =
// (RoPE(phi q) S_c) / (phi q . Z_c + eps) with the block prefix operands the
// scan writes (frags: S_c^T [B H nb][64][64] bf16; zc: Z_c [B H nb][64]
// fp32).  a.L is not used.
hipError_t sva_internal_q_proj_apply(const SvaKvReduceArgs& a, float eps, bool w4a4, const void* x,
                                    const void* wpack, const float* bias, const void* frags, const float* zc,
                                    void* out, hipStream_t stream);

// Workgroups of kernel fn the current device holds at once (CUs times
// workgroups per CU), memoised per (device, kernel, dynamic LDS).
int sva_internal_resident_workgroups(const void* fn, int threads, size_t lds);

// sva_qkv_proj_w4a4 restricted to output features [0, f_end).
sva_status sva_internal_proj_w4a4_features(const sva_proj_desc* desc, const void* xq, const void* wpack,
                                           const float* bias, int f_end, void* q, void* k, void* v, void* stream);

#endif  // SVA_INTERNAL_H
