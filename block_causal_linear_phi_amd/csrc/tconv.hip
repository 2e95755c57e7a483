// Causal temporal convolution with a one-token block cache, for gfx950.
//
// Pages followed: "SANA-Video: Efficient Video Generation with Block Linear
// Diffusion Transformer, [ICLR 2026, Oral]" talk transcript, segment on the
// causal FFN with a temporal convolution (a zero token closes each block,
// the previous block's last token opens the next one); the ICLR 2026 writing
// study of the paper (constant-size convolution cache).  The readings taken
// where they are silent (depthwise, three taps, correlation order) are
// stated in include/sva_tconv.h.
//
// The op is a three-point stencil along t with no reuse across positions or
// channels: every input element is read once and every output written once,
// so it is bound by HBM bandwidth.  One thread owns one 16-byte vector of
// channels (8 bf16 or 4 fp32) at one (b, h, w) and walks the T frames with a
// sliding window in registers, so each frame is read exactly once.  A
// wavefront covers 64 consecutive vectors of a token row: every load and
// store is a contiguous 1 KiB.  Loads run one frame group ahead of the stores.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sva.h"
#include "sva_tconv.h"

namespace {

constexpr int kTconvThreads = 256;
constexpr int kChunk = 1;  // frames per load group; one group ahead of the stores

struct TconvGeo {
  long long vecs;     // B * Hs * Ws * CV: one thread each
  long long fstride;  // vectors between consecutive frames: Hs * Ws * CV
  int T, F, HW, CV;   // CV = vectors per token row
};

typedef __bf16 tc_bf16x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
struct Vec {
  static constexpr int N = BF16 ? 8 : 4;  // elements in 16 bytes
};

template <bool BF16>
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[Vec<BF16>::N]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
}

template <bool BF16>
__device__ __forceinline__ uint4 pack(const float (&f)[Vec<BF16>::N]) {
  uint32_t w[4];
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const tc_bf16x2 p = {(__bf16)f[2 * i], (__bf16)f[2 * i + 1]};  // round to nearest even
      w[i] = __builtin_bit_cast(uint32_t, p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(f[i]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// y[t] for one vector: taps in a fixed order (next, current, previous) on
// top of the bias, each a fused multiply-add in fp32.
template <bool BF16>
__device__ __forceinline__ uint4 stencil(const uint4& prev, const uint4& cur, const uint4& next,
                                         const float (&w0)[Vec<BF16>::N], const float (&w1)[Vec<BF16>::N],
                                         const float (&w2)[Vec<BF16>::N], const float (&bb)[Vec<BF16>::N]) {
  constexpr int N = Vec<BF16>::N;
  float a[N], c[N], n[N], o[N];
  unpack<BF16>(prev, a);
  unpack<BF16>(cur, c);
  unpack<BF16>(next, n);
#pragma unroll
  for (int j = 0; j < N; ++j) o[j] = __builtin_fmaf(w0[j], a[j], __builtin_fmaf(w1[j], c[j], __builtin_fmaf(w2[j], n[j], bb[j])));
  return pack<BF16>(o);
}

typedef uint32_t tc_u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal hint: each input is read once.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const tc_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const tc_u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// One thread per 16-byte channel vector at one (b, h, w); frames t = 0..T-1
// in order.  `prev` carries across block boundaries (the carried token); the
// next frame is replaced by zero at a block's last frame (the separator).
template <bool BF16>
__global__ __launch_bounds__(kTconvThreads) void sva_tconv_kernel(
    const uint4* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const uint4* cache_in, uint4* __restrict__ y, uint4* cache_out, TconvGeo g) {
  constexpr int N = Vec<BF16>::N;
  const long long i = (long long)blockIdx.x * kTconvThreads + threadIdx.x;
  if (i >= g.vecs) return;
  const long long bp = i / g.CV;  // b * HW + p
  const int cv = (int)(i - bp * g.CV);
  const long long b = bp / g.HW;
  const long long p = bp - b * g.HW;

  // taps of channels N*cv .. N*cv + N-1: 3N consecutive floats (16-byte aligned)
  float w0[N], w1[N], w2[N], bb[N];
  {
    const float4* wv = reinterpret_cast<const float4*>(w + (long long)cv * 3 * N);
    float t[3 * N];
#pragma unroll
    for (int k = 0; k < 3 * N / 4; ++k) {
      const float4 q = wv[k];
      t[4 * k] = q.x; t[4 * k + 1] = q.y; t[4 * k + 2] = q.z; t[4 * k + 3] = q.w;
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
      w0[j] = t[3 * j];
      w1[j] = t[3 * j + 1];
      w2[j] = t[3 * j + 2];
    }
    if (bias) {
      const float4* bv = reinterpret_cast<const float4*>(bias + (long long)cv * N);
#pragma unroll
      for (int k = 0; k < N / 4; ++k) {
        const float4 q = bv[k];
        bb[4 * k] = q.x; bb[4 * k + 1] = q.y; bb[4 * k + 2] = q.z; bb[4 * k + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < N; ++j) bb[j] = 0.f;
    }
  }

  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const long long col = (b * g.T * g.HW + p) * g.CV + cv;  // frame 0 of this thread's column
  const uint4* xs = x + col;
  uint4* ys = y + col;
  const long long cidx = bp * g.CV + cv;
  // (A conditional expression over the two lvalues made the compiler select
  // between their addresses and keep `zero` in scratch memory.)
  uint4 prev = make_uint4(0u, 0u, 0u, 0u);
  if (cache_in) prev = cache_in[cidx];
  uint4 cur = load_nt(xs);
  int in_block = 0;  // frame index inside its block
  // Output t from (prev, cur, next) = frames t-1, t, t+1; next is zero at a
  // block's last frame (the separator).
  auto emit = [&](int t, const uint4& next) {
    const bool last_of_block = in_block == g.F - 1;
    ys[(long long)t * g.fstride] = stencil<BF16>(prev, cur, last_of_block ? zero : next, w0, w1, w2, bb);
    in_block = last_of_block ? 0 : in_block + 1;
    prev = cur;
    cur = next;
  };
  // Frames are loaded kChunk at a time into two register sets in turn, one
  // group ahead of the outputs that use them (groups of 1, 2 and 4 frames
  // measured 57.6, 60.6 and 59.7 us at the 720p grid; the previous design,
  // 4 frames loaded then all waited for, 60.2 us).  Loads are unconditional, the
  // frame index clamped to T-1 (a clamped frame is only ever the "next" of
  // frame T-1, the last of its block, and is replaced by zero), and the
  // steady-state loop stores unconditionally: a conditional load or store
  // leaves the compiler unsure how many are in flight, and it then waits for
  // all of them before the next use.
  auto load_chunk = [&](uint4 (&r)[kChunk], int f0) {
#pragma unroll
    for (int j = 0; j < kChunk; ++j) r[j] = load_nt(xs + (long long)min(f0 + j, g.T - 1) * g.fstride);
  };
  uint4 ra[kChunk], rb[kChunk];
  load_chunk(ra, 1);
  int t0 = 0;
  // (The scheduling barriers keep each load group ahead of the outputs that
  // precede its use; the compiler otherwise sinks it next to that use.)
  for (; t0 + 2 * kChunk <= g.T; t0 += 2 * kChunk) {
    load_chunk(rb, t0 + kChunk + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) emit(t0 + j, ra[j]);
    __builtin_amdgcn_sched_barrier(0);
    load_chunk(ra, t0 + 2 * kChunk + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) emit(t0 + kChunk + j, rb[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Fewer than 2 kChunk frames left; ra holds frames t0+1 .. t0+kChunk.
  if (t0 < g.T) {
    load_chunk(rb, t0 + kChunk + 1);
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      if (t0 + j < g.T) emit(t0 + j, ra[j]);
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      if (t0 + kChunk + j < g.T) emit(t0 + kChunk + j, rb[j]);
  }
  if (cache_out) cache_out[cidx] = prev;  // x[T-1], bit for bit
}

// cache <- x[:, T-1]: one thread per 16-byte vector.
__global__ __launch_bounds__(kTconvThreads) void sva_tconv_commit_kernel(const uint4* __restrict__ x,
                                                                        uint4* __restrict__ cache, TconvGeo g) {
  const long long i = (long long)blockIdx.x * kTconvThreads + threadIdx.x;
  if (i >= g.vecs) return;
  const long long bp = i / g.CV;
  const int cv = (int)(i - bp * g.CV);
  const long long b = bp / g.HW;
  const long long p = bp - b * g.HW;
  cache[i] = load_nt(x + ((b * g.T + g.T - 1) * g.HW + p) * g.CV + cv);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bn && y < x + an;
}

struct TconvPlan {
  TconvGeo g;
  bool bf16;
  size_t act_bytes, cache_bytes, w_bytes, b_bytes;
  unsigned blocks;
};

sva_status plan_tconv(const sva_tconv_desc* d, bool one_block, TconvPlan* p) {
  if (!d) return SVA_ERR_INVALID_ARG;
  if (d->dtype != SVA_BF16 && d->dtype != SVA_F32) return SVA_ERR_UNSUPPORTED;
  if (d->B < 1 || d->T < 1 || d->Hs < 1 || d->Ws < 1 || d->C < 1 || d->frames_per_block < 1)
    return SVA_ERR_INVALID_ARG;
  if (d->T % d->frames_per_block != 0) return SVA_ERR_INVALID_ARG;
  if (one_block && d->T != d->frames_per_block) return SVA_ERR_INVALID_ARG;
  const bool bf16 = d->dtype == SVA_BF16;
  const int vec = bf16 ? 8 : 4;
  if (d->C % vec != 0) return SVA_ERR_UNSUPPORTED;
  const long long hw = (long long)d->Hs * d->Ws;
  const long long cv = d->C / vec;
  const long long vecs = (long long)d->B * hw * cv;
  const long long fstride = hw * cv;
  const long long blocks = (vecs + kTconvThreads - 1) / kTconvThreads;
  if (hw > (1LL << 30) || fstride * d->T > (1LL << 40) / d->B || blocks >= (1LL << 31))
    return SVA_ERR_UNSUPPORTED;
  const size_t esz = bf16 ? 2 : 4;
  p->g.vecs = vecs;
  p->g.fstride = fstride;
  p->g.T = d->T;
  p->g.F = d->frames_per_block;
  p->g.HW = (int)hw;
  p->g.CV = (int)cv;
  p->bf16 = bf16;
  p->cache_bytes = (size_t)d->B * hw * d->C * esz;
  p->act_bytes = p->cache_bytes * d->T;
  p->w_bytes = (size_t)d->C * 3 * sizeof(float);
  p->b_bytes = (size_t)d->C * sizeof(float);
  p->blocks = (unsigned)blocks;
  return SVA_OK;
}

sva_status run_tconv(const sva_tconv_desc* desc, bool one_block, const void* x, const float* w,
                     const float* bias, const void* cache_in, void* y, void* cache_out, void* stream) {
  TconvPlan p;
  sva_status s = plan_tconv(desc, one_block, &p);
  if (s != SVA_OK) return s;
  if (!x || !w || !y) return SVA_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w, bias, cache_in, y, cache_out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return SVA_ERR_INVALID_ARG;
  if (overlap(y, p.act_bytes, x, p.act_bytes)) return SVA_ERR_INVALID_ARG;
  if (cache_in && (overlap(cache_in, p.cache_bytes, x, p.act_bytes) || overlap(cache_in, p.cache_bytes, y, p.act_bytes)))
    return SVA_ERR_INVALID_ARG;
  if (cache_out) {
    if (overlap(cache_out, p.cache_bytes, x, p.act_bytes) || overlap(cache_out, p.cache_bytes, y, p.act_bytes))
      return SVA_ERR_INVALID_ARG;
    if (cache_in && cache_in != cache_out && overlap(cache_out, p.cache_bytes, cache_in, p.cache_bytes))
      return SVA_ERR_INVALID_ARG;
  }
  if (overlap(y, p.act_bytes, w, p.w_bytes) || (bias && overlap(y, p.act_bytes, bias, p.b_bytes)))
    return SVA_ERR_INVALID_ARG;
  const uint4* xa = (const uint4*)x;
  const uint4* ci = (const uint4*)cache_in;
  uint4* ya = (uint4*)y;
  uint4* co = (uint4*)cache_out;
  TconvGeo g = p.g;
  void* args[] = {(void*)&xa, (void*)&w, (void*)&bias, (void*)&ci, (void*)&ya, (void*)&co, &g};
  const void* fn = p.bf16 ? (const void*)&sva_tconv_kernel<true> : (const void*)&sva_tconv_kernel<false>;
  if (hipLaunchKernel(fn, dim3(p.blocks), dim3(kTconvThreads), args, 0, (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

}  // namespace

extern "C" {

sva_status sva_tconv_fwd(const sva_tconv_desc* desc, const void* x, const float* w, const float* bias,
                         const void* cache_in, void* y, void* cache_out, void* stream) {
  return run_tconv(desc, false, x, w, bias, cache_in, y, cache_out, stream);
}

sva_status sva_tconv_apply(const sva_tconv_desc* desc, const void* cache, const void* x, const float* w,
                           const float* bias, void* y, void* stream) {
  if (!cache) return SVA_ERR_INVALID_ARG;
  return run_tconv(desc, true, x, w, bias, cache, y, nullptr, stream);
}

sva_status sva_tconv_commit(const sva_tconv_desc* desc, void* cache, const void* x, void* stream) {
  TconvPlan p;
  sva_status s = plan_tconv(desc, true, &p);
  if (s != SVA_OK) return s;
  if (!cache || !x || !aligned16(cache) || !aligned16(x)) return SVA_ERR_INVALID_ARG;
  if (overlap(cache, p.cache_bytes, x, p.act_bytes)) return SVA_ERR_INVALID_ARG;
  const uint4* xa = (const uint4*)x;
  uint4* ca = (uint4*)cache;
  TconvGeo g = p.g;
  void* args[] = {(void*)&xa, (void*)&ca, &g};
  if (hipLaunchKernel((const void*)&sva_tconv_commit_kernel, dim3(p.blocks), dim3(kTconvThreads), args, 0,
                      (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

}  // extern "C"
