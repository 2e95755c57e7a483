// libsva: block-causal ReLU linear attention with numerator-only 3D RoPE and a
// constant-size block KV cache (SANA-Video), hand-written for gfx950 (MI355X).
//
// Pages followed (see include/sva.h for the full statement of the operation):
//   [talk] SANA-Video ICLR 2026 Oral talk transcript (shadowingenglish.com):
//          linear-attention state of fixed d x d shape; block KV cache with
//          additive per-block update; block-causal visibility; 3D RoPE.
//   [news] cstia.com SANA-Video article, positional-encoding paragraph: RoPE
//          in the numerator only, RoPE-free denominator.
//
// Three kernels run per call, all on the caller's stream:
//   1. reduce : per-block state A_c = sum RoPE(phi k) v^T on bf16 MFMA
//               (fp32 MFMA for fp32 inputs) with fp32 accumulation, and
//               zeta_c = sum phi k; phi and RoPE are applied in registers
//               right after the load.  Work is split into equal flattened
//               token ranges, one per workgroup, so every CU streams the
//               same number of bytes; a range that crosses a block boundary
//               emits one partial per block it touches.
//   2. scan   : fixed-order sum of the partials into the inclusive prefix
//               S_c, Z_c (+ initial cache), written once in the exact
//               register layout the output kernel's MFMA A operand wants.
//   3. apply  : out = RoPE(phi q) S_c / (phi q . Z_c + eps); numerator on
//               MFMA (computed transposed so each lane ends up holding a
//               contiguous run of output features), denominator as an fp32
//               dot reduced across the four lane groups, divide and store in
//               one pass.
// Inputs are read exactly once (K, V by reduce, Q by apply) and the output
// written once; the partials and prefix states are <2% of the traffic at
// video sizes.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <map>
#include <type_traits>
#include <mutex>
#include <tuple>

#include "internal.h"
#include "split.h"
#include "sva.h"
#include "sva_proj.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;          // 4 wavefronts of 64 (scan, prep)

// Workgroup sizes of the reduction and output kernels, and how many of their
// workgroups a CU should hold (bf16: 2 waves per SIMD for the reduction, 3
// for the output pass; fp32 needs more registers and runs 1).
template <bool BF16> constexpr int red_threads() { return BF16 ? 512 : 256; }
template <bool BF16> constexpr int app_threads() { return 256; }
template <bool BF16> constexpr int red_min_blocks() { return BF16 ? (512 / red_threads<BF16>() > 0 ? 512 / red_threads<BF16>() : 1) : 1; }
template <bool BF16> constexpr int app_min_blocks() { return BF16 ? (768 / app_threads<BF16>() > 0 ? 768 / app_threads<BF16>() : 1) : 1; }
constexpr int kMaxTableEntries = 3584; // RoPE cos/sin table, 28 KiB of LDS (beside the reduction's 130 KiB)

// ---------------------------------------------------------------------------
// Small integer helpers
// ---------------------------------------------------------------------------

// FastDiv (n / d by multiply and shift) is in internal.h.

// RoPE layout for one call.  The cos/sin table lives in LDS as float2
// entries: [F rows x dt/2] for t (the frames of the block being processed,
// rebuilt per block), then [Hs rows x dh/2] for h, then [Ws rows x dw/2] for
// w.  When every width is a multiple of 4 ("paired"), the two RoPE pairs a
// lane reads next to each other sit in one 16-byte-aligned float4.
struct RopeArgs {
  int dt, dh, dw;
  int off_h, off_w, n_entries;
  int t0;               // global frame of the call's first frame
  int F;                // frames per block (rows of the t part)
  FastDiv fht, fhh, fhw;  // division by dt/2, dh/2, dw/2 (1 for an empty axis)
  double inv_rev[32];   // base^(-2i/d_a) / (2 pi), indexed by global pair p
};

// The frequencies reach the table build through registers: lane l of every
// wave holds that of global pair l % 32, picked from the kernel arguments
// with uniform (scalar) reads at kernel start, and the build takes a pair's
// value from its lane with ds_bpermute.  An indexed read of the
// kernel-argument array inside the build would be a vector memory round trip
// per entry, and since vector loads complete in issue order, each would also
// wait for every streaming load in flight.
__device__ __forceinline__ double load_lane_freq(const RopeArgs& ra) {
  const int p = threadIdx.x & 31;
  double f = ra.inv_rev[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) f = p == i ? ra.inv_rev[i] : f;
  return f;
}

__device__ __forceinline__ double freq_of(double lane_freq, int p) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, lane_freq);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(p << 2, (int)(uint32_t)bits);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(p << 2, (int)(uint32_t)(bits >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// One table entry.  PRECISE (fp32 inputs): fp64 angle reduced to one turn,
// then an accurate single-precision sincos.  Otherwise (bf16 inputs): the
// same reduced angle through the hardware sine/cosine, far below bf16's
// rounding.
template <bool PRECISE>
__device__ __forceinline__ float2 rope_entry(int pos, double inv_rev) {
  double rv = (double)pos * inv_rev;
  rv -= rint(rv);  // angle in turns, within [-1/2, 1/2]
  float c, s;
  if (PRECISE) {
    sincosf((float)(rv * 6.283185307179586), &s, &c);
  } else {
    s = __builtin_amdgcn_sinf((float)rv);  // sin(2 pi x)
    c = __builtin_amdgcn_cosf((float)rv);
  }
  return make_float2(c, s);
}

// The table entries [e_begin, e_end) of NT threads: entry e goes to thread
// e % NT.  The loop runs over whole wavefronts (every lane takes part in the
// cross-lane reads); at(e) gives (position, global pair) of entry e.
template <bool PRECISE, int NT, typename At>
__device__ __forceinline__ void build_rope_range(float2* tab, int e_begin, int e_end, double lane_freq, At at) {
  const int lane = threadIdx.x & 63;
  const int wave_base = (int)(threadIdx.x & ~63u);
  for (int e0 = e_begin + wave_base; e0 < e_end; e0 += NT) {
    const int e = e0 + lane;
    const int2 pp = at(min(e, e_end - 1));
    const double inv = freq_of(lane_freq, pp.y);
    if (e < e_end) tab[e] = rope_entry<PRECISE>(pp.x, inv);
  }
}

// h and w parts of the table (the same for every block).
template <bool PRECISE, int NT>
__device__ void build_rope_hw(float2* tab, const RopeArgs& ra, double lane_freq) {
  const int ht = ra.dt >> 1, hh = ra.dh >> 1;
  build_rope_range<PRECISE, NT>(tab, ra.off_h, ra.n_entries, lane_freq, [&](int e) {
    if (e < ra.off_w) {
      const uint32_t x = (uint32_t)(e - ra.off_h);
      const uint32_t pos = fdiv(x, ra.fhh);
      return make_int2((int)pos, ht + (int)(x - pos * ra.fhh.div));
    }
    const uint32_t x = (uint32_t)(e - ra.off_w);
    const uint32_t pos = fdiv(x, ra.fhw);
    return make_int2((int)pos, ht + hh + (int)(x - pos * ra.fhw.div));
  });
}

// t part of the table for block c: rows are global frames t0 + c*F + row.
template <bool PRECISE, int NT>
__device__ void build_rope_t(float2* tab, const RopeArgs& ra, int c, double lane_freq) {
  const int tbase = ra.t0 + c * ra.F;
  build_rope_range<PRECISE, NT>(tab, 0, ra.off_h, lane_freq, [&](int e) {
    const uint32_t row = fdiv((uint32_t)e, ra.fht);
    return make_int2(tbase + (int)row, e - (int)(row * ra.fht.div));
  });
}

// A token's RoPE coordinates packed in one word, ten bits each: frame within
// its block (the t-table row) in bits 20..29, h in bits 10..19, w in bits
// 0..9, decoded from the block-local token index.  The host rejects RoPE
// grids that do not fit (F, Hs, Ws <= 1024).
__device__ __forceinline__ uint32_t decode_packed(uint32_t n, const FastDiv& fHW, const FastDiv& fWs) {
  const uint32_t frame = fdiv(n, fHW);
  const uint32_t rem = n - frame * fHW.div;
  const uint32_t h = fdiv(rem, fWs);
  const uint32_t w = rem - h * fWs.div;
  return (frame << 20) | (h << 10) | w;
}

// Table entry of one RoPE pair: row base + stride * coordinate, where the
// coordinate is the ten-bit field of the packed word at `shift`.
struct PairLoc {
  int base, stride, shift;
};

__device__ __forceinline__ PairLoc pair_loc(int p, const RopeArgs& ra) {
  const int ht = ra.dt >> 1, hh = ra.dh >> 1;
  PairLoc r;
  if (p < ht) {
    r.base = p; r.stride = ht; r.shift = 20;
  } else if (p < ht + hh) {
    r.base = ra.off_h + (p - ht); r.stride = hh; r.shift = 10;
  } else {
    r.base = ra.off_w + (p - ht - hh); r.stride = ra.dw >> 1; r.shift = 0;
  }
  return r;
}

__device__ __forceinline__ int pair_entry(const PairLoc& pl, uint32_t packed) {
  const uint32_t pos = __builtin_amdgcn_ubfe(packed, (uint32_t)pl.shift, 10u);
  return __mul24((int)pos, pl.stride) + pl.base;  // 24-bit multiply: operands are small
}

// Turn the pair (x, y) by the angle whose (cos, sin) is cs, or by its
// opposite (INV: the transpose of the rotation, for gradients).
template <bool INV = false>
__device__ __forceinline__ void rotate(float& x, float& y, float2 cs) {
  if constexpr (INV) {
    const float xr = x * cs.x + y * cs.y;
    const float yr = y * cs.x - x * cs.y;
    x = xr;
    y = yr;
    return;
  }
  const float xr = x * cs.x - y * cs.y;
  const float yr = x * cs.y + y * cs.x;
  x = xr;
  y = yr;
}

// Rotate a lane's NPAIR consecutive pairs (local elements 2pp, 2pp+1).  In
// paired mode (ROPE >= 2: every axis width a multiple of 4) local pairs
// (2k, 2k+1) are adjacent entries of the same axis at an even index, so one
// 16-byte LDS read serves both.
template <int ROPE, int NPAIR, bool INV = false>
__device__ __forceinline__ void rope_lane(float* x, const float2* tab, const PairLoc* pl, uint32_t co) {
  if constexpr (ROPE >= 2 && NPAIR % 2 == 0) {
    const float4* tab4 = reinterpret_cast<const float4*>(tab);
#pragma unroll
    for (int pp = 0; pp < NPAIR; pp += 2) {
      const float4 cs = tab4[pair_entry(pl[pp], co) >> 1];
      rotate<INV>(x[2 * pp], x[2 * pp + 1], make_float2(cs.x, cs.y));
      rotate<INV>(x[2 * pp + 2], x[2 * pp + 3], make_float2(cs.z, cs.w));
    }
  } else {
#pragma unroll
    for (int pp = 0; pp < NPAIR; ++pp) rotate<INV>(x[2 * pp], x[2 * pp + 1], tab[pair_entry(pl[pp], co)]);
  }
}

// Grouped mode (ROPE == 3: every axis width a multiple of 8) for lanes whose
// elements come in runs of 8 consecutive features starting at a multiple of
// 8: such a run lies in one axis, its four pairs are consecutive entries of
// one table row starting at a multiple of 4, and two 16-byte reads at a
// fixed distance serve them from one computed address.
template <int NRUN, bool INV = false>
__device__ __forceinline__ void rope_lane_runs(float* x, const float2* tab, const PairLoc* pl, uint32_t co) {
  const float4* tab4 = reinterpret_cast<const float4*>(tab);
#pragma unroll
  for (int r = 0; r < NRUN; ++r) {
    const float4* t = tab4 + (pair_entry(pl[r], co) >> 1);
    const float4 c0 = t[0], c1 = t[1];
    float* y = x + 8 * r;
    rotate<INV>(y[0], y[1], make_float2(c0.x, c0.y));
    rotate<INV>(y[2], y[3], make_float2(c0.z, c0.w));
    rotate<INV>(y[4], y[5], make_float2(c1.x, c1.y));
    rotate<INV>(y[6], y[7], make_float2(c1.z, c1.w));
  }
}

// phi = ReLU on the bit pattern: a float with its sign bit set is a negative
// int32, so max_i32(bits, 0) is 0 for every negative float (and -0) and the
// float itself otherwise -- one v_max_i32.
__device__ __forceinline__ float relu_bits(uint32_t bits) {
  return __int_as_float(max((int)bits, 0));
}

// ---------------------------------------------------------------------------
// Element access
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// NW 32-bit words from a 4*NW-byte aligned address.
template <int NW>
__device__ __forceinline__ void load_words(uint32_t* dst, const void* p) {
  if constexpr (NW == 1) {
    dst[0] = *(const uint32_t*)p;
  } else if constexpr (NW == 2) {
    uint2 t = *(const uint2*)p;
    dst[0] = t.x; dst[1] = t.y;
  } else {
    static_assert(NW % 4 == 0, "word count");
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      uint4 t = ((const uint4*)p)[i];
      dst[4 * i] = t.x; dst[4 * i + 1] = t.y; dst[4 * i + 2] = t.z; dst[4 * i + 3] = t.w;
    }
  }
}

template <int NW>
__device__ __forceinline__ void store_words(void* p, const uint32_t* src) {
  if constexpr (NW == 1) {
    *(uint32_t*)p = src[0];
  } else if constexpr (NW == 2) {
    *(uint2*)p = make_uint2(src[0], src[1]);
  } else {
    static_assert(NW % 4 == 0, "word count");
#pragma unroll
    for (int i = 0; i < NW / 4; ++i)
      ((uint4*)p)[i] = make_uint4(src[4 * i], src[4 * i + 1], src[4 * i + 2], src[4 * i + 3]);
  }
}

// Raw buffer access.  A resource covers [base, base + bytes); loads past the
// end return zeros and stores past it are dropped by the hardware, which is
// how the kernels handle a segment's ragged end without branches.
// 0x00020000 is the gfx9 raw-buffer descriptor word 3 (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache policy of the streaming traffic.  Loads of q, k, v (each read
// once) carry the non-temporal bit, which keeps them from churning the
// Infinity Cache; measured on MI355X for this two-pass pattern, this stops
// the output pass's dirty lines from draining into the next reduction
// (memory-only floor of the two passes: 133 -> 112 us at 720p).  Output
// stores keep the default policy: non-temporal stores complete later, and
// since gfx9 counts stores and loads in one in-order counter, the output
// pass's prefetch waits would inherit that latency (77 -> 98 us measured).
constexpr int kLoadPolicy = 2;   // nt
constexpr int kStorePolicy = 0;  // default

// POLICY: kLoadPolicy for the streamed inputs; 0 (default caching) for the
// small per-block operands that many workgroups read.
template <int NW, int POLICY = kLoadPolicy>
__device__ __forceinline__ void buf_load(uint32_t* dst, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (NW == 1) {
    dst[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POLICY);
  } else if constexpr (NW == 2) {
    const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POLICY));
    dst[0] = t.x; dst[1] = t.y;
  } else {
    static_assert(NW % 4 == 0, "word count");
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 t =
          __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, POLICY));
      dst[4 * i] = t.x; dst[4 * i + 1] = t.y; dst[4 * i + 2] = t.z; dst[4 * i + 3] = t.w;
    }
  }
}

template <int NW, int POLICY = kStorePolicy>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint32_t* src) {
  if constexpr (NW == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(src[0], r, off, 0, POLICY);
  } else if constexpr (NW == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, make_uint2(src[0], src[1])), r, off, 0,
                                          POLICY);
  } else {
    static_assert(NW % 4 == 0, "word count");
#pragma unroll
    for (int i = 0; i < NW / 4; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{src[4 * i], src[4 * i + 1], src[4 * i + 2], src[4 * i + 3]}, r, off + 16 * i, 0, POLICY);
  }
}

// Device-scope coherence for the folded prefix's exchange through memory
// (the sc1 bit of gfx94x/gfx950 vector memory instructions): a store is
// acknowledged only once every XCD can see it, and a load does not take a
// line that another XCD's L2 may hold stale.  These are the bits the
// compiler itself gives agent-scope atomic loads and stores; using them on
// the few bytes exchanged avoids the device-scope fences, each of which
// writes back or invalidates a whole L2.
constexpr int kDeviceScope = 16;

// Unpack `CNT` elements (bf16 pairs or fp32 words) into floats.
template <bool BF16, int CNT>
__device__ __forceinline__ void unpack(float* f, const uint32_t* w) {
#pragma unroll
  for (int i = 0; i < CNT; ++i) {
    if (BF16) f[i] = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
    else f[i] = __uint_as_float(w[i]);
  }
}

// phi on a pair of bf16 values in one word: each half is a bf16 bit pattern,
// negative exactly when it is a negative int16, so a packed int16 max with 0
// (v_pk_max_i16) zeroes the negative halves and keeps the rest.
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  const i16x2_t r = __builtin_elementwise_max(__builtin_bit_cast(i16x2_t, w), i16x2_t{0, 0});
  return __builtin_bit_cast(uint32_t, r);
}

// For a pair already through relu_bf16x2: all ones in each 16-bit half that
// is not +0 (where the derivative of ReLU is 1), zeros elsewhere.
__device__ __forceinline__ uint32_t relu_pass_mask(uint32_t relu_w) {
  const i16x2_t one = __builtin_elementwise_min(__builtin_bit_cast(i16x2_t, relu_w), i16x2_t{1, 1});
  return __builtin_bit_cast(uint32_t, i16x2_t{0, 0} - one);
}

// Unpack with phi = ReLU applied on the bits.
template <bool BF16, int CNT>
__device__ __forceinline__ void unpack_relu(float* f, const uint32_t* w) {
  if constexpr (BF16) {
    static_assert(CNT % 2 == 0, "bf16 pairs");
#pragma unroll
    for (int i = 0; i < CNT / 2; ++i) {
      const uint32_t r = relu_bf16x2(w[i]);
      f[2 * i] = bf16_lo(r);
      f[2 * i + 1] = bf16_hi(r);
    }
  } else {
#pragma unroll
    for (int i = 0; i < CNT; ++i) f[i] = relu_bits(w[i]);
  }
}

// Workgroup barrier for LDS data only.  __syncthreads() also orders global
// memory, which on gfx9 means waiting for every outstanding vector load; this
// waits for the wave's LDS operations (lgkmcnt(0), gfx9 s_waitcnt encoding
// 0xC07F leaves vmcnt and expcnt at their maxima) so that prefetched global
// loads stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
}

// Sum of x over the four 16-lane rows of a wavefront, in every lane, with the
// gfx950 lane-swap instructions (no LDS round trip): rows (0+1, 2+3), then
// halves.  Every lane adds the same operands in the same order.
__device__ __forceinline__ float sum_over_rows(float x) {
  auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Wave priority from the share of its steps still to run (done: k of n).
// The instruction arbiter otherwise prefers the oldest waves, so the
// workgroups that share a CU drift apart and the last one runs alone at the
// end; raising the priority of the waves with more work left keeps the
// workgroups of a CU closer together.
__device__ __forceinline__ void prio_by_remaining(int k, int n) {
  const int r4 = 4 * (n - k);
  if (r4 > 3 * n) __builtin_amdgcn_s_setprio(3);
  else if (r4 > 2 * n) __builtin_amdgcn_s_setprio(2);
  else if (r4 > n) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ floatx4 mfma_bf16(const u32x4& a, const u32x4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Geometry shared by the kernels
// ---------------------------------------------------------------------------

struct Geo {
  int N;        // tokens per (b, h) sequence
  int Nb;       // tokens per block
  int nb;       // blocks
  int BH;
  int T, Hs, Ws;
  FastDiv fHW, fWs;
};

__device__ __forceinline__ void add4(float4& a, const float4& b) {
  a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
}

// ---------------------------------------------------------------------------
// The prefix over blocks, folded into the reduction
//
// Every reduction workgroup that writes its last piece of a sequence (b, h)
// counts its arrival on that sequence's counter: its pieces are stored with
// device scope, each wave waits until its stores are acknowledged, the
// workgroup meets at a barrier, and one thread adds 1 with a device-scope
// vector atomic.  The workgroup that brings the count to the number of
// workgroups covering the sequence is the last one: with device-scope loads
// it reads every piece of the sequence, forms the inclusive prefix S_c, Z_c
// over its blocks in a fixed order and writes the output pass's operands
// (and the final cache), then puts the counter back to zero for the next
// call.  No workgroup ever
// waits for another, so there is nothing to bound; the counters only have to
// be zero when a workspace is first used.
// ---------------------------------------------------------------------------

struct FoldArgs {
  unsigned* counters;  // [B*H] arrival counters, zero before and after a call
  const float* S0;     // initial cache [B,H,d,d] in the caller's [fi][fo] layout, or null
  const float* z0;
  float* S_out;        // final cache, or null; may be S0/z0 (each element is read before it is written)
  float* z_out;
  void* frags;         // prefix operands S_c^T [B*H*nb, d, d] in the input dtype, or null
  float* zc;           // Z_c [B*H*nb, d] fp32 (written together with frags)
};

// The prefix of sequence bh, by one workgroup of NT threads: thread t owns
// the 4-element groups t, t + NT, ... of a partial (S^T, then z).  The
// sequence's slots are walked in order, CH per round with all their loads
// issued at once; each block's sum starts from zero, takes the block's
// slots in slot order, then is added to the running prefix (the scan
// kernel's order).  The partials were written by other workgroups during
// this launch, so they are read with device-scope loads.
template <bool BF16, int D, int NT>
__device__ __forceinline__ void scan_sequence(const float* partials, int bh, int nb, int Nb, long long L,
                                              const FoldArgs& fa) {
  constexpr int E = D * D + D;
  constexpr int E4 = E / 4;
  constexpr int NG = (E4 + NT - 1) / NT;
  constexpr int CH = 8;
  // The thread index goes through an empty asm so that the addresses below
  // are computed here, not hoisted to the kernel's start where they would
  // stay live (and spill) across the streaming loop.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  int e[NG];
  float4 run[NG], acc[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    e[i] = min(4 * (tid + i * NT), E - 4);  // threads past the end repeat the last group and store nothing
    run[i] = acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (fa.S0) {  // element e of S^T is S[e % D][e / D]
      if (e[i] < D * D) {
        const float* s0 = fa.S0 + (long long)bh * D * D + (e[i] % D) * D + e[i] / D;
        run[i] = make_float4(s0[0], s0[D], s0[2 * D], s0[3 * D]);
      } else {
        run[i] = *(const float4*)(fa.z0 + (long long)bh * D + (e[i] - D * D));
      }
    }
  }
  auto owns = [&](int i) { return NG * NT == E4 || tid + i * NT < E4; };
  const long long bhc0 = (long long)bh * nb;
  const long long s_first = block_first_slot(bhc0, Nb, L);
  const long long s_last = block_last_slot(bhc0 + nb - 1, Nb, L);
  long long s_beg = s_first;  // slots of the current block c
  long long s_end = block_last_slot(bhc0, Nb, L);
  int c = 0;
  // device-scope loads over the sequence's slots (see kDeviceScope)
  const __amdgpu_buffer_rsrc_t prs =
      make_rsrc(partials + s_first * E, (uint32_t)((s_last - s_first + 1) * E * sizeof(float)));
  for (long long s0 = s_first; s0 <= s_last; s0 += CH) {
    float4 x[CH][NG];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const long long sj = min(s0 + j, s_last);  // slots past the last one repeat it and are not added
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        uint32_t w[4];
        buf_load<4, kDeviceScope>(w, prs, (uint32_t)((sj - s_first) * E + e[i]) * 4);
        x[j][i] = make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                              __uint_as_float(w[3]));
      }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const long long sj = s0 + j;
      if (sj > s_last) break;
      if (sj >= s_beg) {
#pragma unroll
        for (int i = 0; i < NG; ++i) add4(acc[i], x[j][i]);
      }
      if (sj == s_end) {  // block c complete: extend the prefix and emit it
        const long long bhc = bhc0 + c;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          add4(run[i], acc[i]);
          acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (!fa.frags || !owns(i)) continue;
          if (e[i] < D * D) {
            if (BF16) {
              *(uint2*)((__bf16*)fa.frags + bhc * D * D + e[i]) =
                  make_uint2(pack_bf16x2(run[i].x, run[i].y), pack_bf16x2(run[i].z, run[i].w));
            } else {
              *(float4*)((float*)fa.frags + bhc * D * D + e[i]) = run[i];
            }
          } else {
            *(float4*)(fa.zc + bhc * D + (e[i] - D * D)) = run[i];
          }
        }
        ++c;
        if (c < nb) {
          s_beg = block_first_slot(bhc0 + c, Nb, L);
          s_end = block_last_slot(bhc0 + c, Nb, L);
        }
      }
    }
  }
  if (fa.S_out) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (!owns(i)) continue;
      if (e[i] < D * D) {
        float* so = fa.S_out + (long long)bh * D * D + (e[i] % D) * D + e[i] / D;
        so[0] = run[i].x; so[D] = run[i].y; so[2 * D] = run[i].z; so[3 * D] = run[i].w;
      } else {
        *(float4*)(fa.z_out + (long long)bh * D + (e[i] - D * D)) = run[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 1: per-block state reduction
//
// Lane l of a wavefront owns features FPL*(l%16) .. +FPL-1 (FPL = d/16) of
// tokens 4e + l/16, e = 0..7, of a 32-token step, so each load instruction
// reads 4 consecutive token rows.  For bf16 the 8 tokens of a lane become
// the 8 contraction slots of one v_mfma_f32_16x16x32_bf16 operand (K and V
// use the same token->slot map, so the sum over tokens is exact up to
// order); for fp32 each 4-token quad is one v_mfma_f32_16x16x4f32.
// Accumulator (r, s)[i] of lane l holds S[FPL*(4*(l/16)+i)+r][FPL*(l%16)+s].
// ---------------------------------------------------------------------------

template <bool BF16, int D, int ROPE, bool FOLD, int RTT = red_threads<BF16>()>
__global__ __launch_bounds__(RTT, red_min_blocks<BF16>()) void sva_reduce_kernel(
    const void* __restrict__ kp, const void* __restrict__ vp, float* __restrict__ partials,
    Geo geo, SplitArgs sp, RopeArgs ra, FoldArgs fa) {
  constexpr int RT = RTT;
  constexpr int FPL = D / 16;
  constexpr int NPAIR = FPL / 2;
  constexpr int E = D * D + D;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NW = FPL * ESZ / 4;  // 32-bit words per lane per token row piece
  constexpr int ROWB = D * ESZ;      // bytes per token row
  constexpr int STEP = 32;           // tokens per wave per step
  constexpr int WSTRIDE = STEP * (RT / 64);

  extern __shared__ float4 tab_raw[];  // 16-byte aligned
  float2* tab = reinterpret_cast<float2*>(tab_raw);
  // Accumulator tiles for the cross-wave sum, one per wave (bf16, d = 64:
  // 128 KiB; the workgroup has the CU to itself).
  constexpr int NWV = RT / 64;
  __shared__ float red[NWV][D * D];
  __shared__ float zred[NWV][D];
  __shared__ int fold_last;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int cg = lane & 15;
  const int tg = lane >> 4;

  const double lane_freq = ROPE ? load_lane_freq(ra) : 0.0;
  PairLoc pl[NPAIR > 0 ? NPAIR : 1];  // set per segment, once the first loads are out

  const long long g0 = (long long)blockIdx.x * sp.L;
  const long long g1 = min(g0 + sp.L, sp.total);
  const char* kb = (const char*)kp;
  const char* vb = (const char*)vp;

  // Segment parameters: the block (sequence bh, block c) holding the tokens
  // at position p, this workgroup's block-local token range [js, je) in it,
  // buffer resources over the block's rows [0, je) (rows past the segment
  // end read as zeros, so a ragged last step needs no masking: zero k
  // contributes nothing to S or z), and this wave's steps.
  long long bhc, seg_end;
  int bh, c, je, s_first, nsteps;
  __amdgpu_buffer_rsrc_t krs, vrs;
  const uint32_t lane_col = FPL * cg * ESZ;
  auto enter_segment = [&](long long p) {
    const Segment sg = segment_at(p, g1, sp, geo.Nb);
    bhc = sg.bhc;
    seg_end = sg.end;
    bh = (int)(bhc / geo.nb);
    c = (int)(bhc - (long long)bh * geo.nb);
    const int js = sg.js;
    je = sg.je;
    const long long blk_off = ((long long)bh * geo.N + (long long)c * geo.Nb) * ROWB;
    krs = make_rsrc(kb + blk_off, (uint32_t)je * ROWB);
    vrs = make_rsrc(vb + blk_off, (uint32_t)je * ROWB);
    s_first = js + wave * STEP;
    nsteps = s_first < je ? (je - s_first + WSTRIDE - 1) / WSTRIDE : 0;
  };

  floatx4 acc[FPL][FPL];
  float zacc[FPL];

  // A step is 32 consecutive tokens; lane (cg, tg) takes tokens 4e + tg,
  // each load reading 4 consecutive token rows (offsets are immediates).
  auto load_step = [&](uint32_t (&kw)[8][NW], uint32_t (&vw)[8][NW], int s0) {
    const uint32_t off = (uint32_t)(s0 + tg) * ROWB + lane_col;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      buf_load<NW>(kw[e], krs, off + 4 * e * ROWB);
      buf_load<NW>(vw[e], vrs, off + 4 * e * ROWB);
    }
  };

  // Software pipeline over the wave's steps, three register sets in a ring:
  // while step k computes, steps k+1 and k+2 are in flight (16 KiB per wave
  // at bf16, d = 64).  sched_barrier keeps the compiler from sinking a
  // prefetch below the compute it should overlap.  The first two steps of a
  // segment are issued before the previous segment's epilogue.
  uint32_t kA[8][NW], vA[8][NW], kB[8][NW], vB[8][NW], kC[8][NW], vC[8][NW];
  // Every workgroup has at least one token (the grid is ceil(total / L)), so
  // the loop needs no entry test, which would split the reads of the kernel
  // arguments into two dependent rounds.
  long long pos = g0;
  enter_segment(pos);
  load_step(kA, vA, s_first);
  load_step(kB, vB, s_first + WSTRIDE);
  do {
#pragma unroll
    for (int r = 0; r < FPL; ++r)
#pragma unroll
      for (int s = 0; s < FPL; ++s) acc[r][s] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < FPL; ++r) zacc[r] = 0.f;

    auto compute_step = [&](const uint32_t (&kw)[8][NW], const uint32_t (&vw)[8][NW], int s0) {
      // Coordinates: lanes 0..31 decode the step's 32 tokens (clamped to the
      // segment so table indices stay in range), every lane fetches those of
      // its own 8 tokens.
      uint32_t mine = 0;
      if (ROPE)
        mine = decode_packed((uint32_t)min(s0 + (lane & 31), je - 1), geo.fHW, geo.fWs);
      // phi, z and RoPE for token e of this lane, in registers.
      auto prep_token = [&](int e, float (&kf)[FPL]) {
        unpack_relu<BF16, FPL>(kf, kw[e]);
#pragma unroll
        for (int r = 0; r < FPL; ++r) zacc[r] += kf[r];
        if (ROPE) {
          const uint32_t co = (uint32_t)__builtin_amdgcn_ds_bpermute((4 * e + tg) * 4, (int)mine);
          rope_lane<ROPE, NPAIR>(kf, tab, pl, co);
        }
      };
      if (BF16) {
        // V needs no arithmetic: regroup its bf16 halves so slot e of
        // operand s holds feature FPL*cg + s of token e.  Then k-tilde is
        // rounded to bf16 two tokens at a time into the A operands.
        u32x4 A[FPL], Bv[FPL];
#pragma unroll
        for (int s = 0; s < FPL; ++s) {
          const uint32_t sel = (s & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
          for (int m = 0; m < 4; ++m)
            Bv[s][m] = __builtin_amdgcn_perm(vw[2 * m + 1][s >> 1], vw[2 * m][s >> 1], sel);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float k0[FPL], k1[FPL];
          prep_token(2 * m, k0);
          prep_token(2 * m + 1, k1);
#pragma unroll
          for (int r = 0; r < FPL; ++r) A[r][m] = pack_bf16x2(k0[r], k1[r]);
        }
#pragma unroll
        for (int r = 0; r < FPL; ++r)
#pragma unroll
          for (int s = 0; s < FPL; ++s) acc[r][s] = mfma_bf16(A[r], Bv[s], acc[r][s]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float kf[FPL], vf[FPL];
          prep_token(e, kf);
          unpack<false, FPL>(vf, vw[e]);
#pragma unroll
          for (int r = 0; r < FPL; ++r)
#pragma unroll
            for (int s = 0; s < FPL; ++s) acc[r][s] = mfma_f32(kf[r], vf[s], acc[r][s]);
        }
      }
    };

    __builtin_amdgcn_sched_barrier(0);
    // The RoPE layout is read from the kernel arguments only now, so that
    // the streaming loads above wait for no more than the pointers and the
    // split.
    if (ROPE) {
      int cg_seg = cg;  // opaque per segment: keeps this setup below the loads
      asm volatile("" : "+v"(cg_seg));
#pragma unroll
      for (int pp = 0; pp < NPAIR; ++pp) pl[pp] = pair_loc(NPAIR * cg_seg + pp, ra);
    }
    // The RoPE table (h, w rows once; t rows for this block) is built while
    // the first loads are in flight.  Every wave has passed the previous
    // segment's epilogue barrier, so no wave still reads the old t rows.
    if (ROPE) {
      if (pos == g0) build_rope_hw<!BF16, RT>(tab, ra, lane_freq);
      build_rope_t<!BF16, RT>(tab, ra, c, lane_freq);
    }
    lds_barrier();
    int k = 0;
    for (; k + 3 <= nsteps; k += 3) {
      prio_by_remaining(k, nsteps);
      const int s0 = s_first + k * WSTRIDE;
      load_step(kC, vC, s0 + 2 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute_step(kA, vA, s0);
      __builtin_amdgcn_sched_barrier(0);
      load_step(kA, vA, s0 + 3 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute_step(kB, vB, s0 + WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      load_step(kB, vB, s0 + 4 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute_step(kC, vC, s0 + 2 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (k < nsteps) compute_step(kA, vA, s_first + k * WSTRIDE);
    if (k + 1 < nsteps) compute_step(kB, vB, s_first + (k + 1) * WSTRIDE);

    // The next segment's first two steps go out now, in flight across this
    // segment's epilogue (a workgroup whose range crosses a block boundary
    // otherwise waits a full memory round trip after it).  The epilogue
    // below needs only this segment's block and sequence.  In the folded
    // form the epilogue waits for every memory access of the wave, so the
    // next loads follow it instead.
    const long long bhc_done = bhc, seg_end_done = seg_end;
    const int bh_done = bh;
    const bool more = seg_end < g1;
    if (!FOLD && more) {
      enter_segment(seg_end_done);
      load_step(kA, vA, s_first);
      load_step(kB, vB, s_first + WSTRIDE);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Fixed-order reduction over the four lane groups (lane swaps), then over
    // the waves: every wave stores its tile, one barrier, and each thread
    // sums the tiles for 4 contiguous elements in wave order.  (A two-round
    // tree over half as much LDS -- waves 4..7 handing their tiles to waves
    // 0..3 -- cost one more barrier and round of LDS traffic.)
#pragma unroll
    for (int r = 0; r < FPL; ++r) zacc[r] = sum_over_rows(zacc[r]);
    auto tile_elem = [&](int slot, int r, int i) { return red[slot] + (FPL * (4 * tg + i) + r) * D + FPL * cg; };
    auto store_tile = [&](int slot) {
#pragma unroll
      for (int r = 0; r < FPL; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* dst = tile_elem(slot, r, i);
#pragma unroll
          for (int s = 0; s < FPL; ++s) dst[s] = acc[r][s][i];
        }
    };
    store_tile(wave);
    if (tg == 0) {
#pragma unroll
      for (int r = 0; r < FPL; ++r) zred[wave][FPL * cg + r] = zacc[r];
    }
    lds_barrier();
    // Piece (workgroup g, block bhc) goes to slot g + bhc: pieces are ordered
    // along the flattened token axis, so g + bhc strictly increases from one
    // piece to the next and the slots of one block's pieces are contiguous.
    // A partial holds S transposed (row fo, column fi), then z.
    // (Stored with device scope when the prefix is folded in: the last
    // workgroup of the sequence, on any XCD, reads them back.)
    constexpr int PP = FOLD ? kDeviceScope : 0;
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(partials + ((long long)blockIdx.x + bhc_done) * E, E * 4);
    for (int e = tid; e < D * D / 4; e += RT) {
      const int fo = e % D, fi0 = 4 * (e / D);  // consecutive lanes: consecutive fo
      float t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        t[j] = red[0][(fi0 + j) * D + fo];
#pragma unroll
        for (int w = 1; w < NWV; ++w) t[j] += red[w][(fi0 + j) * D + fo];
      }
      const uint32_t w4[4] = {__float_as_uint(t[0]), __float_as_uint(t[1]), __float_as_uint(t[2]),
                              __float_as_uint(t[3])};
      buf_store<4, PP>(prs, (uint32_t)(fo * D + fi0) * 4, w4);
    }
    for (int e = tid; e < D; e += RT) {
      float t = zred[0][e];
#pragma unroll
      for (int w = 1; w < NWV; ++w) t += zred[w][e];
      const uint32_t w1 = __float_as_uint(t);
      buf_store<1, PP>(prs, (uint32_t)(D * D + e) * 4, &w1);
    }
    if constexpr (FOLD) {
      // This workgroup's last piece of sequence bh: count the arrival (see
      // the folded prefix above); the last arrival forms bh's prefix.  The
      // pieces were stored with device scope: each wave waits until its
      // stores are acknowledged, the workgroup meets, then one thread counts
      // with a device-scope atomic.  The empty asm statements keep the
      // compiler from moving memory accesses across these points.
      if (arrives(seg_end_done, g1, bh_done, geo.nb, sp.Nbp)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are visible device-wide
        __builtin_amdgcn_s_barrier();
        if (tid == 0) {
          const long long first = seq_first_wg(bh_done, geo.nb, sp.Nbp, sp.L);
          const long long last = seq_last_wg(bh_done, geo.nb, sp.Nbp, sp.L);
          const unsigned old = __hip_atomic_fetch_add(fa.counters + bh_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          fold_last = old + 1 == (unsigned)(last - first + 1);
        }
        lds_barrier();
        if (fold_last) {
          asm volatile("" ::: "memory");
          scan_sequence<BF16, D, RT>(partials, bh_done, geo.nb, sp.Nbp, sp.L, fa);
          if (tid == 0) __hip_atomic_store(fa.counters + bh_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (more) {
        enter_segment(seg_end_done);
        load_step(kA, vA, s_first);
        load_step(kB, vB, s_first + WSTRIDE);
      }
    }
    // `red` is next written after the next segment's barrier.
    pos = seg_end_done;
  } while (pos < g1);
}

// ---------------------------------------------------------------------------
// Kernel 2: inclusive prefix over blocks, fixed order
//
// One thread per state element per (b, h).  Partials and the emitted prefix
// operands hold S transposed (row fo = value feature, column fi = key
// feature), then z, so consecutive threads read and write consecutive
// addresses; the output kernel reads its MFMA operands straight from that
// layout.  S0 and S_out use the caller's [fi][fo] layout.
// ---------------------------------------------------------------------------

struct ScanArgs {
  int nb, Nb;       // blocks; a block's length on the partials' flattened axis (SplitArgs::Nbp)
  long long L;      // flattened tokens per reduce workgroup
  int cpl;          // blocks per block-lane
  int has_init;     // S0/z0 given
  int write_frags;  // emit the output-kernel operands
  int write_final;  // emit S_out/z_out
  int reverse;      // suffix over blocks (last block first), for the backward
};

constexpr int kScanLanes = 8;                      // block-lanes per element
constexpr int kScanElems = kThreads / kScanLanes;  // 4-element groups per workgroup


// Sum, in slot order, of the partials of flattened block bhc at elements
// e .. e+3.
template <int E>
__device__ __forceinline__ float4 block_sum(const float* __restrict__ partials, long long bhc,
                                            long long L, int Nb, int e) {
  const long long first = block_first_slot(bhc, Nb, L);
  const float* p = partials + first * E + e;
  const int n = (int)(block_last_slot(bhc, Nb, L) - first + 1);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  int i = 0;
  for (; i + 4 <= n; i += 4) {
    const float4 x0 = *(const float4*)(p + (long long)i * E), x1 = *(const float4*)(p + (long long)(i + 1) * E);
    const float4 x2 = *(const float4*)(p + (long long)(i + 2) * E), x3 = *(const float4*)(p + (long long)(i + 3) * E);
    add4(s, x0); add4(s, x1); add4(s, x2); add4(s, x3);
  }
  for (; i < n; ++i) add4(s, *(const float4*)(p + (long long)i * E));
  return s;
}

// kScanElems groups of 4 elements x kScanLanes block-lanes per workgroup.
// Blocks are taken in scan order: 0, 1, ... (prefix), or nb-1, nb-2, ...
// (suffix, `reverse`, for the backward; the initial value is then the
// gradient of the final state and the last value that of the initial one).
// Lane ty owns blocks [ty*cpl, ty*cpl + cpl): pass 1 sums them, the lane
// totals are scanned through LDS in lane order, pass 2 adds each block in
// turn (kept in registers, or re-read: the partials are L2-resident) and
// emits the running prefix.  The order of every sum is fixed by (nb, reduce
// grid), so results are reproducible.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void sva_scan_kernel(
    const float* __restrict__ partials, const float* S0, const float* z0, float* S_out,
    float* z_out, void* __restrict__ frags, float* __restrict__ zc, void* __restrict__ frags_lo,
    ScanArgs a) {
  constexpr int E = D * D + D;
  static_assert(E % 4 == 0 && (D * D) % 4 == 0, "element groups");
  __shared__ float4 lane_tot[kScanLanes][kScanElems];
  const int tx = threadIdx.x % kScanElems;
  const int ty = threadIdx.x / kScanElems;
  const int e = 4 * (blockIdx.x * kScanElems + tx);  // first of 4 consecutive elements
  const int bh = blockIdx.y;
  const bool active = e < E;
  const bool in_S = e < D * D;  // a group never straddles S and z
  const int c_begin = min(ty * a.cpl, a.nb);
  const int c_end = min(c_begin + a.cpl, a.nb);

  // The initial cache is read before the barrier: S_out may alias S0 and is
  // written after it.  Element e of S^T is S[e % D][e / D].
  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
  if (active && a.has_init) {
    if (in_S) {
      const float* s0 = S0 + (long long)bh * D * D + (e % D) * D + e / D;
      run = make_float4(s0[0], s0[D], s0[2 * D], s0[3 * D]);
    } else {
      run = *(const float4*)(z0 + (long long)bh * D + (e - D * D));
    }
  }
  // Pass 1: block sums of this lane's blocks.  Up to kKeep of them stay in
  // registers for pass 2; lanes with more blocks re-read theirs (L2 hits).
  // With one block per sequence (the cached step, block-by-block streaming)
  // the block-lanes split that block's pieces instead: lane ty takes slots
  // ty, ty + 8, ... (all of its loads issued at once), and lane 0 adds the
  // eight lane sums in lane order.
  constexpr int kKeep = 4;
  float4 keep[kKeep];
  float4 tot = make_float4(0.f, 0.f, 0.f, 0.f);
  const bool one = a.nb == 1;
  if (active) {
    if (one) {
      const long long first = block_first_slot(bh, a.Nb, a.L);
      const int n = (int)(block_last_slot(bh, a.Nb, a.L) - first + 1);
      const float* pp = partials + first * E + e;
      for (int i0 = ty; i0 < n; i0 += 4 * kScanLanes) {
        float4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)  // slots past the last repeat it and are not added
          x[j] = *(const float4*)(pp + (long long)min(i0 + j * kScanLanes, n - 1) * E);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (i0 + j * kScanLanes < n) add4(tot, x[j]);
      }
    } else {
      for (int c = c_begin; c < c_end; ++c) {
        const int cb = a.reverse ? a.nb - 1 - c : c;  // the block, in scan order
        const float4 bs = block_sum<E>(partials, (long long)bh * a.nb + cb, a.L, a.Nb, e);
#pragma unroll
        for (int i = 0; i < kKeep; ++i)
          if (c - c_begin == i) keep[i] = bs;
        add4(tot, bs);
      }
    }
  }
  lane_tot[ty][tx] = tot;
  __syncthreads();
  if (!active) return;
  if (one) {
    if (ty != 0) return;  // lane 0 owns the block (c_begin = 0, c_end = 1)
    keep[0] = lane_tot[0][tx];
    for (int l = 1; l < kScanLanes; ++l) add4(keep[0], lane_tot[l][tx]);
  } else {
    for (int l = 0; l < ty; ++l) add4(run, lane_tot[l][tx]);
  }

  for (int c = c_begin; c < c_end; ++c) {
    const long long bhc = (long long)bh * a.nb + (a.reverse ? a.nb - 1 - c : c);
    float4 bs;
    if (c - c_begin < kKeep) {
#pragma unroll
      for (int i = 0; i < kKeep; ++i)
        if (c - c_begin == i) bs = keep[i];
    } else {
      bs = block_sum<E>(partials, bhc, a.L, a.Nb, e);
    }
    add4(run, bs);
    if (a.write_frags) {
      if (in_S) {
        if (BF16) {
          const uint2 hi = make_uint2(pack_bf16x2(run.x, run.y), pack_bf16x2(run.z, run.w));
          *(uint2*)((__bf16*)frags + bhc * D * D + e) = hi;
          if (frags_lo) {
            // the remainder S - hi in bf16: hi + lo carries S to about 16 bits
            const uint2 lo = make_uint2(pack_bf16x2(run.x - bf16_lo(hi.x), run.y - bf16_hi(hi.x)),
                                        pack_bf16x2(run.z - bf16_lo(hi.y), run.w - bf16_hi(hi.y)));
            *(uint2*)((__bf16*)frags_lo + bhc * D * D + e) = lo;
          }
        } else {
          *(float4*)((float*)frags + bhc * D * D + e) = run;
        }
      } else {
        *(float4*)(zc + bhc * D + (e - D * D)) = run;
      }
    }
  }
  if (a.write_final && c_begin < c_end && c_end == a.nb) {
    if (in_S) {
      float* so = S_out + (long long)bh * D * D + (e % D) * D + e / D;
      so[0] = run.x; so[D] = run.y; so[2 * D] = run.z; so[3 * D] = run.w;
    } else {
      *(float4*)(z_out + (long long)bh * D + (e - D * D)) = run;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: output pass
//
// A wavefront handles 16-token tiles.  Lane l takes token l%16 of the tile
// and FPLa = d/4 of its features, chosen so that each 16-byte load or store
// of the four lanes of one token covers 64 contiguous bytes of the row:
//   lane (g = l/16) local element m  <->  feature feat(g, m)
//     bf16: 32*(m/8) + 8*g + m%8        fp32: 16*(m/4) + 4*g + m%4
// Those elements are exactly its B-operand share of out^T = S^T qr^T (k-slot
// e of k-step ks is local element 8*ks + e for bf16, ks for fp32).  The A
// operand rows are permuted (see the prefix scan) so that accumulator rt of
// lane l holds the output features stored by the same contiguous pieces.
// The denominator phi q . Z is, for fp32, an fp32 dot over the lane's
// features plus two lane-swap adds; for bf16, one more MFMA per k-step with
// Z split into two bf16 rows, summed across the lane rows the same way.  The
// lane then scales its accumulators and stores.
// ---------------------------------------------------------------------------

template <bool BF16>
__device__ __forceinline__ int apply_feat(int g, int m) {
  return BF16 ? 32 * (m >> 3) + 8 * g + (m & 7) : 16 * (m >> 2) + 4 * g + (m & 3);
}

template <bool BF16, int D, int ROPE>
__global__ __launch_bounds__(app_threads<BF16>(), app_min_blocks<BF16>()) void sva_apply_kernel(
    const void* __restrict__ qp, void* __restrict__ outp, const void* __restrict__ frags,
    const float* __restrict__ zc, Geo geo, SplitArgs sp, RopeArgs ra, float eps) {
  constexpr int AT = app_threads<BF16>();
  constexpr int FPLa = D / 4;
  constexpr int NRT = D / 16;
  constexpr int NKS = BF16 ? D / 32 : D / 4;
  constexpr int NPAIR = FPLa / 2;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NW = FPLa * ESZ / 4;

  // Tile I/O goes through LDS so that every global load and store
  // instruction covers whole 128-byte lines: PPR lanes per row, RPI rows per
  // instruction.  Each wave has its own tiles (no barrier needed: a wave's
  // LDS operations execute in order).  Piece p of row r sits at unit
  // r*PPR + (p ^ (r & SWM)): the XOR swizzle spreads both the row-order and
  // the MFMA-order 16-byte accesses over all banks (measured on gfx950:
  // about 5 clocks per 64-lane read instead of 8.5 with a padded row).
  constexpr int ROWB = D * ESZ;
  constexpr int PPR = ROWB / 16;  // 16-byte pieces per token row
  constexpr int RPI = 64 / PPR;   // rows per instruction
  constexpr int NLD = 16 / RPI;   // instructions per 16-row tile
  constexpr int SWM = (PPR < 8 ? PPR : 8) - 1;
  static_assert(NLD * 4 == NW, "tile pieces");
  auto tile_at = [](int r, int p) { return r * PPR + (p ^ (r & SWM)); };

  extern __shared__ float4 tab_raw[];  // 16-byte aligned
  float2* tab = reinterpret_cast<float2*>(tab_raw);
  // The block's prefix operand S^T (D rows of CPR 16-byte chunks) is staged
  // in LDS with chunk c of row f at f*CPR + (c ^ (f & (CPR-1))), so that the
  // sixteen rows a k-step's lanes read spread over the banks.
  constexpr int CPR = D * ESZ / 16;
  constexpr int FRAG_U4 = D * CPR;
  __shared__ uint4 fstage[FRAG_U4];
  auto frag_at = [](int f, int c) { return f * CPR + (c ^ (f & (CPR - 1))); };
  constexpr int TPS = 2;          // 16-token tiles per wave step
  constexpr int TSZ = 16 * PPR;   // one tile, in 16-byte units
  __shared__ uint4 tstage[AT / 64][TPS * TSZ];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int row = lane & 15;

  // RoPE lookups: one per pair, or (grouped mode, bf16 runs of 8 features)
  // one per run.
  constexpr bool RUNS = BF16 && ROPE == 3;
  constexpr int NLOC = RUNS ? NKS : NPAIR;
  const double lane_freq = ROPE ? load_lane_freq(ra) : 0.0;
  PairLoc pl[NLOC];  // set per segment, once the first loads are out

  const long long g0 = (long long)blockIdx.x * sp.L;
  const long long g1 = min(g0 + sp.L, sp.total);
  const char* qb = (const char*)qp;
  char* ob = (char*)outp;

  // Every workgroup has at least one token (the grid is ceil(total / L)), so the
  // loop needs no entry test, which would split the reads of the kernel
  // arguments into two dependent rounds.
  long long pos = g0;
  do {
    const Segment sg = segment_at(pos, g1, sp, geo.Nb);
    const long long bhc = sg.bhc;
    const long long seg_end = sg.end;
    const int bh = (int)(bhc / geo.nb);
    const int c = (int)(bhc - (long long)bh * geo.nb);
    const int js = sg.js;
    const int je = sg.je;
    const long long row0 = (long long)bh * geo.N + (long long)c * geo.Nb;

    // Buffer resources over the block's rows [0, je): loads past the segment
    // end read zeros and stores past it are dropped, so ragged tiles need no
    // branches.
    const long long blk_off = row0 * (D * ESZ);
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qb + blk_off, (uint32_t)je * (D * ESZ));
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(ob + blk_off, (uint32_t)je * (D * ESZ));
    // Global side: lane takes piece ld_piece of row ld_row (+ RPI per
    // instruction).  MFMA side: 16-byte piece i of lane (g, row) is bytes
    // 64*i + 16*g of the row.
    const int ld_row = lane / PPR, ld_piece = lane % PPR;
    uint4* wst = tstage[wave];
    auto load_tile = [&](uint32_t (&qw)[NW], int t) {
      const uint32_t off = (uint32_t)(t + ld_row) * ROWB + 16 * ld_piece;
#pragma unroll
      for (int i = 0; i < NLD; ++i) buf_load<4>(qw + 4 * i, qrs, off + i * RPI * ROWB);
    };

    // Segment prologue, in three groups so that no wait covers more than it
    // must (vector loads complete in issue order):
    //   1. loads of this block's prefix operand S_c^T and of Z_c;
    //   2. loads of the segment's first two steps of q;
    //   3. the operand to LDS and the denominator operand to registers (these
    //      wait for group 1 only, while the q loads stay in flight), then the
    //      RoPE table rows.
    // The scheduling barriers keep the groups in this order, and every use
    // of group 1 sits in the same block as its loads, before any branch, so
    // the compiler does not sink those loads below the q loads.
    lds_barrier();  // every wave has read the previous segment's fstage and t rows
    // (Raw buffer loads: the compiler keeps them in program order, whereas
    // plain loads through const restrict pointers count as invariant and may
    // be sunk next to their use, behind the q loads.)
    constexpr int FR = (FRAG_U4 + AT - 1) / AT;
    uint32_t fr[FR][4];
    {
      const __amdgpu_buffer_rsrc_t frs = make_rsrc((const uint4*)frags + bhc * FRAG_U4, FRAG_U4 * 16);
#pragma unroll
      for (int i = 0; i < FR; ++i)  // pieces past the operand read as zeros and are not stored
        buf_load<4, 0>(fr[i], frs, (uint32_t)(tid + i * AT) * 16);
    }
    // Z_c: bf16, the 8-feature runs of the lane's k-steps; fp32, the lane's
    // FPLa features in runs of 4.
    constexpr int NZ4 = BF16 ? 2 * NKS : FPLa / 4;
    uint32_t zr[NZ4][4];
    {
      const __amdgpu_buffer_rsrc_t zrs = make_rsrc(zc + bhc * D, D * 4);
#pragma unroll
      for (int i = 0; i < NZ4; ++i) buf_load<4, 0>(zr[i], zrs, (uint32_t)apply_feat<BF16>(g, 4 * i) * 4);
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int WSTRIDE = 16 * TPS * (AT / 64);
    const int t_first = js + wave * 16 * TPS;
    const int nsteps = t_first < je ? (je - t_first + WSTRIDE - 1) / WSTRIDE : 0;
    uint32_t qa[TPS][NW], qb[TPS][NW], qc[TPS][NW];
    auto load_stepq = [&](uint32_t (&x)[TPS][NW], int t) {
#pragma unroll
      for (int i = 0; i < TPS; ++i) load_tile(x[i], t + 16 * i);
    };
    load_stepq(qa, t_first);
    load_stepq(qb, t_first + WSTRIDE);
    __builtin_amdgcn_sched_barrier(0);
    // the RoPE layout is read from the kernel arguments only now (as in the
    // reduction)
    if (ROPE) {
      int g_seg = g;  // opaque per segment: keeps this setup below the loads
      asm volatile("" : "+v"(g_seg));
#pragma unroll
      for (int i = 0; i < NLOC; ++i) pl[i] = pair_loc(apply_feat<BF16>(g_seg, RUNS ? 8 * i : 2 * i) >> 1, ra);
    }
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int u = tid + i * AT;
      if (FRAG_U4 % AT == 0 || u < FRAG_U4)
        fstage[frag_at(u / CPR, u % CPR)] = make_uint4(fr[i][0], fr[i][1], fr[i][2], fr[i][3]);
    }
    // Denominator operand.  fp32: the lane's FPLa entries of Z.  bf16: the
    // A operand of a 16x16x32 MFMA against the unrotated phi(q) tile, row 0
    // holding Z rounded to bf16 and row 4 the rounding remainder (also in
    // bf16), other rows zero; Z_hi + Z_lo carries Z to about 2^-17 relative,
    // and the MFMA forms the bf16 x bf16 products exactly and sums in fp32.
    float z[BF16 ? 1 : FPLa];
    u32x4 az[BF16 ? NKS : 1];
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        float zz[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) zz[i] = __uint_as_float(zr[2 * ks + i / 4][i % 4]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x2_t hi = {(__bf16)zz[2 * m], (__bf16)zz[2 * m + 1]};
          const bf16x2_t lo = {(__bf16)(zz[2 * m] - (float)hi[0]), (__bf16)(zz[2 * m + 1] - (float)hi[1])};
          az[ks][m] = row == 0 ? __builtin_bit_cast(uint32_t, hi) : row == 4 ? __builtin_bit_cast(uint32_t, lo) : 0u;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NZ4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) z[4 * i + j] = __uint_as_float(zr[i][j]);
    }
    if (ROPE) {
      if (pos == g0) build_rope_hw<!BF16, AT>(tab, ra, lane_freq);
      build_rope_t<!BF16, AT>(tab, ra, c, lane_freq);
    }
    lds_barrier();

    // MFMA A operands.  bf16: accumulator rt, lane row r holds output feature
    //   fo = 32*(rt/2) + 8*(r/4) + 4*(rt%2) + r%4,
    // so that accumulator rt holds the features the lane stores in one
    // contiguous 16-byte piece; k-step ks, lane group g: input features
    // 32*ks + 8*g .. +7 (chunk 4*ks + g of row fo).  fp32: fo = 16*rt + r,
    // k-step ks: input feature feat(g, ks), four consecutive ks in chunk
    // 4*(ks/4) + g.
    u32x4 A16[BF16 ? NRT : 1][BF16 ? NKS : 1];
    float A32[BF16 ? 1 : NRT][BF16 ? 1 : NKS];
    if constexpr (BF16) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int fo = 32 * (rt >> 1) + 8 * (row >> 2) + 4 * (rt & 1) + (row & 3);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 t = fstage[frag_at(fo, 4 * ks + g)];
          A16[rt][ks] = u32x4{t.x, t.y, t.z, t.w};
        }
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int fo = 16 * rt + row;
#pragma unroll
        for (int ks = 0; ks < NKS; ks += 4) {
          const float4 t = __builtin_bit_cast(float4, fstage[frag_at(fo, ks + g)]);
          A32[rt][ks] = t.x; A32[rt][ks + 1] = t.y; A32[rt][ks + 2] = t.z; A32[rt][ks + 3] = t.w;
        }
      }
    }

    // The TPS tiles of a step go through each phase together, so that their
    // LDS round trips and MFMA chains overlap.
    auto compute_stepq = [&](const uint32_t (&x)[TPS][NW], int t) {
      // global row layout -> MFMA layout through the wave's LDS tiles
#pragma unroll
      for (int u = 0; u < TPS; ++u)
#pragma unroll
        for (int i = 0; i < NLD; ++i)
          wst[u * TSZ + tile_at(i * RPI + ld_row, ld_piece)] =
              make_uint4(x[u][4 * i], x[u][4 * i + 1], x[u][4 * i + 2], x[u][4 * i + 3]);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      uint32_t qw[TPS][NW];
#pragma unroll
      for (int u = 0; u < TPS; ++u)
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
          const uint4 v = wst[u * TSZ + tile_at(row, 4 * i + g)];
          qw[u][4 * i] = v.x; qw[u][4 * i + 1] = v.y; qw[u][4 * i + 2] = v.z; qw[u][4 * i + 3] = v.w;
        }
      floatx4 acc[TPS][NRT];
#pragma unroll
      for (int u = 0; u < TPS; ++u)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc[u][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
      float den[TPS];
      if constexpr (BF16) {
        // phi(q) as bf16 pairs is the B operand of the denominator MFMA, and
        // of the numerator too when there is no rotation.
        u32x4 rq[TPS][NKS];
        floatx4 dacc[TPS];
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
#pragma unroll
          for (int i = 0; i < NW; ++i) rq[u][i >> 2][i & 3] = relu_bf16x2(qw[u][i]);
          dacc[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) dacc[u] = mfma_bf16(az[ks], rq[u][ks], dacc[u]);
        }
        if constexpr (ROPE != 0) {
#pragma unroll
          for (int u = 0; u < TPS; ++u) {
            float qf[FPLa];
#pragma unroll
            for (int i = 0; i < NW; ++i) {
              qf[2 * i] = bf16_lo(rq[u][i >> 2][i & 3]);
              qf[2 * i + 1] = bf16_hi(rq[u][i >> 2][i & 3]);
            }
            const uint32_t co = decode_packed((uint32_t)min(t + 16 * u + row, je - 1), geo.fHW, geo.fWs);
            if constexpr (RUNS) rope_lane_runs<NKS>(qf, tab, pl, co);
            else rope_lane<ROPE, NPAIR>(qf, tab, pl, co);
#pragma unroll
            for (int i = 0; i < NW; ++i) rq[u][i >> 2][i & 3] = pack_bf16x2(qf[2 * i], qf[2 * i + 1]);
          }
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int u = 0; u < TPS; ++u)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) acc[u][rt] = mfma_bf16(A16[rt][ks], rq[u][ks], acc[u][rt]);
        // rows 0 and 4 of the denominator product sit in lane rows 0 and 1
#pragma unroll
        for (int u = 0; u < TPS; ++u) den[u] = sum_over_rows(dacc[u][0]);
      } else {
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
          float qf[FPLa];
          unpack_relu<BF16, FPLa>(qf, qw[u]);
          float dn = 0.f;
#pragma unroll
          for (int m = 0; m < FPLa; ++m) dn += qf[m] * z[m];
          if (ROPE) {
            const uint32_t co = decode_packed((uint32_t)min(t + 16 * u + row, je - 1), geo.fHW, geo.fWs);
            rope_lane<ROPE, NPAIR>(qf, tab, pl, co);
          }
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) acc[u][rt] = mfma_f32(A32[rt][ks], qf[ks], acc[u][rt]);
          den[u] = sum_over_rows(dn);
        }
      }
      uint32_t ow[TPS][NW];
#pragma unroll
      for (int u = 0; u < TPS; ++u) {
        // v_rcp_f32 (1 ulp) for bf16 outputs; a correctly rounded divide for fp32.
        const float inv = BF16 ? __builtin_amdgcn_rcpf(den[u] + eps) : 1.0f / (den[u] + eps);
        if (BF16) {
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            ow[u][2 * rt] = pack_bf16x2(acc[u][rt][0] * inv, acc[u][rt][1] * inv);
            ow[u][2 * rt + 1] = pack_bf16x2(acc[u][rt][2] * inv, acc[u][rt][3] * inv);
          }
        } else {
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) ow[u][4 * rt + i] = __float_as_uint(acc[u][rt][i] * inv);
        }
      }
      // MFMA layout -> global row layout through the same LDS tiles
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int u = 0; u < TPS; ++u)
#pragma unroll
        for (int i = 0; i < NW / 4; ++i)
          wst[u * TSZ + tile_at(row, 4 * i + g)] = make_uint4(ow[u][4 * i], ow[u][4 * i + 1], ow[u][4 * i + 2], ow[u][4 * i + 3]);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int u = 0; u < TPS; ++u) {
        const uint32_t off = (uint32_t)(t + 16 * u + ld_row) * ROWB + 16 * ld_piece;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const uint4 v = wst[u * TSZ + tile_at(i * RPI + ld_row, ld_piece)];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
          buf_store<4>(ors, off + i * RPI * ROWB, w4);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    };

    // TPS 16-token tiles per wave step (the first two steps were issued
    // above), software-pipelined over a ring of three register sets: while
    // step k computes (and issues its stores), the loads of steps k+1 and k+2
    // are in flight.  gfx9 counts loads and stores in one in-order counter,
    // so the wait for step k+1's loads never has to cover step k's stores,
    // which were issued after them.
    int k = 0;
    for (; k + 3 <= nsteps; k += 3) {
      const int t0 = t_first + k * WSTRIDE;
      load_stepq(qc, t0 + 2 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute_stepq(qa, t0);
      __builtin_amdgcn_sched_barrier(0);
      load_stepq(qa, t0 + 3 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute_stepq(qb, t0 + WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      load_stepq(qb, t0 + 4 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute_stepq(qc, t0 + 2 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (k < nsteps) compute_stepq(qa, t_first + k * WSTRIDE);
    if (k + 1 < nsteps) compute_stepq(qb, t_first + (k + 1) * WSTRIDE);
    pos = seg_end;
  } while (pos < g1);
}

// ---------------------------------------------------------------------------
// Backward kernels (bf16)
//
// Gradients of L = <out, dout> (+ <S_final, dS_final> + <z_final, dz_final>)
// by the chain rule through the forward's steps.  With num = qt S_c and
// den = phi(q) . Z_c + eps (so out = num / den):
//   dnum = dout / den,  dden = -(dout . num) / den^2 = -(dout . out) / den,
//   dqt = S_c dnum,     dS_c = sum qt dnum^T,  dZ_c = sum dden phi(q),
//   dq  = [q > 0] (RoPE^T dqt + dden Z_c),
// the prefix over blocks becomes a suffix: G_c = sum_{c' >= c} dS_c'
// (+ dS_final), g_c likewise, and for the tokens of block c
//   dkt = G_c v,  dv = G_c^T kt,  dk = [k > 0] (RoPE^T dkt + g_c).
// RoPE^T turns every pair by the opposite angle.  dnum is never rounded or
// stored: the output side forms S_c dout from the exact bf16 dout and scales
// by 1/den in fp32, and the state-gradient pass (the reduction kernel) sums
// (qt / den) dout^T, scaling qt before its bf16 rounding.  The output side
// reads q, dout and out and writes dq, dden and 1/den; the state side reads
// k and v and writes dk and dv.  Both work on 16-token tiles in the layout of the
// forward output pass: lane (g = l/16, row = l%16) holds features
// feat(g, m) = 32(m/8) + 8g + m%8 of token row, which is its share of an
// MFMA B operand whose k index is the feature, and accumulator rt of an
// MFMA whose A operand has rows fo(rt, r) = 32(rt/2) + 8(r/4) + 4(rt%2) +
// r%4 holds the same features of the same token (local element 4rt + i).
// ---------------------------------------------------------------------------

template <int D>
struct BTile {
  static constexpr int ROWB = 2 * D;           // bytes per bf16 token row
  static constexpr int PPR = ROWB / 16;        // 16-byte pieces per row
  static constexpr int RPI = 64 / PPR;         // rows per load instruction
  static constexpr int NLD = 16 / RPI;         // load instructions per tile
  static constexpr int NW = D / 8;             // words per lane in MFMA layout
  static constexpr int SWM = (PPR < 8 ? PPR : 8) - 1;
  static constexpr int TSZ = 16 * PPR;         // one tile, in 16-byte units
  static constexpr int CPR = D / 8;            // 16-byte chunks per operand row
  static constexpr int NRT = D / 16;           // accumulators (16 rows each)
  static constexpr int NKS = D / 32;           // MFMA k-steps
  static_assert(NLD * 4 == NW, "tile pieces");
  __device__ static int at(int r, int p) { return r * PPR + (p ^ (r & SWM)); }
  __device__ static int frag_at(int f, int c) { return f * CPR + (c ^ (f & (CPR - 1))); }
  __device__ static int fo(int rt, int r) { return 32 * (rt >> 1) + 8 * (r >> 2) + 4 * (rt & 1) + (r & 3); }
};

// Global rows t .. t+15 of a bf16 [rows, D] segment into registers, in row
// order (PPR lanes per row).
template <int D>
__device__ __forceinline__ void btile_load(uint32_t* w, __amdgpu_buffer_rsrc_t r, int t, int lane) {
  using T = BTile<D>;
  const uint32_t off = (uint32_t)(t + lane / T::PPR) * T::ROWB + 16 * (lane % T::PPR);
#pragma unroll
  for (int i = 0; i < T::NLD; ++i) buf_load<4>(w + 4 * i, r, off + i * T::RPI * T::ROWB);
}

// Row-order registers -> MFMA-layout words through the wave's LDS tile.
template <int D>
__device__ __forceinline__ void btile_to_mfma(uint4* wst, const uint32_t* w, uint32_t* out, int lane) {
  using T = BTile<D>;
  const int g = lane >> 4, row = lane & 15;
#pragma unroll
  for (int i = 0; i < T::NLD; ++i)
    wst[T::at(i * T::RPI + lane / T::PPR, lane % T::PPR)] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int i = 0; i < T::NW / 4; ++i) {
    const uint4 v = wst[T::at(row, 4 * i + g)];
    out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// MFMA-layout words -> global rows t .. t+15 through the wave's LDS tile.
template <int D>
__device__ __forceinline__ void btile_store(uint4* wst, const uint32_t* ow, __amdgpu_buffer_rsrc_t r, int t,
                                            int lane) {
  using T = BTile<D>;
  const int g = lane >> 4, row = lane & 15;
#pragma unroll
  for (int i = 0; i < T::NW / 4; ++i)
    wst[T::at(row, 4 * i + g)] = make_uint4(ow[4 * i], ow[4 * i + 1], ow[4 * i + 2], ow[4 * i + 3]);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const uint32_t off = (uint32_t)(t + lane / T::PPR) * T::ROWB + 16 * (lane % T::PPR);
#pragma unroll
  for (int i = 0; i < T::NLD; ++i) {
    const uint4 v = wst[T::at(i * T::RPI + lane / T::PPR, lane % T::PPR)];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    buf_store<4>(r, off + i * T::RPI * T::ROWB, w4);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Stage a [D, D] bf16 matrix stored row-major in global memory (M^T of the
// prefix operands, rows = output features) into LDS: as it is (rows a), or
// transposed (rows = its columns) for products with the other side.
template <int D, bool TRANSPOSE>
__device__ __forceinline__ void stage_operand(uint4* fst, const uint4 (&fr)[(D * D / 8 + kThreads - 1) / kThreads],
                                              int tid) {
  using T = BTile<D>;
  constexpr int N = D * T::CPR;
#pragma unroll
  for (int i = 0; i < (N + kThreads - 1) / kThreads; ++i) {
    const int u = tid + i * kThreads;
    if (N % kThreads != 0 && u >= N) continue;
    const int a = u / T::CPR, c = u % T::CPR;
    if constexpr (!TRANSPOSE) {
      fst[T::frag_at(a, c)] = fr[i];
    } else {
      const uint32_t w[4] = {fr[i].x, fr[i].y, fr[i].z, fr[i].w};
      unsigned short* h = reinterpret_cast<unsigned short*>(fst);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        h[T::frag_at(8 * c + j, a >> 3) * 8 + (a & 7)] = (unsigned short)(w[j >> 1] >> (16 * (j & 1)));
    }
  }
}

template <int D>
__device__ __forceinline__ void load_operand(uint4 (&fr)[(D * D / 8 + kThreads - 1) / kThreads], const void* frags,
                                             long long bhc, int tid) {
  constexpr int N = D * D / 8;
  const uint4* src = (const uint4*)frags + bhc * N;
#pragma unroll
  for (int i = 0; i < (N + kThreads - 1) / kThreads; ++i)
    if (N % kThreads == 0 || tid + i * kThreads < N) fr[i] = src[tid + i * kThreads];
}

__device__ __forceinline__ float bf16_elem(const uint32_t* w, int m) {
  return (m & 1) ? bf16_hi(w[m >> 1]) : bf16_lo(w[m >> 1]);
}

// Sum over the 16 lanes of each row of the wavefront (lanes 16r .. 16r+15),
// in every lane, with DPP: mirror, half mirror, then neighbour and pair
// swaps inside quads.  Each lane applies the same sequence, so any one lane's
// result is reproducible.
__device__ __forceinline__ float sum_within_rows(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  return x;
}

// MFMA operand with tokens along k from two 16-token tiles in LDS (row order,
// swizzled as BTile::at): lane (g = l/16, i = l%16) gets features f0 + i of
// tokens 8g .. 8g+7 (tile g/2, rows 8(g%2) ..), through two transposing
// reads.  ds_read_b64_tr_b16 hands lane i of a 16-lane group element i%4 of
// the 8-byte chunks addressed by lanes 4j + i/4 (j = 0..3), so lane x
// addresses row T0 + x/4, features f0 + 4(x%4) .. +3 (measured on gfx950).
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const uint4* t0, const uint4* t1, int f0, int lane) {
  using T = BTile<D>;
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const int g = lane >> 4, x = lane & 15;
  const uint4* tile = (g >> 1) ? t1 : t0;
  const int f = f0 + 4 * (x & 3);
  const int piece = f >> 3, half = (f >> 2) & 1;
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rowi = 8 * (g & 1) + 4 * h + (x >> 2);
    const char* a = reinterpret_cast<const char*>(tile + T::at(rowi, piece)) + 8 * half;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)a);
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    r[2 * h] = w[0];
    r[2 * h + 1] = w[1];
  }
  return r;
}

// Output side: q, dout -> dq, with the gradients of the block states fused
// in: per (workgroup, block) piece it writes dS_c^T = (sum qt dnum^T)^T and
// dZ_c = sum dden phi(q) into `partials` (the reduction's slot layout).
// sfrag holds S_c^T in bf16 and sfrag_lo the remainder S_c^T - sfrag in
// bf16, zc holds Z_c, per (b, h, block).  S_c dout runs on both parts (the
// rounding of S_c to bf16 alone, about 2^-9, is amplified where dout . num
// cancels).  The output itself is not read: the denominator's term needs
// dout . num, which is qt . (S_c dout), the product dq takes anyway, so q and
// dout are the only streams read.  dS takes qt / den (rounded to bf16 once)
// and the exact dout as MFMA operands with tokens along k, read back
// transposed from the wave's LDS tiles.  One workgroup per CU: with the 64 dS accumulators a wave needs
// more than 256 registers, and at one wave per SIMD it gets 512
// (accumulation registers included) instead of spilling.
template <int D, int ROPE>
__global__ __launch_bounds__(kThreads, 1) void sva_bwd_out_kernel(
    const void* __restrict__ qp, const void* __restrict__ dop, void* __restrict__ dqp,
    float* __restrict__ partials, const void* __restrict__ sfrag, const void* __restrict__ sfrag_lo,
    const float* __restrict__ zc, Geo geo, SplitArgs sp, RopeArgs ra, float eps) {
  using T = BTile<D>;
  constexpr int FPLa = D / 4;
  constexpr int NW = T::NW, NKS = T::NKS, NRT = T::NRT;
  constexpr int NPAIR = FPLa / 2;
  constexpr bool RUNS = ROPE == 3;
  constexpr int NLOC = RUNS ? NKS : NPAIR;
  constexpr int FR = (D * D / 8 + kThreads - 1) / kThreads;
  constexpr int E = D * D + D;
  constexpr int NWAVE = kThreads / 64;

  extern __shared__ float4 tab_raw[];
  float2* tab = reinterpret_cast<float2*>(tab_raw);
  __shared__ uint4 fst[D * T::CPR];  // S_c in bf16, rows = key features
  __shared__ uint4 fsl[D * T::CPR];  // S_c - fst in bf16
  __shared__ __align__(16) float zst[D];
  // Per wave: q in / dq out, and for the two steps of a pair the dout tiles
  // and the qt/den tiles.  After the loop the region is the scratch of the
  // cross-wave sum (2 d*d tiles and 4 z rows).
  __shared__ uint4 tiles[NWAVE][5][T::TSZ];
  static_assert(sizeof(tiles) >= (2 * D * D + NWAVE * D) * sizeof(float), "epilogue scratch");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int row = lane & 15;
  uint4* tq = tiles[wave][0];

  const double lane_freq = ROPE ? load_lane_freq(ra) : 0.0;
  PairLoc pl[NLOC];
  if (ROPE) {
#pragma unroll
    for (int i = 0; i < NLOC; ++i) pl[i] = pair_loc(apply_feat<true>(g, RUNS ? 8 * i : 2 * i) >> 1, ra);
  }

  const long long g0 = (long long)blockIdx.x * sp.L;
  const long long g1 = min(g0 + sp.L, sp.total);
  // Every workgroup has at least one token (the grid is ceil(total / L)), so the
  // loop needs no entry test, which would split the reads of the kernel
  // arguments into two dependent rounds.
  long long pos = g0;
  do {
    const long long bhc = pos / geo.Nb;
    const long long seg_end = min(g1, (bhc + 1) * (long long)geo.Nb);
    const int bh = (int)(bhc / geo.nb);
    const int c = (int)(bhc - (long long)bh * geo.nb);
    const int js = (int)(pos - bhc * geo.Nb);
    const int je = (int)(seg_end - bhc * geo.Nb);
    const long long row0 = (long long)bh * geo.N + (long long)c * geo.Nb;
    const long long blk_off = row0 * T::ROWB;
    const uint32_t nbytes = (uint32_t)je * T::ROWB;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc((const char*)qp + blk_off, nbytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc((const char*)dop + blk_off, nbytes);
    const __amdgpu_buffer_rsrc_t dqrs = make_rsrc((char*)dqp + blk_off, nbytes);

    lds_barrier();  // every wave is done with the previous block's operands, t rows and scratch
    uint4 fr[FR], frl[FR];
    load_operand<D>(fr, sfrag, bhc, tid);
    load_operand<D>(frl, sfrag_lo, bhc, tid);
    const float zmine = tid < D ? zc[bhc * D + tid] : 0.f;
    constexpr int WSTRIDE = 16 * NWAVE;
    const int t_first = js + wave * 16;
    const int nsteps = t_first < je ? (je - t_first + WSTRIDE - 1) / WSTRIDE : 0;
    // Two register sets: the next step is in flight while one is computed.
    // (A ring of four, three steps in flight, measured the same: 258.3
    // against 258.1 us per 720p backward.)
    uint32_t x0[2][NW], x1[2][NW];
    auto load2 = [&](uint32_t (&x)[2][NW], int k) {
      const int t = t_first + k * WSTRIDE;
      btile_load<D>(x[0], qrs, t, lane);
      btile_load<D>(x[1], drs, t, lane);
    };
    load2(x0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (ROPE) {
      if (pos == g0) build_rope_hw<false, kThreads>(tab, ra, lane_freq);
      build_rope_t<false, kThreads>(tab, ra, c, lane_freq);
    }
    stage_operand<D, true>(fst, fr, tid);
    stage_operand<D, true>(fsl, frl, tid);
    if (tid < D) zst[tid] = zmine;
    lds_barrier();
    // S_c's A-operand fragments stay in registers for the whole segment (read
    // from LDS per tile they would be the largest LDS stream of the loop)
    u32x4 sh[NRT][NKS], sl[NRT][NKS];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 x = fst[T::frag_at(T::fo(rt, row), 4 * ks + g)];
        const uint4 y = fsl[T::frag_at(T::fo(rt, row), 4 * ks + g)];
        sh[rt][ks] = u32x4{x.x, x.y, x.z, x.w};
        sl[rt][ks] = u32x4{y.x, y.y, y.z, y.w};
      }

    // The denominator operand (rows 0 and 4: Z rounded to bf16 and the
    // remainder), as in the output pass.  Z_c itself is read from LDS where
    // it is needed (registers are scarce here).
    u32x4 az[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float z0 = zst[apply_feat<true>(g, 8 * ks + 2 * m)], z1 = zst[apply_feat<true>(g, 8 * ks + 2 * m + 1)];
        const bf16x2_t hi = {(__bf16)z0, (__bf16)z1};
        const bf16x2_t lo = {(__bf16)(z0 - (float)hi[0]), (__bf16)(z1 - (float)hi[1])};
        az[ks][m] = row == 0 ? __builtin_bit_cast(uint32_t, hi) : row == 4 ? __builtin_bit_cast(uint32_t, lo) : 0u;
      }

    floatx4 sacc[NRT][NRT];  // dS block (rt over key features, st over value features)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int st = 0; st < NRT; ++st) sacc[rt][st] = floatx4{0.f, 0.f, 0.f, 0.f};
    float zacc[FPLa];  // this lane's tokens' dden * phi(q)
#pragma unroll
    for (int m = 0; m < FPLa; ++m) zacc[m] = 0.f;

    // One 16-token tile; `slot` picks the dout and qt/den tiles kept for the
    // pair's dS product.
    auto compute = [&](const uint32_t (&x)[2][NW], int t, int slot) {
      uint4* td = tiles[wave][1 + slot];
      uint4* ts = tiles[wave][3 + slot];
      uint32_t qw[NW], dw[NW];
      btile_to_mfma<D>(tq, x[0], qw, lane);
      btile_to_mfma<D>(td, x[1], dw, lane);  // the dout tile stays for the dS operand
      u32x4 bd[NKS];
#pragma unroll
      for (int i = 0; i < NW; ++i) bd[i >> 2][i & 3] = dw[i];
      floatx4 acc[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc[rt] = mfma_bf16(sh[rt][ks], bd[ks], acc[rt]);  // S_c dout
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc[rt] = mfma_bf16(sl[rt][ks], bd[ks], acc[rt]);
      uint32_t rqw[NW];
      u32x4 rq[NKS];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        rqw[i] = relu_bf16x2(qw[i]);
        rq[i >> 2][i & 3] = rqw[i];
      }
      floatx4 dacc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) dacc = mfma_bf16(az[ks], rq[ks], dacc);
      const float den = sum_over_rows(dacc[0]) + eps;
      // rows past the segment hold zeros; their 1/den is taken as 0 so that
      // they add nothing (also when eps is 0)
      const float inv = t + row < je ? __builtin_amdgcn_rcpf(den) : 0.f;
      uint32_t co = 0;
      if constexpr (ROPE != 0) co = decode_packed((uint32_t)min(t + row, je - 1), geo.fHW, geo.fWs);
      float qf[FPLa];  // qt
#pragma unroll
      for (int m = 0; m < FPLa; ++m) qf[m] = bf16_elem(rqw, m);
      if constexpr (ROPE != 0) {
        if constexpr (RUNS) rope_lane_runs<NKS>(qf, tab, pl, co);
        else rope_lane<ROPE, NPAIR>(qf, tab, pl, co);
      }
      {
        // qt / den, rounded to bf16, into the tile of the dS product
        uint32_t sw[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i) sw[i] = pack_bf16x2(qf[2 * i] * inv, qf[2 * i + 1] * inv);
#pragma unroll
        for (int i = 0; i < NW / 4; ++i)
          ts[T::at(row, 4 * i + g)] = make_uint4(sw[4 * i], sw[4 * i + 1], sw[4 * i + 2], sw[4 * i + 3]);
      }
      // dout . num = qt . (S_c dout): this lane's key features, then the rows
      float dot = 0.f;
#pragma unroll
      for (int m = 0; m < FPLa; ++m) dot += qf[m] * acc[m >> 2][m & 3];
      const float dd = -sum_over_rows(dot) * inv * inv;  // dden: -(dout . num) / den^2
#pragma unroll
      for (int m = 0; m < FPLa; ++m) zacc[m] += dd * bf16_elem(rqw, m);
      float gq[FPLa];
#pragma unroll
      for (int m = 0; m < FPLa; ++m) gq[m] = acc[m >> 2][m & 3] * inv;  // S_c dnum
      if constexpr (ROPE != 0) {
        if constexpr (RUNS) rope_lane_runs<NKS, true>(gq, tab, pl, co);
        else rope_lane<ROPE, NPAIR, true>(gq, tab, pl, co);
      }
      uint32_t dqw[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const float2 zz = *(const float2*)(zst + apply_feat<true>(g, 2 * i));  // runs of 8: pairs stay together
        // masked after packing, so that no branch guards the Z reads
        dqw[i] = pack_bf16x2(gq[2 * i] + dd * zz.x, gq[2 * i + 1] + dd * zz.y) & relu_pass_mask(rqw[i]);
      }
      btile_store<D>(tq, dqw, dqrs, t, lane);
    };
    // dS += (qt/den)^T dout over the 32 tokens of a pair of steps.  The
    // transposing reads always run on the whole wavefront: under a partial
    // exec mask ds_read_b64_tr_b16 still writes the destination registers of
    // the masked-off lanes (measured on gfx950), so a step past the segment
    // is computed on zeros instead of masking lanes.
    auto ds_pair = [&]() {
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      u32x4 bo[NRT];
#pragma unroll
      for (int st = 0; st < NRT; ++st) bo[st] = tr_operand<D>(tiles[wave][1], tiles[wave][2], 16 * st, lane);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const u32x4 ao = tr_operand<D>(tiles[wave][3], tiles[wave][4], 16 * rt, lane);
#pragma unroll
        for (int st = 0; st < NRT; ++st) sacc[rt][st] = mfma_bf16(ao, bo[st], sacc[rt][st]);
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    };

    // Whole pairs of steps: when only the first step of the last pair is
    // inside the segment, the second one reads zeros (the loads past the
    // segment's end return 0), gets 1/den = 0 on every row, adds nothing to
    // dS and dZ, and its stores are dropped, so no slot needs clearing.
    auto step = [&](const uint32_t (&x)[2][NW], int k, int slot) {
      compute(x, t_first + k * WSTRIDE, slot);
    };
    for (int k = 0; k < nsteps; k += 2) {
      load2(x1, k + 1);
      __builtin_amdgcn_sched_barrier(0);
      step(x0, k, 0);
      __builtin_amdgcn_sched_barrier(0);
      load2(x0, k + 2);
      __builtin_amdgcn_sched_barrier(0);
      step(x1, k + 1, 1);
      ds_pair();
      __builtin_amdgcn_sched_barrier(0);
    }

    // Fixed-order sum over the waves: waves 2, 3 store their tiles, waves 0,
    // 1 add theirs and store, then each thread sums the two tiles for one
    // 4-element column of dS^T; z: rows summed within each lane row, then
    // the waves in order.
    float* scr = reinterpret_cast<float*>(&tiles[0][0][0]);  // [2][D*D] then [NWAVE][D]
    float* zscr = scr + 2 * D * D;
#pragma unroll
    for (int m = 0; m < FPLa; ++m) zacc[m] = sum_within_rows(zacc[m]);
    lds_barrier();  // every wave is done with its tiles
    auto tile_elem = [&](int slot, int rt, int st, int i) {
      return scr + slot * D * D + (16 * rt + 4 * g + i) * D + 16 * st + row;
    };
    if (wave >= 2) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int st = 0; st < NRT; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) *tile_elem(wave - 2, rt, st, i) = sacc[rt][st][i];
    }
    if (row == 0) {
#pragma unroll
      for (int m = 0; m < FPLa; ++m) zscr[wave * D + apply_feat<true>(g, m)] = zacc[m];
    }
    lds_barrier();
    if (wave < 2) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int st = 0; st < NRT; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* p = tile_elem(wave, rt, st, i);
            *p = sacc[rt][st][i] + *p;
          }
    }
    lds_barrier();
    float* dst = partials + ((long long)blockIdx.x + bhc) * E;
    for (int e = tid; e < D * D / 4; e += kThreads) {
      const int fo = e % D, fi0 = 4 * (e / D);
      float t4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) t4[j] = scr[(fi0 + j) * D + fo] + scr[D * D + (fi0 + j) * D + fo];
      *(float4*)(dst + fo * D + fi0) = make_float4(t4[0], t4[1], t4[2], t4[3]);
    }
    for (int e = tid; e < D; e += kThreads) {
      float t1 = zscr[e];
#pragma unroll
      for (int w = 1; w < NWAVE; ++w) t1 += zscr[w * D + e];
      dst[D * D + e] = t1;
    }
    pos = seg_end;
  } while (pos < g1);
}

// State side: k, v -> dk, dv.  gfrag holds G_c^T (bf16) and gc holds g_c per
// (b, h, block).
template <int D, int ROPE>
__global__ __launch_bounds__(kThreads, 2) void sva_bwd_kv_kernel(
    const void* __restrict__ kp, const void* __restrict__ vp, void* __restrict__ dkp, void* __restrict__ dvp,
    const void* __restrict__ gfrag, const float* __restrict__ gc, Geo geo, SplitArgs sp, RopeArgs ra) {
  using T = BTile<D>;
  constexpr int FPLa = D / 4;
  constexpr int NW = T::NW, NKS = T::NKS, NRT = T::NRT;
  constexpr int NPAIR = FPLa / 2;
  constexpr bool RUNS = ROPE == 3;
  constexpr int NLOC = RUNS ? NKS : NPAIR;
  constexpr int FR = (D * D / 8 + kThreads - 1) / kThreads;

  extern __shared__ float4 tab_raw[];
  float2* tab = reinterpret_cast<float2*>(tab_raw);
  __shared__ uint4 fsT[D * T::CPR];  // G_c^T, rows = value features (for dv)
  __shared__ uint4 fsN[D * T::CPR];  // G_c, rows = key features (for dkt)
  __shared__ float gst[D];
  __shared__ uint4 tiles[kThreads / 64][2][T::TSZ];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int row = lane & 15;
  uint4* tk = tiles[wave][0];
  uint4* tv = tiles[wave][1];

  const double lane_freq = ROPE ? load_lane_freq(ra) : 0.0;
  PairLoc pl[NLOC];
  if (ROPE) {
#pragma unroll
    for (int i = 0; i < NLOC; ++i) pl[i] = pair_loc(apply_feat<true>(g, RUNS ? 8 * i : 2 * i) >> 1, ra);
  }

  const long long g0 = (long long)blockIdx.x * sp.L;
  const long long g1 = min(g0 + sp.L, sp.total);
  // Every workgroup has at least one token (the grid is ceil(total / L)), so the
  // loop needs no entry test, which would split the reads of the kernel
  // arguments into two dependent rounds.
  long long pos = g0;
  do {
    const long long bhc = pos / geo.Nb;
    const long long seg_end = min(g1, (bhc + 1) * (long long)geo.Nb);
    const int bh = (int)(bhc / geo.nb);
    const int c = (int)(bhc - (long long)bh * geo.nb);
    const int js = (int)(pos - bhc * geo.Nb);
    const int je = (int)(seg_end - bhc * geo.Nb);
    const long long row0 = (long long)bh * geo.N + (long long)c * geo.Nb;
    const long long blk_off = row0 * T::ROWB;
    const uint32_t nbytes = (uint32_t)je * T::ROWB;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc((const char*)kp + blk_off, nbytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const char*)vp + blk_off, nbytes);
    const __amdgpu_buffer_rsrc_t dkrs = make_rsrc((char*)dkp + blk_off, nbytes);
    const __amdgpu_buffer_rsrc_t dvrs = make_rsrc((char*)dvp + blk_off, nbytes);

    lds_barrier();
    uint4 fr[FR];
    load_operand<D>(fr, gfrag, bhc, tid);
    const float gmine = tid < D ? gc[bhc * D + tid] : 0.f;
    constexpr int WSTRIDE = 16 * (kThreads / 64);
    const int t_first = js + wave * 16;
    const int nsteps = t_first < je ? (je - t_first + WSTRIDE - 1) / WSTRIDE : 0;
    uint32_t xa[2][NW], xb[2][NW];
    auto load2 = [&](uint32_t (&x)[2][NW], int t) {
      btile_load<D>(x[0], krs, t, lane);
      btile_load<D>(x[1], vrs, t, lane);
    };
    load2(xa, t_first);
    __builtin_amdgcn_sched_barrier(0);
    if (ROPE) {
      if (pos == g0) build_rope_hw<false, kThreads>(tab, ra, lane_freq);
      build_rope_t<false, kThreads>(tab, ra, c, lane_freq);
    }
    stage_operand<D, false>(fsT, fr, tid);
    stage_operand<D, true>(fsN, fr, tid);
    if (tid < D) gst[tid] = gmine;
    lds_barrier();
    float gz[FPLa];
#pragma unroll
    for (int m = 0; m < FPLa; ++m) gz[m] = gst[apply_feat<true>(g, m)];
    // G_c's A-operand fragments, both orientations, in registers for the
    // segment (not re-read from LDS per tile)
    u32x4 gT[NRT][NKS], gN[NRT][NKS];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 x = fsT[T::frag_at(T::fo(rt, row), 4 * ks + g)];
        const uint4 y = fsN[T::frag_at(T::fo(rt, row), 4 * ks + g)];
        gT[rt][ks] = u32x4{x.x, x.y, x.z, x.w};
        gN[rt][ks] = u32x4{y.x, y.y, y.z, y.w};
      }

    auto compute = [&](const uint32_t (&x)[2][NW], int t) {
      uint32_t kw[NW], vw[NW];
      btile_to_mfma<D>(tk, x[0], kw, lane);
      btile_to_mfma<D>(tv, x[1], vw, lane);
      u32x4 rk[NKS], bv[NKS];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        rk[i >> 2][i & 3] = relu_bf16x2(kw[i]);
        bv[i >> 2][i & 3] = vw[i];
      }
      u32x4 kt[NKS];
      uint32_t co = 0;
      if constexpr (ROPE != 0) {
        co = decode_packed((uint32_t)min(t + row, je - 1), geo.fHW, geo.fWs);
        float kf[FPLa];
#pragma unroll
        for (int m = 0; m < FPLa; ++m) kf[m] = (m & 1) ? bf16_hi(rk[m >> 3][(m >> 1) & 3]) : bf16_lo(rk[m >> 3][(m >> 1) & 3]);
        if constexpr (RUNS) rope_lane_runs<NKS>(kf, tab, pl, co);
        else rope_lane<ROPE, NPAIR>(kf, tab, pl, co);
#pragma unroll
        for (int i = 0; i < NW; ++i) kt[i >> 2][i & 3] = pack_bf16x2(kf[2 * i], kf[2 * i + 1]);
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) kt[ks] = rk[ks];
      }
      floatx4 av[NRT], ak[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        av[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
        ak[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          av[rt] = mfma_bf16(gT[rt][ks], kt[ks], av[rt]);  // dv = G_c^T kt
          ak[rt] = mfma_bf16(gN[rt][ks], bv[ks], ak[rt]);  // dkt = G_c v
        }
      float gk[FPLa];
#pragma unroll
      for (int m = 0; m < FPLa; ++m) gk[m] = ak[m >> 2][m & 3];
      if constexpr (ROPE != 0) {
        if constexpr (RUNS) rope_lane_runs<NKS, true>(gk, tab, pl, co);
        else rope_lane<ROPE, NPAIR, true>(gk, tab, pl, co);
      }
      uint32_t dkw[NW], dvw[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t r = rk[i >> 2][i & 3];
        const float a = (r & 0xffffu) ? gk[2 * i] + gz[2 * i] : 0.f;
        const float b = (r >> 16) ? gk[2 * i + 1] + gz[2 * i + 1] : 0.f;
        dkw[i] = pack_bf16x2(a, b);
        dvw[i] = pack_bf16x2(av[(2 * i) >> 2][(2 * i) & 3], av[(2 * i + 1) >> 2][(2 * i + 1) & 3]);
      }
      btile_store<D>(tk, dkw, dkrs, t, lane);
      btile_store<D>(tv, dvw, dvrs, t, lane);
    };

    // Three register sets in a ring: steps k + 1 and k + 2 in flight while
    // step k computes.  Loads past the segment read zeros and are not used.
    uint32_t xc[2][NW];
    load2(xb, t_first + WSTRIDE);
    int k = 0;
    for (; k + 3 <= nsteps; k += 3) {
      const int t0 = t_first + k * WSTRIDE;
      load2(xc, t0 + 2 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute(xa, t0);
      __builtin_amdgcn_sched_barrier(0);
      load2(xa, t0 + 3 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute(xb, t0 + WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      load2(xb, t0 + 4 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
      compute(xc, t0 + 2 * WSTRIDE);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (k < nsteps) compute(xa, t_first + k * WSTRIDE);
    if (k + 1 < nsteps) compute(xb, t_first + (k + 1) * WSTRIDE);
    pos = seg_end;
  } while (pos < g1);
}

// ---------------------------------------------------------------------------
// Standalone phi + RoPE stage (test entry point): one thread per token.
// ---------------------------------------------------------------------------

template <bool BF16, int D, int ROPE>
__global__ __launch_bounds__(kThreads) void sva_prep_kernel(
    const void* __restrict__ xp, float* __restrict__ xr, float* __restrict__ xphi, Geo geo, RopeArgs ra) {
  // grid: (token chunks of one block, blocks, b*h); one thread per token
  constexpr int ESZ = BF16 ? 2 : 4;
  extern __shared__ float4 tab_raw[];  // 16-byte aligned
  float2* tab = reinterpret_cast<float2*>(tab_raw);
  const int c = blockIdx.y;
  if (ROPE) {
    const double lane_freq = load_lane_freq(ra);
    build_rope_hw<!BF16, kThreads>(tab, ra, lane_freq);
    build_rope_t<!BF16, kThreads>(tab, ra, c, lane_freq);
  }
  __syncthreads();
  const int j = blockIdx.x * kThreads + threadIdx.x;  // block-local token
  if (j >= geo.Nb) return;
  const long long t = (long long)blockIdx.z * geo.N + (long long)c * geo.Nb + j;
  uint32_t w[D * ESZ / 4];
  load_words<D * ESZ / 4>(w, (const char*)xp + t * D * ESZ);
  float f[D];
  unpack_relu<BF16, D>(f, w);
  if (xphi) {
#pragma unroll
    for (int i = 0; i < D; i += 4) *(float4*)(xphi + t * D + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
  }
  if (ROPE) {
    const uint32_t co = decode_packed((uint32_t)j, geo.fHW, geo.fWs);
#pragma unroll
    for (int p = 0; p < D / 2; ++p) rotate(f[2 * p], f[2 * p + 1], tab[pair_entry(pair_loc(p, ra), co)]);
  }
#pragma unroll
  for (int i = 0; i < D; i += 4) *(float4*)(xr + t * D + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
}

// ---------------------------------------------------------------------------
// Host side: validation, planning, launches
// ---------------------------------------------------------------------------

struct Plan {
  int BH, D, N, Nb, nb;
  bool bf16, rope;
  // 0 none, 1 general, 2 paired (every axis width a multiple of 4),
  // 3 grouped (every axis width a multiple of 8; paired where grouping does
  // not apply)
  int rope_mode;
  Geo geo;
  RopeArgs ra;
  SplitArgs red, app;
  int G_red, G_app;
  SplitArgs bwd, bwd_kv;  // backward output side and state side
  int G_bwd_out, G_bwd_kv;
  size_t tab_bytes;
  // The forward's prefix runs inside the reduction (the last workgroup of
  // each sequence forms it) instead of in a separate scan launch.
  bool fold;
  size_t off_counters, off_partials, off_frags, off_zc, off_frags_lo, ws_bytes;
  // Saved prefix states: the operands S_c^T at 0, for bf16 their remainders
  // (S_c^T - operand, in bf16) at states_lo, Z_c at states_zc.
  size_t states_lo, states_zc, states_bytes;
};

constexpr long long kRedWorkgroupsMax = 1024;  // bounds the partials workspace
constexpr long long kAppWorkgroupsMax = 4096;
constexpr int kFoldMinBlocks = 32;  // blocks per sequence from which the prefix is folded

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bn && y < x + an;
}

// How many workgroups of `fn` the current device holds at once (CUs times
// workgroups per CU for its registers and LDS): the streaming kernels' grids
// are at most that many equal token ranges, so that no workgroup waits for a
// slot (make_split, then align_split).
int resident_workgroups(const void* fn, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 512;
  const auto key = std::make_tuple(dev, fn, lds);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, threads, lds) != hipSuccess || per < 1)
    per = 1;
  const int n = cus * per;
  cache[key] = n;
  return n;
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  cache[dev] = cus;
  return cus;
}

sva_status validate_desc(const sva_desc* d, bool one_block) {
  if (!d) return SVA_ERR_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->T < 1 || d->Hs < 1 || d->Ws < 1 || d->frames_per_block < 1 ||
      d->t0 < 0)
    return SVA_ERR_INVALID_ARG;
  if (d->dtype != SVA_F32 && d->dtype != SVA_BF16) return SVA_ERR_UNSUPPORTED;
  if (d->d != 32 && d->d != 64) return SVA_ERR_UNSUPPORTED;
  if (d->T % d->frames_per_block) return SVA_ERR_INVALID_ARG;
  if (one_block && d->T != d->frames_per_block) return SVA_ERR_INVALID_ARG;
  if (!(d->eps >= 0.f) || d->eps > 3.0e38f) return SVA_ERR_INVALID_ARG;
  if (d->rope != 0 && d->rope != 1) return SVA_ERR_INVALID_ARG;
  const long long HW = (long long)d->Hs * d->Ws;
  const long long N = HW * d->T;
  if (N * d->d >= (1ll << 31)) return SVA_ERR_UNSUPPORTED;  // per-sequence 32-bit indexing
  // buffer offsets within a block are 32-bit byte offsets
  if ((long long)d->frames_per_block * HW * d->d * (d->dtype == SVA_BF16 ? 2 : 4) >= (1ll << 31))
    return SVA_ERR_UNSUPPORTED;
  if ((long long)d->B * d->H * N >= (1ll << 40)) return SVA_ERR_UNSUPPORTED;
  if (d->t0 > (1 << 24)) return SVA_ERR_UNSUPPORTED;
  if (d->rope) {
    if (d->rope_dt < 0 || d->rope_dh < 0 || d->rope_dw < 0) return SVA_ERR_UNSUPPORTED;
    if ((d->rope_dt | d->rope_dh | d->rope_dw) & 1) return SVA_ERR_UNSUPPORTED;
    if (d->rope_dt + d->rope_dh + d->rope_dw != d->d) return SVA_ERR_UNSUPPORTED;
    if (!(d->rope_base > 0.f) || d->rope_base > 3.0e38f) return SVA_ERR_UNSUPPORTED;
    const long long entries = (long long)d->frames_per_block * (d->rope_dt / 2) +
                              (long long)d->Hs * (d->rope_dh / 2) + (long long)d->Ws * (d->rope_dw / 2);
    if (entries > kMaxTableEntries) return SVA_ERR_UNSUPPORTED;
    // packed token coordinates: frame-in-block, h and w in 10 bits each
    if (d->frames_per_block > 1024 || d->Hs > 1024 || d->Ws > 1024) return SVA_ERR_UNSUPPORTED;
  }
  return SVA_OK;
}

// Workspace layout for a reduction grid of at most max_red_wg workgroups:
// arrival counters, then the partials (a piece of workgroup g and block c
// sits in slot g + c, so max_red_wg + B*H*nb slots always suffice), then the
// prefix operands and Z_c; every region 256-byte aligned.
void layout_workspace(Plan* p, long long max_red_wg) {
  const size_t E = (size_t)p->D * p->D + p->D;
  const size_t esz = p->bf16 ? 2 : 4;
  size_t off = 0;
  p->off_counters = off;  // B*H arrival counters of the folded prefix: zero between calls
  off = align256(off + (size_t)p->BH * sizeof(unsigned));
  p->off_partials = off;
  off = align256(off + (size_t)(max_red_wg + (long long)p->BH * p->nb) * E * sizeof(float));
  p->off_frags = off;
  off = align256(off + (size_t)p->BH * p->nb * p->D * p->D * esz);
  p->off_zc = off;
  off = align256(off + (size_t)p->BH * p->nb * p->D * sizeof(float));
  p->off_frags_lo = off;  // the backward's remainders of the operands (bf16)
  off = align256(off + (p->bf16 ? (size_t)p->BH * p->nb * p->D * p->D * 2 : 0));
  p->ws_bytes = off;
}

Plan make_plan(const sva_desc* d) {
  Plan p;
  memset(&p, 0, sizeof(p));
  p.BH = d->B * d->H;
  p.D = d->d;
  const int HW = d->Hs * d->Ws;
  p.N = d->T * HW;
  p.Nb = d->frames_per_block * HW;
  p.nb = d->T / d->frames_per_block;
  p.bf16 = d->dtype == SVA_BF16;
  p.rope = d->rope != 0;
  if (!p.rope) {
    p.rope_mode = 0;
  } else {
    const int all = d->rope_dt | d->rope_dh | d->rope_dw;
    p.rope_mode = (all & 7) == 0 ? 3 : (all & 3) == 0 ? 2 : 1;
  }
  p.geo.N = p.N;
  p.geo.Nb = p.Nb;
  p.geo.nb = p.nb;
  p.geo.BH = p.BH;
  p.geo.T = d->T;
  p.geo.Hs = d->Hs;
  p.geo.Ws = d->Ws;
  p.geo.fHW = make_fastdiv((uint32_t)HW);
  p.geo.fWs = make_fastdiv((uint32_t)d->Ws);
  if (p.rope) {
    RopeArgs& ra = p.ra;
    ra.dt = d->rope_dt;
    ra.dh = d->rope_dh;
    ra.dw = d->rope_dw;
    ra.off_h = d->frames_per_block * (ra.dt / 2);
    ra.off_w = ra.off_h + d->Hs * (ra.dh / 2);
    ra.n_entries = ra.off_w + d->Ws * (ra.dw / 2);
    ra.t0 = d->t0;
    ra.F = d->frames_per_block;
    ra.fht = make_fastdiv((uint32_t)(ra.dt / 2 > 0 ? ra.dt / 2 : 1));
    ra.fhh = make_fastdiv((uint32_t)(ra.dh / 2 > 0 ? ra.dh / 2 : 1));
    ra.fhw = make_fastdiv((uint32_t)(ra.dw / 2 > 0 ? ra.dw / 2 : 1));
    const double two_pi = 6.283185307179586476925286766559;
    int p_idx = 0;
    const int widths[3] = {ra.dt, ra.dh, ra.dw};
    for (int ax = 0; ax < 3; ++ax)
      for (int i = 0; i < widths[ax] / 2; ++i)
        ra.inv_rev[p_idx++] = __builtin_pow((double)d->rope_base, -2.0 * i / widths[ax]) / two_pi;
    p.tab_bytes = (size_t)ra.n_entries * sizeof(float2);
  }
  // The prefix folded into the reduction saves the scan launch but makes
  // every reduction workgroup wait for its device-scope stores and atomic,
  // and leaves one workgroup per sequence to read all of that sequence's
  // pieces.  Measured on MI355X it is slower for short sequences (one block
  // of 16 heads: 35.7 against 27.8 us per step; 720p: 125.7 against 110.2
  // us) and slightly faster for long ones (80 blocks: 1214.9 against 1223.6
  // us), where the scan kernel's own read of the partials is large.
  p.fold = p.nb >= kFoldMinBlocks;
  const long long total = (long long)p.BH * p.N;
  // Grids are fixed at launch from the device's occupancy (plan_grids); the
  // workspace is sized for the largest reduce grid.  Piece (g, block) of the
  // reduce lives in slot g + block, so G + B*H*nb slots always suffice.
  p.red = make_split(total, kRedWorkgroupsMax, &p.G_red, p.Nb);
  p.app = make_split(total, kAppWorkgroupsMax, &p.G_app, p.Nb);
  layout_workspace(&p, kRedWorkgroupsMax);
  const size_t esz = p.bf16 ? 2 : 4;
  p.states_lo = align256((size_t)p.BH * p.nb * p.D * p.D * esz);
  p.states_zc = p.states_lo + (p.bf16 ? align256((size_t)p.BH * p.nb * p.D * p.D * 2) : 0);
  p.states_bytes = p.states_zc + align256((size_t)p.BH * p.nb * p.D * sizeof(float));
  return p;
}

// The reduction; with `fold` non-null it also forms the prefix (FoldArgs).
template <bool BF16, int D, int ROPE>
hipError_t launch_reduce(const Plan& p, const void* k, const void* v, float* partials, hipStream_t st,
                         const FoldArgs* fold = nullptr) {
  Geo geo = p.geo;
  SplitArgs sp = p.red;
  RopeArgs ra = p.ra;
  FoldArgs fa = fold ? *fold : FoldArgs{};
  void* args[] = {(void*)&k, (void*)&v, (void*)&partials, &geo, &sp, &ra, &fa};
  constexpr int RM = ROPE == 3 ? 2 : ROPE;
  // bf16 without the folded prefix: 4-wave workgroups, two per CU on
  // block-aligned ranges (448 of them at 480p and 720p, against 224 or 256
  // of 8 waves: the reduction 25.7 -> 24.9 us at 480p, 54.7 -> 54.2 us at
  // 720p), and one per CU for one-block calls, where a range of a few
  // hundred tokens would give 8 waves about one step each (plan_grids_t).
  // Their cross-wave sum adds 4 tiles instead of 8.
  const bool small = BF16 && !fold;
  const void* fn = fold ? (const void*)&sva_reduce_kernel<BF16, D, RM, true>
                 : small ? (const void*)&sva_reduce_kernel<BF16, D, RM, false, 256>
                        : (const void*)&sva_reduce_kernel<BF16, D, RM, false>;
  return hipLaunchKernel(fn, dim3(p.G_red), dim3(small ? 256 : red_threads<BF16>()), args, ROPE ? p.tab_bytes : 0, st);
}

template <bool BF16, int D>
hipError_t launch_scan(const Plan& p, const float* partials, const float* S0, const float* z0,
                       float* S_out, float* z_out, void* frags, float* zc, bool write_frags,
                       hipStream_t st, bool reverse = false, long long L = 0, void* frags_lo = nullptr) {
  ScanArgs a;
  a.nb = p.nb;
  // the split of the kernel that wrote the partials: the reduction's, or
  // (L given) a flat split of L tokens per workgroup
  a.Nb = L ? p.Nb : p.red.Nbp;
  a.L = L ? L : p.red.L;
  a.cpl = (p.nb + kScanLanes - 1) / kScanLanes;
  a.has_init = S0 != nullptr;
  a.write_frags = write_frags;
  a.write_final = S_out != nullptr;
  a.reverse = reverse;
  void* args[] = {(void*)&partials, (void*)&S0, (void*)&z0, (void*)&S_out, (void*)&z_out,
                  (void*)&frags, (void*)&zc, (void*)&frags_lo, &a};
  constexpr int groups = (D * D + D) / 4;
  return hipLaunchKernel((const void*)&sva_scan_kernel<BF16, D>,
                         dim3((groups + kScanElems - 1) / kScanElems, p.BH), dim3(kThreads), args, 0, st);
}

template <bool BF16, int D, int ROPE>
hipError_t launch_apply(const Plan& p, const void* q, void* out, const void* frags, const float* zc,
                        float eps, hipStream_t st) {
  Geo geo = p.geo;
  SplitArgs sp = p.app;
  RopeArgs ra = p.ra;
  void* args[] = {(void*)&q, (void*)&out, (void*)&frags, (void*)&zc, &geo, &sp, &ra, &eps};
  return hipLaunchKernel((const void*)&sva_apply_kernel<BF16, D, (!BF16 && ROPE == 3 ? 2 : ROPE)>, dim3(p.G_app), dim3(app_threads<BF16>()),
                         args, ROPE ? p.tab_bytes : 0, st);
}

template <bool BF16, int D, int ROPE>
hipError_t launch_prep(const Plan& p, const void* x, float* xr, float* xphi, hipStream_t st) {
  Geo geo = p.geo;
  RopeArgs ra = p.ra;
  void* args[] = {(void*)&x, (void*)&xr, (void*)&xphi, &geo, &ra};
  return hipLaunchKernel((const void*)&sva_prep_kernel<BF16, D, (ROPE == 3 ? 2 : ROPE)>,
                         dim3((p.Nb + kThreads - 1) / kThreads, p.nb, p.BH), dim3(kThreads), args,
                         ROPE ? p.tab_bytes : 0, st);
}

// Backward launchers (bf16 only; BF16 is always true where they are used).
template <bool BF16, int D, int ROPE>
hipError_t launch_bwd_out(const Plan& p, const void* q, const void* dout, void* dq, float* partials,
                          const void* frags, const void* frags_lo, const float* zc, float eps, hipStream_t st) {
  static_assert(BF16, "the backward runs on bf16 inputs");
  Geo geo = p.geo;
  SplitArgs sp = p.bwd;
  RopeArgs ra = p.ra;
  void* args[] = {(void*)&q, (void*)&dout, (void*)&dq, (void*)&partials, (void*)&frags, (void*)&frags_lo,
                  (void*)&zc, &geo, &sp, &ra, &eps};
  return hipLaunchKernel((const void*)&sva_bwd_out_kernel<D, ROPE>, dim3(p.G_bwd_out),
                         dim3(kThreads), args, ROPE ? p.tab_bytes : 0, st);
}

template <bool BF16, int D, int ROPE>
hipError_t launch_bwd_kv(const Plan& p, const void* k, const void* v, void* dk, void* dv, const void* gfrags,
                         const float* gc, hipStream_t st) {
  static_assert(BF16, "the backward runs on bf16 inputs");
  Geo geo = p.geo;
  SplitArgs sp = p.bwd_kv;
  RopeArgs ra = p.ra;
  void* args[] = {(void*)&k, (void*)&v, (void*)&dk, (void*)&dv, (void*)&gfrags, (void*)&gc, &geo, &sp, &ra};
  return hipLaunchKernel((const void*)&sva_bwd_kv_kernel<D, ROPE>, dim3(p.G_bwd_kv), dim3(kThreads), args,
                         ROPE ? p.tab_bytes : 0, st);
}

// Template dispatch over (dtype, d, RoPE mode 0 none / 1 general / 2 paired
// / 3 grouped).
#define SVA_DISPATCH_R(P, FN, B, DD, ...)                                              \
  ((P).rope_mode == 3   ? FN<B, DD, 3>(__VA_ARGS__)                                    \
   : (P).rope_mode == 2 ? FN<B, DD, 2>(__VA_ARGS__)                                    \
   : (P).rope_mode == 1 ? FN<B, DD, 1>(__VA_ARGS__)                                    \
                        : FN<B, DD, 0>(__VA_ARGS__))
#define SVA_DISPATCH(P, FN, ...)                                                         \
  ((P).bf16 ? ((P).D == 64 ? SVA_DISPATCH_R(P, FN, true, 64, __VA_ARGS__)                \
                           : SVA_DISPATCH_R(P, FN, true, 32, __VA_ARGS__))               \
            : ((P).D == 64 ? SVA_DISPATCH_R(P, FN, false, 64, __VA_ARGS__)               \
                           : SVA_DISPATCH_R(P, FN, false, 32, __VA_ARGS__)))

#define SVA_DISPATCH2(P, FN, ...)                                                        \
  ((P).bf16 ? ((P).D == 64 ? FN<true, 64>(__VA_ARGS__) : FN<true, 32>(__VA_ARGS__))      \
            : ((P).D == 64 ? FN<false, 64>(__VA_ARGS__) : FN<false, 32>(__VA_ARGS__)))

template <bool BF16, int D, int ROPE>
int plan_grids_t(Plan* p) {
  const long long total = (long long)p->BH * p->N;
  const size_t lds = ROPE ? p->tab_bytes : 0;
  const bool small = BF16 && !p->fold;
  const void* red_fn = p->fold ? (const void*)&sva_reduce_kernel<BF16, D, (ROPE == 3 ? 2 : ROPE), true>
                     : small ? (const void*)&sva_reduce_kernel<BF16, D, (ROPE == 3 ? 2 : ROPE), false, 256>
                               : (const void*)&sva_reduce_kernel<BF16, D, (ROPE == 3 ? 2 : ROPE), false>;
  long long r = resident_workgroups(red_fn, small ? 256 : red_threads<BF16>(), lds);
  if (small && p->nb == 1) r = device_cus();  // one block: one 4-wave workgroup per CU (as measured)
  const long long a = resident_workgroups((const void*)&sva_apply_kernel<BF16, D, (!BF16 && ROPE == 3 ? 2 : ROPE)>, app_threads<BF16>(), lds);
  const long long r_max = r < kRedWorkgroupsMax ? r : kRedWorkgroupsMax;
  const long long a_max = a < kAppWorkgroupsMax ? a : kAppWorkgroupsMax;
  plan_forward_splits(total, (long long)p->BH * p->nb, p->Nb, r_max, a_max, device_cus(), &p->red, &p->G_red,
                      &p->app, &p->G_app);
  return 0;
}

void plan_grids(Plan* p) { (void)SVA_DISPATCH(*p, plan_grids_t, p); }

template <bool BF16, int D, int ROPE>
int plan_bwd_grids_t(Plan* p) {
  const long long total = (long long)p->BH * p->N;
  const size_t lds = ROPE ? p->tab_bytes : 0;
  const long long a = resident_workgroups((const void*)&sva_bwd_out_kernel<D, ROPE>, kThreads, lds);
  const long long b = resident_workgroups((const void*)&sva_bwd_kv_kernel<D, ROPE>, kThreads, lds);
  // its partials use the reduction's slots: at most kRedWorkgroupsMax pieces
  p->bwd = make_split(total, a < kRedWorkgroupsMax ? a : kRedWorkgroupsMax, &p->G_bwd_out, p->Nb);
  p->bwd_kv = make_split(total, b < kAppWorkgroupsMax ? b : kAppWorkgroupsMax, &p->G_bwd_kv, p->Nb);
  return 0;
}

void plan_bwd_grids(Plan* p) {
  (void)(p->D == 64 ? SVA_DISPATCH_R(*p, plan_bwd_grids_t, true, 64, p)
                    : SVA_DISPATCH_R(*p, plan_bwd_grids_t, true, 32, p));
}

size_t qkv_bytes(const Plan& p) { return (size_t)p.BH * p.N * p.D * (p.bf16 ? 2 : 4); }

sva_status check_common(const sva_desc* d, bool one_block, Plan* p) {
  sva_status s = validate_desc(d, one_block);
  if (s != SVA_OK) return s;
  *p = make_plan(d);
  return SVA_OK;
}

// Pointer checks of the forward (before any launch).
sva_status check_fwd_pointers(const Plan& p, const void* q, const void* k, const void* v, const void* out,
                              const float* S0, const float* z0, const float* S_out, const float* z_out) {
  if (!q || !k || !v || !out) return SVA_ERR_INVALID_ARG;
  if (!is_aligned16(q) || !is_aligned16(k) || !is_aligned16(v) || !is_aligned16(out))
    return SVA_ERR_INVALID_ARG;
  if ((S0 == nullptr) != (z0 == nullptr) || (S_out == nullptr) != (z_out == nullptr))
    return SVA_ERR_INVALID_ARG;
  if ((S0 && (!is_aligned16(S0) || !is_aligned16(z0))) ||
      (S_out && (!is_aligned16(S_out) || !is_aligned16(z_out))))
    return SVA_ERR_INVALID_ARG;
  const size_t nbytes = qkv_bytes(p);
  if (overlaps(out, nbytes, q, nbytes) || overlaps(out, nbytes, k, nbytes) ||
      overlaps(out, nbytes, v, nbytes))
    return SVA_ERR_INVALID_ARG;
  return SVA_OK;
}

// The forward's kernels for plan p (grids set) on the workspace at wsb.
sva_status launch_fwd(const Plan& p, const void* q, const void* k, const void* v, void* out, const float* S0,
                      const float* z0, float* S_out, float* z_out, char* wsb, int stages, void* states,
                      float eps, hipStream_t st) {
  float* partials = (float*)(wsb + p.off_partials);
  // the prefix states go to the caller's buffer when it keeps them
  void* frags = states ? states : (void*)(wsb + p.off_frags);
  float* zc = states ? (float*)((char*)states + p.states_zc) : (float*)(wsb + p.off_zc);
  // the backward takes S_c as two bf16 parts (kept states only)
  void* frags_lo = states && p.bf16 ? (void*)((char*)states + p.states_lo) : nullptr;
  if (p.fold) {
    const FoldArgs fa{(unsigned*)(wsb + p.off_counters), S0, z0, S_out, z_out, frags, zc};
    if ((stages & SVA_STAGE_REDUCE) && SVA_DISPATCH(p, launch_reduce, p, k, v, partials, st, &fa) != hipSuccess)
      return SVA_ERR_HIP;
  } else {
    if ((stages & SVA_STAGE_REDUCE) && SVA_DISPATCH(p, launch_reduce, p, k, v, partials, st) != hipSuccess)
      return SVA_ERR_HIP;
    if ((stages & SVA_STAGE_SCAN) &&
        SVA_DISPATCH2(p, launch_scan, p, partials, S0, z0, S_out, z_out, frags, zc, true, st, false, 0,
                      frags_lo) != hipSuccess)
      return SVA_ERR_HIP;
  }
  if ((stages & SVA_STAGE_APPLY) && SVA_DISPATCH(p, launch_apply, p, q, out, frags, zc, eps, st) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

sva_status run_fwd(const sva_desc* desc, const void* q, const void* k, const void* v, void* out,
                   const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                   size_t ws_bytes, void* stream, int stages = SVA_STAGE_ALL, void* states = nullptr) {
  Plan p;
  sva_status s = check_common(desc, false, &p);
  if (s != SVA_OK) return s;
  if ((s = check_fwd_pointers(p, q, k, v, out, S0, z0, S_out, z_out)) != SVA_OK) return s;
  if (!ws || ws_bytes < p.ws_bytes || !is_aligned16(ws)) return SVA_ERR_WORKSPACE;
  if (states && !is_aligned16(states)) return SVA_ERR_INVALID_ARG;
  if (stages < 1 || stages > SVA_STAGE_ALL) return SVA_ERR_INVALID_ARG;
  // kept states carry the operands' bf16 remainders, which the scan kernel
  // writes (the prefix folded into the reduction forms only the operands)
  if (states) p.fold = false;
  plan_grids(&p);
  return launch_fwd(p, q, k, v, out, S0, z0, S_out, z_out, (char*)ws, stages, states, desc->eps,
                    (hipStream_t)stream);
}

sva_status run_bwd(const sva_desc* desc, const void* q, const void* k, const void* v, const void* dout,
                   const float* S0, const float* z0, const float* dS_out, const float* dz_out, void* dq,
                   void* dk, void* dv, float* dS0, float* dz0, const void* states, void* ws, size_t ws_bytes,
                   void* stream) {
  Plan p;
  sva_status s = check_common(desc, false, &p);
  if (s != SVA_OK) return s;
  if (!p.bf16) return SVA_ERR_UNSUPPORTED;
  const void* in[] = {q, k, v, dout};
  void* grads[] = {dq, dk, dv};
  for (const void* x : in)
    if (!x || !is_aligned16(x)) return SVA_ERR_INVALID_ARG;
  for (void* x : grads)
    if (!x || !is_aligned16(x)) return SVA_ERR_INVALID_ARG;
  if ((S0 == nullptr) != (z0 == nullptr) || (dS_out == nullptr) != (dz_out == nullptr) ||
      (dS0 == nullptr) != (dz0 == nullptr))
    return SVA_ERR_INVALID_ARG;
  const float* st_ptr[] = {S0, z0, dS_out, dz_out, dS0, dz0};
  for (const float* x : st_ptr)
    if (x && !is_aligned16(x)) return SVA_ERR_INVALID_ARG;
  const size_t nbytes = qkv_bytes(p);
  for (int i = 0; i < 3; ++i) {
    for (const void* x : in)
      if (overlaps(grads[i], nbytes, x, nbytes)) return SVA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (overlaps(grads[i], nbytes, grads[j], nbytes)) return SVA_ERR_INVALID_ARG;
  }
  if (!ws || ws_bytes < p.ws_bytes || !is_aligned16(ws)) return SVA_ERR_WORKSPACE;
  if (states && !is_aligned16(states)) return SVA_ERR_INVALID_ARG;

  p.fold = false;  // the backward recomputes the prefix with the scan kernel
  plan_grids(&p);
  plan_bwd_grids(&p);
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  float* partials = (float*)(wsb + p.off_partials);
  void* frags = wsb + p.off_frags;
  float* zc = (float*)(wsb + p.off_zc);
#define SVA_BWD(FN, ...) (p.D == 64 ? SVA_DISPATCH_R(p, FN, true, 64, __VA_ARGS__) : SVA_DISPATCH_R(p, FN, true, 32, __VA_ARGS__))
  // The forward's prefix states: saved by sva_lin_attn_fwd_save, or
  // recomputed here (reduction and scan of the forward) into the workspace.
  const void* sfrags = frags;
  const void* sfrags_lo = wsb + p.off_frags_lo;
  const float* szc = zc;
  if (states) {
    sfrags = states;
    sfrags_lo = (const char*)states + p.states_lo;
    szc = (const float*)((const char*)states + p.states_zc);
  } else {
    void* lo = wsb + p.off_frags_lo;
    if (SVA_BWD(launch_reduce, p, k, v, partials, st) != hipSuccess) return SVA_ERR_HIP;
    if ((p.D == 64 ? launch_scan<true, 64>(p, partials, S0, z0, nullptr, nullptr, frags, zc, true, st, false, 0, lo)
                   : launch_scan<true, 32>(p, partials, S0, z0, nullptr, nullptr, frags, zc, true, st, false, 0,
                                           lo)) != hipSuccess)
      return SVA_ERR_HIP;
  }
  if (SVA_BWD(launch_bwd_out, p, q, dout, dq, partials, sfrags, sfrags_lo, szc, desc->eps, st) != hipSuccess)
    return SVA_ERR_HIP;
  if ((p.D == 64 ? launch_scan<true, 64>(p, partials, dS_out, dz_out, dS0, dz0, frags, zc, true, st, true,
                                         p.bwd.L)
                 : launch_scan<true, 32>(p, partials, dS_out, dz_out, dS0, dz0, frags, zc, true, st, true,
                                         p.bwd.L)) != hipSuccess)
    return SVA_ERR_HIP;
  if (SVA_BWD(launch_bwd_kv, p, k, v, dk, dv, frags, zc, st) != hipSuccess) return SVA_ERR_HIP;
#undef SVA_BWD
  return SVA_OK;
}

// Projection + attention with k and v reduced inside the projection.  The
// ranges of the fused kernel take the place of the reduction's workgroup
// ranges: L tokens each, L dividing the block's token count, so that the
// scan finds piece (g, block) at slot g + block exactly as it does for the
// reduction.
struct ProjPlan {
  Plan p;
  long long L, G;
  size_t off_partials, off_frags, off_zc, bytes;
};

sva_status plan_proj_fwd(const sva_desc* a, const sva_proj_desc* pd, ProjPlan* pp) {
  sva_status s = check_common(a, false, &pp->p);
  if (s != SVA_OK) return s;
  const Plan& p = pp->p;
  if (!pd) return SVA_ERR_INVALID_ARG;
  if (!p.bf16 || p.D != 64) return SVA_ERR_UNSUPPORTED;
  if (pd->B != a->B || pd->H != a->H || pd->d != a->d || pd->N != p.N) return SVA_ERR_INVALID_ARG;
  if (a->H % 2 != 0 || pd->C % 256 != 0 || pd->C < 256) return SVA_ERR_UNSUPPORTED;
  if (p.rope && (a->rope_dt % 2 != 0 || a->rope_dh % 2 != 0)) return SVA_ERR_UNSUPPORTED;
  // Range length L: a divisor of the block length (a range never straddles
  // a block), chosen for the k/v kernel's occupancy.  That kernel runs one
  // workgroup per (range, head pair), two per CU, each a loop over ceil(L/64)
  // token tiles; with 256 CUs (512 slots) the estimated time is
  // ceil(workgroups / 512) rounds of ceil(L/64) tiles, plus the partials'
  // write and the scan's read of them (about 1e8 bytes per tile's time).
  // Ties go to the longer range (fewer partials).
  long long L = 1;
  double best = 0.0;
  const long long pairs = a->H / 2;
  for (long long cand = p.Nb < 2048 ? p.Nb : 2048; cand >= 1; --cand) {
    if (p.Nb % cand != 0) continue;
    const long long ranges = (long long)a->B * (p.N / cand);
    const long long wgs = (ranges + 7) / 8 * 8 * pairs;
    const double cost = (double)((wgs + 511) / 512) * (double)((cand + 63) / 64) +
                        (double)ranges * a->H * (p.D * p.D + p.D) * 8.0 / 1e8;
    if (L == 1 || cost < best) {
      L = cand;
      best = cost;
    }
  }
  if (pd->range_tokens != 0) {  // the caller's range length
    const long long v = pd->range_tokens;
    if (v <= 0 || v > p.Nb || p.Nb % v != 0) return SVA_ERR_INVALID_ARG;
    L = v;
  }
  pp->L = L;
  const long long total = (long long)p.BH * p.N;
  pp->G = total / L;
  if (pp->G + (long long)p.BH * p.nb >= (1LL << 31) / (p.D * p.D + p.D)) return SVA_ERR_UNSUPPORTED;
  const size_t E = (size_t)p.D * p.D + p.D;
  size_t off = 0;
  pp->off_partials = off;
  off = align256(off + (size_t)(pp->G + (long long)p.BH * p.nb) * E * sizeof(float));
  pp->off_frags = off;
  off = align256(off + (size_t)p.BH * p.nb * p.D * p.D * 2);
  pp->off_zc = off;
  off = align256(off + (size_t)p.BH * p.nb * p.D * sizeof(float));
  pp->bytes = off;
  return SVA_OK;
}

// x: bf16 activations [B, N, C], or with w4a4 their MXFP4 form (codes, then
// scales, as sva_mxfp4_quant_acts writes them).
sva_status run_proj_fwd(const sva_desc* a, const sva_proj_desc* pd, const void* x, const void* wpack,
                        const float* bias, void* out, const float* S0, const float* z0, float* S_out,
                        float* z_out, void* ws, size_t ws_bytes, void* stream, bool w4a4) {
  ProjPlan pp;
  sva_status s = plan_proj_fwd(a, pd, &pp);
  if (s != SVA_OK) return s;
  Plan& p = pp.p;
  if (!x || !wpack || !out) return SVA_ERR_INVALID_ARG;
  if (!is_aligned16(x) || !is_aligned16(wpack) || !is_aligned16(out) || (bias && !is_aligned16(bias)))
    return SVA_ERR_INVALID_ARG;
  if ((S0 == nullptr) != (z0 == nullptr) || (S_out == nullptr) != (z_out == nullptr))
    return SVA_ERR_INVALID_ARG;
  if ((S0 && (!is_aligned16(S0) || !is_aligned16(z0))) ||
      (S_out && (!is_aligned16(S_out) || !is_aligned16(z_out))))
    return SVA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < pp.bytes || !is_aligned16(ws)) return SVA_ERR_WORKSPACE;
  const size_t nbytes = qkv_bytes(p);
  const size_t M = (size_t)pd->B * pd->N;
  const size_t xbytes = w4a4 ? M * pd->C / 2 + M * pd->C / 32 : M * pd->C * 2;
  const size_t n_out = (size_t)3 * pd->H * pd->d;
  const size_t wbytes = n_out * pd->C / 2 + n_out * pd->C / 32;  // codes, then the scale words
  const size_t s_bytes = (size_t)p.BH * p.D * p.D * sizeof(float), z_bytes = (size_t)p.BH * p.D * sizeof(float);
  if (overlaps(out, nbytes, x, xbytes) || overlaps(out, nbytes, ws, ws_bytes) ||
      overlaps(out, nbytes, wpack, wbytes) || overlaps(ws, ws_bytes, x, xbytes) ||
      overlaps(ws, ws_bytes, wpack, wbytes) || (bias && overlaps(ws, ws_bytes, bias, n_out * sizeof(float))) ||
      (S_out && (overlaps(S_out, s_bytes, ws, ws_bytes) || overlaps(S_out, s_bytes, out, nbytes) ||
                 overlaps(z_out, z_bytes, ws, ws_bytes) || overlaps(z_out, z_bytes, out, nbytes))))
    return SVA_ERR_INVALID_ARG;
  char* wsb = (char*)ws;
  float* partials = (float*)(wsb + pp.off_partials);
  void* frags = wsb + pp.off_frags;
  float* zc = (float*)(wsb + pp.off_zc);
  hipStream_t st = (hipStream_t)stream;

  SvaKvReduceArgs ka;
  ka.B = pd->B;
  ka.N = pd->N;
  ka.C = pd->C;
  ka.H = pd->H;
  ka.Nb = p.Nb;
  ka.nb = p.nb;
  ka.L = (int)pp.L;
  ka.Hs = a->Hs;
  ka.Ws = a->Ws;
  ka.t0 = a->t0;
  ka.rope = p.rope ? 1 : 0;
  ka.dt = a->rope_dt;
  ka.dh = a->rope_dh;
  ka.rope_base = a->rope_base;
  if ((w4a4 ? sva_internal_kv_proj_reduce_w4a4(ka, x, wpack, bias, partials, st)
            : sva_internal_kv_proj_reduce(ka, x, wpack, bias, partials, st)) != hipSuccess)
    return SVA_ERR_HIP;
  plan_grids(&p);
  if (SVA_DISPATCH2(p, launch_scan, p, partials, S0, z0, S_out, z_out, frags, zc, true, st, false, pp.L) !=
      hipSuccess)
    return SVA_ERR_HIP;
  // q is projected inside the output pass, once the prefix exists
  if (sva_internal_q_proj_apply(ka, a->eps, w4a4, x, wpack, bias, frags, zc, out, st) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

}  // namespace

int sva_internal_resident_workgroups(const void* fn, int threads, size_t lds) {
  return resident_workgroups(fn, threads, lds);
}

// ---------------------------------------------------------------------------
// Scratch of sva_block_cache_apply_noalloc
//
// A file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  In host code the array's name is only a stand-in
// for the device symbol, never a device address; the address of each GPU's
// copy comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that pointer is handed to kernels.  Every call on a GPU
// shares that GPU's copy, so calls that overlap on one GPU race.  A one-block
// call forms its prefix with the scan kernel and writes every region it reads
// earlier in the same call (the reduction's pieces, then the prefix operands),
// so nothing in the array has to start at zero.
// ---------------------------------------------------------------------------

static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`.
sva_status device_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SVA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SVA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SVA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SVA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

const char* sva_status_string(int status) {
  switch (status) {
    case SVA_OK: return "ok";
    case SVA_ERR_INVALID_ARG: return "invalid argument (pointer, shape, alignment or overlap)";
    case SVA_ERR_UNSUPPORTED: return "unsupported configuration (dtype, head dim, RoPE split or grid size)";
    case SVA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SVA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int sva_version(void) { return 1; }

sva_status sva_lin_attn_fwd_workspace(const sva_desc* desc, size_t* bytes) {
  if (!bytes) return SVA_ERR_INVALID_ARG;
  Plan p;
  sva_status s = check_common(desc, false, &p);
  if (s != SVA_OK) return s;
  *bytes = p.ws_bytes;
  return SVA_OK;
}

sva_status sva_lin_attn_fwd(const sva_desc* desc, const void* q, const void* k, const void* v,
                            void* out, const float* S0, const float* z0, float* S_out,
                            float* z_out, void* ws, size_t ws_bytes, void* stream) {
  return run_fwd(desc, q, k, v, out, S0, z0, S_out, z_out, ws, ws_bytes, stream);
}

sva_status sva_proj_lin_attn_fwd_workspace(const sva_desc* attn, const sva_proj_desc* proj, size_t* bytes) {
  if (!bytes) return SVA_ERR_INVALID_ARG;
  ProjPlan pp;
  sva_status s = plan_proj_fwd(attn, proj, &pp);
  if (s != SVA_OK) return s;
  *bytes = pp.bytes;
  return SVA_OK;
}

sva_status sva_proj_lin_attn_fwd(const sva_desc* attn, const sva_proj_desc* proj, const void* x,
                                 const void* wpack, const float* bias, void* out, const float* S0,
                                 const float* z0, float* S_out, float* z_out, void* ws, size_t ws_bytes,
                                 void* stream) {
  return run_proj_fwd(attn, proj, x, wpack, bias, out, S0, z0, S_out, z_out, ws, ws_bytes, stream, false);
}

sva_status sva_proj_lin_attn_fwd_w4a4(const sva_desc* attn, const sva_proj_desc* proj, const void* xq,
                                      const void* wpack, const float* bias, void* out, const float* S0,
                                      const float* z0, float* S_out, float* z_out, void* ws, size_t ws_bytes,
                                      void* stream) {
  return run_proj_fwd(attn, proj, xq, wpack, bias, out, S0, z0, S_out, z_out, ws, ws_bytes, stream, true);
}

sva_status sva_lin_attn_fwd_stages(const sva_desc* desc, const void* q, const void* k, const void* v,
                                   void* out, const float* S0, const float* z0, float* S_out,
                                   float* z_out, void* ws, size_t ws_bytes, void* stream, int stages) {
  return run_fwd(desc, q, k, v, out, S0, z0, S_out, z_out, ws, ws_bytes, stream, stages);
}

sva_status sva_lin_attn_bwd_workspace(const sva_desc* desc, size_t* bytes) {
  if (!bytes) return SVA_ERR_INVALID_ARG;
  Plan p;
  sva_status s = check_common(desc, false, &p);
  if (s != SVA_OK) return s;
  if (!p.bf16) return SVA_ERR_UNSUPPORTED;
  *bytes = p.ws_bytes;
  return SVA_OK;
}

sva_status sva_lin_attn_bwd(const sva_desc* desc, const void* q, const void* k, const void* v,
                            const void* dout, const float* S0, const float* z0,
                            const float* dS_out, const float* dz_out, const void* states, void* dq,
                            void* dk, void* dv, float* dS0, float* dz0, void* ws, size_t ws_bytes,
                            void* stream) {
  return run_bwd(desc, q, k, v, dout, S0, z0, dS_out, dz_out, dq, dk, dv, dS0, dz0, states, ws,
                 ws_bytes, stream);
}

sva_status sva_lin_attn_states_bytes(const sva_desc* desc, size_t* bytes) {
  if (!bytes) return SVA_ERR_INVALID_ARG;
  Plan p;
  sva_status s = check_common(desc, false, &p);
  if (s != SVA_OK) return s;
  *bytes = p.states_bytes;
  return SVA_OK;
}

sva_status sva_lin_attn_fwd_save(const sva_desc* desc, const void* q, const void* k, const void* v,
                                 void* out, const float* S0, const float* z0, float* S_out,
                                 float* z_out, void* states, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!states) return SVA_ERR_INVALID_ARG;
  return run_fwd(desc, q, k, v, out, S0, z0, S_out, z_out, ws, ws_bytes, stream, SVA_STAGE_ALL, states);
}

sva_status sva_block_cache_workspace(const sva_desc* desc, size_t* bytes) {
  if (!bytes) return SVA_ERR_INVALID_ARG;
  Plan p;
  sva_status s = check_common(desc, true, &p);
  if (s != SVA_OK) return s;
  *bytes = p.ws_bytes;
  return SVA_OK;
}

sva_status sva_block_cache_apply(const sva_desc* desc, const float* S, const float* z,
                                 const void* q, const void* k, const void* v, void* out,
                                 void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  sva_status s = check_common(desc, true, &p);
  if (s != SVA_OK) return s;
  if (!S || !z) return SVA_ERR_INVALID_ARG;
  return run_fwd(desc, q, k, v, out, S, z, nullptr, nullptr, ws, ws_bytes, stream);
}

sva_status sva_block_cache_apply_noalloc(const sva_desc* desc, const float* S, const float* z, const void* q,
                                         const void* k, const void* v, void* out, void* stream) {
  Plan p;
  sva_status s = check_common(desc, true, &p);
  if (s != SVA_OK) return s;
  if (!S || !z) return SVA_ERR_INVALID_ARG;
  if ((s = check_fwd_pointers(p, q, k, v, out, S, z, nullptr, nullptr)) != SVA_OK) return s;
  void* scr = nullptr;
  if ((s = device_scratch(&scr)) != SVA_OK) return s;
  plan_grids(&p);
  if (p.fold) return SVA_ERR_UNSUPPORTED;  // one block: the prefix is always the scan kernel's
  layout_workspace(&p, p.G_red);           // sized for this launch's reduction grid
  if (p.ws_bytes > kScratchBytes) return SVA_ERR_WORKSPACE;
  return launch_fwd(p, q, k, v, out, S, z, nullptr, nullptr, (char*)scr, SVA_STAGE_ALL, nullptr, desc->eps,
                    (hipStream_t)stream);
}

sva_status sva_block_cache_commit(const sva_desc* desc, float* S, float* z, const void* k,
                                  const void* v, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  sva_status s = check_common(desc, true, &p);
  if (s != SVA_OK) return s;
  if (!S || !z || !k || !v) return SVA_ERR_INVALID_ARG;
  if (!is_aligned16(S) || !is_aligned16(z) || !is_aligned16(k) || !is_aligned16(v))
    return SVA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < p.ws_bytes || !is_aligned16(ws)) return SVA_ERR_WORKSPACE;
  plan_grids(&p);
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  float* partials = (float*)(wsb + p.off_partials);
  if (p.fold) {
    const FoldArgs fa{(unsigned*)(wsb + p.off_counters), S, z, S, z, nullptr, nullptr};
    if (SVA_DISPATCH(p, launch_reduce, p, k, v, partials, st, &fa) != hipSuccess) return SVA_ERR_HIP;
  } else {
    if (SVA_DISPATCH(p, launch_reduce, p, k, v, partials, st) != hipSuccess) return SVA_ERR_HIP;
    if (SVA_DISPATCH2(p, launch_scan, p, partials, S, z, S, z, nullptr, nullptr, false, st) != hipSuccess)
      return SVA_ERR_HIP;
  }
  return SVA_OK;
}

sva_status sva_phi_rope_prep(const sva_desc* desc, const void* x, float* x_rot, float* x_phi,
                             void* stream) {
  Plan p;
  sva_status s = check_common(desc, false, &p);
  if (s != SVA_OK) return s;
  if (!x || !x_rot || !is_aligned16(x) || !is_aligned16(x_rot) || (x_phi && !is_aligned16(x_phi)))
    return SVA_ERR_INVALID_ARG;
  if (SVA_DISPATCH(p, launch_prep, p, x, x_rot, x_phi, (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

}  // extern "C"
