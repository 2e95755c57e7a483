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

#include "sva.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;          // 4 wavefronts of 64
constexpr int kMaxTableEntries = 5632; // RoPE cos/sin table, 44 KiB of LDS

// ---------------------------------------------------------------------------
// Small integer helpers
// ---------------------------------------------------------------------------

// n / d for 0 <= n < 2^31 as (umulhi(n, mul) + n) >> shift, constants from
// the round-up method (Granlund & Montgomery, "Division by invariant
// integers using multiplication", 1994).
struct FastDiv {
  uint32_t mul, shift, div;
};

FastDiv make_fastdiv(uint32_t d) {
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

// ---------------------------------------------------------------------------
// phi + 3D RoPE stage (shared by every kernel)
// ---------------------------------------------------------------------------

// RoPE layout for one call.  The cos/sin table lives in LDS as float2
// entries: [T rows x dt/2] for t (global frame t0 + row), then
// [Hs rows x dh/2] for h, then [Ws rows x dw/2] for w.
struct RopeArgs {
  int dt, dh, dw;
  int off_h, off_w, n_entries;
  int t0;
  int pad_;
  double inv_rev[32];  // base^(-2i/d_a) / (2 pi), indexed by global pair p
};

// Fill the table.  PRECISE (fp32 inputs): fp64 angle reduced to one turn,
// then an accurate single-precision sincos.  Otherwise (bf16 inputs): the
// same reduced angle through the hardware sine/cosine, far below bf16's
// rounding.
template <bool PRECISE>
__device__ void build_rope_table(float2* tab, const RopeArgs& ra) {
  const int ht = ra.dt >> 1, hh = ra.dh >> 1, hw = ra.dw >> 1;
  for (int e = threadIdx.x; e < ra.n_entries; e += blockDim.x) {
    int pos, p;
    if (e < ra.off_h) {
      int row = e / ht;
      p = e - row * ht;
      pos = ra.t0 + row;
    } else if (e < ra.off_w) {
      int x = e - ra.off_h;
      int row = x / hh;
      p = ht + (x - row * hh);
      pos = row;
    } else {
      int x = e - ra.off_w;
      int row = x / hw;
      p = ht + hh + (x - row * hw);
      pos = row;
    }
    double rv = (double)pos * ra.inv_rev[p];
    rv -= rint(rv);  // angle in turns, within [-1/2, 1/2]
    float c, s;
    if (PRECISE) {
      sincosf((float)(rv * 6.283185307179586), &s, &c);
    } else {
      s = __builtin_amdgcn_sinf((float)rv);  // sin(2 pi x)
      c = __builtin_amdgcn_cosf((float)rv);
    }
    tab[e] = make_float2(c, s);
  }
}

// Where the table row of global pair p starts, its row stride, and which
// coordinate (0: frame, 1: h, 2: w) selects the row.
struct PairLoc {
  int base, stride, axis;
};

__device__ __forceinline__ PairLoc pair_loc(int p, const RopeArgs& ra) {
  const int ht = ra.dt >> 1, hh = ra.dh >> 1;
  PairLoc r;
  if (p < ht) {
    r.base = p; r.stride = ht; r.axis = 0;
  } else if (p < ht + hh) {
    r.base = ra.off_h + (p - ht); r.stride = hh; r.axis = 1;
  } else {
    r.base = ra.off_w + (p - ht - hh); r.stride = ra.dw >> 1; r.axis = 2;
  }
  return r;
}

__device__ __forceinline__ int pair_entry(const PairLoc& pl, int frame, int h, int w) {
  const int pos = pl.axis == 0 ? frame : (pl.axis == 1 ? h : w);
  return pl.base + pos * pl.stride;
}

// phi = ReLU
__device__ __forceinline__ float relu(float x) { return x > 0.f ? x : 0.f; }

// Turn the pair (x, y) by the angle whose (cos, sin) is cs.
__device__ __forceinline__ void rotate(float& x, float& y, float2 cs) {
  const float xr = x * cs.x - y * cs.y;
  const float yr = x * cs.y + y * cs.x;
  x = xr;
  y = yr;
}

struct Coord {
  int frame, h, w;
};

__device__ __forceinline__ Coord decode(uint32_t n, const FastDiv& fHW, const FastDiv& fWs) {
  Coord c;
  c.frame = (int)fdiv(n, fHW);
  const uint32_t rem = n - (uint32_t)c.frame * fHW.div;
  c.h = (int)fdiv(rem, fWs);
  c.w = (int)(rem - (uint32_t)c.h * fWs.div);
  return c;
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

// Unpack `CNT` elements (bf16 pairs or fp32 words) into floats.
template <bool BF16, int CNT>
__device__ __forceinline__ void unpack(float* f, const uint32_t* w) {
#pragma unroll
  for (int i = 0; i < CNT; ++i) {
    if (BF16) f[i] = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
    else f[i] = __uint_as_float(w[i]);
  }
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
  FastDiv fHW, fWs;
};

struct SplitArgs {
  long long total;  // BH * N flattened tokens
  long long L;      // flattened tokens per workgroup
  int maxsub;       // most (b, h, block) pieces one workgroup range can touch
  int pad_;
};

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

template <bool BF16, int D, bool ROPE>
__global__ __launch_bounds__(kThreads) void sva_reduce_kernel(
    const void* __restrict__ kp, const void* __restrict__ vp, float* __restrict__ partials,
    Geo geo, SplitArgs sp, RopeArgs ra) {
  constexpr int FPL = D / 16;
  constexpr int NPAIR = FPL / 2;
  constexpr int E = D * D + D;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NW = FPL * ESZ / 4;  // 32-bit words per lane per token row piece

  extern __shared__ float2 tab[];
  __shared__ float red[D * D];
  __shared__ float zred[D];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int cg = lane & 15;
  const int tg = lane >> 4;

  PairLoc pl[NPAIR > 0 ? NPAIR : 1];
  if (ROPE) {
    build_rope_table<!BF16>(tab, ra);
#pragma unroll
    for (int pp = 0; pp < NPAIR; ++pp) pl[pp] = pair_loc(NPAIR * cg + pp, ra);
  }
  __syncthreads();

  const long long g0 = (long long)blockIdx.x * sp.L;
  const long long g1 = min(g0 + sp.L, sp.total);
  const long long first_bhc = g0 / geo.Nb;
  const char* kb = (const char*)kp;
  const char* vb = (const char*)vp;

  for (long long pos = g0; pos < g1;) {
    const long long bhc = pos / geo.Nb;
    const long long seg_end = min(g1, (bhc + 1) * (long long)geo.Nb);
    const int bh = (int)(bhc / geo.nb);
    const int c = (int)(bhc - (long long)bh * geo.nb);
    const int js = (int)(pos - bhc * geo.Nb);        // block-local token range
    const int je = (int)(seg_end - bhc * geo.Nb);
    const long long row0 = (long long)bh * geo.N + (long long)c * geo.Nb;  // token row of j = 0

    floatx4 acc[FPL][FPL];
#pragma unroll
    for (int r = 0; r < FPL; ++r)
#pragma unroll
      for (int s = 0; s < FPL; ++s) acc[r][s] = floatx4{0.f, 0.f, 0.f, 0.f};
    float zacc[FPL];
#pragma unroll
    for (int r = 0; r < FPL; ++r) zacc[r] = 0.f;

    for (int s0 = js + wave * 32; s0 < je; s0 += 4 * 32) {
      uint32_t kw[8][NW], vw[8][NW];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = s0 + 4 * e + tg;
        if (j < je) {
          const long long off = ((row0 + j) * D + FPL * cg) * ESZ;
          load_words<NW>(kw[e], kb + off);
          load_words<NW>(vw[e], vb + off);
        } else {
#pragma unroll
          for (int w = 0; w < NW; ++w) { kw[e][w] = 0u; vw[e][w] = 0u; }
        }
      }
      float kf[8][FPL];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        unpack<BF16, FPL>(kf[e], kw[e]);
#pragma unroll
        for (int r = 0; r < FPL; ++r) {
          kf[e][r] = relu(kf[e][r]);
          zacc[r] += kf[e][r];
        }
      }
      if (ROPE) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = min(s0 + 4 * e + tg, geo.Nb - 1);
          const Coord co = decode((uint32_t)(c * geo.Nb + j), geo.fHW, geo.fWs);
#pragma unroll
          for (int pp = 0; pp < NPAIR; ++pp) {
            const float2 cs = tab[pair_entry(pl[pp], co.frame, co.h, co.w)];
            rotate(kf[e][2 * pp], kf[e][2 * pp + 1], cs);
          }
        }
      }
      if (BF16) {
        u32x4 A[FPL], Bv[FPL];
#pragma unroll
        for (int r = 0; r < FPL; ++r)
#pragma unroll
          for (int m = 0; m < 4; ++m) A[r][m] = pack_bf16x2(kf[2 * m][r], kf[2 * m + 1][r]);
#pragma unroll
        for (int s = 0; s < FPL; ++s) {
          const uint32_t sel = (s & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
          for (int m = 0; m < 4; ++m)
            Bv[s][m] = __builtin_amdgcn_perm(vw[2 * m + 1][s >> 1], vw[2 * m][s >> 1], sel);
        }
#pragma unroll
        for (int r = 0; r < FPL; ++r)
#pragma unroll
          for (int s = 0; s < FPL; ++s) acc[r][s] = mfma_bf16(A[r], Bv[s], acc[r][s]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float vf[FPL];
          unpack<false, FPL>(vf, vw[e]);
#pragma unroll
          for (int r = 0; r < FPL; ++r)
#pragma unroll
            for (int s = 0; s < FPL; ++s) acc[r][s] = mfma_f32(kf[e][r], vf[s], acc[r][s]);
        }
      }
    }

    // Fixed-order reduction over the four lane groups and the four waves.
#pragma unroll
    for (int r = 0; r < FPL; ++r) {
      float z = zacc[r];
      z += __shfl_xor(z, 16);
      z += __shfl_xor(z, 32);
      zacc[r] = z;
    }
    for (int w = 0; w < kThreads / 64; ++w) {
      if (wave == w) {
#pragma unroll
        for (int r = 0; r < FPL; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* dst = red + (FPL * (4 * tg + i) + r) * D + FPL * cg;
#pragma unroll
            for (int s = 0; s < FPL; ++s) dst[s] = (w == 0) ? acc[r][s][i] : dst[s] + acc[r][s][i];
          }
        if (tg == 0) {
#pragma unroll
          for (int r = 0; r < FPL; ++r)
            zred[FPL * cg + r] = (w == 0) ? zacc[r] : zred[FPL * cg + r] + zacc[r];
        }
      }
      __syncthreads();
    }
    float* dst = partials + ((long long)blockIdx.x * sp.maxsub + (bhc - first_bhc)) * E;
    for (int e = tid; e < D * D; e += kThreads) dst[e] = red[e];
    for (int e = tid; e < D; e += kThreads) dst[D * D + e] = zred[e];
    __syncthreads();
    pos = seg_end;
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: inclusive prefix over blocks, fixed order
//
// One thread per state element (d*d entries of S, then d of z) per (b, h).
// Output-kernel A operand layout (the MFMA computes out^T = S^T qr^T):
//   bf16: fragment (rt, ks), lane l, slot e holds
//         S[FPLa*(l/16) + 8*ks + e][fo(rt, l%16)],   FPLa = d/4
//   fp32: fragment (rt, ks), lane l holds S[FPLa*(l/16) + ks][fo(rt, l%16)]
//   with fo(rt, r) = FPLa*(r/4) + 4*rt + r%4, so that accumulator rt of lane
//   l holds output features FPLa*(l/16) + 4*rt + (0..3).
// ---------------------------------------------------------------------------

struct ScanArgs {
  int nb, Nb;
  long long L;
  int maxsub;
  int has_init;     // S0/z0 given
  int write_frags;  // emit the output-kernel operands
  int write_final;  // emit S_out/z_out
};

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void sva_scan_kernel(
    const float* __restrict__ partials, const float* S0, const float* z0, float* S_out,
    float* z_out, void* __restrict__ frags, float* __restrict__ zc, ScanArgs a) {
  constexpr int E = D * D + D;
  constexpr int FPLa = D / 4;
  constexpr int NKS = BF16 ? D / 32 : D / 4;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= E) return;
  const bool in_S = e < D * D;

  int frag_off = 0;
  if (in_S) {
    const int fi = e / D, fo = e % D;
    const int g = fi / FPLa, wi = fi % FPLa;
    const int rem = fo % FPLa;
    const int rt = rem >> 2;
    const int lane = 16 * g + 4 * (fo / FPLa) + (rem & 3);
    if (BF16) frag_off = ((rt * NKS + (wi >> 3)) * 64 + lane) * 8 + (wi & 7);
    else frag_off = (rt * NKS + wi) * 64 + lane;
  }

  float acc = 0.f;
  if (a.has_init) acc = in_S ? S0[(long long)bh * D * D + e] : z0[(long long)bh * D + (e - D * D)];
  for (int c = 0; c < a.nb; ++c) {
    const long long bhc = (long long)bh * a.nb + c;
    const long long start = bhc * a.Nb;
    const long long gf = start / a.L, gl = (start + a.Nb - 1) / a.L;
    for (long long g = gf; g <= gl; ++g) {
      const long long slot = g * a.maxsub + (bhc - (g * a.L) / a.Nb);
      acc += partials[slot * E + e];
    }
    if (a.write_frags) {
      if (in_S) {
        if (BF16) ((__bf16*)frags)[bhc * D * D + frag_off] = (__bf16)acc;
        else ((float*)frags)[bhc * D * D + frag_off] = acc;
      } else {
        zc[bhc * D + (e - D * D)] = acc;
      }
    }
  }
  if (a.write_final) {
    if (in_S) S_out[(long long)bh * D * D + e] = acc;
    else z_out[(long long)bh * D + (e - D * D)] = acc;
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: output pass
//
// A wavefront handles 16-token tiles.  Lane l takes token l%16 of the tile
// and features FPLa*(l/16) .. +FPLa-1 of it (one contiguous 2*FPLa- or
// 4*FPLa-byte piece of the row), which is exactly its B-operand share of
// out^T = S^T qr^T.  The denominator phi q . Z is an fp32 dot over the
// lane's features plus two cross-lane adds; the lane then scales its
// accumulators and stores its contiguous piece of the output row.
// ---------------------------------------------------------------------------

template <bool BF16, int D, bool ROPE>
__global__ __launch_bounds__(kThreads) void sva_apply_kernel(
    const void* __restrict__ qp, void* __restrict__ outp, const void* __restrict__ frags,
    const float* __restrict__ zc, Geo geo, SplitArgs sp, RopeArgs ra, float eps) {
  constexpr int FPLa = D / 4;
  constexpr int NRT = D / 16;
  constexpr int NKS = BF16 ? D / 32 : D / 4;
  constexpr int NPAIR = FPLa / 2;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int NW = FPLa * ESZ / 4;
  constexpr int FRAG_U4 = D * D * ESZ / 16;

  extern __shared__ float2 tab[];
  __shared__ uint4 fstage[FRAG_U4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int row = lane & 15;

  PairLoc pl[NPAIR];
  if (ROPE) {
    build_rope_table<!BF16>(tab, ra);
#pragma unroll
    for (int pp = 0; pp < NPAIR; ++pp) pl[pp] = pair_loc(NPAIR * g + pp, ra);
  }

  const long long g0 = (long long)blockIdx.x * sp.L;
  const long long g1 = min(g0 + sp.L, sp.total);
  const char* qb = (const char*)qp;
  char* ob = (char*)outp;

  for (long long pos = g0; pos < g1;) {
    const long long bhc = pos / geo.Nb;
    const long long seg_end = min(g1, (bhc + 1) * (long long)geo.Nb);
    const int bh = (int)(bhc / geo.nb);
    const int c = (int)(bhc - (long long)bh * geo.nb);
    const int js = (int)(pos - bhc * geo.Nb);
    const int je = (int)(seg_end - bhc * geo.Nb);
    const long long row0 = (long long)bh * geo.N + (long long)c * geo.Nb;

    __syncthreads();  // previous segment done with fstage (and table built)
    {
      const uint4* src = (const uint4*)frags + bhc * FRAG_U4;
      for (int i = tid; i < FRAG_U4; i += kThreads) fstage[i] = src[i];
    }
    float z[FPLa];
    {
      const float* zsrc = zc + bhc * D + FPLa * g;
#pragma unroll
      for (int m = 0; m < FPLa; m += 4) {
        const float4 t = *(const float4*)(zsrc + m);
        z[m] = t.x; z[m + 1] = t.y; z[m + 2] = t.z; z[m + 3] = t.w;
      }
    }
    __syncthreads();

    u32x4 A16[BF16 ? NRT : 1][BF16 ? NKS : 1];
    float A32[BF16 ? 1 : NRT][BF16 ? 1 : NKS];
    if (BF16) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 t = fstage[(rt * NKS + ks) * 64 + lane];
          A16[rt][ks] = u32x4{t.x, t.y, t.z, t.w};
        }
    } else {
      const float* fs = (const float*)fstage;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) A32[rt][ks] = fs[(rt * NKS + ks) * 64 + lane];
    }

    for (int t0 = js + wave * 16; t0 < je; t0 += 4 * 16) {
      const int j = t0 + row;
      const bool valid = j < je;
      const long long off = ((row0 + j) * D + FPLa * g) * ESZ;
      uint32_t qw[NW];
      if (valid) load_words<NW>(qw, qb + off);
      else {
#pragma unroll
        for (int w = 0; w < NW; ++w) qw[w] = 0u;
      }
      float qf[FPLa];
      unpack<BF16, FPLa>(qf, qw);
      float den = 0.f;
#pragma unroll
      for (int m = 0; m < FPLa; ++m) {
        qf[m] = relu(qf[m]);
        den += qf[m] * z[m];
      }
      if (ROPE) {
        const Coord co = decode((uint32_t)(c * geo.Nb + min(j, geo.Nb - 1)), geo.fHW, geo.fWs);
#pragma unroll
        for (int pp = 0; pp < NPAIR; ++pp) {
          const float2 cs = tab[pair_entry(pl[pp], co.frame, co.h, co.w)];
          rotate(qf[2 * pp], qf[2 * pp + 1], cs);
        }
      }
      floatx4 acc[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (BF16) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          u32x4 b;
#pragma unroll
          for (int m = 0; m < 4; ++m) b[m] = pack_bf16x2(qf[8 * ks + 2 * m], qf[8 * ks + 2 * m + 1]);
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) acc[rt] = mfma_bf16(A16[rt][ks], b, acc[rt]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) acc[rt] = mfma_f32(A32[rt][ks], qf[ks], acc[rt]);
      }
      den += __shfl_xor(den, 16);
      den += __shfl_xor(den, 32);
      const float inv = 1.0f / (den + eps);
      if (valid) {
        uint32_t ow[NW];
        if (BF16) {
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            ow[2 * rt] = pack_bf16x2(acc[rt][0] * inv, acc[rt][1] * inv);
            ow[2 * rt + 1] = pack_bf16x2(acc[rt][2] * inv, acc[rt][3] * inv);
          }
        } else {
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) ow[4 * rt + i] = __float_as_uint(acc[rt][i] * inv);
        }
        store_words<NW>(ob + off, ow);
      }
    }
    pos = seg_end;
  }
}

// ---------------------------------------------------------------------------
// Standalone phi + RoPE stage (test entry point): one thread per token.
// ---------------------------------------------------------------------------

template <bool BF16, int D, bool ROPE>
__global__ __launch_bounds__(kThreads) void sva_prep_kernel(
    const void* __restrict__ xp, float* __restrict__ xr, float* __restrict__ xphi,
    long long total, int N, Geo geo, RopeArgs ra) {
  constexpr int ESZ = BF16 ? 2 : 4;
  extern __shared__ float2 tab[];
  if (ROPE) build_rope_table<!BF16>(tab, ra);
  __syncthreads();
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (t >= total) return;
  const int n = (int)(t % N);
  uint32_t w[D * ESZ / 4];
  load_words<D * ESZ / 4>(w, (const char*)xp + t * D * ESZ);
  float f[D];
  unpack<BF16, D>(f, w);
#pragma unroll
  for (int i = 0; i < D; ++i) f[i] = relu(f[i]);
  if (xphi) {
#pragma unroll
    for (int i = 0; i < D; i += 4) *(float4*)(xphi + t * D + i) = make_float4(f[i], f[i + 1], f[i + 2], f[i + 3]);
  }
  if (ROPE) {
    const Coord co = decode((uint32_t)n, geo.fHW, geo.fWs);
#pragma unroll
    for (int p = 0; p < D / 2; ++p) {
      const PairLoc pl = pair_loc(p, ra);
      rotate(f[2 * p], f[2 * p + 1], tab[pair_entry(pl, co.frame, co.h, co.w)]);
    }
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
  Geo geo;
  RopeArgs ra;
  SplitArgs red, app;
  int G_red, G_app;
  size_t tab_bytes;
  size_t off_partials, off_frags, off_zc, ws_bytes;
};

constexpr long long kRedWorkgroups = 512;   // 2 per CU on 256 CUs
constexpr long long kAppWorkgroups = 1024;  // 4 per CU on 256 CUs
constexpr long long kMinTokensPerWG = 256;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bn && y < x + an;
}

SplitArgs make_split(long long total, long long target_wg, int Nb, int* G_out) {
  long long G = target_wg;
  const long long g_min_tokens = (total + kMinTokensPerWG - 1) / kMinTokensPerWG;
  if (G > g_min_tokens) G = g_min_tokens;
  if (G < 1) G = 1;
  SplitArgs s;
  s.total = total;
  s.L = (total + G - 1) / G;
  G = (total + s.L - 1) / s.L;
  s.maxsub = (int)((s.L - 1) / Nb + 2);
  s.pad_ = 0;
  *G_out = (int)G;
  return s;
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
  if ((long long)d->B * d->H * N >= (1ll << 40)) return SVA_ERR_UNSUPPORTED;
  if (d->t0 > (1 << 24)) return SVA_ERR_UNSUPPORTED;
  if (d->rope) {
    if (d->rope_dt < 0 || d->rope_dh < 0 || d->rope_dw < 0) return SVA_ERR_UNSUPPORTED;
    if ((d->rope_dt | d->rope_dh | d->rope_dw) & 1) return SVA_ERR_UNSUPPORTED;
    if (d->rope_dt + d->rope_dh + d->rope_dw != d->d) return SVA_ERR_UNSUPPORTED;
    if (!(d->rope_base > 0.f) || d->rope_base > 3.0e38f) return SVA_ERR_UNSUPPORTED;
    const long long entries = (long long)d->T * (d->rope_dt / 2) +
                              (long long)d->Hs * (d->rope_dh / 2) + (long long)d->Ws * (d->rope_dw / 2);
    if (entries > kMaxTableEntries) return SVA_ERR_UNSUPPORTED;
  }
  return SVA_OK;
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
  p.geo.N = p.N;
  p.geo.Nb = p.Nb;
  p.geo.nb = p.nb;
  p.geo.BH = p.BH;
  p.geo.fHW = make_fastdiv((uint32_t)HW);
  p.geo.fWs = make_fastdiv((uint32_t)d->Ws);
  if (p.rope) {
    RopeArgs& ra = p.ra;
    ra.dt = d->rope_dt;
    ra.dh = d->rope_dh;
    ra.dw = d->rope_dw;
    ra.off_h = d->T * (ra.dt / 2);
    ra.off_w = ra.off_h + d->Hs * (ra.dh / 2);
    ra.n_entries = ra.off_w + d->Ws * (ra.dw / 2);
    ra.t0 = d->t0;
    const double two_pi = 6.283185307179586476925286766559;
    int p_idx = 0;
    const int widths[3] = {ra.dt, ra.dh, ra.dw};
    for (int ax = 0; ax < 3; ++ax)
      for (int i = 0; i < widths[ax] / 2; ++i)
        ra.inv_rev[p_idx++] = __builtin_pow((double)d->rope_base, -2.0 * i / widths[ax]) / two_pi;
    p.tab_bytes = (size_t)ra.n_entries * sizeof(float2);
  }
  const long long total = (long long)p.BH * p.N;
  p.red = make_split(total, kRedWorkgroups, p.Nb, &p.G_red);
  p.app = make_split(total, kAppWorkgroups, p.Nb, &p.G_app);
  const size_t E = (size_t)p.D * p.D + p.D;
  const size_t esz = p.bf16 ? 2 : 4;
  size_t off = 0;
  p.off_partials = off;
  off = align256(off + (size_t)p.G_red * p.red.maxsub * E * sizeof(float));
  p.off_frags = off;
  off = align256(off + (size_t)p.BH * p.nb * p.D * p.D * esz);
  p.off_zc = off;
  off = align256(off + (size_t)p.BH * p.nb * p.D * sizeof(float));
  p.ws_bytes = off;
  return p;
}

template <bool BF16, int D, bool ROPE>
hipError_t launch_reduce(const Plan& p, const void* k, const void* v, float* partials, hipStream_t st) {
  Geo geo = p.geo;
  SplitArgs sp = p.red;
  RopeArgs ra = p.ra;
  void* args[] = {(void*)&k, (void*)&v, (void*)&partials, &geo, &sp, &ra};
  return hipLaunchKernel((const void*)&sva_reduce_kernel<BF16, D, ROPE>, dim3(p.G_red), dim3(kThreads),
                         args, ROPE ? p.tab_bytes : 0, st);
}

template <bool BF16, int D>
hipError_t launch_scan(const Plan& p, const float* partials, const float* S0, const float* z0,
                       float* S_out, float* z_out, void* frags, float* zc, bool write_frags,
                       hipStream_t st) {
  ScanArgs a;
  a.nb = p.nb;
  a.Nb = p.Nb;
  a.L = p.red.L;
  a.maxsub = p.red.maxsub;
  a.has_init = S0 != nullptr;
  a.write_frags = write_frags;
  a.write_final = S_out != nullptr;
  void* args[] = {(void*)&partials, (void*)&S0, (void*)&z0, (void*)&S_out, (void*)&z_out,
                  (void*)&frags, (void*)&zc, &a};
  const int E = D * D + D;
  return hipLaunchKernel((const void*)&sva_scan_kernel<BF16, D>,
                         dim3((E + kThreads - 1) / kThreads, p.BH), dim3(kThreads), args, 0, st);
}

template <bool BF16, int D, bool ROPE>
hipError_t launch_apply(const Plan& p, const void* q, void* out, const void* frags, const float* zc,
                        float eps, hipStream_t st) {
  Geo geo = p.geo;
  SplitArgs sp = p.app;
  RopeArgs ra = p.ra;
  void* args[] = {(void*)&q, (void*)&out, (void*)&frags, (void*)&zc, &geo, &sp, &ra, &eps};
  return hipLaunchKernel((const void*)&sva_apply_kernel<BF16, D, ROPE>, dim3(p.G_app), dim3(kThreads),
                         args, ROPE ? p.tab_bytes : 0, st);
}

template <bool BF16, int D, bool ROPE>
hipError_t launch_prep(const Plan& p, const void* x, float* xr, float* xphi, hipStream_t st) {
  Geo geo = p.geo;
  RopeArgs ra = p.ra;
  long long total = (long long)p.BH * p.N;
  int N = p.N;
  void* args[] = {(void*)&x, (void*)&xr, (void*)&xphi, &total, &N, &geo, &ra};
  return hipLaunchKernel((const void*)&sva_prep_kernel<BF16, D, ROPE>,
                         dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), args,
                         ROPE ? p.tab_bytes : 0, st);
}

// Template dispatch over (dtype, d, rope).
#define SVA_DISPATCH(P, FN, ...)                                                         \
  ((P).bf16 ? ((P).D == 64 ? ((P).rope ? FN<true, 64, true>(__VA_ARGS__)                 \
                                       : FN<true, 64, false>(__VA_ARGS__))               \
                           : ((P).rope ? FN<true, 32, true>(__VA_ARGS__)                 \
                                       : FN<true, 32, false>(__VA_ARGS__)))              \
            : ((P).D == 64 ? ((P).rope ? FN<false, 64, true>(__VA_ARGS__)                \
                                       : FN<false, 64, false>(__VA_ARGS__))              \
                           : ((P).rope ? FN<false, 32, true>(__VA_ARGS__)                \
                                       : FN<false, 32, false>(__VA_ARGS__))))

#define SVA_DISPATCH2(P, FN, ...)                                                        \
  ((P).bf16 ? ((P).D == 64 ? FN<true, 64>(__VA_ARGS__) : FN<true, 32>(__VA_ARGS__))      \
            : ((P).D == 64 ? FN<false, 64>(__VA_ARGS__) : FN<false, 32>(__VA_ARGS__)))

size_t qkv_bytes(const Plan& p) { return (size_t)p.BH * p.N * p.D * (p.bf16 ? 2 : 4); }

sva_status check_common(const sva_desc* d, bool one_block, Plan* p) {
  sva_status s = validate_desc(d, one_block);
  if (s != SVA_OK) return s;
  *p = make_plan(d);
  return SVA_OK;
}

sva_status run_fwd(const sva_desc* desc, const void* q, const void* k, const void* v, void* out,
                   const float* S0, const float* z0, float* S_out, float* z_out, void* ws,
                   size_t ws_bytes, void* stream, void* const* events) {
  Plan p;
  sva_status s = check_common(desc, false, &p);
  if (s != SVA_OK) return s;
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
  if (!ws || ws_bytes < p.ws_bytes || !is_aligned16(ws)) return SVA_ERR_WORKSPACE;
  if (events) {
    for (int i = 0; i < 4; ++i)
      if (!events[i]) return SVA_ERR_INVALID_ARG;
  }

  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  float* partials = (float*)(wsb + p.off_partials);
  void* frags = wsb + p.off_frags;
  float* zc = (float*)(wsb + p.off_zc);
  hipError_t e = hipSuccess;
  if (events && (e = hipEventRecord((hipEvent_t)events[0], st)) != hipSuccess) return SVA_ERR_HIP;
  if ((e = SVA_DISPATCH(p, launch_reduce, p, k, v, partials, st)) != hipSuccess) return SVA_ERR_HIP;
  if (events && (e = hipEventRecord((hipEvent_t)events[1], st)) != hipSuccess) return SVA_ERR_HIP;
  if ((e = SVA_DISPATCH2(p, launch_scan, p, partials, S0, z0, S_out, z_out, frags, zc, true, st)) !=
      hipSuccess)
    return SVA_ERR_HIP;
  if (events && (e = hipEventRecord((hipEvent_t)events[2], st)) != hipSuccess) return SVA_ERR_HIP;
  if ((e = SVA_DISPATCH(p, launch_apply, p, q, out, frags, zc, desc->eps, st)) != hipSuccess)
    return SVA_ERR_HIP;
  if (events && (e = hipEventRecord((hipEvent_t)events[3], st)) != hipSuccess) return SVA_ERR_HIP;
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
  return run_fwd(desc, q, k, v, out, S0, z0, S_out, z_out, ws, ws_bytes, stream, nullptr);
}

sva_status sva_lin_attn_fwd_traced(const sva_desc* desc, const void* q, const void* k,
                                   const void* v, void* out, const float* S0, const float* z0,
                                   float* S_out, float* z_out, void* ws, size_t ws_bytes,
                                   void* stream, void* const events[4]) {
  if (!events) return SVA_ERR_INVALID_ARG;
  return run_fwd(desc, q, k, v, out, S0, z0, S_out, z_out, ws, ws_bytes, stream, events);
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
  return run_fwd(desc, q, k, v, out, S, z, nullptr, nullptr, ws, ws_bytes, stream, nullptr);
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
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  float* partials = (float*)(wsb + p.off_partials);
  if (SVA_DISPATCH(p, launch_reduce, p, k, v, partials, st) != hipSuccess) return SVA_ERR_HIP;
  if (SVA_DISPATCH2(p, launch_scan, p, partials, S, z, S, z, nullptr, nullptr, false, st) !=
      hipSuccess)
    return SVA_ERR_HIP;
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
