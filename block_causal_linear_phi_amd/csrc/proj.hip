// QKV projection with MXFP4 weights on gfx950 MFMA, writing q, k, v in the
// attention's [B, H, N, d] layout.
//
// Pages followed: the cstia.com SANA-Video article (4-bit QKV projections
// with SVDQuant; NVFP4 deployment) and the OCP Microscaling Formats (MX)
// specification for the MXFP4 format; readings in include/sva_proj.h.
//
// The product is computed transposed, y^T = W^T x^T, on
// v_mfma_f32_16x16x32_bf16: the A operand is a 16-feature slice of the
// decoded weights, the B operand 16 tokens, so a lane's accumulators hold
// consecutive output features of one token and the epilogue writes 16-byte
// pieces of the [B, H, N, d] rows directly.  A workgroup (4 waves) owns 256
// output features x 64 tokens; a wave 64 features x 64 tokens (4 x 4
// accumulators).  Two workgroups share a CU (198 registers a lane), so one's
// epilogue overlaps the other's MFMAs (8-wave workgroups of 256 x 128, one
// per CU, took 7% longer).  The input channels advance 128 per stage.
//
// Only x goes through LDS (64 x 128 bf16 a stage, double-buffered, the
// stage after next in registers).  Each wave loads its own weights straight
// from global memory into registers, one stage ahead, in the packed layout
// sva_mxfp4_pack_weights writes (4 KiB of codes and 256 bytes of scales per
// wave and stage, contiguous), and decodes them per k-step with
// v_cvt_scalef32_pk_bf16_fp4 (two 4-bit codes and their E8M0 block scale per
// instruction, exact).  Staging decoded weights in LDS instead (the previous
// design) made the operand reads from LDS as long as the MFMAs (0.5 KB an
// MFMA at this tile); the natural [row][channel] code layout, read straight
// from global memory, stalled the texture path on 16 rows per load.
// Consecutive workgroup indices go to the eight XCDs in turn, so the tiles
// are ordered to keep every workgroup that reads one x tile on the same XCD
// (its L2 then serves the 12 output tiles of a 720p QKV projection; x is
// fetched from HBM once).  Outputs are stored non-temporally: written
// through the L2 like the x tiles, they cost 8% more time.  A persistent
// version (a grid of resident workgroups, the stages of consecutive tiles in
// one pipeline, outputs leaving through LDS one piece per stage) was no
// faster.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "sva.h"
#include "sva_proj.h"

namespace {

typedef float pj_floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t pj_u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 pj_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pj_bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;  // LDS destination of direct loads

constexpr int kPjThreads = 256;  // 4 waves
constexpr int kTileN = 256;      // output features per workgroup
constexpr int kTileM = 64;       // tokens per workgroup
constexpr int kTileK = 128;      // input channels per stage
constexpr int kPieces = kTileK * 2 / 16;        // 16-byte pieces of an x row per stage
constexpr int kXU4 = kTileM * kPieces;          // x tile, 16-byte units
constexpr int kXLoads = kXU4 / kPjThreads;      // x pieces per thread per stage

struct ProjGeo {
  int M;          // B * N tokens
  int N;          // tokens per sample
  int C;          // input channels
  int H, d;
  int n_out;      // features computed: [0, n_out) of the packed weights
  int n_pack;     // rows of the packed weights (3 * H * d)
  int Mt, Nt;     // token tiles, feature tiles
  int stages;     // C / kTileK
  FastDiv fN, fHD, fd;  // division by N, H * d and d (the epilogue's indices)
};

struct KvGeo {
  int N, C, H;      // tokens per sample, input channels, heads (head dimension 64)
  int n_pack;       // rows of the packed weights (3 * H * 64)
  int stages;       // C / kTileK
  int L;            // tokens per range; divides Nb
  int ranges;       // N / L
  int Nb, nb;       // tokens per block, blocks per sample
  int npairs;       // H / 2
  int nrg;          // B * ranges
  FastDiv fHW, fWs; // division by Hs * Ws and by Ws
  int Hs, Ws, t0;   // latent grid rows and columns, first frame
  int rope, dt, dh; // RoPE on, t and h axis widths (w takes the rest)
  double log2_base_d;  // log2 of the RoPE base
  int F;            // frames per block
  int tab_entries;  // F dt/2 + Hs dh/2 + Ws dw/2 (the RoPE table's size)
};

struct QaGeo {
  int N, C, H;      // tokens per sample, input channels, heads (head dimension 64)
  int n_pack;       // rows of the packed weights (3 * H * 64)
  int stages;       // C / kTileK
  int Nb, nb;       // tokens per block, blocks per sample
  int tiles_blk;    // 64-token tiles per block (the last one ragged)
  int tpw;          // tiles per workgroup
  int groups;       // workgroups per block and head quad: ceil(tiles_blk / tpw)
  int ngrp;         // B * nb * groups
  int nquads;       // ceil(H / 4)
  FastDiv fHW, fWs; // division by Hs * Ws and by Ws
  int Hs, Ws, t0;   // latent grid rows and columns, first frame
  int rope, dt, dh; // RoPE on, t and h axis widths (w takes the rest)
  double log2_base_d;  // log2 of the RoPE base
  int F;            // frames per block
  int tab_entries;  // F dt/2 + Hs dh/2 + Ws dw/2
  float eps;
};

// LDS RoPE table of the fused k, v kernel: cos/sin of every (axis position,
// frequency) one workgroup's range can need: [F frames of its block][dt/2],
// then [Hs][dh/2], then [Ws][dw/2].  Sized so that two workgroups still fit
// in a CU's 160 KB of LDS; larger grids rotate on the fly.
constexpr int kRopeTab = 1728;

// Piece p of row r of the x tile, XOR-swizzled by r & 7: the B operand's
// 16-byte reads (served eight lanes at a time) take one piece of eight
// consecutive rows, and the tile writes eight consecutive pieces of one row;
// both land in eight distinct 16-byte bank groups.
__device__ __forceinline__ int sw(int r, int p) { return r * kPieces + (p ^ (r & 15)); }

// A-operand row permutation: accumulator rt, element i of lane (g, .) holds
// feature fo(rt, 4g + i) = 32(rt/2) + 8g + 4(rt%2) + i, so accumulators 0, 1
// (and 2, 3) of a lane cover 8 consecutive features.
__device__ __forceinline__ int fo(int rt, int r) {
  return 32 * (rt >> 1) + 8 * (r >> 2) + 4 * (rt & 1) + (r & 3);
}

__device__ __forceinline__ pj_floatx4 mfma(const uint4& a, const uint4& b, pj_floatx4 c) {
  const pj_u32x4 av = {a.x, a.y, a.z, a.w}, bv = {b.x, b.y, b.z, b.w};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pj_bf16x8, av),
                                                 __builtin_bit_cast(pj_bf16x8, bv), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// E8M0 scale byte -> the fp32 factor 2^(e - 127) (0 gives the denormal
// 2^-127), or NaN for 255; selects, no branches.
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  const uint32_t bits = e == 0 ? 0x00400000u : e << 23;
  return __uint_as_float(e == 255 ? 0x7fc00000u : bits);
}

// One word of codes (8 channels, low nibble first) -> the 8 bf16 weights of
// an A operand.
__device__ __forceinline__ uint4 decode8(uint32_t c, float s) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, s, 3)));
}

// A wave's weights for one stage: per accumulator row tile rt, the lane's 16
// bytes of codes (one MX block: 32 channels), and one word whose byte rt is
// that block's scale.
struct WRegs {
  uint4 c[4];
  uint32_t s;
};

// The fused k, v kernel's: two row tiles of a k block and two of a v block,
// each block with its own scale word.
struct KvWRegs {
  uint4 c[4];
  uint32_t sk, sv;
};

// Workgroup barrier for LDS only: waits for this wave's LDS accesses
// (lgkmcnt(0); 0xC07F leaves vmcnt and expcnt at their maxima), so global
// loads in flight stay in flight across it.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const pj_bf16x2 v = {(__bf16)a, (__bf16)b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Epilogue of a wave's 64 x 64 tile: lane (lg, lr) holds, for token tile
// tt, features f0 + 8 lg + 0..7 (accumulators 0, 1) and f0 + 32 + 8 lg +
// 0..7 (2, 3) of token t0 + 16 tt + lr.  Adds the bias, rounds to bf16 and
// stores 16-byte pieces straight into the [B, H, N, d] rows (non-temporal).
__device__ __forceinline__ void store_qkv(const pj_floatx4 (&acc)[4][4], const ProjGeo& g,
                                          const float* __restrict__ bias, void* __restrict__ qp,
                                          void* __restrict__ kp, void* __restrict__ vp, int f0, int t0, int lg,
                                          int lr) {
  const int HD = g.H * g.d;
#pragma unroll
  for (int run = 0; run < 2; ++run) {
    const int f = f0 + 32 * run + 8 * lg;  // first of 8 features
    if (f >= g.n_out) continue;
    const int which = (int)fdiv((uint32_t)f, g.fHD);
    const int h = (int)fdiv((uint32_t)(f - which * HD), g.fd);
    const int fd = f - which * HD - h * g.d;
    char* dst = (char*)(which == 0 ? qp : which == 1 ? kp : vp);
    float bb[8];
    if (bias) {
      const float4 b0 = *(const float4*)(bias + f), b1 = *(const float4*)(bias + f + 4);
      bb[0] = b0.x; bb[1] = b0.y; bb[2] = b0.z; bb[3] = b0.w;
      bb[4] = b1.x; bb[5] = b1.y; bb[6] = b1.z; bb[7] = b1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) bb[i] = 0.f;
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int m = t0 + tt * 16 + lr;
      if (m < g.M) {
        const int b = (int)fdiv((uint32_t)m, g.fN), t = m - b * g.N;
        const pj_floatx4 lo = acc[2 * run][tt], hi = acc[2 * run + 1][tt];
        const uint4 v = make_uint4(pack2(lo[0] + bb[0], lo[1] + bb[1]), pack2(lo[2] + bb[2], lo[3] + bb[3]),
                                   pack2(hi[0] + bb[4], hi[1] + bb[5]), pack2(hi[2] + bb[6], hi[3] + bb[7]));
        __builtin_nontemporal_store(__builtin_bit_cast(pj_u32x4, v),
                                    (pj_u32x4*)(dst + ((((size_t)b * g.H + h) * g.N + t) * g.d + fd) * 2));
      }
    }
  }
}

__global__ __launch_bounds__(kPjThreads, 2) void sva_qkv_proj_kernel(
    const void* __restrict__ xp, const uint8_t* __restrict__ wpack, const float* __restrict__ bias,
    void* __restrict__ qp, void* __restrict__ kp, void* __restrict__ vp, ProjGeo g) {
  __shared__ uint4 xs[2][kXU4];

  // Tile order: workgroup i runs on XCD i % 8; within an XCD, consecutive
  // workgroups take the feature tiles of one token tile.
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int mt = (local / g.Nt) * 8 + xcd;
  const int nt = local % g.Nt;
  if (mt >= g.Mt) return;
  const int m0 = mt * kTileM, n0 = nt * kTileN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lg = lane >> 4, lr = lane & 15;
  const int wn = wave & 3, wm = wave >> 2;  // 64 features x 64 tokens each (wm = 0)

  // x rows m0 .. m0 + 63 (rows past M read as zeros)
  const int rows = min(kTileM, g.M - m0);
  const size_t row_bytes = (size_t)g.C * 2;
  const __amdgpu_buffer_rsrc_t xr = rsrc((const char*)xp + (size_t)m0 * row_bytes, (uint32_t)(rows * row_bytes));

  // The MFMA contraction slots of a stage are assigned so that lane group lg
  // takes channels 32 lg + 8 j + e in k-step j: the lane's weights of a stage
  // are then one MX block per accumulator row tile, 16 bytes of codes and one
  // scale byte, and its x operands are pieces 4 lg + j of the token row.  The
  // packed layout puts a wave's codes of one stage in 4 KiB and its scales in
  // one word per lane, so each load is contiguous across the wave.  A wave
  // past n_out (a partial last tile) reads the last block and stores nothing.
  const int blk = min(n0 / 64 + wn, g.n_out / 64 - 1);
  const uint8_t* cbase = wpack + ((size_t)blk * g.stages * 4) * 1024 + lane * 16;
  const uint8_t* sbase = wpack + (size_t)g.n_pack * (g.C / 2) + ((size_t)blk * g.stages * 64 + lane) * 4;

  auto load_x = [&](uint4 (&r)[kXLoads], int s) {
    const int k0 = s * kTileK;
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int u = tid + j * kPjThreads;
      const uint32_t off = (uint32_t)((u / kPieces) * row_bytes + (size_t)k0 * 2 + 16 * (u % kPieces));
      r[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
  };
  auto store_x = [&](const uint4 (&r)[kXLoads], int buf) {
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int u = tid + j * kPjThreads;
      xs[buf][sw(u / kPieces, u % kPieces)] = r[j];
    }
  };
  auto load_w = [&](WRegs& w, int s) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) w.c[rt] = *(const uint4*)(cbase + ((size_t)s * 4 + rt) * 1024);
    w.s = *(const uint32_t*)(sbase + (size_t)s * 256);
  };

  pj_floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = pj_floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const WRegs& w, int buf) {
    // The scale bytes pass through an empty asm here: otherwise the
    // compiler converts them right after their loads, one stage early, and
    // waits there for every load in flight (one in-order counter).
    uint32_t e = w.s;
    asm volatile("" : "+v"(e));
    float sc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) sc[rt] = e8m0_scale((e >> (8 * rt)) & 0xffu);
#pragma unroll
    for (int j = 0; j < kTileK / 32; ++j) {
      uint4 a[4], b[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const uint32_t cw = j == 0 ? w.c[rt].x : j == 1 ? w.c[rt].y : j == 2 ? w.c[rt].z : w.c[rt].w;
        a[rt] = decode8(cw, sc[rt]);
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) b[tt] = xs[buf][sw(wm * 64 + tt * 16 + lr, 4 * lg + j)];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = mfma(a[rt], b[tt], acc[rt][tt]);
    }
  };

  // Pipeline: stage s is computed from LDS buffer s % 2 and weight registers
  // s % 2 while stage s + 1's x waits in registers and stage s + 2's x loads
  // are in flight; stage s + 1's weights are requested before stage s's
  // MFMAs.  Every load is issued, with the stage index clamped to the last
  // one (repeat loads at the tail are in bounds and unused): a conditional
  // load leaves the compiler unsure how many loads are in flight after it,
  // and it then waits for all of them.
  const int last = g.stages - 1;
  uint4 x0[kXLoads], x1[kXLoads];
  WRegs w0, w1;
  load_w(w0, 0);
  load_x(x0, 0);
  load_x(x1, min(1, last));
  store_x(x0, 0);
  load_x(x0, min(2, last));
  __syncthreads();
  auto step = [&](int s, const WRegs& wc, WRegs& wn_, uint4 (&xn)[kXLoads]) {
    load_w(wn_, min(s + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    compute(wc, s & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < g.stages) store_x(xn, (s + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    load_x(xn, min(s + 3, last));
    __syncthreads();
  };
  int s = 0;
  for (; s + 2 <= g.stages; s += 2) {
    step(s, w0, w1, x1);
    step(s + 1, w1, w0, x0);
  }
  if (s < g.stages) step(s, w0, w1, x1);

  store_qkv(acc, g, bias, qp, kp, vp, n0 + wn * 64, m0 + wm * 64, lg, lr);
}

// ---------------------------------------------------------------------------
// W4A4: the activations in MXFP4 as well.
//
// The pages deploy the 4-bit projections through SVDQuant in NVFP4, which
// puts both operands of the projection in 4 bits; gfx950's counterpart is
// MXFP4 on the scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4), four times
// the bf16 rate.  sva_mxfp4_quant_kernel converts the activations once
// (OCP MX conversion, per token row and 32 input channels); the GEMM then
// reads 4-bit x straight from global memory in the MFMA's B layout (lane
// (lg, lr): token lr, channels 32 lg .. 32 lg + 31 of the stage, 16 bytes)
// with its E8M0 scale, and the packed weights exactly as the bf16 kernel
// does: the packed layout is already the A layout of the scaled MFMA (lane
// (lg, lr): row lr, channels 32 lg .. + 31), and the word of four scale
// bytes per lane is its scale operand, the row tile picking the byte.  No
// decode instructions and no LDS.
// ---------------------------------------------------------------------------

constexpr int kQuantThreads = 256;

// One thread per 32-channel block of a token row.  The shared exponent
// comes from the exponent field of the block's largest magnitude (bf16
// magnitudes order as their bit patterns): floor(log2 amax) - 2, at least
// -127 (scale byte 0, also for an all-zero block).  The elements go through
// v_cvt_scalef32_pk_fp4_f32, which rounds x / scale to E2M1 (nearest, ties
// to even, clamped at 6, the sign kept); measured on gfx950 to equal that
// rule for every finite bf16 input at power-of-two scales.  Below scale
// byte 64 both x and the scale are multiplied by 2^64 (exact), so that the
// scale is a normal fp32 number.  Non-finite inputs are outside the
// contract.
__global__ __launch_bounds__(kQuantThreads) void sva_mxfp4_quant_kernel(const uint32_t* __restrict__ x,
                                                                       uint8_t* __restrict__ codes,
                                                                       uint8_t* __restrict__ scales,
                                                                       long long nblk) {
  const long long i = (long long)blockIdx.x * kQuantThreads + threadIdx.x;
  if (i >= nblk) return;
  const uint4* src = (const uint4*)(x + i * 16);  // 32 bf16, two a word, low half first
  uint32_t w[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 v = src[j];
    w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) amax = max(amax, max(w[j] & 0x7fffu, (w[j] >> 16) & 0x7fffu));
  const uint32_t e = amax >> 7;  // the bf16 (and fp32) exponent field
  const uint32_t code = e > 2 ? e - 2 : 0;
  const bool pre = code < 64;
  const float mul = pre ? 0x1p64f : 1.0f;
  const float scale = __uint_as_float((code + (pre ? 64u : 0u)) << 23);
  // channels 2j, 2j + 1 of input word j -> byte j % 4 of output word j / 4
  auto lo = [&](int j) { return __uint_as_float(w[j] << 16) * mul; };
  auto hi = [&](int j) { return __uint_as_float(w[j] & 0xffff0000u) * mul; };
  uint32_t out[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo(4 * q), hi(4 * q), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo(4 * q + 1), hi(4 * q + 1), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo(4 * q + 2), hi(4 * q + 2), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo(4 * q + 3), hi(4 * q + 3), scale, 3);
    out[q] = r;
  }
  *(uint4*)(codes + i * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  scales[i] = (uint8_t)code;
}

typedef int pj_v8i __attribute__((ext_vector_type(8)));

// acc += (A * 2^(sa byte RT)) (B * 2^(sb)) with A, B 16 x 128 and 128 x 16
// fp4 (E2M1) tiles; RT picks the A scale's byte.
template <int RT>
__device__ __forceinline__ pj_floatx4 mfma_fp4(const uint4& a, uint32_t sa, const uint4& b, uint32_t sb,
                                               pj_floatx4 c) {
  const pj_v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const pj_v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, RT, (int)sa, 0, (int)sb);
}

// The workgroup's 64 x-rows of up to kXChunk channels live in LDS: codes at
// a pitch of 32 16-byte pieces a row, piece p of row r at p ^ (r & 31) (the
// B reads of one instruction -- 16 rows, 4 pieces each -- fall in distinct
// bank groups), and one word of four scale bytes per row and stage.  They
// come straight from global memory (buffer loads with the lds bit), which
// leaves the registers to the accumulators and weights.
constexpr int kXChunk = 1024;                 // channels per LDS chunk
constexpr int kXChunkStages = kXChunk / kTileK;
constexpr int kXPitch = kXChunk / 32;         // 16-byte pieces per row

__global__ __launch_bounds__(kPjThreads, 2) void sva_qkv_proj_w4a4_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xsc, const uint8_t* __restrict__ wpack,
    const float* __restrict__ bias, void* __restrict__ qp, void* __restrict__ kp, void* __restrict__ vp,
    ProjGeo g) {
  __shared__ uint4 xcs[kTileM * kXPitch];
  __shared__ uint32_t xss[kTileM * kXChunkStages];

  // Tile order as in the bf16 kernel: the feature tiles of one token tile on
  // one XCD, whose L2 then serves its x.
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int mt = (local / g.Nt) * 8 + xcd;
  const int nt = local % g.Nt;
  if (mt >= g.Mt) return;
  const int m0 = mt * kTileM, n0 = nt * kTileN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lg = lane >> 4, lr = lane & 15;
  const int wn = wave & 3;

  // x rows m0 .. m0 + 63 (rows past M read as zero codes and zero scales)
  const int rows = min(kTileM, g.M - m0);
  const uint32_t crow = (uint32_t)g.C / 2, srow = (uint32_t)g.C / 32;
  const __amdgpu_buffer_rsrc_t xr = rsrc(xq + (size_t)m0 * crow, (uint32_t)rows * crow);
  const __amdgpu_buffer_rsrc_t sr = rsrc(xsc + (size_t)m0 * srow, (uint32_t)rows * srow);

  const int blk = min(n0 / 64 + wn, g.n_out / 64 - 1);
  const uint8_t* cbase = wpack + ((size_t)blk * g.stages * 4) * 1024 + lane * 16;
  const uint8_t* sbase = wpack + (size_t)g.n_pack * (g.C / 2) + ((size_t)blk * g.stages * 64 + lane) * 4;

  auto load_w = [&](WRegs& w, int s) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) w.c[rt] = *(const uint4*)(cbase + ((size_t)s * 4 + rt) * 1024);
    w.s = *(const uint32_t*)(sbase + (size_t)s * 256);
  };
  // The chunk of x at stage s0 straight into LDS (buffer loads with the lds
  // bit, as in the fused k, v kernel): load i of wave w fills code slots
  // 64 (8 w + i) + lane, rows 2 (8 w + i) + lane / 32 at swizzled position
  // lane % 32; scale load i fills words 64 (2 w + i) + lane.  Pieces and
  // stages past the chunk get an offset past the descriptor: zeros.
  constexpr uint32_t kPast = 0x80000000u;
  auto load_chunk = [&](int s0) {
    const int ns = min(kXChunkStages, g.stages - s0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 2 * (8 * wave + i) + (lane >> 5);
      const int piece = (lane & 31) ^ (row & 31);
      const uint32_t off = piece < 4 * ns ? (uint32_t)row * crow + 64 * s0 + 16 * piece : kPast;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_ptr)(xcs + 64 * (8 * wave + i)), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = 64 * (2 * wave + i) + lane;
      const int sl = u % kXChunkStages;
      const uint32_t off = sl < ns ? (uint32_t)(u / kXChunkStages) * srow + 4 * (s0 + sl) : kPast;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void_ptr)(xss + 64 * (2 * wave + i)), 4, off, 0, 0, 0);
    }
  };

  pj_floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = pj_floatx4{0.f, 0.f, 0.f, 0.f};

  // One stage from chunk-local stage sl: B operands and scales from LDS,
  // the weights from registers.
  auto compute = [&](const WRegs& w, int sl) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int r = tt * 16 + lr;
      const uint4 b = xcs[r * kXPitch + ((4 * sl + lg) ^ (r & 31))];
      const uint32_t sb = (xss[r * kXChunkStages + sl] >> (8 * lg)) & 0xffu;
      acc[0][tt] = mfma_fp4<0>(w.c[0], w.s, b, sb, acc[0][tt]);
      acc[1][tt] = mfma_fp4<1>(w.c[1], w.s, b, sb, acc[1][tt]);
      acc[2][tt] = mfma_fp4<2>(w.c[2], w.s, b, sb, acc[2][tt]);
      acc[3][tt] = mfma_fp4<3>(w.c[3], w.s, b, sb, acc[3][tt]);
    }
  };

  // Weights one stage ahead, two register sets: every load is issued, the
  // stage clamped to the last (repeat loads at the tail are in bounds and
  // unused).  (Two stages ahead in a ring of register pairs raised the
  // registers past three workgroups a CU, and was no faster.)
  WRegs w0, w1;
  load_w(w0, 0);
  load_chunk(0);
  const int nch = (g.stages + kXChunkStages - 1) / kXChunkStages;
  const int last = g.stages - 1;
  for (int j = 0; j < nch; ++j) {
    if (j > 0) {  // past 1024 channels: the next chunk, once every wave is done with this one
      __syncthreads();
      load_chunk(j * kXChunkStages);
    }
    // every wave's loads of the chunk have landed: vmcnt(0), then the workgroup meets
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    asm volatile("" ::: "memory");
    const int s0 = j * kXChunkStages;
    const int ns = min(kXChunkStages, g.stages - s0);
    int sl = 0;
    for (; sl + 2 <= ns; sl += 2) {
      load_w(w1, min(s0 + sl + 1, last));
      __builtin_amdgcn_sched_barrier(0);
      compute(w0, sl);
      __builtin_amdgcn_sched_barrier(0);
      load_w(w0, min(s0 + sl + 2, last));
      __builtin_amdgcn_sched_barrier(0);
      compute(w1, sl + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (sl < ns) {  // an odd stage count (C an odd multiple of 128): the last stage
      load_w(w1, min(s0 + sl + 1, last));
      __builtin_amdgcn_sched_barrier(0);
      compute(w0, sl);
      __builtin_amdgcn_sched_barrier(0);
      w0 = w1;
    }
  }

  store_qkv(acc, g, bias, qp, kp, vp, n0 + wn * 64, m0, lg, lr);
}

// ---------------------------------------------------------------------------
// k and v projections fused with the per-block state reduction.
//
// A workgroup takes a range of L tokens of one sample (L divides the block's
// token count, so a range lies in one block) and two heads h0, h0 + 1; its
// waves compute k and v of those heads (64 features each) for 64-token
// tiles with the projection's GEMM.  Instead of storing k and v, each tile's
// epilogue rounds them to bf16 (as a stored tensor would be), applies phi
// and the numerator-only 3D RoPE to k, stages both in LDS and adds the
// tile's v^T RoPE(phi k) to the head's state on MFMA (operands read with
// LDS transpose reads), and phi k to its normaliser.  At the end of the
// range each head's state and normaliser go to the partial slot the block
// scan reads for (range, block): slot g + bhc with g the range's index along
// the flattened (b, h, token) axis in units of L.  So k and v never reach
// HBM.
//
// The GEMM pipeline runs on across the tiles of a range (the next tile's
// first x and weight stages load during the epilogue), the accumulators
// start from the bias, and RoPE reads cos/sin from a per-workgroup LDS
// table of the positions the range can hold, or computes them on the fly
// for grids whose table would not fit beside two workgroups per CU.
// ---------------------------------------------------------------------------

constexpr int kKvThreads = 256;  // waves: (h0, half 0), (h0, half 1), (h0+1, 0), (h0+1, 1)
static_assert(kKvThreads == kPjThreads, "the GEMM part assumes the projection's workgroup size");

// Pieces shared by the fused k, v kernels (bf16 and 4-bit activations):
// both GEMMs leave a wave's 64 features x 64 tokens in the same accumulator
// layout, so the epilogue, the state update and the partial are common.

// The LDS RoPE table of block c (see kRopeTab; any geometry with KvGeo's
// RoPE fields): cos, sin of pos *
// base^(-2i/width) turns, the angle in fp64 reduced to [-1/2, 1/2] turn,
// then the hardware sine and cosine (which take turns).
template <typename Geo>
__device__ __forceinline__ void kv_build_rope_table(float2* rtab, const Geo& g, int c, int tid) {
  const int ht = g.dt >> 1, hh = g.dh >> 1, hwd = (64 - g.dt - g.dh) >> 1;
  const int off_h = g.F * ht, off_w = off_h + g.Hs * hh;
  for (int e = tid; e < g.tab_entries; e += kKvThreads) {
    int pos, i, width;
    if (e < off_h) {
      pos = g.t0 + c * g.F + e / ht, i = e % ht, width = g.dt;
    } else if (e < off_w) {
      pos = (e - off_h) / hh, i = (e - off_h) % hh, width = g.dh;
    } else {
      pos = (e - off_w) / hwd, i = (e - off_w) % hwd, width = 64 - g.dt - g.dh;
    }
    double rv = (double)pos * exp2(-(double)(2 * i) / (double)width * g.log2_base_d) * 0.15915494309189535;
    rv -= rint(rv);
    rtab[e] = make_float2(__builtin_amdgcn_cosf((float)rv), __builtin_amdgcn_sinf((float)rv));
  }
}

// Epilogue of one 64-token tile (tokens n0 ..) of the range [.., n_end) of
// block c.  Lane (lg, lr) holds features 32 half + 8 lg + 0..7 of the head's
// k (accumulators 0, 1) and v (2, 3) for token 16 tt + lr, bias included
// (the accumulators start from it).  Values are rounded to bf16 as the
// stored tensors would be; k then gets phi (its normaliser share goes to the
// lane's zt, which kv_z_reduce sums at the end) and the rotation of its
// position, and is rounded to bf16 again.  Only v is zeroed past the range
// (its zero rows keep those tokens out of S; the normaliser masks k
// itself), and only in a ragged tile (kFull false).
// The head's k and v tiles go to LDS row-major, for kv_state_mfma_tr after
// a barrier: row = token, 128 bytes of 64 bf16 features, 16-byte piece p of
// row t at p ^ (t & 7); a lane's 8 features of one token are one piece, so
// a token tile takes two 16-byte writes a lane.  lgv is lg, through an
// empty asm where registers are short: the compiler would otherwise hoist
// the RoPE constants out of the tile loop, and they would occupy registers
// through the GEMM.  RoPE: kRope 0 takes the cos/sin table with the lane's
// 4 pairs on one axis (every axis width a multiple of 8: the pairs' entries
// are consecutive), 1 the table pair by pair, 2 computes the angles.
__device__ __forceinline__ int kv_rm_off(int t, int p) { return t * 128 + ((p ^ (t & 7)) << 4); }

template <int kRope, bool kFull>
__device__ __forceinline__ void kv_tile_epilogue_rm(const pj_floatx4 (&acc)[4][4], const KvGeo& g,
                                                    const float2* rtab, uint4* kvt, float (&zt)[8], int wave,
                                                    int half, int lg, int lgv, int lr, int n0, int n_end, int c) {
  const int off_h = g.F * (g.dt >> 1), off_w = off_h + g.Hs * (g.dh >> 1);
  float inv[4], tbase[4];
  int axis[4], eoff[4], estr[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int f = 32 * half + 8 * lgv + 2 * pp;
    const int ax = f < g.dt ? 0 : f < g.dt + g.dh ? 1 : 2;
    const int start = ax == 0 ? 0 : ax == 1 ? g.dt : g.dt + g.dh;
    const int width = ax == 0 ? g.dt : ax == 1 ? g.dh : 64 - g.dt - g.dh;
    axis[pp] = ax;
    if constexpr (kRope < 2) {
      eoff[pp] = (ax == 0 ? 0 : ax == 1 ? off_h : off_w) + ((f - start) >> 1);
      estr[pp] = width >> 1;
    } else {
      const double inv_d = exp2(-(double)(f - start) / (double)width * g.log2_base_d) * 0.15915494309189535;
      double tb = ax == 0 ? (double)(g.t0 + c * g.F) * inv_d : 0.0;
      tb -= rint(tb);
      inv[pp] = (float)inv_d;
      tbase[pp] = (float)tb;
    }
  }
  char* const ktile = reinterpret_cast<char*>(kvt + (wave & 2) * 512);
  char* const vtile = reinterpret_cast<char*>(kvt + ((wave & 2) + 1) * 512);
  const int piece = 4 * half + lg;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int tok = 16 * tt + lr;
    const int n = n0 + tok;
    const bool valid = kFull || n < n_end;
    // element i of the lane's 8 features: accumulator 2 run + i / 4, entry i % 4
    uint4 vw = make_uint4(pack2(acc[2][tt][0], acc[2][tt][1]), pack2(acc[2][tt][2], acc[2][tt][3]),
                          pack2(acc[3][tt][0], acc[3][tt][1]), pack2(acc[3][tt][2], acc[3][tt][3]));
    if (!kFull && !valid) vw = make_uint4(0u, 0u, 0u, 0u);
    float kv8[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w = pack2(acc[m >> 1][tt][2 * (m & 1)], acc[m >> 1][tt][2 * (m & 1) + 1]);
      // phi on the bit pattern, as in the attention kernels: every value
      // with the sign bit set (negative numbers, -0, a negative-signed NaN)
      // becomes +0, every other value passes unchanged
      kv8[2 * m] = __int_as_float(max((int)(w << 16), 0));
      kv8[2 * m + 1] = __int_as_float(max((int)(w & 0xffff0000u), 0));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) zt[i] += valid ? kv8[i] : 0.f;
    if (g.rope) {
      const uint32_t np = (uint32_t)(valid ? n : n_end - 1);  // positions past the range: any in it
      const uint32_t fr = fdiv(np, g.fHW), rem = np - fr * g.fHW.div;
      const uint32_t row = fdiv(rem, g.fWs);
      const int pt = (int)fr - c * g.F;  // the frame within the block
      const int ph = (int)row, pw = (int)(rem - row * g.fWs.div);
      const int ps0 = axis[0] == 0 ? pt : axis[0] == 1 ? ph : pw;
      const int e0 = eoff[0] + ps0 * estr[0];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        float sn, cs;
        if constexpr (kRope == 0) {
          const float2 e = rtab[e0 + pp];
          cs = e.x, sn = e.y;
        } else if constexpr (kRope == 1) {
          const int ax = axis[pp];
          const int ps = ax == 0 ? pt : ax == 1 ? ph : pw;
          const float2 e = rtab[eoff[pp] + ps * estr[pp]];
          cs = e.x, sn = e.y;
        } else {
          const int ax = axis[pp];
          const int ps = ax == 0 ? pt : ax == 1 ? ph : pw;
          const float turn = __builtin_amdgcn_fractf(tbase[pp] + (float)ps * inv[pp]);
          sn = __builtin_amdgcn_sinf(turn), cs = __builtin_amdgcn_cosf(turn);
        }
        const float x = kv8[2 * pp], y = kv8[2 * pp + 1];
        kv8[2 * pp] = x * cs - y * sn;
        kv8[2 * pp + 1] = x * sn + y * cs;
      }
    }
    const uint4 kw = make_uint4(pack2(kv8[0], kv8[1]), pack2(kv8[2], kv8[3]), pack2(kv8[4], kv8[5]),
                                pack2(kv8[6], kv8[7]));
    *reinterpret_cast<uint4*>(ktile + kv_rm_off(tok, piece)) = kw;
    *reinterpret_cast<uint4*>(vtile + kv_rm_off(tok, piece)) = vw;
  }
}

// The lanes' normaliser shares summed over the 16 token lanes: features
// 32 half + 8 lg + i of the head, into zhead (one wave per half writes).
__device__ __forceinline__ void kv_z_reduce(const float (&zt)[8], float* zhead, int half, int lg, int lr) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float t = zt[i];
    t += __shfl_xor(t, 1);
    t += __shfl_xor(t, 2);
    t += __shfl_xor(t, 4);
    t += __shfl_xor(t, 8);
    if (lr == 0) zhead[32 * half + 8 * lg + i] = t;
  }
}

typedef short pj_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) pj_i16x4* lds_i16x4_ptr;

// State rows (value features) 32 half .. + 31 of the wave's head, from the
// tiles kv_tile_epilogue_rm wrote: S^T[fo][fi] += sum over the tile's tokens
// of v[fo] RoPE(phi k)[fi]; sa[ft][fc] element i of lane (lg, lr) is row
// 16 (2 half + ft) + 4 lg + i, column 16 fc + lr.  The operands come with
// LDS transpose reads (ds_read_b64_tr_b16): within each 16-lane group,
// output lane i's element m
// is element i % 4 of the 8 bytes input lane 4 m + i / 4 points at.  So
// input lane j pointing at row tb + j / 4, features f0 + 4 (j % 4) .. + 3
// hands output lane i feature f0 + i of rows tb .. tb + 3: the 4 token
// slots of an MFMA operand, for the feature the lane's operand row needs.
__device__ __forceinline__ void kv_state_mfma_tr(pj_floatx4 (&sa)[2][4], const uint4* kvt, int wave, int half,
                                                 int lane) {
  const char* const vt = reinterpret_cast<const char*>(kvt + ((wave & 2) + 1) * 512);
  const char* const kt = reinterpret_cast<const char*>(kvt + (wave & 2) * 512);
  const int grp = lane >> 4, j = lane & 15;
  auto rd = [&](const char* tile, int tb, int f0) {
    const int row = tb + (j >> 2);
    const int f = f0 + 4 * (j & 3);
    const int off = row * 128 + (((f >> 3) ^ (row & 7)) << 4) + (f & 7) * 2;
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(tile + off)));
  };
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int tb = 32 * ks + 8 * grp;  // the lane group's 8 tokens of this k-step
    uint4 a[2], bo[4];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      const uint2 lo = rd(vt, tb, 32 * half + 16 * ft), hi = rd(vt, tb + 4, 32 * half + 16 * ft);
      a[ft] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
#pragma unroll
    for (int fc = 0; fc < 4; ++fc) {
      const uint2 lo = rd(kt, tb, 16 * fc), hi = rd(kt, tb + 4, 16 * fc);
      bo[fc] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int fc = 0; fc < 4; ++fc) sa[ft][fc] = mfma(a[ft], bo[fc], sa[ft][fc]);
  }
}

// The wave's share of the partial of (range r of sample b, block c) for
// head `head`: S^T rows 32 half .. + 31 (row fo, column fi), and from the
// waves of half 0 the head's z.  The partial sits at slot gv + bhc, with gv
// the range's index along the flattened (b, h, token) axis in units of L.
__device__ __forceinline__ void kv_store_partial(const pj_floatx4 (&sa)[2][4], const float* zhead,
                                                 float* __restrict__ partials, const KvGeo& g, int b, int head,
                                                 int r, int c, int half, int lg, int lr, int lane) {
  const long long bh = (long long)b * g.H + head;
  const long long gv = bh * g.ranges + r;
  const long long bhc = bh * g.nb + c;
  float* dst = partials + (gv + bhc) * (64 * 64 + 64);
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int fc = 0; fc < 4; ++fc) {
      const pj_floatx4 v4 = sa[ft][fc];
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * (2 * half + ft) + 4 * lg + i) * 64 + 16 * fc + lr] = v4[i];
    }
  if (half == 0) dst[64 * 64 + lane] = zhead[lane];
}

// kRope: as for kv_tile_epilogue_rm (0, 1: the LDS table; 2: on the fly).
template <int kRope>
__global__ __launch_bounds__(kKvThreads, 2) void sva_kv_proj_reduce_kernel(
    const void* __restrict__ xp, const uint8_t* __restrict__ wpack, const float* __restrict__ bias,
    float* __restrict__ partials, KvGeo g) {
  // The x stages double as the epilogue's k and v tiles (the GEMM is done
  // with them by then); the head states accumulate in LDS, lane by lane, so
  // that nothing beyond the projection's registers lives across the GEMM.
  __shared__ uint4 xs[2][kXU4];
  __shared__ pj_floatx4 sacc[kKvThreads / 64][8][64];
  __shared__ float zs[2][64];
  __shared__ float bs[kKvThreads / 64][64];
  __shared__ float2 rtab[kRope < 2 ? kRopeTab : 1];
  static_assert(sizeof(xs) == (kKvThreads / 64) * 64 * 8 * sizeof(uint4), "tiles alias the x stages");
  uint4* const kvt = &xs[0][0];  // wave w's tile at kvt + w * 512

  // Tile order: workgroup i runs on XCD i % 8; consecutive workgroups of one
  // XCD take the head pairs of one token range (they read the same x).
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int rg = (local / g.npairs) * 8 + xcd;
  const int pair = local % g.npairs;
  if (rg >= g.nrg) return;
  const int b = rg / g.ranges, r = rg - b * g.ranges;
  const int n_begin = r * g.L, n_end = n_begin + g.L;
  const int c = n_begin / g.Nb;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lg = lane >> 4, lr = lane & 15;
  // A wave computes features 32 half .. + 31 of both k and v of its head
  // (row tiles 2 half, 2 half + 1 of each packed 64-row block), so that
  // every wave takes an equal share of the epilogue's phi and RoPE.
  const int half = wave & 1;
  const int head = 2 * pair + (wave >> 1);
  const int blk_k = g.H + head, blk_v = 2 * g.H + head;
  // the v block lies H blocks past the k block (offsets uniform over the wave)
  const uint8_t* cbase = wpack + ((size_t)blk_k * g.stages * 4 + 2 * half) * 1024 + lane * 16;
  const uint8_t* sbase = wpack + (size_t)g.n_pack * (g.C / 2) + ((size_t)blk_k * g.stages * 64 + lane) * 4;
  const size_t cvoff = (size_t)g.H * g.stages * 4 * 1024, svoff = (size_t)g.H * g.stages * 256;
  const int sshift = 16 * half;  // the scale bytes of row tiles 2 half, 2 half + 1
  const size_t row_bytes = (size_t)g.C * 2;
  const long long M = (long long)(g.nrg / g.ranges) * g.N;  // B * N rows of x

#pragma unroll
  for (int k = 0; k < 8; ++k) sacc[wave][k][lane] = pj_floatx4{0.f, 0.f, 0.f, 0.f};
  float zt[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zt[i] = 0.f;
  bs[wave][lane] = bias ? bias[(lane < 32 ? blk_k : blk_v) * 64 + 32 * half + (lane & 31)] : 0.f;
  if constexpr (kRope < 2) kv_build_rope_table(rtab, g, c, tid);

  // x rows of token tile t of the range; past the last tile the descriptor
  // is empty (its loads return zeros and touch no memory).
  const int ntiles = (g.L + kTileM - 1) / kTileM;
  auto tile_rsrc = [&](int t) {
    const long long m0 = (long long)b * g.N + n_begin + (long long)t * kTileM;
    const int rows = t < ntiles ? (int)min((long long)kTileM, M - m0) : 0;
    return rsrc((const char*)xp + m0 * row_bytes, (uint32_t)(rows * row_bytes));
  };
  auto load_x = [&](uint4 (&rg4)[kXLoads], __amdgpu_buffer_rsrc_t xr, int s) {
    const int k0 = s * kTileK;
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int u = tid + j * kKvThreads;
      const uint32_t off = (uint32_t)((u / kPieces) * row_bytes + (size_t)k0 * 2 + 16 * (u % kPieces));
      rg4[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
  };
  auto store_x = [&](const uint4 (&rg4)[kXLoads], int buf) {
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int u = tid + j * kKvThreads;
      xs[buf][sw(u / kPieces, u % kPieces)] = rg4[j];
    }
  };
  // accumulators 0, 1: k row tiles; 2, 3: v row tiles
  auto load_w = [&](KvWRegs& w, int s) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      w.c[rt] = *(const uint4*)(cbase + (rt < 2 ? 0 : cvoff) + ((size_t)s * 4 + (rt & 1)) * 1024);
    w.sk = *(const uint32_t*)(sbase + (size_t)s * 256);
    w.sv = *(const uint32_t*)(sbase + svoff + (size_t)s * 256);
  };

  // The GEMM pipeline runs on across tiles: the last steps of a tile load
  // the next tile's first two x stages and first weight stage, which stay in
  // registers through the epilogue (the stage count is even, so they land in
  // x0, x1 and w0, where the prologue expects them).
  const int last = g.stages - 1;
  uint4 x0[kXLoads], x1[kXLoads];
  KvWRegs w0, w1;
  load_w(w0, 0);
  {
    const __amdgpu_buffer_rsrc_t xr0 = tile_rsrc(0);
    load_x(x0, xr0, 0);
    load_x(x1, xr0, 1);
  }
  for (int it = 0; it < ntiles; ++it) {
    const int n0 = n_begin + it * kTileM;
    const __amdgpu_buffer_rsrc_t xr = tile_rsrc(it), xr_next = tile_rsrc(it + 1);
    // x stage vs of this tile, or vs - stages of the next one
    auto load_v = [&](uint4 (&rg4)[kXLoads], int vs) {
      const bool nx = vs >= g.stages;
      load_x(rg4, nx ? xr_next : xr, nx ? vs - g.stages : vs);
    };
    // The accumulators start from the bias (row tile rt, entry i of lane
    // (lg, .): feature 8 lg + 4 (rt % 2) + i of the wave's k or v features).
    pj_floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 b4 = *reinterpret_cast<const float4*>(&bs[wave][32 * (i >> 1) + 8 * lg + 4 * (i & 1)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = pj_floatx4{b4.x, b4.y, b4.z, b4.w};
    }
    auto compute = [&](const KvWRegs& w, int buf) {
      uint32_t ek = w.sk, ev = w.sv;
      asm volatile("" : "+v"(ek));  // see the projection kernel
      asm volatile("" : "+v"(ev));
      const uint32_t e = ((ek >> sshift) & 0xffffu) | ((ev >> sshift) << 16);
      float sc[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) sc[rt] = e8m0_scale((e >> (8 * rt)) & 0xffu);
#pragma unroll
      for (int j = 0; j < kTileK / 32; ++j) {
        uint4 a[4], bo[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const uint32_t cw = j == 0 ? w.c[rt].x : j == 1 ? w.c[rt].y : j == 2 ? w.c[rt].z : w.c[rt].w;
          a[rt] = decode8(cw, sc[rt]);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) bo[tt] = xs[buf][sw(tt * 16 + lr, 4 * lg + j)];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = mfma(a[rt], bo[tt], acc[rt][tt]);
      }
    };
    // The barrier first: every wave has read the previous tile's k and v
    // from xs.
    __syncthreads();
    store_x(x0, 0);
    load_v(x0, 2);
    __syncthreads();
    auto step = [&](int s, const KvWRegs& wc, KvWRegs& wn_, uint4 (&xn)[kXLoads]) {
      load_w(wn_, s + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(wc, s & 1);
      __builtin_amdgcn_sched_barrier(0);
      store_x(xn, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      load_v(xn, s + 3);
      __syncthreads();
    };
    int s = 0;
    for (; s + 2 < g.stages; s += 2) {
      step(s, w0, w1, x1);
      step(s + 1, w1, w0, x0);
    }
    step(s, w0, w1, x1);
    // the tile's last stage: weights of stage 0 for the next tile, no x
    load_w(w0, 0);
    __builtin_amdgcn_sched_barrier(0);
    compute(w1, 1);
    __syncthreads();  // every wave is done with xs, which the epilogue overwrites

    int lgv = lg;
    asm volatile("" : "+v"(lgv));
    if (n0 + kTileM <= n_end)
      kv_tile_epilogue_rm<kRope, true>(acc, g, rtab, kvt, zt, wave, half, lg, lgv, lr, n0, n_end, c);
    else
      kv_tile_epilogue_rm<kRope, false>(acc, g, rtab, kvt, zt, wave, half, lg, lgv, lr, n0, n_end, c);
    __syncthreads();
    pj_floatx4 sa[2][4];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int fc = 0; fc < 4; ++fc) sa[ft][fc] = sacc[wave][4 * ft + fc][lane];
    kv_state_mfma_tr(sa, kvt, wave, half, lane);
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int fc = 0; fc < 4; ++fc) sacc[wave][4 * ft + fc][lane] = sa[ft][fc];
  }

  kv_z_reduce(zt, zs[wave >> 1], half, lg, lr);
  __syncthreads();
  pj_floatx4 sa[2][4];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int fc = 0; fc < 4; ++fc) sa[ft][fc] = sacc[wave][4 * ft + fc][lane];
  kv_store_partial(sa, zs[wave >> 1], partials, g, b, head, r, c, half, lg, lr, lane);
}

// The fused k, v kernel on 4-bit activations: the work split, the tile order
// and the epilogue of sva_kv_proj_reduce_kernel, with the GEMM of
// sva_qkv_proj_w4a4_kernel (the scaled fp4 MFMA on the 4-bit x tile from
// LDS, the packed weights one stage ahead in registers).  A token tile's x
// codes (64 rows of up to 1024 channels a chunk, rows XOR-swizzled) and
// scale words go straight from global memory to LDS (buffer loads with the
// lds bit, which take no registers): the next tile's are issued once every
// wave is done with the current ones, after the tile's last weight loads
// (vector loads complete in issue order, so no weight wait also waits for
// them), and land while the epilogue runs on its own LDS tiles.  Grids
// with more than 1024 channels reload the x buffer per chunk, in turn.  The
// head states stay in registers.
constexpr int kRopeTabW4 = 1536;  // this kernel's RoPE table: two workgroups a CU with both x and k, v tiles

// kRope: as for kv_tile_epilogue_rm (0, 1: the LDS table; 2: on the fly).
template <int kRope>
__global__ __launch_bounds__(kKvThreads, 2) void sva_kv_proj_reduce_w4a4_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xsc, const uint8_t* __restrict__ wpack,
    const float* __restrict__ bias, float* __restrict__ partials, KvGeo g) {
  __shared__ uint4 xcs[kTileM * kXPitch];
  __shared__ uint32_t xss[kTileM * kXChunkStages];
  __shared__ uint4 kvt[(kKvThreads / 64) * 512];  // wave w's k or v tile at kvt + w * 512
  __shared__ float zs[2][64];
  __shared__ float bs[kKvThreads / 64][64];
  __shared__ float2 rtab[kRope < 2 ? kRopeTabW4 : 1];
  static_assert(kTileM * kXPitch == 32 * 64 && kTileM * kXChunkStages == 8 * 64,
                "x unit: 32 code and 8 scale loads of 64 lanes, 8 and 2 a wave");

  // Tile order as in the bf16 kernel: the head pairs of one range on one XCD.
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int rg = (local / g.npairs) * 8 + xcd;
  const int pair = local % g.npairs;
  if (rg >= g.nrg) return;
  const int b = rg / g.ranges, r = rg - b * g.ranges;
  const int n_begin = r * g.L, n_end = n_begin + g.L;
  const int c = n_begin / g.Nb;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lg = lane >> 4, lr = lane & 15;
  const int half = wave & 1;
  const int head = 2 * pair + (wave >> 1);
  const int blk_k = g.H + head, blk_v = 2 * g.H + head;
  const uint8_t* cbase = wpack + ((size_t)blk_k * g.stages * 4 + 2 * half) * 1024 + lane * 16;
  const uint8_t* sbase = wpack + (size_t)g.n_pack * (g.C / 2) + ((size_t)blk_k * g.stages * 64 + lane) * 4;
  const size_t cvoff = (size_t)g.H * g.stages * 4 * 1024, svoff = (size_t)g.H * g.stages * 256;
  const int sshift = 16 * half;
  const uint32_t crow = (uint32_t)g.C / 2, srow = (uint32_t)g.C / 32;
  const long long M = (long long)(g.nrg / g.ranges) * g.N;
  const int nch = (g.stages + kXChunkStages - 1) / kXChunkStages;

  bs[wave][lane] = bias ? bias[(lane < 32 ? blk_k : blk_v) * 64 + 32 * half + (lane & 31)] : 0.f;
  if constexpr (kRope < 2) kv_build_rope_table(rtab, g, c, tid);

  // x unit (tile t, chunk j) into LDS.  Load i of wave w fills code slots
  // 64 (8 w + i) + lane, i.e. rows 2 (8 w + i) + lane / 32 at swizzled
  // position lane % 32, so the lane fetches piece (lane % 32) ^ (row & 31);
  // scale load i fills words 64 (2 w + i) + lane = (row, stage) (u / 8,
  // u % 8).  Pieces and stages past the chunk, rows past the tokens, and
  // every load past the last tile get an offset past the descriptor's
  // range: they write zeros and touch no memory.
  const int ntiles = (g.L + kTileM - 1) / kTileM;
  constexpr uint32_t kPast = 0x80000000u;
  auto load_unit = [&](int t, int j) {
    const long long m0 = (long long)b * g.N + n_begin + (long long)t * kTileM;
    const int rows = t < ntiles ? (int)min((long long)kTileM, M - m0) : 0;
    const __amdgpu_buffer_rsrc_t cr = rsrc(xq + m0 * crow, (uint32_t)rows * crow);
    const __amdgpu_buffer_rsrc_t sr = rsrc(xsc + m0 * srow, (uint32_t)rows * srow);
    const int s0 = j * kXChunkStages;
    const int ns = min(kXChunkStages, g.stages - s0);
    // Where registers are short (the per-pair RoPE modes) the lane index
    // goes through an empty asm: the offsets are then recomputed per call
    // rather than kept live (and spilled) across the tile loop.
    int ln = lane;
    if constexpr (kRope != 0) asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 2 * (8 * wave + i) + (ln >> 5);
      const int piece = (ln & 31) ^ (row & 31);
      const uint32_t off = piece < 4 * ns ? (uint32_t)row * crow + 64 * s0 + 16 * piece : kPast;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (lds_void_ptr)(xcs + 64 * (8 * wave + i)), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = 64 * (2 * wave + i) + ln;
      const int sl = u % kXChunkStages;
      const uint32_t off = sl < ns ? (uint32_t)(u / kXChunkStages) * srow + 4 * (s0 + sl) : kPast;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void_ptr)(xss + 64 * (2 * wave + i)), 4, off, 0, 0, 0);
    }
  };
  // Every wave's loads of the unit have landed in LDS: each wave waits for
  // its own (vmcnt(0)), then the workgroup meets.  The empty asm statements
  // keep the compiler from moving LDS accesses across.
  auto unit_ready = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    asm volatile("" ::: "memory");
  };
  // accumulators 0, 1: k row tiles; 2, 3: v row tiles
  auto load_w = [&](KvWRegs& w, int s) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
      w.c[rt] = *(const uint4*)(cbase + (rt < 2 ? 0 : cvoff) + ((size_t)s * 4 + (rt & 1)) * 1024);
    w.sk = *(const uint32_t*)(sbase + (size_t)s * 256);
    w.sv = *(const uint32_t*)(sbase + svoff + (size_t)s * 256);
  };

  pj_floatx4 sa[2][4];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int fc = 0; fc < 4; ++fc) sa[ft][fc] = pj_floatx4{0.f, 0.f, 0.f, 0.f};
  float zt[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zt[i] = 0.f;

  // The weights go by pairs of stages (C is a multiple of 256) in a ring of
  // two register pairs: pair q + 1 loads while pair q computes, so every
  // load is issued two stages before its use (one stage ahead left each
  // stage waiting for L2).  The weights do not depend on the token tile: the
  // pair after a tile's last is its pair 0, for the next tile, and it loads
  // during the tile's last pair.
  const int np = g.stages / 2;
  auto load_pair = [&](KvWRegs (&w)[2], int q) {
    load_w(w[0], 2 * q);
    load_w(w[1], 2 * q + 1);
  };
  KvWRegs P0[2], P1[2];
  load_pair(P0, 0);
  load_unit(0, 0);
  for (int it = 0; it < ntiles; ++it) {
    const int n0 = n_begin + it * kTileM;
    // The accumulators start from the bias: row tile rt, entry i of lane
    // (lg, .) is feature 8 lg + 4 (rt % 2) + i of the wave's k (rt < 2) or
    // v features.
    pj_floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 b4 = *reinterpret_cast<const float4*>(&bs[wave][32 * (i >> 1) + 8 * lg + 4 * (i & 1)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = pj_floatx4{b4.x, b4.y, b4.z, b4.w};
    }
    // one stage from chunk-local stage sl: B operands and scales from LDS,
    // the weights' scale bytes of this wave's row tiles gathered into one
    // word (k tiles in bytes 0, 1; v tiles in 2, 3) for op_sel
    auto compute = [&](const KvWRegs& w, int sl) {
      uint32_t ek = w.sk, ev = w.sv;
      asm volatile("" : "+v"(ek));
      asm volatile("" : "+v"(ev));
      const uint32_t e = ((ek >> sshift) & 0xffffu) | ((ev >> sshift) << 16);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int row = tt * 16 + lr;
        const uint4 bo = xcs[row * kXPitch + ((4 * sl + lg) ^ (row & 31))];
        const uint32_t sb = (xss[row * kXChunkStages + sl] >> (8 * lg)) & 0xffu;
        acc[0][tt] = mfma_fp4<0>(w.c[0], e, bo, sb, acc[0][tt]);
        acc[1][tt] = mfma_fp4<1>(w.c[1], e, bo, sb, acc[1][tt]);
        acc[2][tt] = mfma_fp4<2>(w.c[2], e, bo, sb, acc[2][tt]);
        acc[3][tt] = mfma_fp4<3>(w.c[3], e, bo, sb, acc[3][tt]);
      }
    };
    for (int j = 0; j < nch; ++j) {
      if (j > 0) {  // past 1024 channels: the next chunk, once every wave is done with this one
        __syncthreads();
        load_unit(it, j);
      }
      unit_ready();
      const int q0 = j * (kXChunkStages / 2);                   // the chunk's first pair
      const int nq = min(kXChunkStages, g.stages - 2 * q0) / 2;  // its pairs
      int ql = 0;
      for (; ql + 2 <= nq; ql += 2) {
        const int q = q0 + ql;
        load_pair(P1, (q + 1) % np);
        __builtin_amdgcn_sched_barrier(0);
        compute(P0[0], 2 * ql);
        compute(P0[1], 2 * ql + 1);
        __builtin_amdgcn_sched_barrier(0);
        load_pair(P0, (q + 2) % np);
        __builtin_amdgcn_sched_barrier(0);
        compute(P1[0], 2 * ql + 2);
        compute(P1[1], 2 * ql + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ql < nq) {  // an odd pair count: the last pair, then the ring shifts
        load_pair(P1, (q0 + ql + 1) % np);
        __builtin_amdgcn_sched_barrier(0);
        compute(P0[0], 2 * ql);
        compute(P0[1], 2 * ql + 1);
        __builtin_amdgcn_sched_barrier(0);
        P0[0] = P1[0];
        P0[1] = P1[1];
      }
    }
    // Every wave is done with the x buffer: the next tile's first chunk
    // loads into it during the epilogue.  (Barriers on LDS alone from here
    // on: the weight and x loads in flight stay in flight.)
    asm volatile("" ::: "memory");
    lds_sync();
    asm volatile("" ::: "memory");
    load_unit(it + 1, 0);
    // (in the per-pair modes, lg through an empty asm: their RoPE constants
    // are then set per tile instead of occupying registers through the GEMM)
    int lgv = lg;
    if constexpr (kRope != 0) asm volatile("" : "+v"(lgv));
    if (n0 + kTileM <= n_end)
      kv_tile_epilogue_rm<kRope, true>(acc, g, rtab, kvt, zt, wave, half, lg, lgv, lr, n0, n_end, c);
    else
      kv_tile_epilogue_rm<kRope, false>(acc, g, rtab, kvt, zt, wave, half, lg, lgv, lr, n0, n_end, c);
    asm volatile("" ::: "memory");
    lds_sync();
    asm volatile("" ::: "memory");
    kv_state_mfma_tr(sa, kvt, wave, half, lane);
  }
  kv_z_reduce(zt, zs[wave >> 1], half, lg, lr);
  __syncthreads();  // zs complete
  kv_store_partial(sa, zs[wave >> 1], partials, g, b, head, r, c, half, lg, lr, lane);
}

// ---------------------------------------------------------------------------
// The q projection fused with the output pass, on 4-bit activations.
//
// A workgroup takes `tpw` consecutive 64-token tiles of one block of one
// sample and four heads (a quad): wave w computes q of head 4 quad + w (all 64
// features) with the 4-bit GEMM of the k, v kernel (the x tile in LDS by
// buffer loads with the lds bit, the weights two stages ahead), and applies
// the output pass in its epilogue: q (bias included: the accumulators start
// from it) is rounded to bf16 as a stored tensor would be; phi gives phi q
// for the RoPE-free denominator and the rotation of its position q~ for the
// numerator; out = (q~ S_c) / (phi q . Z_c + eps) with the block's prefix
// state S_c, Z_c from the scan.  The numerator runs on MFMA, transposed
// (out^T = S_c^T q~^T): the GEMM leaves lane (lg, lr) features 8 lg + 0..7
// and 32 + 8 lg + 0..7 of token lr -- exactly the B operand of the two
// k-steps over the 64 q features -- and A holds rows of S_c^T (the scan's
// bf16 operands, in registers for the whole workgroup), its rows permuted
// like the projection's so that the lane's outputs are again two runs of 8
// consecutive features, stored as 16-byte pieces.  The denominator is an
// fp32 dot on the VALU.  q never reaches HBM; out past the block's last
// token falls outside the store descriptor and is dropped.
// ---------------------------------------------------------------------------

// kRope: as for kv_tile_epilogue_rm (0, 1: the LDS table; 2: on the fly).
// kW4: 4-bit activations (xin: the codes, xsc: the scales), else bf16
// activations (xin: x [B, N, C]; xsc unused).
template <int kRope, bool kW4>
__global__ __launch_bounds__(kKvThreads, 2) void sva_q_proj_apply_kernel(
    const void* __restrict__ xin, const uint8_t* __restrict__ xsc, const uint8_t* __restrict__ wpack,
    const float* __restrict__ bias, const uint16_t* __restrict__ frags, const float* __restrict__ zc,
    uint16_t* __restrict__ out, QaGeo g) {
  // x: a 4-bit tile's codes (one chunk) and scale words, or two 128-channel
  // bf16 stages of the tile (the same 32 KiB)
  __shared__ uint4 xcs[kTileM * kXPitch];
  __shared__ uint32_t xss[kW4 ? kTileM * kXChunkStages : 1];
  static_assert(kTileM * kXPitch == 2 * kXU4, "two bf16 stages fill the 4-bit chunk's buffer");
  __shared__ float2 rtab[kRope < 2 ? kRopeTabW4 : 1];
  __shared__ float bz[kKvThreads / 64][2][64];  // per wave: the head's q bias, then Z_c
  // The S_c^T operands stay in registers for the 4-bit GEMM; the bf16 GEMM
  // needs those registers, so there they wait in LDS (one uint4 a lane per
  // output row tile and k-step) and are read per tile.
  constexpr bool kSaLds = !kW4;
  __shared__ uint4 sal[kSaLds ? (kKvThreads / 64) * 8 * 64 : 1];

  // Tile order: the four head quads of one tile group on one XCD (they read
  // the same x).
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int tg = (local / g.nquads) * 8 + xcd;
  const int quad = local % g.nquads;
  if (tg >= g.ngrp) return;
  const int b = tg / (g.nb * g.groups);
  const int rem = tg - b * g.nb * g.groups;
  const int c = rem / g.groups, grp = rem - c * g.groups;
  const int t_begin = grp * g.tpw, t_end = min(t_begin + g.tpw, g.tiles_blk);
  const int blk0 = c * g.Nb;               // the block's first token
  const int n_end = blk0 + g.Nb;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lg = lane >> 4, lr = lane & 15;
  // With H not a multiple of 4 the last quad's waves past the heads compute
  // head H - 1 again (every load stays in bounds) and store nothing.
  const bool live = 4 * quad + wave < g.H;
  const int head = min(4 * quad + wave, g.H - 1);
  const uint8_t* cbase = wpack + ((size_t)head * g.stages * 4) * 1024 + lane * 16;
  const uint8_t* sbase = wpack + (size_t)g.n_pack * (g.C / 2) + ((size_t)head * g.stages * 64 + lane) * 4;
  const long long M = (long long)(g.ngrp / (g.nb * g.groups)) * g.N;
  const long long bh = (long long)b * g.H + head;
  const long long bhc = bh * g.nb + c;

  if constexpr (kRope < 2) kv_build_rope_table(rtab, g, c, tid);

  // The block's prefix state for this head: A operands of S_c^T rows
  // fo(ot, lr) (the projection's row permutation), k-steps of 32 q features;
  // Z_c at the lane's 16 features.
  uint4 sA[kSaLds ? 1 : 4][2];
#pragma unroll
  for (int ot = 0; ot < 4; ++ot) {
    const int fo_row = 32 * (ot >> 1) + 8 * (lr >> 2) + 4 * (ot & 1) + (lr & 3);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4*>(frags + (bhc * 64 + fo_row) * 64 + 32 * ks + 8 * lg);
      if constexpr (kSaLds) sal[(wave * 8 + 2 * ot + ks) * 64 + lane] = v;
      else sA[ot][ks] = v;
    }
  }
  // the head's q bias and Z_c, read per tile from LDS (read first after
  // the first barrier)
  bz[wave][0][lane] = bias ? bias[head * 64 + lane] : 0.f;
  bz[wave][1][lane] = zc[bhc * 64 + lane];

  // The output rows of this head: a store past the block's last token is
  // outside the descriptor and dropped.
  const __amdgpu_buffer_rsrc_t orr =
      rsrc(out + (bh * g.N + blk0) * 64, (uint32_t)g.Nb * 128u);

  // RoPE of the lane's 8 pairs: features 8 lg + 2 pp (group 0) and
  // 32 + 8 lg + 2 pp (group 1), pp = 0..3
  const int off_h = g.F * (g.dt >> 1), off_w = off_h + g.Hs * (g.dh >> 1);
  int lgv = lg;
  if constexpr (kRope != 0) asm volatile("" : "+v"(lgv));

  auto load_w = [&](WRegs& w, int s) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) w.c[rt] = *(const uint4*)(cbase + ((size_t)s * 4 + rt) * 1024);
    w.s = *(const uint32_t*)(sbase + (size_t)s * 256);
  };
  // The output pass of tile n0 .. n0 + 63 from the GEMM's accumulators.
  auto output_pass = [&](const pj_floatx4 (&acc)[4][4], int n0) {
      // RoPE constants of the lane's two 8-feature groups
      float inv[2][4], tbase[2][4];
      int axis[2][4], eoff[2][4], estr[2][4];
  #pragma unroll
      for (int gq = 0; gq < 2; ++gq)
  #pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int f = 32 * gq + 8 * lgv + 2 * pp;
          const int ax = f < g.dt ? 0 : f < g.dt + g.dh ? 1 : 2;
          const int start = ax == 0 ? 0 : ax == 1 ? g.dt : g.dt + g.dh;
          const int width = ax == 0 ? g.dt : ax == 1 ? g.dh : 64 - g.dt - g.dh;
          axis[gq][pp] = ax;
          if constexpr (kRope < 2) {
            eoff[gq][pp] = (ax == 0 ? 0 : ax == 1 ? off_h : off_w) + ((f - start) >> 1);
            estr[gq][pp] = width >> 1;
          } else {
            const double inv_d = exp2(-(double)(f - start) / (double)width * g.log2_base_d) * 0.15915494309189535;
            double tb = ax == 0 ? (double)(g.t0 + c * g.F) * inv_d : 0.0;
            tb -= rint(tb);
            inv[gq][pp] = (float)inv_d;
            tbase[gq][pp] = (float)tb;
          }
        }
  #pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int tok = 16 * tt + lr;
        const int n = n0 + tok;
        // q rounded to bf16, then phi on the bit pattern (every value with the
        // sign bit set becomes +0): features 32 gq + 8 lg + i, i = 0..7, from
        // accumulators 2 gq + i / 4, entry i % 4
        float ph[2][8];
  #pragma unroll
        for (int gq = 0; gq < 2; ++gq)
  #pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int rt = 2 * gq + (m >> 1);
            const uint32_t w = pack2(acc[rt][tt][2 * (m & 1)], acc[rt][tt][2 * (m & 1) + 1]);
            ph[gq][2 * m] = __int_as_float(max((int)(w << 16), 0));
            ph[gq][2 * m + 1] = __int_as_float(max((int)(w & 0xffff0000u), 0));
          }
        // denominator: phi q . Z_c over the 64 features (16 a lane, then the
        // four lane groups), fp32
        float den = 0.f;
  #pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
          const float4 z0 = *reinterpret_cast<const float4*>(&bz[wave][1][32 * gq + 8 * lg]);
          const float4 z1 = *reinterpret_cast<const float4*>(&bz[wave][1][32 * gq + 8 * lg + 4]);
          const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
  #pragma unroll
          for (int i = 0; i < 8; ++i) den = fmaf(ph[gq][i], zz[i], den);
        }
        den += __shfl_xor(den, 16);
        den += __shfl_xor(den, 32);
        if (g.rope) {
          const uint32_t np_ = (uint32_t)min(n, n_end - 1);  // positions past the block: any in it
          const uint32_t fr = fdiv(np_, g.fHW), rm = np_ - fr * g.fHW.div;
          const uint32_t row = fdiv(rm, g.fWs);
          const int pt = (int)fr - c * g.F;
          const int phh = (int)row, pw = (int)(rm - row * g.fWs.div);
  #pragma unroll
          for (int gq = 0; gq < 2; ++gq) {
            const int ps0 = axis[gq][0] == 0 ? pt : axis[gq][0] == 1 ? phh : pw;
            const int e0 = eoff[gq][0] + ps0 * estr[gq][0];
  #pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              float sn, cs;
              if constexpr (kRope == 0) {
                const float2 e = rtab[e0 + pp];
                cs = e.x, sn = e.y;
              } else if constexpr (kRope == 1) {
                const int ax = axis[gq][pp];
                const int ps = ax == 0 ? pt : ax == 1 ? phh : pw;
                const float2 e = rtab[eoff[gq][pp] + ps * estr[gq][pp]];
                cs = e.x, sn = e.y;
              } else {
                const int ax = axis[gq][pp];
                const int ps = ax == 0 ? pt : ax == 1 ? phh : pw;
                const float turn = __builtin_amdgcn_fractf(tbase[gq][pp] + (float)ps * inv[gq][pp]);
                sn = __builtin_amdgcn_sinf(turn), cs = __builtin_amdgcn_cosf(turn);
              }
              const float x = ph[gq][2 * pp], y = ph[gq][2 * pp + 1];
              ph[gq][2 * pp] = x * cs - y * sn;
              ph[gq][2 * pp + 1] = x * sn + y * cs;
            }
          }
        }
        // numerator: out^T rows fo(ot, .) = sum over the 64 q features
        const uint4 B0 = make_uint4(pack2(ph[0][0], ph[0][1]), pack2(ph[0][2], ph[0][3]), pack2(ph[0][4], ph[0][5]),
                                    pack2(ph[0][6], ph[0][7]));
        const uint4 B1 = make_uint4(pack2(ph[1][0], ph[1][1]), pack2(ph[1][2], ph[1][3]), pack2(ph[1][4], ph[1][5]),
                                    pack2(ph[1][6], ph[1][7]));
        pj_floatx4 o[4];
  #pragma unroll
        for (int ot = 0; ot < 4; ++ot) {
          uint4 a0, a1;
          if constexpr (kSaLds) {
            a0 = sal[(wave * 8 + 2 * ot) * 64 + lane];
            a1 = sal[(wave * 8 + 2 * ot + 1) * 64 + lane];
          } else {
            a0 = sA[ot][0];
            a1 = sA[ot][1];
          }
          o[ot] = mfma(a0, B0, pj_floatx4{0.f, 0.f, 0.f, 0.f});
          o[ot] = mfma(a1, B1, o[ot]);
        }
        const float r = __builtin_amdgcn_rcpf(den + g.eps);
        // lane (lg, lr): output features 8 lg + 0..7 (accumulators 0, 1) and
        // 32 + 8 lg + 0..7 (2, 3) of token lr
  #pragma unroll
        for (int gq = 0; gq < 2 && live; ++gq) {
          const pj_floatx4 a0 = o[2 * gq], a1 = o[2 * gq + 1];
          const uint32_t w4[4] = {pack2(a0[0] * r, a0[1] * r), pack2(a0[2] * r, a0[3] * r),
                                  pack2(a1[0] * r, a1[1] * r), pack2(a1[2] * r, a1[3] * r)};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(pj_u32x4, make_uint4(w4[0], w4[1], w4[2], w4[3])),
                                                 orr, (uint32_t)(n - blk0) * 128u + 64 * gq + 16 * lg, 0, 0);
        }
      }
  };

  if constexpr (kW4) {
    // x unit (tile t of the block, chunk j): as in the k, v kernel.
    const uint8_t* const xq = (const uint8_t*)xin;
    const uint32_t crow = (uint32_t)g.C / 2, srow = (uint32_t)g.C / 32;
    const int nch = (g.stages + kXChunkStages - 1) / kXChunkStages;
    constexpr uint32_t kPast = 0x80000000u;
    auto load_unit = [&](int t, int j) {
      const long long m0 = (long long)b * g.N + blk0 + (long long)t * kTileM;
      const int rows = t < t_end ? (int)min((long long)kTileM, M - m0) : 0;
      const __amdgpu_buffer_rsrc_t cr = rsrc(xq + m0 * crow, (uint32_t)rows * crow);
      const __amdgpu_buffer_rsrc_t sr = rsrc(xsc + m0 * srow, (uint32_t)rows * srow);
      const int s0 = j * kXChunkStages;
      const int ns = min(kXChunkStages, g.stages - s0);
      int ln = lane;
      if constexpr (kRope != 0) asm volatile("" : "+v"(ln));
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 2 * (8 * wave + i) + (ln >> 5);
        const int piece = (ln & 31) ^ (row & 31);
        const uint32_t off = piece < 4 * ns ? (uint32_t)row * crow + 64 * s0 + 16 * piece : kPast;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (lds_void_ptr)(xcs + 64 * (8 * wave + i)), 16, off, 0, 0, 0);
      }
  #pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int u = 64 * (2 * wave + i) + ln;
        const int sl = u % kXChunkStages;
        const uint32_t off = sl < ns ? (uint32_t)(u / kXChunkStages) * srow + 4 * (s0 + sl) : kPast;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void_ptr)(xss + 64 * (2 * wave + i)), 4, off, 0, 0, 0);
      }
    };
    auto unit_ready = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      asm volatile("" ::: "memory");
    };
    const int np = g.stages / 2;
    auto load_pair = [&](WRegs (&w)[2], int q) {
      load_w(w[0], 2 * q);
      load_w(w[1], 2 * q + 1);
    };

    WRegs P0[2], P1[2];
    load_pair(P0, 0);
    load_unit(t_begin, 0);
    for (int t = t_begin; t < t_end; ++t) {
      const int n0 = blk0 + t * kTileM;
      // the accumulators start from the bias: row tile rt, entry i of lane
      // (lg, .) is feature 32 (rt / 2) + 8 lg + 4 (rt % 2) + i
      pj_floatx4 acc[4][4];
  #pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float4 b4 = *reinterpret_cast<const float4*>(&bz[wave][0][32 * (rt >> 1) + 8 * lg + 4 * (rt & 1)]);
  #pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = pj_floatx4{b4.x, b4.y, b4.z, b4.w};
      }
      auto compute = [&](const WRegs& w, int sl) {
  #pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int row = tt * 16 + lr;
          const uint4 bo = xcs[row * kXPitch + ((4 * sl + lg) ^ (row & 31))];
          const uint32_t sb = (xss[row * kXChunkStages + sl] >> (8 * lg)) & 0xffu;
          acc[0][tt] = mfma_fp4<0>(w.c[0], w.s, bo, sb, acc[0][tt]);
          acc[1][tt] = mfma_fp4<1>(w.c[1], w.s, bo, sb, acc[1][tt]);
          acc[2][tt] = mfma_fp4<2>(w.c[2], w.s, bo, sb, acc[2][tt]);
          acc[3][tt] = mfma_fp4<3>(w.c[3], w.s, bo, sb, acc[3][tt]);
        }
      };
      for (int j = 0; j < nch; ++j) {
        if (j > 0) {  // past 1024 channels: the next chunk, once every wave is done with this one
          __syncthreads();
          load_unit(t, j);
        }
        unit_ready();
        const int q0 = j * (kXChunkStages / 2);
        const int nq = min(kXChunkStages, g.stages - 2 * q0) / 2;
        int ql = 0;
        for (; ql + 2 <= nq; ql += 2) {
          const int q = q0 + ql;
          load_pair(P1, (q + 1) % np);
          __builtin_amdgcn_sched_barrier(0);
          compute(P0[0], 2 * ql);
          compute(P0[1], 2 * ql + 1);
          __builtin_amdgcn_sched_barrier(0);
          load_pair(P0, (q + 2) % np);
          __builtin_amdgcn_sched_barrier(0);
          compute(P1[0], 2 * ql + 2);
          compute(P1[1], 2 * ql + 3);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (ql < nq) {
          load_pair(P1, (q0 + ql + 1) % np);
          __builtin_amdgcn_sched_barrier(0);
          compute(P0[0], 2 * ql);
          compute(P0[1], 2 * ql + 1);
          __builtin_amdgcn_sched_barrier(0);
          P0[0] = P1[0];
          P0[1] = P1[1];
        }
      }
      // Every wave is done with the x buffer: the next tile loads into it
      // while this one's output pass runs (registers and global memory only,
      // apart from the RoPE table).
      asm volatile("" ::: "memory");
      lds_sync();
      asm volatile("" ::: "memory");
      load_unit(t + 1, 0);

      output_pass(acc, n0);
    }
  } else {
    // bf16 activations: the W4A16 projection's GEMM per tile (x stages
    // through registers into the two LDS buffers, the weights decoded per
    // k-step one stage ahead), its pipeline restarted per tile.
    const size_t row_bytes = (size_t)g.C * 2;
    const int last = g.stages - 1;
    for (int t = t_begin; t < t_end; ++t) {
      const int n0 = blk0 + t * kTileM;
      const long long m0 = (long long)b * g.N + n0;
      const int rows = (int)min((long long)kTileM, M - m0);
      const __amdgpu_buffer_rsrc_t xr = rsrc((const char*)xin + m0 * row_bytes, (uint32_t)(rows * row_bytes));
      auto load_x = [&](uint4 (&r)[kXLoads], int s) {
        const int k0 = s * kTileK;
  #pragma unroll
        for (int j = 0; j < kXLoads; ++j) {
          const int u = tid + j * kKvThreads;
          const uint32_t off = (uint32_t)((u / kPieces) * row_bytes + (size_t)k0 * 2 + 16 * (u % kPieces));
          r[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
        }
      };
      auto store_x = [&](const uint4 (&r)[kXLoads], int buf) {
  #pragma unroll
        for (int j = 0; j < kXLoads; ++j) {
          const int u = tid + j * kKvThreads;
          xcs[buf * kXU4 + sw(u / kPieces, u % kPieces)] = r[j];
        }
      };
      // the accumulators start from the bias: row tile rt, entry i of lane
      // (lg, .) is feature 32 (rt / 2) + 8 lg + 4 (rt % 2) + i
      pj_floatx4 acc[4][4];
  #pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float4 b4 = *reinterpret_cast<const float4*>(&bz[wave][0][32 * (rt >> 1) + 8 * lg + 4 * (rt & 1)]);
  #pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = pj_floatx4{b4.x, b4.y, b4.z, b4.w};
      }
      auto compute = [&](const WRegs& w, int buf) {
        uint32_t e = w.s;
        asm volatile("" : "+v"(e));  // see the projection kernel
        float sc[4];
  #pragma unroll
        for (int rt = 0; rt < 4; ++rt) sc[rt] = e8m0_scale((e >> (8 * rt)) & 0xffu);
  #pragma unroll
        for (int j = 0; j < kTileK / 32; ++j) {
          uint4 a[4], bo[4];
  #pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const uint32_t cw = j == 0 ? w.c[rt].x : j == 1 ? w.c[rt].y : j == 2 ? w.c[rt].z : w.c[rt].w;
            a[rt] = decode8(cw, sc[rt]);
          }
  #pragma unroll
          for (int tt = 0; tt < 4; ++tt) bo[tt] = xcs[buf * kXU4 + sw(tt * 16 + lr, 4 * lg + j)];
  #pragma unroll
          for (int rt = 0; rt < 4; ++rt)
  #pragma unroll
            for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = mfma(a[rt], bo[tt], acc[rt][tt]);
        }
      };
      // the projection kernel's pipeline: stage s from LDS buffer s % 2, stage
      // s + 1's x in registers, stage s + 2's x in flight, stage s + 1's
      // weights requested before stage s's MFMAs
      uint4 x0[kXLoads], x1[kXLoads];
      WRegs w0, w1;
      load_w(w0, 0);
      load_x(x0, 0);
      load_x(x1, min(1, last));
      store_x(x0, 0);
      load_x(x0, min(2, last));
      __syncthreads();
      auto step = [&](int st, const WRegs& wc, WRegs& wn_, uint4 (&xn)[kXLoads]) {
        load_w(wn_, min(st + 1, last));
        __builtin_amdgcn_sched_barrier(0);
        compute(wc, st & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 < g.stages) store_x(xn, (st + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        load_x(xn, min(st + 3, last));
        __syncthreads();
      };
      int st = 0;
      for (; st + 2 <= g.stages; st += 2) {
        step(st, w0, w1, x1);
        step(st + 1, w1, w0, x0);
      }
      if (st < g.stages) step(st, w0, w1, x1);
      output_pass(acc, n0);
    }
  }
}

// Repacks natural-layout MXFP4 weights (codes [n_out, C/2], scales
// [n_out, C/32]) into the projection's layout: thread (blk, s, lane) writes
// the lane's 16 code bytes of each row tile rt of 64-feature block blk and
// stage s, and the word of their four scale bytes.
__global__ void sva_mxfp4_pack_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                      uint8_t* __restrict__ wpack, int n_out, int C, int stages, int total) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int lane = t & 63, lg = lane >> 4, lr = lane & 15;
  const int s = (t >> 6) % stages, blk = (t >> 6) / stages;
  uint32_t sw_word = 0;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int n = blk * 64 + fo(rt, lr);
    const uint4 c = *(const uint4*)(codes + (size_t)n * (C / 2) + 64 * s + 16 * lg);
    *(uint4*)(wpack + (((size_t)blk * stages + s) * 4 + rt) * 1024 + lane * 16) = c;
    sw_word |= (uint32_t)scales[(size_t)n * (C / 32) + 4 * s + lg] << (8 * rt);
  }
  *(uint32_t*)(wpack + (size_t)n_out * (C / 2) + (((size_t)blk * stages + s) * 64 + lane) * 4) = sw_word;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bn && y < x + an;
}

// Shape checks shared by both entry points.
sva_status check_desc(const sva_proj_desc* desc) {
  if (!desc) return SVA_ERR_INVALID_ARG;
  const sva_proj_desc& d = *desc;
  if (d.B < 1 || d.N < 1 || d.C < 1 || d.H < 1 || d.d < 1) return SVA_ERR_INVALID_ARG;
  if (d.C % kTileK != 0 || (d.H * (long long)d.d) % 64 != 0 || d.d % 8 != 0) return SVA_ERR_UNSUPPORTED;
  const long long M = (long long)d.B * d.N;
  const long long Mt = (M + kTileM - 1) / kTileM;
  const long long Nt = (3LL * d.H * d.d + kTileN - 1) / kTileN;
  if (M >= (1LL << 31) || (long long)kTileM * d.C * 2 >= (1LL << 31) || (Mt + 7) / 8 * 8 * Nt >= (1LL << 31) ||
      3LL * d.H * d.d * d.C >= (1LL << 31))
    return SVA_ERR_UNSUPPORTED;
  return SVA_OK;
}

size_t packed_bytes(const sva_proj_desc& d) {
  const size_t n_out = 3 * (size_t)d.H * d.d;
  return n_out * d.C / 2 + n_out * d.C / 32;
}

// 4-bit activations: codes [B N, C / 2] then scales [B N, C / 32].
size_t acts_bytes(const sva_proj_desc& d) {
  const size_t M = (size_t)d.B * d.N;
  return M * d.C / 2 + M * d.C / 32;
}

}  // namespace

extern "C" sva_status sva_mxfp4_pack_weights(const sva_proj_desc* desc, const void* codes, const void* scales,
                                             void* wpack, void* stream) {
  const sva_status st = check_desc(desc);
  if (st != SVA_OK) return st;
  const sva_proj_desc& d = *desc;
  if (!codes || !scales || !wpack) return SVA_ERR_INVALID_ARG;
  if (!aligned(codes, 16) || !aligned(wpack, 16)) return SVA_ERR_INVALID_ARG;
  const int n_out = 3 * d.H * d.d;
  const size_t cb = (size_t)n_out * d.C / 2, sb = (size_t)n_out * d.C / 32, pb = packed_bytes(d);
  if (overlap(wpack, pb, codes, cb) || overlap(wpack, pb, scales, sb)) return SVA_ERR_INVALID_ARG;
  const int stages = d.C / kTileK;
  const int total = n_out / 64 * stages * 64;
  const uint8_t* cp = (const uint8_t*)codes;
  const uint8_t* sp = (const uint8_t*)scales;
  uint8_t* wp = (uint8_t*)wpack;
  int C = d.C;
  int n = n_out;
  void* args[] = {(void*)&cp, (void*)&sp, (void*)&wp, &n, &C, (void*)&stages, (void*)&total};
  if (hipLaunchKernel((const void*)&sva_mxfp4_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), args,
                      0, (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

sva_status sva_internal_proj_features(const sva_proj_desc* desc, const void* x, const void* wpack,
                                      const float* bias, int f_end, void* q, void* k, void* v, void* stream) {
  const sva_status st = check_desc(desc);
  if (st != SVA_OK) return st;
  const sva_proj_desc& d = *desc;
  if (!x || !wpack || !q || !k || !v) return SVA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(wpack, 16) ||
      (bias && !aligned(bias, 16)))
    return SVA_ERR_INVALID_ARG;
  const int n_pack = 3 * d.H * d.d;
  if (f_end < 64 || f_end > n_pack || f_end % 64 != 0) return SVA_ERR_INVALID_ARG;
  const long long M = (long long)d.B * d.N;
  const long long Mt = (M + kTileM - 1) / kTileM;
  const long long Nt = (f_end + kTileN - 1) / kTileN;
  const long long grid = (Mt + 7) / 8 * 8 * Nt;
  const size_t xb = (size_t)M * d.C * 2, ob = (size_t)M * d.H * d.d * 2, pb = packed_bytes(d);
  const size_t bb = 3 * (size_t)d.H * d.d * 4;
  // the outputs that features [0, f_end) reach
  void* outs[3] = {q, k, v};
  const int n_outs = (f_end + d.H * d.d - 1) / (d.H * d.d);
  for (int i = 0; i < n_outs; ++i) {
    if (overlap(outs[i], ob, x, xb) || overlap(outs[i], ob, wpack, pb) || (bias && overlap(outs[i], ob, bias, bb)))
      return SVA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], ob, outs[j], ob)) return SVA_ERR_INVALID_ARG;
  }
  ProjGeo g;
  g.M = (int)M;
  g.N = d.N;
  g.C = d.C;
  g.H = d.H;
  g.d = d.d;
  g.n_out = f_end;
  g.n_pack = n_pack;
  g.Mt = (int)Mt;
  g.Nt = (int)Nt;
  g.stages = d.C / kTileK;
  g.fN = make_fastdiv((uint32_t)d.N);
  g.fHD = make_fastdiv((uint32_t)(d.H * d.d));
  g.fd = make_fastdiv((uint32_t)d.d);
  const uint8_t* wp = (const uint8_t*)wpack;
  void* args[] = {(void*)&x, (void*)&wp, (void*)&bias, (void*)&q, (void*)&k, (void*)&v, &g};
  if (hipLaunchKernel((const void*)&sva_qkv_proj_kernel, dim3((unsigned)grid), dim3(kPjThreads), args, 0,
                      (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

namespace {

// The fused k, v kernels' geometry; false where the kernels' pipeline does
// not apply (it carries the next tile's first weight stage through the
// epilogue in fixed registers, which takes an even stage count).
bool make_kv_geo(const SvaKvReduceArgs& a, KvGeo* out) {
  if (a.C % (2 * kTileK) != 0 || a.C < 2 * kTileK || a.H % 2 != 0 || a.L <= 0 || a.N % a.L != 0) return false;
  KvGeo& g = *out;
  g.N = a.N;
  g.C = a.C;
  g.H = a.H;
  g.n_pack = 3 * a.H * 64;
  g.stages = a.C / kTileK;
  g.L = a.L;
  g.ranges = a.N / a.L;
  g.Nb = a.Nb;
  g.nb = a.nb;
  g.npairs = a.H / 2;
  g.nrg = a.B * g.ranges;
  g.Hs = a.Hs;
  g.Ws = a.Ws;
  g.fHW = make_fastdiv((uint32_t)(a.Hs * a.Ws));
  g.fWs = make_fastdiv((uint32_t)a.Ws);
  g.t0 = a.t0;
  g.rope = a.rope;
  g.dt = a.dt;
  g.dh = a.dh;
  g.log2_base_d = log2((double)a.rope_base);
  g.F = a.Nb / (a.Hs * a.Ws);
  g.tab_entries = g.F * (a.dt / 2) + a.Hs * (a.dh / 2) + a.Ws * ((64 - a.dt - a.dh) / 2);
  return true;
}

}  // namespace

hipError_t sva_internal_kv_proj_reduce(const SvaKvReduceArgs& a, const void* x, const void* wpack,
                                       const float* bias, float* partials, hipStream_t stream) {
  KvGeo g;
  if (!make_kv_geo(a, &g)) return hipErrorInvalidValue;
  const int mode = !a.rope ? 0 : g.tab_entries > kRopeTab ? 2 : (a.dt % 8 == 0 && a.dh % 8 == 0) ? 0 : 1;
  const long long grid = ((long long)g.nrg + 7) / 8 * 8 * g.npairs;
  const uint8_t* wp = (const uint8_t*)wpack;
  void* args[] = {(void*)&x, (void*)&wp, (void*)&bias, (void*)&partials, &g};
  const void* fn = mode == 0   ? (const void*)&sva_kv_proj_reduce_kernel<0>
                   : mode == 1 ? (const void*)&sva_kv_proj_reduce_kernel<1>
                               : (const void*)&sva_kv_proj_reduce_kernel<2>;
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kKvThreads), args, 0, stream);
}

hipError_t sva_internal_kv_proj_reduce_w4a4(const SvaKvReduceArgs& a, const void* xq, const void* wpack,
                                            const float* bias, float* partials, hipStream_t stream) {
  KvGeo g;
  if (!make_kv_geo(a, &g)) return hipErrorInvalidValue;
  // RoPE: the LDS table where it fits, the lane's 4 pairs on one axis
  // where every axis width is a multiple of 8; without RoPE the mode does
  // not matter (the epilogue skips the rotation)
  const int mode = !a.rope ? 0 : g.tab_entries > kRopeTabW4 ? 2 : (a.dt % 8 == 0 && a.dh % 8 == 0) ? 0 : 1;
  const long long grid = ((long long)g.nrg + 7) / 8 * 8 * g.npairs;
  const long long M = (long long)a.B * a.N;
  const uint8_t* codes = (const uint8_t*)xq;
  const uint8_t* scales = codes + (size_t)M * a.C / 2;
  const uint8_t* wp = (const uint8_t*)wpack;
  void* args[] = {(void*)&codes, (void*)&scales, (void*)&wp, (void*)&bias, (void*)&partials, &g};
  const void* fn = mode == 0   ? (const void*)&sva_kv_proj_reduce_w4a4_kernel<0>
                   : mode == 1 ? (const void*)&sva_kv_proj_reduce_w4a4_kernel<1>
                               : (const void*)&sva_kv_proj_reduce_w4a4_kernel<2>;
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kKvThreads), args, 0, stream);
}

hipError_t sva_internal_q_proj_apply(const SvaKvReduceArgs& a, float eps, bool w4a4, const void* x,
                                    const void* wpack, const float* bias, const void* frags, const float* zc,
                                    void* out, hipStream_t stream) {
  if (a.C % (2 * kTileK) != 0 || a.C < 2 * kTileK || a.H < 1 || a.Nb <= 0 || a.N % a.Nb != 0)
    return hipErrorInvalidValue;
  QaGeo g;
  g.N = a.N;
  g.C = a.C;
  g.H = a.H;
  g.n_pack = 3 * a.H * 64;
  g.stages = a.C / kTileK;
  g.Nb = a.Nb;
  g.nb = a.nb;
  g.tiles_blk = (a.Nb + kTileM - 1) / kTileM;
  g.nquads = (a.H + 3) / 4;
  g.fHW = make_fastdiv((uint32_t)(a.Hs * a.Ws));
  g.fWs = make_fastdiv((uint32_t)a.Ws);
  g.Hs = a.Hs;
  g.Ws = a.Ws;
  g.t0 = a.t0;
  g.rope = a.rope;
  g.dt = a.dt;
  g.dh = a.dh;
  g.log2_base_d = log2((double)a.rope_base);
  g.F = a.Nb / (a.Hs * a.Ws);
  g.tab_entries = g.F * (a.dt / 2) + a.Hs * (a.dh / 2) + a.Ws * ((64 - a.dt - a.dh) / 2);
  g.eps = eps;
  const int mode = !a.rope ? 0 : g.tab_entries > kRopeTabW4 ? 2 : (a.dt % 8 == 0 && a.dh % 8 == 0) ? 0 : 1;
  const void* fn = w4a4 ? (mode == 0   ? (const void*)&sva_q_proj_apply_kernel<0, true>
                           : mode == 1 ? (const void*)&sva_q_proj_apply_kernel<1, true>
                                       : (const void*)&sva_q_proj_apply_kernel<2, true>)
                        : (mode == 0   ? (const void*)&sva_q_proj_apply_kernel<0, false>
                           : mode == 1 ? (const void*)&sva_q_proj_apply_kernel<1, false>
                                       : (const void*)&sva_q_proj_apply_kernel<2, false>);
  // Tiles per workgroup: each workgroup pays about one tile's time for its
  // set-up (the RoPE table, the state operands, the first x tile), and the
  // workgroups run in rounds of the resident count, so take the tpw with
  // the fewest rounds x (tpw + 1) tile times.
  const long long slots = sva_internal_resident_workgroups(fn, kKvThreads, 0);
  long long best = -1;
  g.tpw = 1;
  for (int tpw = 1; tpw <= 32 && tpw <= g.tiles_blk; ++tpw) {
    const long long groups = (g.tiles_blk + tpw - 1) / tpw;
    const long long wgs = ((long long)a.B * a.nb * groups + 7) / 8 * 8 * g.nquads;
    const long long cost = (wgs + slots - 1) / slots * (tpw + 1);
    if (best < 0 || cost < best) {
      best = cost;
      g.tpw = tpw;
    }
  }
  g.groups = (g.tiles_blk + g.tpw - 1) / g.tpw;
  g.ngrp = a.B * a.nb * g.groups;
  const long long grid = ((long long)g.ngrp + 7) / 8 * 8 * g.nquads;
  if (grid >= (1LL << 31)) return hipErrorInvalidValue;
  const long long M = (long long)a.B * a.N;
  const uint8_t* scales = w4a4 ? (const uint8_t*)x + (size_t)M * a.C / 2 : nullptr;
  const uint8_t* wp = (const uint8_t*)wpack;
  const uint16_t* fr = (const uint16_t*)frags;
  uint16_t* op = (uint16_t*)out;
  void* args[] = {(void*)&x, (void*)&scales, (void*)&wp, (void*)&bias, (void*)&fr, (void*)&zc, (void*)&op, &g};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kKvThreads), args, 0, stream);
}

extern "C" sva_status sva_qkv_proj_mxfp4(const sva_proj_desc* desc, const void* x, const void* wpack,
                                         const float* bias, void* q, void* k, void* v, void* stream) {
  if (!desc) return SVA_ERR_INVALID_ARG;
  return sva_internal_proj_features(desc, x, wpack, bias, 3 * desc->H * desc->d, q, k, v, stream);
}

extern "C" sva_status sva_mxfp4_acts_bytes(const sva_proj_desc* desc, size_t* bytes) {
  if (!bytes) return SVA_ERR_INVALID_ARG;
  const sva_status st = check_desc(desc);
  if (st != SVA_OK) return st;
  *bytes = acts_bytes(*desc);
  return SVA_OK;
}

extern "C" sva_status sva_mxfp4_quant_acts(const sva_proj_desc* desc, const void* x, void* xq, void* stream) {
  const sva_status st = check_desc(desc);
  if (st != SVA_OK) return st;
  const sva_proj_desc& d = *desc;
  if (!x || !xq || !aligned(x, 16) || !aligned(xq, 16)) return SVA_ERR_INVALID_ARG;
  const long long M = (long long)d.B * d.N;
  if (overlap(xq, acts_bytes(d), x, (size_t)M * d.C * 2)) return SVA_ERR_INVALID_ARG;
  long long nblk = M * (d.C / 32);
  const long long grid = (nblk + kQuantThreads - 1) / kQuantThreads;
  if (grid >= (1LL << 31)) return SVA_ERR_UNSUPPORTED;
  const uint32_t* xp = (const uint32_t*)x;
  uint8_t* codes = (uint8_t*)xq;
  uint8_t* scales = codes + (size_t)M * d.C / 2;
  void* args[] = {(void*)&xp, (void*)&codes, (void*)&scales, (void*)&nblk};
  if (hipLaunchKernel((const void*)&sva_mxfp4_quant_kernel, dim3((unsigned)grid), dim3(kQuantThreads), args, 0,
                      (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

sva_status sva_internal_proj_w4a4_features(const sva_proj_desc* desc, const void* xq, const void* wpack,
                                           const float* bias, int f_end, void* q, void* k, void* v, void* stream) {
  const sva_status st = check_desc(desc);
  if (st != SVA_OK) return st;
  const sva_proj_desc& d = *desc;
  if (!xq || !wpack || !q || !k || !v) return SVA_ERR_INVALID_ARG;
  if (!aligned(xq, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(wpack, 16) ||
      (bias && !aligned(bias, 16)))
    return SVA_ERR_INVALID_ARG;
  const int n_pack = 3 * d.H * d.d;
  if (f_end < 64 || f_end > n_pack || f_end % 64 != 0) return SVA_ERR_INVALID_ARG;
  const long long M = (long long)d.B * d.N;
  const size_t ab = acts_bytes(d), ob = (size_t)M * d.H * d.d * 2, pb = packed_bytes(d);
  const size_t bb = (size_t)n_pack * 4;
  // the outputs that features [0, f_end) reach
  void* outs[3] = {q, k, v};
  const int n_outs = (f_end + d.H * d.d - 1) / (d.H * d.d);
  for (int i = 0; i < n_outs; ++i) {
    if (overlap(outs[i], ob, xq, ab) || overlap(outs[i], ob, wpack, pb) || (bias && overlap(outs[i], ob, bias, bb)))
      return SVA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], ob, outs[j], ob)) return SVA_ERR_INVALID_ARG;
  }
  ProjGeo g;
  g.M = (int)M;
  g.N = d.N;
  g.C = d.C;
  g.H = d.H;
  g.d = d.d;
  g.n_out = f_end;
  g.n_pack = n_pack;
  g.Mt = (int)((M + kTileM - 1) / kTileM);
  g.Nt = (f_end + kTileN - 1) / kTileN;
  g.stages = d.C / kTileK;
  g.fN = make_fastdiv((uint32_t)d.N);
  g.fHD = make_fastdiv((uint32_t)(d.H * d.d));
  g.fd = make_fastdiv((uint32_t)d.d);
  const long long grid = ((long long)g.Mt + 7) / 8 * 8 * g.Nt;
  const uint8_t* codes = (const uint8_t*)xq;
  const uint8_t* scales = codes + (size_t)M * d.C / 2;
  const uint8_t* wp = (const uint8_t*)wpack;
  void* args[] = {(void*)&codes, (void*)&scales, (void*)&wp, (void*)&bias, (void*)&q, (void*)&k, (void*)&v, &g};
  if (hipLaunchKernel((const void*)&sva_qkv_proj_w4a4_kernel, dim3((unsigned)grid), dim3(kPjThreads), args, 0,
                      (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

extern "C" sva_status sva_qkv_proj_w4a4(const sva_proj_desc* desc, const void* xq, const void* wpack,
                                        const float* bias, void* q, void* k, void* v, void* stream) {
  if (!desc) return SVA_ERR_INVALID_ARG;
  return sva_internal_proj_w4a4_features(desc, xq, wpack, bias, 3 * desc->H * desc->d, q, k, v, stream);
}
