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

#include "sva.h"
#include "sva_proj.h"

namespace {

typedef float pj_floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t pj_u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 pj_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pj_bf16x2 __attribute__((ext_vector_type(2)));

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
  int n_out;      // 3 * H * d
  int Mt, Nt;     // token tiles, feature tiles
  int stages;     // C / kTileK
};

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

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const pj_bf16x2 v = {(__bf16)a, (__bf16)b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
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
  const uint8_t* sbase = wpack + (size_t)g.n_out * (g.C / 2) + ((size_t)blk * g.stages * 64 + lane) * 4;

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

  // Epilogue: lane (lg, lr) holds, for token tile tt, features
  // fb + 8 lg + 0..7 (accumulators 0, 1) and fb + 32 + 8 lg + 0..7 (2, 3).
  const int HD = g.H * g.d;
#pragma unroll
  for (int run = 0; run < 2; ++run) {
    const int f = n0 + wn * 64 + 32 * run + 8 * lg;  // first of 8 features
    if (f >= g.n_out) continue;
    const int which = f / HD;
    const int h = (f - which * HD) / g.d;
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
      const int m = m0 + wm * 64 + tt * 16 + lr;
      if (m < g.M) {
        const int b = m / g.N, t = m - b * g.N;
        const pj_floatx4 lo = acc[2 * run][tt], hi = acc[2 * run + 1][tt];
        const uint4 v = make_uint4(pack2(lo[0] + bb[0], lo[1] + bb[1]), pack2(lo[2] + bb[2], lo[3] + bb[3]),
                                   pack2(hi[0] + bb[4], hi[1] + bb[5]), pack2(hi[2] + bb[6], hi[3] + bb[7]));
        __builtin_nontemporal_store(__builtin_bit_cast(pj_u32x4, v),
                                    (pj_u32x4*)(dst + ((((size_t)b * g.H + h) * g.N + t) * g.d + fd) * 2));
      }
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

extern "C" sva_status sva_qkv_proj_mxfp4(const sva_proj_desc* desc, const void* x, const void* wpack,
                                         const float* bias, void* q, void* k, void* v, void* stream) {
  const sva_status st = check_desc(desc);
  if (st != SVA_OK) return st;
  const sva_proj_desc& d = *desc;
  if (!x || !wpack || !q || !k || !v) return SVA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(wpack, 16) ||
      (bias && !aligned(bias, 16)))
    return SVA_ERR_INVALID_ARG;
  const long long M = (long long)d.B * d.N;
  const long long Mt = (M + kTileM - 1) / kTileM;
  const long long Nt = (3LL * d.H * d.d + kTileN - 1) / kTileN;
  const long long grid = (Mt + 7) / 8 * 8 * Nt;
  const size_t xb = (size_t)M * d.C * 2, ob = (size_t)M * d.H * d.d * 2, pb = packed_bytes(d);
  const size_t bb = 3 * (size_t)d.H * d.d * 4;
  void* outs[3] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
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
  g.n_out = 3 * d.H * d.d;
  g.Mt = (int)Mt;
  g.Nt = (int)Nt;
  g.stages = d.C / kTileK;
  const uint8_t* wp = (const uint8_t*)wpack;
  void* args[] = {(void*)&x, (void*)&wp, (void*)&bias, (void*)&q, (void*)&k, (void*)&v, &g};
  if (hipLaunchKernel((const void*)&sva_qkv_proj_kernel, dim3((unsigned)grid), dim3(kPjThreads), args, 0,
                      (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}
