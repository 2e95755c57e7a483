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
// pieces of the [B, H, N, d] rows directly.  A workgroup (8 waves) owns 128
// output features x 256 tokens; a wave 64 features x 64 tokens (4 x 4
// accumulators).  The input channels advance 64 per stage: a stage's x tile
// (256 x 64 bf16) and weight tile (128 x 64, decoded to bf16 with
// v_cvt_scalef32_pk_bf16_fp4: two 4-bit codes and their E8M0 block scale per
// instruction, exact) sit in LDS, double-buffered, with the global loads of
// the stage after next in registers.  At this tile the operand reads from LDS
// (0.5 KB an MFMA, 128 KB a stage per CU) take about as long as the MFMAs
// (measured: without them the kernel ran twice as fast).  Tried and slower:
// 128 x 128 per wave (one wave per SIMD, the accumulators in AGPRs, then
// room for one stage of prefetch only), decoding the weights per wave from
// staged 4-bit codes, two 4-wave workgroups per CU.  Consecutive workgroup
// indices go to the eight XCDs in turn, so the tiles are ordered to keep
// every workgroup that reads one x tile on the same XCD (its L2 then serves
// the 24 output tiles of a 720p QKV projection).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sva.h"
#include "sva_proj.h"

namespace {

typedef float pj_floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t pj_u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 pj_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pj_bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kPjThreads = 512;  // 8 waves
constexpr int kTileN = 128;      // output features per workgroup
constexpr int kTileM = 256;      // tokens per workgroup
constexpr int kTileK = 64;       // input channels per stage
constexpr int kPieces = kTileK * 2 / 16;        // 16-byte pieces of a row per stage
constexpr int kXU4 = kTileM * kPieces;          // x tile, 16-byte units
constexpr int kWU4 = kTileN * kPieces;          // weight tile, 16-byte units
constexpr int kXLoads = kXU4 / kPjThreads;      // x pieces per thread per stage

struct ProjGeo {
  int M;          // B * N tokens
  int N;          // tokens per sample
  int C;          // input channels
  int H, d;
  int Mt, Nt;     // token tiles, feature tiles
  int stages;     // C / kTileK
};

// Piece p of row r, XOR-swizzled with f(r) = (r & 7) ^ ((r >> 1) & 4).  A
// 16-byte LDS read is served eight lanes at a time, so the eight rows one
// such group reads must get distinct f: the B operand's groups are eight
// consecutive rows from a multiple of 8, the A operand's (fo order) rows
// {0-3, 8-11} or {4-7, 12-15} (+32): both are conflict-free, and so are the
// tile writes (8 pieces of one row; pieces {0, 2, 4, 6} of two adjacent
// rows).  r & 7 alone gave the A reads 2-way conflicts.
__device__ __forceinline__ int sw(int r, int p) { return r * kPieces + (p ^ ((r & 7) ^ ((r >> 1) & 4))); }

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

// Eight bytes of codes (16 channels, low nibble first) -> 16 bf16 weights.
__device__ __forceinline__ void decode16(uint2 c, float s, uint32_t (&o)[8]) {
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c.x, s, 0));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c.x, s, 1));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c.x, s, 2));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c.x, s, 3));
  o[4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c.y, s, 0));
  o[5] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c.y, s, 1));
  o[6] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c.y, s, 2));
  o[7] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c.y, s, 3));
}

// A stage's global data in registers: 4 pieces of x, 8 bytes of codes and
// the aligned word holding the thread's scale byte.
struct StageRegs {
  uint4 x[kXLoads];
  uint2 c;
  uint32_t s;
};

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const pj_bf16x2 v = {(__bf16)a, (__bf16)b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(kPjThreads, 1) void sva_qkv_proj_kernel(
    const void* __restrict__ xp, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ bias, void* __restrict__ qp, void* __restrict__ kp, void* __restrict__ vp,
    ProjGeo g) {
  __shared__ uint4 xs[2][kXU4];
  __shared__ uint4 ws[2][kWU4];

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
  const int wn = wave & 1, wm = wave >> 1;  // 64 features x 64 tokens each

  // x rows m0 .. m0 + 255 (rows past M read as zeros)
  const int rows = min(kTileM, g.M - m0);
  const size_t row_bytes = (size_t)g.C * 2;
  const __amdgpu_buffer_rsrc_t xr = rsrc((const char*)xp + (size_t)m0 * row_bytes, (uint32_t)(rows * row_bytes));
  // weights: thread t decodes 16 channels (half an MX block) of feature t / 4
  const int w_row = tid >> 2, w_q = tid & 3;
  const uint8_t* crow = codes + (size_t)(n0 + w_row) * (g.C / 2);
  const uint8_t* srow = scales + (size_t)(n0 + w_row) * (g.C / 32);

  auto load = [&](StageRegs& r, int s) {
    const int k0 = s * kTileK;
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int u = tid + j * kPjThreads;
      const uint32_t off = (uint32_t)((u / kPieces) * row_bytes + (size_t)k0 * 2 + 16 * (u % kPieces));
      r.x[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
    r.c = *(const uint2*)(crow + k0 / 2 + 8 * w_q);
    r.s = *(const uint32_t*)(srow + (((k0 + 16 * w_q) / 32) & ~3));
  };
  auto store = [&](const StageRegs& r, int s, int buf) {
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const int u = tid + j * kPjThreads;
      xs[buf][sw(u / kPieces, u % kPieces)] = r.x[j];
    }
    // The scale byte passes through an empty asm here: otherwise the
    // compiler masks it at the end of the previous iteration, right after
    // its load, and waits there for every load in flight.
    uint32_t sb = r.s;
    asm volatile("" : "+v"(sb));
    const int sbyte = ((s * kTileK + 16 * w_q) / 32) & 3;
    uint32_t o[8];
    decode16(r.c, e8m0_scale((sb >> (8 * sbyte)) & 0xffu), o);
    ws[buf][sw(w_row, 2 * w_q)] = make_uint4(o[0], o[1], o[2], o[3]);
    ws[buf][sw(w_row, 2 * w_q + 1)] = make_uint4(o[4], o[5], o[6], o[7]);
  };

  pj_floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = pj_floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kTileK / 32; ++ks) {
      uint4 a[4], b[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) a[rt] = ws[buf][sw(wn * 64 + fo(rt, lr), 4 * ks + lg)];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) b[tt] = xs[buf][sw(wm * 64 + tt * 16 + lr, 4 * ks + lg)];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = mfma(a[rt], b[tt], acc[rt][tt]);
    }
  };

  // Pipeline: stage s is computed from LDS buffer s % 2 while stage s + 1
  // waits in registers set (s + 1) % 2 and stage s + 2's loads are in flight.
  // Every prefetch is issued, with the stage index clamped to the last one
  // (repeat loads at the tail are in bounds and unused): a conditional load
  // leaves the compiler unsure how many loads are in flight after it, and it
  // then waits for all of them.
  const int last = g.stages - 1;
  StageRegs r0, r1;
  load(r0, 0);
  load(r1, min(1, last));
  store(r0, 0, 0);
  load(r0, min(2, last));
  __syncthreads();
  // The scheduling barriers keep the next stage's decode below the MFMAs:
  // hoisted above them, its first use of a just-loaded scale byte made the
  // wave wait for every load in flight (one in-order counter) each stage.
  auto step = [&](int s, StageRegs& nxt) {
    compute(s & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < g.stages) store(nxt, s + 1, (s + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    load(nxt, min(s + 3, last));
    __syncthreads();
  };
  int s = 0;
  for (; s + 2 <= g.stages; s += 2) {
    step(s, r1);
    step(s + 1, r0);
  }
  if (s < g.stages) step(s, r1);

  // Epilogue: lane (lg, lr) holds, for token tile tt, features
  // fb + 8 lg + 0..7 (accumulators 0, 1) and fb + 32 + 8 lg + 0..7 (2, 3).
  const int HD = g.H * g.d;
#pragma unroll
  for (int run = 0; run < 2; ++run) {
    const int f = n0 + wn * 64 + 32 * run + 8 * lg;  // first of 8 features
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
        *(uint4*)(dst + ((((size_t)b * g.H + h) * g.N + t) * g.d + fd) * 2) = v;
      }
    }
  }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bn && y < x + an;
}

}  // namespace

extern "C" sva_status sva_qkv_proj_mxfp4(const sva_proj_desc* desc, const void* x, const void* codes,
                                         const void* scales, const float* bias, void* q, void* k, void* v,
                                         void* stream) {
  if (!desc) return SVA_ERR_INVALID_ARG;
  const sva_proj_desc& d = *desc;
  if (d.B < 1 || d.N < 1 || d.C < 1 || d.H < 1 || d.d < 1) return SVA_ERR_INVALID_ARG;
  // C: whole stages, and word-aligned rows of scale bytes (C / 32 a multiple of 4)
  if (d.C % 128 != 0 || (d.H * d.d) % kTileN != 0 || d.d % 8 != 0) return SVA_ERR_UNSUPPORTED;
  const long long M = (long long)d.B * d.N;
  const long long Mt = (M + kTileM - 1) / kTileM;
  const long long Nt = 3LL * d.H * d.d / kTileN;
  const long long grid = (Mt + 7) / 8 * 8 * Nt;
  if (M >= (1LL << 31) || (long long)kTileM * d.C * 2 >= (1LL << 31) || grid >= (1LL << 31))
    return SVA_ERR_UNSUPPORTED;
  if (!x || !codes || !scales || !q || !k || !v) return SVA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(codes, 8) ||
      !aligned(scales, 4) || (bias && !aligned(bias, 16)))
    return SVA_ERR_INVALID_ARG;
  const size_t xb = (size_t)M * d.C * 2, ob = (size_t)M * d.H * d.d * 2;
  const size_t cb = 3 * (size_t)d.H * d.d * d.C / 2, sb = 3 * (size_t)d.H * d.d * d.C / 32;
  const size_t bb = 3 * (size_t)d.H * d.d * 4;
  void* outs[3] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], ob, x, xb) || overlap(outs[i], ob, codes, cb) || overlap(outs[i], ob, scales, sb) ||
        (bias && overlap(outs[i], ob, bias, bb)))
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
  g.Mt = (int)Mt;
  g.Nt = (int)Nt;
  g.stages = d.C / kTileK;
  const uint8_t* cp = (const uint8_t*)codes;
  const uint8_t* sp = (const uint8_t*)scales;
  void* args[] = {(void*)&x, (void*)&cp, (void*)&sp, (void*)&bias, (void*)&q, (void*)&k, (void*)&v, &g};
  if (hipLaunchKernel((const void*)&sva_qkv_proj_kernel, dim3((unsigned)grid), dim3(kPjThreads), args, 0,
                      (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}
