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
  float log2_base;  // log2 of the RoPE base
  double log2_base_d;
  int F;            // frames per block
  int tab_entries;  // F dt/2 + Hs dh/2 + Ws dw/2 (the RoPE table's size)
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

// ---------------------------------------------------------------------------
// k and v projections fused with the per-block state reduction.
//
// A workgroup takes a range of L tokens of one sample (L divides the block's
// token count, so a range lies in one block) and two heads h0, h0 + 1; its
// waves compute k and v of those heads (64 features each) for 64-token
// tiles with the projection's GEMM.  Instead of storing k and v, each tile's
// epilogue rounds them to bf16 (as a stored tensor would be), applies phi
// and the numerator-only 3D RoPE to k, stages both transposed in LDS and
// adds the tile's v^T RoPE(phi k) to the head's state on MFMA, and phi k to
// its normaliser.  At the end of the range each head's state and normaliser
// go to the partial slot the block scan reads for (range, block): slot g + bhc
// with g the range's index along the flattened (b, h, token) axis in units
// of L.  So k and v never reach HBM.
//
// The GEMM pipeline runs on across the tiles of a range (the next tile's
// first x and weight stages load during the epilogue), the bias sits in LDS,
// and RoPE reads cos/sin from a per-workgroup LDS table of the positions the
// range can hold (kTab), or computes them on the fly for grids whose table
// would not fit beside two workgroups per CU.
// ---------------------------------------------------------------------------

constexpr int kKvThreads = 256;  // waves: (h0, half 0), (h0, half 1), (h0+1, 0), (h0+1, 1)
static_assert(kKvThreads == kPjThreads, "the GEMM part assumes the projection's workgroup size");

// A wave's 64 x 64 bf16 tile, transposed: feature row f (128 bytes = 64
// tokens), 16-byte piece p = token / 8 at p ^ (f & 7).
__device__ __forceinline__ int kv_piece(int f, int p) { return f * 8 + (p ^ (f & 7)); }

template <bool kTab>
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
  __shared__ float2 rtab[kTab ? kRopeTab : 1];
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
  if (tid < 128) zs[tid >> 6][tid & 63] = 0.f;
  bs[wave][lane] = bias ? bias[(lane < 32 ? blk_k : blk_v) * 64 + 32 * half + (lane & 31)] : 0.f;
  const int ht = g.dt >> 1, hh = g.dh >> 1, hwd = (64 - g.dt - g.dh) >> 1;
  const int off_h = g.F * ht, off_w = off_h + g.Hs * hh;
  if constexpr (kTab) {
    // cos, sin of pos * base^(-2i/width) turns: the angle in fp64, reduced
    // to [-1/2, 1/2] turn, then the hardware sine and cosine (which take
    // turns); read by the tile loop after its first barrier.
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
    pj_floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = pj_floatx4{0.f, 0.f, 0.f, 0.f};
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

    // Epilogue.  Lane (lg, lr) holds features 32 run + 8 lg + 0..7
    // (accumulators 2 run, 2 run + 1) of token 16 tt + lr.  Values are
    // rounded to bf16 as the stored tensor would be; k then gets phi (and its
    // normaliser share) and the rotation of its position, and is rounded to
    // bf16 again; tokens past the range contribute zeros.
    // (lg through an empty asm: otherwise the compiler hoists the bias and
    // the RoPE constants out of the tile loop, and they occupy registers
    // through the GEMM.)
    int lgv = lg;
    asm volatile("" : "+v"(lgv));
    float bb[2][8];
#pragma unroll
    for (int run = 0; run < 2; ++run)
#pragma unroll
      for (int i = 0; i < 8; ++i) bb[run][i] = bs[wave][32 * run + 8 * lgv + i];
    // RoPE of the lane's 4 k pairs (features 32 half + 8 lg + 0..7 of the
    // head): the axis, and either the table entry of position 0 and the
    // entries per position step, or base^(-2i/width)/(2 pi)
    float inv[4];
    int axis[4], eoff[4], estr[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int f = 32 * half + 8 * lgv + 2 * pp;
      const int ax = f < g.dt ? 0 : f < g.dt + g.dh ? 1 : 2;
      const int start = ax == 0 ? 0 : ax == 1 ? g.dt : g.dt + g.dh;
      const int width = ax == 0 ? g.dt : ax == 1 ? g.dh : 64 - g.dt - g.dh;
      axis[pp] = ax;
      if constexpr (kTab) {
        eoff[pp] = (ax == 0 ? 0 : ax == 1 ? off_h : off_w) + ((f - start) >> 1);
        estr[pp] = width >> 1;
      } else {
        inv[pp] = exp2f(-(float)(f - start) / (float)width * g.log2_base) * 0.15915494309189535f;
      }
    }
    float zt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) zt[i] = 0.f;
    // k rows to the head's k tile, v rows to its v tile
    char* const ktile = reinterpret_cast<char*>(kvt + (wave & 2) * 512);
    char* const vtile = reinterpret_cast<char*>(kvt + ((wave & 2) + 1) * 512);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = 16 * tt + lr;
      const int n = n0 + tok;
      const bool valid = n < n_end;
      float val[2][8];  // [0]: k, [1]: v
#pragma unroll
      for (int run = 0; run < 2; ++run)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          val[run][i] = (float)(__bf16)(acc[2 * run + (i >> 2)][tt][i & 3] + bb[run][i]);
      const uint32_t np = (uint32_t)(valid ? n : n_end - 1);  // positions past the range: any in it
      const uint32_t fr = fdiv(np, g.fHW), rem = np - fr * g.fHW.div;
      const uint32_t row = fdiv(rem, g.fWs);
      const int pt = kTab ? (int)fr - c * g.F : g.t0 + (int)fr;  // table: the frame within the block
      const int ph = (int)row, pw = (int)(rem - row * g.fWs.div);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        val[0][i] = fmaxf(val[0][i], 0.f);
        zt[i] += valid ? val[0][i] : 0.f;
      }
      if (g.rope) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int ax = axis[pp];
          const int ps = ax == 0 ? pt : ax == 1 ? ph : pw;
          float sn, cs;
          if constexpr (kTab) {
            const float2 e = rtab[eoff[pp] + ps * estr[pp]];
            cs = e.x, sn = e.y;
          } else {
            const float turn = __builtin_amdgcn_fractf((float)ps * inv[pp]);
            sn = __builtin_amdgcn_sinf(turn), cs = __builtin_amdgcn_cosf(turn);
          }
          const float x = val[0][2 * pp], y = val[0][2 * pp + 1];
          val[0][2 * pp] = x * cs - y * sn;
          val[0][2 * pp + 1] = x * sn + y * cs;
        }
      }
#pragma unroll
      for (int run = 0; run < 2; ++run)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int f = 32 * half + 8 * lg + i;
          const __bf16 h = (__bf16)(valid ? val[run][i] : 0.f);
          *reinterpret_cast<__bf16*>((run ? vtile : ktile) + kv_piece(f, tok >> 3) * 16 + (tok & 7) * 2) = h;
        }
    }
    // the tile's normaliser share, summed over the 16 token lanes
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t = zt[i];
      t += __shfl_xor(t, 1);
      t += __shfl_xor(t, 2);
      t += __shfl_xor(t, 4);
      t += __shfl_xor(t, 8);
      if (lr == 0) zs[wave >> 1][32 * half + 8 * lg + i] += t;
    }
    __syncthreads();
    // State rows (value features) 32 half .. + 31 of this wave's head:
    // S^T[fo][fi] += sum over the tile's tokens of v[fo] RoPE(phi k)[fi].
    const uint4* vt = kvt + ((wave & 2) + 1) * 512;
    const uint4* kt = kvt + (wave & 2) * 512;
    pj_floatx4 sa[2][4];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int fc = 0; fc < 4; ++fc) sa[ft][fc] = sacc[wave][4 * ft + fc][lane];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 a[2], bo[4];
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) a[ft] = vt[kv_piece(16 * (2 * half + ft) + lr, 4 * ks + lg)];
#pragma unroll
      for (int fc = 0; fc < 4; ++fc) bo[fc] = kt[kv_piece(16 * fc + lr, 4 * ks + lg)];
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int fc = 0; fc < 4; ++fc) sa[ft][fc] = mfma(a[ft], bo[fc], sa[ft][fc]);
    }
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int fc = 0; fc < 4; ++fc) sacc[wave][4 * ft + fc][lane] = sa[ft][fc];
  }

  // Partial of (range, block): S^T (row fo, column fi), then z.
  __syncthreads();
  const long long bh = (long long)b * g.H + head;
  const long long gv = bh * g.ranges + r;
  const long long bhc = bh * g.nb + c;
  float* dst = partials + (gv + bhc) * (64 * 64 + 64);
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int fc = 0; fc < 4; ++fc) {
      const pj_floatx4 v4 = sacc[wave][4 * ft + fc][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * (2 * half + ft) + 4 * lg + i) * 64 + 16 * fc + lr] = v4[i];
    }
  if (half == 0) dst[64 * 64 + lane] = zs[wave >> 1][lane];
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
  const uint8_t* wp = (const uint8_t*)wpack;
  void* args[] = {(void*)&x, (void*)&wp, (void*)&bias, (void*)&q, (void*)&k, (void*)&v, &g};
  if (hipLaunchKernel((const void*)&sva_qkv_proj_kernel, dim3((unsigned)grid), dim3(kPjThreads), args, 0,
                      (hipStream_t)stream) != hipSuccess)
    return SVA_ERR_HIP;
  return SVA_OK;
}

hipError_t sva_internal_kv_proj_reduce(const SvaKvReduceArgs& a, const void* x, const void* wpack,
                                       const float* bias, float* partials, hipStream_t stream) {
  // The kernel's pipeline carries the next tile's first stages through the
  // epilogue in fixed registers, which takes an even stage count.
  if (a.C % (2 * kTileK) != 0 || a.C < 2 * kTileK || a.H % 2 != 0 || a.L <= 0 || a.N % a.L != 0)
    return hipErrorInvalidValue;
  KvGeo g;
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
  g.log2_base = log2f(a.rope_base);
  g.log2_base_d = log2((double)a.rope_base);
  g.F = a.Nb / (a.Hs * a.Ws);
  g.tab_entries = g.F * (a.dt / 2) + a.Hs * (a.dh / 2) + a.Ws * ((64 - a.dt - a.dh) / 2);
  const bool tab = a.rope && g.tab_entries <= kRopeTab;
  const long long grid = ((long long)g.nrg + 7) / 8 * 8 * g.npairs;
  const uint8_t* wp = (const uint8_t*)wpack;
  void* args[] = {(void*)&x, (void*)&wp, (void*)&bias, (void*)&partials, &g};
  const void* fn = tab ? (const void*)&sva_kv_proj_reduce_kernel<true> : (const void*)&sva_kv_proj_reduce_kernel<false>;
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kKvThreads), args, 0,
                         stream);
}

extern "C" sva_status sva_qkv_proj_mxfp4(const sva_proj_desc* desc, const void* x, const void* wpack,
                                         const float* bias, void* q, void* k, void* v, void* stream) {
  if (!desc) return SVA_ERR_INVALID_ARG;
  return sva_internal_proj_features(desc, x, wpack, bias, 3 * desc->H * desc->d, q, k, v, stream);
}
