// Grouped bf16 GEMMs of the expert MLP (forward and backward) on gfx950.
//
// One grouped GEMM call covers every expert: the tile scheduler reads the
// per-expert row offsets (split_sizes) on the device, so experts with no
// tokens produce no tiles and the host never waits ("NVIDIA presents an
// efficient path for training biological MoE models", section "Grouped
// experts instead of a Python loop"; "Efficient MoE training for biological
// foundation models (NVIDIA)", section "1) Fragmented expert kernels").
// The gate/up GEMM carries ScaledSwiGLU times the routing weight in its
// epilogue, so the gate/up product never goes through HBM ("NVIDIA presents
// ...", section "Reducing memory and quantisation cost"; "Efficient MoE
// training ...", section "3) Quantisation overhead in low-precision
// training").
//
// Kernel shape: 256 x 256 output tile, K step 64, 256 threads = 4 waves in a
// 2 (M) x 2 (N) grid; each wave owns 128 x 128 = 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (256 float32 accumulators per lane, which the
// compiler keeps in AGPRs).  Operand tiles sit in LDS as [mn][k] rows of
// 128 bytes with an XOR swizzle on the eight 16-byte chunks of a row; two
// stages, one barrier per K step.
//  * K-contiguous operands go global -> LDS directly (global_load_lds_dwordx4:
//    each wave instruction fills one contiguous KiB of LDS, so every lane
//    picks the global chunk that belongs at its LDS slot).
//  * MN-contiguous operands (backward) go through registers and are
//    transposed 8 x 8 on the way into LDS.
// Tiles are ordered so that each XCD (blocks b = x mod 8) works through one
// contiguous run of tiles, M fastest inside groups of 4 N tiles: the tiles in
// flight on one XCD share activation rows and weight panels in its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
#define MOE_LDS __attribute__((address_space(3)))

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * BK * 2;     // 32 KiB per operand tile
constexpr int kGroupN = 4;                  // N tiles per scheduling group
constexpr int kXcds = 8;

enum Layout { KC = 0, MC = 1 };  // memory: [mn][k] or [k][mn]
enum Group { RAGGED_M = 0, RAGGED_K = 1 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2 };

struct Params {
  const uint16_t* a;      // operand A (rows = M)
  int64_t lda;
  const uint16_t* b;      // operand B (rows = N), expert e at b + e * b_es
  int64_t ldb, b_es;
  int M, N, K;            // RAGGED_M: M per expert from offsets; RAGGED_K: K
  int F;                  // EPI_SWIGLU / EPI_SWIGLU_BWD: expert FFN size
  int E;
  const int32_t* offsets;     // [E+1] rows per expert
  const int32_t* tile_start;  // RAGGED_M: [E+1] tile prefix
  int tiles_n;                // tiles along N
  int tiles_m;                // RAGGED_K: tiles along M
  uint16_t* c;                // main output
  int64_t ldc, c_es;
  uint16_t* c2;               // EPI_SWIGLU: h1 save [rows, 2F] (nullable)
  const uint16_t* h1;         // EPI_SWIGLU_BWD: saved (g, u) [rows, 2F]
  const float* w;             // routing weight per row (nullable -> 1)
  float* dw_part;             // EPI_SWIGLU_BWD: [tiles_n][rows]
  int64_t rows;
};

// Swizzle of the 16-byte chunk c of LDS tile row r.  Eight consecutive rows
// (one MFMA fragment read per 8 lanes) and eight rows 8 apart (one transposed
// register write per 8 lanes) both land on eight distinct chunk positions.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * (BK * 2) + ((c ^ swz(r)) << 4);
}

struct TileCoord {
  int e;        // expert
  int m0;       // first row of the tile inside the expert's M range
  int seg0;     // offsets[e]
  int seg_len;  // rows of expert e
  int nt;       // N tile index
};

template <int G>
__device__ __forceinline__ bool decode_tile(const Params& p, TileCoord& tc) {
  const int b = blockIdx.x;
  int total;
  if constexpr (G == RAGGED_M) total = p.tile_start[p.E];
  else total = p.E * p.tiles_m * p.tiles_n;
  const int per = (total + kXcds - 1) / kXcds;
  const int idx = b / kXcds;
  if (idx >= per) return false;
  const int L = (b % kXcds) * per + idx;
  if (L >= total) return false;
  int e, local, mt_e;
  if constexpr (G == RAGGED_M) {
    // tile_start[e] <= L < tile_start[e+1]; experts without tiles have
    // tile_start[e] == tile_start[e+1] and are never selected
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_start[mid] <= L) lo = mid; else hi = mid;
    }
    e = lo;
    local = L - p.tile_start[e];
    const int len = p.offsets[e + 1] - p.offsets[e];
    mt_e = (len + BM - 1) / BM;
  } else {
    const int per_e = p.tiles_m * p.tiles_n;
    e = L / per_e;
    local = L - e * per_e;
    mt_e = p.tiles_m;
  }
  // groups of kGroupN N-tiles, M tiles fastest inside a group
  const int ng = local / (mt_e * kGroupN);
  const int in_g = local - ng * mt_e * kGroupN;
  tc.e = e;
  tc.m0 = (in_g % mt_e) * BM;
  tc.nt = ng * kGroupN + in_g / mt_e;
  tc.seg0 = p.offsets[e];
  tc.seg_len = p.offsets[e + 1] - tc.seg0;
  return true;
}

// ---- K-contiguous operand: direct global -> LDS ----------------------------
// Wave w, instruction j fills KiB q = 4 j + w of the tile = tile rows
// 8q .. 8q+7; lane i lands at row 8q + i/8, chunk slot i%8, which holds the
// logical chunk (i%8) ^ swz(row).
struct KcDirect {
  const uint16_t* g[8];  // per instruction: global address at k = 0
  __device__ __forceinline__ void issue(char* lds_tile, int k0,
                                        int wave) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      MOE_LDS void* dst =
          (MOE_LDS void*)(lds_tile + (4 * j + wave) * 1024);
      __builtin_amdgcn_global_load_lds((const void*)(g[j] + k0), dst, 16, 0,
                                       0);
    }
  }
};

// ---- MN-contiguous operand through registers --------------------------------
// Thread t covers mn chunk (t & 31) (8 values) for k rows 8 (t >> 5) .. +7;
// the 8 x 8 block is transposed in registers and written as 8 row chunks.
struct McStaged {
  const uint16_t* base;   // element (mn = this thread's chunk, k = 0)
  int64_t ld;             // elements between consecutive k rows
  int kvalid;             // k rows >= kvalid read as zero
  int kr;                 // first k row of the staged block
  uint4 v0, v1, v2, v3, v4, v5, v6, v7;

  // Rows past kvalid load the last valid row; store() zeroes them, so the
  // loads stay in flight until the LDS store (callers never load with
  // kvalid == 0).
  __device__ __forceinline__ uint4 row(int k) const {
    const int kc = min(k, kvalid - 1);
    return *reinterpret_cast<const uint4*>(base + (int64_t)kc * ld);
  }
  __device__ __forceinline__ void load(int k0) {
    kr = k0 + 8 * (threadIdx.x >> 5);
    v0 = row(kr + 0); v1 = row(kr + 1); v2 = row(kr + 2); v3 = row(kr + 3);
    v4 = row(kr + 4); v5 = row(kr + 5); v6 = row(kr + 6); v7 = row(kr + 7);
  }
  static __device__ __forceinline__ uint4 keep(uint4 v, bool ok) {
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u,
                      ok ? v.w : 0u);
  }
  // lo: halves 0 of the two inputs (k even, k odd); hi: halves 1
  static __device__ __forceinline__ uint32_t plo(uint32_t ke, uint32_t ko) {
    return __builtin_amdgcn_perm(ko, ke, 0x05040100u);
  }
  static __device__ __forceinline__ uint32_t phi(uint32_t ke, uint32_t ko) {
    return __builtin_amdgcn_perm(ko, ke, 0x07060302u);
  }
  static __device__ __forceinline__ void put(char* lds, int r, int c,
                                             uint4 val) {
    *reinterpret_cast<uint4*>(lds + lds_off(r, c)) = val;
  }
  __device__ __forceinline__ void store(char* lds) const {
    const int kg = threadIdx.x >> 5;          // k chunk 0..7
    const int r0 = (threadIdx.x & 31) * 8;    // first mn row
    const uint4 w0 = keep(v0, kr + 0 < kvalid), w1 = keep(v1, kr + 1 < kvalid);
    const uint4 w2 = keep(v2, kr + 2 < kvalid), w3 = keep(v3, kr + 3 < kvalid);
    const uint4 w4 = keep(v4, kr + 4 < kvalid), w5 = keep(v5, kr + 5 < kvalid);
    const uint4 w6 = keep(v6, kr + 6 < kvalid), w7 = keep(v7, kr + 7 < kvalid);
    // column pair d of the inputs holds mn 2d (low half) and 2d+1 (high)
    put(lds, r0 + 0, kg, make_uint4(plo(w0.x, w1.x), plo(w2.x, w3.x),
                                    plo(w4.x, w5.x), plo(w6.x, w7.x)));
    put(lds, r0 + 1, kg, make_uint4(phi(w0.x, w1.x), phi(w2.x, w3.x),
                                    phi(w4.x, w5.x), phi(w6.x, w7.x)));
    put(lds, r0 + 2, kg, make_uint4(plo(w0.y, w1.y), plo(w2.y, w3.y),
                                    plo(w4.y, w5.y), plo(w6.y, w7.y)));
    put(lds, r0 + 3, kg, make_uint4(phi(w0.y, w1.y), phi(w2.y, w3.y),
                                    phi(w4.y, w5.y), phi(w6.y, w7.y)));
    put(lds, r0 + 4, kg, make_uint4(plo(w0.z, w1.z), plo(w2.z, w3.z),
                                    plo(w4.z, w5.z), plo(w6.z, w7.z)));
    put(lds, r0 + 5, kg, make_uint4(phi(w0.z, w1.z), phi(w2.z, w3.z),
                                    phi(w4.z, w5.z), phi(w6.z, w7.z)));
    put(lds, r0 + 6, kg, make_uint4(plo(w0.w, w1.w), plo(w2.w, w3.w),
                                    plo(w4.w, w5.w), plo(w6.w, w7.w)));
    put(lds, r0 + 7, kg, make_uint4(phi(w0.w, w1.w), phi(w2.w, w3.w),
                                    phi(w4.w, w5.w), phi(w6.w, w7.w)));
  }
};

__device__ __forceinline__ float fast_sigmoid(float x) {
  return 1.0f / (1.0f + __expf(-x));
}

// Zero one operand stage (a padding K step past the end of K).
__device__ __forceinline__ void zero_tile(char* lds) {
#pragma unroll
  for (int i = 0; i < kTileBytes / (16 * kThreads); ++i)
    *reinterpret_cast<uint4*>(lds + (i * kThreads + threadIdx.x) * 16) =
        make_uint4(0, 0, 0, 0);
}

// MFMA operand fragments of one 16-wide K slice of the wave's 128 x 128
// block: lane l holds row l%32 (of each 32-row block), k 8 (l/32) .. +7.
struct Frags {
  bf16x8_t a0, a1, a2, a3, b0, b1, b2, b3;
};

__device__ __forceinline__ bf16x8_t frag_at(const char* s, int r, int ch) {
  return *reinterpret_cast<const bf16x8_t*>(s + lds_off(r, ch));
}

__device__ __forceinline__ void load_frags(const char* sa, const char* sb,
                                           int kk, int wm, int wn, int lane,
                                           Frags& f) {
  const int frow = lane & 31;
  const int ch = kk * 2 + (lane >> 5);
  f.a0 = frag_at(sa, wm * 128 + 0 * 32 + frow, ch);
  f.a1 = frag_at(sa, wm * 128 + 1 * 32 + frow, ch);
  f.a2 = frag_at(sa, wm * 128 + 2 * 32 + frow, ch);
  f.a3 = frag_at(sa, wm * 128 + 3 * 32 + frow, ch);
  f.b0 = frag_at(sb, wn * 128 + 0 * 32 + frow, ch);
  f.b1 = frag_at(sb, wn * 128 + 1 * 32 + frow, ch);
  f.b2 = frag_at(sb, wn * 128 + 2 * 32 + frow, ch);
  f.b3 = frag_at(sb, wn * 128 + 3 * 32 + frow, ch);
}

#define MOE_MFMA(i, j, A, B) \
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[i][j], 0, 0, 0)

__device__ __forceinline__ void mfma_frags(const Frags& f,
                                           f32x16_t (&acc)[4][4]) {
  MOE_MFMA(0, 0, f.a0, f.b0); MOE_MFMA(0, 1, f.a0, f.b1);
  MOE_MFMA(0, 2, f.a0, f.b2); MOE_MFMA(0, 3, f.a0, f.b3);
  MOE_MFMA(1, 0, f.a1, f.b0); MOE_MFMA(1, 1, f.a1, f.b1);
  MOE_MFMA(1, 2, f.a1, f.b2); MOE_MFMA(1, 3, f.a1, f.b3);
  MOE_MFMA(2, 0, f.a2, f.b0); MOE_MFMA(2, 1, f.a2, f.b1);
  MOE_MFMA(2, 2, f.a2, f.b2); MOE_MFMA(2, 3, f.a2, f.b3);
  MOE_MFMA(3, 0, f.a3, f.b0); MOE_MFMA(3, 1, f.a3, f.b1);
  MOE_MFMA(3, 2, f.a3, f.b2); MOE_MFMA(3, 3, f.a3, f.b3);
}
#undef MOE_MFMA

template <int LA, int LB, int G, int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) char sA0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kTileBytes];
  TileCoord tc;
  if (!decode_tile<G>(p, tc)) return;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1;   // 0..1
  const int wn = wave & 1;    // 0..1

  // ---- tile geometry ----
  int kdim, n0;
  if constexpr (G == RAGGED_M) kdim = p.K;
  else kdim = tc.seg_len;
  if constexpr (EPI == EPI_SWIGLU) n0 = tc.nt * (BN / 2);   // f units
  else n0 = tc.nt * BN;

  // ---- operand sources ----
  KcDirect da, db;
  McStaged ma, mb;
  if constexpr (LA == KC) {
    // RAGGED_M rows seg0 + m0 + r, clamped to the expert's last row
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = 8 * (4 * j + wave) + (lane >> 3);
      const int c = (lane & 7) ^ swz(rr);
      const int r = min(tc.m0 + rr, tc.seg_len - 1);
      da.g[j] = p.a + (int64_t)(tc.seg0 + r) * p.lda + c * 8;
    }
  } else {
    // A element (m, k) at a[(seg0 + k) * lda + m] (RAGGED_K: k = token)
    const int mc = min(tc.m0 + (t & 31) * 8, p.M - 8);
    ma.base = p.a + (int64_t)tc.seg0 * p.lda + mc;
    ma.ld = p.lda;
    ma.kvalid = kdim;
  }
  const uint16_t* bexp = p.b + (int64_t)tc.e * p.b_es;
  if constexpr (LB == KC) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = 8 * (4 * j + wave) + (lane >> 3);
      const int c = (lane & 7) ^ swz(rr);
      int brow;
      if constexpr (EPI == EPI_SWIGLU) {
        // 32-row blocks alternate gate / up for the same 32 f columns
        const int blk = rr >> 5;
        const int f = min(n0 + (blk >> 1) * 32 + (rr & 31), p.F - 1);
        brow = (blk & 1) ? p.F + f : f;
      } else {
        brow = min(n0 + rr, p.N - 1);
      }
      db.g[j] = bexp + (int64_t)brow * p.ldb + c * 8;
    }
  } else {
    const int nc = min(n0 + (t & 31) * 8, p.N - 8);
    if constexpr (G == RAGGED_M) mb.base = bexp + nc;  // b_e[k * ldb + n]
    else mb.base = p.b + (int64_t)tc.seg0 * p.ldb + nc;
    mb.ld = p.ldb;
    mb.kvalid = kdim;
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  const int nk = (kdim + BK - 1) / BK;
  // Two K steps per loop trip, one per LDS stage, so each stage is a
  // distinct LDS object: the compiler then knows that direct loads into one
  // stage never alias fragment reads of the other and waits for them only
  // at the barrier.  An odd last step computes on a zero-filled stage.
  // Fragment reads run one 16-wide K slice ahead of the MFMAs; the barrier
  // that publishes the next stage sits before the last slice's MFMAs so the
  // first reads of the next stage overlap them.
  const int nk2 = (nk + 1) & ~1;
  if (nk > 0) {
    if constexpr (LA == KC) da.issue(sA0, 0, wave); else ma.load(0);
    if constexpr (LB == KC) db.issue(sB0, 0, wave); else mb.load(0);
    if constexpr (LA == MC) ma.store(sA0);
    if constexpr (LB == MC) mb.store(sB0);
  }
  __syncthreads();
  Frags cur, nxt;
  load_frags(sA0, sB0, 0, wm, wn, lane, cur);

  for (int kt = 0; kt < nk2; kt += 2) {
    // stage kt from buffers 0 while stage kt+1 loads into buffers 1
    const bool real1 = kt + 1 < nk;
    if (real1) {
      if constexpr (LA == KC) da.issue(sA1, (kt + 1) * BK, wave);
      else ma.load((kt + 1) * BK);
      if constexpr (LB == KC) db.issue(sB1, (kt + 1) * BK, wave);
      else mb.load((kt + 1) * BK);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16 - 1; ++kk) {
      load_frags(sA0, sB0, kk + 1, wm, wn, lane, nxt);
      mfma_frags(cur, acc);
      cur = nxt;
    }
    if (real1) {
      if constexpr (LA == MC) ma.store(sA1);
      if constexpr (LB == MC) mb.store(sB1);
    } else {
      zero_tile(sA1);
      zero_tile(sB1);
    }
    __syncthreads();
    load_frags(sA1, sB1, 0, wm, wn, lane, nxt);
    mfma_frags(cur, acc);
    cur = nxt;

    // stage kt+1 from buffers 1 while stage kt+2 loads into buffers 0
    const bool real2 = kt + 2 < nk;
    if (real2) {
      if constexpr (LA == KC) da.issue(sA0, (kt + 2) * BK, wave);
      else ma.load((kt + 2) * BK);
      if constexpr (LB == KC) db.issue(sB0, (kt + 2) * BK, wave);
      else mb.load((kt + 2) * BK);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16 - 1; ++kk) {
      load_frags(sA1, sB1, kk + 1, wm, wn, lane, nxt);
      mfma_frags(cur, acc);
      cur = nxt;
    }
    if (real2) {
      if constexpr (LA == MC) ma.store(sA0);
      if constexpr (LB == MC) mb.store(sB0);
    }
    __syncthreads();
    if (real2) load_frags(sA0, sB0, 0, wm, wn, lane, nxt);
    mfma_frags(cur, acc);
    cur = nxt;
  }

  // ---- epilogue ----
  // acc[i][j][r] is C[row][col] of the wave's block with
  //   row = wm*128 + i*32 + (r/4)*8 + (lane/32)*4 + r%4,
  //   col = wn*128 + j*32 + lane%32
  const int colw = lane & 31;
  const int rsub = (lane >> 5) * 4;
  if constexpr (EPI == EPI_SWIGLU) {
    // B rows of block j: gate f-block (2 wn + j/2) for even j, up for odd j
    const int64_t ld1 = 2 * (int64_t)p.F;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int f = n0 + (2 * wn + jj) * 32 + colw;
      if (f >= p.F) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mrow =
              tc.m0 + wm * 128 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          if (mrow < tc.seg_len) {
            const int64_t row = tc.seg0 + mrow;
            const float g = acc[i][2 * jj][r], u = acc[i][2 * jj + 1][r];
            const float wr = p.w ? p.w[row] : 1.0f;
            const float a = wr * (g * fast_sigmoid(g)) * u;
            p.c[row * p.ldc + f] = (uint16_t)f32_to_bf16(a);
            if (p.c2) {
              p.c2[row * ld1 + f] = (uint16_t)f32_to_bf16(g);
              p.c2[row * ld1 + p.F + f] = (uint16_t)f32_to_bf16(u);
            }
          }
        }
    }
  } else if constexpr (EPI == EPI_STORE) {
    uint16_t* cbase = p.c;
    if constexpr (G == RAGGED_K) cbase += (int64_t)tc.e * p.c_es;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + colw;
      if (col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mrow =
              tc.m0 + wm * 128 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          int64_t row;
          if constexpr (G == RAGGED_M) {
            if (mrow >= tc.seg_len) continue;
            row = tc.seg0 + mrow;
          } else {
            if (mrow >= p.M) continue;
            row = mrow;
          }
          cbase[row * p.ldc + col] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        }
    }
  } else {  // EPI_SWIGLU_BWD: acc = dA[row][f], f = n0 + wn*128 + j*32 + col
    float* red = reinterpret_cast<float*>(sA0);  // [2 N-waves][256 rows]
    const int64_t ld1 = 2 * (int64_t)p.F;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float rs[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) rs[r] = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = n0 + wn * 128 + j * 32 + colw;
        const bool fok = f < p.F;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mrow =
              tc.m0 + wm * 128 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          if (mrow < tc.seg_len && fok) {
            const int64_t row = tc.seg0 + mrow;
            const float g = bf16_to_f32(p.h1[row * ld1 + f]);
            const float u = bf16_to_f32(p.h1[row * ld1 + p.F + f]);
            const float wr = p.w ? p.w[row] : 1.0f;
            const float s = fast_sigmoid(g);
            const float sg = g * s;
            const float da = acc[i][j][r];
            const float dg = da * wr * u * (s * (1.0f + g * (1.0f - s)));
            const float du = da * wr * sg;
            p.c[row * ld1 + f] = (uint16_t)f32_to_bf16(dg);
            p.c[row * ld1 + p.F + f] = (uint16_t)f32_to_bf16(du);
            rs[r] += da * sg * u;
          }
        }
      }
      if (p.dw_part) {
        // sum over the 32 columns held by the lanes with the same lane / 32
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = rs[r];
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off, 64);
          if (colw == 0) {
            const int tr = wm * 128 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
            red[wn * 256 + tr] = v;
          }
        }
      }
    }
    if (p.dw_part) {
      // across the 2 N-waves, fixed order
      __syncthreads();
      const int mrow = tc.m0 + t;
      if (mrow < tc.seg_len) {
        const float s = red[t] + red[256 + t];
        p.dw_part[(int64_t)tc.nt * p.rows + tc.seg0 + mrow] = s;
      }
    }
  }
}

// Tile prefix over experts: tile_start[e] = sum_{e' < e} ceil(M_e'/BM) * tn.
__global__ __launch_bounds__(1024) void tile_table_kernel(
    const int32_t* __restrict__ offsets, int E, int tn,
    int32_t* __restrict__ tile_start) {
  __shared__ int32_t wsum[16];
  const int e = threadIdx.x;
  const int lane = e & 63, wid = e >> 6;
  int32_t v = 0;
  if (e < E) v = ((offsets[e + 1] - offsets[e] + BM - 1) / BM) * tn;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  if (e == 0) {
    int32_t acc = 0;
    for (int w = 0; w < 16; ++w) {
      const int32_t s = wsum[w];
      wsum[w] = acc;
      acc += s;
    }
  }
  __syncthreads();
  const int32_t excl = incl - v + wsum[wid];
  if (e < E) tile_start[e] = excl;
  if (e == E - 1) tile_start[E] = excl + v;
}

// dw_perm[r] = sum over N tiles (ascending) of the partial row sums.
__global__ __launch_bounds__(256) void reduce_parts_kernel(
    const float* __restrict__ part, int nparts, int64_t rows,
    float* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float s = 0.0f;
  for (int i = 0; i < nparts; ++i) s += part[(int64_t)i * rows + r];
  out[r] = s;
}

int ragged_m_grid(int64_t rows, int E, int tn) {
  // sum_e ceil(M_e / BM) <= rows / BM + E
  const int64_t mt = rows / BM + E;
  int64_t g = mt * tn;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return (int)g;
}

template <int LA, int LB, int G, int EPI>
hipError_t launch(const Params& p, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<LA, LB, G, EPI>), dim3(grid),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t mlp_fwd_bf16_ws_bytes(int E, int H, int F, int64_t rows, bool need_a) {
  size_t b = 2 * align256((size_t)(E + 1) * sizeof(int32_t));
  if (need_a) b += align256((size_t)rows * F * 2);
  return b;
}

hipError_t launch_mlp_fwd_bf16(int E, int H, int F, int64_t rows,
                               const void* x_perm, const void* w_gu,
                               const void* w_dn, const float* w_perm,
                               const int32_t* offsets, void* z_perm,
                               void* h1_save, void* a_save, void* ws,
                               hipStream_t stream) {
  char* wp = static_cast<char*>(ws);
  int32_t* ts1 = reinterpret_cast<int32_t*>(wp);
  wp += align256((size_t)(E + 1) * sizeof(int32_t));
  int32_t* ts2 = reinterpret_cast<int32_t*>(wp);
  wp += align256((size_t)(E + 1) * sizeof(int32_t));
  uint16_t* a_buf = static_cast<uint16_t*>(a_save);
  if (!a_buf) a_buf = reinterpret_cast<uint16_t*>(wp);
  if (rows == 0) return hipSuccess;

  const int tn1 = (F + BN / 2 - 1) / (BN / 2);
  const int tn2 = (H + BN - 1) / BN;
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream,
                     offsets, E, tn1, ts1);
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream,
                     offsets, E, tn2, ts2);

  Params p1{};
  p1.a = static_cast<const uint16_t*>(x_perm);
  p1.lda = H;
  p1.b = static_cast<const uint16_t*>(w_gu);
  p1.ldb = H;
  p1.b_es = (int64_t)2 * F * H;
  p1.N = 2 * F;
  p1.K = H;
  p1.F = F;
  p1.E = E;
  p1.offsets = offsets;
  p1.tile_start = ts1;
  p1.tiles_n = tn1;
  p1.c = a_buf;
  p1.ldc = F;
  p1.c2 = static_cast<uint16_t*>(h1_save);
  p1.w = w_perm;
  p1.rows = rows;
  hipError_t err = launch<KC, KC, RAGGED_M, EPI_SWIGLU>(
      p1, ragged_m_grid(rows, E, tn1), stream);
  if (err != hipSuccess) return err;

  Params p2{};
  p2.a = a_buf;
  p2.lda = F;
  p2.b = static_cast<const uint16_t*>(w_dn);
  p2.ldb = F;
  p2.b_es = (int64_t)H * F;
  p2.N = H;
  p2.K = F;
  p2.E = E;
  p2.offsets = offsets;
  p2.tile_start = ts2;
  p2.tiles_n = tn2;
  p2.c = static_cast<uint16_t*>(z_perm);
  p2.ldc = H;
  p2.rows = rows;
  return launch<KC, KC, RAGGED_M, EPI_STORE>(p2, ragged_m_grid(rows, E, tn2),
                                             stream);
}

size_t mlp_bwd_bf16_ws_bytes(int E, int H, int F, int64_t rows) {
  const int tnf = (F + BN - 1) / BN;
  size_t b = 2 * align256((size_t)(E + 1) * sizeof(int32_t));
  b += align256((size_t)rows * 2 * F * 2);        // dH1
  b += align256((size_t)tnf * rows * sizeof(float));  // dw partials
  return b;
}

hipError_t launch_mlp_bwd_bf16(int E, int H, int F, int64_t rows,
                               const void* x_perm, const void* w_gu,
                               const void* w_dn, const float* w_perm,
                               const int32_t* offsets, const void* h1_save,
                               const void* a_save, const void* dz_perm,
                               void* dx_perm, void* dw_gu, void* dw_dn,
                               float* dw_perm, void* ws, hipStream_t stream) {
  const int tnf = (F + BN - 1) / BN;
  const int tnh = (H + BN - 1) / BN;
  char* wp = static_cast<char*>(ws);
  int32_t* ts_f = reinterpret_cast<int32_t*>(wp);
  wp += align256((size_t)(E + 1) * sizeof(int32_t));
  int32_t* ts_h = reinterpret_cast<int32_t*>(wp);
  wp += align256((size_t)(E + 1) * sizeof(int32_t));
  uint16_t* dh1 = reinterpret_cast<uint16_t*>(wp);
  wp += align256((size_t)rows * 2 * F * 2);
  float* part = reinterpret_cast<float*>(wp);

  hipError_t err;
  if (rows > 0) {
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream,
                       offsets, E, tnf, ts_f);
    hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream,
                       offsets, E, tnh, ts_h);
    // dgrad2 + SwiGLU backward: dA = dZ W_dn[e]  (B = W_dn[e] [H, F] is
    // N-contiguous)
    Params p{};
    p.a = static_cast<const uint16_t*>(dz_perm);
    p.lda = H;
    p.b = static_cast<const uint16_t*>(w_dn);
    p.ldb = F;
    p.b_es = (int64_t)H * F;
    p.N = F;
    p.K = H;
    p.F = F;
    p.E = E;
    p.offsets = offsets;
    p.tile_start = ts_f;
    p.tiles_n = tnf;
    p.c = dh1;
    p.h1 = static_cast<const uint16_t*>(h1_save);
    p.w = w_perm;
    p.dw_part = dw_perm ? part : nullptr;
    p.rows = rows;
    err = launch<KC, MC, RAGGED_M, EPI_SWIGLU_BWD>(p, ragged_m_grid(rows, E, tnf),
                                                   stream);
    if (err != hipSuccess) return err;
    if (dw_perm) {
      hipLaunchKernelGGL(reduce_parts_kernel, dim3((unsigned)((rows + 255) / 256)),
                         dim3(256), 0, stream, part, tnf, rows, dw_perm);
    }
    // dgrad1: dX = dH1 W_gu[e]  (B = W_gu[e] [2F, H] is N-contiguous)
    Params q{};
    q.a = dh1;
    q.lda = 2 * F;
    q.b = static_cast<const uint16_t*>(w_gu);
    q.ldb = H;
    q.b_es = (int64_t)2 * F * H;
    q.N = H;
    q.K = 2 * F;
    q.E = E;
    q.offsets = offsets;
    q.tile_start = ts_h;
    q.tiles_n = tnh;
    q.c = static_cast<uint16_t*>(dx_perm);
    q.ldc = H;
    q.rows = rows;
    err = launch<KC, MC, RAGGED_M, EPI_STORE>(q, ragged_m_grid(rows, E, tnh),
                                              stream);
    if (err != hipSuccess) return err;
  }
  // wgrad2: dW_dn[e] [H, F] = dZ_e^T A_e   (K = rows of expert e)
  {
    Params p{};
    p.a = static_cast<const uint16_t*>(dz_perm);
    p.lda = H;
    p.b = static_cast<const uint16_t*>(a_save);
    p.ldb = F;
    p.M = H;
    p.N = F;
    p.E = E;
    p.offsets = offsets;
    p.tiles_m = (H + BM - 1) / BM;
    p.tiles_n = (F + BN - 1) / BN;
    p.c = static_cast<uint16_t*>(dw_dn);
    p.ldc = F;
    p.c_es = (int64_t)H * F;
    p.rows = rows;
    const int grid = (E * p.tiles_m * p.tiles_n + kXcds - 1) / kXcds * kXcds;
    err = launch<MC, MC, RAGGED_K, EPI_STORE>(p, grid, stream);
    if (err != hipSuccess) return err;
  }
  // wgrad1: dW_gu[e] [2F, H] = dH1_e^T X_e
  {
    Params p{};
    p.a = dh1;
    p.lda = 2 * F;
    p.b = static_cast<const uint16_t*>(x_perm);
    p.ldb = H;
    p.M = 2 * F;
    p.N = H;
    p.E = E;
    p.offsets = offsets;
    p.tiles_m = (2 * F + BM - 1) / BM;
    p.tiles_n = (H + BN - 1) / BN;
    p.c = static_cast<uint16_t*>(dw_gu);
    p.ldc = H;
    p.c_es = (int64_t)2 * F * H;
    p.rows = rows;
    const int grid = (E * p.tiles_m * p.tiles_n + kXcds - 1) / kXcds * kXcds;
    err = launch<MC, MC, RAGGED_K, EPI_STORE>(p, grid, stream);
  }
  return err;
}

}  // namespace moe
