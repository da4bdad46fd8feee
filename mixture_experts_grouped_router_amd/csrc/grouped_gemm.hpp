// Persistent-free ragged grouped GEMM kernel template for gfx950, shared by
// the bf16 and MXFP8 expert-MLP GEMMs.
//
// One launch covers every expert: the tile decoder reads the per-expert row
// offsets (split_sizes) on the device, so experts with no tokens produce no
// tiles and the host never waits ("NVIDIA presents an efficient path for
// training biological MoE models", section "Grouped experts instead of a
// Python loop"; "Efficient MoE training for biological foundation models
// (NVIDIA)", section "1) Fragmented expert kernels").
//
// Tile: 256 x 256 outputs, K step = one 128-byte row per operand (64 bf16 or
// 128 E4M3 values), 256 threads = 4 waves in a 2 (M) x 2 (N) grid; each wave
// owns 128 x 128 outputs = 4 x 4 MFMA blocks of 32 x 32 with 256 float32
// accumulators per lane (kept in AGPRs).
//  * bf16: v_mfma_f32_32x32x16_bf16, four 16-wide K slices per step.
//  * MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, one E8M0 scale
//    per 32 consecutive K values of each row and column), two 64-wide K
//    slices per step.  Lane l holds row l%32; with g = l/32 its 32 bytes are
//    K [16g, 16g+16) and [32+16g, 32+16g+16) of the slice, and its scale
//    byte is the one of K block g of the slice (block 2kk+g of the step).
// Operand tiles sit in LDS as [mn][k] rows of 128 bytes with an XOR swizzle
// on the eight 16-byte chunks of a row; two stages, one barrier per step.
//  * K-contiguous operands go global -> LDS directly (global_load_lds_dwordx4:
//    each wave instruction fills one contiguous KiB of LDS, so every lane
//    picks the global chunk that belongs at its LDS slot).
//  * MN-contiguous operands (bf16 backward) also go global -> LDS directly,
//    as [k][mn] rows, and the MFMA fragments are read with the transposing
//    LDS read (ds_read_b64_tr_b16).
// Tiles are ordered so that each XCD (blocks b = x mod 8) works through one
// contiguous run of tiles, M fastest inside groups of 4 N tiles: the tiles in
// flight on one XCD share activation rows and weight panels in its L2.
#pragma once

#include <type_traits>
#include <algorithm>

#include "common.hpp"
#include "work_items.hpp"
#include "timer.hpp"

namespace moe {
namespace gg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
#define MOE_LDS __attribute__((address_space(3)))

constexpr int kRowBytes = 128;              // bytes of one K step per row
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * kRowBytes;  // 32 KiB per operand stage
// RAGGED_K launches: consecutive tiles (largest expert first) are dealt to
// the XCDs in runs of this many, so every XCD gets a share of each expert
constexpr int kDealK = 4;

enum Layout { KC = 0, MC = 1 };  // memory: [mn][k] or [k][mn]
enum Group { RAGGED_M = 0, RAGGED_K = 1 };
enum Epi {
  EPI_STORE = 0,       // bf16 C
  EPI_SWIGLU = 1,      // bf16 A = w * silu(g) * u (+ g, u save)
  EPI_SWIGLU_BWD = 2,  // dgrad of the down projection + SwiGLU backward
  EPI_SWIGLU_MX = 3    // as EPI_SWIGLU, A quantised to MXFP8 along f
};
// P_FP8: MXFP8 (E8M0 scale per 32 along K, scaled MFMA); P_FP8T: E4M3
// with one float32 scale per tensor (unit MFMA scales, the tensor scales
// applied to the accumulators before the epilogue)
enum Prec { P_BF16 = 0, P_FP8 = 1, P_FP8T = 2 };



// Instruction schedule of one MFMA region: NR LDS reads interleaved one to
// one with the first NR of the region's NM MFMAs, then the remaining MFMAs,
// so the reads for the next K slice go out early and their latency hides
// under the MFMAs (the default schedule issued them after most MFMAs).
template <int NR, int NM>
__device__ __forceinline__ void sched_reads_mfma() {
  if constexpr (NR <= NM) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
    if constexpr (NM > NR)
      __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
  } else {   // NR / NM reads before each MFMA
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, NR / NM, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  }
}

// As sched_reads_mfma, with the region's NV vector-memory instructions (the
// next K step's direct loads) issued VPM per MFMA from the first MFMA on:
// issued all at once they fill the texture unit's queue and the wave stalls
// on the load issue instead of issuing MFMAs.
template <int NV, int NR, int NM, int VPM, int MPV = 1, int I = 0>
__device__ __forceinline__ void sched_vmem_reads_mfma() {
  if constexpr (I < NM) {
    // before every MPV-th MFMA, VPM vector-memory instructions
    constexpr int rem = NV - (I / MPV) * VPM;
    constexpr int v = (I % MPV != 0 || rem <= 0) ? 0 : (rem < VPM ? rem : VPM);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x010, v, 0);
    if constexpr (I < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched_vmem_reads_mfma<NV, NR, NM, VPM, MPV, I + 1>();
  }
}

// Direct loads of the next K step issued per MFMA of the first slice(s):
// bf16 (4 slices, loads spread over two of them) one per MFMA; the 8-bit
// modes (2 slices, all 24 loads in the first) three per MFMA, which leaves
// the loads more of the step to land before the barrier (Mixtral-shaped
// MXFP8 gate/up: 1.98 -> 1.95 ms; bf16 gate/up with three: 3.32 -> 3.39).
constexpr int kLoadVpmBf16 = 1;
constexpr int kLoadVpm8 = 3;

struct Params {
  const char* a;          // operand A (rows = M)
  int64_t lda;            // bytes between rows (KC) or k rows (MC)
  const char* b;          // operand B (rows = N), expert e at b + e * b_es
  int64_t ldb, b_es;      // bytes
  int M, N, K;            // K in elements; RAGGED_K: K per expert
  int F;                  // SwiGLU epilogues: expert FFN size
  int E;
  const int32_t* offsets;     // [E+1] rows per expert
  const int32_t* tile_start;  // RAGGED_M: [E+1] tile prefix
  const int32_t* mrec;        // RAGGED_M, nullable: M-tile records (the
                              // tile_start search when null)
  const int32_t* order;       // RAGGED_K: experts by decreasing rows
  int tiles_n;                // tiles along N
  int tiles_m;                // RAGGED_K: tiles along M
  int b_rows;                 // rows of one expert's B (KC direct loads)
  // MXFP8 scales in the GEMM layout (mx_tile_off); ldsa / ldsb: K steps
  // (128 values) per row of A / B; sb_es: scale bytes per expert of B
  const uint8_t* sa;
  int64_t ldsa;
  const uint8_t* sb;
  int64_t ldsb, sb_es;
  uint16_t* c;                // bf16 output (EPI_SWIGLU_MX: optional A save)
  int64_t ldc, c_es;          // elements
  uint16_t* c2;               // SwiGLU epilogues: (g, u) save [rows, 2F]
  uint8_t* cq;                // EPI_SWIGLU_MX: A codes [rows, F]
  uint8_t* cs;                // EPI_SWIGLU_MX: A scales (GEMM layout)
  uint8_t* cs_rm;             // EPI_SWIGLU_MX: optional row-major copy
  const uint16_t* h1;         // EPI_SWIGLU_BWD: saved (g, u) [rows, 2F]
  const float* w;             // routing weight per row (nullable -> 1)
  float* dw_part;             // EPI_SWIGLU_BWD: [tiles_n][rows]
  int64_t rows;
  // P_FP8T: tensor scales of A (tsa[0]) and of expert e's B (tsb[e])
  const float* tsa;
  const float* tsb;
  // EPI_SWIGLU, nullable: amax of the bf16 A output (float32 bits,
  // atomic max)
  uint32_t* amax_out;
  // Eight-wave forward kernel, nullable: float32 partial tiles and arrival
  // counters (zero on entry) of the last, partly filled round of tiles,
  // whose K range is split over several work-groups; split_slots_x slots
  // and counters per XCD; cus_per_xcd work-groups make one round
  float* split_part;
  uint32_t* split_cnt;
  int split_slots_x;
  int cus_per_xcd;
  // Ragged-M launches, nullable: kQueueWords counters (zero on entry) of a
  // persistent launch, one work-group per CU taking items from them
  uint32_t* queue;
};

// Swizzle of the 16-byte chunk c of LDS tile row r.  It depends only on
// r mod 32, so the four 32-row blocks a wave reads sit at constant offsets
// from each other.  Eight consecutive rows (one MFMA fragment read per 8
// lanes) land on eight distinct chunk positions; so do rows 8 apart within
// 32 rows (transposed register writes, 4 per 8 lanes).
__device__ __forceinline__ int swz32(int r) {
  return (r & 7) ^ ((r >> 3) & 3);
}
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * kRowBytes + ((c ^ swz32(r)) << 4);
}

// Coordinates of tile L of a RAGGED_M launch (work_items.hpp).
__device__ __forceinline__ void ragged_m_tile(const Params& p, int L,
                                              TileCoord& tc) {
  ragged_m_tile_at(p.tile_start, p.offsets, p.E, L, tc, p.mrec, p.tiles_n);
}

template <int G>
__device__ __forceinline__ bool decode_tile(const Params& p, TileCoord& tc) {
  const int b = blockIdx.x;
  if constexpr (G == RAGGED_M) {
    // XCD x (= b mod 8) takes the x-th contiguous eighth of the tile list,
    // so an expert's tiles share one L2
    const int total = p.tile_start[p.E];
    const int per = (total + kXcds - 1) / kXcds;
    const int idx = b / kXcds;
    if (idx >= per) return false;
    const int L = (b % kXcds) * per + idx;
    if (L >= total) return false;
    ragged_m_tile(p, L, tc);
  } else {
    // a tile's cost is its expert's row count: tiles are taken largest
    // expert first and dealt round the XCDs in runs of kDealK, so every
    // XCD gets an even share of the long tiles and runs them first
    const int per_e = p.tiles_m * p.tiles_n;
    const int x = b % kXcds, idx = b / kXcds;
    const int L = ((idx / kDealK) * kXcds + x) * kDealK + idx % kDealK;
    if (L >= p.E * per_e) return false;
    const int rank = L / per_e;
    const int e = p.order[rank];
    if (e < 0) return false;   // offsets were invalid: nothing runs
    const int local = L - rank * per_e;
    const int mt_e = p.tiles_m;
    // groups of kGroupN N-tiles, M tiles fastest inside a group
    const int ng = local / (mt_e * kGroupN);
    const int in_g = local - ng * mt_e * kGroupN;
    tc.e = e;
    tc.m0 = (in_g % mt_e) * BM;
    tc.nt = ng * kGroupN + in_g / mt_e;
    tc.seg0 = p.offsets[e];
    tc.seg_len = p.offsets[e + 1] - tc.seg0;
  }
  return true;
}

// ---- K-contiguous operand: direct global -> LDS ----------------------------
// buffer_load_dwordx4 ... lds: each wave instruction fills one contiguous KiB
// of LDS.  Wave w, instruction j fills KiB 4 j + w of the tile = tile rows
// 32 j + (8 w + i/8) for lane i, chunk slot i%8, which holds the logical
// chunk (i%8) ^ swz32(row).  The buffer descriptor covers exactly the
// operand's valid bytes from the current K offset, so rows past the end of
// an expert and a padding K step (descriptor of 0 bytes) read as zeros with
// no branch.
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data format

template <int EPI, bool IS_B>
struct KcDirect {
  const char* base;  // wave-uniform: operand base of the expert
  uint32_t rec;      // valid bytes from base
  int64_t ld;        // bytes per row
  int q;             // row inside each 32-row block: 8 w + lane / 8
  int cl;            // the lane's logical chunk
  int r0;            // A: first tile row (expert-relative)
  int n0, F, N;      // B: tile's first output unit, FFN size, rows
  uint32_t off[8];   // per instruction: byte offset of the lane's chunk

  __device__ __forceinline__ int row(int j) const {
    if constexpr (!IS_B) {
      return r0 + 32 * j + q;   // past the expert's rows: out of range -> 0
    } else if constexpr (EPI == EPI_SWIGLU) {
      // 32-row blocks alternate gate / up rows for the same 32 f columns
      const int f = min(n0 + (j >> 1) * 32 + q, F - 1);
      return (j & 1) ? F + f : f;
    } else {
      return min(n0 + 32 * j + q, N - 1);
    }
  }
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      off[j] = (uint32_t)row(j) * (uint32_t)ld + (uint32_t)(cl * 16);
  }
  __device__ __forceinline__ void issue(char* lds_tile, uint32_t kbyte,
                                        bool real, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + kbyte), (short)0, (int)(real ? rec - kbyte : 0u),
        kBufFlags);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      MOE_LDS void* dst =
          (MOE_LDS void*)(lds_tile + (4 * j + wave) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off[j], 0, 0, 0);
    }
  }
};

// ---- MXFP8 scales of one K step --------------------------------------------
// Lane l needs, for each of its 4 A row blocks and 4 B row blocks, the scale
// bytes of K blocks g and 2+g of the step (g = l/32): one dword (4 blocks)
// per row, rearranged so that byte 0 feeds slice 0 and byte 1 slice 1 (the
// MFMA's opsel picks the byte).  In the GEMM scale layout the 32 rows of a
// row block read one 128-byte line per step (two when an expert's rows
// start inside a 32-row group).
struct MxScales {
  const uint8_t* a;  // wave-uniform: A scales at the first K step
  const uint8_t* b;  // wave-uniform: B scales of the expert
  uint32_t oa[4], ob[4];  // lane's row offsets (bytes, K step 0)
  uint32_t na[4], nb[4];  // next step, raw
  __device__ __forceinline__ void load(int kstep) {
    const uint8_t* ka = a + kstep * 128;
    const uint8_t* kb = b + kstep * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      na[i] = *reinterpret_cast<const uint32_t*>(ka + oa[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      nb[j] = *reinterpret_cast<const uint32_t*>(kb + ob[j]);
  }
  // bytes (g, 2+g) -> (0, 1)
  static __device__ __forceinline__ uint32_t pick(uint32_t d, uint32_t sel) {
    return __builtin_amdgcn_perm(0u, d, sel);
  }
};

// 1 / (1 + e^-x) with the hardware reciprocal (1 ulp) instead of an IEEE
// division (about ten instructions per value, most of a SwiGLU epilogue's
// VALU time); every use rounds the result to bf16 or E4M3 afterwards
__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// ---- MFMA fragments ---------------------------------------------------------
template <int P>
struct Frags;

// Byte offset of chunk c in the lane's fragment row fr (0..31) of a 32-row
// block; a block's rows start at a multiple of 32, where the swizzle
// repeats, so block offsets are plain constants.
__device__ __forceinline__ int frag_off(int fr, int c) {
  return fr * kRowBytes + ((c ^ swz32(fr)) << 4);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

template <>
struct Frags<P_BF16> {
  static constexpr int kSlices = 4;  // 16-wide K slices per step
  bf16x8_t a0, a1, a2, a3, b0, b1, b2, b3;
  static __device__ __forceinline__ bf16x8_t at(const char* s, int off) {
    return *reinterpret_cast<const bf16x8_t*>(s + off);
  }
  // lane l: row l%32 of each 32-row block, k 8 (l/32) .. +7 of the slice
  __device__ __forceinline__ void load_a(const char* sa, int kk, int wm,
                                         int lane) {
    const char* pa = sa + wm * (128 * kRowBytes) +
                     frag_off(lane & 31, kk * 2 + (lane >> 5));
    a0 = at(pa, 0 * 32 * kRowBytes);
    a1 = at(pa, 1 * 32 * kRowBytes);
    a2 = at(pa, 2 * 32 * kRowBytes);
    a3 = at(pa, 3 * 32 * kRowBytes);
  }
  __device__ __forceinline__ void load_b(const char* sb, int kk, int wn,
                                         int lane) {
    const char* pb = sb + wn * (128 * kRowBytes) +
                     frag_off(lane & 31, kk * 2 + (lane >> 5));
    b0 = at(pb, 0 * 32 * kRowBytes);
    b1 = at(pb, 1 * 32 * kRowBytes);
    b2 = at(pb, 2 * 32 * kRowBytes);
    b3 = at(pb, 3 * 32 * kRowBytes);
  }
  __device__ __forceinline__ void load(const char* sa, const char* sb, int kk,
                                       int wm, int wn, int lane) {
    load_a(sa, kk, wm, lane);
    load_b(sb, kk, wn, lane);
  }
  // 8 k values of the lane from a [k][mn] stage (McDirect8 layout): two
  // transposed 8-byte reads, k and k + 4 rows apart
  static __device__ __forceinline__ bf16x8_t tr8(const char* p) {
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MOE_LDS i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MOE_LDS i16x4_t*)(p + 4 * 512));
    const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

template <>
struct Frags<P_FP8> {
  static constexpr int kSlices = 2;  // 64-wide K slices per step
  i32x8_t a0, a1, a2, a3, b0, b1, b2, b3;
  static __device__ __forceinline__ i32x8_t at(const char* s0, const char* s1,
                                               int off) {
    const uint4 lo = *reinterpret_cast<const uint4*>(s0 + off);
    const uint4 hi = *reinterpret_cast<const uint4*>(s1 + off);
    i32x8_t v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
  }
  // lane l (g = l/32): chunks 4kk+g and 4kk+2+g of its row
  __device__ __forceinline__ void load(const char* sa, const char* sb, int kk,
                                       int wm, int wn, int lane) {
    const int c0 = kk * 4 + (lane >> 5);
    const int o0 = frag_off(lane & 31, c0), o1 = frag_off(lane & 31, c0 + 2);
    const char* pa0 = sa + wm * (128 * kRowBytes) + o0;
    const char* pa1 = sa + wm * (128 * kRowBytes) + o1;
    const char* pb0 = sb + wn * (128 * kRowBytes) + o0;
    const char* pb1 = sb + wn * (128 * kRowBytes) + o1;
    a0 = at(pa0, pa1, 0 * 32 * kRowBytes);
    a1 = at(pa0, pa1, 1 * 32 * kRowBytes);
    a2 = at(pa0, pa1, 2 * 32 * kRowBytes);
    a3 = at(pa0, pa1, 3 * 32 * kRowBytes);
    b0 = at(pb0, pb1, 0 * 32 * kRowBytes);
    b1 = at(pb0, pb1, 1 * 32 * kRowBytes);
    b2 = at(pb0, pb1, 2 * 32 * kRowBytes);
    b3 = at(pb0, pb1, 3 * 32 * kRowBytes);
  }
};

// The 16 MFMAs of one K slice in row-block order; HALF = 0 issues row
// blocks 0-1, HALF = 1 row blocks 2-3, HALF = 2 all four.
#define MOE_MFMA_BF(i, j, A, B) \
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[i][j], 0, 0, 0)

template <int HALF>
__device__ __forceinline__ void mfma_bf16(const Frags<P_BF16>& f,
                                          f32x16_t (&acc)[4][4]) {
  if constexpr (HALF == 0 || HALF == 2 || HALF == 3) {
    MOE_MFMA_BF(0, 0, f.a0, f.b0); MOE_MFMA_BF(0, 1, f.a0, f.b1);
    MOE_MFMA_BF(0, 2, f.a0, f.b2); MOE_MFMA_BF(0, 3, f.a0, f.b3);
    MOE_MFMA_BF(1, 0, f.a1, f.b0); MOE_MFMA_BF(1, 1, f.a1, f.b1);
    MOE_MFMA_BF(1, 2, f.a1, f.b2); MOE_MFMA_BF(1, 3, f.a1, f.b3);
  }
  if constexpr (HALF == 1 || HALF == 2 || HALF == 3) {
    MOE_MFMA_BF(2, 0, f.a2, f.b0); MOE_MFMA_BF(2, 1, f.a2, f.b1);
    MOE_MFMA_BF(2, 2, f.a2, f.b2); MOE_MFMA_BF(2, 3, f.a2, f.b3);
  }
  if constexpr (HALF == 1 || HALF == 2 || HALF == 4) {
    MOE_MFMA_BF(3, 0, f.a3, f.b0); MOE_MFMA_BF(3, 1, f.a3, f.b1);
    MOE_MFMA_BF(3, 2, f.a3, f.b2); MOE_MFMA_BF(3, 3, f.a3, f.b3);
  }
}
#undef MOE_MFMA_BF

// MXFP8 slice KK: scales sa[i], sb[j] hold slice 0 in byte 0, slice 1 in
// byte 1 (opsel = KK); format code 0 = E4M3 for both operands.
#define MOE_MFMA_MX(i, j, A, B)                                            \
  acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(             \
      A, B, acc[i][j], 0, 0, KK, (int)sa[i], KK, (int)sb[j])

template <int KK, int HALF>
__device__ __forceinline__ void mfma_fp8(const Frags<P_FP8>& f,
                                         const uint32_t (&sa)[4],
                                         const uint32_t (&sb)[4],
                                         f32x16_t (&acc)[4][4]) {
  if constexpr (HALF == 0 || HALF == 2 || HALF == 3) {
    MOE_MFMA_MX(0, 0, f.a0, f.b0); MOE_MFMA_MX(0, 1, f.a0, f.b1);
    MOE_MFMA_MX(0, 2, f.a0, f.b2); MOE_MFMA_MX(0, 3, f.a0, f.b3);
    MOE_MFMA_MX(1, 0, f.a1, f.b0); MOE_MFMA_MX(1, 1, f.a1, f.b1);
    MOE_MFMA_MX(1, 2, f.a1, f.b2); MOE_MFMA_MX(1, 3, f.a1, f.b3);
  }
  if constexpr (HALF == 1 || HALF == 2 || HALF == 3) {
    MOE_MFMA_MX(2, 0, f.a2, f.b0); MOE_MFMA_MX(2, 1, f.a2, f.b1);
    MOE_MFMA_MX(2, 2, f.a2, f.b2); MOE_MFMA_MX(2, 3, f.a2, f.b3);
  }
  if constexpr (HALF == 1 || HALF == 2 || HALF == 4) {
    MOE_MFMA_MX(3, 0, f.a3, f.b0); MOE_MFMA_MX(3, 1, f.a3, f.b1);
    MOE_MFMA_MX(3, 2, f.a3, f.b2); MOE_MFMA_MX(3, 3, f.a3, f.b3);
  }
}
#undef MOE_MFMA_MX

template <int P>
struct Mma;

template <>
struct Mma<P_BF16> {
  template <int KK, int HALF = 2>
  static __device__ __forceinline__ void run(const Frags<P_BF16>& f,
                                             const uint32_t (&)[4],
                                             const uint32_t (&)[4],
                                             f32x16_t (&acc)[4][4]) {
    mfma_bf16<HALF>(f, acc);
  }
};

template <>
struct Mma<P_FP8> {
  template <int KK, int HALF = 2>
  static __device__ __forceinline__ void run(const Frags<P_FP8>& f,
                                             const uint32_t (&sa)[4],
                                             const uint32_t (&sb)[4],
                                             f32x16_t (&acc)[4][4]) {
    mfma_fp8<KK & 1, HALF>(f, sa, sb, acc);
  }
};

// ---- the kernel -------------------------------------------------------------
// ---- LDS-staged epilogue helpers ---------------------------------------------
// A wave stages its outputs in its own 32 KiB LDS array: 128 rows of 256
// bytes (64 float32 or 128 bf16), 16-byte chunk c of row r stored at chunk
// c ^ (r & 3).  A staging write (one row, 32 lanes, 128 contiguous bytes)
// is free of bank conflicts.  Readback gives consecutive lanes consecutive
// 16-byte chunks of a row (16 lanes per bf16 row, 8 lanes per 32 float32
// of a row), so each wave-wide global store covers whole 128-byte lines.
__device__ __forceinline__ int stg_off(int r, int c) {
  return r * 256 + ((c ^ (r & 3)) << 4);
}
// row of accumulator element (i, r) inside the wave's 128 rows
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
__device__ __forceinline__ void stage_f32(char* buf, int row, int col,
                                          float v) {
  *reinterpret_cast<float*>(buf + stg_off(row, col >> 2) + (col & 3) * 4) = v;
}
__device__ __forceinline__ void stage_bf16(char* buf, int row, int col,
                                           float v) {
  *reinterpret_cast<uint16_t*>(buf + stg_off(row, col >> 3) + (col & 7) * 2) =
      (uint16_t)f32_to_bf16(v);
}
__device__ __forceinline__ uint4 stage_chunk(const char* buf, int row, int c) {
  return *reinterpret_cast<const uint4*>(buf + stg_off(row, c));
}

// ---- epilogues -------------------------------------------------------------
// acc[i][j][r] is C[row][col] of the wave's 128 x 128 block with
//   row = wm*128 + i*32 + (r/4)*8 + (lane/32)*4 + r%4,
//   col = wn*128 + j*32 + lane%32
// Routing weights of the wave's 128 rows in the wave's own LDS array: lane l
// loads rows l and 64 + l (clamped to the expert; 1 without weights) before
// any store of the epilogue, so the wait for them waits for no store.
__device__ __forceinline__ float* row_weights(const Params& p,
                                              const TileCoord& tc, int mw,
                                              int lane, int t) {
  __shared__ float wrow_all[kThreads / 64][128];
  float* wrow = wrow_all[t >> 6];
  float w0 = 1.0f, w1 = 1.0f;
  if (p.w) {
    w0 = p.w[tc.seg0 + min(mw + lane, tc.seg_len - 1)];
    w1 = p.w[tc.seg0 + min(mw + 64 + lane, tc.seg_len - 1)];
  }
  wrow[lane] = w0;
  wrow[64 + lane] = w1;
  return wrow;
}

// SwiGLU epilogues: gate block 2 jj of each row block becomes
// silu(g) * u, with u from block 2 jj + 1
__device__ __forceinline__ void silu_mul_in_place(f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float g = acc[i][2 * jj][r];
        acc[i][2 * jj][r] = (g * fast_sigmoid(g)) * acc[i][2 * jj + 1][r];
      }
}

// Global loads and stores share one in-order counter (vmcnt): a wait for a
// load also waits for every store issued before it.  So each epilogue issues
// its loads (routing weights, saved g and u) ahead of the stores they would
// otherwise wait behind, and reads LDS in batches before storing.
template <int G, int EPI>
__device__ __forceinline__ void epilogue(const Params& p, const TileCoord& tc,
                                         f32x16_t (&acc)[4][4], int n0,
                                         int wm, int wn, int lane, int t,
                                         char* wbuf) {
  // acc[i][j][r] is C[row][col] of the wave's block with
  //   row = wm*128 + i*32 + (r/4)*8 + (lane/32)*4 + r%4,
  //   col = wn*128 + j*32 + lane%32
  const int colw = lane & 31;
  const int mw = tc.m0 + wm * 128;   // first row of the wave's block
  if constexpr (EPI == EPI_SWIGLU) {
    // B rows of block j: gate f-block (2 wn + j/2) for even j, up for odd j.
    // silu(g) * u goes through LDS (float32); the routing weight, the bf16
    // rounding and the stores happen per row on readback, where lane l owns
    // rows 8 q + l / 8 and f values 8 (l % 8) .. + 7 of the wave's 64.
    const int64_t ld1 = 2 * (int64_t)p.F;
    const bool fvalid = n0 + 64 * wn < p.F;   // F % 64 == 0: whole runs
    float* wrow = row_weights(p, tc, mw, lane, t);
    if (p.c2) {
      // (g, u) save for the backward pass, through LDS as bf16: row r holds
      // g of the wave's 64 f in columns 0..63 and u in 64..127; on readback
      // lane l takes chunk l % 16 of row 4 q + l / 16 (chunks 0-7 g, 8-15 u)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            stage_bf16(wbuf, acc_row(i, r, lane), jj * 32 + colw,
                       acc[i][2 * jj][r]);
            stage_bf16(wbuf, acc_row(i, r, lane), 64 + jj * 32 + colw,
                       acc[i][2 * jj + 1][r]);
          }
      silu_mul_in_place(acc);   // frees the u registers for the readback
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging written
      const int ch = lane & 15;
      const int coff = (ch >> 3) * p.F + n0 + 64 * wn + 8 * (ch & 7);
#pragma unroll
      for (int qb = 0; qb < 32; qb += 4) {
        uint4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = stage_chunk(wbuf, 4 * (qb + q) + (lane >> 4), ch);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mrow = mw + 4 * (qb + q) + (lane >> 4);
          if (fvalid && mrow < tc.seg_len)
            *reinterpret_cast<uint4*>(p.c2 + (tc.seg0 + mrow) * ld1 + coff) =
                v[q];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);   // readback done before reuse
    } else {
      silu_mul_in_place(acc);
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stage_f32(wbuf, acc_row(i, r, lane), jj * 32 + colw,
                    acc[i][2 * jj][r]);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging written
    const int c8 = lane & 7;
    const int f = n0 + 64 * wn + 8 * c8;
#pragma unroll
    for (int qb = 0; qb < 16; qb += 4) {
      uint4 c0[4], c1[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = 8 * (qb + q) + (lane >> 3);
        c0[q] = stage_chunk(wbuf, lr, 2 * c8);
        c1[q] = stage_chunk(wbuf, lr, 2 * c8 + 1);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mrow = mw + 8 * (qb + q) + (lane >> 3);
        const bool ok = fvalid && mrow < tc.seg_len;
        const int64_t row = tc.seg0 + mrow;
        const float wr = wrow[8 * (qb + q) + (lane >> 3)];
        float v[8] = {__uint_as_float(c0[q].x), __uint_as_float(c0[q].y),
                      __uint_as_float(c0[q].z), __uint_as_float(c0[q].w),
                      __uint_as_float(c1[q].x), __uint_as_float(c1[q].y),
                      __uint_as_float(c1[q].z), __uint_as_float(c1[q].w)};
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] *= wr;
        if (ok)
          *reinterpret_cast<uint4*>(p.c + row * p.ldc + f) =
              make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                         pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      }
    }
  } else if constexpr (EPI == EPI_STORE) {
    // bf16 C through LDS; on readback lane l takes chunk l % 16 (8 columns)
    // of row 4 q + l / 16
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stage_bf16(wbuf, acc_row(i, r, lane), j * 32 + colw, acc[i][j][r]);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging written
    uint16_t* cbase = p.c;
    const int ch = lane & 15;
    const int col = n0 + wn * 128 + 8 * ch;   // N % 64 == 0
    const int mlim = tc.seg_len;
    const int64_t rbase = tc.seg0;
#pragma unroll
    for (int qb = 0; qb < 32; qb += 16) {
      uint4 v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        v[q] = stage_chunk(wbuf, 4 * (qb + q) + (lane >> 4), ch);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int mrow = mw + 4 * (qb + q) + (lane >> 4);
        if (col < p.N && mrow < mlim)
          *reinterpret_cast<uint4*>(cbase + (rbase + mrow) * p.ldc + col) =
              v[q];
      }
    }
  } else {  // EPI_SWIGLU_BWD: acc = dA[row][f], f = n0 + wn*128 + j*32 + col
    // Two passes of 64 f columns through the wave's LDS buffer (float32).
    // On readback lane l owns rows 8 q + l / 8 and 8 f values (l % 8) of
    // the pass: it reads (g, u) of those f with 16-byte loads, writes dg
    // and du with 16-byte stores and sums dA * silu(g) * u for dw; the
    // eight lanes of a row then add their sums in a fixed tree.  The
    // (g, u) loads of the next batch of four rows go out before the
    // stores of the current one.
    __shared__ float red[2 * BM];   // row sums of the two N-waves
    const int64_t ld1 = 2 * (int64_t)p.F;
    const int c8 = lane & 7;
    float* wrow = row_weights(p, tc, mw, lane, t);
    float rsum[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) rsum[q] = 0.0f;
    // batch b: pass b / 4, rows q = 4 (b % 4) .. + 3
    auto fcol = [&](int pass) { return n0 + wn * 128 + 64 * pass; };
    auto load_gu = [&](int b, uint4 (&g4)[4], uint4 (&u4)[4]) {
      const int f = fcol(b >> 2) + 8 * c8;
      if (fcol(b >> 2) >= p.F) return;   // F % 64 == 0
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mrow = min(mw + 8 * (4 * (b & 3) + q) + (lane >> 3),
                             tc.seg_len - 1);
        const uint16_t* h = p.h1 + (tc.seg0 + mrow) * ld1 + f;
        g4[q] = *reinterpret_cast<const uint4*>(h);
        u4[q] = *reinterpret_cast<const uint4*>(h + p.F);
      }
    };
    auto stage_pass = [&](int pass) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            stage_f32(wbuf, acc_row(i, r, lane), jj * 32 + colw,
                      acc[i][2 * pass + jj][r]);
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging written
    };
    uint4 gA[4], uA[4], gB[4], uB[4];
    load_gu(0, gA, uA);
    stage_pass(0);
    auto run_batch = [&](int b, const uint4 (&g4)[4], const uint4 (&u4)[4]) {
      const int pass = b >> 2;
      const int f = fcol(pass) + 8 * c8;
      if (fcol(pass) >= p.F) return;
      uint4 c0[4], c1[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = 8 * (4 * (b & 3) + q) + (lane >> 3);
        c0[q] = stage_chunk(wbuf, lr, 2 * c8);
        c1[q] = stage_chunk(wbuf, lr, 2 * c8 + 1);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qq = 4 * (b & 3) + q;
        const int mrow = mw + 8 * qq + (lane >> 3);
        const float da[8] = {
            __uint_as_float(c0[q].x), __uint_as_float(c0[q].y),
            __uint_as_float(c0[q].z), __uint_as_float(c0[q].w),
            __uint_as_float(c1[q].x), __uint_as_float(c1[q].y),
            __uint_as_float(c1[q].z), __uint_as_float(c1[q].w)};
        const uint32_t gw[4] = {g4[q].x, g4[q].y, g4[q].z, g4[q].w};
        const uint32_t uw[4] = {u4[q].x, u4[q].y, u4[q].z, u4[q].w};
        const float wr = wrow[8 * qq + (lane >> 3)];
        uint32_t dgw[4], duw[4];
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float dgv[2], duv[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const float g = hh ? bf16hi(gw[e]) : bf16lo(gw[e]);
            const float u = hh ? bf16hi(uw[e]) : bf16lo(uw[e]);
            const float a = da[2 * e + hh];
            const float sgm = fast_sigmoid(g);
            const float sg = g * sgm;
            dgv[hh] = a * wr * u * (sgm * (1.0f + g * (1.0f - sgm)));
            duv[hh] = a * wr * sg;
            part += a * sg * u;
          }
          dgw[e] = pack_bf16x2(dgv[0], dgv[1]);
          duw[e] = pack_bf16x2(duv[0], duv[1]);
        }
        if (mrow < tc.seg_len) {
          uint16_t* d = p.c + (tc.seg0 + mrow) * ld1 + f;
          *reinterpret_cast<uint4*>(d) =
              make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]);
          *reinterpret_cast<uint4*>(d + p.F) =
              make_uint4(duw[0], duw[1], duw[2], duw[3]);
          rsum[qq] += part;
        }
      }
    };
#pragma unroll
    for (int b = 0; b < 8; b += 2) {
      if (b == 4) {
        __builtin_amdgcn_s_waitcnt(0xc07f);   // pass 0 readback done
        stage_pass(1);
      }
      load_gu(b + 1, gB, uB);
      run_batch(b, gA, uA);
      if (b + 2 < 8) load_gu(b + 2, gA, uA);
      run_batch(b + 1, gB, uB);
    }
    if (p.dw_part) {
      // the eight lanes of a row, then the two N-waves in a fixed order
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        float v = rsum[q];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        if (c8 == 0) red[wn * BM + wm * 128 + 8 * q + (lane >> 3)] = v;
      }
      __syncthreads();
      const int mrow = tc.m0 + t;
      if (mrow < tc.seg_len) {
        const float s = red[t] + red[BM + t];
        p.dw_part[(int64_t)tc.nt * p.rows + tc.seg0 + mrow] = s;
      }
    }
  }
}

// ---- The last round of tiles, split along K ---------------------------------
// An XCD runs its contiguous run of tiles in rounds of one tile per CU.  A
// run of R rounds plus `rem` more tiles takes R + 1 tile times even when rem
// is small (a tile with a few valid rows costs as much as a full one: the
// weight panel and the MFMAs are the same).  When rem is at most half a
// round, each of those rem tiles is split into S <= kMaxSplit ranges of K
// steps (rem * S <= CUs of the XCD), run by S work-groups that each write
// their float32 partial tile to a slot of the workspace; the last to arrive
// (an arrival counter per tile) adds the S partials in slot order and runs
// the tile's epilogue.  The sums are fixed by the tile list alone, so the
// result is deterministic.  Items and pieces: work_items.hpp.

__device__ __forceinline__ SplitCfg split_cfg(const Params& p) {
  return SplitCfg{p.split_part != nullptr, p.cus_per_xcd, p.split_slots_x};
}

// Item idx of XCD x: a whole tile, or a range of K steps of one of the
// last round's tiles.
__device__ __forceinline__ bool decode_item(const Params& p, int nk, int x,
                                            int idx, TileCoord& tc,
                                            SplitRange& sr) {
  return decode_item_at(p.tile_start, p.offsets, p.E, split_cfg(p), nk, x,
                        idx, tc, sr, p.mrec, p.tiles_n);
}

// ---- persistent ragged-M launches -------------------------------------------
// One work-group per CU.  Per item a work-group on XCD x first takes the
// next index of its own XCD's counter (so an expert's tiles keep sharing
// that XCD's L2, as with one work-group per item), and once that share is
// used up the next index of the other XCDs' counters in turn: an XCD that
// runs slow (one of them takes ~5% longer per tile on the same work) no
// longer holds the whole launch back, and no work-group waits for a new
// launch between tiles (3-4 us per tile measured between one work-group's
// end and the next one's start on a CU).
constexpr int kQueueWords = 16;   // counters 0..7 used

// This CU's XCD (hardware register XCC_ID).
__device__ __forceinline__ int hw_xcd() {
  return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcds - 1));
}

// Thread 0: the next item (x, idx), or x = -1 when none is left.
__device__ __forceinline__ void take_item(const Params& p, int nk, int xh,
                                          int& x, int& idx) {
  uint32_t* q = p.queue;
  take_item_with(
      p.tile_start[p.E], split_cfg(p), nk, xh,
      [q](int y) {
        return __hip_atomic_load(q + y, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      },
      [q](int y) {
        return __hip_atomic_fetch_add(q + y, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      },
      x, idx);
}

// Partial tile of a split work-group: float4 q of accumulator block (i, j)
// of thread t at float4 index ((i NJ + j) 4 + q) NT + t of its slot, so
// every wave-wide store and load covers one contiguous KiB.  Returns true
// for the last arrival, whose accumulators then hold the sum of the S
// partials, added in slot order.  arrived: one word of LDS.
template <int NT, int MI, int NJ>
__device__ __forceinline__ bool split_reduce(const Params& p,
                                             const SplitRange& sr,
                                             f32x16_t (&acc)[MI][NJ], int t,
                                             uint32_t* arrived) {
  constexpr int kSlot4 = BM * BN / 4;   // float4 per slot
  float4* own = reinterpret_cast<float4*>(p.split_part) +
                (int64_t)(sr.slot0 + sr.s) * kSlot4;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        own[((i * NJ + j) * 4 + q) * NT + t] =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                        acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
  // Every wave's partial stores have reached the L2 (vmcnt(0)) before the
  // barrier; then one release at agent scope (an L2 write-back ahead of the
  // counter increment) publishes them all, instead of one per wave.
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  __syncthreads();
  if (t == 0)
    *arrived = __hip_atomic_fetch_add(p.split_cnt + sr.id, 1u,
                                     __ATOMIC_RELEASE,
                                     __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*arrived != (uint32_t)(sr.S - 1)) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16_t{};
  const float4* part =
      reinterpret_cast<const float4*>(p.split_part) + (int64_t)sr.slot0 * kSlot4;
  for (int s = 0; s < sr.S; ++s) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v =
              part[(int64_t)s * kSlot4 + ((i * NJ + j) * 4 + q) * NT + t];
          acc[i][j][4 * q] += v.x;
          acc[i][j][4 * q + 1] += v.y;
          acc[i][j][4 * q + 2] += v.z;
          acc[i][j][4 * q + 3] += v.w;
        }
  }
  // the counter is zero again for the next launch
  if (t == 0)
    __hip_atomic_store(p.split_cnt + sr.id, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

template <int EPI>
struct Shape8 {
  static constexpr int MI =                             // 32-row A blocks
      EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX ? 2 : 4;
  static constexpr int NJ = 8 / MI;                     // 32-row B blocks
  static constexpr int WN = 8 / (8 / MI);               // waves along N
};

// The four-wave kernel serves the GEMMs the eight-wave kernels do not take,
// all ragged M with K-contiguous operands: the per-expert loop's plain
// store, the bf16 gate/up GEMM with H above kW8MaxGateUpK, and the MXFP8
// dgrad of the down projection with the SwiGLU-backward epilogue.
template <int P, int LA, int LB, int G, int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(Params p) {
  static_assert(G == RAGGED_M && LA == KC && LB == KC,
                "ragged M, K-contiguous operands");
  static_assert(P == P_BF16 || P == P_FP8, "bf16 or MXFP8");
  static_assert(EPI != EPI_SWIGLU_MX, "the MXFP8 gate/up is eight-wave");
  constexpr int PF = P;
  using Fr = Frags<PF>;
  constexpr int kSl = Fr::kSlices;
  constexpr int kElemBytes = P == P_BF16 ? 2 : 1;
  constexpr int kStepK = kRowBytes / kElemBytes;  // K elements per step

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
  const int kdim = p.K;
  const int n0 = EPI == EPI_SWIGLU ? tc.nt * (BN / 2)   // f units
                                   : tc.nt * BN;

  // ---- operand sources ----
  KcDirect<EPI, false> da;
  KcDirect<EPI, true> db;
  MxScales ms;
  const int q = 8 * wave + (lane >> 3);   // direct-load row inside 32 rows
  const int cl = (lane & 7) ^ swz32(q);   // its logical chunk
  // rows seg0 + m0 + r; rows past the expert's last read as zeros
  da.base = p.a + (int64_t)tc.seg0 * p.lda;
  da.rec = (uint32_t)tc.seg_len * (uint32_t)p.lda;
  da.ld = p.lda;
  da.q = q;
  da.cl = cl;
  da.r0 = tc.m0;
  da.init();
  const char* bexp = p.b + (int64_t)tc.e * p.b_es;
  db.base = bexp;
  db.rec = (uint32_t)p.b_rows * (uint32_t)p.ldb;
  db.ld = p.ldb;
  db.q = q;
  db.cl = cl;
  db.n0 = n0;
  db.F = p.F;
  db.N = p.N;
  db.init();
  // E8M0 scale bytes of the current K step
  uint32_t sa_cur[4] = {0, 0, 0, 0}, sb_cur[4] = {0, 0, 0, 0};
  // byte selector for v_perm: lane group g takes scale bytes (g, 2 + g)
  const uint32_t sel = (lane >> 5) ? 0x0c0c0301u : 0x0c0c0200u;
  if constexpr (P == P_FP8) {
    // scales of K step s at byte 128 s of a row block's run
    ms.a = p.sa;
    ms.b = p.sb + (int64_t)tc.e * p.sb_es;
    KcDirect<EPI, true> m;   // B row mapping of the lane's 32-row blocks
    m.q = lane & 31;
    m.n0 = n0;
    m.F = p.F;
    m.N = p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = min(tc.m0 + wm * 128 + 32 * i + (lane & 31),
                         tc.seg_len - 1);
      const uint32_t rabs = (uint32_t)(tc.seg0 + ra);
      ms.oa[i] = mx_tile_off(rabs, 0, (uint32_t)p.ldsa);
      // B tile row wn*128 + 32 i + lane%32 is direct-load block 4 wn + i
      ms.ob[i] = mx_tile_off((uint32_t)m.row(4 * wn + i), 0,
                             (uint32_t)p.ldsb);
    }
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  const int nk = (kdim + kStepK - 1) / kStepK;
  // LDS reads per K slice: 4 per K-contiguous side (16-byte reads), 8 for
  // an N-contiguous B (two 8-byte transposed reads per block); MXFP8 16
  constexpr int kNR = P != P_BF16 ? 16 : 8;
  // part 1: A (and the MXFP8 scales), part 2: B, 3: both
  auto issue_part = [&](char* bufa, char* bufb, int kt, bool real, int part) {
    // a padding step (real == false) reads zeros: empty descriptors for
    // direct loads, k rows past kvalid for staged loads; its scales are
    // those of the last real step (finite; they multiply zeros)
    if (part & 1) {
      da.issue(bufa, (uint32_t)kt * kRowBytes, real, wave);
      if constexpr (P == P_FP8) ms.load(min(kt, nk - 1));
    }
    if (part & 2) {
      db.issue(bufb, (uint32_t)kt * kRowBytes, real, wave);
    }
  };
  auto issue = [&](char* bufa, char* bufb, int kt, bool real) {
    issue_part(bufa, bufb, kt, real, 3);
  };
  // The next K step's loads go out over the first slice (or, split, A over
  // the first slice and B over the second), spread between the MFMAs.
  constexpr bool kSplit = kSl >= 3;
  constexpr int kVmA = 8 + (P == P_FP8 ? 8 : 0);   // A loads (+ scales)
  constexpr int kVpm = P != P_BF16 ? kLoadVpm8 : kLoadVpmBf16;
  // 8-bit modes: the stage barrier after three of the last slice's four
  // row blocks of MFMAs, the last four overlapping the next stage's first
  // fragment reads (MXFP8 gate/up 1.888-1.903 -> 1.857-1.868 ms, down
  // 0.962-0.966 -> 0.947); bf16: after the last MFMA (three quarters:
  // gate/up 3.229 -> 3.236 ms)
  constexpr bool kBarQ = P != P_BF16;
  constexpr int kVmB = 8;
  auto slice_sched = [&](int kk) {
    if (kk == 0) {
      if constexpr (kSplit) sched_vmem_reads_mfma<kVmA, kNR, 16, kVpm>();
      else sched_vmem_reads_mfma<kVmA + kVmB, kNR, 16, kVpm>();
    } else if (kSplit && kk == 1) {
      sched_vmem_reads_mfma<kVmB, kNR, 16, kVpm>();
    } else {
      sched_reads_mfma<kNR, 16>();
    }
  };
  // fragments of K slice kk from stage (sa, sb)
  auto fload = [&](Fr& f, const char* sa, const char* sb, int kk) {
    f.load(sa, sb, kk, wm, wn, lane);
  };
  auto take_scales = [&]() {
    if constexpr (P == P_FP8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa_cur[i] = MxScales::pick(ms.na[i], sel);
        sb_cur[i] = MxScales::pick(ms.nb[i], sel);
      }
    }
  };

  {
    // Two K steps per loop trip, one per LDS stage, so each stage is a
    // distinct LDS object: the compiler then knows that direct loads into one
    // stage never alias fragment reads of the other and waits for them only
    // at the barrier.  An odd last step computes on a zero stage.  The trip
    // has no branches, so the MFMAs stay where they are written.
    // Fragment reads run one K slice ahead of the MFMAs; the barrier that
    // publishes the next stage follows the step's last MFMA (8-bit modes: the
    // last slice's third row block of MFMAs), so the next stage's loads get
    // (nearly) the whole step to land.  (With the barrier halfway
    // through the last slice, the next stage's first fragment reads overlapped
    // the MFMAs after it but the loads had half a slice less: Mixtral-shaped
    // gate/up 3.298 -> 3.206 ms, MXFP8 gate/up 1.963 -> 1.911 ms, MXFP8 down
    // 1.000 -> 0.971 ms with the barrier at the end.)
    const int nk2 = (nk + 1) & ~1;
    if (nk > 0) issue(sA0, sB0, 0, true);
    __syncthreads();
    take_scales();
    Fr cur, nxt;
    fload(cur, sA0, sB0, 0);

    for (int kt = 0; kt < nk2; kt += 2) {
      // stage kt from buffers 0 while stage kt+1 loads into buffers 1
      issue_part(sA1, sB1, kt + 1, kt + 1 < nk, kSplit ? 1 : 3);
  #pragma unroll
      for (int kk = 0; kk < kSl - 1; ++kk) {
        if (kSplit && kk == 1) issue_part(sA1, sB1, kt + 1, kt + 1 < nk, 2);
        fload(nxt, sA0, sB0, kk + 1);
        if (kk == 0) Mma<PF>::template run<0>(cur, sa_cur, sb_cur, acc);
        else Mma<PF>::template run<1>(cur, sa_cur, sb_cur, acc);
        cur = nxt;
        slice_sched(kk);
        // keep the scheduler from hoisting later slices' reads (registers)
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kBarQ) {
        Mma<PF>::template run<kSl - 1, 3>(cur, sa_cur, sb_cur, acc);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        fload(nxt, sA1, sB1, 0);
        Mma<PF>::template run<kSl - 1, 4>(cur, sa_cur, sb_cur, acc);
        cur = nxt;
        take_scales();
        sched_reads_mfma<kNR, 4>();
        __builtin_amdgcn_sched_barrier(0);
      } else {
        Mma<PF>::template run<kSl - 1>(cur, sa_cur, sb_cur, acc);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        fload(nxt, sA1, sB1, 0);
        cur = nxt;
        take_scales();
        __builtin_amdgcn_sched_barrier(0);
      }

      // stage kt+1 from buffers 1 while stage kt+2 loads into buffers 0 (a
      // step past nk2 is never computed; its zero loads are harmless)
      issue_part(sA0, sB0, kt + 2, kt + 2 < nk, kSplit ? 1 : 3);
  #pragma unroll
      for (int kk = 0; kk < kSl - 1; ++kk) {
        if (kSplit && kk == 1) issue_part(sA0, sB0, kt + 2, kt + 2 < nk, 2);
        fload(nxt, sA1, sB1, kk + 1);
        if (kk == 0) Mma<PF>::template run<0>(cur, sa_cur, sb_cur, acc);
        else Mma<PF>::template run<1>(cur, sa_cur, sb_cur, acc);
        cur = nxt;
        slice_sched(kk);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kBarQ) {
        Mma<PF>::template run<kSl - 1, 3>(cur, sa_cur, sb_cur, acc);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        fload(nxt, sA0, sB0, 0);
        Mma<PF>::template run<kSl - 1, 4>(cur, sa_cur, sb_cur, acc);
        cur = nxt;
        take_scales();
        sched_reads_mfma<kNR, 4>();
        __builtin_amdgcn_sched_barrier(0);
      } else {
        Mma<PF>::template run<kSl - 1>(cur, sa_cur, sb_cur, acc);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        fload(nxt, sA0, sB0, 0);
        cur = nxt;
        take_scales();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // every wave is past its last LDS read of the operand stages (and every
  // direct load has landed) before the stages become epilogue staging
  __syncthreads();
  char* wbuf = wave == 0 ? sA0 : wave == 1 ? sB0 : wave == 2 ? sA1 : sB1;
  epilogue<G, EPI>(p, tc, acc, n0, wm, wn, lane, t, wbuf);
}

// Prefix over experts: tile_start[e] = sum_{e' < e} ceil(M_e'/unit) * tn
// (all zero, and MOE_DEVERR_OFFSETS recorded, for invalid offsets); with
// mrec, also the M-tile records (work_items.hpp).
__global__ __launch_bounds__(1024) void tile_table_kernel(
    const int32_t* __restrict__ offsets, int E, int64_t rows, int unit,
    int tn, int32_t* __restrict__ tile_start, uint32_t* __restrict__ zero,
    int nzero, int32_t* status, int32_t* __restrict__ mrec);

// Workspace bytes of a tile table with M-tile records (tile_table_ints)
inline size_t tile_table_bytes(int E, int64_t rows) {
  return ((size_t)tile_table_ints(E, rows) * sizeof(int32_t) + 255) &
         ~(size_t)255;
}
// The records of a tile table of that size
inline const int32_t* tile_records(const int32_t* tile_start, int E) {
  return tile_start + tile_rec_offset(E);
}

// Grid for a RAGGED_M launch: sum_e ceil(M_e / BM) <= rows / BM + E tiles
// per N tile, rounded up to whole XCD rounds.
inline int ragged_m_grid(int64_t rows, int E, int tn) {
  const int64_t mt = rows / BM + E;
  int64_t g = mt * tn;
  g = (g + kXcds - 1) / kXcds * kXcds;
  return (int)g;
}

// Grid of a RAGGED_M launch that may split its tail: ragged_m_grid plus
// one round of split work-groups per XCD.
inline int ragged_m_grid_split(int64_t rows, int E, int tn, const Params& p) {
  return ragged_m_grid(rows, E, tn) +
         (p.split_part ? kXcds * p.split_slots_x : 0);
}

// Partial-tile slots per XCD worth allocating for a launch with at most
// `tiles` tiles and nk K steps (0: no split); float32 partials of BM x BN
// per slot, plus one counter per slot.
inline int split_slots_x(int64_t tiles, int nk) {
  if (nk < 4) return 0;
  const int64_t per = (tiles + kXcds - 1) / kXcds;
  return (int)std::min<int64_t>(kMaxSplitSlotsX, per * kMaxSplit);
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace bytes of the float32 partial tiles and of the arrival counters
// for slots_x slots per XCD.
inline size_t split_part_bytes(int slots_x) {
  return align256((size_t)kXcds * slots_x * BM * BN * sizeof(float));
}
inline size_t split_cnt_bytes(int slots_x) {
  return align256((size_t)kXcds * slots_x * sizeof(uint32_t));
}
// Workspace bytes of nq persistent launches' counters followed by the split
// arrival counters (one zeroed range).
inline size_t counters_bytes(int nq, int slots_x) {
  return align256(((size_t)nq * kQueueWords + (size_t)kXcds * slots_x) *
                  sizeof(uint32_t));
}
// Grid of a persistent launch: one work-group per CU (whole XCD rounds),
// never more than the one-item-per-work-group grid.
inline int persistent_grid(int cu_count, int grid) {
  const int g = std::max(kXcds, cu_count / kXcds * kXcds);
  return std::min(g, grid);
}
// Lets launch p split its tail (slots_x > 0); the counters must be zero.
inline void enable_split(Params& p, float* part, uint32_t* cnt, int slots_x,
                         int cu_count) {
  if (slots_x <= 0) return;
  p.split_part = part;
  p.split_cnt = cnt;
  p.split_slots_x = slots_x;
  p.cus_per_xcd = cu_count / kXcds;
}

inline int ragged_k_grid(int E, int tiles_m, int tiles_n) {
  constexpr int r = kXcds * kDealK;
  return (E * tiles_m * tiles_n + r - 1) / r * r;
}

template <int P, int LA, int LB, int G, int EPI>
hipError_t launch(const char* name, const Params& p, int grid,
                  hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  KernelScope ks(name, stream);
  hipLaunchKernelGGL((grouped_gemm_kernel<P, LA, LB, G, EPI>), dim3(grid),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// Each of these checks offsets (non-decreasing from 0 to rows) and, if
// they are not, records MOE_DEVERR_OFFSETS in *status and publishes an
// empty table, so that no GEMM tile and no segment is processed.
// (also clears zero[0 .. nzero), e.g. the split tiles' arrival counters).
// tile_start holds tile_table_bytes(E, rows): the prefix and the M-tile
// records.
hipError_t launch_tile_table(const int32_t* offsets, int E, int64_t rows,
                             int tn, int32_t* tile_start, int32_t* status,
                             hipStream_t stream, uint32_t* zero = nullptr,
                             int nzero = 0);
// order[i] = the expert with the i-th most rows (equal counts: lower index
// first); E <= 1024
hipError_t launch_expert_order(const int32_t* offsets, int E, int64_t rows,
                               int32_t* order, int32_t* status,
                               hipStream_t stream);
// poff[e] = sum_{e' < e} ceil(M_e' / pad) * pad, poff[E] the total
hipError_t launch_padded_offsets(const int32_t* offsets, int E, int64_t rows,
                                 int pad, int32_t* poff, int32_t* status,
                                 hipStream_t stream);


}  // namespace gg
}  // namespace moe
