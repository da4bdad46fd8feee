// The bf16 forward grouped GEMM with eight waves per 256 x 256 tile, two per
// SIMD: while one wave of a SIMD waits (its load queue, an LDS read, the
// barrier) the other issues MFMAs.  Tile, LDS stages, direct loads, tile
// order and arithmetic are those of grouped_gemm.hpp (the results are bit
// for bit the same); the wave layout and the epilogues' staging differ.
// K-contiguous operands, ragged M, EPI_STORE and EPI_SWIGLU.
//
// Wave shapes: EPI_STORE, 128 rows x 64 columns (a 2 x 4 wave grid);
// EPI_SWIGLU, 64 rows x 128 B rows (4 x 2), i.e. gate and up of 64 f, so
// each wave stores whole 128-byte lines of A and of the (g, u) save.
#pragma once

#include <algorithm>

#include "grouped_gemm.hpp"

namespace moe {
namespace gg {

constexpr int kThreads8 = 512;
// largest K (= H) for which the gate/up GEMM runs with eight waves (with
// the five-buffer rotation; without it, four waves were 3% faster at
// H = 4096: Mixtral-shaped gate/up 3.15 ms four waves, 3.01-3.03 eight)
constexpr int kW8MaxGateUpK = 4096;

// Direct loads with eight waves: wave w, instruction j (of 4) fills KiB
// 8 j + w of the stage = tile rows 32 (2 j + w / 4) + 8 (w % 4) + lane / 8,
// the same bytes as the four-wave loader puts there.
template <int EPI, bool IS_B>
struct KcDirect8 {
  const char* base;
  uint32_t rec;
  int64_t ld;
  int q;             // row inside the 32-row block: 8 (w % 4) + lane / 8
  int cl;            // the lane's logical chunk
  int r0;
  int n0, F, N;
  uint32_t off[4];
  __device__ __forceinline__ int row(int blk) const {
    if constexpr (!IS_B) {
      return r0 + 32 * blk + q;
    } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX) {
      const int f = min(n0 + (blk >> 1) * 32 + q, F - 1);
      return (blk & 1) ? F + f : f;
    } else {
      return min(n0 + 32 * blk + q, N - 1);
    }
  }
  __device__ __forceinline__ void init(int wave) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      off[j] = (uint32_t)row(2 * j + (wave >> 2)) * (uint32_t)ld +
               (uint32_t)(cl * 16);
  }
  __device__ __forceinline__ void issue(char* lds_tile, uint32_t kbyte,
                                        bool real, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + kbyte), (short)0, (int)(real ? rec - kbyte : 0u),
        kBufFlags);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      MOE_LDS void* dst = (MOE_LDS void*)(lds_tile + (8 * j + wave) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off[j], 0, 0, 0);
    }
  }
};

// Fragments of one 16-wide K slice: MI A blocks and NJ B blocks (six reads).
template <int MI, int NJ>
struct Frags8 {
  bf16x8_t a[MI], b[NJ];
  static __device__ __forceinline__ bf16x8_t at(const char* s, int off) {
    return *reinterpret_cast<const bf16x8_t*>(s + off);
  }
  // reads at lane offsets oa, ob (slice and wave block included; from
  // offsets())
  __device__ __forceinline__ void load_at(const char* sa, const char* sb,
                                          uint32_t oa, uint32_t ob) {
#pragma unroll
    for (int i = 0; i < MI; ++i) a[i] = at(sa + oa, i * 32 * kRowBytes);
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = at(sb + ob, j * 32 * kRowBytes);
  }
  static __device__ __forceinline__ void offsets(int kk, int wm, int wn,
                                                 int lane, uint32_t& oa,
                                                 uint32_t& ob) {
    const int o = frag_off(lane & 31, kk * 2 + (lane >> 5));
    oa = (uint32_t)(wm * (MI * 32 * kRowBytes) + o);
    ob = (uint32_t)(wn * (NJ * 32 * kRowBytes) + o);
  }
};

// The slice's eight MFMAs (HALF 0 / 1: those of the first / second half of
// the A blocks; 2: all)
template <int HALF, int MI, int NJ>
__device__ __forceinline__ void mfma_bf16_w8(const Frags8<MI, NJ>& f,
                                             f32x16_t (&acc)[MI][NJ]) {
  constexpr int i0 = HALF == 1 ? MI / 2 : 0;
  constexpr int i1 = HALF == 0 ? MI / 2 : MI;
#pragma unroll
  for (int i = i0; i < i1; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j],
                                                          acc[i][j], 0, 0, 0);
}

// Staging with 128-byte rows: 16-byte chunk c of row r at chunk c ^ (r & 7).
__device__ __forceinline__ int stg8(int r, int c) {
  return r * 128 + ((c ^ (r & 7)) << 4);
}

// EPI_STORE of a wave's 128 x 64 block (acc[i][j][r]: row acc_row(i, r),
// column 32 j + lane % 32) through its 16 KiB of LDS: 128-byte rows of 64
// bf16; on readback lane l takes chunk l % 8 of row 8 q + l / 8.  RAGGED_K
// (weight gradients): rows are those of expert e's [M, N] output.
template <int G = RAGGED_M>
__device__ __forceinline__ void epilogue_w8_store(const Params& p,
                                                  const TileCoord& tc,
                                                  f32x16_t (&acc)[4][2],
                                                  int n0, int wm, int wn,
                                                  int lane, char* wbuf) {
  const int colw = lane & 31;
  const int mw = tc.m0 + wm * 128;
  // Accumulator row acc_row(i, r) = 32 i + 8 (r / 4) + lo with lo =
  // 4 (lane / 32) + r % 4, so its swizzle depends on lo alone: a staging
  // address is one of a few per-lane bases plus a constant.
  int bb[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r3 = 0; r3 < 4; ++r3) {
      const int lo = 4 * (lane >> 5) + r3;
      const int c = 4 * j + (colw >> 3);
      bb[j][r3] = lo * 128 + ((c ^ lo) << 4) + (colw & 7) * 2;
    }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *reinterpret_cast<uint16_t*>(wbuf + bb[j][r & 3] +
                                     (32 * i + 8 * (r >> 2)) * 128) =
            (uint16_t)f32_to_bf16(acc[i][j][r]);
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging written
  const int ch = lane & 7;
  const int col = n0 + wn * 64 + 8 * ch;   // N % 64 == 0
  uint16_t* cbase = p.c;
  if constexpr (G == RAGGED_K) cbase += (int64_t)tc.e * p.c_es;
  const int mlim = G == RAGGED_M ? tc.seg_len : p.M;
  const int64_t rbase = G == RAGGED_M ? tc.seg0 : 0;
#pragma unroll
  for (int qb = 0; qb < 16; qb += 8) {
    uint4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      v[q] = *reinterpret_cast<const uint4*>(
          wbuf + stg8(8 * (qb + q) + (lane >> 3), ch));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int mrow = mw + 8 * (qb + q) + (lane >> 3);
      if (col < p.N && mrow < mlim)
        *reinterpret_cast<uint4*>(cbase + (rbase + mrow) * p.ldc + col) = v[q];
    }
  }
}

// EPI_SWIGLU of a wave's 64 rows x 64 f: acc[i][2 jj] is g and
// acc[i][2 jj + 1] is u of f = n0 + 64 wn + 32 jj + lane % 32 at row
// acc_row(i, r).  Staging in 256-byte rows (stg_off): (g, u) as bf16 for the
// save, then silu(g) * u as float32; the routing weight and the bf16
// rounding of A (EPI_SWIGLU_MX: its MXFP8 quantisation, a quad of lanes per
// 32-value block) happen per row on readback, as in the four-wave epilogue.
template <int EPI = EPI_SWIGLU>
__device__ __forceinline__ void epilogue_w8_swiglu(const Params& p,
                                                   const TileCoord& tc,
                                                   f32x16_t (&acc)[2][4],
                                                   int n0, int wm, int wn,
                                                   int lane, int wave,
                                                   char* wbuf, float* wrow) {
  const int colw = lane & 31;
  const int mw = tc.m0 + wm * 64;
  // routing weights of the wave's 64 rows (wrow: 64 floats of LDS per
  // wave), loaded before any store
  wrow[lane] = p.w ? p.w[tc.seg0 + min(mw + lane, tc.seg_len - 1)] : 1.0f;
  const int64_t ld1 = 2 * (int64_t)p.F;
  const int f0 = n0 + 64 * wn;
  const bool fvalid = f0 < p.F;   // F % 64 == 0: whole runs
  auto silu_mul = [&]() {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float g = acc[i][2 * jj][r];
          acc[i][2 * jj][r] = (g * fast_sigmoid(g)) * acc[i][2 * jj + 1][r];
        }
  };
  if (p.c2) {
    // row r: g of the wave's 64 f in columns 0..63, u in 64..127; on
    // readback lane l takes chunk l % 16 of row 4 q + l / 16
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          stage_bf16(wbuf, acc_row(i, r, lane), jj * 32 + colw,
                     acc[i][2 * jj][r]);
          stage_bf16(wbuf, acc_row(i, r, lane), 64 + jj * 32 + colw,
                     acc[i][2 * jj + 1][r]);
        }
    silu_mul();
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging written
    const int ch = lane & 15;
    const int coff = (ch >> 3) * p.F + f0 + 8 * (ch & 7);
#pragma unroll
    for (int qb = 0; qb < 16; qb += 8) {
      uint4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = stage_chunk(wbuf, 4 * (qb + q) + (lane >> 4), ch);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int mrow = mw + 4 * (qb + q) + (lane >> 4);
        if (fvalid && mrow < tc.seg_len)
          *reinterpret_cast<uint4*>(p.c2 + (tc.seg0 + mrow) * ld1 + coff) =
              v[q];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // readback done before reuse
  } else {
    silu_mul();
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stage_f32(wbuf, acc_row(i, r, lane), jj * 32 + colw,
                  acc[i][2 * jj][r]);
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging written
  // lane l: rows 8 q + l / 8, f values 8 (l % 8) .. + 7
  const int c8 = lane & 7;
  const int f = f0 + 8 * c8;
  uint32_t amx = 0;   // amax_out: largest |A| of the lane, bf16 bits
#pragma unroll
  for (int qb = 0; qb < 8; qb += 4) {
    uint4 c0[4], c1[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lr = 8 * (qb + q) + (lane >> 3);
      c0[q] = stage_chunk(wbuf, lr, 2 * c8);
      c1[q] = stage_chunk(wbuf, lr, 2 * c8 + 1);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lr = 8 * (qb + q) + (lane >> 3);
      const int mrow = mw + lr;
      const float wr = wrow[lr];
      const bool ok = fvalid && mrow < tc.seg_len;
      const int64_t row = tc.seg0 + mrow;
      const float v[8] = {
          __uint_as_float(c0[q].x) * wr, __uint_as_float(c0[q].y) * wr,
          __uint_as_float(c0[q].z) * wr, __uint_as_float(c0[q].w) * wr,
          __uint_as_float(c1[q].x) * wr, __uint_as_float(c1[q].y) * wr,
          __uint_as_float(c1[q].z) * wr, __uint_as_float(c1[q].w) * wr};
      if constexpr (EPI == EPI_SWIGLU_MX) {
        // F % 128 == 0: blocks are whole; every lane takes part in the
        // quad reduction, rows past the expert just do not store
        int sx;
        const uint2 w8 = mx_quad_encode_f32(v, &sx);
        if (ok) {
          *reinterpret_cast<uint2*>(p.cq + row * p.F + f) = w8;
          if ((c8 & 3) == 0) {
            p.cs[mx_tile_off((uint32_t)row, (uint32_t)(f / 32),
                             (uint32_t)(p.F / 128))] = (uint8_t)(sx + 127);
            if (p.cs_rm)
              p.cs_rm[row * (p.F / 32) + f / 32] = (uint8_t)(sx + 127);
          }
        }
      }
      if (ok && (EPI == EPI_SWIGLU || p.c)) {
        const uint4 o =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        *reinterpret_cast<uint4*>(p.c + row * p.ldc + f) = o;
        if (p.amax_out) {
          const uint32_t w4[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
          for (int d = 0; d < 4; ++d)
            amx = max(amx, max(w4[d] & 0x7fffu, (w4[d] >> 16) & 0x7fffu));
        }
      }
    }
  }
  if (p.amax_out) {
    // the bf16 magnitudes order like their float32 bits
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
      amx = max(amx, (uint32_t)__shfl_xor((int)amx, off, 64));
    if (lane == 0) atomicMax(p.amax_out, amx << 16);
  }
}

// EPI_SWIGLU_BWD (dgrad of the down projection and the SwiGLU backward) of
// a wave's 128 rows x 64 f (acc[i][j][r] = dA at row acc_row(i, r), f =
// n0 + 64 wn + 32 j + lane % 32), in two passes of 32 f through the wave's
// 16 KiB of LDS (float32, 128-byte rows, stg8).  On readback lane l owns
// rows 16 q + l / 4 and f values 8 (l % 4) .. + 7 of the pass: it reads the
// saved (g, u) of those f with 16-byte loads, writes dg and du with 16-byte
// stores and sums dA silu(g) u for the routing-weight gradient; the four
// lanes of a row, then the tile's four N waves (in wave order, through red)
// add their sums.  wrow: 128 floats per wave; red: 4 x 256 floats.  A wave
// without rows (act false) only meets the barrier.
__device__ __forceinline__ void epilogue_w8_swiglu_bwd(
    const Params& p, const TileCoord& tc, f32x16_t (&acc)[4][2], int n0,
    int wm, int wn, int lane, int t, bool act, char* wbuf, float* wrow,
    float* red) {
  const int64_t ld1 = 2 * (int64_t)p.F;
  const int mw = tc.m0 + wm * 128;
  const int c4 = lane & 3;
  float rsum[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) rsum[q] = 0.0f;
  if (act) {
    const int colw = lane & 31;
    wrow[lane] = p.w ? p.w[tc.seg0 + min(mw + lane, tc.seg_len - 1)] : 1.0f;
    wrow[64 + lane] =
        p.w ? p.w[tc.seg0 + min(mw + 64 + lane, tc.seg_len - 1)] : 1.0f;
    auto fpass = [&](int pass) { return n0 + wn * 64 + 32 * pass; };
    // batch b: pass b / 2, rows q = 4 (b % 2) .. + 3
    auto load_gu = [&](int b, uint4 (&g4)[4], uint4 (&u4)[4]) {
      const int f = fpass(b >> 1) + 8 * c4;
      if (fpass(b >> 1) >= p.F) return;   // F % 32 == 0
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mrow = min(mw + 16 * (4 * (b & 1) + q) + (lane >> 2),
                             tc.seg_len - 1);
        const uint16_t* h = p.h1 + (tc.seg0 + mrow) * ld1 + f;
        g4[q] = *reinterpret_cast<const uint4*>(h);
        u4[q] = *reinterpret_cast<const uint4*>(h + p.F);
      }
    };
    auto stage_pass = [&](int pass) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row(i, r, lane);
          *reinterpret_cast<float*>(wbuf + stg8(row, colw >> 2) +
                                    (colw & 3) * 4) = acc[i][pass][r];
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): staging written
    };
    auto run_batch = [&](int b, const uint4 (&g4)[4], const uint4 (&u4)[4]) {
      const int pass = b >> 1;
      const int f = fpass(pass) + 8 * c4;
      if (fpass(pass) >= p.F) return;
      uint4 c0[4], c1[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = 16 * (4 * (b & 1) + q) + (lane >> 2);
        c0[q] = *reinterpret_cast<const uint4*>(wbuf + stg8(lr, 2 * c4));
        c1[q] = *reinterpret_cast<const uint4*>(wbuf + stg8(lr, 2 * c4 + 1));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qq = 4 * (b & 1) + q;
        const int lr = 16 * qq + (lane >> 2);
        const int mrow = mw + lr;
        const float da[8] = {
            __uint_as_float(c0[q].x), __uint_as_float(c0[q].y),
            __uint_as_float(c0[q].z), __uint_as_float(c0[q].w),
            __uint_as_float(c1[q].x), __uint_as_float(c1[q].y),
            __uint_as_float(c1[q].z), __uint_as_float(c1[q].w)};
        const uint32_t gw[4] = {g4[q].x, g4[q].y, g4[q].z, g4[q].w};
        const uint32_t uw[4] = {u4[q].x, u4[q].y, u4[q].z, u4[q].w};
        const float wr = wrow[lr];
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
    uint4 gA[4], uA[4], gB[4], uB[4];
    load_gu(0, gA, uA);
    stage_pass(0);
    load_gu(1, gB, uB);
    run_batch(0, gA, uA);
    load_gu(2, gA, uA);
    run_batch(1, gB, uB);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // pass 0 readback done
    stage_pass(1);
    load_gu(3, gB, uB);
    run_batch(2, gA, uA);
    run_batch(3, gB, uB);
  }
  if (p.dw_part) {
    if (act) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float v = rsum[q];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        if (c4 == 0) red[wn * BM + wm * 128 + 16 * q + (lane >> 2)] = v;
      }
    }
    __syncthreads();
    if (t < BM) {
      const int mrow = tc.m0 + t;
      if (mrow < tc.seg_len) {
        const float s = ((red[t] + red[BM + t]) + red[2 * BM + t]) +
                        red[3 * BM + t];
        p.dw_part[(int64_t)tc.nt * p.rows + tc.seg0 + mrow] = s;
      }
    }
  }
}


// The barrier that publishes the next step sits halfway through the last
// slice: the next step's first fragment reads overlap the last four MFMAs.
// (Before the rotation, long K loops did better with it after the step's
// last MFMA, which gives the next step's loads the whole step to land:
// Mixtral-shaped down GEMM 1.679 -> 1.656 ms; with the rotation, whose
// weight loads have two steps, halfway is faster there too: gate/up
// 3.104-3.116 -> 3.085-3.089, down 1.659-1.668 -> 1.633-1.634 ms.)

// Five 32 KiB operand buffers in rotation instead of two 64 KiB stages with
// one K step in flight (ms per launch, same box: Qwen3-shaped gate/up 0.884
// -> 0.838-0.845, down 0.529 -> 0.500-0.507; Mixtral-shaped down 1.627 ->
// 1.591; Mixtral-shaped gate/up with eight waves 3.01-3.03 against 3.15
// with four), so that the weight rows (B) are loaded two K steps ahead and the
// token rows (A) one: buffer n % 5 takes B of step k for n = 2 k and A of
// step k for n = 2 k + 1, and step k computes on B_k, A_k while A_{k+1}
// (issued over its first slice) and B_{k+2} (over its second) land in the
// two buffers that B_{k-1} and A_{k-1} have just left.  A weight row that
// no other tile on the XCD is reading (an expert with few rows) comes from
// HBM or the MALL, and one step in flight does not cover that latency;
// token rows are shared by the tile group's N tiles and mostly hit L2.
// The barrier that publishes step k + 1 waits for everything of the wave
// but B_{k+2}: vmcnt counts in issue order.  The buffer that is free in the
// epilogue holds the routing weights, the persistent hand-over and the
// split tail's arrival count.
template <int EPI>
__global__ __launch_bounds__(kThreads8) void grouped_gemm_w8_kernel(Params p) {
  static_assert(EPI == EPI_STORE || EPI == EPI_SWIGLU, "forward epilogues");
  using S = Shape8<EPI>;
  constexpr int MI = S::MI, NJ = S::NJ;
  constexpr int kSl = 4;         // 16-wide K slices per 64-wide step
  constexpr int kStepK = 64;
  __shared__ __attribute__((aligned(1024))) char sA0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kTileBytes];
  // small LDS: routing weights (64 floats per wave), then the persistent
  // hand-over (2 ints) and the split tail's arrival count
  constexpr int kMiscBytes = kThreads8 / 64 * 64 * 4 + 16;
  __shared__ __attribute__((aligned(1024))) char sX4[kTileBytes];
  char* const misc = sX4;
  int* const s_item = reinterpret_cast<int*>(misc + kMiscBytes - 16);
  uint32_t* const arrived =
      reinterpret_cast<uint32_t*>(misc + kMiscBytes - 8);
  const int nk_all = (p.K + kStepK - 1) / kStepK;
  const int t = threadIdx.x;
  // persistent launch (p.queue): items from the XCD counters, the next one
  // taken during the last trip of the current one's K loop (an atomic's
  // round trip then hides under a K step) and handed over through LDS
  // (the down GEMM's items are too long for per-item gaps to matter, and a
  // slow XCD's items are all taken before other XCDs run dry: there the
  // one-item launch is kept)
  constexpr bool kPers = EPI == EPI_SWIGLU;
  const bool pers = kPers && p.queue != nullptr;
  int ix, iidx, xh = 0;
  if (pers) {
    xh = hw_xcd();
    if (t == 0) take_item(p, nk_all, xh, s_item[0], s_item[1]);
    __syncthreads();
    ix = s_item[0];
    iidx = s_item[1];
  } else {
    ix = blockIdx.x % kXcds;
    iidx = blockIdx.x / kXcds;
  }
  for (;;) {
  TileCoord tc;
  SplitRange sr;
  if (ix < 0 || !decode_item(p, nk_all, ix, iidx, tc, sr)) return;

  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / S::WN;
  const int wn = wave % S::WN;
  const int n0 = EPI == EPI_SWIGLU ? tc.nt * (BN / 2) : tc.nt * BN;

  KcDirect8<EPI, false> da;
  KcDirect8<EPI, true> db;
  const int q = 8 * (wave & 3) + (lane >> 3);
  const int cl = (lane & 7) ^ swz32(q);
  // rows past the expert's last read as zeros (buffer descriptor range);
  // a split work-group starts at K step ks
  const uint32_t kofs = (uint32_t)sr.ks * kRowBytes;
  da.base = p.a + (int64_t)tc.seg0 * p.lda + kofs;
  da.rec = (uint32_t)tc.seg_len * (uint32_t)p.lda - kofs;
  da.ld = p.lda;
  da.q = q;
  da.cl = cl;
  da.r0 = tc.m0;
  da.init(wave);
  db.base = p.b + (int64_t)tc.e * p.b_es + kofs;
  db.rec = (uint32_t)p.b_rows * (uint32_t)p.ldb - kofs;
  db.ld = p.ldb;
  db.q = q;
  db.cl = cl;
  db.n0 = n0;
  db.F = p.F;
  db.N = p.N;
  db.init(wave);

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16_t{};

  const int nk = sr.ke - sr.ks;
  // 6 LDS reads and 8 MFMAs per slice; the next step's four A loads go out
  // together ahead of the first slice's first MFMA, its four B loads ahead
  // of the second slice's (Mixtral-shaped down GEMM, ms: one load per MFMA
  // 1.771, two 1.750, four 1.709-1.723; all eight ahead of the first slice
  // 1.749-1.753; Qwen3-shaped gate/up 0.985 -> 0.972 with four)
  auto slice_sched = [&](int kk) {
    if (kk <= 1) sched_vmem_reads_mfma<4, 6, 8, 4>();
    else sched_reads_mfma<6, 8>();
  };
  // A wave whose rows all lie past the expert's last row (the last tile of
  // an expert with few rows) issues its share of the direct loads and meets
  // the barriers, but reads no fragments and runs no MFMAs: with at most
  // half a tile of valid rows, every SIMD then computes for one of its two
  // waves.  Its accumulators stay zero and its epilogue would store nothing.
  const bool act = __builtin_amdgcn_readfirstlane(
                       tc.m0 + wm * MI * 32 < tc.seg_len ? 1 : 0) != 0;
  int nx = -1, ni = 0;   // thread 0 (always in an active wave): next item
  Frags8<MI, NJ> cur, nxt;

  using std::integral_constant;
  auto buf = [&](auto nc) -> char* {
    constexpr int n = decltype(nc)::value % 5;
    if constexpr (n == 0) return sA0;
    else if constexpr (n == 1) return sB0;
    else if constexpr (n == 2) return sA1;
    else if constexpr (n == 3) return sB1;
    else return misc;
  };
  // Lane offsets of each slice's fragments, passed through an empty asm
  // at each use, so that the compiler adds them to a buffer's address per
  // read instead of holding an address per buffer, slice and operand.
  uint32_t fo_a[kSl], fo_b[kSl];
#pragma unroll
  for (int kk = 0; kk < kSl; ++kk)
    Frags8<MI, NJ>::offsets(kk, wm, wn, lane, fo_a[kk], fo_b[kk]);
  struct Offs { uint32_t a, b; };
  auto launder = [&](int kk) {
    Offs o = {fo_a[kk], fo_b[kk]};
    asm volatile("" : "+v"(o.a), "+v"(o.b));
    return o;
  };
  // this wave's loads but the last four (B two steps ahead) have landed
  // and its reads of the step's buffers are done, then every wave's
  constexpr int kWait = (4 & 0xf) | (0x7 << 4);   // vmcnt(4) lgkmcnt(0)
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  int k = 0;
  auto rstep = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    char* const sb = buf(integral_constant<int, 2 * j>{});
    char* const sa = buf(integral_constant<int, 2 * j + 1>{});
    char* const nb = buf(integral_constant<int, 2 * j + 2>{});
    char* const na = buf(integral_constant<int, 2 * j + 3>{});
    char* const nb2 = buf(integral_constant<int, 2 * j + 4>{});
#pragma unroll
    for (int kk = 0; kk < kSl - 1; ++kk) {
      const Offs o = launder(kk + 1);
      if (kk == 0)
        da.issue(na, (uint32_t)(k + 1) * kRowBytes, k + 1 < nk, wave);
      if (kk == 1)
        db.issue(nb2, (uint32_t)(k + 2) * kRowBytes, k + 2 < nk, wave);
      nxt.load_at(sa, sb, o.a, o.b);
      mfma_bf16_w8<2>(cur, acc);
      cur = nxt;
      slice_sched(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
    const Offs o0 = launder(0);
    mfma_bf16_w8<0>(cur, acc);
    __builtin_amdgcn_sched_barrier(0);
    publish();
    nxt.load_at(na, nb, o0.a, o0.b);
    mfma_bf16_w8<1>(cur, acc);
    cur = nxt;
    sched_reads_mfma<6, 4>();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto rstep_idle = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    char* const na = buf(integral_constant<int, 2 * j + 3>{});
    char* const nb2 = buf(integral_constant<int, 2 * j + 4>{});
    da.issue(na, (uint32_t)(k + 1) * kRowBytes, k + 1 < nk, wave);
    db.issue(nb2, (uint32_t)(k + 2) * kRowBytes, k + 2 < nk, wave);
    __builtin_amdgcn_sched_barrier(0);
    publish();
    __builtin_amdgcn_sched_barrier(0);
  };
  // prologue: B_0, A_0, then B_1 (left in flight)
  db.issue(sA0, 0u, true, wave);
  da.issue(sB0, 0u, true, wave);
  db.issue(sA1, (uint32_t)kRowBytes, 1 < nk, wave);
  publish();
  if (act) {
    const Offs o = launder(0);
    cur.load_at(sB0, sA0, o.a, o.b);
  }
  // whole trips of five steps, then the last nk % 5 (before which the
  // persistent launch takes its next item)
  const int trips = nk / 5, rem = nk - 5 * trips;
  auto run = [&](auto st) {
    for (int tr = 0; tr < trips; ++tr) {
      st(integral_constant<int, 0>{});
      ++k;
      st(integral_constant<int, 1>{});
      ++k;
      st(integral_constant<int, 2>{});
      ++k;
      st(integral_constant<int, 3>{});
      ++k;
      st(integral_constant<int, 4>{});
      ++k;
    }
    if (pers && t == 0) take_item(p, nk_all, xh, nx, ni);
    if (rem > 0) {
      st(integral_constant<int, 0>{});
      ++k;
      if (rem > 1) {
        st(integral_constant<int, 1>{});
        ++k;
        if (rem > 2) {
          st(integral_constant<int, 2>{});
          ++k;
          if (rem > 3) st(integral_constant<int, 3>{});
        }
      }
    }
  };
  if (act) run(rstep);
  else run(rstep_idle);

  // every wave is past its last read of the stages (and every direct load
  // has landed) before they become epilogue staging: 16 KiB per wave
  __syncthreads();
  if (pers && t == 0) {
    s_item[0] = nx;
    s_item[1] = ni;
  }
  // (every wave takes part in the hand-over of a split tile's partials)
  const bool last =
      sr.S == 1 || split_reduce<kThreads8>(p, sr, acc, t, arrived);
  if (last && act) {
    char* wbuf = (wave < 2 ? sA0 : wave < 4 ? sB0 : wave < 6 ? sA1 : sB1) +
                 (wave & 1) * (kTileBytes / 2);
    if constexpr (EPI == EPI_STORE)
      epilogue_w8_store(p, tc, acc, n0, wm, wn, lane, wbuf);
    else
      epilogue_w8_swiglu(p, tc, acc, n0, wm, wn, lane, wave, wbuf,
                         reinterpret_cast<float*>(misc) + 64 * wave);
  }
  if (!pers) return;
  // every wave's staging reads are done before the next item's loads
  // write the stages (its stores may still be in flight: they read
  // registers, not LDS), and thread 0's next item is visible
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  ix = s_item[0];
  iidx = s_item[1];
  }
}

template <int EPI>
hipError_t launch_w8(const char* name, const Params& p, int grid,
                     hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  KernelScope ks(name, stream);
  hipLaunchKernelGGL((grouped_gemm_w8_kernel<EPI>), dim3(grid),
                     dim3(kThreads8), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gg
}  // namespace moe
