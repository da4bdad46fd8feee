// The bf16 backward grouped GEMMs with a plain store (the dgrad of the
// gate/up projection: ragged M, K-contiguous A, N-contiguous weights; the
// weight gradients: ragged K, both operands M- / N-contiguous) with eight
// waves per 256 x 256 tile, two per SIMD, and the five-buffer operand
// rotation of grouped_gemm_w8.hpp (B two K steps ahead, A one).  The tile
// lists, operand ranges, LDS stage layouts (K-contiguous: 256 rows of 128
// bytes; N-contiguous: 64 k rows of 512 bytes, read with transposing LDS
// reads) and MFMAs are those of the four-wave kernel in grouped_gemm.hpp, so
// every output is the same sum of the same products.
//
// Wave shape: 128 rows x 64 columns (a 2 x 4 wave grid), four 32-row A
// blocks and two 32-column B blocks, eight 32 x 32 x 16 MFMAs per 16-wide K
// slice, four slices per 64-wide K step; fragments are read one slice ahead.
#pragma once

#include "grouped_gemm_w8.hpp"

namespace moe {
namespace gg {

// ---- MN-contiguous bf16 operand: direct global -> LDS, transposed reads -----
// The stage holds the step's 64 k rows of the tile's 256 mn values (512
// bytes each) as they lie in memory; 16-byte chunk c of row k sits at chunk
// c ^ 4 (k & 3).  With eight waves, wave w, instruction j (of 4) fills KiB
// 8 j + w of the stage = k rows 2 (8 j + w) + lane / 32, each lane loading
// the logical chunk that belongs at its slot.  MFMA fragments come from
// ds_read_b64_tr_b16: in a group of 16 lanes, lane i receives element i % 4
// of the 8 bytes addressed by lane 4 j + i / 4 as its element j; with lane
// 4 j + q addressing row k0 + j, mn mb + 4 q .. +3, lane i gets mn mb + i
// at k0 .. k0 + 3.  Two such reads (k and k + 4) give a lane its 8 k values;
// the swizzle puts the 4 rows x 2 groups of a read on 16 distinct chunks (no
// bank conflicts).  Rows at or past kvalid read as zeros through the buffer
// descriptor; mn past the operand's end reads the next row (or zeros):
// those outputs are never stored.
struct McDirect8 {
  const char* base;  // wave-uniform: element (k = 0, mn = tile start)
  uint32_t rec;      // valid bytes from base
  int64_t ld;        // bytes per k row
  uint32_t off[4];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 2 * (8 * j + wave) + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (row & 3));
      off[j] = (uint32_t)row * (uint32_t)ld + (uint32_t)(c * 16);
    }
  }
  __device__ __forceinline__ void issue(char* lds_tile, int kt, bool real,
                                        int wave) const {
    const uint32_t kb = (uint32_t)kt * 64u * (uint32_t)ld;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + kb), (short)0, (int)(real ? rec - kb : 0u),
        kBufFlags);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      MOE_LDS void* dst = (MOE_LDS void*)(lds_tile + (8 * j + wave) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off[j], 0, 0, 0);
    }
  }
  // lane's byte offsets of its nb 32-wide blocks (K slice 0, first of the
  // two reads) starting at mn chunk xb of the stage rows
  template <int NB>
  static __device__ __forceinline__ void frag_offsets(int xb, int lane,
                                                      uint32_t (&o)[NB]) {
    const int G = lane >> 4, s = lane & 15, j = s >> 2, q = s & 3;
    const int k0 = 8 * (G >> 1) + j;
    const int x = 2 * (G & 1) + (q >> 1) + xb;   // chunk, bits 2-3 clear
#pragma unroll
    for (int i = 0; i < NB; ++i)
      o[i] = (uint32_t)(k0 * 512 + (((x + 4 * i) ^ (4 * j)) * 16) +
                        (q & 1) * 8);
  }
};

template <int LA, int LB, int G, int EPI = EPI_STORE>
__global__ __launch_bounds__(kThreads8) void grouped_gemm_w8b_kernel(Params p) {
  static_assert((G == RAGGED_M && LA == KC && LB == MC) ||
                    (G == RAGGED_K && LA == MC && LB == MC),
                "backward operand layouts");
  // the dgrad of the down projection may carry the SwiGLU backward
  static_assert(EPI == EPI_STORE || (EPI == EPI_SWIGLU_BWD && G == RAGGED_M),
                "plain store, or the SwiGLU backward on a ragged-M dgrad");
  constexpr int MI = 4, NJ = 2;   // 32-row A / 32-column B blocks of a wave
  constexpr int kSl = 4;          // 16-wide K slices per 64-wide step
  constexpr int kStepK = 64;
  __shared__ __attribute__((aligned(1024))) char sA0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sX4[kTileBytes];
  const int t = threadIdx.x;
  TileCoord tc;
  if (!decode_tile<G>(p, tc)) return;
  const int kdim = G == RAGGED_M ? p.K : tc.seg_len;
  const int nk = (kdim + kStepK - 1) / kStepK;   // 0: an empty expert

  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 2;   // rows wm * 128
  const int wn = wave & 3;    // columns wn * 64
  const int n0 = tc.nt * BN;

  KcDirect8<EPI_STORE, false> da;
  McDirect8 ma, mb;
  if constexpr (LA == KC) {
    // rows seg0 + m0 + r; rows past the expert's last read as zeros
    const int q = 8 * (wave & 3) + (lane >> 3);
    da.base = p.a + (int64_t)tc.seg0 * p.lda;
    da.rec = (uint32_t)tc.seg_len * (uint32_t)p.lda;
    da.ld = p.lda;
    da.q = q;
    da.cl = (lane & 7) ^ swz32(q);
    da.r0 = tc.m0;
    da.init(wave);
  } else {
    // A element (m, k) at a + (seg0 + k) * lda + 2 m (k = token)
    ma.base = p.a + (int64_t)tc.seg0 * p.lda + 2 * (int64_t)tc.m0;
    ma.rec = (uint32_t)kdim * (uint32_t)p.lda - 2u * (uint32_t)tc.m0;
    ma.ld = p.lda;
    ma.init(wave, lane);
  }
  // B element (n, k) at b_e + k * ldb + 2 n (ragged K: b + (seg0 + k) ...)
  if constexpr (G == RAGGED_M)
    mb.base = p.b + (int64_t)tc.e * p.b_es + 2 * (int64_t)n0;
  else
    mb.base = p.b + (int64_t)tc.seg0 * p.ldb + 2 * (int64_t)n0;
  mb.rec = (uint32_t)kdim * (uint32_t)p.ldb - 2u * (uint32_t)n0;
  mb.ld = p.ldb;
  mb.init(wave, lane);
  auto issue_a = [&](char* dst, int kt) {
    if constexpr (LA == KC)
      da.issue(dst, (uint32_t)kt * kRowBytes, kt < nk, wave);
    else
      ma.issue(dst, kt, kt < nk, wave);
  };
  auto issue_b = [&](char* dst, int kt) { mb.issue(dst, kt, kt < nk, wave); };

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16_t{};

  // A wave whose rows all lie past the end (ragged M: the expert's rows;
  // ragged K: M) issues its share of the direct loads and meets the
  // barriers only (see grouped_gemm_w8.hpp)
  const bool act =
      __builtin_amdgcn_readfirstlane(
          tc.m0 + wm * 128 < (G == RAGGED_M ? tc.seg_len : p.M) ? 1 : 0) != 0;

  using std::integral_constant;
  auto buf = [&](auto nc) -> char* {
    constexpr int n = decltype(nc)::value % 5;
    if constexpr (n == 0) return sA0;
    else if constexpr (n == 1) return sB0;
    else if constexpr (n == 2) return sA1;
    else if constexpr (n == 3) return sB1;
    else return sX4;
  };
  // Per-lane fragment offsets, passed through an empty asm at each use so
  // that the compiler forms the addresses when they are needed.
  // K-contiguous A: slice kk's chunk of the lane's row (frag_off);
  // N-contiguous: the blocks' offsets of slice 0 (a slice adds 16 k rows).
  uint32_t fa[kSl], tra[MI], trb[NJ];
  if constexpr (LA == KC) {
#pragma unroll
    for (int kk = 0; kk < kSl; ++kk)
      fa[kk] = (uint32_t)(wm * 128 * kRowBytes +
                          frag_off(lane & 31, kk * 2 + (lane >> 5)));
  } else {
    McDirect8::frag_offsets<MI>(16 * wm, lane, tra);
  }
  McDirect8::frag_offsets<NJ>(8 * wn, lane, trb);
  struct Frg { bf16x8_t a[MI], b[NJ]; };
  auto read = [&](Frg& f, const char* sa, const char* sb, int kk) {
    if constexpr (LA == KC) {
      uint32_t o = fa[kk];
      asm volatile("" : "+v"(o));
#pragma unroll
      for (int i = 0; i < MI; ++i)
        f.a[i] = *reinterpret_cast<const bf16x8_t*>(sa + o +
                                                    i * 32 * kRowBytes);
    } else {
      uint32_t o[MI];
#pragma unroll
      for (int i = 0; i < MI; ++i) o[i] = tra[i];
      asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
#pragma unroll
      for (int i = 0; i < MI; ++i)
        f.a[i] = Frags<P_BF16>::tr8(sa + kk * 16 * 512 + o[i]);
    }
    uint32_t ob[NJ] = {trb[0], trb[1]};
    asm volatile("" : "+v"(ob[0]), "+v"(ob[1]));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      f.b[j] = Frags<P_BF16>::tr8(sb + kk * 16 * 512 + ob[j]);
  };
  // MFMAs of A blocks [I0, I1) x both B blocks
  auto mma = [&](const Frg& f, auto i0c, auto i1c) {
    constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j],
                                                            acc[i][j], 0, 0, 0);
  };
  using I0 = integral_constant<int, 0>;
  using I2 = integral_constant<int, 2>;
  using I4 = integral_constant<int, 4>;
  // LDS reads per slice: A 4 (K-contiguous) or 8 (two transposed reads per
  // block), B 4
  constexpr int kNR = (LA == KC ? 4 : 8) + 4;
  // this wave's loads but the last four (B two steps ahead) have landed and
  // its reads of the step's buffers are done, then every wave's
  constexpr int kWait = (4 & 0xf) | (0x7 << 4);   // vmcnt(4) lgkmcnt(0)
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  Frg cur, nxt;
  int k = 0;
  // Step k: B_k in buffer 2 j, A_k in 2 j + 1 (j = k % 5); A_{k+1} goes to
  // 2 j + 3 over the first slice, B_{k+2} to 2 j + 4 over the second.
  auto rstep = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    char* const b = buf(integral_constant<int, 2 * j>{});
    char* const a = buf(integral_constant<int, 2 * j + 1>{});
    char* const bn = buf(integral_constant<int, 2 * j + 2>{});
    char* const an = buf(integral_constant<int, 2 * j + 3>{});
    char* const bn2 = buf(integral_constant<int, 2 * j + 4>{});
#pragma unroll
    for (int kk = 0; kk < kSl - 1; ++kk) {
      if (kk == 0) issue_a(an, k + 1);
      if (kk == 1) issue_b(bn2, k + 2);
      read(nxt, a, b, kk + 1);
      mma(cur, I0{}, I4{});
      cur = nxt;
      if (kk <= 1) sched_vmem_reads_mfma<4, kNR, 8, 2>();
      else sched_reads_mfma<kNR, 8>();
      __builtin_amdgcn_sched_barrier(0);
    }
    // last slice: half the MFMAs, publish step k + 1, its first fragments
    // under the other half
    mma(cur, I0{}, I2{});
    __builtin_amdgcn_sched_barrier(0);
    publish();
    read(nxt, an, bn, 0);
    mma(cur, I2{}, I4{});
    cur = nxt;
    sched_reads_mfma<kNR, 4>();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto rstep_idle = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    char* const an = buf(integral_constant<int, 2 * j + 3>{});
    char* const bn2 = buf(integral_constant<int, 2 * j + 4>{});
    issue_a(an, k + 1);
    issue_b(bn2, k + 2);
    __builtin_amdgcn_sched_barrier(0);
    publish();
    __builtin_amdgcn_sched_barrier(0);
  };
  // prologue: B_0 into buffer 0, A_0 into buffer 1, then B_1 into buffer 2
  // (left in flight)
  issue_b(sA0, 0);
  issue_a(sB0, 0);
  issue_b(sA1, 1);
  publish();
  if (act) read(cur, sB0, sA0, 0);
  // whole trips of five steps, then the last nk % 5
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

  // every wave is past its last read of the buffers (and every direct load
  // has landed) before they become epilogue staging: 16 KiB per wave
  __syncthreads();
  char* wbuf = (wave < 2 ? sA0 : wave < 4 ? sB0 : wave < 6 ? sA1 : sB1) +
               (wave & 1) * (kTileBytes / 2);
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    // routing weights (128 per wave), then the four N waves' row sums, in
    // the fifth buffer; every wave meets the row-sum barrier
    float* misc = reinterpret_cast<float*>(sX4);
    epilogue_w8_swiglu_bwd(p, tc, acc, n0, wm, wn, lane, t, act, wbuf,
                           misc + 128 * wave, misc + 128 * 8);
    return;
  }
  if (!act) return;
  epilogue_w8_store<G>(p, tc, acc, n0, wm, wn, lane, wbuf);
}

template <int LA, int LB, int G, int EPI = EPI_STORE>
hipError_t launch_w8b(const char* name, const Params& p, int grid,
                      hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  KernelScope ks(name, stream);
  hipLaunchKernelGGL((grouped_gemm_w8b_kernel<LA, LB, G, EPI>), dim3(grid),
                     dim3(kThreads8), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gg
}  // namespace moe
