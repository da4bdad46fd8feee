// The 8-bit forward grouped GEMMs (MXFP8, or E4M3 with tensor scales;
// ragged M, K-contiguous operands) with eight waves per 256 x 256 tile, two
// per SIMD, and the five-buffer operand rotation of grouped_gemm_w8.hpp (the
// weight rows two K steps ahead, the token rows one).  The tile list, the
// split tail, the LDS layout of a step, the per-lane fragment chunks, the
// scale bytes and the scaled MFMA are those of the four-wave kernel in
// grouped_gemm.hpp, so every output element is the same sum of the same
// products (outputs are bit for bit those of the four-wave kernel, except in
// split tiles, whose partial sums run in another order).
//
// Ragged K (weight gradients, EPI_STORE): the tile list, operand ranges and
// scales of the four-wave kernel's RAGGED_K case (expert e's [M, N] tiles,
// K = its padded tokens; an expert without tokens stores zeros).
//
// Wave shapes as in grouped_gemm_w8.hpp: EPI_STORE (down GEMM) 128 rows x 64
// columns, four 32-row A blocks and two B blocks; the SwiGLU epilogues
// (gate/up GEMM) 64 rows x 128 B rows, two A blocks and four B blocks (gate
// and up of 64 f).  Eight MFMAs (32 x 32 x 64, one scale per 32 K values)
// per 64-wide K slice, two slices per 128-wide K step.  With 256 registers
// per wave, fragments are read half a slice ahead (two of the four blocks
// of the operand that has four, the other operand's two once per slice)
// instead of a whole slice: 64 registers of fragments instead of 96.
#pragma once

#include "grouped_gemm_w8.hpp"

namespace moe {
namespace gg {

// One operand fragment of a 64-wide K slice for the lane's row of a 32-row
// block: chunks 4 kk + g and 4 kk + 2 + g (g = lane / 32), as in Frags<P_FP8>.
__device__ __forceinline__ i32x8_t q_frag(const char* s, uint32_t o0,
                                          uint32_t o1, int blk_off) {
  const uint4 lo = *reinterpret_cast<const uint4*>(s + o0 + blk_off);
  const uint4 hi = *reinterpret_cast<const uint4*>(s + o1 + blk_off);
  i32x8_t v;
  v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
  v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
  return v;
}

template <int P, int EPI, int G>
__global__ __launch_bounds__(kThreads8) void grouped_gemm_w8q_kernel(Params p) {
  static_assert(P == P_FP8 || P == P_FP8T, "8-bit operands");
  static_assert(EPI == EPI_STORE ||
                    (P == P_FP8 ? EPI == EPI_SWIGLU_MX : EPI == EPI_SWIGLU),
                "forward epilogues");
  static_assert(G == RAGGED_M || EPI == EPI_STORE, "ragged K: plain store");
  using S = Shape8<EPI>;
  constexpr int MI = S::MI, NJ = S::NJ;   // 32-row A / B blocks of a wave
  // the operand with four blocks is read in halves (X), the other (Y)
  // once per slice
  constexpr bool kXa = MI == 4;
  constexpr int kStepK = 128;     // K values per step (one byte each)
  __shared__ __attribute__((aligned(1024))) char sA0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sX4[kTileBytes];
  const int t = threadIdx.x;
  TileCoord tc;
  SplitRange sr;
  if constexpr (G == RAGGED_M) {
    const int nk_all = (p.K + kStepK - 1) / kStepK;
    if (!decode_item(p, nk_all, blockIdx.x % kXcds, blockIdx.x / kXcds, tc,
                     sr))
      return;
  } else {
    if (!decode_tile<RAGGED_K>(p, tc)) return;
    sr.ks = 0;
    sr.ke = (tc.seg_len + kStepK - 1) / kStepK;   // 0 for an empty expert
    sr.S = 1;
  }

  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / S::WN;   // rows wm * 32 MI
  const int wn = wave % S::WN;   // B rows wn * 32 NJ
  const int n0 = EPI == EPI_STORE ? tc.nt * BN : tc.nt * (BN / 2);

  KcDirect8<EPI, false> da;
  KcDirect8<EPI, true> db;
  const int q = 8 * (wave & 3) + (lane >> 3);
  const int cl = (lane & 7) ^ swz32(q);
  // rows past the expert's last read as zeros (buffer descriptor range);
  // a split work-group starts at K step ks
  // (ragged K: the expert's K range starts at byte seg0 of every row of
  // both operands, a multiple of the K step; rows past M read as zeros)
  const uint32_t kofs =
      G == RAGGED_M ? (uint32_t)sr.ks * kRowBytes : (uint32_t)tc.seg0;
  if constexpr (G == RAGGED_M) {
    da.base = p.a + (int64_t)tc.seg0 * p.lda + kofs;
    da.rec = (uint32_t)tc.seg_len * (uint32_t)p.lda - kofs;
    db.base = p.b + (int64_t)tc.e * p.b_es + kofs;
  } else {
    da.base = p.a + kofs;
    da.rec = (uint32_t)p.M * (uint32_t)p.lda - kofs;
    db.base = p.b + kofs;
  }
  da.ld = p.lda;
  da.q = q;
  da.cl = cl;
  da.r0 = tc.m0;
  da.init(wave);
  db.rec = (uint32_t)p.b_rows * (uint32_t)p.ldb - kofs;
  db.ld = p.ldb;
  db.q = q;
  db.cl = cl;
  db.n0 = n0;
  db.F = p.F;
  db.N = p.N;
  db.init(wave);

  // E8M0 scale bytes (P_FP8T: 127 = 2^0 throughout).  Lane l needs, for
  // each of its A and B blocks, the dword of its row's four block scales of
  // the step, bytes (g, 2 + g) moved to (0, 1) so that the MFMA's opsel
  // picks slice kk's byte (as in the four-wave kernel).
  constexpr uint32_t kS0 = P == P_FP8T ? 0x7f7f7f7fu : 0u;
  uint32_t sa[MI], sb[NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i) sa[i] = kS0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) sb[j] = kS0;
  uint32_t na[MI], nb[NJ];
  uint32_t soa[MI], sob[NJ];
  const uint8_t* sca = nullptr;
  const uint8_t* scb = nullptr;
  const uint32_t sel = (lane >> 5) ? 0x0c0c0301u : 0x0c0c0200u;
  if constexpr (P == P_FP8) {
    // scales of K step s at byte 128 s of a row block's run (ragged K: the
    // expert's first K step at byte seg0)
    sca = p.sa + kofs;
    scb = p.sb + (G == RAGGED_M ? (int64_t)tc.e * p.sb_es : 0) + kofs;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int ra = min(tc.m0 + wm * 32 * MI + 32 * i + (lane & 31),
                         (G == RAGGED_M ? tc.seg_len : p.M) - 1);
      const uint32_t rabs = G == RAGGED_M ? (uint32_t)(tc.seg0 + ra) : ra;
      soa[i] = mx_tile_off(rabs, 0, (uint32_t)p.ldsa);
    }
    KcDirect8<EPI, true> m;   // B row of the lane's 32-row blocks
    m.q = lane & 31;
    m.n0 = n0;
    m.F = p.F;
    m.N = p.N;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      sob[j] = mx_tile_off((uint32_t)m.row(NJ * wn + j), 0, (uint32_t)p.ldsb);
  }
  auto load_scales = [&](int ks) {
    if constexpr (P == P_FP8) {
      const uint8_t* ka = sca + ks * 128;
      const uint8_t* kb = scb + ks * 128;
#pragma unroll
      for (int i = 0; i < MI; ++i)
        na[i] = *reinterpret_cast<const uint32_t*>(ka + soa[i]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        nb[j] = *reinterpret_cast<const uint32_t*>(kb + sob[j]);
    }
  };
  auto take_scales = [&]() {
    if constexpr (P == P_FP8) {
#pragma unroll
      for (int i = 0; i < MI; ++i) sa[i] = __builtin_amdgcn_perm(0u, na[i], sel);
#pragma unroll
      for (int j = 0; j < NJ; ++j) sb[j] = __builtin_amdgcn_perm(0u, nb[j], sel);
    }
  };

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16_t{};

  const int nk = sr.ke - sr.ks;
  // A wave whose rows all lie past the expert's last row issues its share
  // of the direct loads and meets the barriers only (see grouped_gemm_w8.hpp)
  const bool act =
      __builtin_amdgcn_readfirstlane(
          tc.m0 + wm * 32 * MI < (G == RAGGED_M ? tc.seg_len : p.M) ? 1
                                                                     : 0) != 0;

  using std::integral_constant;
  auto buf = [&](auto nc) -> char* {
    constexpr int n = decltype(nc)::value % 5;
    if constexpr (n == 0) return sA0;
    else if constexpr (n == 1) return sB0;
    else if constexpr (n == 2) return sA1;
    else if constexpr (n == 3) return sB1;
    else return sX4;
  };
  // Fragment addresses: lane row r = lane % 32 of a block, chunk c ^ swz(r)
  // with c = 4 kk + 2 e + g, i.e. (4 kk + 2 e) ^ (g ^ swz(r)).  The two
  // per-lane values pass through an empty asm at each use, so that the
  // compiler forms each address when it is needed instead of holding one
  // per buffer, slice, chunk and operand.
  const uint32_t rowoff = (uint32_t)((lane & 31) * kRowBytes);
  const uint32_t xsw = (uint32_t)(swz32(lane & 31) ^ (lane >> 5));
  const int a_wave = wm * 32 * MI * kRowBytes;
  const int b_wave = wn * 32 * NJ * kRowBytes;
  struct Offs { uint32_t o0, o1; };
  auto offs = [&](int kk) {
    uint32_t r = rowoff, x = xsw;
    asm volatile("" : "+v"(r), "+v"(x));
    return Offs{r + (((uint32_t)(4 * kk) ^ x) << 4),
                r + (((uint32_t)(4 * kk + 2) ^ x) << 4)};
  };
  // fragments: X blocks 0-1 (X0) and 2-3 (X1) of a slice, Y of the slice
  // (Yc for slice 0, Yn for slice 1); X = A for EPI_STORE, else B
  i32x8_t X0[2], X1[2], Yc[2], Yn[2];
  const int x_wave = kXa ? a_wave : b_wave, y_wave = kXa ? b_wave : a_wave;
  // (x, y: the step's A and B buffers in X / Y order)
  auto read_x = [&](i32x8_t (&f)[2], const char* s, const Offs& o, int half) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      f[b] = q_frag(s, o.o0, o.o1, x_wave + (2 * half + b) * 32 * kRowBytes);
  };
  auto read_y = [&](i32x8_t (&f)[2], const char* s, const Offs& o) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
      f[b] = q_frag(s, o.o0, o.o1, y_wave + b * 32 * kRowBytes);
  };
  // MFMAs of X half `half` x Y of slice KK; first / last n of the four
  auto mma = [&](auto kkc, auto halfc, const i32x8_t (&fx)[2],
                 const i32x8_t (&fy)[2], auto m0c, auto m1c) {
    constexpr int KK = decltype(kkc)::value, H = decltype(halfc)::value;
    constexpr int M0 = decltype(m0c)::value, M1 = decltype(m1c)::value;
#pragma unroll
    for (int m = M0; m < M1; ++m) {
      const int xx = m >> 1, yy = m & 1;
      const int i = kXa ? 2 * H + xx : yy, j = kXa ? yy : 2 * H + xx;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          kXa ? fx[xx] : fy[yy], kXa ? fy[yy] : fx[xx], acc[i][j], 0, 0, KK,
          (int)sa[i], KK, (int)sb[j]);
    }
  };
  using I0 = integral_constant<int, 0>;
  using I1 = integral_constant<int, 1>;
  using I2 = integral_constant<int, 2>;
  using I4 = integral_constant<int, 4>;
  // this wave's loads but the last four (B two steps ahead) have landed and
  // its reads of the step's buffers are done, then every wave's
  constexpr int kWait = (4 & 0xf) | (0x7 << 4);   // vmcnt(4) lgkmcnt(0)
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  constexpr int kVmA = 4 + (P == P_FP8 ? MI + NJ : 0);   // A (+ scales)
  int k = 0;
  // Step k: B_k in buffer 2 j, A_k in 2 j + 1 (j = k % 5); A_{k+1} goes to
  // 2 j + 3 (with the scales of step k + 1), B_{k+2} to 2 j + 4.
  auto rstep = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    char* const b = buf(integral_constant<int, 2 * j>{});
    char* const a = buf(integral_constant<int, 2 * j + 1>{});
    char* const bn = buf(integral_constant<int, 2 * j + 2>{});
    char* const an = buf(integral_constant<int, 2 * j + 3>{});
    char* const bn2 = buf(integral_constant<int, 2 * j + 4>{});
    const char* const x = kXa ? a : b;
    const char* const y = kXa ? b : a;
    const char* const xn = kXa ? an : bn;
    const char* const yn = kXa ? bn : an;
    // slice 0, X blocks 0-1: A_{k+1} and the scales out; X blocks 2-3 in
    {
      const Offs o = offs(0);
      da.issue(an, (uint32_t)(k + 1) * kRowBytes, k + 1 < nk, wave);
      load_scales(min(k + 1, nk - 1));
      read_x(X1, x, o, 1);
      mma(I0{}, I0{}, X0, Yc, I0{}, I4{});
      sched_vmem_reads_mfma<kVmA, 4, 4, 3>();
      __builtin_amdgcn_sched_barrier(0);
    }
    // slice 0, X blocks 2-3; slice 1's X blocks 0-1 and Y in
    {
      const Offs o = offs(1);
      read_x(X0, x, o, 0);
      read_y(Yn, y, o);
      mma(I0{}, I1{}, X1, Yc, I0{}, I4{});
      sched_reads_mfma<8, 4>();
      __builtin_amdgcn_sched_barrier(0);
    }
    // slice 1, X blocks 0-1: B_{k+2} out; X blocks 2-3 in
    {
      const Offs o = offs(1);
      db.issue(bn2, (uint32_t)(k + 2) * kRowBytes, k + 2 < nk, wave);
      read_x(X1, x, o, 1);
      mma(I1{}, I0{}, X0, Yn, I0{}, I4{});
      sched_vmem_reads_mfma<4, 4, 4, 2>();
      __builtin_amdgcn_sched_barrier(0);
    }
    // slice 1, X blocks 2-3: two MFMAs, publish step k + 1, its first
    // fragments under the last two
    {
      const Offs o = offs(0);
      mma(I1{}, I1{}, X1, Yn, I0{}, I2{});
      __builtin_amdgcn_sched_barrier(0);
      publish();
      read_x(X0, xn, o, 0);
      read_y(Yc, yn, o);
      mma(I1{}, I1{}, X1, Yn, I2{}, I4{});
      take_scales();
      sched_reads_mfma<8, 2>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto rstep_idle = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    char* const an = buf(integral_constant<int, 2 * j + 3>{});
    char* const bn2 = buf(integral_constant<int, 2 * j + 4>{});
    da.issue(an, (uint32_t)(k + 1) * kRowBytes, k + 1 < nk, wave);
    db.issue(bn2, (uint32_t)(k + 2) * kRowBytes, k + 2 < nk, wave);
    __builtin_amdgcn_sched_barrier(0);
    publish();
    __builtin_amdgcn_sched_barrier(0);
  };
  // prologue: B_0 into buffer 0, A_0 (+ scales of step 0) into buffer 1,
  // then B_1 into buffer 2 (left in flight)
  db.issue(sA0, 0u, nk > 0, wave);
  da.issue(sB0, 0u, nk > 0, wave);
  if (act && nk > 0) load_scales(0);
  db.issue(sA1, (uint32_t)kRowBytes, 1 < nk, wave);
  publish();
  if (act) {
    take_scales();
    const Offs o = offs(0);
    read_x(X0, kXa ? sB0 : sA0, o, 0);
    read_y(Yc, kXa ? sA0 : sB0, o);
  }
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
  // (every wave takes part in the hand-over of a split tile's partials;
  // the fifth buffer holds the arrival count)
  if (sr.S > 1 && !split_reduce<kThreads8>(p, sr, acc, t,
                                           reinterpret_cast<uint32_t*>(sX4)))
    return;
  if (!act) return;
  if constexpr (P == P_FP8T) {
    // the two tensor scales
    const float f = p.tsa[0] * p.tsb[tc.e];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] *= f;
  }
  char* wbuf = (wave < 2 ? sA0 : wave < 4 ? sB0 : wave < 6 ? sA1 : sB1) +
               (wave & 1) * (kTileBytes / 2);
  if constexpr (EPI == EPI_STORE)
    epilogue_w8_store<G>(p, tc, acc, n0, wm, wn, lane, wbuf);
  else   // routing weights in the fifth buffer (64 floats per wave)
    epilogue_w8_swiglu<EPI>(p, tc, acc, n0, wm, wn, lane, wave, wbuf,
                            reinterpret_cast<float*>(sX4) + 64 * wave);
}

template <int P, int EPI, int G = RAGGED_M>
hipError_t launch_w8q(const char* name, const Params& p, int grid,
                      hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  KernelScope ks(name, stream);
  hipLaunchKernelGGL((grouped_gemm_w8q_kernel<P, EPI, G>), dim3(grid),
                     dim3(kThreads8), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gg
}  // namespace moe
