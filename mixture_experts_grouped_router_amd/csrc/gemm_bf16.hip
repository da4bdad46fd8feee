// Grouped bf16 GEMMs of the expert MLP (forward and backward) on gfx950.
//
// One grouped GEMM call covers every expert: the tile scheduler reads the
// per-expert row offsets (split_sizes) on the device, so experts with no
// tokens produce no tiles and the host never waits ("NVIDIA presents an
// efficient path for training biological MoE models", section "Grouped
// experts instead of a Python loop"; "Efficient MoE training for biological
// foundation models (NVIDIA)", section "1) Fragmented expert kernels").
// The gate/up GEMM carries ScaledSwiGLU times the routing weight in its
// epilogue, so the intermediate h1 never has to go through HBM ("NVIDIA
// presents ...", section "Reducing memory and quantisation cost";
// "Efficient MoE training ...", section "3) Quantisation overhead in
// low-precision training").
//
// Kernel shape: 256 x 256 output tile, K step 64, 512 threads = 8 waves in a
// 2 (M) x 4 (N) grid, each wave 128 x 64 = 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 with float32 accumulators.  Operands are staged
// through LDS (two buffers, one barrier per K step) in a [mn][k] layout with
// an XOR swizzle on 16-byte chunks; operands whose memory layout is
// MN-contiguous (backward) are transposed in registers on the way in.
// Tiles are ordered so that each XCD (blocks b = x mod 8) works on one
// contiguous run of tiles: consecutive tiles share an expert's weight panel
// and activation rows in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 512;
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
  const int32_t* tile_start;  // RAGGED_M: [E+1] tile prefix; [E+1]: total
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

// byte offset of 16-byte chunk c (0..7) of LDS tile row r: XOR swizzle that
// keeps 8 consecutive rows at one chunk (MFMA fragment reads) and rows
// 8 apart at one chunk (transposed writes) on distinct bank groups.
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * (BK * 2) + (((c ^ r ^ (r >> 3)) & 7) << 4);
}

// Register transpose of a 4 (k) x 8 (mn) block of bf16: in[i] holds row k=i
// (8 values); out[j] gets the 4 k-values of column j packed as 2 dwords.
__device__ __forceinline__ void transpose4x8(const uint4 in[4], uint2 out[8]) {
  const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&in[0]);
  const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&in[1]);
  const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&in[2]);
  const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&in[3]);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // column 2d takes the low halves, column 2d+1 the high halves
    out[2 * d].x = __builtin_amdgcn_perm(r1[d], r0[d], 0x05040100u);
    out[2 * d].y = __builtin_amdgcn_perm(r3[d], r2[d], 0x05040100u);
    out[2 * d + 1].x = __builtin_amdgcn_perm(r1[d], r0[d], 0x07060302u);
    out[2 * d + 1].y = __builtin_amdgcn_perm(r3[d], r2[d], 0x07060302u);
  }
}

struct TileCoord {
  int e;        // expert
  int m0;       // first row of the tile inside the expert's M range
  int n0;       // first column (output units; f units for EPI_SWIGLU)
  int seg0;     // offsets[e]
  int seg_len;  // rows of expert e
  int nt;       // N tile index
};

template <int G>
__device__ __forceinline__ bool decode_tile(const Params& p, TileCoord& tc) {
  const int b = blockIdx.x;
  int total;
  if (G == RAGGED_M) total = p.tile_start[p.E];
  else total = p.E * p.tiles_m * p.tiles_n;
  const int per = (total + kXcds - 1) / kXcds;
  const int idx = b / kXcds;
  if (idx >= per) return false;
  const int L = (b % kXcds) * per + idx;
  if (L >= total) return false;
  int e, local, mt_e;
  if (G == RAGGED_M) {
    // binary search: tile_start[e] <= L < tile_start[e+1]
    int lo = 0, hi = p.E;  // invariant: tile_start[lo] <= L < tile_start[hi]
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
  const int gsz = min(kGroupN, p.tiles_n - ng * kGroupN);
  const int mt = in_g % mt_e;
  const int nt = ng * kGroupN + in_g / mt_e;
  (void)gsz;
  tc.e = e;
  tc.m0 = mt * BM;
  tc.nt = nt;
  tc.seg0 = p.offsets[e];
  tc.seg_len = p.offsets[e + 1] - tc.seg0;
  return true;
}

// ---- operand staging ------------------------------------------------------
// K-contiguous operand: tile rows r = 0..255, 8 chunks of 16 B per row.
// Thread t loads chunk (t & 7) of rows (t >> 3) + 64 i, i = 0..3.
struct KcLoader {
  const uint16_t* ptr[4];
  __device__ __forceinline__ void load(uint4 (&v)[4], int k0) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = *reinterpret_cast<const uint4*>(ptr[i] + k0);
  }
  __device__ __forceinline__ static void store(char* lds, const uint4 (&v)[4]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (t >> 3) + 64 * i;
      *reinterpret_cast<uint4*>(lds + lds_off(r, t & 7)) = v[i];
    }
  }
};

// MN-contiguous operand ([k][mn] in memory): thread t covers mn chunk
// (t & 31) (8 values) for k rows 4 (t >> 5) .. +3; transposed in registers.
struct McLoader {
  const uint16_t* base;   // element (mn = 0, k = 0)
  int64_t ld;             // elements between consecutive k rows
  int kvalid;             // k rows < kvalid are real (rest read as zero)
  __device__ __forceinline__ void load(uint4 (&v)[4], int k0) const {
    const int t = threadIdx.x;
    const int kr = k0 + 4 * (t >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kr + i < kvalid)
        v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)(kr + i) * ld);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ static void store(char* lds, const uint4 (&v)[4]) {
    const int t = threadIdx.x;
    uint2 o[8];
    transpose4x8(v, o);
    const int kg = t >> 5;            // k group of 4 (0..15)
    const int mn0 = (t & 31) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = mn0 + j;
      *reinterpret_cast<uint2*>(lds + lds_off(r, kg >> 1) + (kg & 1) * 8) = o[j];
    }
  }
};

__device__ __forceinline__ float fast_sigmoid(float x) {
  return 1.0f / (1.0f + __expf(-x));
}

template <int LA, int LB, int G, int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * kTileBytes];
  TileCoord tc;
  if (!decode_tile<G>(p, tc)) return;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 2;   // 0..1
  const int wn = wave & 3;    // 0..3

  // ---- tile geometry ----
  int kdim, n0;
  if (G == RAGGED_M) kdim = p.K;
  else kdim = tc.seg_len;
  if (EPI == EPI_SWIGLU) n0 = tc.nt * (BN / 2);   // f units
  else n0 = tc.nt * BN;

  // ---- loaders ----
  KcLoader la_kc, lb_kc;
  McLoader la_mc, lb_mc;
  if (LA == KC) {
    // RAGGED_M: rows seg0 + m0 + r, clamped to the expert's last row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = tc.m0 + (t >> 3) + 64 * i;
      r = min(r, tc.seg_len - 1);
      la_kc.ptr[i] = p.a + (int64_t)(tc.seg0 + r) * p.lda + (t & 7) * 8;
    }
  } else {
    // RAGGED_K: A element (m, k) at a[(seg0 + k) * lda + m]
    int mc = tc.m0 + (t & 31) * 8;
    mc = min(mc, p.M - 8);
    la_mc.base = p.a + (int64_t)tc.seg0 * p.lda + mc;
    la_mc.ld = p.lda;
    la_mc.kvalid = kdim;
  }
  const uint16_t* bexp = p.b + (int64_t)tc.e * p.b_es;
  if (LB == KC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (t >> 3) + 64 * i;
      int brow;
      if (EPI == EPI_SWIGLU) {
        // 32-row blocks alternate gate / up for the same 32 f columns
        const int blk = rr >> 5;
        int f = n0 + (blk >> 1) * 32 + (rr & 31);
        f = min(f, p.F - 1);
        brow = (blk & 1) ? p.F + f : f;
      } else {
        brow = min(n0 + rr, p.N - 1);
      }
      lb_kc.ptr[i] = bexp + (int64_t)brow * p.ldb + (t & 7) * 8;
    }
  } else {
    int nc = n0 + (t & 31) * 8;
    nc = min(nc, p.N - 8);
    if (G == RAGGED_M) {
      lb_mc.base = bexp + nc;     // B element (n, k) at b_e[k * ldb + n]
      lb_mc.kvalid = kdim;
    } else {
      lb_mc.base = p.b + (int64_t)tc.seg0 * p.ldb + nc;
      lb_mc.kvalid = kdim;
    }
    lb_mc.ld = p.ldb;
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (kdim + BK - 1) / BK;
  uint4 va[4], vb[4];
  auto gload = [&](int kt) {
    if (LA == KC) la_kc.load(va, kt * BK); else la_mc.load(va, kt * BK);
    if (LB == KC) lb_kc.load(vb, kt * BK); else lb_mc.load(vb, kt * BK);
  };
  auto sstore = [&](int buf) {
    char* sa = smem + buf * 2 * kTileBytes;
    char* sb = sa + kTileBytes;
    if (LA == KC) KcLoader::store(sa, va); else McLoader::store(sa, va);
    if (LB == KC) KcLoader::store(sb, vb); else McLoader::store(sb, vb);
  };

  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  const int frow = lane & 31;
  const int fk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const char* sa = smem + buf * 2 * kTileBytes;
    const char* sb = sa + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t fa[4], fb[2];
      const int ch = kk * 2 + fk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t*>(
            sa + lds_off(wm * 128 + i * 32 + frow, ch));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8_t*>(
            sb + lds_off(wn * 64 + j * 32 + frow, ch));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j],
                                                              acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  // acc[i][j][r] is C[row][col] with
  //   row = wm*128 + i*32 + (r/4)*8 + (lane/32)*4 + r%4,  col = lane%32 (+ j*32)
  const int colw = lane & 31;
  const int rsub = (lane >> 5) * 4;
  if (EPI == EPI_SWIGLU) {
    const int f = n0 + wn * 32 + colw;
    const bool fok = f < p.F;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mrow = tc.m0 + wm * 128 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
        if (mrow < tc.seg_len && fok) {
          const int64_t row = tc.seg0 + mrow;
          const float g = acc[i][0][r], u = acc[i][1][r];
          const float wr = p.w ? p.w[row] : 1.0f;
          const float a = wr * (g * fast_sigmoid(g)) * u;
          p.c[row * p.ldc + f] = (uint16_t)f32_to_bf16(a);
          if (p.c2) {
            p.c2[row * (2 * (int64_t)p.F) + f] = (uint16_t)f32_to_bf16(g);
            p.c2[row * (2 * (int64_t)p.F) + p.F + f] = (uint16_t)f32_to_bf16(u);
          }
        }
      }
  } else if (EPI == EPI_STORE) {
    uint16_t* cbase = p.c + (G == RAGGED_K ? (int64_t)tc.e * p.c_es : 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + colw;
      if (col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mrow = tc.m0 + wm * 128 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          int64_t row;
          if (G == RAGGED_M) {
            if (mrow >= tc.seg_len) continue;
            row = tc.seg0 + mrow;
          } else {
            if (mrow >= p.M) continue;
            row = mrow;
          }
          cbase[row * p.ldc + col] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        }
    }
  } else {  // EPI_SWIGLU_BWD: acc = dA[row][f], f = n0 + wn*64 + j*32 + col
    // One 32-row block at a time so only 16 partial row sums are live.
    float* red = reinterpret_cast<float*>(smem);  // [4 N-waves][256 rows]
    const int64_t ld1 = 2 * (int64_t)p.F;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float rs[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) rs[r] = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int f = n0 + wn * 64 + j * 32 + colw;
        const bool fok = f < p.F;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mrow = tc.m0 + wm * 128 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
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
      // across the 4 N-waves, fixed order
      __syncthreads();
      if (t < 256) {
        const int mrow = tc.m0 + t;
        if (mrow < tc.seg_len) {
          const float s = red[t] + red[256 + t] + red[512 + t] + red[768 + t];
          p.dw_part[(int64_t)tc.nt * p.rows + tc.seg0 + mrow] = s;
        }
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
