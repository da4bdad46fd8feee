// MXFP8 quantisation of bf16 tensors: E4M3 elements, one E8M0 scale per
// block of 32 consecutive values ("NVIDIA presents an efficient path for
// training biological MoE models", section "Reducing memory and quantisation
// cost"; "Efficient MoE training for biological foundation models
// (NVIDIA)", section "2) Model size and activation memory").  16-bit master
// weights are quantised from bf16 on the fly ("Efficient MoE training ...",
// section "3) Quantisation overhead in low-precision training").
//
// Scale exponent s = floor(log2 amax) - 8 (integer operations on the bf16
// amax, mx_codec.hpp); elements E4M3(v * 2^-s) with round to nearest even
// and saturation at 448, by the gfx950 scaled conversion (common.hpp).  All
// kernels are HBM-bound streaming passes: 2 bytes read, 1 + 1/32 bytes
// written per element.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "timer.hpp"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) {
  return a > b ? a : b;
}


__device__ __forceinline__ uint32_t amax8(const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a = umax(a, w[i] & 0x7fffu);
    a = umax(a, (w[i] >> 16) & 0x7fffu);
  }
  return a;
}

// Row-wise with row-major scales [rows, cols / 32]: 4 consecutive lanes own
// one block of 32 along a row; every thread keeps U independent 16-byte
// loads in flight.
constexpr int kRowsUnroll = 4;

__global__ __launch_bounds__(256) void mx_rows_kernel(
    const uint4* __restrict__ src, int64_t n_chunks,
    uint2* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t S = (int64_t)gridDim.x * blockDim.x;
  // n_chunks and S are multiples of 4: groups of 4 lanes stay aligned to
  // blocks and are either wholly in range or wholly out
  for (int64_t c0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
       c0 - threadIdx.x % 4 < n_chunks; c0 += kRowsUnroll * S) {
    uint4 v[kRowsUnroll];
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
      const int64_t c = c0 + u * S;
      v[u] = c < n_chunks ? ld_nt(src + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
      const int64_t c = c0 + u * S;
      uint32_t a = amax8(v[u]);
      a = umax(a, __shfl_xor(a, 1, 64));
      a = umax(a, __shfl_xor(a, 2, 64));
      const int s = e8m0_exp_from_bf16_amax(a);
      if (c < n_chunks) {
        codes[c] = e4m3x8_hw(v[u], s);
        if ((c & 3) == 0) scales[c >> 2] = (uint8_t)(s + 127);
      }
    }
  }
}

// Row-wise into the GEMM scale layout: a block covers 32 rows x 256 values
// (two K steps of 128).  Wave w takes rows 8w .. 8w+7; lane l row 8w + l/8
// and, for load u, chunk 8u + l%8 of the window, so the 8 lanes of a row
// read 128 contiguous bytes and 4 consecutive lanes hold one block of 32.
// The block's scale bytes (32 rows x 2 steps x 4 blocks) are gathered in
// LDS and leave as whole 128-byte lines, one per step (in the GEMM layout
// the 32 rows x 4 blocks of one step are one line); single-byte stores
// scattered over those lines cost the HBM-bound pass ~15% extra write
// traffic.  Rows past the end of the last group get the scale of an
// all-zero block (storage covers rows rounded up to 32).
constexpr int kTiledWin = 32;   // 16-byte chunks per window (256 values)

__global__ __launch_bounds__(256) void mx_rows_tiled_kernel(
    const uint4* __restrict__ src, int64_t rows, int cols8, int nwin,
    uint32_t nks, uint2* __restrict__ codes, uint32_t* __restrict__ scales) {
  __shared__ uint32_t sc[64];   // [step][row]: the 4 block scales of a step
  const int64_t g = blockIdx.x / nwin;
  const int win = (int)(blockIdx.x - g * nwin);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int rr = 8 * wave + (lane >> 3);
  const int64_t row = g * 32 + rr;
  const bool rv = row < rows;
  const int cw0 = win * kTiledWin;
  const uint4* srow = src + row * cols8;
  uint4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = cw0 + 8 * u + (lane & 7);
    v[u] = (rv && c < cols8) ? ld_nt(srow + c) : make_uint4(0, 0, 0, 0);
  }
  uint8_t* scb = reinterpret_cast<uint8_t*>(sc);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = cw0 + 8 * u + (lane & 7);
    uint32_t a = amax8(v[u]);
    a = umax(a, __shfl_xor(a, 1, 64));
    a = umax(a, __shfl_xor(a, 2, 64));
    const int s = e8m0_exp_from_bf16_amax(a);
    if (rv && c < cols8) codes[row * cols8 + c] = e4m3x8_hw(v[u], s);
    if ((lane & 3) == 0) {
      const int blk = (8 * u + (lane & 7)) >> 2;   // block of the window
      scb[((blk >> 2) * 32 + rr) * 4 + (blk & 3)] = (uint8_t)(s + 127);
    }
  }
  __syncthreads();
  if (t < 64) {
    const int step = t >> 5;
    if (cw0 + 16 * step < cols8)
      scales[(g * nks + 2 * win + step) * 32 + (t & 31)] = sc[t];
  }
}

// Column-wise tile kernel: a block covers 32 rows x 64 columns of one batch
// entry; blocks run down the columns (32 values); output transposed.
// Segment mode: rows come from one segment (zero-padded past its end) and
// land at output offsets where every segment starts on a multiple of
// 32 * pad_tiles.
template <bool SEG, bool TILED>
__global__ __launch_bounds__(256) void mx_cols_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
    const int32_t* __restrict__ seg_offsets, int n_seg, int pad_tiles,
    int64_t ld_out, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int32_t* status) {
  __shared__ uint16_t tile[32][64 + 2];
  __shared__ int32_t tprefix[1025];
  const int t = threadIdx.x;
  const int64_t b = blockIdx.z;
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  int64_t r0, rend, out0;
  if (SEG) {
    // tile prefix over segments (ceil(n_s / (32 pad_tiles)) * pad_tiles
    // row tiles each): thread t owns segments 4t .. 4t+3, then a block-wide
    // exclusive scan.
    const int pad = 32 * pad_tiles;
    if (!seg_offsets_ok(seg_offsets, n_seg, rows, t, status)) return;
    int32_t cnt4[4], own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = 4 * t + i;
      cnt4[i] = sg < n_seg
                    ? (seg_offsets[sg + 1] - seg_offsets[sg] + pad - 1) / pad *
                          pad_tiles
                    : 0;
      own += cnt4[i];
    }
    int32_t total;
    int32_t run = block_exclusive_scan_256(own, &total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = 4 * t + i;
      if (sg < n_seg) tprefix[sg] = run;
      run += cnt4[i];
    }
    if (t == 0) tprefix[n_seg] = total;
    __syncthreads();
    const int g = blockIdx.x;
    if (g >= tprefix[n_seg]) return;
    int lo = 0, hi = n_seg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tprefix[mid] <= g) lo = mid; else hi = mid;
    }
    const int lt = g - tprefix[lo];
    r0 = seg_offsets[lo] + (int64_t)lt * 32;
    rend = seg_offsets[lo + 1];
    out0 = (int64_t)g * 32;
  } else {
    r0 = (int64_t)blockIdx.x * 32;
    rend = rows;
    out0 = r0;
  }
  const uint16_t* base = src + b * rows * cols;
  // load 32 x 64: thread t -> row t / 8, 16-byte chunk t % 8
  {
    const int rr = t >> 3, ch = t & 7;
    const int64_t r = r0 + rr;
    const int64_t c = c0 + ch * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rend && c < cols)
      v = *reinterpret_cast<const uint4*>(base + r * cols + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[rr][ch * 8 + 2 * i] = (uint16_t)(w[i] & 0xffffu);
      tile[rr][ch * 8 + 2 * i + 1] = (uint16_t)(w[i] >> 16);
    }
  }
  __syncthreads();
  // thread t -> column t / 4, rows 8 (t % 4) .. +7
  const int col = t >> 2, q = t & 3;
  uint32_t a = 0;
  uint32_t vals[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    vals[i] = tile[q * 8 + i][col];
    a = umax(a, vals[i] & 0x7fffu);
  }
  a = umax(a, __shfl_xor(a, 1, 64));
  a = umax(a, __shfl_xor(a, 2, 64));
  const int s = e8m0_exp_from_bf16_amax(a);
  const int64_t c = c0 + col;
  if (c < cols) {
    const float sc = mx_scale_f32(s);
    const uint32_t lo = e4m3x4_hw(vals[0] | (vals[1] << 16),
                                  vals[2] | (vals[3] << 16), sc);
    const uint32_t hi = e4m3x4_hw(vals[4] | (vals[5] << 16),
                                  vals[6] | (vals[7] << 16), sc);
    const int64_t orow = b * cols + c;   // output row
    *reinterpret_cast<uint2*>(codes + orow * ld_out + out0 + q * 8) =
        make_uint2(lo, hi);
    if (q == 0) {
      const int64_t kb = out0 / 32;
      if (TILED)
        scales[mx_tile_off((uint32_t)orow, (uint32_t)kb,
                           (uint32_t)(ld_out / 128))] = (uint8_t)(s + 127);
      else
        scales[orow * (ld_out / 32) + kb] = (uint8_t)(s + 127);
    }
  }
}

// Column-wise with 128-row tiles: a block covers 128 rows x 64 columns
// (four blocks of 32 down each column) and writes 128 contiguous code bytes
// per column.  Thread t loads rows 4 (t >> 3) .. +3 of 16-byte column chunk
// t & 7 and writes them transposed into LDS ([column][row]); then thread t
// quantises rows 32 (t & 3) .. +31 of column t >> 2 from four 16-byte LDS
// reads.  Segment mode: tiles of one segment (zero past its end), output at
// offsets where every segment starts on a multiple of 128 * pad_tiles; a
// block there takes NCB consecutive 64-column chunks of its row tile, so
// that its prologue (offsets check, segment scan and search) is paid once
// per NCB chunks.  ROWS: the same pass also writes the row-wise codes
// [rows][cols] and scales (GEMM layout) of the rows it loads, each thread
// encoding the four 8-value runs it holds, a quad of lanes per 32-value
// block: one read of the tensor serves both directions.
template <bool SEG, bool TILED, int NCB = 1, bool ROWS = false>
__global__ __launch_bounds__(256) void mx_cols128_kernel(
    const uint4* __restrict__ src, int64_t rows, int64_t cols,
    const int32_t* __restrict__ seg_offsets, int n_seg, int pad_tiles,
    int64_t ld_out, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int32_t* status,
    uint2* __restrict__ row_codes = nullptr,
    uint8_t* __restrict__ row_scales = nullptr) {
  __shared__ __attribute__((aligned(16))) uint16_t tileT[64][128 + 8];
  __shared__ int32_t tprefix[1025];
  // ROWS: the row-wise scale bytes of the block's rows, [row][block of 32
  // along the NCB chunks], stored after the chunks as one dword per row and
  // four blocks (the GEMM layout keeps those four bytes together)
  __shared__ __attribute__((aligned(4))) uint8_t rsc[ROWS ? 128 : 1]
                                                    [ROWS ? 2 * NCB : 1];
  const int t = threadIdx.x;
  const int64_t b = blockIdx.z;
  int64_t r0, rend, out0;
  if (SEG) {
    const int pad = 128 * pad_tiles;
    if (!seg_offsets_ok(seg_offsets, n_seg, rows, t, status)) return;
    int32_t cnt4[4], own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = 4 * t + i;
      cnt4[i] = sg < n_seg
                    ? (seg_offsets[sg + 1] - seg_offsets[sg] + pad - 1) / pad *
                          pad_tiles
                    : 0;
      own += cnt4[i];
    }
    int32_t total;
    int32_t run = block_exclusive_scan_256(own, &total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = 4 * t + i;
      if (sg < n_seg) tprefix[sg] = run;
      run += cnt4[i];
    }
    if (t == 0) tprefix[n_seg] = total;
    __syncthreads();
    const int g = blockIdx.x;
    if (g >= tprefix[n_seg]) return;
    int lo = 0, hi = n_seg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tprefix[mid] <= g) lo = mid; else hi = mid;
    }
    r0 = seg_offsets[lo] + (int64_t)(g - tprefix[lo]) * 128;
    rend = seg_offsets[lo + 1];
    out0 = (int64_t)g * 128;
  } else {
    r0 = (int64_t)blockIdx.x * 128;
    rend = rows;
    out0 = r0;
  }
  const int64_t cpr = cols / 8;   // 16-byte chunks per row (cols % 8 == 0)
  const uint4* base = src + b * rows * cpr;
  uint2 pend[4];   // ROWS: row codes of the previous (even) chunk
  for (int cb = 0; cb < NCB; ++cb) {
    const int64_t c0 = ((int64_t)blockIdx.y * NCB + cb) * 64;
    if (c0 >= cols) break;
    if (cb > 0) __syncthreads();   // the previous chunk's LDS reads are done
    {
      const int ch = t & 7, rq = t >> 3;
      const int64_t c = c0 / 8 + ch;
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 4 * rq + i;
        v[i] = (r < rend && c < cpr) ? ld_nt(base + r * cpr + c)
                                     : make_uint4(0, 0, 0, 0);
      }
      if constexpr (ROWS) {
        // every lane of a quad takes part; rows past the end do not store
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t a = amax8(v[i]);
          a = umax(a, __shfl_xor(a, 1, 64));
          a = umax(a, __shfl_xor(a, 2, 64));
          const int s = e8m0_exp_from_bf16_amax(a);
          const int64_t r = r0 + 4 * rq + i;
          // a 128-byte line of codes spans two chunks: the even chunk's
          // codes wait in registers and go out with the odd chunk's
          const uint2 cw = e4m3x8_hw(v[i], s);
          if (cb & 1) {
            if (r < rend && c < cpr) {
              uint2* rc = row_codes + (b * rows + r) * cpr + c;
              rc[-8] = pend[i];
              rc[0] = cw;
            }
          } else {
            pend[i] = cw;
          }
          if ((ch & 3) == 0) rsc[4 * rq + i][2 * cb + (ch >> 2)] =
              (uint8_t)(s + 127);
        }
      }
      const uint32_t w[4][4] = {{v[0].x, v[0].y, v[0].z, v[0].w},
                                {v[1].x, v[1].y, v[1].z, v[1].w},
                                {v[2].x, v[2].y, v[2].z, v[2].w},
                                {v[3].x, v[3].y, v[3].z, v[3].w}};
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int sh = (cc & 1) * 16;
        const uint32_t e0 = (w[0][cc >> 1] >> sh) & 0xffffu;
        const uint32_t e1 = (w[1][cc >> 1] >> sh) & 0xffffu;
        const uint32_t e2 = (w[2][cc >> 1] >> sh) & 0xffffu;
        const uint32_t e3 = (w[3][cc >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(&tileT[8 * ch + cc][4 * rq]) =
            make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
      }
    }
    __syncthreads();
    const int col = t >> 2, q = t & 3;
    const int64_t c = c0 + col;
    const uint4* lp = reinterpret_cast<const uint4*>(&tileT[col][32 * q]);
    uint32_t x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = lp[i];
      x[4 * i] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
    }
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      a = umax(a, umax(x[i] & 0x7fffu, (x[i] >> 16) & 0x7fffu));
    const int s = e8m0_exp_from_bf16_amax(a);
    const float sc = mx_scale_f32(s);
    uint32_t o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = e4m3x4_hw(x[2 * d], x[2 * d + 1], sc);
    if (c < cols) {
      const int64_t orow = b * cols + c;   // output row
      uint4* dst = reinterpret_cast<uint4*>(codes + orow * ld_out + out0 + 32 * q);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
      const int64_t kb = out0 / 32 + q;
      if (TILED)
        scales[mx_tile_off((uint32_t)orow, (uint32_t)kb,
                           (uint32_t)(ld_out / 128))] = (uint8_t)(s + 127);
      else
        scales[orow * (ld_out / 32) + kb] = (uint8_t)(s + 127);
    }
  }
  if constexpr (ROWS) {
    // thread t: row t % 128, group g = t / 128 of four 32-value blocks
    // (NCB = 4: two groups)
    static_assert(NCB == 4, "two groups of four blocks per row");
    __syncthreads();
    const int lr = t & 127, g = t >> 7;
    const int64_t r = r0 + lr;
    const int64_t kb0 = (int64_t)blockIdx.y * NCB * 2 + 4 * g;   // first block
    if (r < rend && 32 * kb0 < cols) {
      const int64_t orow = b * rows + r;
      const uint32_t wd = *reinterpret_cast<const uint32_t*>(&rsc[lr][4 * g]);
      *reinterpret_cast<uint32_t*>(
          row_scales + mx_tile_off((uint32_t)orow, (uint32_t)kb0,
                                   (uint32_t)(cols / 128))) = wd;
    }
  }
}

// Row-major scales [rows][4 nks] -> the GEMM layout; one thread per row and
// K step (a dword), consecutive threads write consecutive dwords.
__global__ __launch_bounds__(256) void mx_retile_kernel(
    const uint32_t* __restrict__ src, int64_t rows, uint32_t nks,
    uint32_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rb = i / (32 * (int64_t)nks);
  const uint32_t rem = (uint32_t)(i - rb * 32 * (int64_t)nks);
  const uint32_t st = rem / 32, rr = rem % 32;
  const int64_t r = rb * 32 + rr;
  if (r >= rows) return;
  dst[i] = src[r * nks + st];
}

}  // namespace

hipError_t launch_mx_quant_rows(const void* src, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales,
                                hipStream_t stream, bool tiled) {
  const int64_t n_chunks = rows * cols / 8;
  if (n_chunks == 0) return hipSuccess;
  int64_t blocks = (n_chunks + 256 * kRowsUnroll - 1) / (256 * kRowsUnroll);
  if (blocks > 65536) blocks = 65536;
  if (n_chunks / 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const uint32_t nks = (uint32_t)(cols / 128);
  KernelScope ks("mxfp8_quantize_rows", stream);
  if (tiled) {
    // cols is a multiple of 128 (whole K steps); scales 4-byte aligned
    if (cols % 128 != 0 || reinterpret_cast<uintptr_t>(scales) % 4 != 0)
      return hipErrorInvalidValue;
    const int cols8 = (int)(cols / 8);
    const int nwin = (cols8 + kTiledWin - 1) / kTiledWin;
    const int64_t nblk = (rows + 31) / 32 * nwin;
    if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx_rows_tiled_kernel, dim3((unsigned)nblk), dim3(256),
                       0, stream, static_cast<const uint4*>(src), rows, cols8,
                       nwin, nks, reinterpret_cast<uint2*>(codes),
                       reinterpret_cast<uint32_t*>(scales));
  } else {
    hipLaunchKernelGGL(mx_rows_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       stream, static_cast<const uint4*>(src), n_chunks,
                       reinterpret_cast<uint2*>(codes), scales);
  }
  return hipGetLastError();
}

hipError_t launch_mx_quant_cols(const void* src, int64_t batch, int64_t rows,
                                int64_t cols, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream, bool tiled) {
  if (batch * rows * cols == 0) return hipSuccess;
  KernelScope ks("mxfp8_quantize_cols", stream);
  if (rows % 128 == 0) {
    const dim3 g128((unsigned)(rows / 128), (unsigned)((cols + 63) / 64),
                    (unsigned)batch);
    if (tiled)
      hipLaunchKernelGGL((mx_cols128_kernel<false, true>), g128, dim3(256), 0,
                         stream, static_cast<const uint4*>(src), rows, cols,
                         (const int32_t*)nullptr, 0, 1, rows, codes, scales,
                       nullptr);
    else
      hipLaunchKernelGGL((mx_cols128_kernel<false, false>), g128, dim3(256),
                         0, stream, static_cast<const uint4*>(src), rows,
                         cols, (const int32_t*)nullptr, 0, 1, rows, codes,
                         scales, nullptr);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(rows / 32), (unsigned)((cols + 63) / 64),
                  (unsigned)batch);
  if (tiled)
    hipLaunchKernelGGL((mx_cols_kernel<false, true>), grid, dim3(256), 0,
                       stream, static_cast<const uint16_t*>(src), rows, cols,
                       (const int32_t*)nullptr, 0, 1, rows, codes, scales,
                       nullptr);
  else
    hipLaunchKernelGGL((mx_cols_kernel<false, false>), grid, dim3(256), 0,
                       stream, static_cast<const uint16_t*>(src), rows, cols,
                       (const int32_t*)nullptr, 0, 1, rows, codes, scales,
                       nullptr);
  return hipGetLastError();
}

hipError_t launch_mx_quant_segments(const void* src, int64_t rows,
                                    int64_t cols, const int32_t* seg_offsets,
                                    int n_seg, int pad, int64_t ld,
                                    uint8_t* codes, uint8_t* scales,
                                    int32_t* status, hipStream_t stream,
                                    bool tiled, uint8_t* row_codes,
                                    uint8_t* row_scales) {
  if (rows * cols == 0) return hipSuccess;
  if (row_codes && (pad % 128 != 0 || !tiled || cols % 128 != 0))
    return hipErrorInvalidValue;
  KernelScope ks(row_codes ? "mxfp8_quantize_segments_and_rows"
                           : "mxfp8_quantize_segments",
                 stream);
  if (pad % 128 == 0) {
    const int pt = pad / 128;
    // sum_s ceil(n_s / pad) * pad / 128 <= rows / 128 + n_seg * pad / 128
    const int64_t tiles = rows / 128 + (int64_t)n_seg * pt;
    constexpr int kNcb = 4;
    const dim3 g128((unsigned)tiles, (unsigned)((cols + 64 * kNcb - 1) /
                                                (64 * kNcb)), 1);
    if (row_codes)
      hipLaunchKernelGGL((mx_cols128_kernel<true, true, kNcb, true>), g128,
                         dim3(256), 0, stream,
                         static_cast<const uint4*>(src), rows, cols,
                         seg_offsets, n_seg, pt, ld, codes, scales, status,
                         reinterpret_cast<uint2*>(row_codes), row_scales);
    else if (tiled)
      hipLaunchKernelGGL((mx_cols128_kernel<true, true, kNcb>), g128,
                         dim3(256), 0, stream,
                         static_cast<const uint4*>(src), rows, cols,
                         seg_offsets, n_seg, pt, ld, codes, scales, status);
    else
      hipLaunchKernelGGL((mx_cols128_kernel<true, false, kNcb>), g128,
                         dim3(256), 0, stream,
                         static_cast<const uint4*>(src), rows, cols,
                         seg_offsets, n_seg, pt, ld, codes, scales, status);
    return hipGetLastError();
  }
  const int pad_tiles = pad / 32;
  // sum_s ceil(n_s / pad) * pad / 32 <= rows / 32 + n_seg * pad / 32
  const int64_t tiles = rows / 32 + (int64_t)n_seg * pad_tiles;
  const dim3 grid((unsigned)tiles, (unsigned)((cols + 63) / 64), 1);
  if (tiled)
    hipLaunchKernelGGL((mx_cols_kernel<true, true>), grid, dim3(256), 0,
                       stream, static_cast<const uint16_t*>(src), rows, cols,
                       seg_offsets, n_seg, pad_tiles, ld, codes, scales,
                       status);
  else
    hipLaunchKernelGGL((mx_cols_kernel<true, false>), grid, dim3(256), 0,
                       stream, static_cast<const uint16_t*>(src), rows, cols,
                       seg_offsets, n_seg, pad_tiles, ld, codes, scales,
                       status);
  return hipGetLastError();
}

namespace {
// Row-wise MXFP8 of float32 values, a quad of lanes per block of 32 (lane l
// holds values 8 l .. 8 l + 7 of the flat array): the encoder the MXFP8
// gate/up epilogue runs on its float32 ScaledSwiGLU outputs.
__global__ __launch_bounds__(256) void mx_f32_kernel(
    const float4* __restrict__ src, int64_t n8, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // n8 is a multiple of 4, so a quad is either wholly in range or wholly out
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += stride) {
    const float4 a = src[2 * i], b = src[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    int sx;
    codes[i] = mx_quad_encode_f32(v, &sx);
    if ((i & 3) == 0) scales[i >> 2] = (uint8_t)(sx + 127);
  }
}
}  // namespace

hipError_t launch_mx_quant_f32(const float* src, int64_t n, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  KernelScope ks("mxfp8_quantize_f32", stream);
  const int64_t n8 = n / 8;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 65536);
  hipLaunchKernelGGL(mx_f32_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     stream, reinterpret_cast<const float4*>(src), n8,
                     reinterpret_cast<uint2*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_mx_scales_retile(const uint8_t* src, int64_t rows,
                                   int64_t k, uint8_t* dst,
                                   hipStream_t stream) {
  const uint32_t nks = (uint32_t)(k / 128);
  const int64_t n = (rows + 31) / 32 * 32 * nks;   // dwords
  if (n == 0) return hipSuccess;
  KernelScope ks("mxfp8_scales_retile", stream);
  hipLaunchKernelGGL(mx_retile_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(src), rows, nks,
                     reinterpret_cast<uint32_t*>(dst));
  return hipGetLastError();
}

}  // namespace moe
