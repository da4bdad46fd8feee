// Expert-order permutation, row gather, combine.
//
// The grouped GEMM needs every expert's tokens contiguous plus the
// per-expert counts split_sizes ("NVIDIA presents an efficient path for
// training biological MoE models", section "Grouped experts instead of a
// Python loop"; "Efficient MoE training for biological foundation models
// (NVIDIA)", section "1) Fragmented expert kernels").  The combine sums each
// token's k expert outputs back in token order.
//
// Index build (deterministic, no order-dependent atomics):
//   1. count:  each block histograms a chunk of pairs per expert -> cnt[b][e]
//   2. scan:   per expert, exclusive scan of cnt over blocks (in place);
//              split_sizes, offsets = exclusive scan over experts
//   3. rank:   each block re-walks its chunk in order, one wave, 64 pairs at a
//              time; the rank of a pair among equal experts inside the wave
//              comes from ballots; running per-expert counters sit in LDS.
//              row = offsets[e] + cnt[b][e] + running + rank.
// Row copy: one block per token reads x[t] once and writes it to its k
// destination rows (16-byte vectors); optional row-wise MXFP8 quantisation on
// the way.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "timer.hpp"

namespace moe {

namespace {

constexpr int kChunk = 1024;  // pairs per block in the index build

__global__ __launch_bounds__(256) void perm_count_kernel(
    const int32_t* __restrict__ topk_idx, int64_t n_pairs, int E,
    int32_t* __restrict__ cnt, int32_t* status) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
    const int64_t p = base + i;
    if (p < n_pairs) {
      const int e = topk_idx[p];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
      else report_error(status, 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    cnt[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One block of 1024 threads.  cnt[b][e] becomes the exclusive prefix over
// blocks; split_sizes / offsets from the column totals.  Threads form
// G = 1024 / E' groups (E' = E rounded up to a power of two); group g owns a
// contiguous range of blocks, so each thread walks nblk / G blocks.
__global__ __launch_bounds__(1024) void perm_scan_kernel(
    int32_t* __restrict__ cnt, int nblk, int E, int32_t* __restrict__ split,
    int32_t* __restrict__ offsets) {
  __shared__ int32_t part[1024];
  __shared__ int32_t wsum[16];
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int G = 1024 / Ep;
  const int e = threadIdx.x % Ep, g = threadIdx.x / Ep;
  const int per = (nblk + G - 1) / G;
  const int b0 = g * per, b1 = min(nblk, b0 + per);
  // phase 1: range sums
  int32_t s = 0;
  if (e < E) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int32_t c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = cnt[(int64_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += c[i];
    }
    for (; b < b1; ++b) s += cnt[(int64_t)b * E + e];
  }
  part[threadIdx.x] = s;
  __syncthreads();
  // phase 2: prefix over groups for this expert, total per expert
  int32_t pre = 0, tot = 0;
  for (int gg = 0; gg < G; ++gg) {
    const int32_t v = part[gg * Ep + e];
    if (gg < g) pre += v;
    tot += v;
  }
  // phase 3: rewrite the range as exclusive prefixes
  if (e < E) {
    int32_t run = pre;
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      int32_t c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = cnt[(int64_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        cnt[(int64_t)(b + i) * E + e] = run;
        run += c[i];
      }
    }
    for (; b < b1; ++b) {
      const int32_t c = cnt[(int64_t)b * E + e];
      cnt[(int64_t)b * E + e] = run;
      run += c;
    }
    if (g == 0) split[e] = tot;
  }
  __syncthreads();
  // exclusive scan of the per-expert totals over e (threads 0..E-1 of group 0
  // hold e = threadIdx.x when g == 0)
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int32_t v = (g == 0 && e < E) ? tot : 0;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int w = 0; w < 16; ++w) {
      const int32_t t = wsum[w];
      wsum[w] = acc;
      acc += t;
    }
  }
  __syncthreads();
  const int32_t excl = incl - v + wsum[wid];
  if (g == 0 && e < E) {
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + v;
  }
}

// One wave per block walks its chunk in order.
__global__ __launch_bounds__(64) void perm_rank_kernel(
    const int32_t* __restrict__ topk_idx, int64_t n_pairs, int E,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_map, int32_t* __restrict__ src_row) {
  extern __shared__ int32_t run[];  // [E] running count inside this chunk
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64)
    run[e] = offsets[e] + cnt[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  // every expert id of the chunk is loaded up front (the loop's barriers
  // would otherwise hold each load's latency)
  constexpr int kPer = kChunk / 64;
  int ev[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t p = base + 64 * u + lane;
    ev[u] = p < n_pairs ? topk_idx[p] : -1;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t p = base + 64 * u + lane;
    const int e = ev[u];
    const bool ok = (unsigned)e < (unsigned)E;
    // lanes holding the same expert id: intersect ballots bit by bit
    uint64_t same = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bal = __ballot(ok && ((e >> b) & 1));
      same &= ((e >> b) & 1) ? bal : ~bal;
    }
    int rank = 0, basev = 0;
    if (ok) {
      rank = __popcll(same & lt_mask);
      basev = run[e];
    }
    // the block is one wave, whose LDS accesses complete in program order:
    // the compiler barriers keep that order (a block barrier would also
    // wait for the previous pairs' global stores)
    asm volatile("" ::: "memory");
    // the highest lane of each group advances the running counter
    if (ok && (same >> lane) == 1ull) run[e] = basev + rank + 1;
    asm volatile("" ::: "memory");
    if (p < n_pairs) {
      if (ok) {
        const int32_t r = basev + rank;
        row_map[p] = r;
        src_row[r] = (int32_t)p;
      } else {
        row_map[p] = -1;
      }
    }
  }
}

// Row kernels below: one block per token; every thread issues the loads of
// all its 16-byte chunks of the row (kRowU per pass) before the first use,
// and the row_map read overlaps them.
constexpr int kRowU = 4;

// bf16 row copy: x[t] -> x_perm[row_map[t*k+j]] for j < k.
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ row_map,
    const float* __restrict__ topk_w, int64_t T, int H8, int k,
    uint4* __restrict__ x_perm, float* __restrict__ w_perm) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t rows[64];
  const uint4* src = x + t * (int64_t)H8;
  for (int c0 = 0; c0 < H8; c0 += 256 * kRowU) {
    uint4 v[kRowU];
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int c = c0 + 256 * u + threadIdx.x;
      v[u] = c < H8 ? ld_nt(src + c) : make_uint4(0, 0, 0, 0);
    }
    if (c0 == 0) {
      if (threadIdx.x < k) {
        const int32_t r = row_map[t * k + threadIdx.x];
        rows[threadIdx.x] = r;
        if (w_perm && r >= 0) w_perm[r] = topk_w[t * k + threadIdx.x];
      }
      __syncthreads();
    }
    for (int j = 0; j < k; ++j) {
      const int32_t r = rows[j];
      if (r < 0) continue;
      uint4* dst = x_perm + (int64_t)r * H8;
#pragma unroll
      for (int u = 0; u < kRowU; ++u) {
        const int c = c0 + 256 * u + threadIdx.x;
        if (c < H8) st_nt(dst + c, v[u]);
      }
    }
  }
}

// Row copy with row-wise MXFP8 quantisation: 4 lanes per block of 32 bf16
// (64 bytes); block amax via two lane shuffles.
__global__ __launch_bounds__(256) void gather_rows_mx_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ row_map,
    const float* __restrict__ topk_w, int64_t T, int H, int k,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ w_perm) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t rows[64];
  const int H8 = H >> 3;
  const uint4* src = x + t * (int64_t)H8;
  // H8 is a multiple of 4, so the 4 lanes of a block stay in one pass
  for (int c0 = 0; c0 < H8; c0 += 256 * kRowU) {
    uint4 v[kRowU];
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int c = c0 + 256 * u + threadIdx.x;
      v[u] = c < H8 ? ld_nt(src + c) : make_uint4(0, 0, 0, 0);
    }
    if (c0 == 0) {
      if (threadIdx.x < k) {
        const int32_t r = row_map[t * k + threadIdx.x];
        rows[threadIdx.x] = r;
        if (w_perm && r >= 0) w_perm[r] = topk_w[t * k + threadIdx.x];
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < kRowU; ++u) {
      const int c = c0 + 256 * u + threadIdx.x;
      if (c0 + 256 * u >= H8) break;   // uniform: the pass ends here
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
        amax = amax > lo ? amax : lo;
        amax = amax > hi ? amax : hi;
      }
      uint32_t o = __shfl_xor(amax, 1, 64);
      amax = amax > o ? amax : o;
      o = __shfl_xor(amax, 2, 64);
      amax = amax > o ? amax : o;
      const int s = e8m0_exp_from_bf16_amax(amax);
      const uint2 qq = e4m3x8_hw(v[u], s);
      if (c < H8) {
        for (int j = 0; j < k; ++j) {
          const int32_t r = rows[j];
          if (r < 0) continue;
          reinterpret_cast<uint2*>(codes + (int64_t)r * H)[c] = qq;
          if ((c & 3) == 0)
            scales[(int64_t)r * (H >> 5) + (c >> 2)] = (uint8_t)(s + 127);
        }
      }
    }
  }
}

// The MXFP8 row copy for rows of at most 256 U chunks, TPB tokens per
// block (all loads issued before the row_map reads and the stores): codes
// leave as streaming 8-byte stores, and with sc4 (H % 128 == 0 and 4-byte aligned scales: a 16-lane
// group's four blocks sit in one aligned word of its row) the lane at the
// head of 16 gathers their scale bytes (three lane reads) for one 4-byte
// store.
template <int TPB, int U>
__global__ __launch_bounds__(256) void gather_rows_mx_multi_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ row_map,
    const float* __restrict__ topk_w, int64_t T, int H, int k,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ w_perm, bool sc4) {
  const int64_t t0 = (int64_t)blockIdx.x * TPB;
  __shared__ int32_t rows[TPB * 32];   // k <= 32
  const int H8 = H >> 3;
  uint4 v[TPB][U];
#pragma unroll
  for (int tk = 0; tk < TPB; ++tk)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = 256 * u + threadIdx.x;
      const int64_t t = t0 + tk;
      v[tk][u] = (t < T && c < H8) ? ld_nt(x + t * H8 + c)
                                   : make_uint4(0, 0, 0, 0);
    }
  if (threadIdx.x < TPB * k) {
    const int tk = threadIdx.x / k, j = threadIdx.x - tk * k;
    const int64_t t = t0 + tk;
    int32_t r = -1;
    if (t < T) {
      r = row_map[t * k + j];
      if (w_perm && r >= 0) w_perm[r] = topk_w[t * k + j];
    }
    rows[threadIdx.x] = r;
  }
  const int lane = threadIdx.x & 63;
  __syncthreads();
#pragma unroll
  for (int tk = 0; tk < TPB; ++tk)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = 256 * u + threadIdx.x;
      // every lane takes part in the shuffles (zeros past the row)
      const uint32_t w[4] = {v[tk][u].x, v[tk][u].y, v[tk][u].z, v[tk][u].w};
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
        amax = amax > lo ? amax : lo;
        amax = amax > hi ? amax : hi;
      }
      uint32_t o = __shfl_xor(amax, 1, 64);
      amax = amax > o ? amax : o;
      o = __shfl_xor(amax, 2, 64);
      amax = amax > o ? amax : o;
      const int s = e8m0_exp_from_bf16_amax(amax);
      const uint2 qq = e4m3x8_hw(v[tk][u], s);
      const uint32_t sb = (uint32_t)(s + 127);
      // scale bytes of the 16-lane group's four blocks, low byte first
      const uint32_t s4 = sb | (__shfl(sb, lane + 4, 64) << 8) |
                          (__shfl(sb, lane + 8, 64) << 16) |
                          (__shfl(sb, lane + 12, 64) << 24);
      if (c >= H8) continue;
      for (int j = 0; j < k; ++j) {
        const int32_t r = rows[tk * k + j];
        if (r < 0) continue;
        u32x2_t q2 = {qq.x, qq.y};
        __builtin_nontemporal_store(
            q2, reinterpret_cast<u32x2_t*>(codes + (int64_t)r * H) + c);
        uint8_t* srow = scales + (int64_t)r * (H >> 5);
        if (sc4) {
          if ((c & 15) == 0)
            *reinterpret_cast<uint32_t*>(srow + (c >> 2)) = s4;
        } else if ((c & 3) == 0) {
          srow[c >> 2] = (uint8_t)sb;
        }
      }
    }
}

// y[t] = sum_j c_j * z[row_map[t*k+j]] in float32, ascending j; the rows of
// up to kUnpJ slots are loaded before they are added.
constexpr int kUnpU = 2, kUnpJ = 4;

__global__ __launch_bounds__(256) void unpermute_kernel(
    const uint4* __restrict__ z, const int32_t* __restrict__ row_map,
    const float* __restrict__ topk_w, int64_t T, int H8, int k,
    uint4* __restrict__ y) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t rows[64];
  __shared__ float cw[64];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_map[t * k + threadIdx.x];
    cw[threadIdx.x] = topk_w ? topk_w[t * k + threadIdx.x] : 1.0f;
  }
  __syncthreads();
  for (int c0 = 0; c0 < H8; c0 += 256 * kUnpU) {
    float acc[kUnpU][8];
#pragma unroll
    for (int u = 0; u < kUnpU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kUnpJ) {
      uint4 v[kUnpJ][kUnpU];
#pragma unroll
      for (int jj = 0; jj < kUnpJ; ++jj) {
        const int j = j0 + jj;
        const int32_t r = j < k ? rows[j] : -1;
#pragma unroll
        for (int u = 0; u < kUnpU; ++u) {
          const int c = c0 + 256 * u + threadIdx.x;
          v[jj][u] = (r >= 0 && c < H8) ? ld_nt(z + (int64_t)r * H8 + c)
                                        : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kUnpJ; ++jj) {
        const int j = j0 + jj;
        if (j >= k || rows[j] < 0) continue;   // uniform over the block
        const float cj = cw[j];
#pragma unroll
        for (int u = 0; u < kUnpU; ++u) {
          const uint32_t w[4] = {v[jj][u].x, v[jj][u].y, v[jj][u].z,
                                 v[jj][u].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[u][2 * i] += cj * bf16lo(w[i]);
            acc[u][2 * i + 1] += cj * bf16hi(w[i]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnpU; ++u) {
      const int c = c0 + 256 * u + threadIdx.x;
      if (c >= H8) continue;
      uint4 o;
      o.x = pack_bf16x2(acc[u][0], acc[u][1]);
      o.y = pack_bf16x2(acc[u][2], acc[u][3]);
      o.z = pack_bf16x2(acc[u][4], acc[u][5]);
      o.w = pack_bf16x2(acc[u][6], acc[u][7]);
      st_nt(y + t * (int64_t)H8 + c, o);
    }
  }
}

__global__ __launch_bounds__(256) void probs_grad_kernel(
    const float* __restrict__ dw_perm, const int32_t* __restrict__ row_map,
    int64_t n, float* __restrict__ dprobs) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p < n) {
    const int32_t r = row_map[p];
    dprobs[p] = r >= 0 ? dw_perm[r] : 0.0f;
  }
}

}  // namespace

namespace {
// Scratch of moe_permute_noalloc: the per-block expert histograms of the
// index build (what moe_permute keeps in its workspace), in a static device
// array, so that the call allocates nothing.  Every GPU holds its own copy,
// at its own address, for the life of the process; host code reaches it
// only through the address hipGetSymbolAddress returns for the current
// device (the array's name is a host-side stand-in).
constexpr size_t kPermScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) int32_t scratch[kPermScratchBytes /
                                                 sizeof(int32_t)];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t permute_scratch_bytes() { return kPermScratchBytes; }

hipError_t permute_scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

size_t permute_ws_bytes(int64_t T, int E, int k) {
  const int64_t n = T * (int64_t)k;
  const int64_t nblk = (n + kChunk - 1) / kChunk;
  return (size_t)(nblk > 0 ? nblk : 1) * (size_t)E * sizeof(int32_t);
}

hipError_t launch_permute_index(const int32_t* topk_idx, int64_t T, int E,
                                int k, int32_t* row_map, int32_t* src_row,
                                int32_t* split, int32_t* offsets, void* ws,
                                int32_t* status, hipStream_t stream) {
  const int64_t n = T * (int64_t)k;
  const int nblk = (int)((n + kChunk - 1) / kChunk);
  int32_t* cnt = static_cast<int32_t*>(ws);
  KernelScope ks("permute_index", stream);
  if (nblk > 0)
    hipLaunchKernelGGL(perm_count_kernel, dim3(nblk), dim3(256),
                       E * sizeof(int32_t), stream, topk_idx, n, E, cnt, status);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, stream, cnt,
                     nblk, E, split, offsets);
  if (nblk > 0)
    hipLaunchKernelGGL(perm_rank_kernel, dim3(nblk), dim3(64),
                       E * sizeof(int32_t), stream, topk_idx, n, E, cnt,
                       offsets, row_map, src_row);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_map,
                              const float* topk_w, int64_t T, int H, int k,
                              void* x_perm, float* w_perm, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  KernelScope ks("permute_gather", stream);
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)T), dim3(256), 0,
                     stream, static_cast<const uint4*>(x), row_map, topk_w, T,
                     H / 8, k, static_cast<uint4*>(x_perm), w_perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows_mx(const void* x, const int32_t* row_map,
                                 const float* topk_w, int64_t T, int H, int k,
                                 uint8_t* codes, uint8_t* scales,
                                 float* w_perm, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  KernelScope ks("permute_gather_mxfp8", stream);
  const int H8 = H / 8;
  const uint4* xs = static_cast<const uint4*>(x);
  const bool sc4 = (H % 128) == 0 &&
                   (reinterpret_cast<uintptr_t>(scales) & 3u) == 0;
  // Mixtral shapes (H = 4096, k = 2): two tokens per block, 4.38 -> 4.77
  // TB/s with the streaming code and word scale stores (caches flushed).
  // bf16 rows of 2048 values to k = 8 rows copied four tokens per block ran
  // slower than one per block (4.88 vs 5.25 TB/s): one token per block there.
  if (H8 <= 256)
    hipLaunchKernelGGL((gather_rows_mx_multi_kernel<1, 1>), dim3((unsigned)T),
                       dim3(256), 0, stream, xs, row_map, topk_w, T, H, k,
                       codes, scales, w_perm, sc4);
  else if (H8 <= 512)
    hipLaunchKernelGGL((gather_rows_mx_multi_kernel<2, 2>),
                       dim3((unsigned)((T + 1) / 2)), dim3(256), 0, stream, xs,
                       row_map, topk_w, T, H, k, codes, scales, w_perm, sc4);
  else
    hipLaunchKernelGGL(gather_rows_mx_kernel, dim3((unsigned)T), dim3(256), 0,
                       stream, xs, row_map, topk_w, T, H, k, codes, scales,
                       w_perm);
  return hipGetLastError();
}

hipError_t launch_unpermute(const void* z, const int32_t* row_map,
                            const float* topk_w, int64_t T, int H, int k,
                            void* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  KernelScope ks("unpermute", stream);
  hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)T), dim3(256), 0, stream,
                     static_cast<const uint4*>(z), row_map, topk_w, T, H / 8,
                     k, static_cast<uint4*>(y));
  return hipGetLastError();
}

hipError_t launch_probs_grad(const float* dw_perm, const int32_t* row_map,
                             int64_t T, int k, float* dprobs,
                             hipStream_t stream) {
  const int64_t n = T * (int64_t)k;
  if (n == 0) return hipSuccess;
  KernelScope ks("probs_grad", stream);
  hipLaunchKernelGGL(probs_grad_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream, dw_perm, row_map, n, dprobs);
  return hipGetLastError();
}

}  // namespace moe
