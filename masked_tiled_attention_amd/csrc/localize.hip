// Mask localization for one context-parallel rank.
//
// "FlashMask-3" page (iitog.ru), contributions paragraph and "Key facts": the
// mask is indexed by key position but stores query-axis bounds, so when a
// rank holds several fragments of the context its local mask is obtained by
// clip, shift and max on the bound vectors, without communication. Here, for
// chunk c = [s_c, s_c + len_c) at local offset off_c (chunks ascending):
//   x  = clamp(bound, 0, Sq_glob)                  (clip to the query axis)
//   t_c = min(x - s_c + off_c, off_c + len_c)      (shift into chunk c, clip at its end)
//   x' = max(0, max_c t_c)                         (max over chunks, clip at 0)
// which counts the local rows below the bound. Pure int32; one thread per
// (bm, hm, key column), handling all four vectors.
#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {
namespace {

__device__ __forceinline__ int32_t localize_one(const LocalizeArgs& a, int32_t v) {
  const int32_t x = min(max(v, 0), a.seq_q_global);
  int32_t best = 0;
  for (int c = 0; c < a.num_chunks; ++c) {
    const int32_t t = min(x - a.chunk_start[c] + a.chunk_off[c], a.chunk_off[c] + a.chunk_len[c]);
    best = max(best, t);
  }
  return best;
}

__global__ __launch_bounds__(256) void localize_kernel(LocalizeArgs a) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= a.seq_k) return;
  const int bh = blockIdx.y;
  const int bm = bh / a.mask.hm, hm = bh % a.mask.hm;
  const int64_t in = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h + j;
  const int64_t out = (int64_t)bh * a.seq_k + j;
  if (a.mask.has_lower) {
    a.out[0][out] = localize_one(a, a.mask.lts[in]);
    a.out[1][out] = localize_one(a, a.mask.lte[in]);
  }
  if (a.mask.has_upper) {
    a.out[2][out] = localize_one(a, a.mask.uts[in]);
    a.out[3][out] = localize_one(a, a.mask.ute[in]);
  }
}

// Mask-pruned K/V transfer set of one rank. Same page, contributions
// paragraph and "Key facts": the overlap of computation with communication
// drops the transfers that the mask makes useless. With the rank's (localized)
// vectors, key j is needed when some row of [0, Sq) escapes both of its
// intervals. The first open row is found by stepping from row 0 past an
// interval that contains it; two passes over the two intervals suffice (once
// the row has stepped past an interval it never re-enters it). A key tile is
// needed when any of its keys is. Pure int32, exact for any bound values.
__device__ __forceinline__ bool key_needed(int32_t n, int32_t a0, int32_t a1, int32_t b0, int32_t b1) {
  int32_t r = 0;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (a0 <= r && r < a1) r = a1;
    if (b0 <= r && r < b1) r = b1;
  }
  return r < n;
}

// grid (key tiles, bm * hm): one flag per key tile
__global__ __launch_bounds__(256) void transfer_set_kernel(TransferArgs a) {
  const int bh = blockIdx.y;
  const int bm = bh / a.mask.hm, hm = bh % a.mask.hm;
  const int64_t base = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const int64_t j0 = (int64_t)blockIdx.x * a.block_k;
  const int64_t j1 = min(j0 + a.block_k, (int64_t)a.seq_k);
  bool any = false;
  for (int64_t j = j0 + threadIdx.x; j < j1 && !any; j += 256) {
    const int32_t a0 = a.mask.has_lower ? a.mask.lts[base + j] : 0;
    const int32_t a1 = a.mask.has_lower ? a.mask.lte[base + j] : 0;
    const int32_t b0 = a.mask.has_upper ? a.mask.uts[base + j] : 0;
    const int32_t b1 = a.mask.has_upper ? a.mask.ute[base + j] : 0;
    any = key_needed(a.seq_q, a0, a1, b0, b1);
  }
  any = __syncthreads_or(any);
  if (threadIdx.x == 0) a.need[(int64_t)bh * a.tk + blockIdx.x] = any ? 1 : 0;
}

// grid (bm * hm): number of needed tiles per mask row
__global__ __launch_bounds__(256) void transfer_count_kernel(TransferArgs a) {
  const uint8_t* row = a.need + (int64_t)blockIdx.x * a.tk;
  int c = 0;
  for (int t = threadIdx.x; t < a.tk; t += 256) c += row[t];
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  __shared__ int red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) a.count[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// Open (row, key) pairs per chunk of the global query axis, the work that a
// sparsity-aware chunk -> rank assignment balances (same page: the HCC-IPO
// balancer is named, nothing more). For key j, the masked rows are the union
// of its two intervals A and B, so within chunk [s, e) it hides
// |A n [s,e)| + |B n [s,e)| - |A n B n [s,e)| rows; the rest are open.
// Workgroups take kWorkKeys keys of one mask row each and add their int64
// sums into the (zeroed) output with atomics: exact for any bounds, and the
// integer sums do not depend on the order.
constexpr int kWorkThreads = 256;
constexpr int kWorkKeys = 4096;
constexpr int kWorkChunks = 8;

__device__ __forceinline__ int64_t overlap(int64_t a, int64_t b, int64_t s, int64_t e) {
  return max((int64_t)0, min(b, e) - max(a, s));
}

__global__ __launch_bounds__(256) void chunk_work_zero_kernel(ChunkWorkArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (int64_t)a.mask.bm * a.mask.hm * a.num_chunks) a.work[i] = 0;
}

// grid (key blocks, bm * hm)
__global__ __launch_bounds__(kWorkThreads) void chunk_work_kernel(ChunkWorkArgs a) {
  const int mr = blockIdx.y;
  const int bm = mr / a.mask.hm, hm = mr % a.mask.hm;
  const int64_t base = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const int j0 = blockIdx.x * kWorkKeys, j1 = min(j0 + kWorkKeys, a.seq_k);
  __shared__ int64_t red[kWorkThreads / 64][kWorkChunks];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int c0 = 0; c0 < a.num_chunks; c0 += kWorkChunks) {
    int64_t acc[kWorkChunks];
#pragma unroll
    for (int k = 0; k < kWorkChunks; ++k) acc[k] = 0;
    for (int j = j0 + threadIdx.x; j < j1; j += kWorkThreads) {
      const int64_t a0 = a.mask.has_lower ? a.mask.lts[base + j] : 0;
      const int64_t a1 = a.mask.has_lower ? a.mask.lte[base + j] : 0;
      const int64_t b0 = a.mask.has_upper ? a.mask.uts[base + j] : 0;
      const int64_t b1 = a.mask.has_upper ? a.mask.ute[base + j] : 0;
      const int64_t i0 = max(a0, b0), i1 = min(a1, b1);   // A n B
#pragma unroll
      for (int k = 0; k < kWorkChunks; ++k) {
        if (c0 + k < a.num_chunks) {
          const int64_t s = a.chunk_start[c0 + k], e = s + a.chunk_len[c0 + k];
          acc[k] += (e - s) - overlap(a0, a1, s, e) - overlap(b0, b1, s, e) + overlap(i0, i1, s, e);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kWorkChunks; ++k) {
      int64_t v = acc[k];
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0) red[wv][k] = v;
    }
    __syncthreads();
    if (threadIdx.x < kWorkChunks && c0 + (int)threadIdx.x < a.num_chunks) {
      int64_t t = 0;
      for (int w = 0; w < kWorkThreads / 64; ++w) t += red[w][threadIdx.x];
      atomicAdd(reinterpret_cast<unsigned long long*>(a.work + (int64_t)mr * a.num_chunks + c0 + threadIdx.x),
                (unsigned long long)t);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_chunk_work(const ChunkWorkArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.mask.bm * a.mask.hm * a.num_chunks;
  hipLaunchKernelGGL(chunk_work_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_work_kernel, dim3((a.seq_k + kWorkKeys - 1) / kWorkKeys, a.mask.bm * a.mask.hm),
                     dim3(kWorkThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_transfer_set(const TransferArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(transfer_set_kernel, dim3(a.tk, a.mask.bm * a.mask.hm), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.count) return e;
  hipLaunchKernelGGL(transfer_count_kernel, dim3(a.mask.bm * a.mask.hm), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_localize(const LocalizeArgs& a, hipStream_t stream) {
  dim3 grid((a.seq_k + 255) / 256, a.mask.bm * a.mask.hm);
  hipLaunchKernelGGL(localize_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fm
