// Tile classification pre-pass.
//
// The pages do not describe a tile pre-pass; its rule is the reading stated in
// fm_attn.h (fm_tile_classify). Two kernels:
//   summary: one workgroup per (bm, hm, key tile) reduces min / max of the four
//            bound vectors over the tile's columns -> 8 int32;
//   map:     one thread per (query tile, key tile) applies the rule to the
//            summary and writes one class byte, row-major in either order.
// Both are integer-only and bound by launch latency and HBM at these sizes.
#include <climits>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {
namespace {

constexpr int kSumThreads = 256;

__device__ __forceinline__ int wave_min(int x) {
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}

__global__ __launch_bounds__(kSumThreads) void classify_summary_kernel(ClassifyArgs a) {
  const int kt = blockIdx.x;
  const int bh = blockIdx.y;
  const int bm = bh / a.mask.hm, hm = bh % a.mask.hm;
  const int64_t base = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const int c0 = kt * a.block_k;
  const int c1 = min(c0 + a.block_k, a.seq_k);

  // lanes accumulate (min, max) of lts, lte, uts, ute
  int mn[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
  int mx[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
  for (int c = c0 + (int)threadIdx.x; c < c1; c += kSumThreads) {
    int v[4];
    if (a.mask.has_lower) {
      v[0] = a.mask.lts[base + c];
      v[1] = a.mask.lte[base + c];
    } else {
      v[0] = a.seq_q;
      v[1] = a.seq_q;
    }
    if (a.mask.has_upper) {
      v[2] = a.mask.uts[base + c];
      v[3] = a.mask.ute[base + c];
    } else {
      v[2] = 0;
      v[3] = 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mn[i] = min(mn[i], v[i]);
      mx[i] = max(mx[i], v[i]);
    }
  }
  __shared__ int red[kSumThreads / 64][8];
  const int w = threadIdx.x / 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int a0 = wave_min(mn[i]);
    int a1 = wave_max(mx[i]);
    if (lane_id() == 0) {
      red[w][2 * i] = a0;
      red[w][2 * i + 1] = a1;
    }
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int i = threadIdx.x;
    int r = red[0][i];
    for (int ww = 1; ww < kSumThreads / 64; ++ww) r = (i & 1) ? max(r, red[ww][i]) : min(r, red[ww][i]);
    a.summary[((int64_t)bh * a.tk + kt) * 8 + i] = r;
  }
}

__device__ __forceinline__ uint8_t classify_one(const int* s, int r0, int r1) {
  // s: min lts, max lts, min lte, max lte, min uts, max uts, min ute, max ute
  const bool covers_l = s[1] <= r0 && s[2] >= r1;
  const bool covers_u = s[5] <= r0 && s[6] >= r1;
  if (covers_l || covers_u) return (uint8_t)FM_TILE_SKIP;
  const bool misses_l = s[3] <= r0 || s[0] >= r1;
  const bool misses_u = s[7] <= r0 || s[4] >= r1;
  return (uint8_t)((misses_l && misses_u) ? FM_TILE_FULL : FM_TILE_PARTIAL);
}

// Not transposed: grid (ceil(tk/256), tq, bm*hm); thread -> key tile.
// Transposed:     grid (ceil(tq/256), tk, bm*hm); thread -> query tile.
__global__ __launch_bounds__(256) void classify_map_kernel(ClassifyArgs a) {
  const int bh = blockIdx.z;
  const int t = blockIdx.x * 256 + threadIdx.x;
  int qt, kt;
  if (a.transposed) {
    kt = blockIdx.y;
    qt = t;
    if (qt >= a.tq) return;
  } else {
    qt = blockIdx.y;
    kt = t;
    if (kt >= a.tk) return;
  }
  const int* sp = a.summary + ((int64_t)bh * a.tk + kt) * 8;
  int s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = sp[i];
  const int r0 = qt * a.block_q;
  const int r1 = min(r0 + a.block_q, a.seq_q);
  const uint8_t c = classify_one(s, r0, r1);
  if (a.transposed)
    a.classes[((int64_t)bh * a.tk + kt) * a.tq + qt] = c;
  else
    a.classes[((int64_t)bh * a.tq + qt) * a.tk + kt] = c;
}

// grid (rows): counts[r] = number of non-SKIP entries of class-map line r.
__global__ __launch_bounds__(256) void order_count_kernel(OrderArgs a) {
  const int r = blockIdx.x;
  const uint8_t* line = a.classes + (int64_t)(r / a.inner) * a.outer_stride + (int64_t)(r % a.inner) * a.line_stride;
  int c = 0;
  for (int gi = 0; gi < a.group; ++gi)
    for (int i = threadIdx.x; i < a.len; i += 256) c += line[gi * a.group_stride + i * a.elem_stride] != FM_TILE_SKIP;
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  __shared__ int red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) a.counts[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// One workgroup of 1024: counting sort of the rows by count, descending, with
// the counts grouped into at most 4096 buckets (order within a bucket is
// arbitrary; only the launch order depends on it).
constexpr int kOrderBuckets = 4096;
__global__ __launch_bounds__(1024) void order_sort_kernel(OrderArgs a) {
  __shared__ int hist[kOrderBuckets];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // a line counts up to len entries in each of its `group` class-map lines
  const int64_t cmax = (int64_t)a.len * a.group;
  const int nb = (int)min(cmax + 1, (int64_t)kOrderBuckets);
  auto key = [&](int r) {   // descending count -> ascending key in [0, nb)
    const int64_t c = min(max((int64_t)a.counts[r], (int64_t)0), cmax);
    return nb - 1 - (int)(c * nb / (cmax + 1));
  };
  for (int i = tid; i < nb; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int r = tid; r < a.rows; r += 1024) atomicAdd(&hist[key(r)], 1);
  __syncthreads();
  // exclusive scan: thread t owns buckets 4t .. 4t+3
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    v[i] = b < nb ? hist[b] : 0;
    s += v[i];
  }
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int pre = incl - s;
  for (int k = 0; k < wv; ++k) pre += wsum[k];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    if (b < nb) hist[b] = pre;
    pre += v[i];
  }
  __syncthreads();
  for (int r = tid; r < a.rows; r += 1024)
    a.order[atomicAdd(&hist[key(r)], 1)] = (int32_t)((uint32_t)r | (a.mark_empty && a.counts[r] <= 0 ? kEmptyLine : 0u));
}

}  // namespace

hipError_t launch_order(const OrderArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(order_count_kernel, dim3(a.rows), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(order_sort_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_classify_summary(const ClassifyArgs& a, hipStream_t stream) {
  dim3 grid(a.tk, a.mask.bm * a.mask.hm);
  hipLaunchKernelGGL(classify_summary_kernel, grid, dim3(kSumThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_classify_map(const ClassifyArgs& a, hipStream_t stream) {
  dim3 grid;
  if (a.transposed)
    grid = dim3((a.tq + 255) / 256, a.tk, a.mask.bm * a.mask.hm);
  else
    grid = dim3((a.tk + 255) / 256, a.tq, a.mask.bm * a.mask.hm);
  hipLaunchKernelGGL(classify_map_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fm
