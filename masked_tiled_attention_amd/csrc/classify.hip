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

}  // namespace

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
