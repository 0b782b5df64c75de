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

}  // namespace

hipError_t launch_localize(const LocalizeArgs& a, hipStream_t stream) {
  dim3 grid((a.seq_k + 255) / 256, a.mask.bm * a.mask.hm);
  hipLaunchKernelGGL(localize_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fm
