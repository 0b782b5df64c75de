// Pre-pass kernels: tile classification, launch orders and, for the
// backward, the row pass and the stored-dS slot plan.
//
// The pages do not describe a tile pre-pass; its rule is the reading stated in
// fm_attn.h (fm_tile_classify). The bodies live in prep.hpp. Forward (and
// fm_tile_classify):
//   summary   one wavefront per (mask row, key tile), four per workgroup:
//             min / max of the four bound vectors over the tile's columns
//             -> 8 int32;
//   map       one workgroup per (mask row, map line): the line's classes from
//             the summaries, and its non-SKIP count;
//   order     one workgroup: lines sorted by count, longest first.
// The backward runs the same steps fused into four launches whose workgroups
// pick their task by index, since each launch in a chain of dependent ones
// costs a few microseconds whatever its size.
// Everything here is integer work bound by launch latency and HBM.
#include <climits>

#include "fm_device.hpp"
#include "fm_internal.hpp"
#include "prep.hpp"

namespace fm {
namespace {

// grid (ceil(tk / 4), bm * hm): wavefront w takes key tile 4 * blockIdx.x + w
__global__ __launch_bounds__(256) void classify_summary_kernel(ClassifyArgs a) {
  const int kt = 4 * blockIdx.x + (int)(threadIdx.x >> 6);
  if (kt < a.tk) prep::summary_tile(a, kt, blockIdx.y);
}

// grid (lines, bm * hm): lines = tq, or tk when transposed
__global__ __launch_bounds__(256) void classify_map_kernel(ClassifyArgs a) {
  prep::map_line(a, blockIdx.x, blockIdx.y);
}

__global__ __launch_bounds__(1024) void order_sort_kernel(OrderArgs a) { prep::sort_lines(a); }

// Backward launch 1: summaries of the dK/dV tiling (ct), then of the dQ
// tiling (cq).
// (one wavefront per tile, four per workgroup)
__global__ __launch_bounds__(256) void bwd_summaries_kernel(ClassifyArgs ct, ClassifyArgs cq) {
  const int mrows = ct.mask.bm * ct.mask.hm;
  const int t = 4 * blockIdx.x + (int)(threadIdx.x >> 6);
  if (t < ct.tk * mrows) return prep::summary_tile(ct, t % ct.tk, t / ct.tk);
  const int t2 = t - ct.tk * mrows;
  if (t2 < cq.tk * mrows) prep::summary_tile(cq, t2 % cq.tk, t2 / cq.tk);
}

// Backward launch 2: the lines of both class maps (ct transposed: key-tile
// lines; cq: query-tile lines).
__global__ __launch_bounds__(256) void bwd_maps_kernel(ClassifyArgs ct, ClassifyArgs cq) {
  const int mrows = ct.mask.bm * ct.mask.hm;
  const int blk = blockIdx.x;
  if (blk < ct.tk * mrows) return prep::map_line(ct, blk % ct.tk, blk / ct.tk);
  const int b2 = blk - ct.tk * mrows;
  prep::map_line(cq, b2 % cq.tq, b2 / cq.tq);
}

// Backward launch 3: workgroup 0 sorts the dK/dV order, the next ones the
// recompute dQ kernel's and the stored-dS dQ kernel's block order (each when
// set), and the last one scans the slot offsets (when the plan is set).
__global__ __launch_bounds__(1024) void bwd_orders_kernel(OrderArgs ok, OrderArgs oq, BwdArgs a) {
  int blk = blockIdx.x;
  if (blk == 0) return prep::sort_lines(ok);
  if (oq.order && --blk == 0) return prep::sort_lines(oq);
  if (a.dq_blocks && --blk == 0) return prep::sort_dq_blocks(a);
  prep::scan_slots(a, a.mask.bm * a.mask.hm * a.tk);
}

// Stored dS: slots_q[mr][qt][kt] = the slot of tile (kt, qt) for non-SKIP
// tiles (row_off of the key-tile row + non-SKIP tiles before its 64-tile chunk
// + its rank within the chunk), -1 for SKIP ones. Block (kb, ch, mr) of
// ceil(tk / 16) x ceil(tq / 64) x mask rows: each wavefront ranks four
// key-tile rows of a 64-tile chunk (one ballot each); the 16 x 64 block goes
// out through LDS so that the query-major writes are 64-byte runs.
__device__ __forceinline__ void slots_block(const BwdArgs& a, int kb, int ch, int mr) {
  __shared__ int32_t t[16][65];
  const int kt0 = kb * 16, q0 = ch * 64;
  const int w = threadIdx.x >> 6, c = threadIdx.x & 63;
  const int nch = (a.tq + 63) / 64;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = w + 4 * j, kt = kt0 + r, q = q0 + c;   // kt is uniform per wavefront
    bool open = false;
    if (kt < a.tk && q < a.tq) open = a.classes_t[((int64_t)mr * a.tk + kt) * a.tq + q] != FM_TILE_SKIP;
    const uint64_t bal = __ballot(open);
    int32_t v = -1;
    if (open) {
      const int64_t row = (int64_t)mr * a.tk + kt;
      const int64_t s = (int64_t)a.row_off[row] + a.chunk_pre[row * nch + ch] + __popcll(bal & ((1ull << c) - 1));
      v = (int32_t)min(s, (int64_t)INT_MAX);   // beyond INT_MAX the plan disables the store
    }
    t[r][c] = v;
  }
  __syncthreads();
  const int kk = threadIdx.x & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int qq = (threadIdx.x >> 4) + 16 * j, q = q0 + qq, kt = kt0 + kk;
    if (q < a.tq && kt < a.tk) a.slots_q[((int64_t)mr * a.tq + q) * a.tk + kt] = t[kk][qq];
  }
}

// Backward launch 4: n_slots blocks of the slot map (stored dS), then the row
// pass (D and LSE * log2(e)), which the dK/dV kernel reads next, together with
// dO.
template <int D, bool F32>
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdArgs a, int n_slots) {
  const int blk = blockIdx.x;
  if (blk < n_slots) {
    const int gx = (a.tk + 15) / 16, gy = (a.tq + 63) / 64;
    return slots_block(a, blk % gx, (blk / gx) % gy, blk / (gx * gy));
  }
  prep::row_stats<D, F32>(a, blk - n_slots);
}

template <int D, bool F32>
hipError_t launch_rows_t(const BwdArgs& a, bool slots, bool rows, hipStream_t s) {
  const int64_t n_slots = slots ? (int64_t)((a.tk + 15) / 16) * ((a.tq + 63) / 64) * a.mask.bm * a.mask.hm : 0;
  int64_t nblk = n_slots;
  if (rows) {
    const int64_t nrows = (int64_t)a.batch * a.seq_pad * a.heads;
    const int rpb = 256 / (D / 8);
    nblk += (nrows + rpb - 1) / rpb;
  }
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_rows_kernel<D, F32>), dim3((unsigned)nblk), dim3(256), 0, s, a, (int)n_slots);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_order(const OrderArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(order_sort_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_classify_summary(const ClassifyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(classify_summary_kernel, dim3((a.tk + 3) / 4, a.mask.bm * a.mask.hm), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_classify_map(const ClassifyArgs& a, hipStream_t stream) {
  const dim3 grid(a.transposed ? a.tk : a.tq, a.mask.bm * a.mask.hm);
  hipLaunchKernelGGL(classify_map_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Each of these launches does the work of two or more small kernels: each
// such kernel is far too small to fill the chip, and in a chain of dependent
// launches each costs a few microseconds whatever its size.
hipError_t launch_bwd_summaries(const ClassifyArgs& ct, const ClassifyArgs& cq, hipStream_t stream) {
  const int64_t mrows = (int64_t)ct.mask.bm * ct.mask.hm;
  hipLaunchKernelGGL(bwd_summaries_kernel, dim3((unsigned)(((ct.tk + cq.tk) * mrows + 3) / 4)), dim3(256), 0, stream,
                     ct, cq);
  return hipGetLastError();
}

hipError_t launch_bwd_maps(const ClassifyArgs& ct, const ClassifyArgs& cq, hipStream_t stream) {
  const int64_t mrows = (int64_t)ct.mask.bm * ct.mask.hm;
  hipLaunchKernelGGL(bwd_maps_kernel, dim3((unsigned)((ct.tk + cq.tq) * mrows)), dim3(256), 0, stream, ct, cq);
  return hipGetLastError();
}

hipError_t launch_bwd_orders(const OrderArgs& ok, const OrderArgs& oq, const BwdArgs& a, hipStream_t stream) {
  const int nblk = 1 + (oq.order ? 1 : 0) + (a.dq_blocks ? 1 : 0) + (a.plan ? 1 : 0);
  hipLaunchKernelGGL(bwd_orders_kernel, dim3(nblk), dim3(1024), 0, stream, ok, oq, a);
  return hipGetLastError();
}

hipError_t launch_bwd_rows(const BwdArgs& a, bool slots, bool rows, int head_dim, bool f32, hipStream_t stream) {
  if (head_dim == 128)
    return f32 ? launch_rows_t<128, true>(a, slots, rows, stream) : launch_rows_t<128, false>(a, slots, rows, stream);
  return f32 ? launch_rows_t<64, true>(a, slots, rows, stream) : launch_rows_t<64, false>(a, slots, rows, stream);
}

}  // namespace fm
