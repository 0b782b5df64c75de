// Pre-pass bodies shared by the standalone pre-pass kernels and the fused
// backward launches (classify.hip): tile summaries, class maps with their line
// counts, the longest-first launch order, the stored-dS slot offsets and the
// backward's per-row statistics. Each body is written for one workgroup of the
// stated size; a fused launch picks the body by workgroup index.
//
// The pages do not describe a tile pre-pass; the classification rule is the
// reading stated in fm_attn.h (fm_tile_classify).
#pragma once

#include <climits>
#include <cmath>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {
namespace prep {

static_assert(kBwdListCap % 256 == 0, "list passes end on a map-pass iteration");
constexpr int kOrderBuckets = 4096;
constexpr int64_t kTileBytes = (int64_t)kBwdBlockQ * kBwdBlockK * 2;   // one bf16 dS tile

__device__ __forceinline__ int wave_min(int x) {
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}

// One wavefront: min and max of the four bound vectors over the columns of key
// tile kt of mask row bh -> summary[bh][kt][8] (min lts, max lts, min lte, max
// lte, min uts, max uts, min ute, max ute). A missing pair reads as the empty
// interval [Sq, Sq) (lower) or [0, 0) (upper).
__device__ __forceinline__ void summary_tile(const ClassifyArgs& a, int kt, int bh) {
  // one wavefront per tile (a workgroup's wavefronts take consecutive tiles)
  const int lane = (int)(threadIdx.x & 63);
  const int bm = bh / a.mask.hm, hm = bh % a.mask.hm;
  const int64_t base = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const int c0 = kt * a.block_k;
  const int c1 = min(c0 + a.block_k, a.seq_k);
  int mn[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
  int mx[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
  for (int c = c0 + lane; c < c1; c += 64) {
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
  int r = 0;   // lane i < 8 keeps summary value i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int a0 = wave_min(mn[i]);
    const int a1 = wave_max(mx[i]);
    r = lane == 2 * i ? a0 : (lane == 2 * i + 1 ? a1 : r);
  }
  if (lane < 8) a.summary[((int64_t)bh * a.tk + kt) * 8 + lane] = r;
}

// The class of query rows [r0, r1) against a key tile with summary s: SKIP
// when one interval covers the rows for every key, FULL when both intervals
// miss them for every key, else PARTIAL.
__device__ __forceinline__ uint8_t classify_one(const int* s, int r0, int r1) {
  const bool covers_l = s[1] <= r0 && s[2] >= r1;
  const bool covers_u = s[5] <= r0 && s[6] >= r1;
  if (covers_l || covers_u) return (uint8_t)FM_TILE_SKIP;
  const bool misses_l = s[3] <= r0 || s[0] >= r1;
  const bool misses_u = s[7] <= r0 || s[4] >= r1;
  return (uint8_t)((misses_l && misses_u) ? FM_TILE_FULL : FM_TILE_PARTIAL);
}

// 256 threads: one line of the class map of mask row bh (a query tile's
// row of [tq][tk], or with `transposed` a key tile's row of [tk][tq]),
// classified from the summaries and written. With a.counts set, its number of
// non-SKIP entries goes to counts[bh * lines + line]; with a.chunk_pre set,
// the number of non-SKIP entries before each 64-entry chunk of the line goes
// to chunk_pre[bh * lines + line][chunk].
// With a.first set (transposed maps), the line's first entry in the dK/dV
// kernel's list order goes to first[bh * lines + line]: of the first
// kBwdListCap-entry pass that has a non-SKIP entry, its first FULL entry, else
// its first PARTIAL one (all entries count as PARTIAL for the ragged last key
// tile); -1 for a line with none.
__device__ __forceinline__ void map_line(const ClassifyArgs& a, int line, int bh) {
  __shared__ int wcnt[4];
  __shared__ int wmin[2][4];   // per wavefront: first FULL, first non-SKIP entry
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool tr = a.transposed != 0;
  const int len = tr ? a.tq : a.tk;
  const int64_t lid = (int64_t)bh * (tr ? a.tk : a.tq) + line;
  uint8_t* out = a.classes + lid * len;
  const int* sb = a.summary + (int64_t)bh * a.tk * 8;
  int s[8];
  int r0 = 0, r1 = 0;
  if (tr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = sb[line * 8 + i];
  } else {
    r0 = line * a.block_q;
    r1 = min(r0 + a.block_q, a.seq_q);
  }
  const int nch = (len + 63) / 64;
  const bool want_first = tr && a.first != nullptr;
  const bool all_partial = (a.seq_k % a.block_k) != 0 && line == a.tk - 1;   // the ragged last key tile
  int carry = 0;
  int pass_full = INT_MAX, pass_open = INT_MAX, first = -1;   // (uniform over the workgroup)
  for (int base = 0; base < len; base += 256) {
    const int i = base + tid;
    bool open = false, full = false;
    if (i < len) {
      if (tr) {
        r0 = i * a.block_q;
        r1 = min(r0 + a.block_q, a.seq_q);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] = sb[i * 8 + k];
      }
      const uint8_t c = classify_one(s, r0, r1);
      out[i] = c;
      open = c != FM_TILE_SKIP;
      full = c == FM_TILE_FULL && !all_partial;
    }
    const uint64_t bo = __ballot(open), bf = __ballot(full);
    const int wc = __popcll(bo);
    __syncthreads();   // every thread is done with the previous iteration's counts
    if (lane == 0) {
      wcnt[wv] = wc;
      wmin[0][wv] = bf ? base + 64 * wv + __builtin_ctzll(bf) : INT_MAX;
      wmin[1][wv] = bo ? base + 64 * wv + __builtin_ctzll(bo) : INT_MAX;
    }
    __syncthreads();
    int pre = carry, tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < wv) pre += wcnt[k];
      tot += wcnt[k];
      pass_full = min(pass_full, wmin[0][k]);
      pass_open = min(pass_open, wmin[1][k]);
    }
    const int ch = base / 64 + wv;
    if (a.chunk_pre && lane == 0 && ch < nch) a.chunk_pre[lid * nch + ch] = pre;
    carry += tot;
    // end of a list pass (kBwdListCap is a multiple of 256): its first entry
    if ((base + 256) % kBwdListCap == 0 || base + 256 >= len) {
      if (first < 0 && pass_open != INT_MAX) first = pass_full != INT_MAX ? pass_full : pass_open;
      pass_full = pass_open = INT_MAX;
    }
  }
  if (a.counts && tid == 0) a.counts[lid] = carry;
  if (want_first && tid == 0) a.first[lid] = first;
}

// 1024 threads: a.order = the lines sorted by their count, descending (a
// counting sort over at most 4096 buckets; the order within a bucket is
// arbitrary, only the launch order depends on it). Line r counts the sum of
// `group` entries of a.counts (see OrderArgs); with mark_empty, lines whose
// count is 0 carry kEmptyLine.
__device__ __forceinline__ void sort_lines(const OrderArgs& a) {
  __shared__ int hist[kOrderBuckets];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t cmax = (int64_t)a.len * a.group;
  // with mark_empty, lines with no work take a bucket of their own, the last
  const int nb = (int)min(cmax + 1, (int64_t)kOrderBuckets - (a.mark_empty ? 1 : 0));
  const int nbt = nb + (a.mark_empty ? 1 : 0);
  auto count = [&](int r) {
    const int64_t at = (int64_t)(r / a.inner) * a.outer_stride + r % a.inner;
    int64_t c = 0;
    for (int gi = 0; gi < a.group; ++gi) c += a.counts[at + gi * a.group_stride];
    return min(max(c, (int64_t)0), cmax);
  };
  auto key = [&](int64_t c) {   // descending count
    return a.mark_empty && c == 0 ? nb : nb - 1 - (int)(c * nb / (cmax + 1));
  };
  for (int i = tid; i < nbt; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int r = tid; r < a.rows; r += 1024) atomicAdd(&hist[key(count(r))], 1);
  __syncthreads();
  // exclusive scan: thread t owns buckets 4t .. 4t+3
  int v[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    v[i] = b < nbt ? hist[b] : 0;
    sum += v[i];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int pre = incl - sum;
  for (int k = 0; k < wv; ++k) pre += wsum[k];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    if (b < nbt) hist[b] = pre;
    if (a.live != nullptr && b == nbt - 1) *a.live = pre;   // lines before the empty ones
    pre += v[i];
  }
  __syncthreads();
  for (int r = tid; r < a.rows; r += 1024) {
    const int64_t c = count(r);
    const int pos = atomicAdd(&hist[key(c)], 1);
    a.order[pos] = (int32_t)((uint32_t)r | (a.mark_empty && c == 0 ? kEmptyLine : 0u));
    if (a.first_out) a.first_out[pos] = a.first_in[r];
  }
}

// 1024 threads: the stored-dS dQ kernel's launch order over blocks of
// kDqBlockPairs query-tile pairs (block b holds pairs npair - 1 - 16 b - i,
// i < 16: later pairs first within a block, so neighbouring workgroups still
// share K tiles), the block with the longest list first; ties keep the later
// block first. A pair's list length is its dQ-map line count (the 128-row
// line is the pair); one mask row.
constexpr int kMaxDqBlocks = 4096;   // beyond this, the blocks keep their natural order
__device__ __forceinline__ void sort_dq_blocks(const BwdArgs& a) {
  __shared__ int bkey[kMaxDqBlocks];
  const int npair = a.tq_q;
  const int nblk = (npair + kDqBlockPairs - 1) / kDqBlockPairs;
  const int tid = threadIdx.x;
  if (nblk > kMaxDqBlocks) {
    for (int b = tid; b < nblk; b += 1024) a.dq_blocks[b] = b;
    return;
  }
  for (int b = tid; b < nblk; b += 1024) {
    int m = 0;
    for (int i = 0; i < kDqBlockPairs; ++i) {
      const int p = npair - 1 - kDqBlockPairs * b - i;
      if (p >= 0) m = max(m, a.counts_q[p]);
    }
    bkey[b] = m;
  }
  __syncthreads();
  for (int b = tid; b < nblk; b += 1024) {
    const int kb = bkey[b];
    int rank = 0;
    for (int o = 0; o < nblk; ++o) {
      const int ko = bkey[o];
      rank += (ko > kb) || (ko == kb && o < b);
    }
    a.dq_blocks[rank] = b;
  }
}

// 1024 threads: row_off = exclusive prefix sums of row_cnt over the nrows =
// mask rows * tk key-tile rows, plan[0] = the total, plan[1] = 1 when rep *
// total dS tiles fit into ds_capacity bytes (and slots fit in int32).
__device__ __forceinline__ void scan_slots(const BwdArgs& a, int nrows) {
  __shared__ int wsum[16];
  __shared__ int64_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nrows; base += 1024) {
    const int i = base + tid;
    const int v = i < nrows ? a.row_cnt[i] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int64_t pre = carry;
    int chunk = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < wv) pre += wsum[k];
      chunk += wsum[k];
    }
    if (i < nrows) a.row_off[i] = (int32_t)min(pre + incl - v, (int64_t)INT_MAX);
    __syncthreads();
    if (tid == 0) carry += chunk;
    __syncthreads();
  }
  if (tid == 0) {
    const int64_t total = carry;
    a.plan[0] = (int32_t)min(total, (int64_t)INT_MAX);
    a.plan[1] = (total < INT_MAX && total * a.rep * kTileBytes <= a.ds_capacity) ? 1 : 0;
  }
}

// 256 threads: rows RPB blk .. RPB blk + RPB - 1 (RPB = 2048 / D) of the
// backward's row pass over (b, m, h), m < Sp: D = rowsum(dO * O) and
// LSE * log2(e), the latter +inf where the row sees no key (LSE = -inf) so
// that P = 0 there; rows past Sq get +inf and 0, so tiles may read whole
// padded row blocks.
template <int D, bool F32>
__device__ __forceinline__ void row_stats(const BwdArgs& a, int blk) {
  constexpr int TPR = D / 8;            // threads per row
  constexpr int RPB = 256 / TPR;        // rows per block
  const int sub = threadIdx.x % TPR;
  const int64_t row = (int64_t)blk * RPB + threadIdx.x / TPR;   // (b, m, h) linear, m < Sp
  const int64_t nrows = (int64_t)a.batch * a.seq_pad * a.heads;
  float part = 0.f;
  int b = 0, m = 0, h = 0;
  if (row < nrows) {
    h = (int)(row % a.heads);
    m = (int)((row / a.heads) % a.seq_pad);
    b = (int)(row / ((int64_t)a.heads * a.seq_pad));
  }
  if (row < nrows && m < a.seq_q) {
    const int64_t off = (int64_t)b * a.o_sb + (int64_t)m * a.o_ss + (int64_t)h * a.o_sh + 8 * sub;
    float x[8], y[8];
    if constexpr (F32) {
      const float* po = reinterpret_cast<const float*>(a.o) + off;
      const float* pd = reinterpret_cast<const float*>(a.dout) + off;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = po[i];
        y[i] = pd[i];
      }
    } else {
      const u32x4 vo = ld16(reinterpret_cast<const uint16_t*>(a.o) + off);
      const u32x4 vd = ld16(reinterpret_cast<const uint16_t*>(a.dout) + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(vo[i]);
        x[2 * i + 1] = bf16_hi(vo[i]);
        y[2 * i] = bf16_lo(vd[i]);
        y[2 * i + 1] = bf16_hi(vd[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part = fmaf(x[i], y[i], part);
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (row < nrows && sub == 0) {
    const int64_t r = ((int64_t)b * a.heads + h) * a.seq_pad + m;
    float l2 = INFINITY;
    if (m < a.seq_q) {
      const float lse = a.lse[((int64_t)b * a.heads + h) * a.seq_q + m];
      l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
    }
    a.lse2[r] = l2;
    a.drow[r] = part;
  }
}

}  // namespace prep
}  // namespace fm
