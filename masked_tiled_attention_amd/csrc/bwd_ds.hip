// Backward with stored dS: slot plan and dQ = scale * dS K.
//
// "FlashAttention-2 ... GPU work partitioning" (iplexlaw.co.kr), section
// "Block processing keeps the global normalization": dQ = scale * dS K with
// dS = P (dP - D) is exact attention's gradient; how dS reaches the product
// is an implementation choice. The dK/dV kernel forms every non-SKIP bf16 dS
// tile anyway (as an MFMA operand); when the workspace holds them all, it
// writes them out and dQ becomes a plain product over the stored tiles,
// instead of a second kernel that recomputes S and dP (6 d flops per open
// pair then, 2 d flops and 2 bytes of dS traffic per pair here).
//
// Kernels:
//   plan_count  non-SKIP tiles per key-tile row of the dK/dV class map;
//   plan_scan   one workgroup: exclusive prefix sums (slot offsets), the total
//               and whether the workspace holds every tile for every (b, h);
//   dq_ds       one workgroup per (b, h, pair of 64-row query tiles), or per
//               part of the pair's list when few pairs have long key ranges:
//               for each key tile non-SKIP for either, K and the pair's stored
//               dS tiles go straight into LDS (one stage; two workgroups per
//               CU) and
//               dQ^T += K^T dS^T accumulates in registers;
//   dq_merge    split lists: dQ = the sum of the parts' float32 partials.
#include <climits>
#include <cmath>

#include "fm_device.hpp"
#include "fm_internal.hpp"
#include "fm_tile.hpp"

namespace fm {
namespace {

constexpr int BQ = kBwdBlockQ;   // rows per dS tile
constexpr int BK = kBwdBlockK;   // keys per dS tile
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int LIST_CAP = 1024;
constexpr int64_t kTileBytes = (int64_t)BQ * BK * 2;

// ------------------------------------------------------------------ plan
// grid (tk, mask rows): row_cnt[mr][kt] = non-SKIP entries of class row (mr, kt).
__global__ __launch_bounds__(256) void plan_count_kernel(BwdArgs a) {
  const int kt = blockIdx.x, mr = blockIdx.y;
  const uint8_t* row = a.classes_t + ((int64_t)mr * a.tk + kt) * a.tq;
  int c = 0;
  for (int q = threadIdx.x; q < a.tq; q += 256) c += row[q] != FM_TILE_SKIP;
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  __shared__ int red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) a.row_cnt[(int64_t)mr * a.tk + kt] = red[0] + red[1] + red[2] + red[3];
}

// grid (tk, mask rows): slots[mr][kt][qt] = row_off[mr][kt] + rank of qt
// among the row's non-SKIP entries (entries of SKIP tiles are not written).
__global__ __launch_bounds__(256) void plan_slots_kernel(BwdArgs a) {
  const int kt = blockIdx.x, mr = blockIdx.y;
  const int64_t r = (int64_t)mr * a.tk + kt;
  const uint8_t* row = a.classes_t + r * a.tq;
  int32_t* out = a.slots + r * a.tq;
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = a.row_off[r];
  for (int base = 0; base < a.tq; base += 256) {
    const int q = base + tid;
    const int v = q < a.tq && row[q] != FM_TILE_SKIP;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int pre = carry, chunk = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < wv) pre += wsum[k];
      chunk += wsum[k];
    }
    if (v) out[q] = pre + incl - 1;
    carry += chunk;
    __syncthreads();
  }
}

// One workgroup of 1024: row_off = exclusive prefix sums of row_cnt over the
// nrows = mask rows * tk rows in order, plan[0] = total, plan[1] = 1 when
// rep * total tiles fit into ds_capacity bytes (and slots fit in int32).
__global__ __launch_bounds__(1024) void plan_scan_kernel(BwdArgs a, int32_t nrows) {
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

// ------------------------------------------------------------------ dQ from dS
// One workgroup per (b, h, pair of adjacent 64-row query tiles). It walks the
// key tiles that are non-SKIP for either query tile of the pair; each K tile
// staged in LDS serves the stored dS tiles of both (two thirds of the bytes
// staged per tile of work, against one K tile per dS tile).
constexpr int PAIR = 2;   // query tiles per workgroup
// One staged key tile per workgroup (K and the pair's dS tiles, 76 KiB with the
// lists), so that two workgroups share a CU: one's loads overlap the other's
// products (1.22 ms at 128K, against 1.34 with two stages and one workgroup
// per CU).
constexpr int NSTAGE = 1;

template <int D>
struct alignas(16) DsSmem {
  uint16_t k[NSTAGE][BK * D];          // key tiles, row-major, swizzled
  uint16_t ds[NSTAGE][PAIR][BK * BQ];  // dS tiles as stored: 16 MFMA operand fragments of 1 KiB
  uint32_t list[LIST_CAP];             // key tiles of the pair's list
  int32_t slot[LIST_CAP][PAIR];        // stored-dS slot per query tile of the pair; -1: SKIP
  int32_t scan[NW];
};

// The pair's key-tile list: ascending key tiles that are non-SKIP for query
// tile qt0 or qt0 + 1 (the latter only when has1), with both slots. Starts and
// ends with a barrier.
__device__ __forceinline__ int compact_pair(const uint8_t* ccol, const int32_t* scol, int64_t stride, int first,
                                            int count, bool has1, uint32_t* sm_list, int32_t (*sm_slot)[PAIR],
                                            int32_t* sm_scan, int tid) {
  constexpr int PER = LIST_CAP / NT;
  const int lane = tid & 63, wave = tid >> 6;
  bool on[PER][PAIR];
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid * PER + e;
    const int64_t o = (int64_t)(first + idx) * stride;
    on[e][0] = idx < count && ccol[o] != FM_TILE_SKIP;
    on[e][1] = idx < count && has1 && ccol[o + 1] != FM_TILE_SKIP;
    cnt += on[e][0] || on[e][1];
  }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == 63) sm_scan[wave] = incl;
  __syncthreads();
  int pos = incl - cnt, n_list = 0;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    if (ww < wave) pos += sm_scan[ww];
    n_list += sm_scan[ww];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (on[e][0] || on[e][1]) {
      const int kt = first + tid * PER + e;
      const int64_t o = (int64_t)kt * stride;
      sm_list[pos] = (uint32_t)kt;
      sm_slot[pos][0] = on[e][0] ? scol[o] : -1;
      sm_slot[pos][1] = on[e][1] ? scol[o + 1] : -1;
      ++pos;
    }
  }
  __syncthreads();
  return n_list;
}

template <int D, bool F32>
__global__ __launch_bounds__(NT) void bwd_dq_ds_kernel(BwdArgs a) {
  if (a.plan == nullptr || a.plan[1] == 0) return;   // dQ comes from the recompute kernel
  constexpr int CB = D / 32;              // 32-channel blocks of dQ^T
  constexpr int RB = 2 * PAIR;            // 32-row blocks of the pair
  constexpr int BLK = CB * RB / NW;       // (channel block, row block) pairs per wavefront
  constexpr int KR = (BK * D / 8) / NT;   // 16-byte chunks per thread of a float32 key tile
  constexpr int ES = F32 ? 4 : 2;
  __shared__ DsSmem<D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 31;
  const int g = l >> 5;

  // Later query tiles first, heads interleaved: neighbouring workgroups work
  // on nearby rows and share K tiles in L2 (this kernel is bound by memory
  // traffic, so that beats ordering by length).
  // With split lists (a.dq_split > 1), consecutive workgroups take the
  // parts of one pair's key-tile list and write float32 partial dQ.
  const int ks = a.dq_split > 1 ? a.dq_split : 1;
  const int sp = (int)(blockIdx.x % ks);   // this workgroup's part
  const int wg = (int)(blockIdx.x / ks);
  const int nbh = a.batch * a.heads;
  const int npair = (a.tq + PAIR - 1) / PAIR;
  const int qt0 = PAIR * (npair - 1 - wg / nbh);
  const bool has1 = qt0 + 1 < a.tq;
  const int bh = wg % nbh;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  const int mrow = (a.mask.bm > 1 ? b : 0) * a.mask.hm + (a.mask.hm > 1 ? h : 0);
  const int rep_i = (a.mask.bm > 1 ? 0 : b) * (a.mask.hm > 1 ? 1 : a.heads) + (a.mask.hm > 1 ? 0 : h);
  const int64_t total = __builtin_amdgcn_readfirstlane(a.plan[0]);   // uniform
  const uint16_t* ds_rep = a.ds + (int64_t)rep_i * total * (BK * BQ);
  const uint8_t* ccol = a.classes_t + (int64_t)mrow * a.tk * a.tq + qt0;   // stride tq over kt
  const int32_t* scol = a.slots + (int64_t)mrow * a.tk * a.tq + qt0;

  // This wavefront's channel block and row blocks (row block rb: query tile
  // rb / 2 of the pair, rows 32 (rb % 2) ..). For d = 128 a wavefront owns one
  // channel block and all four row blocks; for d = 64 one channel block and
  // one row block of each query tile.
  const int cbw = CB == 4 ? w : (w & 1);
  auto rb_of = [&](int j) { return CB == 4 ? j : (w >> 1) + 2 * j; };
  f32x16 acc[BLK];
#pragma unroll
  for (int j = 0; j < BLK; ++j) acc[j] = f32x16{};

  // ---- staging: K (bf16: direct loads; float32: through registers) and the
  // present dS tiles ----
  const int64_t k_ld = a.k_ss * ES;
  const char* kbh = reinterpret_cast<const char*>(a.k) + ((int64_t)b * a.k_sb + (int64_t)__builtin_amdgcn_readfirstlane(h / a.group) * a.k_sh) * ES;
  using DmaK = DmaTile<D, BK, NT>;
  constexpr int NOFF = F32 ? KR : 1;
  uint32_t koff[NOFF];
  if constexpr (F32) {
    tile_offsets<D, F32, KR, NT>(koff, k_ld, tid);
  } else {
    koff[0] = DmaK::offset(k_ld, tid);
  }
  constexpr int SPER = BK * BQ * 2 / 1024 / NW;   // dS fragments per wavefront and tile
  const uint32_t sdst = lds_address(sm.ds) + (uint32_t)__builtin_amdgcn_readfirstlane(w) * 1024u;
  auto stage = [&](int idx, int buf) {   // list entry idx -> stage buf
    const int kt = __builtin_amdgcn_readfirstlane((int)sm.list[idx]);   // uniform
    const int n0 = kt * BK;
    if constexpr (F32) {
      u32x4 rk[KR];
      load_tile_rows<D, F32, KR, NT>(rk, kbh + n0 * k_ld, koff, k_ld, tid, a.seq_k - n0);
      store_tile_rows<D, KR, NT>(reinterpret_cast<char*>(sm.k[buf]), rk, tid);
    } else {
      DmaK::load(reinterpret_cast<char*>(sm.k[buf]), kbh + n0 * k_ld, koff[0], k_ld, tid, a.seq_k - n0);
    }
#pragma unroll
    for (int q = 0; q < PAIR; ++q) {
      const int64_t slot = __builtin_amdgcn_readfirstlane(sm.slot[idx][q]);   // uniform
      if (slot < 0) continue;
      // the tile is copied as stored, fragment i * NW + w by this wavefront
      const char* src = reinterpret_cast<const char*>(ds_rep + slot * (BK * BQ)) + w * 1024;
      const uint32_t dst = sdst + (uint32_t)(buf * PAIR + q) * (BK * BQ * 2);
#pragma unroll
      for (int i = 0; i < SPER; ++i)
        DmaK::dma16_nt(src + i * NW * 1024, 16u * (uint32_t)l, dst + (uint32_t)(i * NW) * 1024u);
    }
  };

  // dQ^T (channels x rows) += K^T (channels x keys) dS^T (keys x rows), 16
  // keys per step: K^T read transposed, dS^T as the stored fragment lane, both
  // with the same key order per lane half. Only the present query tiles' row
  // blocks take part (P0, P1: query tile 0, 1 present).
  auto products = [&](const char* kb, const char* sb, auto p0_c, auto p1_c) {
    constexpr bool P0 = decltype(p0_c)::value, P1 = decltype(p1_c)::value;
    constexpr int NJ = (P0 ? BLK / 2 : 0) + (P1 ? BLK / 2 : 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int r0 = 16 * s + 4 * g;
      const u32x4 ka = tr_operand<D>(kb, l, 32 * cbw, r0, r0 + 8);
#pragma unroll
      for (int j = 0; j < BLK; ++j) {
        const int rb = rb_of(j);
        const int q = rb >> 1;
        if ((q == 0 && !P0) || (q == 1 && !P1)) continue;
        acc[j] = mfma32(ka, *reinterpret_cast<const u32x4*>(sb + q * (BK * BQ * 2) + ((rb & 1) * 8 + s) * 1024 + l * 16),
                        acc[j]);
      }
    }
    sched_lds_mfma<(BK / 16) * NJ, (1 + 2 * NJ) / NJ, 2>();
  };

  for (int kt0 = 0; kt0 < a.tk; kt0 += LIST_CAP) {
    const int n_list = compact_pair(ccol, scol, (int64_t)a.tq, kt0, min(LIST_CAP, a.tk - kt0), has1, sm.list,
                                    sm.slot, sm.scan, tid);
    // this workgroup's part of the list (all of it unless lists are split)
    const int lo = (int)((int64_t)n_list * sp / ks), hi = (int)((int64_t)n_list * (sp + 1) / ks);
    if (lo == hi) continue;
    stage(lo, 0);

    for (int it = lo; it < hi; ++it) {
      const int buf = 0;
      wait_vmem();       // this stage landed (nothing younger is in flight)
      __syncthreads();   // the stage is visible to all
      const char* kb = reinterpret_cast<const char*>(sm.k[buf]);
      const char* sb = reinterpret_cast<const char*>(sm.ds[buf]);
      const bool p0 = sm.slot[it][0] >= 0, p1 = sm.slot[it][1] >= 0;
      if (p0 && p1) products(kb, sb, std::true_type{}, std::true_type{});
      else if (p0) products(kb, sb, std::true_type{}, std::false_type{});
      else products(kb, sb, std::false_type{}, std::true_type{});
      __syncthreads();   // every wavefront is done with the stage
      if (it + 1 < hi) stage(it + 1, 0);
    }
  }

  // ---- epilogue: dQ = scale * (dQ^T)^T; lane = query row, registers = channels ----
  // Column c of stored fragment row block rb is row 32 rb + 16 t + 4 g +
  // (j < 4 ? j : j + 4) with g, t = bits 4, 3 of c, j = c % 8.
#pragma unroll
  for (int j = 0; j < BLK; ++j) {
    const int rb = rb_of(j);
    const int c = lr;
    const int jj = c & 7;
    const int m = (qt0 + (rb >> 1)) * BQ + 32 * (rb & 1) + 16 * ((c >> 3) & 1) + 4 * (c >> 4) + (jj < 4 ? jj : jj + 4);
    if (m < a.seq_q && ks > 1) {   // float32 partial [ks][B][H][Sq][D]
      float* out = a.dqpart + ((((int64_t)sp * a.batch + b) * a.heads + h) * a.seq_q + m) * D;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(out + 32 * cbw + 8 * q4 + 4 * g) =
            f32x4{acc[j][4 * q4] * a.scale, acc[j][4 * q4 + 1] * a.scale, acc[j][4 * q4 + 2] * a.scale,
                  acc[j][4 * q4 + 3] * a.scale};
    } else if (m < a.seq_q) {
      const int64_t qoff = (int64_t)b * a.q_sb + (int64_t)m * a.q_ss + (int64_t)h * a.q_sh;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = 32 * cbw + 8 * q4 + 4 * g;
        const float x0 = acc[j][4 * q4] * a.scale, x1 = acc[j][4 * q4 + 1] * a.scale;
        const float x2 = acc[j][4 * q4 + 2] * a.scale, x3 = acc[j][4 * q4 + 3] * a.scale;
        if constexpr (F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dq) + qoff + c0) = f32x4{x0, x1, x2, x3};
        } else {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.dq) + qoff + c0) =
              u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
        }
      }
    }
  }
}

// Split lists: dQ = the sum of the parts' float32 partials (fixed order), one
// thread per 4 channels of one row. Exits when the plan chose the recompute
// path.
template <int D, bool F32>
__global__ __launch_bounds__(256) void dq_merge_kernel(BwdArgs a) {
  if (a.plan == nullptr || a.plan[1] == 0) return;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // ((b * H + h) * Sq + m) * D / 4 + c4
  const int64_t rows = (int64_t)a.batch * a.heads * a.seq_q;
  if (i >= rows * (D / 4)) return;
  const int64_t r = i / (D / 4);
  const int c0 = (int)(i % (D / 4)) * 4;
  f32x4 x = f32x4{};
  for (int s = 0; s < a.dq_split; ++s) x += *reinterpret_cast<const f32x4*>(a.dqpart + (s * rows + r) * D + c0);
  const int m = (int)(r % a.seq_q);
  const int h = (int)((r / a.seq_q) % a.heads);
  const int b = (int)(r / ((int64_t)a.seq_q * a.heads));
  const int64_t off = (int64_t)b * a.q_sb + (int64_t)m * a.q_ss + (int64_t)h * a.q_sh + c0;
  if constexpr (F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dq) + off) = x;
  } else {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.dq) + off) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
  }
}

template <int D, bool F32>
hipError_t launch_dq_ds_t(const BwdArgs& a, hipStream_t s) {
  const int ks = a.dq_split > 1 ? a.dq_split : 1;
  const int npair = (a.tq + PAIR - 1) / PAIR;
  hipLaunchKernelGGL((bwd_dq_ds_kernel<D, F32>), dim3(npair * a.batch * a.heads * ks), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  const int64_t n = (int64_t)a.batch * a.heads * a.seq_q * (D / 4);
  hipLaunchKernelGGL((dq_merge_kernel<D, F32>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_plan(const BwdArgs& a, bool with_slots, hipStream_t stream) {
  const int mrows = a.mask.bm * a.mask.hm;
  hipLaunchKernelGGL(plan_count_kernel, dim3(a.tk, mrows), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, stream, a, (int32_t)(mrows * a.tk));
  if ((e = hipGetLastError()) != hipSuccess || !with_slots) return e;
  hipLaunchKernelGGL(plan_slots_kernel, dim3(a.tk, mrows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds(const BwdArgs& a, int head_dim, bool f32, hipStream_t s) {
  if (head_dim == 128) return f32 ? launch_dq_ds_t<128, true>(a, s) : launch_dq_ds_t<128, false>(a, s);
  return f32 ? launch_dq_ds_t<64, true>(a, s) : launch_dq_ds_t<64, false>(a, s);
}

}  // namespace fm
