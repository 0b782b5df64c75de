// Forward kernel: masked attention with an online softmax over K/V tiles.
//
// "FlashAttention-2 ... GPU work partitioning" (iplexlaw.co.kr):
//   - "Block processing keeps the global normalization": inputs are tiled in
//     on-chip memory and the softmax is streamed, rescaling the running
//     statistics and partial output so that the result is normalised over
//     the whole key sequence; no score matrix goes to HBM.
//   - "Three ways to raise GPU utilization": less non-matmul work (the output
//     is normalised once at the end; no per-tile row maximum: probabilities
//     are formed against a reference that moves, with a rescale of the
//     running output, only when one of them would exceed 2^8; the mask is
//     evaluated only on PARTIAL tiles), work split over batch, heads and
//     query tiles, and the query rows of a tile split among the wavefronts
//     while K/V are shared.
// "FlashMask-3" page (iitog.ru), predecessor paragraph: the mask arrives as
// four bound vectors per key column; fully masked tiles are skipped using the
// classification pre-pass.
//
// CDNA4 mapping (one workgroup = 4 wavefronts = 128 query rows of one
// (batch, head); each wavefront owns 32 rows):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = the
//         wavefront's Q rows held in registers for the whole kernel. In the
//         accumulator each lane holds one query row (its column), so row max,
//         row sum and the rescale are per-lane scalars, combined with the
//         other half-wave once per tile (max) or once at the end (sum).
//   O^T += V^T P^T: B = P straight from the S^T accumulator (rounded to bf16),
//         A = V^T read with ds_read_b64_tr_b16 from the row-major V tile, with
//         the contraction index permuted identically on both sides.
// K and V tiles are double-buffered in LDS; the next tile's global loads are
// issued before the current tile's math. Each 64-key tile runs as two 32-key
// halves so that one half's softmax sits beside the other half's MFMAs.
#include <climits>
#include <cmath>
#include <type_traits>

#include "fm_device.hpp"
#include "fm_internal.hpp"
#include "fm_tile.hpp"

namespace fm {
namespace {

constexpr int BQ = kFwdBlockQ;   // 128 query rows per workgroup
constexpr int BK = kFwdBlockK;   // 64 keys per K/V tile
constexpr int NW = BQ / 32;      // 4 wavefronts
constexpr int NT = NW * 64;      // 256 threads
constexpr int LIST_CAP = 1024;   // class bytes compacted per pass (4 per thread)
// The running output is rescaled only when a row maximum grows by more than
// 2^kRescaleLog2; until then probabilities are taken relative to the older,
// smaller maximum (at most 2^kRescaleLog2, far from float overflow). O and the
// row sum always share the same reference, so the result is unchanged.
constexpr float kRescaleLog2 = 8.0f;
constexpr float kRescaleMax = 256.0f;   // 2^kRescaleLog2

template <int D>
struct alignas(16) FwdSmem {
  uint16_t k[2][BK * D];      // double-buffered K tile, row-major, swizzled
  uint16_t v[2][BK * D];      // double-buffered V tile, row-major, swizzled
  int32_t bnd[2][4][BK];      // lts, lte, uts, ute of the tile's keys
  uint32_t list[LIST_CAP];    // non-SKIP key tiles (kt | partial bit)
  int32_t scan[NW];
};

template <int D, bool F32>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs a) {
  constexpr int KSTEPS = D / 16;         // MFMA k-steps over the head dimension
  constexpr int CB = D / 32;             // 32-channel blocks of O^T
  constexpr int NB = BK / 32;            // 32-key blocks of a tile
  constexpr int KR = (BK * D / 8) / NT;  // 16-byte chunks per thread of a K (or V) tile
  constexpr int ES = F32 ? 4 : 2;
  __shared__ FwdSmem<D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 31;
  const int g = l >> 5;

  // Query tiles longest first (order from the class map), then the (b, h)
  // pairs that share the tile's mask row, then (split lists) the parts of the
  // tile's key-tile list.
  const int ks = a.ksplit > 1 ? a.ksplit : 1;
  const int sp = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % ks));   // this workgroup's part
  const int wg = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / ks));
  const int line = __builtin_amdgcn_readfirstlane(a.order[wg / a.rep]);   // mask row * tq + query tile
  const int j = wg % a.rep;
  const int qt = line % a.tq;
  const int mr = line / a.tq;
  const int bm = mr / a.mask.hm;
  const int hm = mr % a.mask.hm;
  const int b = a.mask.bm > 1 ? bm : j / (a.mask.hm > 1 ? 1 : a.heads);
  const int h = a.mask.hm > 1 ? hm : j % a.heads;
  const int64_t mbase = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const uint8_t* crow = a.classes + ((int64_t)(bm * a.mask.hm + hm) * a.tq + qt) * a.tk;

  const int m = qt * BQ + w * 32 + lr;   // this lane's query row
  const bool row_ok = m < a.seq_q;

  // The wavefront's Q rows as MFMA B operands (rows past the end re-read the
  // last row; their results are never stored).
  u32x4 qf[KSTEPS];
  {
    const int mq = min(m, a.seq_q - 1);
    const int64_t qoff = (int64_t)b * a.q_sb + (int64_t)mq * a.q_ss + (int64_t)h * a.q_sh + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = load8_as_bf16<F32>(a.q, qoff + 16 * s);
  }

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;   // reference maximum (raw score units)
  float l_run = 0.f;         // this lane's share of the row sum
  const float C = a.scale_log2;
  const bool ragged_k = (a.seq_k % BK) != 0;

  // ---- tile staging ----
  // bf16: straight from global memory into LDS (no staging registers);
  // float32: through registers, rounded to bf16 on the way.
  const int64_t k_ld = a.k_ss * ES, v_ld = a.v_ss * ES;
  const int hk = __builtin_amdgcn_readfirstlane(h / a.group);   // K/V head (grouped-query attention)
  const char* kbh = reinterpret_cast<const char*>(a.k) + ((int64_t)b * a.k_sb + (int64_t)hk * a.k_sh) * ES;
  const char* vbh = reinterpret_cast<const char*>(a.v) + ((int64_t)b * a.v_sb + (int64_t)hk * a.v_sh) * ES;
  using Dma = DmaTile<D, BK, NT>;
  constexpr int NOFF = F32 ? KR : 1;
  constexpr int NREG = F32 ? KR : 1;
  uint32_t koff[NOFF], voff[NOFF];
  if constexpr (F32) {
    tile_offsets<D, F32, KR, NT>(koff, k_ld, tid);
    tile_offsets<D, F32, KR, NT>(voff, v_ld, tid);
  } else {
    koff[0] = Dma::offset(k_ld, tid);
    voff[0] = Dma::offset(v_ld, tid);
  }
  u32x4 rk[NREG], rv[NREG];
  int32_t rb[4] = {INT_MIN, INT_MAX, 0, 0};

  // Start fetching key tile kt into LDS buffer `buf` (bf16) or registers (f32),
  // and its bounds into registers.
  auto load_tile = [&](int kt, bool masked, int buf) {
    const int n0 = kt * BK;
    if constexpr (F32) {
      load_tile_rows<D, F32, KR, NT>(rk, kbh + n0 * k_ld, koff, k_ld, tid, a.seq_k - n0);
      load_tile_rows<D, F32, KR, NT>(rv, vbh + n0 * v_ld, voff, v_ld, tid, a.seq_k - n0);
    } else {
      Dma::load(reinterpret_cast<char*>(sm.k[buf]), kbh + n0 * k_ld, koff[0], k_ld, tid, a.seq_k - n0);
      Dma::load(reinterpret_cast<char*>(sm.v[buf]), vbh + n0 * v_ld, voff[0], v_ld, tid, a.seq_k - n0);
    }
    if (masked && tid < BK) {
      const int n = n0 + tid;
      if (n < a.seq_k) {
        rb[0] = a.mask.has_lower ? a.mask.lts[mbase + n] : a.seq_q;
        rb[1] = a.mask.has_lower ? a.mask.lte[mbase + n] : a.seq_q;
        rb[2] = a.mask.has_upper ? a.mask.uts[mbase + n] : 0;
        rb[3] = a.mask.has_upper ? a.mask.ute[mbase + n] : 0;
      } else {   // keys past the end: masked for every row
        rb[0] = INT_MIN;
        rb[1] = INT_MAX;
        rb[2] = 0;
        rb[3] = 0;
      }
    }
  };
  // Finish staging into buffer `buf` what load_tile() left in registers.
  auto store_tile = [&](int buf, bool masked) {
    if constexpr (F32) {
      store_tile_rows<D, KR, NT>(reinterpret_cast<char*>(sm.k[buf]), rk, tid);
      store_tile_rows<D, KR, NT>(reinterpret_cast<char*>(sm.v[buf]), rv, tid);
    }
    if (masked && tid < BK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.bnd[buf][j][tid] = rb[j];
    }
  };
  // Interval mask on one 32-key half of a PARTIAL (or ragged) tile.
  auto mask_half = [&](f32x16& sc, int nb, int buf) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int nl = nb * 32 + 8 * q4 + 4 * g;   // 4 consecutive keys
      const i32x4 l0 = *reinterpret_cast<const i32x4*>(&sm.bnd[buf][0][nl]);
      const i32x4 l1 = *reinterpret_cast<const i32x4*>(&sm.bnd[buf][1][nl]);
      const i32x4 u0 = *reinterpret_cast<const i32x4*>(&sm.bnd[buf][2][nl]);
      const i32x4 u1 = *reinterpret_cast<const i32x4*>(&sm.bnd[buf][3][nl]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool mk = ((l0[r] <= m) & (m < l1[r])) | ((u0[r] <= m) & (m < u1[r]));
        sc[4 * q4 + r] = mk ? -INFINITY : sc[4 * q4 + r];
      }
    }
  };

  // Probabilities of one 32-key half against the current reference:
  // p = 2^(C s + nmC), rounded to bf16 as the MFMA consumes them; returns the
  // lane's sum of the same rounded values (two per v_dot2c), so O and l share
  // one set of weights.
  float nmC = INFINITY;   // -C * reference, or +inf while the row has no reference
  u32x4 pf[NB][2];
  auto soft_half = [&](const f32x16& sc, int nb) {
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(fmaf(sc[8 * t + 2 * j], C, nmC));
        const float p1 = fast_exp2(fmaf(sc[8 * t + 2 * j + 1], C, nmC));
        pf[nb][t][j] = pack_bf16(p0, p1);
        if (j & 1) r1 = add_bf16_pair(pf[nb][t][j], r1);
        else r0 = add_bf16_pair(pf[nb][t][j], r0);
      }
    return r0 + r1;
  };
  // The common path keeps the reference while every p of the half is at most
  // 2^kRescaleLog2 (a lane sum within that bound implies it; a row without a
  // reference yields inf or NaN here). Otherwise, wave-uniformly: the row
  // maximum of the half, a move of the reference to it when it is larger,
  // the rescale of O and l, and the half's probabilities again.
  auto settle_half = [&](const f32x16& sc, int nb, float rs) {
    if (__any(!(rs <= kRescaleMax))) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[i]);
      mx = pair_max(mx);
      const bool move = mx > m_run;   // false while both are -inf
      const float alpha = move ? fast_exp2((m_run - mx) * C) : 1.f;   // 0 from -inf
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
      m_run = move ? mx : m_run;
      nmC = m_run == -INFINITY ? 0.f : -m_run * C;   // fully masked so far: p = 0
      rs = soft_half(sc, nb);
      if (m_run == -INFINITY) nmC = INFINITY;
    }
    l_run += rs;
  };

  // Offsets of the transposed V reads, computed once. The swizzle depends on
  // the row modulo 16 only, so the 16-key steps of a tile (+16 rows) are
  // immediate offsets on the same address, and per tile only the buffer is
  // added. The offsets are made opaque so that the compiler keeps them whole
  // rather than rebuilding them per read.
  uint32_t vo[CB][2];
  {
    const uint32_t vbase = lds_address(sm.v[0]);
    const int i = l & 15;
    const int r = 4 * g + (i >> 2);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = 32 * cb + 16 * ((l >> 4) & 1) + 4 * (i & 3);
      vo[cb][0] = vbase + (uint32_t)rm_byte<D>(r, col);
      vo[cb][1] = vbase + (uint32_t)rm_byte<D>(r + 8, col);
      asm volatile("" : "+v"(vo[cb][0]));
      asm volatile("" : "+v"(vo[cb][1]));
    }
  }

  int it_global = 0;   // iteration count across passes (selects the LDS buffer)
  auto iteration = [&](auto masked_c, int it, int n_list, uint32_t& ent) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int buf = it_global & 1;
    store_tile(buf, MASKED);
    wait_vmem();
    __syncthreads();   // tile `buf` complete and visible; the other buffer is free
    if (it + 1 < n_list) {   // next tile's global loads overlap this tile's math
      ent = __builtin_amdgcn_readfirstlane(sm.list[it + 1]);
      load_tile((int)(ent & ~kPartialBit), (ent & kPartialBit) != 0, buf ^ 1);
    }
    const char* kb = reinterpret_cast<const char*>(sm.k[buf]);
    const uint32_t bo = (uint32_t)buf * (BK * D * 2);
    uint32_t vt_addr[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      vt_addr[cb][0] = vo[cb][0] + bo;
      vt_addr[cb][1] = vo[cb][1] + bo;
    }
    // V^T operand of the 16 keys from row 16 rr of the tile (rr = 0..3)
    auto vt = [&](int cb, int rr) {
      const u32x2 x = lds_tr16(vt_addr[cb][0], (uint32_t)rr * (16 * 2 * D));
      const u32x2 y = lds_tr16(vt_addr[cb][1], (uint32_t)rr * (16 * 2 * D));
      return u32x4{x[0], x[1], y[0], y[1]};
    };
    f32x16 sacc[NB];

    // S^T = K Q^T, first 32 keys
    sacc[0] = f32x16{};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      sacc[0] = mfma32(*reinterpret_cast<const u32x4*>(kb + rm_byte<D>(lr, 16 * s + 8 * g)), qf[s], sacc[0]);
    sched_lds_mfma<KSTEPS, 1, 4>();
    __builtin_amdgcn_sched_barrier(0);

    // S^T, second 32 keys, under the first half's mask and softmax
    sacc[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      sacc[1] = mfma32(*reinterpret_cast<const u32x4*>(kb + rm_byte<D>(32 + lr, 16 * s + 8 * g)), qf[s], sacc[1]);
    if constexpr (MASKED) mask_half(sacc[0], 0, buf);
    const float rs0 = soft_half(sacc[0], 0);
    settle_half(sacc[0], 0, rs0);

    // O^T += V^T P^T over the first 32 keys, under the second half's softmax
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) oacc[cb] = mfma32(vt(cb, t), pf[0][t], oacc[cb]);
    if constexpr (MASKED) mask_half(sacc[1], 1, buf);
    const float rs1 = soft_half(sacc[1], 1);
    settle_half(sacc[1], 1, rs1);

    // O^T += V^T P^T over the second 32 keys
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) oacc[cb] = mfma32(vt(cb, 2 + t), pf[1][t], oacc[cb]);
    sched_lds_mfma<2 * CB, 2, 3>();
  };

  // FULL tiles first (no mask), then PARTIAL ones and the ragged last tile.
  for (int kt0 = 0; kt0 < a.tk; kt0 += LIST_CAP) {
    int n_full;
    const int n_list = compact_classes_split<LIST_CAP, NT>(crow, kt0, min(LIST_CAP, a.tk - kt0), sm.list, nullptr,
                                                           sm.scan, tid, false, &n_full, ragged_k ? a.tk - 1 : -1);
    // this workgroup's part of the list (all of it unless lists are split)
    const int lo = (int)((int64_t)n_list * sp / ks), hi = (int)((int64_t)n_list * (sp + 1) / ks);
    if (lo == hi) continue;

    uint32_t ent = __builtin_amdgcn_readfirstlane(sm.list[lo]);
    load_tile((int)(ent & ~kPartialBit), (ent & kPartialBit) != 0, it_global & 1);
    int it = lo;
    for (; it < min(n_full, hi); ++it, ++it_global) iteration(std::false_type{}, it, hi, ent);
    for (; it < hi; ++it, ++it_global) iteration(std::true_type{}, it, hi, ent);
  }

  // ---- epilogue: normalise once, write O and LSE ----
  const float lt = pair_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (ks > 1) {   // split lists: float32 partial O and LSE of this part
    if (row_ok) {
      const int64_t r = (((int64_t)sp * a.batch + b) * a.heads + h) * a.seq_q + m;
      float* op = a.opart + r * D;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(op + cb * 32 + 8 * q4 + 4 * g) =
              f32x4{oacc[cb][4 * q4] * inv, oacc[cb][4 * q4 + 1] * inv, oacc[cb][4 * q4 + 2] * inv,
                    oacc[cb][4 * q4 + 3] * inv};
      if (g == 0) a.lpart[r] = lt > 0.f ? (m_run * C + __log2f(lt)) * kLn2 : -INFINITY;
    }
  } else if (row_ok) {
    const int64_t ooff = (int64_t)b * a.o_sb + (int64_t)m * a.o_ss + (int64_t)h * a.o_sh;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = cb * 32 + 8 * q4 + 4 * g;
        const float x0 = oacc[cb][4 * q4 + 0] * inv, x1 = oacc[cb][4 * q4 + 1] * inv;
        const float x2 = oacc[cb][4 * q4 + 2] * inv, x3 = oacc[cb][4 * q4 + 3] * inv;
        if constexpr (F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + ooff + c0) = f32x4{x0, x1, x2, x3};
        } else {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.o) + ooff + c0) =
              u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
        }
      }
    }
    if (g == 0)
      a.lse[((int64_t)b * a.heads + h) * a.seq_q + m] =
          lt > 0.f ? (m_run * C + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// Split lists: O and LSE of each row from the parts' normalised partial O_s
// and LSE_s: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s (the
// parts' softmax weights). A row no part sees keeps O = 0, LSE = -inf. One
// thread per 4 channels of one row; KS (the part count) is a compile-time
// constant so that every part's loads go out before any is used.
template <int D, bool F32, int KS>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // ((b * H + h) * Sq + m) * D / 4 + c4
  const int64_t rows = (int64_t)a.batch * a.heads * a.seq_q;
  if (i >= rows * (D / 4)) return;
  const int64_t r = i / (D / 4);
  const int c0 = (int)(i % (D / 4)) * 4;
  float lp[KS];
  f32x4 op[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    lp[s] = a.lpart[s * rows + r];
    op[s] = *reinterpret_cast<const f32x4*>(a.opart + (s * rows + r) * D + c0);
  }
  // no branch (it would hold the O loads back behind the LSE loads): with no
  // part seeing the row every weight is exp(-inf) = 0 against a zero reference
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < KS; ++s) mx = fmaxf(mx, lp[s]);
  const bool seen = mx > -INFINITY;
  const float mref = seen ? mx : 0.f;
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) sum += __expf(lp[s] - mref);
  const float lse = seen ? mref + __logf(sum) : -INFINITY;
  const float lref = seen ? lse : 0.f;
  f32x4 o = f32x4{};
#pragma unroll
  for (int s = 0; s < KS; ++s) o += __expf(lp[s] - lref) * op[s];
  const int m = (int)(r % a.seq_q);
  const int h = (int)((r / a.seq_q) % a.heads);
  const int b = (int)(r / ((int64_t)a.seq_q * a.heads));
  const int64_t ooff = (int64_t)b * a.o_sb + (int64_t)m * a.o_ss + (int64_t)h * a.o_sh + c0;
  if constexpr (F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + ooff) = o;
  } else {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.o) + ooff) = u32x2{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
  }
  if (c0 == 0) a.lse[r] = lse;
}

template <int D, bool F32>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int ks = a.ksplit > 1 ? a.ksplit : 1;
  if (ks > 8) return hipErrorInvalidValue;
  const int nblk = a.tq * a.batch * a.heads * ks;
  hipLaunchKernelGGL((fwd_kernel<D, F32>), dim3(nblk), dim3(NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  const int64_t n = (int64_t)a.batch * a.heads * a.seq_q * (D / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (ks) {
    case 2: hipLaunchKernelGGL((fwd_merge_kernel<D, F32, 2>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((fwd_merge_kernel<D, F32, 3>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((fwd_merge_kernel<D, F32, 4>), grid, dim3(256), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((fwd_merge_kernel<D, F32, 5>), grid, dim3(256), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((fwd_merge_kernel<D, F32, 6>), grid, dim3(256), 0, stream, a); break;
    case 7: hipLaunchKernelGGL((fwd_merge_kernel<D, F32, 7>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((fwd_merge_kernel<D, F32, 8>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool f32, hipStream_t stream) {
  if (head_dim == 128) return f32 ? launch_fwd_t<128, true>(a, stream) : launch_fwd_t<128, false>(a, stream);
  return f32 ? launch_fwd_t<64, true>(a, stream) : launch_fwd_t<64, false>(a, stream);
}

}  // namespace fm
