// Backward kernels: exact gradients of masked attention.
//
// "FlashAttention-2 ... GPU work partitioning" (iplexlaw.co.kr), section
// "Block processing keeps the global normalization": outputs and gradients
// are those of exact attention and are checked with tolerances. The
// gradients recompute the probabilities from the saved logsumexp instead of
// storing them (no score matrix in HBM):
//   P  = exp(scale * Q K^T - LSE)  (0 on masked pairs)
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),  D = rowsum(dO * O)
//   dK = scale * dS^T Q,   dQ = scale * dS K.
// Section "Three ways to raise GPU utilization": work is split over batch,
// heads and sequence tiles, and each wavefront owns its own output rows.
//
// Kernels (the row pass D = rowsum(dO * O) runs with the pre-passes):
//   bwd_dkdv  one workgroup per (batch, head, 128-key tile) with K and V in
//             LDS; each pair of wavefronts owns 32 keys, forms S and dP for
//             half the rows of every non-SKIP 64-row query tile each, and one
//             accumulates dV, the other dK, in registers;
//   bwd_dq    one workgroup per (batch, head, 128-row query tile); each
//             wavefront owns 32 query rows whose Q, dO, LSE, D stay in
//             registers and whose dQ accumulates over all non-SKIP 64-key
//             tiles. It recomputes S and dP (two extra matrix products) so
//             that no workgroup ever adds into another one's output: no
//             atomics, deterministic results.
#include <climits>
#include <cstddef>
#include <type_traits>
#include <cmath>

#include "fm_device.hpp"
#include "fm_internal.hpp"
#include "fm_tile.hpp"

namespace fm {
namespace {

constexpr int NW = 4;            // wavefronts per workgroup
constexpr int NT = NW * 64;      // threads per workgroup
constexpr int LIST_CAP = 1024;   // class bytes compacted per pass (4 per thread)

// ------------------------------------------------------------------ dK / dV
// One workgroup per (batch, K/V head, 128-key tile), eight wavefronts, two per
// SIMD. Wavefronts w and w + 4 (one SIMD) own keys 32 (w % 4) .. + 31 of the
// tile and split the products of every non-SKIP 64-row query tile by kind:
//   the P wavefront (w < 4) holds its keys' K rows in registers, forms
//     S = Q K^T and P for all 64 rows, hands the bf16 P to its partner through
//     LDS and accumulates dV^T += dO^T P;
//   the dS wavefront (w >= 4) holds its keys' V rows in registers and works
//     one query tile behind: dP = dO V^T of the previous tile, dS = P (dP - D)
//     with the P handed over one iteration earlier, dK^T += Q^T dS (and the
//     dS tile to HBM when dQ is formed from it).
// With K and V in registers only Q and dO are read from LDS (each once as
// rows and once transposed per wavefront pair), and working one tile behind
// frees the dS wavefront from waiting for its partner's exponentials, so the
// two wavefronts of a SIMD overlap their matrix products with each other's
// vector work. Three query tiles live in LDS: the P wavefronts' current one,
// the dS wavefronts' previous one, and the next one loading.
namespace kv {
constexpr int BQ = kBwdBlockQ;   // 64 query rows per inner tile
constexpr int BK = kBwdBlockK;   // 128 keys per workgroup
constexpr int WAVES = 8;         // 4 key groups x (P, dS)
constexpr int THREADS = WAVES * 64;
constexpr int NBUF = 3;          // query tiles in LDS
constexpr int QCAP = kBwdListCap;   // query tiles compacted per list pass (2 per thread)
constexpr int kZeroShare = 4;    // empty lines written per workgroup with work, at most

template <int D>
struct alignas(16) Smem {
  uint16_t q[NBUF][BQ * D];      // query tiles, row-major, swizzled
  uint16_t dout[NBUF][BQ * D];   // dO tiles
  float lse2[NBUF][BQ];          // LSE * log2(e); +inf for rows that see nothing / past the end
  float dd[NBUF][BQ];            // D = rowsum(dO * O)
  uint32_t list[QCAP];
  uint16_t rank[QCAP];           // ascending rank of each list entry (stored-dS slot)
  // per key group, two buffers of 4 KiB: the bf16 P of one query tile (64 rows
  // x 32 keys in MFMA operand order), then the dS wavefront's store staging
  uint16_t xch[4][2][BQ * 32];
  int32_t scan[WAVES];
};
}  // namespace kv

// GROUPED: more than one query head per K/V head. The head loop runs the
// group's a.group heads, or only the workgroup's own head with split heads
// (a.part set); without GROUPED it has one trip and folds away.
template <int D, bool F32, bool GROUPED>
__global__ __launch_bounds__(kv::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(BwdArgs a) {
  using namespace kv;
  constexpr int KSTEPS = D / 16;
  constexpr int CB = D / 32;
  constexpr int QR = (BQ * D / 8) / THREADS;   // 16-byte chunks per thread of a float32 Q (or dO) tile
  __shared__ Smem<D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int kg = __builtin_amdgcn_readfirstlane(w & 3);          // key group
  const bool is_p = __builtin_amdgcn_readfirstlane(w >> 2) == 0;  // P wavefront (else dS wavefront)
  const int l = tid & 63;
  const int lr = l & 31;
  const int g = l >> 5;

  // Key tiles longest first, then the (b, K/V head) pairs sharing the K/V
  // mask row; the workgroup runs the `group` query heads of its K/V head one
  // after the other, with dK, dV accumulating over all of them.
  // With split heads (a.part set; a mask shared by all heads), each of the
  // `group` query heads of a K/V head has a workgroup of its own, which writes
  // float32 partial dK, dV that a second kernel sums.
  const int split = GROUPED && a.part != nullptr;
  const int rep = split ? a.rep_kv * a.group : a.rep_kv;
  const uint32_t ent = (uint32_t)__builtin_amdgcn_readfirstlane(a.order_k[blockIdx.x / rep]);
  // A line whose key tile no query tile sees (flagged by the order sort, which
  // puts those lines last): its dK and dV are zero. The first kZeroShare
  // workgroups' worth of them are written by the workgroups with work (each
  // takes up to kZeroShare, strided), so that the stores drain while those
  // run; the workgroups of such lines end at once. Any others write their own.
  const int64_t busy = (int64_t)__builtin_amdgcn_readfirstlane(*a.order_live) * rep;
  const int64_t zeros = min((int64_t)gridDim.x - busy, kZeroShare * busy);   // lines zeroed by others
  const bool empty = (ent & kEmptyLine) != 0;
  if (empty && (int64_t)blockIdx.x - busy < zeros) return;
  const int line = (int)(ent & ~kEmptyLine);   // K/V mask row * tk + key tile
  // (by launch position, so that it loads beside the order entry; without a
  // head loop the line is also the class column's mask row and key tile)
  const int first_q =
      !GROUPED && a.first_k != nullptr ? __builtin_amdgcn_readfirstlane(a.first_k[blockIdx.x / rep]) : -1;
  // (integer divisions by launch constants expand to vector code: the results
  // are taken back to scalar registers so that the addresses stay scalar)
  const int kt = __builtin_amdgcn_readfirstlane(line % a.tk);
  const int kr = __builtin_amdgcn_readfirstlane(line / a.tk);
  const int hkm = a.mask.hm > 1 ? a.heads_kv : 1;   // K/V mask rows per batch row
  const int jr = __builtin_amdgcn_readfirstlane((blockIdx.x % rep) / (split ? a.group : 1));
  const int gsel = __builtin_amdgcn_readfirstlane(split ? blockIdx.x % a.group : 0);   // the head (split heads)
  const int b = __builtin_amdgcn_readfirstlane(a.mask.bm > 1 ? kr / hkm : jr / (a.mask.hm > 1 ? 1 : a.heads_kv));
  const int hk = __builtin_amdgcn_readfirstlane(a.mask.hm > 1 ? kr % hkm : jr % a.heads_kv);
  const int bm = __builtin_amdgcn_readfirstlane(kr / hkm);
  constexpr int ES = F32 ? 4 : 2;

  // workgroup i with work writes the zeros of the empty workgroups busy + j,
  // j = i, i + busy, ... below zeros: dK then dV rows of the line's 128 keys,
  // 16 bytes per lane
  for (int64_t j = blockIdx.x; j < zeros; j += busy) {
    const int64_t wg = busy + j;
    const int zl = (int)((uint32_t)__builtin_amdgcn_readfirstlane(a.order_k[wg / rep]) & ~kEmptyLine);
    const int zkt = __builtin_amdgcn_readfirstlane(zl % a.tk);
    const int zkr = __builtin_amdgcn_readfirstlane(zl / a.tk);
    const int zjr = __builtin_amdgcn_readfirstlane((int)((wg % rep) / (split ? a.group : 1)));
    const int zg = __builtin_amdgcn_readfirstlane(split ? (int)(wg % a.group) : 0);
    const int zb = __builtin_amdgcn_readfirstlane(a.mask.bm > 1 ? zkr / hkm : zjr / (a.mask.hm > 1 ? 1 : a.heads_kv));
    const int zh = __builtin_amdgcn_readfirstlane(a.mask.hm > 1 ? zkr % hkm : zjr % a.heads_kv);
    const int lc = split ? __builtin_ctz(D * 4 / 16) : __builtin_ctz(D * ES / 16);   // log2 of chunks per row
    for (int c = tid; c < (2 * BK) << lc; c += THREADS) {
      const int row = c >> lc, ch = c & ((1 << lc) - 1);
      const bool is_k = row < BK;
      const int nz = zkt * BK + (row & (BK - 1));
      if (nz >= a.seq_k) continue;
      char* out;
      if (split) {   // float32 partials [2][B][H][Sk][D]: dK, then dV
        out = reinterpret_cast<char*>(a.part + (is_k ? 0 : (int64_t)a.batch * a.heads * a.seq_k * D) +
                                      (((int64_t)zb * a.heads + zh * a.group + zg) * a.seq_k + nz) * D);
      } else {
        const int64_t off = is_k ? (int64_t)zb * a.k_sb + (int64_t)nz * a.k_ss + (int64_t)zh * a.k_sh
                                 : (int64_t)zb * a.v_sb + (int64_t)nz * a.v_ss + (int64_t)zh * a.v_sh;
        out = reinterpret_cast<char*>(is_k ? a.dk : a.dv) + off * ES;
      }
      *reinterpret_cast<u32x4*>(out + 16 * ch) = u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int n = kt * BK + 32 * kg + lr;   // this lane's key
  const bool key_ok = n < a.seq_k;
  const bool ragged_k = (a.seq_k % BK) != 0 && kt == a.tk - 1;
  const bool store_ds = a.plan != nullptr && a.plan[1] != 0;

  // ---- the lane's key row as MFMA B operands, once: K for the P wavefront,
  // V for the dS wavefront, channels 16 s + 8 g .. + 7 in step s (keys past
  // the end re-read the last key; their pairs are masked) ----
  u32x4 kvf[KSTEPS];
  {
    const int nn = min(n, a.seq_k - 1);
    const int64_t off = is_p ? (int64_t)b * a.k_sb + (int64_t)nn * a.k_ss + (int64_t)hk * a.k_sh + 8 * g
                             : (int64_t)b * a.v_sb + (int64_t)nn * a.v_ss + (int64_t)hk * a.v_sh + 8 * g;
    const void* src = is_p ? a.k : a.v;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) kvf[s] = load8_as_bf16<F32>(src, off + 16 * s);
  }
  if (empty) {   // dK = dV = 0 for this tile's keys: no list, bounds or tiles
    if (!key_ok) return;
    const bool is_k = !is_p;
    if (split) {   // float32 partials [2][B][H][Sk][D]: dK, then dV
      float* out = a.part + (is_k ? 0 : (int64_t)a.batch * a.heads * a.seq_k * D) +
                   (((int64_t)b * a.heads + hk * a.group + gsel) * a.seq_k + n) * D;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) *reinterpret_cast<f32x4*>(out + 8 * c + 4 * g) = f32x4{};
    } else {
      const int64_t off = is_k ? (int64_t)b * a.k_sb + (int64_t)n * a.k_ss + (int64_t)hk * a.k_sh
                               : (int64_t)b * a.v_sb + (int64_t)n * a.v_ss + (int64_t)hk * a.v_sh;
      char* out = reinterpret_cast<char*>(is_k ? a.dk : a.dv) + off * ES;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        if constexpr (F32) *reinterpret_cast<f32x4*>(out + (8 * c + 4 * g) * 4) = f32x4{};
        else *reinterpret_cast<u32x2*>(out + (8 * c + 4 * g) * 2) = u32x2{0u, 0u};
      }
    }
    return;
  }

  // Per query head (set at the start of each head): the lane's key bounds
  // and interval widths, the class column, the stored-dS slot base and
  // stream, the LSE / D rows and the Q / dO bases.
  int h = 0;
  uint32_t b_lw = 0, b_uw = 0;
  int32_t b_lts = 0, b_uts = 0;
  const uint8_t* ccol = nullptr;
  int64_t slot0 = 0, lrow = 0;
  uint16_t* ds_rep = nullptr;
  f32x16 acc[CB];   // dV^T (P wavefront) or dK^T (dS wavefront) of the wavefront's keys
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  const float C = a.scale_log2;

  // ---- query tile staging ----
  // Q and dO (bf16) and the rows' LSE*log2(e) and D go straight from global
  // memory into LDS one tile ahead of the math; float32 Q and dO pass through
  // registers (rounded to bf16) when their tile is staged. Rows past the end
  // re-read the last row; their LSE*log2(e) is +inf, so P = dS = 0.
  const int64_t q_ld = a.q_ss * ES, o_ld = a.o_ss * ES;
  const char* qbh = nullptr;
  const char* dbh = nullptr;
  using Dma = DmaTile<D, BQ, THREADS>;
  constexpr int NOFF = F32 ? QR : 1;
  uint32_t qoff[NOFF], doff[NOFF];
  if constexpr (F32) {
    tile_offsets<D, F32, QR, THREADS>(qoff, q_ld, tid);
    tile_offsets<D, F32, QR, THREADS>(doff, o_ld, tid);
  } else {
    qoff[0] = Dma::offset(q_ld, tid);
    doff[0] = Dma::offset(o_ld, tid);
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto stage_q = [&](int qt, int buf) {
    const int m0 = qt * BQ;
    if constexpr (F32) {
      u32x4 rq[QR], rd[QR];
      load_tile_rows<D, F32, QR, THREADS>(rq, qbh + m0 * q_ld, qoff, q_ld, tid, a.seq_q - m0);
      load_tile_rows<D, F32, QR, THREADS>(rd, dbh + m0 * o_ld, doff, o_ld, tid, a.seq_q - m0);
      store_tile_rows<D, QR, THREADS>(reinterpret_cast<char*>(sm.q[buf]), rq, tid);
      store_tile_rows<D, QR, THREADS>(reinterpret_cast<char*>(sm.dout[buf]), rd, tid);
    } else {
      Dma::load(reinterpret_cast<char*>(sm.q[buf]), qbh + m0 * q_ld, qoff[0], q_ld, tid, a.seq_q - m0);
      Dma::load(reinterpret_cast<char*>(sm.dout[buf]), dbh + m0 * o_ld, doff[0], o_ld, tid, a.seq_q - m0);
    }
    if (wu == 0) dma4(a.lse2 + lrow + m0, 4u * (uint32_t)l, lds_address(sm.lse2[buf]));
    else if (wu == 1) dma4(a.drow + lrow + m0, 4u * (uint32_t)l, lds_address(sm.dd[buf]));
  };

  // Where the two wavefronts of a SIMD both want the matrix unit, the P
  // wavefront goes first: its exponentials then overlap the other's products.
  if (is_p) __builtin_amdgcn_s_setprio(1);

  // LDS byte offsets of this lane's operand reads within a tile, computed
  // once; the tile's base is added per iteration, row blocks and row steps go
  // into the reads' immediate offsets (none of them changes the swizzle).
  // Row operands (Q for the P wavefront, dO for the dS wavefront) of step s:
  // row lr (+ 32 per row block), channels 16 s + 8 g.
  uint32_t fo[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) fo[s] = (uint32_t)rm_byte<D>(lr, 16 * s + 8 * g);
  // Transposed operands (dO^T for the P wavefront, Q^T for the dS wavefront)
  // of channel block cb: the two 4-row groups of tr_operand() (+ 16 rows per
  // row step).
  uint32_t to[CB][2];
  {
    const int i = l & 15;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int r0 = 4 * g + (i >> 2);
      const int col = 32 * cb + 16 * ((l >> 4) & 1) + 4 * (i & 3);
      to[cb][0] = (uint32_t)rm_byte<D>(r0, col);
      to[cb][1] = (uint32_t)rm_byte<D>(r0 + 8, col);
    }
  }
  // (kept whole: otherwise the compiler splits them into shared parts and
  // adds those again in every tile)
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) asm volatile("" : "+v"(fo[s]));
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    asm volatile("" : "+v"(to[cb][0]));
    asm volatile("" : "+v"(to[cb][1]));
  }
  constexpr uint32_t QTILE = BQ * D * 2;             // bytes per Q (or dO) tile
  constexpr uint32_t DOUT = NBUF * QTILE;            // sm.dout[0] - sm.q[0]
  constexpr uint32_t RB = 32 * 2 * D;                // bytes of 32 tile rows
  static_assert(offsetof(Smem<D>, dout) - offsetof(Smem<D>, q) == DOUT, "tile layout");
  static_assert(DOUT + QTILE <= 65536, "immediate offsets");
  const uint32_t q0 = lds_address(sm.q[0]);
  char* xgrp = reinterpret_cast<char*>(sm.xch[kg]);

  // One query tile of this wavefront's role: entry list[e] in LDS buffer
  // buf, its P in xch[kg][par], its stored-dS slot (dS wavefront, storing).
  // Both roles run the same products on different operands, so that the
  // accumulators stay in place; only the vector work between the products
  // differs by role.
  auto work = [&](auto masked_c, int e, int buf, int par, int64_t slot) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const uint32_t tile = q0 + (uint32_t)buf * QTILE;
    const uint32_t fbase = tile + (is_p ? 0u : DOUT);   // rows: Q (P) or dO (dS)
    const uint32_t tbase = tile + (is_p ? DOUT : 0u);   // transposed: dO^T (P) or Q^T (dS)
    char* xp = xgrp + par * (BQ * 32 * 2);

    // S (P wavefront) or dP (dS wavefront) for the tile's 64 rows x the
    // wavefront's 32 keys: row operands from LDS, the key operands in
    // registers (lane = key, registers = rows). Operands read three MFMAs
    // ahead.
    f32x16 sp[2] = {f32x16{}, f32x16{}};
    {
      constexpr int NJ = 2 * KSTEPS;   // (step, row block)
      u32x4 op[NJ];
      auto rd = [&](int j) { op[j] = lds16(fo[j >> 1] + fbase, (j & 1) * RB); };
#pragma unroll
      for (int j = 0; j < 3; ++j) rd(j);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j + 3 < NJ) rd(j + 3);
        sp[j & 1] = mfma32(op[j], kvf[j >> 1], sp[j & 1]);
      }
      sched_lds_mfma<NJ, 1, 3>();
      __builtin_amdgcn_sched_barrier(0);
    }

    // The transposed operands of the first three column products, read
    // before the vector work so that it covers their latency.
    constexpr int NS = 4 * CB;   // (row step, channel block)
    u32x4 ta[NS];
    auto tread = [&](int j) {
      const int t = j / CB, cb = j % CB;
      const u32x2 x = lds_tr16(to[cb][0] + tbase, t * 16 * 2 * D);
      const u32x2 y = lds_tr16(to[cb][1] + tbase, t * 16 * 2 * D);
      ta[j] = u32x4{x[0], x[1], y[0], y[1]};
    };
#pragma unroll
    for (int j = 0; j < 3; ++j) tread(j);
    __builtin_amdgcn_sched_barrier(0);

    u32x4 bop[4];   // B operands of the column products, one per 16-row step
    if (is_p) {
      // P = exp2(S * scale * log2(e) - LSE * log2(e)), 0 on masked pairs
      const int m0 = (int)(sm.list[e] & ~kPartialBit) * BQ;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int ml = 32 * rb + 8 * q4 + 4 * g;
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][ml]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * q4 + r;
            float p = fast_exp2(fmaf(sp[rb][i], C, -l2[r]));
            if constexpr (MASKED) {
              const uint32_t mm = (uint32_t)(m0 + ml + r);
              const bool mk = (mm - (uint32_t)b_lts < b_lw) | (mm - (uint32_t)b_uts < b_uw);
              p = mk ? 0.f : p;
            }
            sp[rb][i] = p;
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) bop[2 * rb + t][j] = pack_bf16(sp[rb][8 * t + 2 * j], sp[rb][8 * t + 2 * j + 1]);
      }
      // hand P over (lane-linear, 1 KiB per row step)
#pragma unroll
      for (int t = 0; t < 4; ++t) *reinterpret_cast<u32x4*>(xp + (t * 64 + l) * 16) = bop[t];
    } else {
      // dS = P (dP - D), with the bf16 P the dV product used
      u32x4 pr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) pr[t] = *reinterpret_cast<const u32x4*>(xp + (t * 64 + l) * 16);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int ml = 32 * rb + 8 * q4 + 4 * g;
          const f32x4 dd = *reinterpret_cast<const f32x4*>(&sm.dd[buf][ml]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * q4 + r;
            const uint32_t wd = pr[2 * rb + i / 8][(i % 8) / 2];
            const float p = (i & 1) ? bf16_hi(wd) : bf16_lo(wd);
            sp[rb][i] = p * (sp[rb][i] - dd[r]);
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) bop[2 * rb + t][j] = pack_bf16(sp[rb][8 * t + 2 * j], sp[rb][8 * t + 2 * j + 1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // dV^T += dO^T P (P wavefront) or dK^T += Q^T dS (dS wavefront) over the
    // 64 rows; transposed operands three MFMAs ahead.
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j + 3 < NS) tread(j + 3);
      acc[j % CB] = mfma32(ta[j], bop[j / CB], acc[j % CB]);
    }
#pragma unroll
    for (int j = 0; j < NS - 3; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    __builtin_amdgcn_sched_barrier(0);

    if (!is_p && store_ds) {   // 4 stores per lane, counted by the wait at the top of the next iteration
      // The stored tile is 16 MFMA operand fragments of 1 KiB, fragment
      // (rb, s) = query rows 32 rb .. 32 rb + 31 x keys 16 s .. 16 s + 15.
      // Lane L's 16 bytes at L * 16 hold the row of fragment column
      // c = L % 32 (row 32 rb + 16 c[3] + 8 j[2] + 4 c[4] + j[1:0] for
      // element j's half, the order in which the accumulator holds rows) and
      // keys 16 s + 4 h + 0..3, 16 s + 8 + 4 h + 0..3 (h = L / 32), the
      // order in which the dQ kernel's transposing K^T reads take the keys.
      // The wavefront's 32 keys are fragments (rb, 2 kg) and (rb, 2 kg + 1).
      // They go through the LDS buffer P came in (P is in registers now) as
      // two row-major [key][column] tiles; transposing reads of them yield
      // whole fragment lanes, so each non-temporal store writes one
      // contiguous KiB. LDS accesses of one wavefront execute in order.
      // The tiles' 64-byte rows keep 16-byte chunk c of row r at c ^ sw(r),
      // sw(r) = (r[2], r[1] ^ r[3]): each 8 consecutive rows of a 16-byte
      // write (lane = row) then cover 128 distinct bytes modulo 128, and each
      // 16 consecutive rows 256 modulo 256, and a transposing read of four
      // rows covers one 256-byte block. (Chunk c ^ r[3:2], the swizzle of the
      // 64-byte rows elsewhere, puts rows r and r + 2 in the same banks of
      // such a write: 4.4e7 conflict cycles at 128K document-causal.)
      auto sbyte = [](int r, int col) {
        const int sw = (((r >> 2) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1);
        return r * 64 + (((col >> 3) ^ sw) << 4) + ((col & 7) << 1);
      };
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          *reinterpret_cast<u32x4*>(xp + rb * 2048 + sbyte(lr, 8 * (2 * g + t))) = bop[2 * rb + t];
      char* dst = reinterpret_cast<char*>(ds_rep + slot * (BK * BQ));
      const int i16 = l & 15;
      const int col = 16 * ((l >> 4) & 1) + 4 * (i16 & 3);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int sp2 = 0; sp2 < 2; ++sp2) {
          const int r0 = 16 * sp2 + 4 * g + (i16 >> 2);
          const u32x2 x = tr16(xp + rb * 2048, sbyte(r0, col));
          const u32x2 y = tr16(xp + rb * 2048, sbyte(r0 + 8, col));
          __builtin_nontemporal_store(u32x4{x[0], x[1], y[0], y[1]},
                                      reinterpret_cast<u32x4*>(dst + (rb * 8 + 2 * kg + sp2) * 1024 + l * 16));
        }
    }
  };

  int it_global = 0;   // iteration count over heads and passes (selects the LDS buffers)
  const int ngroup = GROUPED ? a.group : 1;
  for (int gi = gsel; gi < (split ? gsel + 1 : ngroup); ++gi) {
    h = hk * ngroup + gi;
    {
      const int hm = a.mask.hm > 1 ? h : 0;
      const int64_t mbase = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
      const int mrow = bm * a.mask.hm + hm;
      ccol = a.classes_t + ((int64_t)mrow * a.tk + kt) * a.tq;
      // The lane's key bounds (keys past the end are masked for every row) and
      // interval widths (0 for empty intervals): row mm is masked by [s, e) iff
      // (uint)mm - (uint)s < width (modulo 2^32, so no signed overflow), exact
      // for every int32 s, e.
      int32_t lte = INT_MAX, ute = 0;
      b_lts = INT_MIN;
      b_uts = 0;
      if (key_ok) {
        b_lts = a.mask.has_lower ? a.mask.lts[mbase + n] : a.seq_q;
        lte = a.mask.has_lower ? a.mask.lte[mbase + n] : a.seq_q;
        b_uts = a.mask.has_upper ? a.mask.uts[mbase + n] : 0;
        ute = a.mask.has_upper ? a.mask.ute[mbase + n] : 0;
      }
      b_lw = lte > b_lts ? (uint32_t)lte - (uint32_t)b_lts : 0u;
      b_uw = ute > b_uts ? (uint32_t)ute - (uint32_t)b_uts : 0u;
      // Stored dS: when the plan enables it, every processed tile's bf16 dS goes
      // to slot row_off[mask row][kt] + (rank of its query tile among this key
      // tile's non-SKIP ones) of the (b, h) pair's tile stream.
      if (store_ds) {
        const int rep_i = (a.mask.bm > 1 ? 0 : b) * (a.mask.hm > 1 ? 1 : a.heads) + (a.mask.hm > 1 ? 0 : h);
        slot0 = a.row_off[(int64_t)mrow * a.tk + kt];
        ds_rep = a.ds + (int64_t)rep_i * a.plan[0] * (BK * BQ);
      }
      lrow = ((int64_t)b * a.heads + h) * a.seq_pad;
      qbh = reinterpret_cast<const char*>(a.q) + ((int64_t)b * a.q_sb + (int64_t)h * a.q_sh) * ES;
      dbh = reinterpret_cast<const char*>(a.dout) + ((int64_t)b * a.o_sb + (int64_t)h * a.o_sh) * ES;
    }
    const int head_base = it_global;   // non-SKIP tiles of earlier heads
    // Without a head loop, the first list entry is known from the class map
    // pass: its tile loads go out before the list is compacted.
    bool prestaged = false;
    if constexpr (!GROUPED) {
      if (first_q >= 0) {
        stage_q(first_q, it_global % NBUF);
        prestaged = true;
      }
    }
    for (int qt0 = 0; qt0 < a.tq; qt0 += QCAP) {
      int n_full;
      const int n_list = compact_classes_split<QCAP, THREADS>(ccol, qt0, min(QCAP, a.tq - qt0), sm.list,
                                                              sm.rank, sm.scan, tid, ragged_k, &n_full);
      if (n_list == 0) continue;
      const int base = it_global;
      const int pass_base = base - head_base;   // this head's non-SKIP tiles in earlier passes
      if (!prestaged) stage_q((int)(sm.list[0] & ~kPartialBit), base % NBUF);
      prestaged = false;

      // Iteration it: the P wavefronts take list entry it, the dS wavefronts
      // entry it - 1. FULL entries come first, then PARTIAL ones (only the P
      // wavefronts evaluate the mask); the first iteration has work for the P
      // wavefronts alone and one more at the end for the dS wavefronts alone.
      auto top = [&](int it) {
        // This tile's loads done (and, at a pass's first tile, the key rows).
        // Younger vector-memory operations that may stay in flight: the dS
        // wavefront's stores of the previous iteration (vmcnt counts stores).
        if (!is_p && store_ds && it >= 2) wait_vmem_le<4>();
        else wait_vmem();
        // the tile visible to all, the P handed over last iteration too; the
        // buffer of entry it - 2 is free
        __syncthreads();
        if (it + 1 < n_list) stage_q((int)(sm.list[it + 1] & ~kPartialBit), (base + it + 1) % NBUF);
      };
      auto run = [&](auto masked_c, int it) {
        const int e = is_p ? it : it - 1;
        work(masked_c, e, (base + e) % NBUF, (base + e) & 1,
             !is_p && store_ds ? slot0 + pass_base + sm.rank[e] : 0);
      };
      top(0);
      if (is_p) {
        if (n_full > 0) run(std::false_type{}, 0);
        else run(std::true_type{}, 0);
      }
      int it = 1;
      for (; it < n_full; ++it) {
        top(it);
        run(std::false_type{}, it);
      }
      for (; it < n_list; ++it) {
        top(it);
        run(std::true_type{}, it);
      }
      top(it);
      if (!is_p) run(std::false_type{}, it);
      it_global += n_list;
    }
  }
  if (is_p) __builtin_amdgcn_s_setprio(0);
  // A key tile that no query tile sees skips the loop above with its key row
  // loads possibly still in flight: they land before the workgroup ends.
  wait_vmem();

  // ---- epilogue: dV = dV^T (P wavefront), dK = scale * dK^T (dS wavefront),
  // transposed back on store ----
  if (key_ok && split) {   // float32 partials [2][B][H][Sk][D]: dK, then dV
    const bool is_k = !is_p;
    float* out = a.part + (is_k ? 0 : (int64_t)a.batch * a.heads * a.seq_k * D) +
                 (((int64_t)b * a.heads + hk * a.group + gsel) * a.seq_k + n) * D;
    const float sc = is_k ? a.scale : 1.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(out + 32 * cb + 8 * q4 + 4 * g) =
            f32x4{acc[cb][4 * q4] * sc, acc[cb][4 * q4 + 1] * sc, acc[cb][4 * q4 + 2] * sc, acc[cb][4 * q4 + 3] * sc};
  } else if (key_ok) {
    const bool is_k = !is_p;
    const int64_t off = is_k ? (int64_t)b * a.k_sb + (int64_t)n * a.k_ss + (int64_t)hk * a.k_sh
                             : (int64_t)b * a.v_sb + (int64_t)n * a.v_ss + (int64_t)hk * a.v_sh;
    void* out = is_k ? a.dk : a.dv;
    const float sc = is_k ? a.scale : 1.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = 32 * cb + 8 * q4 + 4 * g;
        const float x0 = acc[cb][4 * q4] * sc, x1 = acc[cb][4 * q4 + 1] * sc;
        const float x2 = acc[cb][4 * q4 + 2] * sc, x3 = acc[cb][4 * q4 + 3] * sc;
        if constexpr (F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off + c0) = f32x4{x0, x1, x2, x3};
        } else {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + off + c0) =
              u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
        }
      }
    }
  }
}

// ------------------------------------------------------------------ dQ
namespace dqk {
constexpr int BQ = kDqBlockQ;   // 128 query rows per workgroup (32 per wavefront)
constexpr int BK = kDqBlockK;   // 64 keys per inner tile

template <int D>
struct alignas(16) Smem {
  uint16_t k[2][BK * D];      // double-buffered key tile, row-major
  uint16_t v[2][BK * D];      // double-buffered value tile, row-major
  int32_t bnd[2][4][BK];      // lts, lte, uts, ute of the tile's keys
  uint32_t list[LIST_CAP];
  int32_t scan[NW];
};
}  // namespace dqk

template <int D, bool F32>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdArgs a) {
  using namespace dqk;
  if (a.plan != nullptr && a.plan[1] != 0) return;   // dQ comes from the stored dS instead
  constexpr int KSTEPS = D / 16;
  constexpr int CB = D / 32;
  constexpr int NB = BK / 32;
  constexpr int KR = (BK * D / 8) / NT;   // 16-byte chunks per thread of a K (or V) tile
  __shared__ Smem<D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 31;
  const int g = l >> 5;

  // Query tiles longest first, then the (b, h) pairs sharing the mask row;
  // without an order, later tiles first with heads interleaved.
  int qt, mr, b, h;
  if (a.order_qq != nullptr) {
    const int line = __builtin_amdgcn_readfirstlane(a.order_qq[blockIdx.x / a.rep]);   // mask row * tq_q + tile
    qt = line % a.tq_q;
    mr = line / a.tq_q;
    ordered_bh(mr, blockIdx.x % a.rep, a.mask, a.heads, &b, &h);
  } else {
    const int nbh = a.batch * a.heads;
    qt = a.tq_q - 1 - (int)(blockIdx.x / nbh);
    b = (blockIdx.x % nbh) / a.heads;
    h = (blockIdx.x % nbh) % a.heads;
    mr = (a.mask.bm > 1 ? b : 0) * a.mask.hm + (a.mask.hm > 1 ? h : 0);
  }
  const int bm = mr / a.mask.hm;
  const int hm = mr % a.mask.hm;
  const int64_t mbase = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const uint8_t* crow = a.classes_q + ((int64_t)(bm * a.mask.hm + hm) * a.tq_q + qt) * a.tk_q;

  const int m = qt * BQ + 32 * w + lr;   // this lane's query row
  const bool row_ok = m < a.seq_q;

  // Q and dO rows of this lane's query as MFMA B operands; its LSE and D.
  // (rows past the end re-read the last row; their results are never stored)
  u32x4 qf[KSTEPS], df[KSTEPS];
  float l2 = INFINITY, dd = 0.f;
  {
    const int mq = min(m, a.seq_q - 1);
    const int64_t qoff = (int64_t)b * a.q_sb + (int64_t)mq * a.q_ss + (int64_t)h * a.q_sh + 8 * g;
    const int64_t doff = (int64_t)b * a.o_sb + (int64_t)mq * a.o_ss + (int64_t)h * a.o_sh + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qf[s] = load8_as_bf16<F32>(a.q, qoff + 16 * s);
      df[s] = load8_as_bf16<F32>(a.dout, doff + 16 * s);
    }
    const int64_t lrow = ((int64_t)b * a.heads + h) * a.seq_pad + m;   // m < Sp
    l2 = a.lse2[lrow];
    dd = a.drow[lrow];
  }

  f32x16 dqacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) dqacc[cb] = f32x16{};
  const float C = a.scale_log2;
  const bool ragged_k = (a.seq_k % BK) != 0;

  // ---- key tile staging (K, V; bounds through registers) ----
  // bf16: straight from global memory into LDS; float32: through registers,
  // rounded to bf16 on the way.
  constexpr int ES = F32 ? 4 : 2;
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
  auto load_k = [&](int kt, bool masked, int buf) {
    const int n0 = kt * BK;
    if constexpr (F32) {
      load_tile_rows<D, F32, KR, NT>(rk, kbh + n0 * k_ld, koff, k_ld, tid, a.seq_k - n0);
      load_tile_rows<D, F32, KR, NT>(rv, vbh + n0 * v_ld, voff, v_ld, tid, a.seq_k - n0);
    } else {
      Dma::load(reinterpret_cast<char*>(sm.k[buf]), kbh + n0 * k_ld, koff[0], k_ld, tid, a.seq_k - n0);
      Dma::load(reinterpret_cast<char*>(sm.v[buf]), vbh + n0 * v_ld, voff[0], v_ld, tid, a.seq_k - n0);
    }
    if (masked && tid < BK) {
      const int nn = n0 + tid;
      if (nn < a.seq_k) {
        rb[0] = a.mask.has_lower ? a.mask.lts[mbase + nn] : a.seq_q;
        rb[1] = a.mask.has_lower ? a.mask.lte[mbase + nn] : a.seq_q;
        rb[2] = a.mask.has_upper ? a.mask.uts[mbase + nn] : 0;
        rb[3] = a.mask.has_upper ? a.mask.ute[mbase + nn] : 0;
      } else {   // keys past the end: masked for every row
        rb[0] = INT_MIN;
        rb[1] = INT_MAX;
        rb[2] = 0;
        rb[3] = 0;
      }
    }
  };
  auto store_k = [&](int buf, bool masked) {
    if constexpr (F32) {
      store_tile_rows<D, KR, NT>(reinterpret_cast<char*>(sm.k[buf]), rk, tid);
      store_tile_rows<D, KR, NT>(reinterpret_cast<char*>(sm.v[buf]), rv, tid);
    }
    if (masked && tid < BK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.bnd[buf][j][tid] = rb[j];
    }
  };
  auto masked_of = [&](uint32_t ent) {
    return (ent & kPartialBit) || (ragged_k && (int)(ent & ~kPartialBit) == a.tk_q - 1);
  };

  int it_global = 0;
  for (int kt0 = 0; kt0 < a.tk_q; kt0 += LIST_CAP) {
    const int n_list = compact_classes<LIST_CAP, NT>(crow, kt0, min(LIST_CAP, a.tk_q - kt0), sm.list, sm.scan, tid);
    if (n_list == 0) continue;

    uint32_t ent = sm.list[0];
    load_k((int)(ent & ~kPartialBit), masked_of(ent), it_global & 1);

    for (int it = 0; it < n_list; ++it, ++it_global) {
      const int buf = it_global & 1;
      const bool masked_tile = masked_of(ent);
      store_k(buf, masked_tile);
      wait_vmem();
      __syncthreads();   // tile `buf` complete and visible; the other buffer is free
      if (it + 1 < n_list) {   // the next key tile's loads overlap this tile's math
        ent = sm.list[it + 1];
        load_k((int)(ent & ~kPartialBit), masked_of(ent), buf ^ 1);
      }
      const char* kb = reinterpret_cast<const char*>(sm.k[buf]);
      const char* vb = reinterpret_cast<const char*>(sm.v[buf]);

      // ---- S^T = K Q^T and dP^T = V dO^T (lane = query row, registers = keys) ----
      f32x16 sacc[NB], dpacc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sacc[nb] = f32x16{};
        dpacc[nb] = f32x16{};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const int off = rm_byte<D>(32 * nb + lr, 16 * s + 8 * g);
          sacc[nb] = mfma32(*reinterpret_cast<const u32x4*>(kb + off), qf[s], sacc[nb]);
          dpacc[nb] = mfma32(*reinterpret_cast<const u32x4*>(vb + off), df[s], dpacc[nb]);
        }
      }
      sched_lds_mfma<2 * NB * KSTEPS, 1, 4>();

      // ---- P and dS for this lane's row ----
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          i32x4 l0, l1, u0, u1;
          if (masked_tile) {
            const int nl = 32 * nb + 8 * q4 + 4 * g;   // 4 consecutive keys
            l0 = *reinterpret_cast<const i32x4*>(&sm.bnd[buf][0][nl]);
            l1 = *reinterpret_cast<const i32x4*>(&sm.bnd[buf][1][nl]);
            u0 = *reinterpret_cast<const i32x4*>(&sm.bnd[buf][2][nl]);
            u1 = *reinterpret_cast<const i32x4*>(&sm.bnd[buf][3][nl]);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * q4 + r;
            float p = fast_exp2(fmaf(sacc[nb][i], C, -l2));
            if (masked_tile) {
              const bool mk = ((l0[r] <= m) & (m < l1[r])) | ((u0[r] <= m) & (m < u1[r]));
              p = mk ? 0.f : p;
            }
            dpacc[nb][i] = p * (dpacc[nb][i] - dd);
          }
        }
      }

      // ---- dQ^T += K^T dS^T (contraction over the tile's keys) ----
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 dsp;
#pragma unroll
          for (int j = 0; j < 4; ++j) dsp[j] = pack_bf16(dpacc[nb][8 * t + 2 * j], dpacc[nb][8 * t + 2 * j + 1]);
          const int r0 = 32 * nb + 16 * t + 4 * g;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            dqacc[cb] = mfma32(tr_operand<D>(kb, l, 32 * cb, r0, r0 + 8), dsp, dqacc[cb]);
        }
      }
      sched_lds_mfma<NB * 2 * CB, 2, 3>();
    }
  }

  // ---- epilogue: dQ = scale * dQ^T, transposed back on store ----
  if (row_ok) {
    const int64_t qoff = (int64_t)b * a.q_sb + (int64_t)m * a.q_ss + (int64_t)h * a.q_sh;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = 32 * cb + 8 * q4 + 4 * g;
        const float x0 = dqacc[cb][4 * q4] * a.scale, x1 = dqacc[cb][4 * q4 + 1] * a.scale;
        const float x2 = dqacc[cb][4 * q4 + 2] * a.scale, x3 = dqacc[cb][4 * q4 + 3] * a.scale;
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

// Split heads: dK, dV of K/V head hk = the sum of the float32 partials of its
// `group` query heads; one thread per 4 channels of one key.
template <int D, bool F32>
__global__ __launch_bounds__(256) void kv_reduce_kernel(BwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (b, hk, n, c4)
  const int64_t total = (int64_t)a.batch * a.heads_kv * a.seq_k * (D / 4);
  if (i >= total) return;
  const int c0 = (int)(i % (D / 4)) * 4;
  const int n = (int)((i / (D / 4)) % a.seq_k);
  const int hk = (int)((i / ((int64_t)(D / 4) * a.seq_k)) % a.heads_kv);
  const int b = (int)(i / ((int64_t)(D / 4) * a.seq_k * a.heads_kv));
  const int64_t half = (int64_t)a.batch * a.heads * a.seq_k * D;
#pragma unroll
  for (int kind = 0; kind < 2; ++kind) {   // 0: dK, 1: dV
    f32x4 x = f32x4{};
    for (int gi = 0; gi < a.group; ++gi)
      x += *reinterpret_cast<const f32x4*>(a.part + kind * half +
                                           (((int64_t)b * a.heads + hk * a.group + gi) * a.seq_k + n) * D + c0);
    const int64_t off = kind == 0 ? (int64_t)b * a.k_sb + (int64_t)n * a.k_ss + (int64_t)hk * a.k_sh + c0
                                  : (int64_t)b * a.v_sb + (int64_t)n * a.v_ss + (int64_t)hk * a.v_sh + c0;
    void* out = kind == 0 ? a.dk : a.dv;
    if constexpr (F32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off) = x;
    } else {
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + off) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    }
  }
}

template <int D, bool F32>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t s) {
  if (a.group > 1 && a.part != nullptr) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, F32, true>), dim3(a.tk * a.batch * a.heads), dim3(kv::THREADS), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)a.batch * a.heads_kv * a.seq_k * (D / 4);
    hipLaunchKernelGGL((kv_reduce_kernel<D, F32>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  } else if (a.group > 1) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, F32, true>), dim3(a.tk * a.batch * a.heads_kv), dim3(kv::THREADS), 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, F32, false>), dim3(a.tk * a.batch * a.heads_kv), dim3(kv::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, F32>), dim3(a.tq_q * a.batch * a.heads), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, bool f32, hipStream_t s) {
  if (head_dim == 128) return f32 ? launch_dkdv_t<128, true>(a, s) : launch_dkdv_t<128, false>(a, s);
  return f32 ? launch_dkdv_t<64, true>(a, s) : launch_dkdv_t<64, false>(a, s);
}

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, bool f32, hipStream_t s) {
  if (head_dim == 128) return f32 ? launch_dq_t<128, true>(a, s) : launch_dq_t<128, false>(a, s);
  return f32 ? launch_dq_t<64, true>(a, s) : launch_dq_t<64, false>(a, s);
}

}  // namespace fm
