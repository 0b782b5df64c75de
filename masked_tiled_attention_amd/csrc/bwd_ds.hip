// Backward with stored dS: dQ = scale * dS K.
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
// The slot plan (each non-SKIP tile's slot, the total, and whether the
// workspace holds every tile for every (b, h)) comes from the pre-passes.
// Kernels:
//   dq_ds       one workgroup per (b, h, pair of 64-row query tiles), or per
//               part of the pair's list when few pairs have long key ranges:
//               for each key tile non-SKIP for either, K goes into LDS and
//               each wavefront's stored dS fragments straight into registers,
//               and dQ^T += K^T dS^T accumulates in registers;
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

// ------------------------------------------------------------------ dQ from dS
// One workgroup per (b, h, pair of adjacent 64-row query tiles): four
// wavefronts, wavefront w owning rows 32 w .. 32 w + 31 of the pair (query tile
// w / 2) and all channels. It walks the key tiles that are non-SKIP for either
// query tile of the pair. A stored dS tile is a set of MFMA operand fragments,
// and each fragment is used by exactly one wavefront, so the wavefronts load
// their fragments straight into registers, two key tiles ahead; only the K
// tile, which all four use, is staged in LDS (two buffers).
constexpr int PAIR = 2;   // query tiles per workgroup
constexpr int DS_FRAGS = BK / 16;   // dS fragments per wavefront and key tile

template <int D>
struct alignas(16) DsSmem {
  uint16_t k[2][BK * D];       // key tiles, row-major, swizzled
  uint32_t list[LIST_CAP];     // key tiles of the pair's list
  int32_t slot[LIST_CAP][PAIR];   // stored-dS slot per query tile of the pair; -1: SKIP
  int32_t scan[NW];
};

// The pair's key-tile list: ascending key tiles in [first, first + count)
// that are non-SKIP for either query tile of the pair, with both slots, read
// from the two query tiles' rows of the query-major slot map (row1 == nullptr
// when the pair has one query tile). Starts and ends with a barrier.
__device__ __forceinline__ int compact_pair(const int32_t* row0, const int32_t* row1, int first, int count,
                                            uint32_t* sm_list, int32_t (*sm_slot)[PAIR], int32_t* sm_scan, int tid) {
  constexpr int PER = LIST_CAP / NT;
  const int lane = tid & 63, wave = tid >> 6;
  int32_t sl[PER][PAIR];
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid * PER + e;
    sl[e][0] = idx < count ? row0[first + idx] : -1;
    sl[e][1] = idx < count && row1 ? row1[first + idx] : -1;
    cnt += sl[e][0] >= 0 || sl[e][1] >= 0;
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
    if (sl[e][0] >= 0 || sl[e][1] >= 0) {
      sm_list[pos] = (uint32_t)(first + tid * PER + e);
      sm_slot[pos][0] = sl[e][0];
      sm_slot[pos][1] = sl[e][1];
      ++pos;
    }
  }
  __syncthreads();
  return n_list;
}

template <int D, bool F32>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_ds_kernel(BwdArgs a) {
  if (a.plan == nullptr || a.plan[1] == 0) return;   // dQ comes from the recompute kernel
  constexpr int CB = D / 32;              // 32-channel blocks of dQ^T
  constexpr int KR = (BK * D / 8) / NT;   // 16-byte chunks per thread of a float32 key tile
  constexpr int ES = F32 ? 4 : 2;
  __shared__ DsSmem<D> sm;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int g = l >> 5;
  const int q = w >> 1;        // this wavefront's query tile within the pair
  const int half = w & 1;      // its 32-row half of that tile

  // Later query tiles first, heads interleaved: neighbouring workgroups work
  // on nearby rows and share K tiles in L2 (this kernel is bound by memory
  // traffic, so that beats ordering by length). With one mask row, blocks of
  // 16 pairs (later pairs first within each) launch longest block first, which
  // keeps that sharing within a block and cuts the tail.
  // With split lists (a.dq_split > 1), consecutive workgroups take the
  // parts of one pair's key-tile list and write float32 partial dQ.
  // With a block order (one mask row), launch position p takes block
  // dq_blocks[p / 16] of 16 pairs counted from the last pair, later pairs
  // first within it; the launch is padded to whole blocks.
  const int ks = a.dq_split > 1 ? a.dq_split : 1;
  const int sp = (int)(blockIdx.x % ks);   // this workgroup's part
  const int wg = (int)(blockIdx.x / ks);
  const int nbh = a.batch * a.heads;
  const int npair = (a.tq + PAIR - 1) / PAIR;
  const int pos = wg / nbh;
  int pair = npair - 1 - pos;
  if (a.dq_blocks != nullptr) {
    const int blk = __builtin_amdgcn_readfirstlane(a.dq_blocks[pos / kDqBlockPairs]);
    pair = npair - 1 - kDqBlockPairs * blk - pos % kDqBlockPairs;
    if (pair < 0) return;   // padding of the earliest block
  }
  const int qt0 = PAIR * pair;
  const bool has1 = qt0 + 1 < a.tq;
  const int bh = wg % nbh;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  const int mrow = (a.mask.bm > 1 ? b : 0) * a.mask.hm + (a.mask.hm > 1 ? h : 0);
  const int rep_i = (a.mask.bm > 1 ? 0 : b) * (a.mask.hm > 1 ? 1 : a.heads) + (a.mask.hm > 1 ? 0 : h);
  const int64_t total = __builtin_amdgcn_readfirstlane(a.plan[0]);   // uniform
  // this wavefront's fragments of a stored tile start here (bytes)
  const char* ds_rep = reinterpret_cast<const char*>(a.ds + (int64_t)rep_i * total * (BK * BQ)) +
                       half * (DS_FRAGS * 1024) + l * 16;
  const int32_t* srow0 = a.slots_q + ((int64_t)mrow * a.tq + qt0) * a.tk;
  const int32_t* srow1 = has1 ? srow0 + a.tk : nullptr;

  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};

  // ---- K staging (bf16: direct loads; float32: through registers) ----
  const int64_t k_ld = a.k_ss * ES;
  const char* kbh = reinterpret_cast<const char*>(a.k) +
                    ((int64_t)b * a.k_sb + (int64_t)__builtin_amdgcn_readfirstlane(h / a.group) * a.k_sh) * ES;
  using DmaK = DmaTile<D, BK, NT>;
  constexpr int NOFF = F32 ? KR : 1;
  uint32_t koff[NOFF];
  if constexpr (F32) {
    tile_offsets<D, F32, KR, NT>(koff, k_ld, tid);
  } else {
    koff[0] = DmaK::offset(k_ld, tid);
  }
  auto stage_k = [&](int idx, int buf) {
    const int kt = __builtin_amdgcn_readfirstlane((int)sm.list[idx]);   // uniform
    const int n0 = kt * BK;
    if constexpr (F32) {
      u32x4 rk[KR];
      load_tile_rows<D, F32, KR, NT>(rk, kbh + n0 * k_ld, koff, k_ld, tid, a.seq_k - n0);
      store_tile_rows<D, KR, NT>(reinterpret_cast<char*>(sm.k[buf]), rk, tid);
    } else {
      DmaK::load(reinterpret_cast<char*>(sm.k[buf]), kbh + n0 * k_ld, koff[0], k_ld, tid, a.seq_k - n0);
    }
  };
  // ---- this wavefront's dS fragments of list entry idx, into registers ----
  // Returns whether its query tile has the tile (wavefront-uniform). The loads
  // are issued either way (an absent tile re-reads the other query tile's,
  // which the entry always has), so that every entry issues the same number
  // of loads and the waits below count them exactly.
  u32x4 dsr[3][DS_FRAGS];
  auto load_ds = [&](int idx, u32x4 (&r)[DS_FRAGS]) __attribute__((always_inline)) {
    const int32_t own = __builtin_amdgcn_readfirstlane(sm.slot[idx][q]);
    const int32_t other = __builtin_amdgcn_readfirstlane(sm.slot[idx][q ^ 1]);
    const int64_t slot = own >= 0 ? own : other;
    const char* src = ds_rep + slot * (BK * BQ * 2);
#pragma unroll
    for (int s = 0; s < DS_FRAGS; ++s) r[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + s * 1024));
    return own >= 0;
  };

  // LDS addresses of this lane's two transposing K reads per channel block in
  // buffer 0, first 16-key step. The swizzle depends on the row modulo 16, so
  // step s adds s * 16 rows as an immediate offset and buffer 1 adds one
  // tile. Kept opaque so that the compiler does not rebuild them per read.
  uint32_t ko[CB][2];
  {
    const uint32_t kbase = lds_address(sm.k[0]);
    const int i = l & 15;
    const int r = 4 * g + (i >> 2);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = 32 * cb + 16 * ((l >> 4) & 1) + 4 * (i & 3);
      ko[cb][0] = kbase + (uint32_t)rm_byte<D>(r, col);
      ko[cb][1] = kbase + (uint32_t)rm_byte<D>(r + 8, col);
      asm volatile("" : "+v"(ko[cb][0]));
      asm volatile("" : "+v"(ko[cb][1]));
    }
  }

  // dQ^T (channels x rows) += K^T (channels x keys) dS^T (keys x rows), 16
  // keys per step: K^T read transposed from LDS, dS^T the wavefront's
  // fragment, both with the same key order per lane half.
  auto products = [&](int buf, const u32x4 (&r)[DS_FRAGS]) __attribute__((always_inline)) {
    const uint32_t tb = (uint32_t)buf * (BK * D * 2);
    uint32_t ka[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      ka[cb][0] = ko[cb][0] + tb;
      ka[cb][1] = ko[cb][1] + tb;
    }
#pragma unroll
    for (int s = 0; s < DS_FRAGS; ++s) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const u32x2 x = lds_tr16(ka[cb][0], (uint32_t)s * (16 * 2 * D));
        const u32x2 y = lds_tr16(ka[cb][1], (uint32_t)s * (16 * 2 * D));
        acc[cb] = mfma32(u32x4{x[0], x[1], y[0], y[1]}, r[s], acc[cb]);
      }
    }
    sched_lds_mfma<DS_FRAGS * CB, 2, 2>();
  };

  for (int kt0 = 0; kt0 < a.tk; kt0 += LIST_CAP) {
    const int n_list = compact_pair(srow0, srow1, kt0, min(LIST_CAP, a.tk - kt0), sm.list, sm.slot, sm.scan, tid);
    // this workgroup's part of the list (all of it unless lists are split)
    const int lo = (int)((int64_t)n_list * sp / ks), hi = (int)((int64_t)n_list * (sp + 1) / ks);
    if (lo == hi) continue;

    // Pipeline: K of entry i is issued one entry ahead, this wavefront's dS
    // fragments two ahead. In the main loop every entry issues its eight dS
    // loads (an entry near the end re-loads the last one), and each of them
    // is consumed by a later entry, so none is dropped by the compiler. At
    // the top of entry i the loads in flight are then, oldest first, dS(i),
    // K(i) and dS(i + 1): waiting until only dS(i + 1)'s remain covers entry
    // i. The last two entries (the tail) issue no dS loads and wait for all.
    bool pres[3];
    stage_k(lo, 0);
    pres[0] = load_ds(lo, dsr[0]);
    pres[1] = load_ds(min(lo + 1, hi - 1), dsr[1]) && lo + 1 < hi;
    pres[2] = false;
    auto entry = [&](auto ring_c, auto tail_c, int it) __attribute__((always_inline)) {
      constexpr int R = decltype(ring_c)::value;
      constexpr int R2 = (R + 2) % 3;
      constexpr bool TAIL = decltype(tail_c)::value;
      const int buf = (it - lo) & 1;
      if constexpr (TAIL) wait_vmem();
      else wait_vmem_le<DS_FRAGS>();
      __syncthreads();   // K(it) visible to all; every wavefront is done with K(it - 1)
      if (it + 1 < hi) stage_k(it + 1, buf ^ 1);
      if constexpr (!TAIL) pres[R2] = load_ds(min(it + 2, hi - 1), dsr[R2]) && it + 2 < hi;
      if (pres[R]) products(buf, dsr[R]);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int it = lo;
    for (; it + 2 < hi; it += 3) {
      entry(I0{}, std::false_type{}, it);
      entry(I1{}, std::false_type{}, it + 1);
      entry(I2{}, std::false_type{}, it + 2);
    }
    if (it < hi) entry(I0{}, std::true_type{}, it);
    if (it + 1 < hi) entry(I1{}, std::true_type{}, it + 1);
    __syncthreads();   // K buffers free before the next pass restages them
  }

  // ---- epilogue: dQ = scale * (dQ^T)^T; lane = query row, registers = channels ----
  // Column c of a stored fragment of row half t is row 32 t + 16 u + 4 v +
  // (j < 4 ? j : j + 4) with v, u = bits 4, 3 of c, j = c % 8.
  {
    const int c = l & 31;
    const int jj = c & 7;
    const int m = (qt0 + q) * BQ + 32 * half + 16 * ((c >> 3) & 1) + 4 * (c >> 4) + (jj < 4 ? jj : jj + 4);
    if (m < a.seq_q && ks > 1) {   // float32 partial [ks][B][H][Sq][D]
      float* out = a.dqpart + ((((int64_t)sp * a.batch + b) * a.heads + h) * a.seq_q + m) * D;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(out + 32 * cb + 8 * q4 + 4 * g) =
              f32x4{acc[cb][4 * q4] * a.scale, acc[cb][4 * q4 + 1] * a.scale, acc[cb][4 * q4 + 2] * a.scale,
                    acc[cb][4 * q4 + 3] * a.scale};
    } else if (m < a.seq_q) {
      const int64_t qoff = (int64_t)b * a.q_sb + (int64_t)m * a.q_ss + (int64_t)h * a.q_sh;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int c0 = 32 * cb + 8 * q4 + 4 * g;
          const float x0 = acc[cb][4 * q4] * a.scale, x1 = acc[cb][4 * q4 + 1] * a.scale;
          const float x2 = acc[cb][4 * q4 + 2] * a.scale, x3 = acc[cb][4 * q4 + 3] * a.scale;
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
template <int D, bool F32, int KS>
__global__ __launch_bounds__(256) void dq_merge_kernel(BwdArgs a) {
  if (a.plan == nullptr || a.plan[1] == 0) return;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // ((b * H + h) * Sq + m) * D / 4 + c4
  const int64_t rows = (int64_t)a.batch * a.heads * a.seq_q;
  if (i >= rows * (D / 4)) return;
  const int64_t r = i / (D / 4);
  const int c0 = (int)(i % (D / 4)) * 4;
  // KS (the part count) is a compile-time constant so that every part's load
  // goes out before the sum
  f32x4 y[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) y[s] = *reinterpret_cast<const f32x4*>(a.dqpart + (s * rows + r) * D + c0);
  f32x4 x = y[0];
#pragma unroll
  for (int s = 1; s < KS; ++s) x += y[s];
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
  if (ks != 1 && ks != 2 && ks != 4 && ks != 8) return hipErrorInvalidValue;
  const int npair = (a.tq + PAIR - 1) / PAIR;
  const int npos = a.dq_blocks ? (npair + kDqBlockPairs - 1) / kDqBlockPairs * kDqBlockPairs : npair;
  hipLaunchKernelGGL((bwd_dq_ds_kernel<D, F32>), dim3(npos * a.batch * a.heads * ks), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  const int64_t n = (int64_t)a.batch * a.heads * a.seq_q * (D / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (ks == 2) hipLaunchKernelGGL((dq_merge_kernel<D, F32, 2>), grid, dim3(256), 0, s, a);
  else if (ks == 4) hipLaunchKernelGGL((dq_merge_kernel<D, F32, 4>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((dq_merge_kernel<D, F32, 8>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_ds(const BwdArgs& a, int head_dim, bool f32, hipStream_t s) {
  if (head_dim == 128) return f32 ? launch_dq_ds_t<128, true>(a, s) : launch_dq_ds_t<128, false>(a, s);
  return f32 ? launch_dq_ds_t<64, true>(a, s) : launch_dq_ds_t<64, false>(a, s);
}

}  // namespace fm
