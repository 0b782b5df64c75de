// Forward kernel: masked attention with an online softmax over K/V tiles.
//
// "FlashAttention-2 ... GPU work partitioning" (iplexlaw.co.kr):
//   - "Block processing keeps the global normalization": inputs are tiled in
//     on-chip memory and the softmax is streamed, rescaling the running
//     statistics and partial output so that the result is normalised over
//     the whole key sequence; no score matrix goes to HBM.
//   - "Three ways to raise GPU utilization": less non-matmul work (here the
//     output is normalised once at the end and the mask is evaluated only on
//     PARTIAL tiles), work split over batch, heads and query tiles, and the
//     query rows of a tile split among the wavefronts while K/V are shared.
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
//         A = V^T read from a transposed LDS copy of the V tile, with the
//         contraction index permuted identically on both sides.
#include <climits>
#include <cmath>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {
namespace {

constexpr int BQ = kFwdBlockQ;   // 128 query rows per workgroup
constexpr int BK = kFwdBlockK;   // 64 keys per K/V tile
constexpr int NW = BQ / 32;      // 4 wavefronts
constexpr int NT = NW * 64;      // 256 threads
constexpr int LIST_CAP = 1024;   // class bytes compacted per pass (4 per thread)
constexpr uint32_t kPartialBit = 0x80000000u;

// V^T rows hold the tile's keys in groups of 4 (8 bytes). Group kg of channel
// row c is stored at group kg ^ vswz(c): with unpadded 128-byte rows this makes
// both the transposing writes (16 lanes -> 16 rows 8 apart) and the MFMA
// operand reads (16 lanes -> 16 consecutive rows) hit 16 distinct 8-byte bank
// slots.
__device__ __forceinline__ int vswz(int c) { return (c & 15) ^ ((c >> 3) & 15); }

template <int D>
struct alignas(16) FwdSmem {
  static constexpr int KP = D + 8;    // padded K row (elements): 8 consecutive rows, 8 bank slots
  uint16_t k[2][BK][KP];              // double-buffered K tile, row-major
  uint16_t vt[2][D][BK];              // double-buffered V tile, transposed and swizzled
  int32_t bnd[2][4][BK];              // lts, lte, uts, ute of the tile's columns
  uint32_t list[LIST_CAP];            // non-SKIP key tiles (kt | partial bit)
  int32_t scan[NW];
};

// Registers carrying one K/V tile from global memory to LDS.
template <int D>
struct TileRegs {
  static constexpr int KR = (BK * D / 8) / NT;                 // 16-byte K chunks per thread
  static constexpr int VG = (BK / 4) * (D / 8);                // 4-key x 8-channel V groups
  static constexpr int VR = (VG + NT - 1) / NT;                // V groups per thread
  u32x4 k[KR];
  u32x4 v[VR][4];
  int32_t b[4];
};

template <int D, bool F32>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs a) {
  constexpr int KSTEPS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int CB = D / 32;       // 32-channel blocks of O^T
  constexpr int NB = BK / 32;      // 32-key blocks of a tile
  using TR = TileRegs<D>;
  __shared__ FwdSmem<D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 31;
  const int g = l >> 5;

  // Heaviest query tiles first (for causal-like masks later rows see more keys).
  const int nbh = a.batch * a.heads;
  const int bid = blockIdx.x;
  const int qt = a.tq - 1 - bid / nbh;
  const int bh = bid % nbh;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  const int bm = a.mask.bm > 1 ? b : 0;
  const int hm = a.mask.hm > 1 ? h : 0;
  const int64_t mbase = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const uint8_t* crow = a.classes + ((int64_t)(bm * a.mask.hm + hm) * a.tq + qt) * a.tk;

  const int m = qt * BQ + w * 32 + lr;   // this lane's query row
  const bool row_ok = m < a.seq_q;

  u32x4 qf[KSTEPS];
  {
    const int64_t qoff = (int64_t)b * a.q_sb + (int64_t)m * a.q_ss + (int64_t)h * a.q_sh + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (row_ok)
        qf[s] = load8_as_bf16<F32>(a.q, qoff + 16 * s);
      else
        qf[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float C = a.scale_log2;
  const bool ragged_k = (a.seq_k % BK) != 0;

  // ---- global -> registers for key tile kt ----
  auto load_tile = [&](TR& r, int kt, bool masked) {
    const int n0 = kt * BK;
#pragma unroll
    for (int i = 0; i < TR::KR; ++i) {
      const int ci = tid + i * NT;
      const int n = n0 + ci / (D / 8);
      const int c8 = ci % (D / 8);
      r.k[i] = n < a.seq_k ? load8_as_bf16<F32>(a.k, (int64_t)b * a.k_sb + (int64_t)n * a.k_ss +
                                                         (int64_t)h * a.k_sh + 8 * c8)
                           : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < TR::VR; ++i) {
      const int gi = tid + i * NT;
      const int kq = gi / (D / 8);
      const int c8 = gi % (D / 8);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int n = n0 + 4 * kq + rr;
        r.v[i][rr] = (gi < TR::VG && n < a.seq_k)
                         ? load8_as_bf16<F32>(a.v, (int64_t)b * a.v_sb + (int64_t)n * a.v_ss +
                                                       (int64_t)h * a.v_sh + 8 * c8)
                         : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (masked && tid < BK) {
      const int n = n0 + tid;
      if (n < a.seq_k) {
        r.b[0] = a.mask.has_lower ? a.mask.lts[mbase + n] : a.seq_q;
        r.b[1] = a.mask.has_lower ? a.mask.lte[mbase + n] : a.seq_q;
        r.b[2] = a.mask.has_upper ? a.mask.uts[mbase + n] : 0;
        r.b[3] = a.mask.has_upper ? a.mask.ute[mbase + n] : 0;
      } else {   // keys past the end: masked for every row
        r.b[0] = INT_MIN;
        r.b[1] = INT_MAX;
        r.b[2] = 0;
        r.b[3] = 0;
      }
    }
  };

  // ---- registers -> LDS buffer buf (K row-major, V transposed) ----
  auto store_tile = [&](const TR& r, int buf, bool masked) {
#pragma unroll
    for (int i = 0; i < TR::KR; ++i) {
      const int ci = tid + i * NT;
      *reinterpret_cast<u32x4*>(&sm.k[buf][ci / (D / 8)][8 * (ci % (D / 8))]) = r.k[i];
    }
#pragma unroll
    for (int i = 0; i < TR::VR; ++i) {
      const int gi = tid + i * NT;
      if (gi < TR::VG) {
        const int kq = gi / (D / 8);
        const int c8 = gi % (D / 8);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int ce = 8 * c8 + 2 * p;
          u32x2 ev, od;
          ev[0] = (r.v[i][0][p] & 0xffffu) | (r.v[i][1][p] << 16);
          ev[1] = (r.v[i][2][p] & 0xffffu) | (r.v[i][3][p] << 16);
          od[0] = (r.v[i][0][p] >> 16) | (r.v[i][1][p] & 0xffff0000u);
          od[1] = (r.v[i][2][p] >> 16) | (r.v[i][3][p] & 0xffff0000u);
          *reinterpret_cast<u32x2*>(&sm.vt[buf][ce][4 * (kq ^ vswz(ce))]) = ev;
          *reinterpret_cast<u32x2*>(&sm.vt[buf][ce + 1][4 * (kq ^ vswz(ce + 1))]) = od;
        }
      }
    }
    if (masked && tid < BK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.bnd[buf][j][tid] = r.b[j];
    }
  };

  TR regs;
  int it_global = 0;   // iteration count across chunks (selects the LDS buffer)

  for (int kt0 = 0; kt0 < a.tk; kt0 += LIST_CAP) {
    // ---- compact the non-SKIP key tiles of this row of the class map ----
    const int n_in = min(LIST_CAP, a.tk - kt0);
    uint8_t cls[LIST_CAP / NT];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < LIST_CAP / NT; ++e) {
      const int idx = tid * (LIST_CAP / NT) + e;
      cls[e] = idx < n_in ? crow[kt0 + idx] : (uint8_t)FM_TILE_SKIP;
      cnt += cls[e] != FM_TILE_SKIP;
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (l >= o) incl += y;
    }
    __syncthreads();   // all waves are done with sm.list, sm.scan and both LDS buffers
    if (l == 63) sm.scan[w] = incl;
    __syncthreads();
    int pos = incl - cnt, n_list = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      if (ww < w) pos += sm.scan[ww];
      n_list += sm.scan[ww];
    }
#pragma unroll
    for (int e = 0; e < LIST_CAP / NT; ++e) {
      if (cls[e] != FM_TILE_SKIP) {
        const uint32_t kt = (uint32_t)(kt0 + tid * (LIST_CAP / NT) + e);
        sm.list[pos++] = kt | (cls[e] == FM_TILE_PARTIAL ? kPartialBit : 0u);
      }
    }
    __syncthreads();
    if (n_list == 0) continue;

    auto masked_of = [&](uint32_t ent) {
      return (ent & kPartialBit) || (ragged_k && (int)(ent & ~kPartialBit) == a.tk - 1);
    };
    uint32_t ent = sm.list[0];
    load_tile(regs, (int)(ent & ~kPartialBit), masked_of(ent));

    for (int it = 0; it < n_list; ++it, ++it_global) {
      const int buf = it_global & 1;
      const bool masked_tile = masked_of(ent);
      store_tile(regs, buf, masked_tile);
      __syncthreads();   // tile `buf` visible; the other buffer is free
      if (it + 1 < n_list) {   // next tile's global loads overlap this tile's math
        ent = sm.list[it + 1];
        load_tile(regs, (int)(ent & ~kPartialBit), masked_of(ent));
      }

      // ---- S^T = K Q^T ----
      f32x16 sacc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sacc[nb] = f32x16{};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(&sm.k[buf][nb * 32 + lr][16 * s + 8 * g]);
          sacc[nb] = mfma32(kf, qf[s], sacc[nb]);
        }
      }

      // ---- interval mask on PARTIAL (and ragged) tiles only ----
      if (masked_tile) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int nl = nb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            const bool mk = (sm.bnd[buf][0][nl] <= m && m < sm.bnd[buf][1][nl]) ||
                            (sm.bnd[buf][2][nl] <= m && m < sm.bnd[buf][3][nl]);
            if (mk) sacc[nb][i] = -INFINITY;
          }
        }
      }

      // ---- online softmax (per-lane row) ----
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[nb][i]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * C);
      const float mC = m_use * C;
      float rs = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sacc[nb][i], C, -mC));
          sacc[nb][i] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (__any(alpha != 1.f)) {   // wave-uniform: skipped once the row maxima settle
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
      }

      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 pf;
#pragma unroll
          for (int j = 0; j < 4; ++j) pf[j] = pack_bf16(sacc[nb][8 * t + 2 * j], sacc[nb][8 * t + 2 * j + 1]);
          const int kg = 8 * nb + 4 * t + g;   // 4-key group of this lane's first 4 keys
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const int c = cb * 32 + lr;
            const int sw = vswz(c);
            const u32x2 lo = *reinterpret_cast<const u32x2*>(&sm.vt[buf][c][4 * (kg ^ sw)]);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(&sm.vt[buf][c][4 * ((kg + 2) ^ sw)]);
            oacc[cb] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, oacc[cb]);
          }
        }
      }
    }
  }

  // ---- epilogue: normalise once, write O and LSE ----
  const float lt = l_run + xor32(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (row_ok) {
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

template <int D, bool F32>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nblk = a.tq * a.batch * a.heads;
  hipLaunchKernelGGL((fwd_kernel<D, F32>), dim3(nblk), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int head_dim, bool f32, hipStream_t stream) {
  if (head_dim == 128) return f32 ? launch_fwd_t<128, true>(a, stream) : launch_fwd_t<128, false>(a, stream);
  return f32 ? launch_fwd_t<64, true>(a, stream) : launch_fwd_t<64, false>(a, stream);
}

}  // namespace fm
