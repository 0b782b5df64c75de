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
// Kernels:
//   bwd_pre     D per query row and zeroing of the float32 dQ accumulator;
//   bwd         one workgroup per (batch, head, 128-key tile); K and V rows
//               stay in registers, dK and dV accumulate in registers across
//               all non-SKIP 64-row query tiles; dQ partial sums are added to
//               the float32 accumulator with global atomics;
//   dq_finalize dQ = scale * accumulator, cast to the output dtype.
#include <climits>
#include <cmath>

#include "fm_device.hpp"
#include "fm_internal.hpp"

namespace fm {
namespace {

constexpr int BQ = kBwdBlockQ;   // 64 query rows per inner tile
constexpr int BK = kBwdBlockK;   // 128 keys per workgroup
constexpr int NW = BK / 32;      // 4 wavefronts, 32 keys each
constexpr int NT = NW * 64;
constexpr int LIST_CAP = 1024;
constexpr uint32_t kPartialBit = 0x80000000u;

// ------------------------------------------------------------------ pre-pass
template <int D, bool F32>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;            // threads per row
  constexpr int RPB = 256 / TPR;        // rows per block
  const int sub = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;   // (b, m, h) linear
  const int64_t nrows = (int64_t)a.batch * a.seq_q * a.heads;
  float part = 0.f;
  int b = 0, m = 0, h = 0;
  if (row < nrows) {
    h = (int)(row % a.heads);
    m = (int)((row / a.heads) % a.seq_q);
    b = (int)(row / ((int64_t)a.heads * a.seq_q));
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
    float* acc = a.dq_acc + row * D + 8 * sub;
    *reinterpret_cast<f32x4*>(acc) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(acc + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (row < nrows && sub == 0) a.drow[((int64_t)b * a.heads + h) * a.seq_q + m] = part;
}

// ------------------------------------------------------------------ finalize
template <int D, bool F32>
__global__ __launch_bounds__(256) void dq_finalize_kernel(BwdArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8-element chunk
  const int64_t nchunk = (int64_t)a.batch * a.seq_q * a.heads * (D / 8);
  if (idx >= nchunk) return;
  const int64_t row = idx / (D / 8);
  const int c8 = (int)(idx % (D / 8));
  const int h = (int)(row % a.heads);
  const int m = (int)((row / a.heads) % a.seq_q);
  const int b = (int)(row / ((int64_t)a.heads * a.seq_q));
  const float* src = a.dq_acc + row * D + 8 * c8;
  const f32x4 u = *reinterpret_cast<const f32x4*>(src);
  const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4);
  const int64_t off = (int64_t)b * a.q_sb + (int64_t)m * a.q_ss + (int64_t)h * a.q_sh + 8 * c8;
  const float s = a.scale;
  if constexpr (F32) {
    float* d = reinterpret_cast<float*>(a.dq) + off;
    *reinterpret_cast<f32x4*>(d) = f32x4{u[0] * s, u[1] * s, u[2] * s, u[3] * s};
    *reinterpret_cast<f32x4*>(d + 4) = f32x4{v[0] * s, v[1] * s, v[2] * s, v[3] * s};
  } else {
    st16(reinterpret_cast<uint16_t*>(a.dq) + off,
         u32x4{pack_bf16(u[0] * s, u[1] * s), pack_bf16(u[2] * s, u[3] * s), pack_bf16(v[0] * s, v[1] * s),
               pack_bf16(v[2] * s, v[3] * s)});
  }
}

// ------------------------------------------------------------------ main
template <int D>
struct alignas(16) BwdSmem {
  static constexpr int RP = D + 8;     // padded row-major row (elements)
  static constexpr int QTP = BQ + 4;   // padded transposed row over query rows
  static constexpr int KTP = BK + 8;   // padded transposed row over keys
  uint16_t q[BQ][RP];
  uint16_t qt[D][QTP];
  uint16_t dout[BQ][RP];
  uint16_t doutt[D][QTP];
  uint16_t ds[BQ][BK + 8];
  uint16_t kt[D][KTP];
  float lse2[BQ];
  float dd[BQ];
  uint32_t list[LIST_CAP];
  int32_t scan[NW];
};

// Write 4 rows x 8 channels (packed bf16, one u32x4 per row) into a
// row-major tile and its transpose.
template <int ROWP, int TP>
__device__ __forceinline__ void store_rows_and_transpose(uint16_t (*rm)[ROWP], uint16_t (*tr)[TP], int r0, int c0,
                                                         const u32x4 (&rv)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x4*>(&rm[r0 + r][c0]) = rv[r];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    u32x2 ev, od;
    ev[0] = (rv[0][p] & 0xffffu) | (rv[1][p] << 16);
    ev[1] = (rv[2][p] & 0xffffu) | (rv[3][p] << 16);
    od[0] = (rv[0][p] >> 16) | (rv[1][p] & 0xffff0000u);
    od[1] = (rv[2][p] >> 16) | (rv[3][p] & 0xffff0000u);
    *reinterpret_cast<u32x2*>(&tr[c0 + 2 * p][r0]) = ev;
    *reinterpret_cast<u32x2*>(&tr[c0 + 2 * p + 1][r0]) = od;
  }
}

template <int TP>
__device__ __forceinline__ void store_transpose(uint16_t (*tr)[TP], int r0, int c0, const u32x4 (&rv)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    u32x2 ev, od;
    ev[0] = (rv[0][p] & 0xffffu) | (rv[1][p] << 16);
    ev[1] = (rv[2][p] & 0xffffu) | (rv[3][p] << 16);
    od[0] = (rv[0][p] >> 16) | (rv[1][p] & 0xffff0000u);
    od[1] = (rv[2][p] >> 16) | (rv[3][p] & 0xffff0000u);
    *reinterpret_cast<u32x2*>(&tr[c0 + 2 * p][r0]) = ev;
    *reinterpret_cast<u32x2*>(&tr[c0 + 2 * p + 1][r0]) = od;
  }
}

template <int D, bool F32>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdArgs a) {
  constexpr int KSTEPS = D / 16;
  constexpr int CB = D / 32;
  __shared__ BwdSmem<D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 31;
  const int g = l >> 5;

  // Key tiles in ascending order first: under causal-like masks the early
  // keys are seen by the most query rows.
  const int nbh = a.batch * a.heads;
  const int kt = blockIdx.x / nbh;
  const int bh = blockIdx.x % nbh;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  const int bm = a.mask.bm > 1 ? b : 0;
  const int hm = a.mask.hm > 1 ? h : 0;
  const int64_t mbase = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const uint8_t* ccol = a.classes_t + ((int64_t)(bm * a.mask.hm + hm) * a.tk + kt) * a.tq;

  const int n0 = kt * BK;
  const int n = n0 + 32 * w + lr;   // this lane's key
  const bool key_ok = n < a.seq_k;

  // K and V rows of this lane's key as MFMA B operands (channels 16s + 8g ..).
  u32x4 kf[KSTEPS], vf[KSTEPS];
  {
    const int64_t koff = (int64_t)b * a.k_sb + (int64_t)n * a.k_ss + (int64_t)h * a.k_sh + 8 * g;
    const int64_t voff = (int64_t)b * a.v_sb + (int64_t)n * a.v_ss + (int64_t)h * a.v_sh + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      kf[s] = key_ok ? load8_as_bf16<F32>(a.k, koff + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      vf[s] = key_ok ? load8_as_bf16<F32>(a.v, voff + 16 * s) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // The lane's key bounds (keys past the end are masked for every row).
  int32_t b_lts = INT_MIN, b_lte = INT_MAX, b_uts = 0, b_ute = 0;
  if (key_ok) {
    b_lts = a.mask.has_lower ? a.mask.lts[mbase + n] : a.seq_q;
    b_lte = a.mask.has_lower ? a.mask.lte[mbase + n] : a.seq_q;
    b_uts = a.mask.has_upper ? a.mask.uts[mbase + n] : 0;
    b_ute = a.mask.has_upper ? a.mask.ute[mbase + n] : 0;
  }
  const bool ragged_k = (a.seq_k % BK) != 0 && kt == a.tk - 1;

  // K^T of the whole 128-key tile in LDS (B operand of dQ = dS K).
  for (int gi = tid; gi < (BK / 4) * (D / 8); gi += NT) {
    const int kq = gi / (D / 8);
    const int c8 = gi % (D / 8);
    u32x4 rv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nn = n0 + 4 * kq + r;
      rv[r] = nn < a.seq_k ? load8_as_bf16<F32>(a.k, (int64_t)b * a.k_sb + (int64_t)nn * a.k_ss +
                                                         (int64_t)h * a.k_sh + 8 * c8)
                           : u32x4{0u, 0u, 0u, 0u};
    }
    store_transpose<BwdSmem<D>::KTP>(sm.kt, 4 * kq, 8 * c8, rv);
  }

  f32x16 dvacc[CB], dkacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    dvacc[cb] = f32x16{};
    dkacc[cb] = f32x16{};
  }
  const float C = a.scale_log2;
  const int64_t lrow = ((int64_t)b * a.heads + h) * a.seq_q;

  for (int qt0 = 0; qt0 < a.tq; qt0 += LIST_CAP) {
    const int n_in = min(LIST_CAP, a.tq - qt0);
    uint8_t cls[LIST_CAP / NT];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < LIST_CAP / NT; ++e) {
      const int idx = tid * (LIST_CAP / NT) + e;
      cls[e] = idx < n_in ? ccol[qt0 + idx] : (uint8_t)FM_TILE_SKIP;
      cnt += cls[e] != FM_TILE_SKIP;
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (l >= o) incl += y;
    }
    __syncthreads();
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
        const uint32_t qt = (uint32_t)(qt0 + tid * (LIST_CAP / NT) + e);
        sm.list[pos++] = qt | (cls[e] == FM_TILE_PARTIAL ? kPartialBit : 0u);
      }
    }
    __syncthreads();

    for (int it = 0; it < n_list; ++it) {
      const uint32_t ent = sm.list[it];
      const int qt = (int)(ent & ~kPartialBit);
      const bool masked_tile = (ent & kPartialBit) || ragged_k;
      const int m0 = qt * BQ;

      // ---- stage Q, dO (row-major and transposed), LSE*log2e and D ----
      for (int gi = tid; gi < (BQ / 4) * (D / 8); gi += NT) {
        const int rq = gi / (D / 8);
        const int c8 = gi % (D / 8);
        u32x4 rq_[4], rd_[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mm = m0 + 4 * rq + r;
          if (mm < a.seq_q) {
            rq_[r] = load8_as_bf16<F32>(a.q, (int64_t)b * a.q_sb + (int64_t)mm * a.q_ss + (int64_t)h * a.q_sh + 8 * c8);
            rd_[r] = load8_as_bf16<F32>(a.dout, (int64_t)b * a.o_sb + (int64_t)mm * a.o_ss + (int64_t)h * a.o_sh + 8 * c8);
          } else {
            rq_[r] = u32x4{0u, 0u, 0u, 0u};
            rd_[r] = u32x4{0u, 0u, 0u, 0u};
          }
        }
        store_rows_and_transpose<BwdSmem<D>::RP, BwdSmem<D>::QTP>(sm.q, sm.qt, 4 * rq, 8 * c8, rq_);
        store_rows_and_transpose<BwdSmem<D>::RP, BwdSmem<D>::QTP>(sm.dout, sm.doutt, 4 * rq, 8 * c8, rd_);
      }
      if (tid < BQ) {
        const int mm = m0 + tid;
        float l2 = INFINITY, dv = 0.f;
        if (mm < a.seq_q) {
          const float lse = a.lse[lrow + mm];
          l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
          dv = a.drow[lrow + mm];
        }
        sm.lse2[tid] = l2;
        sm.dd[tid] = dv;
      }
      __syncthreads();

      // ---- S = Q K^T and dP = dO V^T (lane = key, registers = query rows) ----
      f32x16 sacc[2], dpacc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        sacc[mb] = f32x16{};
        dpacc[mb] = f32x16{};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const u32x4 qa = *reinterpret_cast<const u32x4*>(&sm.q[32 * mb + lr][16 * s + 8 * g]);
          sacc[mb] = mfma32(qa, kf[s], sacc[mb]);
          const u32x4 da = *reinterpret_cast<const u32x4*>(&sm.dout[32 * mb + lr][16 * s + 8 * g]);
          dpacc[mb] = mfma32(da, vf[s], dpacc[mb]);
        }
      }

      // ---- P and dS ----
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int ml = 32 * mb + 8 * q4 + 4 * g;
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(&sm.lse2[ml]);
          const f32x4 dd = *reinterpret_cast<const f32x4*>(&sm.dd[ml]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * q4 + r;
            float p = fast_exp2(fmaf(sacc[mb][i], C, -l2[r]));
            if (masked_tile) {
              const int mm = m0 + ml + r;
              const bool mk = (b_lts <= mm && mm < b_lte) || (b_uts <= mm && mm < b_ute);
              p = mk ? 0.f : p;
            }
            sacc[mb][i] = p;
            dpacc[mb][i] = p * (dpacc[mb][i] - dd[r]);
          }
        }
      }
      // dS (bf16) to LDS, row-major [query][key], for the dQ product
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ml = 32 * mb + 8 * (i >> 2) + 4 * g + (i & 3);
          const __bf16 x = (__bf16)dpacc[mb][i];
          sm.ds[ml][32 * w + lr] = __builtin_bit_cast(uint16_t, x);
        }

      // ---- dV^T += dO^T P,  dK^T += Q^T dS (contraction over query rows) ----
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 pp, dsp;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pp[j] = pack_bf16(sacc[mb][8 * t + 2 * j], sacc[mb][8 * t + 2 * j + 1]);
            dsp[j] = pack_bf16(dpacc[mb][8 * t + 2 * j], dpacc[mb][8 * t + 2 * j + 1]);
          }
          const int kb = 32 * mb + 16 * t + 4 * g;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const u32x2 d0 = *reinterpret_cast<const u32x2*>(&sm.doutt[32 * cb + lr][kb]);
            const u32x2 d1 = *reinterpret_cast<const u32x2*>(&sm.doutt[32 * cb + lr][kb + 8]);
            dvacc[cb] = mfma32(u32x4{d0[0], d0[1], d1[0], d1[1]}, pp, dvacc[cb]);
            const u32x2 q0 = *reinterpret_cast<const u32x2*>(&sm.qt[32 * cb + lr][kb]);
            const u32x2 q1 = *reinterpret_cast<const u32x2*>(&sm.qt[32 * cb + lr][kb + 8]);
            dkacc[cb] = mfma32(u32x4{q0[0], q0[1], q1[0], q1[1]}, dsp, dkacc[cb]);
          }
        }
      }
      __syncthreads();   // dS tile complete

      // ---- dQ += dS K over the workgroup's 128 keys; float32 atomics ----
      constexpr int NBLK = 2 * CB;            // (query block, channel block) pairs
      constexpr int PER_W = NBLK / NW;        // 2 for D = 128, 1 for D = 64
#pragma unroll
      for (int u = 0; u < PER_W; ++u) {
        const int blk = w * PER_W + u;
        const int mb = blk % 2;
        const int cb = blk / 2;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
          const u32x4 da = *reinterpret_cast<const u32x4*>(&sm.ds[32 * mb + lr][16 * s + 8 * g]);
          const u32x4 kb2 = *reinterpret_cast<const u32x4*>(&sm.kt[32 * cb + lr][16 * s + 8 * g]);
          acc = mfma32(da, kb2, acc);
        }
        // acc holds dQ[m][c]: column c = 32cb + lr, rows m = 32mb + 8(i/4) + 4g + (i&3)
        const int c = 32 * cb + lr;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int mm = m0 + 32 * mb + 8 * (i >> 2) + 4 * g + (i & 3);
          if (mm < a.seq_q)
            unsafeAtomicAdd(a.dq_acc + (((int64_t)b * a.seq_q + mm) * a.heads + h) * D + c, acc[i]);
        }
      }
      __syncthreads();   // LDS tiles are overwritten by the next query tile
    }
  }

  // ---- epilogue: dK = scale * dK^T, dV = dV^T, transposed back on store ----
  if (key_ok) {
    const int64_t koff = (int64_t)b * a.k_sb + (int64_t)n * a.k_ss + (int64_t)h * a.k_sh;
    const int64_t voff = (int64_t)b * a.v_sb + (int64_t)n * a.v_ss + (int64_t)h * a.v_sh;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = 32 * cb + 8 * q4 + 4 * g;
        const float k0 = dkacc[cb][4 * q4] * a.scale, k1 = dkacc[cb][4 * q4 + 1] * a.scale;
        const float k2 = dkacc[cb][4 * q4 + 2] * a.scale, k3 = dkacc[cb][4 * q4 + 3] * a.scale;
        const float v0 = dvacc[cb][4 * q4], v1 = dvacc[cb][4 * q4 + 1];
        const float v2 = dvacc[cb][4 * q4 + 2], v3 = dvacc[cb][4 * q4 + 3];
        if constexpr (F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dk) + koff + c0) = f32x4{k0, k1, k2, k3};
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dv) + voff + c0) = f32x4{v0, v1, v2, v3};
        } else {
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.dk) + koff + c0) =
              u32x2{pack_bf16(k0, k1), pack_bf16(k2, k3)};
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.dv) + voff + c0) =
              u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
        }
      }
    }
  }
}

template <int D, bool F32>
hipError_t launch_pre_t(const BwdArgs& a, hipStream_t s) {
  const int64_t nrows = (int64_t)a.batch * a.seq_q * a.heads;
  const int rpb = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D, F32>), dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_kernel<D, F32>), dim3(a.tk * a.batch * a.heads), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_fin_t(const BwdArgs& a, hipStream_t s) {
  const int64_t nchunk = (int64_t)a.batch * a.seq_q * a.heads * (D / 8);
  hipLaunchKernelGGL((dq_finalize_kernel<D, F32>), dim3((unsigned)((nchunk + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const BwdArgs& a, int head_dim, bool f32, hipStream_t s) {
  if (head_dim == 128) return f32 ? launch_pre_t<128, true>(a, s) : launch_pre_t<128, false>(a, s);
  return f32 ? launch_pre_t<64, true>(a, s) : launch_pre_t<64, false>(a, s);
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, bool f32, hipStream_t s) {
  if (head_dim == 128) return f32 ? launch_bwd_t<128, true>(a, s) : launch_bwd_t<128, false>(a, s);
  return f32 ? launch_bwd_t<64, true>(a, s) : launch_bwd_t<64, false>(a, s);
}

hipError_t launch_dq_finalize(const BwdArgs& a, int head_dim, bool f32, hipStream_t s) {
  if (head_dim == 128) return f32 ? launch_fin_t<128, true>(a, s) : launch_fin_t<128, false>(a, s);
  return f32 ? launch_fin_t<64, true>(a, s) : launch_fin_t<64, false>(a, s);
}

}  // namespace fm
