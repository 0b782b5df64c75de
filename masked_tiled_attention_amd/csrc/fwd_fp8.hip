// Forward kernel on 8-bit floating-point inputs (OCP E4M3, per-tensor
// descales), head dimension 64 or 128.
//
// "Современное состояние Flash Attention на ROCm" (kripta.biz), paragraphs on
// the attention variants and their ranking: the fastest variant runs the
// FlashAttention-2 forward with FP8 operands. The page fixes nothing else;
// the readings taken are: Q, K, V stored as E4M3 codes with one descale
// factor each; both products on the FP8 matrix cores with fp32 accumulation;
// the probabilities taken to E4M3 for the second product; softmax state,
// row sums, O before its final rounding and LSE in fp32.
//
// The tiling, online softmax, class-map driven tile list and mask handling
// are those of the bf16 forward ("FlashAttention-2 ... GPU work
// partitioning", iplexlaw.co.kr, "Block processing keeps the global
// normalization"; FlashMask-3 page, predecessor paragraph). What changes on
// CDNA4 with FP8:
//   S^T = K Q^T with v_mfma_scale_f32_32x32x64_f8f6f4 (scales fixed at 1):
//     lane l holds row (l & 31) and 32 consecutive bytes of the contraction
//     for half l >> 5, so a K row feeds A with two 16-byte LDS reads per 64
//     channels and the wavefront's Q rows sit in registers (8 per 64
//     channels) for the whole kernel.
//   O^T += V^T P^T contracts 64 keys per instruction: P comes straight from
//     the two S^T accumulators of a tile, register i of 32-key block nb being
//     byte 16 nb + i of the lane's operand, converted with v_cvt_pk_fp8_f32.
//     The A operand needs V^T with the same key order; a pre-pass writes,
//     per 64-key tile, four planes (lane half g, 16-key group kc) of
//     [D channels][16 bytes] whose byte t is key 32 kc + 8 (t / 4) + 4 g +
//     t % 4, zero past the sequence end. The kernel copies these D * 64-byte tiles
//     into LDS unchanged, and each lane reads its channel's two 16-byte
//     pieces, 16 bytes apart from the neighbouring lane's.
// Probabilities never exceed 2^8 (the rescale threshold of the max-free
// softmax, checked here per 64-key tile), below 448, the largest finite E4M3
// value. The row sum adds the
// unrounded probabilities, so LSE carries no FP8 rounding.
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
constexpr int LIST_CAP = 1024;
constexpr float kRescaleMax = 256.0f;
template <int D> constexpr int kTileBytes = BK * D;   // one K tile or one V^T tile
template <int D> constexpr int kPlane = D * 16;       // one (g, kc) plane of a V^T tile

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // E8M0 block scales of 127 = 2^0 on both operands: a plain FP8 product.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// ---------------------------------------------------------------- V^T pre-pass
// One workgroup per (b, K/V head, 64-key tile): the tile's V rows go to LDS
// as loaded, then each thread assembles D / 64 16-byte plane pieces (plane
// u / D, channel u % D) from bytes of 16 keys of one channel.
template <int D>
__global__ __launch_bounds__(256) void vt_kernel(VtArgs a) {
  constexpr int CPT = D / 64;   // 16-byte pieces per thread, in and out
  __shared__ uint8_t s[BK][D];
  const int tid = threadIdx.x;
  const int kt = blockIdx.x % a.tk;
  const int bh = blockIdx.x / a.tk;   // b * heads_kv + hk
  const int hk = bh % a.heads_kv, b = bh / a.heads_kv;
  const int n0 = kt * BK;
  {
    const int r = tid >> 2, c0 = (D / 4) * (tid & 3);
    const bool ok = n0 + r < a.seq_k;
    const uint8_t* src = a.v + (int64_t)b * a.v_sb + (int64_t)(n0 + r) * a.v_ss + (int64_t)hk * a.v_sh + c0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) st16(&s[r][c0 + 16 * i], ok ? ld16(src + 16 * i) : u32x4{0u, 0u, 0u, 0u});
  }
  __syncthreads();
  uint8_t* dst = a.vt + ((int64_t)bh * a.tk + kt) * kTileBytes<D>;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int u = tid + 256 * i;
    const int plane = u / D, c = u % D;
    const int g = plane >> 1, kc = plane & 1;
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int key = 32 * kc + 8 * d + 4 * g;   // bytes 4d .. 4d+3
      o[d] = (uint32_t)s[key][c] | ((uint32_t)s[key + 1][c] << 8) | ((uint32_t)s[key + 2][c] << 16) |
             ((uint32_t)s[key + 3][c] << 24);
    }
    st16(dst + u * 16, o);
  }
}

// ---------------------------------------------------------------- forward
template <int D>
struct alignas(16) Fp8Smem {
  uint8_t k[2][kTileBytes<D>];    // K tiles: D-byte rows, 16-byte chunks swizzled by row
  uint8_t vt[3][kTileBytes<D>];   // V^T tiles as the pre-pass wrote them (three: a tile's PV runs in the next iteration)
  int32_t bnd[2][4][BK];       // lts, lte, uts, ute of the tile's keys
  uint32_t list[LIST_CAP];     // non-SKIP key tiles (kt | partial bit)
  int32_t scan[NW];
};

template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_fp8_kernel(FwdArgs a) {
  constexpr int CB = D / 32;       // 32-channel blocks of O^T
  constexpr int KS = D / 64;       // 64-channel contraction steps of S
  constexpr int TILE_BYTES = kTileBytes<D>;
  constexpr int PLANE = kPlane<D>;
  // A D-byte K row has the chunk layout of a (D / 2)-element bf16 row.
  constexpr int DB = D / 2;
  using Dma = DmaTile<DB, BK, NT>;
  __shared__ Fp8Smem<D> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lr = l & 31;
  const int g = l >> 5;

  const int line = __builtin_amdgcn_readfirstlane(a.order[blockIdx.x / a.rep]);
  const int j = blockIdx.x % a.rep;
  const int qt = line % a.tq;
  const int mr = line / a.tq;
  const int bm = mr / a.mask.hm;
  const int hm = mr % a.mask.hm;
  const int b = a.mask.bm > 1 ? bm : j / (a.mask.hm > 1 ? 1 : a.heads);
  const int h = a.mask.hm > 1 ? hm : j % a.heads;
  const int64_t mbase = (int64_t)bm * a.mask.stride_b + (int64_t)hm * a.mask.stride_h;
  const uint8_t* crow = a.classes + ((int64_t)(bm * a.mask.hm + hm) * a.tq + qt) * a.tk;

  const int m = qt * BQ + w * 32 + lr;
  const bool row_ok = m < a.seq_q;

  // Q rows as B operands: bytes 64 s + 32 g .. + 31 of the lane's row.
  i32x8 qf[KS];
  {
    const int mq = min(m, a.seq_q - 1);
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.q) + (int64_t)b * a.q_sb + (int64_t)mq * a.q_ss +
                        (int64_t)h * a.q_sh + 32 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = cat8(ld16(qp + 64 * s), ld16(qp + 64 * s + 16));
  }

  f32x16 oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float C = a.scale_log2;   // includes the Q and K descales
  const bool ragged_k = (a.seq_k % BK) != 0;

  const int hk = __builtin_amdgcn_readfirstlane(h / a.group);
  const int64_t k_ld = a.k_ss;
  const char* kbh = reinterpret_cast<const char*>(a.k) + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh;
  const char* vth = reinterpret_cast<const char*>(a.vt) + ((int64_t)b * a.heads_kv + hk) * a.tk * TILE_BYTES;
  const uint32_t koff = Dma::offset(k_ld, tid);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int32_t rb[4] = {INT_MIN, INT_MAX, 0, 0};

  auto load_tile = [&](int kt, bool masked, int buf, int vbuf) {
    const int n0 = kt * BK;
    Dma::load(reinterpret_cast<char*>(sm.k[buf]), kbh + n0 * k_ld, koff, k_ld, tid, a.seq_k - n0);
    const char* src = vth + (int64_t)kt * TILE_BYTES;
    const uint32_t dst = Dma::lds_address(reinterpret_cast<const char*>(sm.vt[vbuf]));
#pragma unroll
    for (int i = 0; i < TILE_BYTES / 1024 / NW; ++i) {
      const int blk = i * NW + wu;
      Dma::dma16(src + blk * 1024, 16 * l, dst + (uint32_t)blk * 1024u);
    }
    if (masked && tid < BK) {
      const int n = n0 + tid;
      if (n < a.seq_k) {
        rb[0] = a.mask.has_lower ? a.mask.lts[mbase + n] : a.seq_q;
        rb[1] = a.mask.has_lower ? a.mask.lte[mbase + n] : a.seq_q;
        rb[2] = a.mask.has_upper ? a.mask.uts[mbase + n] : 0;
        rb[3] = a.mask.has_upper ? a.mask.ute[mbase + n] : 0;
      } else {
        rb[0] = INT_MIN;
        rb[1] = INT_MAX;
        rb[2] = 0;
        rb[3] = 0;
      }
    }
  };
  auto store_bounds = [&](int buf, bool masked) {
    if (masked && tid < BK) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sm.bnd[buf][jj][tid] = rb[jj];
    }
  };
  auto mask_half = [&](f32x16& sc, int nb, int buf) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int nl = nb * 32 + 8 * q4 + 4 * g;
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

  // Probabilities of one 32-key block against the current reference, as E4M3
  // bytes 16 nb .. 16 nb + 15 of the PV operand; returns the lane's sum of
  // the unrounded values.
  float nmC = INFINITY;
  i32x8 pf;
  auto soft_half = [&](const f32x16& sc, int nb) {
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float p0 = fast_exp2(fmaf(sc[4 * d + 0], C, nmC));
      const float p1 = fast_exp2(fmaf(sc[4 * d + 1], C, nmC));
      const float p2 = fast_exp2(fmaf(sc[4 * d + 2], C, nmC));
      const float p3 = fast_exp2(fmaf(sc[4 * d + 3], C, nmC));
      // The low-half conversion keeps the register's upper bytes, which the
      // high-half conversion then replaces: passing the dead old contents
      // (rather than 0) saves zeroing the register first.
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf[4 * nb + d], false);
      pf[4 * nb + d] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, lo, true);
      r0 += p0 + p2;
      r1 += p1 + p3;
    }
    return r0 + r1;
  };
  // Keep the reference while every probability of the tile is at most 2^8
  // (a lane sum over the tile within that bound implies it), else
  // (wave-uniformly) move it to the tile's row maximum, rescale O and l, and
  // form both halves again. Unlike the bf16 forward, which adds each 32-key
  // half into O before the next half may move the reference, both halves
  // here enter O in one 64-key product, so they must share one reference.
  auto settle_tile = [&](const f32x16* sc, float rs) {
    if (__any(!(rs <= kRescaleMax))) {
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[nb][i]);
      mx = pair_max(mx);
      const bool move = mx > m_run;
      const float alpha = move ? fast_exp2((m_run - mx) * C) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
      m_run = move ? mx : m_run;
      nmC = m_run == -INFINITY ? 0.f : -m_run * C;
      rs = soft_half(sc[0], 0) + soft_half(sc[1], 1);
      if (m_run == -INFINITY) nmC = INFINITY;
    }
    l_run += rs;
  };

  // O^T += V^T P^T for a tile whose probabilities are in `p`, its V^T in
  // LDS buffer vbuf.
  auto pv = [&](const i32x8& p, int vbuf) {
    const char* vb = reinterpret_cast<const char*>(sm.vt[vbuf]);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = 32 * cb + lr;
      const i32x8 va = cat8(*reinterpret_cast<const u32x4*>(vb + (2 * g) * PLANE + 16 * c),
                            *reinterpret_cast<const u32x4*>(vb + (2 * g + 1) * PLANE + 16 * c));
      oacc[cb] = mfma_fp8(va, p, oacc[cb]);
    }
  };

  // Software pipeline: iteration t forms S and the probabilities of tile t
  // while the PV product of tile t-1 runs on the matrix cores. The reference
  // may move at tile t only after that product has entered O, which the
  // program order guarantees (the rescale reads O after the MFMAs wrote it).
  // The first iteration's "previous tile" is V^T buffer 2, zeroed here, with
  // zero probabilities, so that every iteration runs the same straight-line
  // code (a branch would split the block and keep the scheduler from
  // interleaving the product with the softmax). Buffer 2 is first written in
  // the second iteration, after a barrier.
#pragma unroll
  for (int o = 16 * tid; o < TILE_BYTES; o += 16 * NT) st16(sm.vt[2] + o, u32x4{0u, 0u, 0u, 0u});
  int it_global = 0;
  int vrot = 0;             // V^T buffer of the current tile (it_global mod 3)
  i32x8 pf_prev = {0, 0, 0, 0, 0, 0, 0, 0};   // probabilities of the previous tile, not yet in O
  auto iteration = [&](auto masked_c, int it, int n_list, uint32_t& ent) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int buf = it_global & 1;
    const int vnext = vrot == 2 ? 0 : vrot + 1;
    const int vprev = vrot == 0 ? 2 : vrot - 1;
    store_bounds(buf, MASKED);
    wait_vmem();
    __syncthreads();
    if (it + 1 < n_list) {
      ent = __builtin_amdgcn_readfirstlane(sm.list[it + 1]);
      load_tile((int)(ent & ~kPartialBit), (ent & kPartialBit) != 0, buf ^ 1, vnext);
    }
    const char* kb = reinterpret_cast<const char*>(sm.k[buf]);
    f32x16 sacc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      sacc[nb] = f32x16{};
      const int row = 32 * nb + lr;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const i32x8 ka = cat8(*reinterpret_cast<const u32x4*>(kb + rm_byte<DB>(row, 32 * s + 16 * g)),
                              *reinterpret_cast<const u32x4*>(kb + rm_byte<DB>(row, 32 * s + 16 * g + 8)));
        sacc[nb] = mfma_fp8(ka, qf[s], sacc[nb]);
      }
    }
    pv(pf_prev, vprev);
    if constexpr (MASKED) mask_half(sacc[0], 0, buf);
    const float rs0 = soft_half(sacc[0], 0);
    if constexpr (MASKED) mask_half(sacc[1], 1, buf);
    const float rs1 = soft_half(sacc[1], 1);
    settle_tile(sacc, rs0 + rs1);
    pf_prev = pf;
    vrot = vnext;
  };

  for (int kt0 = 0; kt0 < a.tk; kt0 += LIST_CAP) {
    int n_full;
    const int n_list = compact_classes_split<LIST_CAP, NT>(crow, kt0, min(LIST_CAP, a.tk - kt0), sm.list, nullptr,
                                                           sm.scan, tid, false, &n_full, ragged_k ? a.tk - 1 : -1);
    if (n_list == 0) continue;
    uint32_t ent = __builtin_amdgcn_readfirstlane(sm.list[0]);
    load_tile((int)(ent & ~kPartialBit), (ent & kPartialBit) != 0, it_global & 1, vrot);
    int it = 0;
    for (; it < n_full; ++it, ++it_global) iteration(std::false_type{}, it, n_list, ent);
    for (; it < n_list; ++it, ++it_global) iteration(std::true_type{}, it, n_list, ent);
  }
  pv(pf_prev, vrot == 0 ? 2 : vrot - 1);   // the last tile's product
  // Hold the product here, with every lane active: left alone, the compiler
  // sinks these MFMAs into the row_ok branch below, and an MFMA issued with
  // lanes masked off loses the operand rows those lanes hold.
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) asm volatile("" : "+v"(oacc[cb]));

  // ---- epilogue: normalise once (the V descale folded in), write bf16 O and LSE ----
  const float lt = pair_sum(l_run);
  const float inv = lt > 0.f ? a.o_scale / lt : 0.f;
  if (row_ok) {
    const int64_t ooff = (int64_t)b * a.o_sb + (int64_t)m * a.o_ss + (int64_t)h * a.o_sh;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = cb * 32 + 8 * q4 + 4 * g;
        const float x0 = oacc[cb][4 * q4 + 0] * inv, x1 = oacc[cb][4 * q4 + 1] * inv;
        const float x2 = oacc[cb][4 * q4 + 2] * inv, x3 = oacc[cb][4 * q4 + 3] * inv;
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.o) + ooff + c0) =
            u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
      }
    }
    if (g == 0)
      a.lse[((int64_t)b * a.heads + h) * a.seq_q + m] =
          lt > 0.f ? (m_run * C + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_vt(const VtArgs& a, int head_dim, hipStream_t stream) {
  const int64_t nblk = (int64_t)a.batch * a.heads_kv * a.tk;
  if (head_dim == 128) hipLaunchKernelGGL(vt_kernel<128>, dim3((unsigned)nblk), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(vt_kernel<64>, dim3((unsigned)nblk), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a, int head_dim, hipStream_t stream) {
  const int nblk = a.tq * a.batch * a.heads;
  if (head_dim == 128) hipLaunchKernelGGL(fwd_fp8_kernel<128>, dim3(nblk), dim3(NT), 0, stream, a);
  else hipLaunchKernelGGL(fwd_fp8_kernel<64>, dim3(nblk), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fm
