// LDS tile layout, transposing operand reads and class-list compaction shared
// by the attention kernels (gfx950).
#pragma once

#include "fm_attn.h"
#include "fm_device.hpp"

namespace fm {

constexpr uint32_t kPartialBit = 0x80000000u;   // list entry flag: tile needs the mask

// Row-major bf16 tiles (rows of D elements) store 16-byte chunk ch of row r at
// chunk ch ^ swz<D>(r). The gfx950 LDS has 64 four-byte banks; a 16-byte read
// is served 16 lanes per cycle and an 8-byte read 32 lanes per cycle. With the
// swizzle, 16-byte operand reads of 16 consecutive rows, 16-byte staging
// writes of one row, and 4-row x 32-column transposing reads
// (ds_read_b64_tr_b16) each touch every bank once per cycle.
//   D = 128 (256-byte rows, one bank sweep per row): the two low bit pairs of
//     r swapped, so 16 consecutive rows get distinct chunk offsets and 4
//     consecutive rows differ in the chunk-group bits [3:2].
//   D = 64 (128-byte rows, two rows per bank sweep): a bijection of r[3:1]
//     with r[1] on chunk bit 2.
//   D = 32 (64-byte rows, four rows per bank sweep; the 64-byte FP8 rows of
//     head dimension 64): r[3:2] on the two chunk bits.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else if constexpr (D == 32) {
    return (r >> 2) & 3;
  } else {
    return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
  }
}

template <int D>
__device__ __forceinline__ int rm_byte(int row, int col) {   // col: element index, multiple of 4
  return row * (2 * D) + (((col >> 3) ^ swz<D>(row)) << 4) + ((col & 7) << 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each 16-lane
// group, lane j receives element (j % 4) of the 4-value row addressed by lane
// 4k + j / 4, for k = 0..3. When the 16 lanes address rows r..r+3 x columns
// c..c+15 of a row-major bf16 tile (lane i -> row r + i/4, columns
// c + 4(i%4) .. +3), lane j receives column c + j of rows r..r+3.
__device__ __forceinline__ u32x2 tr16(const char* lds_base, int byte) {
  lds_s16x4* p = (lds_s16x4*)((__attribute__((address_space(3))) char*)lds_base + byte);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}

// 16-byte LDS read and transposing read (as tr16) at an LDS byte address.
// Kernels that precompute per-lane addresses use these, so that constant
// parts of an address end up in the instruction's immediate offset.
// The constant part `imm` is added as a pointer offset (it cannot wrap), which
// lets it fold into the instruction.
typedef __attribute__((address_space(3))) const char lds_char;
__device__ __forceinline__ u32x4 lds16(uint32_t addr, uint32_t imm = 0) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((lds_char*)(size_t)addr + imm);
}
__device__ __forceinline__ u32x2 lds_tr16(uint32_t addr, uint32_t imm = 0) {
  return __builtin_bit_cast(u32x2,
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((lds_char*)(size_t)addr + imm)));
}

// MFMA operand (32 output indices x 16 contraction values) read transposed from
// a row-major tile whose rows are the contraction index: lane l gets output
// index obase + (l & 31) and contraction rows r0 + 0..3 (elements 0..3) and
// r1 + 0..3 (elements 4..7), r0 / r1 chosen per lane half by the caller.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const char* base, int lane, int obase, int r0, int r1) {
  const int i = lane & 15;
  const int col = obase + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
  const u32x2 x = tr16(base, rm_byte<D>(r0 + (i >> 2), col));
  const u32x2 y = tr16(base, rm_byte<D>(r1 + (i >> 2), col));
  return u32x4{x[0], x[1], y[0], y[1]};
}

// Compact the non-SKIP entries of one class-map row (entries [first,
// first + count), entry e at row[e * stride]) into sm_list in ascending
// order, flagging PARTIAL ones; returns the number of entries. CAP / NT
// entries per thread. Starts and ends with a barrier, so callers may reuse
// every LDS buffer around it.
template <int CAP, int NT>
__device__ __forceinline__ int compact_classes(const uint8_t* row, int first, int count, uint32_t* sm_list,
                                               int32_t* sm_scan, int tid, int64_t stride = 1) {
  constexpr int PER = CAP / NT;
  constexpr int NWAVE = NT / 64;
  const int lane = tid & 63, wave = tid >> 6;
  uint8_t cls[PER];
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid * PER + e;
    cls[e] = idx < count ? row[(first + idx) * stride] : (uint8_t)FM_TILE_SKIP;
    cnt += cls[e] != FM_TILE_SKIP;
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
  for (int ww = 0; ww < NWAVE; ++ww) {
    if (ww < wave) pos += sm_scan[ww];
    n_list += sm_scan[ww];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (cls[e] != FM_TILE_SKIP) {
      const uint32_t id = (uint32_t)(first + tid * PER + e);
      sm_list[pos++] = id | (cls[e] == FM_TILE_PARTIAL ? kPartialBit : 0u);
    }
  }
  __syncthreads();
  return n_list;
}

// As compact_classes(), but the list holds the FULL entries first and the
// PARTIAL ones after them (each group ascending); *n_full receives the number
// of FULL entries. With all_partial, every entry counts as PARTIAL; entry
// partial_id (if not negative) counts as PARTIAL too. When sm_rank is not
// null, sm_rank[i] receives list entry i's rank among all non-SKIP entries in
// ascending order.
template <int CAP, int NT>
__device__ __forceinline__ int compact_classes_split(const uint8_t* row, int first, int count, uint32_t* sm_list,
                                                     uint16_t* sm_rank, int32_t* sm_scan, int tid,
                                                     bool all_partial, int* n_full, int partial_id = -1) {
  constexpr int PER = CAP / NT;
  constexpr int NWAVE = NT / 64;
  const int lane = tid & 63, wave = tid >> 6;
  uint8_t cls[PER];
  int cf = 0, cp = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid * PER + e;
    uint8_t c = idx < count ? row[first + idx] : (uint8_t)FM_TILE_SKIP;
    if ((all_partial || first + idx == partial_id) && c == FM_TILE_FULL) c = FM_TILE_PARTIAL;
    cls[e] = c;
    cf += c == FM_TILE_FULL;
    cp += c == FM_TILE_PARTIAL;
  }
  // both counts in one scan: FULL in the low 16 bits, PARTIAL in the high
  int incl = cf | (cp << 16);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == 63) sm_scan[wave] = incl;
  __syncthreads();
  int pos = incl - (cf | (cp << 16)), tot = 0;
#pragma unroll
  for (int ww = 0; ww < NWAVE; ++ww) {
    if (ww < wave) pos += sm_scan[ww];
    tot += sm_scan[ww];
  }
  const int nf = tot & 0xffff, np = tot >> 16;
  int pf = pos & 0xffff, pp = nf + (pos >> 16);
  int rank = (pos & 0xffff) + (pos >> 16);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const uint32_t id = (uint32_t)(first + tid * PER + e);
    if (cls[e] == FM_TILE_FULL) {
      if (sm_rank) sm_rank[pf] = (uint16_t)rank;
      ++rank;
      sm_list[pf++] = id;
    } else if (cls[e] == FM_TILE_PARTIAL) {
      if (sm_rank) sm_rank[pp] = (uint16_t)rank;
      ++rank;
      sm_list[pp++] = id | kPartialBit;
    }
  }
  __syncthreads();
  *n_full = nf;
  return nf + np;
}

// Global -> registers for a row-major [rows][D] tile slice: 16-byte chunk
// ci = tid + i * NT holds row ci / (D/8), elements 8 * (ci % (D/8)) .. +8.
// tile_offsets() gives each chunk's byte offset from the tile's first row
// (computed once per kernel); `tile` is that row's byte address (uniform).
// In a ragged tile, rows at or past `nvalid` are re-read from row nvalid - 1
// (callers mask or discard them), so no load leaves the tensor.
template <int D, bool F32, int CHUNKS, int NT>
__device__ __forceinline__ void tile_offsets(uint32_t (&off)[CHUNKS], int64_t ld, int tid) {
  constexpr int ES = F32 ? 4 : 2;
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int ci = tid + i * NT;
    off[i] = (uint32_t)((ci / (D / 8)) * ld + (ci % (D / 8)) * 8 * ES);
  }
}

template <int D, bool F32, int CHUNKS, int NT>
__device__ __forceinline__ void load_tile_rows(u32x4 (&r)[CHUNKS], const char* tile, const uint32_t (&off)[CHUNKS],
                                               int64_t ld, int tid, int nvalid) {
  constexpr int ES = F32 ? 4 : 2;
  constexpr int ROWS = CHUNKS * NT / (D / 8);
  if (nvalid >= ROWS) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) r[i] = load8_as_bf16<F32>(tile + off[i], 0);
  } else {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int ci = tid + i * NT;
      const int row = min(ci / (D / 8), nvalid - 1);
      r[i] = load8_as_bf16<F32>(tile + (int64_t)row * ld + (ci % (D / 8)) * 8 * ES, 0);
    }
  }
}

// Registers -> LDS for the same slice (row-major, swizzled).
template <int D, int CHUNKS, int NT>
__device__ __forceinline__ void store_tile_rows(char* lds, const u32x4 (&r)[CHUNKS], int tid) {
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int ci = tid + i * NT;
    *reinterpret_cast<u32x4*>(lds + rm_byte<D>(ci / (D / 8), 8 * (ci % (D / 8)))) = r[i];
  }
}

// A wavefront-uniform address moved into scalar registers (the direct loads
// below take their base there); free when the compiler already keeps it so.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Direct global -> LDS staging (gfx950 global_load_lds, 16 bytes per lane) of
// a [ROWS][D] bf16 tile into the swizzled row-major layout, without passing
// through registers. One wave instruction fills one contiguous KiB of LDS
// (lane l writes bytes 16 l .. 16 l + 15 of it), so lane l fetches the logical
// chunk that the swizzle stores at that position. KiB block b = i * NW + w is
// written by wavefront w's i-th instruction; its rows are b * RPB + 16 l / 2D.
// Successive instructions of a wavefront step NW * RPB rows (a multiple of 16),
// which leaves swz() unchanged, so a lane needs one offset for all of them and
// the step goes into the uniform base address.
template <int D, int ROWS, int NT>
struct DmaTile {
  static constexpr int NW = NT / 64;
  static constexpr int BLOCKS = ROWS * D * 2 / 1024;
  static constexpr int PER = BLOCKS / NW;   // instructions per wavefront
  static constexpr int RPB = 512 / D;       // rows per KiB block
  static constexpr int STEP = NW * RPB;     // rows between a wavefront's instructions
  static_assert(PER * NW == BLOCKS, "tile must split evenly over the wavefronts");
  static_assert(STEP % 16 == 0, "the row step must keep the swizzle");

  // This lane's first row and its logical chunk in every instruction.
  __device__ static __forceinline__ int row0(int tid) { return (tid >> 6) * RPB + (16 * (tid & 63)) / (2 * D); }
  __device__ static __forceinline__ int chunk(int tid) {
    return (((16 * (tid & 63)) % (2 * D)) / 16) ^ swz<D>(row0(tid));
  }
  // Byte offset, from the tile's first row, of what this lane fetches in a
  // wavefront's first instruction.
  __device__ static __forceinline__ uint32_t offset(int64_t ld, int tid) {
    return (uint32_t)(row0(tid) * ld + chunk(tid) * 16);
  }

  // Issue the tile's loads; `lds` is the tile's LDS base, `off` = offset().
  // Rows at or past `nvalid` re-read row nvalid - 1. The caller awaits
  // completion with wait_vmem() before the barrier that publishes the tile.
  template <bool STREAM = false>
  __device__ static __forceinline__ void load(char* lds, const char* tile, uint32_t off, int64_t ld, int tid,
                                              int nvalid) {
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t base = lds_address(lds) + (uint32_t)w * 1024u;
    if (nvalid >= ROWS) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if constexpr (STREAM) dma16_nt(tile + i * STEP * ld, off, base + (uint32_t)(i * NW) * 1024u);
        else dma16(tile + i * STEP * ld, off, base + (uint32_t)(i * NW) * 1024u);
      }
    } else {
      const int r0 = row0(tid), ch = chunk(tid);
#pragma unroll
      for (int i = 0; i < PER; ++i)
        dma16(tile, (uint32_t)(min(r0 + i * STEP, nvalid - 1) * ld + ch * 16), base + (uint32_t)(i * NW) * 1024u);
    }
  }

  __device__ static __forceinline__ uint32_t lds_address(const char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  }

  // One global_load_lds_dwordx4: lane l copies 16 bytes from base + voff(l)
  // to LDS byte lds_dst + 16 l. Written as inline assembly so that the
  // compiler, which cannot tell the two LDS buffers apart, does not hold back
  // reads of the other buffer until this load lands; the M0 write is followed
  // by the one wait state the LDS-DMA hazard needs.
  // No other code in these kernels keeps a value in M0, so clobbering it here
  // is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  __device__ static __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t lds_dst) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds_dst), "v"(voff), "s"(uniform_ptr(base))
        : "memory", "m0");
  }
  // The same with the non-temporal hint, for data read once (kept out of the
  // caches' way of reused tiles).
  __device__ static __forceinline__ void dma16_nt(const char* base, uint32_t voff, uint32_t lds_dst) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt"
        :
        : "s"(lds_dst), "v"(voff), "s"(uniform_ptr(base))
        : "memory", "m0");
  }
#pragma clang diagnostic pop
};

// One global_load_lds_dword: lane l copies 4 bytes from base + voff(l) to LDS
// byte lds_dst + 4 l (same reasoning as DmaTile::dma16).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds_dst) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2"
      :
      : "s"(lds_dst), "v"(voff), "s"(uniform_ptr(base))
      : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Wait until at most N of this wavefront's global loads (including direct
// loads into LDS) are outstanding: s_waitcnt vmcnt(N). Loads complete in
// issue order, so this awaits everything but the N most recent.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_le<0>(); }

}  // namespace fm
