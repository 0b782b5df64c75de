// Device-side helpers for the gfx950 (CDNA4) kernels of libfmattn.
//
// Wavefronts are 64 lanes. Matrix products use v_mfma_f32_32x32x16_bf16:
//   A (32 x 16): lane l holds row (l & 31), 8 consecutive k of half (l >> 5);
//   B (16 x 32): lane l holds column (l & 31), the same 8 k;
//   C/D (32 x 32, fp32): lane l holds column (l & 31) and, in register i,
//                        row 8*(i/4) + 4*(l >> 5) + (i & 3).
// A and B share the k-to-(lane, element) assignment, so any consistent
// permutation of the contraction index between them gives the same product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// acc + lo(x) + hi(x) for a packed bf16 pair, one v_dot2c_f32_bf16.
__device__ __forceinline__ float add_bf16_pair(uint32_t x, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// 8 consecutive elements of a row as 8 packed bf16 (4 dwords). For float32
// storage the values are rounded to bf16 here.
template <bool kF32>
__device__ __forceinline__ u32x4 load8_as_bf16(const void* base, int64_t elem_off) {
  if constexpr (kF32) {
    const float* p = reinterpret_cast<const float*>(base) + elem_off;
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    u32x4 r;
    r[0] = pack_bf16(a[0], a[1]);
    r[1] = pack_bf16(a[2], a[3]);
    r[2] = pack_bf16(b[0], b[1]);
    r[3] = pack_bf16(b[2], b[3]);
    return r;
  } else {
    return ld16(reinterpret_cast<const uint16_t*>(base) + elem_off);
  }
}

// Instruction-order hints for the machine scheduler (one basic block):
// N MFMAs, each consuming R LDS reads, with the reads of the next DEPTH MFMAs
// issued ahead, so that DEPTH * R reads stay in flight behind each MFMA.
// Masks: 0x008 MFMA, 0x100 LDS read.
template <int N, int R, int DEPTH>
__device__ __forceinline__ void sched_lds_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, DEPTH * R, 0);
#pragma unroll
  for (int j = 0; j < N - DEPTH; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, DEPTH, 0);
}

// Lane id within the wavefront.
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// max / sum of x over the lane pair (l, l ^ 32), one v_permlane32_swap (no
// LDS round trip). Both lanes of a pair get bit-identical results.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace fm
