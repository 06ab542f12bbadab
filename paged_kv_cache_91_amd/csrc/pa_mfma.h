// Matrix-core and cross-lane helpers shared by the head-dim-128 decode and
// prefill kernels (gfx950, wave64): the MFMA shapes per 16-bit type, exact
// fp8 -> 16-bit widening, and lane exchanges that stay on the VALU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_common.h"

namespace pa_impl {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <typename QS> struct Mma;
template <> struct Mma<BF16S> {
  using V8 = bf16x8_t;
  using V4 = bf16x4_t;
  static __device__ __forceinline__ f32x4_t run(V8 a, V8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t run16(V4 a, V4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  // two floats -> two bf16 (round to nearest even) in one dword
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(x), static_cast<__bf16>(y)});
  }
  // acc + the two bf16 values of a packed dword (a dot product with (1, 1))
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, 0x3F803F80u),
                                           acc, false);
  }
  // two e4m3 codes (low or high half of w) -> two bf16 values, exact
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_fp8(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
};
template <> struct Mma<F16S> {
  using V8 = f16x8_t;
  using V4 = f16x4_t;
  static __device__ __forceinline__ f32x4_t run(V8 a, V8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t run16(V4 a, V4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, f16x2_t{static_cast<_Float16>(x), static_cast<_Float16>(y)});
  }
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, 0x3C003C00u), acc, false);
  }
  template <bool HI>
  static __device__ __forceinline__ uint32_t from_fp8(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
};

// Combine each lane's value with the lane 16 (resp. 32) away, on the VALU
// (v_permlane16_swap / v_permlane32_swap), so no LDS traffic is involved.
// The swaps are written as inline assembly: given the same value twice, the
// compiler's model of the intrinsics treats both results as that value and
// drops the exchange.  The leading s_nop covers the VALU-write -> permlane
// read hazard on the operands.
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// IEEE maximum (NaN-propagating), one v_max / v_maximum3 with no
// canonicalising moves (fmaxf first quiets each operand it cannot prove
// canonical, one extra instruction per operand)
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float xor16_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  return max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float xor32_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  return max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float xor16_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float xor32_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Values every lane of the wave agrees on, marked as such for the compiler:
// results of cross-lane reductions are otherwise treated as per-lane, which
// turns loops over them into exec-masked loops with copied registers.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// lane l's value, l uniform: two lane reads rather than an LDS permute
__device__ __forceinline__ int64_t lane_value(int64_t x, int l) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Inclusive sum over the wave's 64 lanes of 32-bit values, with DPP moves
// (no LDS): shifts by 1, 2, 4 and 8 within each row of 16 lanes, then each
// row's last lane added into the rows after it (row broadcasts of lanes 15
// and 31).  Lanes a move has no source for contribute 0.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2 and 3
  return v;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

}  // namespace
}  // namespace pa_impl
