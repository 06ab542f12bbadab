// Device helpers shared by the HIP kernels: element conversions and the
// per-dtype rules for loading and widening a lane's run of a K/V row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa_impl {
namespace {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------

typedef _Float16 half2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void f16x2(uint32_t w, float &a, float &b) {
  half2_v h = __builtin_bit_cast(half2_v, w);
  a = static_cast<float>(h.x);
  b = static_cast<float>(h.y);
}

// Two OCP e4m3 codes (bytes 0,1 or, with HIGH, bytes 2,3 of w) to float; exact.
template <bool HIGH>
__device__ __forceinline__ void fp8x2(uint32_t w, float &a, float &b) {
  auto f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HIGH);
  a = f[0];
  b = f[1];
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  _Float16 h = static_cast<_Float16>(x);   // v_cvt_f16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// float -> OCP e4m3 code: round to nearest even, saturate to +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;            // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;           // |x| >= 448 (incl. inf): saturate
  if (a >= 0x3c800000u) {                              // |x| >= 2^-6: normal e4m3
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);  // round mantissa to 3 bits, ties even
    return sign | (((r >> 20) - (120u << 3)) & 0x7fu);   // rebias exponent 127 -> 7
  }
  // subnormal e4m3: multiples of 2^-9; 8 * 2^-9 is the smallest normal (code 8)
  const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
  return sign | static_cast<uint32_t>(m);
}

// First position a sliding window of `window` positions (0: none) leaves
// visible to the query at position n - 1: the query and the window - 1
// positions before it.  Blocks wholly before it may have been released, so
// their table entries are never read.
__host__ __device__ __forceinline__ int window_lo(int n, int window) {
  return (window > 0 && n > window) ? n - window : 0;
}

// ---------------------------------------------------------------------------
// storage traits: how one lane loads and widens its run of a K/V row
// ---------------------------------------------------------------------------

struct F32S {};
struct F16S {};
struct BF16S {};
struct FP8S {};

template <typename S> struct Kv;

template <> struct Kv<F32S> {
  static constexpr int kElems = 4;     // elements per lane load (16 bytes)
  static constexpr int kSize = 4;
  using Raw = uint4;
  static __device__ __forceinline__ void widen(const Raw &r, float *f) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
};
template <> struct Kv<BF16S> {
  static constexpr int kElems = 8;
  static constexpr int kSize = 2;
  using Raw = uint4;
  static __device__ __forceinline__ void widen(const Raw &r, float *f) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  }
};
template <> struct Kv<F16S> {
  static constexpr int kElems = 8;
  static constexpr int kSize = 2;
  using Raw = uint4;
  static __device__ __forceinline__ void widen(const Raw &r, float *f) {
    f16x2(r.x, f[0], f[1]); f16x2(r.y, f[2], f[3]);
    f16x2(r.z, f[4], f[5]); f16x2(r.w, f[6], f[7]);
  }
};
template <> struct Kv<FP8S> {
  static constexpr int kElems = 8;     // 8-byte loads keep per-lane registers small
  static constexpr int kSize = 1;
  using Raw = uint2;
  static __device__ __forceinline__ void widen(const Raw &r, float *f) {
    fp8x2<false>(r.x, f[0], f[1]); fp8x2<true>(r.x, f[2], f[3]);
    fp8x2<false>(r.y, f[4], f[5]); fp8x2<true>(r.y, f[6], f[7]);
  }
};

// q / out element access (scalar; only once per workgroup)
template <typename S> struct Qv;
template <> struct Qv<F32S> {
  static __device__ __forceinline__ float get(const void *p, int64_t i) {
    return static_cast<const float *>(p)[i];
  }
  static __device__ __forceinline__ void put(void *p, int64_t i, float x) {
    static_cast<float *>(p)[i] = x;
  }
};
template <> struct Qv<BF16S> {
  static __device__ __forceinline__ float get(const void *p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
  }
  static __device__ __forceinline__ void put(void *p, int64_t i, float x) {
    static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
  }
};
template <> struct Qv<F16S> {
  static __device__ __forceinline__ float get(const void *p, int64_t i) {
    return static_cast<float>(static_cast<const _Float16 *>(p)[i]);
  }
  static __device__ __forceinline__ void put(void *p, int64_t i, float x) {
    static_cast<uint16_t *>(p)[i] = f32_to_f16(x);
  }
};

}  // namespace
}  // namespace pa_impl
