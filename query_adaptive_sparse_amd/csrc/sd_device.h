// Device helpers shared by the gfx950 kernels of the decode step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sd_internal.h"

namespace sd {

using bf16x8 = __attribute__((ext_vector_type(8))) __bf16;
using f32x4 = __attribute__((ext_vector_type(4))) float;
using u16x8 = __attribute__((ext_vector_type(8))) unsigned short;
using bf16x4 = __attribute__((ext_vector_type(4))) __bf16;
using u16x4 = __attribute__((ext_vector_type(4))) unsigned short;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr double kNegInfD = -__builtin_huge_val();
constexpr double kPosInfD = __builtin_huge_val();

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <typename T>
__device__ __forceinline__ float elem_f32(const T* p);
template <>
__device__ __forceinline__ float elem_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float elem_f32<uint16_t>(const uint16_t* p) { return bf2f(*p); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Monotone map of fp64 to uint64: larger score -> larger key; -0 and +0 share a key.
__device__ __forceinline__ uint64_t dkey(double s) {
  s = s + 0.0;
  uint64_t b = static_cast<uint64_t>(__double_as_longlong(s));
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double dkey_inv(uint64_t k) {
  uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double(static_cast<long long>(b));
}

__device__ __forceinline__ double wave_max(double v) {
  for (int o = 32; o; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_min(double v) {
  for (int o = 32; o; o >>= 1) v = fmin(v, __shfl_xor(v, o));
  return v;
}

// Bits of word w (entries 32w .. 32w+31) that fall in [0, first) or [n - last, n).
__device__ __forceinline__ uint32_t edge_bits(int64_t w, int64_t n, int64_t first, int64_t last) {
  uint32_t m = 0;
  const int64_t e0 = w * 32;
  const int64_t lo_end = first < n ? first : n;           // [0, lo_end)
  const int64_t hi_beg = n - last > 0 ? n - last : 0;      // [hi_beg, n)
  for (int i = 0; i < 32; ++i) {
    const int64_t e = e0 + i;
    if (e < n && (e < lo_end || e >= hi_beg)) m |= 1u << i;
  }
  return m;
}

template <typename T>
inline T* at(char* ws, size_t off) {
  return reinterpret_cast<T*>(ws + off);
}

}  // namespace sd
