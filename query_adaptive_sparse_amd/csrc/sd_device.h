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
// Streaming 16-byte load, marked non-temporal: data read once per call (the gathered K / V rows)
// should not displace reusable lines from the caches.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

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

// Tokens sequence b's cache holds: ctx_len[b] clamped to [0, cap], or cap when no lengths are given
// (a growing cache: workspace rows and tensor strides keep the capacity, the lengths vary per call).
__device__ __forceinline__ int64_t seq_tokens(const int32_t* ctx_len, int b, int64_t cap) {
  if (!ctx_len) return cap;
  const int64_t n = ctx_len[b];
  return n < 0 ? 0 : (n < cap ? n : cap);
}

// Per-sequence cache lengths of one step. The step's first kernel publishes them (from the caller's
// array, or the capacity where it gives none) into the workspace copy `out`; every later kernel of
// the step reads that copy, so all stages see the lengths the scores were computed for.
struct StepLens {
  const int32_t* in;  // caller's device array [B] of tokens, or NULL (every sequence: cap)
  int32_t* out;       // workspace copy [B], or NULL where nothing is published
  int B;
  int64_t cap;        // capacity (tokens)
  int shift;          // entries = tokens >> shift (chunks; 0 for token rows)
  __device__ __forceinline__ void publish(int tid, int nt) const {
    if (out)
      for (int b = tid; b < B; b += nt) out[b] = int32_t(seq_tokens(in, b, cap));
  }
  // entries of sequence b's rows, at most `limit` (the row length a kernel was launched for)
  __device__ __forceinline__ int64_t entries(int b, int64_t limit) const {
    const int64_t e = seq_tokens(in, b, cap) >> shift;
    return e < limit ? e : limit;
  }
};

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

// ---- wave-level reductions and scans on DPP (no LDS round trip). Each has a fixed association,
// and reductions return one lane's value through readlane, so every lane holds the same bits.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
  return __hiloint2double(hi, lo);
}

// max / min of two doubles as one instruction each, for values that come from arithmetic (never
// signalling NaNs): fmax / fmin would first quiet an operand that passed through a branch or a
// lane exchange with an extra instruction. A quiet NaN operand yields the other operand.
__device__ __forceinline__ double max_f64(double x, double y) {
  double r;
  asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ double min_f64(double x, double y) {
  double r;
  asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}

// Clears one long row's coarse bin totals: kBins1 fixed-point mass words (high, low) and counts.
__device__ __forceinline__ void zero_long_totals(unsigned long long* hh, unsigned long long* hl, uint32_t* hc,
                                                 int64_t row, int tid, int nt) {
  for (int i = tid; i < kBins1; i += nt) {
    hh[row * kBins1 + i] = 0ull;
    hl[row * kBins1 + i] = 0ull;
    hc[row * kBins1 + i] = 0u;
  }
}

// x clamped into [0, 1] (NaN to 0) with two instructions and inline constants
__device__ __forceinline__ double clamp01_f64(double x) {
  double r;
  asm("v_max_f64 %0, %1, 0\n\tv_min_f64 %0, %0, 1.0" : "=&v"(r) : "v"(x));
  return r;
}

// x clamped into [0, hi] (NaN to 0); hi is uniform (a scalar register)
__device__ __forceinline__ double clamp0_f64(double x, double hi) {
  double r;
  asm("v_max_f64 %0, %1, 0\n\tv_min_f64 %0, %0, %2" : "=&v"(r) : "v"(x), "s"(hi));
  return r;
}

// Row-of-16 reduction: every lane of a row ends with the row's result.
#define SD_ROW_REDUCE(v, OP)                      \
  v = OP(v, dpp_f64<kDppQuadXor1>(v));            \
  v = OP(v, dpp_f64<kDppQuadXor2>(v));            \
  v = OP(v, dpp_f64<kDppRowRor4>(v));             \
  v = OP(v, dpp_f64<kDppRowRor8>(v));

__device__ __forceinline__ double dpp_add(double a, double b) { return a + b; }

__device__ __forceinline__ double wave_max_dpp(double v) {
  SD_ROW_REDUCE(v, fmax)
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}
__device__ __forceinline__ double wave_min_dpp(double v) {
  SD_ROW_REDUCE(v, fmin)
  return fmin(fmin(readlane_f64(v, 0), readlane_f64(v, 16)), fmin(readlane_f64(v, 32), readlane_f64(v, 48)));
}
__device__ __forceinline__ double wave_sum_dpp(double v) {
  SD_ROW_REDUCE(v, dpp_add)
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}
__device__ __forceinline__ int wave_min_i32_dpp(int v) {
  v = min(v, dpp_i32<kDppQuadXor1>(v));
  v = min(v, dpp_i32<kDppQuadXor2>(v));
  v = min(v, dpp_i32<kDppRowRor4>(v));
  v = min(v, dpp_i32<kDppRowRor8>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_sum_i32_dpp(int v) {
  v += dpp_i32<kDppQuadXor1>(v);
  v += dpp_i32<kDppQuadXor2>(v);
  v += dpp_i32<kDppRowRor4>(v);
  v += dpp_i32<kDppRowRor8>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
// Inclusive scans across the wave: shifts within rows of 16, then the earlier rows' totals.
__device__ __forceinline__ double wave_scan_dpp(double v, int lane) {
  v += dpp_f64<kDppRowShr1>(v);
  v += dpp_f64<kDppRowShr2>(v);
  v += dpp_f64<kDppRowShr4>(v);
  v += dpp_f64<kDppRowShr8>(v);
  const double t0 = readlane_f64(v, 15), t1 = readlane_f64(v, 31), t2 = readlane_f64(v, 47);
  const int r = lane >> 4;
  const double off = r == 0 ? 0.0 : (r == 1 ? t0 : (r == 2 ? t0 + t1 : (t0 + t1) + t2));
  return v + off;
}
__device__ __forceinline__ int wave_scan_i32_dpp(int v, int lane) {
  v += dpp_i32<kDppRowShr1>(v);
  v += dpp_i32<kDppRowShr2>(v);
  v += dpp_i32<kDppRowShr4>(v);
  v += dpp_i32<kDppRowShr8>(v);
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31),
            t2 = __builtin_amdgcn_readlane(v, 47);
  const int r = lane >> 4;
  return v + (r == 0 ? 0 : (r == 1 ? t0 : (r == 2 ? t0 + t1 : t0 + t1 + t2)));
}

// Element offset of query row r of sequence b. Rows are ordered by KV group, then query token,
// then head: r = g Gr + t Gq + j (Gr = T Gq rows per group) is token t, head g Gq + j.
struct QRows {
  int64_t sb, st, sh;
  int Gr, Gq;
};
__device__ __forceinline__ int64_t q_offset(const QRows& m, int b, int r) {
  const int g = r / m.Gr, rr = r - g * m.Gr, t = rr / m.Gq, j = rr - t * m.Gq;
  return int64_t(b) * m.sb + int64_t(t) * m.st + int64_t(g * m.Gq + j) * m.sh;
}

template <typename T>
inline T* at(char* ws, size_t off) {
  return reinterpret_cast<T*>(ws + off);
}

}  // namespace sd
