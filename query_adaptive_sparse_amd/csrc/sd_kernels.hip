// gfx950 kernels of one query-adaptive sparse decode step.
//
// Compiled with -ffp-contract=off: every fused multiply-add below is an
// explicit fma(); nothing is contracted behind our back, so the fp64 score
// arithmetic can be matched bit for bit by a sequential CPU evaluation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sd_internal.h"

namespace sd {
namespace {

using bf16x8 = __attribute__((ext_vector_type(8))) __bf16;
using f32x4 = __attribute__((ext_vector_type(4))) float;
using u16x8 = __attribute__((ext_vector_type(8))) unsigned short;

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

// ---------------------------------------------------------------------------------------------
// Scores. One workgroup scores 64 rows of summary keys (or per-head candidate rows) against the
// group's queries. The key tile is staged in LDS as fp32 (exact for bf16 and fp32 inputs); each
// thread owns one (row, head) score and accumulates it in fp64 over d in index order. Each
// product of two bf16 or two fp32 values is exact in fp64, so fma(q, k, acc) equals the CPU's
// acc + q*k, step for step.
// ---------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_score_rows(const T* __restrict__ q, int64_t q_sb, int64_t q_sh,
                                                    const T* __restrict__ keys, int64_t k_sb, int64_t k_sh,
                                                    int64_t k_st, const int32_t* __restrict__ cand,
                                                    int64_t n_rows, int64_t n_keys, int G, int Hq,
                                                    uint64_t local_mask, double* __restrict__ out, int64_t out_len,
                                                    uint32_t* __restrict__ status) {
  constexpr int R = 64;
  __shared__ float tile[R][D + 1];
  __shared__ float qs[kMaxGroup][D];
  const int b = blockIdx.z, y = blockIdx.y, tid = threadIdx.x;
  if (status && blockIdx.x == 0 && y == 0 && b == 0 && tid < 4) status[tid] = 0;
  const int g = cand ? y / G : y;
  if ((local_mask >> g) & 1) return;
  const int h0 = cand ? y : y * G;
  const int nh = cand ? 1 : G;
  const int64_t r0 = int64_t(blockIdx.x) * R;
  for (int i = tid; i < nh * D; i += 256) {
    const int j = i / D, dd = i - j * D;
    qs[j][dd] = elem_f32<T>(q + b * q_sb + (h0 + j) * q_sh + dd);
  }
  constexpr int EPV = 16 / sizeof(T);
  constexpr int PPR = D / EPV;
  const T* kb = keys + b * k_sb + int64_t(g) * k_sh;
  for (int i = tid; i < R * PPR; i += 256) {
    const int r = i / PPR, pc = i - r * PPR;
    const int64_t row = r0 + r;
    if (row < n_rows) {
      int64_t src = cand ? int64_t(cand[(int64_t(b) * Hq + h0) * out_len + row]) : row;
      src = src < 0 ? 0 : (src < n_keys ? src : n_keys - 1);
      const uint4 v = ld16(kb + src * k_st + pc * EPV);
      const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int u = 0; u < EPV; ++u) tile[r][pc * EPV + u] = elem_f32<T>(e + u);
    }
  }
  __syncthreads();
  const int r = tid % R;
  const int64_t row = r0 + r;
  if (row >= n_rows) return;
  for (int j = tid / R; j < nh; j += 256 / R) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) acc = fma(double(qs[j][i]), double(tile[r][i]), acc);
    out[(int64_t(b) * Hq + h0 + j) * out_len + row] = acc;
  }
}

// Projected query q_p = q P (d -> 16) per scored head, fp64, index order. A bf16 or fp32 query
// times an fp32 projection entry is exact in fp64.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_proxy_query(const T* __restrict__ q, int64_t q_sb, int64_t q_sh,
                                                     const float* __restrict__ proj, int G, int Hq,
                                                     uint64_t local_mask, double* __restrict__ qp,
                                                     uint32_t* __restrict__ status) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && b == 0 && threadIdx.x < 4) status[threadIdx.x] = 0;
  const int h = t >> 4, j = t & 15;
  if (h >= Hq) return;
  const int g = h / G;
  double acc = 0.0;
  if (!((local_mask >> g) & 1)) {
    const float* P = proj + int64_t(g) * D * 16;
    const T* qh = q + b * q_sb + h * q_sh;
    for (int i = 0; i < D; ++i) acc = fma(double(elem_f32<T>(qh + i)), double(P[i * 16 + j]), acc);
  }
  qp[(int64_t(b) * Hq + h) * 16 + j] = acc;
}

// Proxy scores s_t = q_p . k_p[t] over the 16 proxy dims, separate multiply and add in index
// order (q_p has 53 significant bits, so the products round). One thread per token; the
// group's G heads share the token's proxy key. Also writes per-block max / min per head.
__global__ __launch_bounds__(256) void k_score_proxy(const uint16_t* __restrict__ kp, int64_t kp_sb,
                                                     int64_t kp_sh, int64_t kp_st, const double* __restrict__ qp,
                                                     int G, int Hq, int64_t N, uint64_t local_mask,
                                                     double* __restrict__ s0, double* __restrict__ pmax,
                                                     double* __restrict__ pmin, int nblk) {
  const int b = blockIdx.z, g = blockIdx.y, tid = threadIdx.x;
  if ((local_mask >> g) & 1) return;
  __shared__ double qs[kMaxGroup][16];
  __shared__ double rmax[kMaxGroup][4], rmin[kMaxGroup][4];
  if (tid < G * 16) qs[tid >> 4][tid & 15] = qp[(int64_t(b) * Hq + g * G + (tid >> 4)) * 16 + (tid & 15)];
  __syncthreads();
  const int64_t t = int64_t(blockIdx.x) * 256 + tid;
  const bool valid = t < N;
  double kd[16];
  if (valid) {
    const uint16_t* row = kp + b * kp_sb + int64_t(g) * kp_sh + t * kp_st;
    const uint4 a = ld16(row), c = ld16(row + 8);
    const _Float16* ha = reinterpret_cast<const _Float16*>(&a);
    const _Float16* hc = reinterpret_cast<const _Float16*>(&c);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kd[j] = double(float(ha[j]));
      kd[j + 8] = double(float(hc[j]));
    }
  }
  const int lane = tid & 63, wave = tid >> 6;
  for (int j = 0; j < G; ++j) {
    double acc = 0.0;
    if (valid) {
#pragma unroll
      for (int u = 0; u < 16; ++u) acc = acc + qs[j][u] * kd[u];
      s0[(int64_t(b) * Hq + g * G + j) * N + t] = acc;
    }
    const double mx = wave_max(valid ? acc : kNegInfD);
    const double mn = wave_min(valid ? acc : kPosInfD);
    if (lane == 0) {
      rmax[j][wave] = mx;
      rmin[j][wave] = mn;
    }
  }
  __syncthreads();
  if (tid < G) {
    const double mx = fmax(fmax(rmax[tid][0], rmax[tid][1]), fmax(rmax[tid][2], rmax[tid][3]));
    const double mn = fmin(fmin(rmin[tid][0], rmin[tid][1]), fmin(rmin[tid][2], rmin[tid][3]));
    pmax[(int64_t(b) * Hq + g * G + tid) * nblk + blockIdx.x] = mx;
    pmin[(int64_t(b) * Hq + g * G + tid) * nblk + blockIdx.x] = mn;
  }
}

// Per-256-entry max / min of score rows that take the long-row path on summary routing.
__global__ __launch_bounds__(256) void k_row_minmax(const double* __restrict__ s0, int64_t len, int G, int Hq,
                                                    uint64_t local_mask, double* __restrict__ pmax,
                                                    double* __restrict__ pmin, int nblk) {
  const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
  if ((local_mask >> (h / G)) & 1) return;
  __shared__ double rmax[4], rmin[4];
  const int64_t t = int64_t(blockIdx.x) * 256 + tid;
  const int64_t row = int64_t(b) * Hq + h;
  const double v = t < len ? s0[row * len + t] : 0.0;
  const double mx = wave_max(t < len ? v : kNegInfD), mn = wave_min(t < len ? v : kPosInfD);
  if ((tid & 63) == 0) {
    rmax[tid >> 6] = mx;
    rmin[tid >> 6] = mn;
  }
  __syncthreads();
  if (tid == 0) {
    pmax[row * nblk + blockIdx.x] = fmax(fmax(rmax[0], rmax[1]), fmax(rmax[2], rmax[3]));
    pmin[row * nblk + blockIdx.x] = fmin(fmin(rmin[0], rmin[1]), fmin(rmin[2], rmin[3]));
  }
}

// ---------------------------------------------------------------------------------------------
// Block-wide helpers for 512-thread workgroups.
// ---------------------------------------------------------------------------------------------
constexpr int kSelThreads = 512;

// Sort keys[0..Lp) (Lp a power of two) so that larger keys come first and equal keys by
// smaller index: a bitonic network over LDS.
template <typename Idx>
__device__ void bitonic_desc(uint64_t* keys, Idx* idx, int Lp) {
  for (int kk = 2; kk <= Lp; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < Lp; i += kSelThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t ka = keys[i], kb = keys[ixj];
          const Idx ia = idx[i], ib = idx[ixj];
          const bool a_first = ka > kb || (ka == kb && ia < ib);
          const bool want_a_first = (i & kk) == 0;
          if (a_first != want_a_first) {
            keys[i] = kb;
            keys[ixj] = ka;
            idx[i] = ib;
            idx[ixj] = ia;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Exclusive prefix sum of one double per thread, in thread order (fixed association).
__device__ double block_excl_scan(double v, double* buf, double* total) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const double add = t >= off ? buf[t - off] : 0.0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  const double incl = buf[t];
  *total = buf[kSelThreads - 1];
  __syncthreads();
  return incl - v;
}

// First sorted position (< n) at which the running weight base + w_0 + ... + w_i reaches
// `target`, or -1. Positions are split into contiguous per-thread segments; weights come from
// weight(i). Returns the same value to every thread.
template <typename WF>
__device__ int block_first_crossing(int n, double base, double target, WF weight, double* buf, int* ibuf) {
  const int per = (n + kSelThreads - 1) / kSelThreads;
  const int i0 = threadIdx.x * per;
  const int i1 = min(n, i0 + per);
  double local = 0.0;
  for (int i = i0; i < i1; ++i) local += weight(i);
  double total;
  const double excl = block_excl_scan(local, buf, &total);
  if (threadIdx.x == 0) *ibuf = 0x7FFFFFFF;
  __syncthreads();
  double c = base + excl;
  for (int i = i0; i < i1; ++i) {
    c += weight(i);
    if (c >= target) {
      atomicMin(ibuf, i);
      break;
    }
  }
  __syncthreads();
  const int r = *ibuf;
  __syncthreads();
  return r == 0x7FFFFFFF ? -1 : r;
}

// ---------------------------------------------------------------------------------------------
// Selection of rows up to kSmallRowMax entries: one workgroup per (sequence, query head) sorts
// the row by (score desc, index asc) in LDS, then takes the first k (top-k) or the shortest
// prefix whose softmax mass reaches p * Z (top-p; masses and their prefix sums in fp64, fixed
// reduction order). kind 0: bitmap of the row's entries. kind 1 (two-level, level 0): the kept
// segments' chunks as ascending candidate lists. kind 2 (level 1): bitmap over the chunks named
// by the candidate list.
// ---------------------------------------------------------------------------------------------
constexpr int kLdsBitsWords = 4096;

__global__ __launch_bounds__(kSelThreads) void k_select_small(
    const double* __restrict__ s, int64_t len, int Hq, int G, uint64_t local_mask, int topp, int k, double p,
    double scale, int kind, const int32_t* __restrict__ cand_in, int32_t* __restrict__ cand_out, int seg_size,
    int64_t cand_len, uint32_t* __restrict__ bits, int64_t words) {
  __shared__ uint64_t keys[kSmallRowMax];
  __shared__ uint16_t idx[kSmallRowMax];
  __shared__ double buf[kSelThreads];
  __shared__ int ibuf;
  __shared__ uint32_t lbits[kLdsBitsWords];
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  const int64_t row = int64_t(b) * Hq + h;
  const bool local = (local_mask >> (h / G)) & 1;
  if (local) {
    if (kind != 1)
      for (int64_t w = tid; w < words; w += kSelThreads) bits[row * words + w] = 0;
    return;
  }
  const int L = int(len);
  int Lp = 2;
  while (Lp < L) Lp <<= 1;
  for (int i = tid; i < Lp; i += kSelThreads) {
    keys[i] = i < L ? dkey(s[row * len + i]) : 0ull;
    idx[i] = uint16_t(i);
  }
  const int bw = kind == 1 ? (L + 31) / 32 : int(words);
  for (int w = tid; w < bw; w += kSelThreads) lbits[w] = 0;
  __syncthreads();
  bitonic_desc<uint16_t>(keys, idx, Lp);
  int n_sel;
  if (!topp) {
    n_sel = k < L ? k : L;
  } else if (p >= 1.0) {
    n_sel = L;
  } else {
    const double ellmax = scale * dkey_inv(keys[0]);
    auto mass = [&](int i) { return exp(scale * dkey_inv(keys[i]) - ellmax); };
    // Z over every entry, then the first prefix reaching p * Z
    const int per = (L + kSelThreads - 1) / kSelThreads;
    double local_z = 0.0;
    for (int i = tid * per; i < min(L, tid * per + per); ++i) local_z += mass(i);
    double Z;
    block_excl_scan(local_z, buf, &Z);
    const int pos = block_first_crossing(L, 0.0, p * Z, mass, buf, &ibuf);
    n_sel = pos < 0 ? L : pos + 1;
  }
  for (int i = tid; i < n_sel; i += kSelThreads) {
    int e = idx[i];
    if (kind == 2) {
      e = cand_in[row * len + e];
      e = e < 0 ? 0 : (e < int(words) * 32 ? e : int(words) * 32 - 1);
    }
    atomicOr(&lbits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (kind != 1) {
    for (int64_t w = tid; w < words; w += kSelThreads) bits[row * words + w] = lbits[w];
    return;
  }
  // kind 1: kept segments in ascending order -> candidate chunk lists
  const int per = (bw + kSelThreads - 1) / kSelThreads;
  int cntl = 0;
  for (int w = tid * per; w < min(bw, tid * per + per); ++w) cntl += __popc(lbits[w]);
  double tot;
  int rank = int(block_excl_scan(double(cntl), buf, &tot));
  for (int w = tid * per; w < min(bw, tid * per + per); ++w) {
    uint32_t m = lbits[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      const int seg = w * 32 + bit;
      for (int j = 0; j < seg_size; ++j) cand_out[row * cand_len + int64_t(rank) * seg_size + j] = seg * seg_size + j;
      ++rank;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Selection of long rows (token-level): the order is resolved through a coarse histogram of
// (smax - s) over the row's score range, a fine histogram inside the coarse bin where the
// running weight crosses the target, and an exact sort of the entries of the crossing fine bin.
// Weight = softmax mass exp(scale*s - scale*smax) for top-p, 1 for top-k. Bins are monotone in
// the score, so every entry of an earlier bin precedes every entry of a later one in the
// (score desc, index asc) order.
// ---------------------------------------------------------------------------------------------
struct LongArgs {
  const double* s0;
  int64_t len;
  int Hq, G;
  uint64_t local_mask;
  int topp, k;
  double p, scale;
  RowInfo* info;
  const double* pmax;
  const double* pmin;
  int nblk;
  double* h1m;
  uint32_t* h1c;
  double* h2m;
  uint32_t* h2c;
  uint64_t* ckey;
  int32_t* cidx;
  int32_t* ccnt;
  uint32_t* bits;
  int64_t words;
  uint32_t* status;
};

__device__ __forceinline__ void long_bins(double s, const RowInfo& ri, int* b1, int* b2) {
  double delta = (ri.smax - s) * ri.binscale;
  delta = delta >= 0.0 ? (delta < double(kBins1) ? delta : double(kBins1)) : 0.0;  // NaN -> 0
  int c1 = int(delta);
  c1 = c1 < kBins1 - 1 ? c1 : kBins1 - 1;
  *b1 = c1;
  const double f = delta - double(c1);
  int c2 = int(f * double(kBins2));
  c2 = c2 < 0 ? 0 : (c2 < kBins2 - 1 ? c2 : kBins2 - 1);
  *b2 = c2;
}

__device__ __forceinline__ double long_weight(const LongArgs& a, const RowInfo& ri, double s) {
  return a.topp ? exp(a.scale * s - a.scale * ri.smax) : 1.0;
}

__global__ __launch_bounds__(256) void k_long_prep(LongArgs a) {
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  __shared__ double rmax[4], rmin[4];
  double mx = kNegInfD, mn = kPosInfD;
  for (int i = tid; i < a.nblk; i += 256) {
    mx = fmax(mx, a.pmax[row * a.nblk + i]);
    mn = fmin(mn, a.pmin[row * a.nblk + i]);
  }
  mx = wave_max(mx);
  mn = wave_min(mn);
  if ((tid & 63) == 0) {
    rmax[tid >> 6] = mx;
    rmin[tid >> 6] = mn;
  }
  for (int i = tid; i < kBins1; i += 256) {
    a.h1m[row * kBins1 + i] = 0.0;
    a.h1c[row * kBins1 + i] = 0;
  }
  for (int i = tid; i < kBins2; i += 256) {
    a.h2m[row * kBins2 + i] = 0.0;
    a.h2c[row * kBins2 + i] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    RowInfo ri = {};
    ri.smax = fmax(fmax(rmax[0], rmax[1]), fmax(rmax[2], rmax[3]));
    ri.smin = fmin(fmin(rmin[0], rmin[1]), fmin(rmin[2], rmin[3]));
    const double range = ri.smax - ri.smin;
    ri.binscale = range > 0.0 ? double(kBins1) / range : 0.0;
    ri.all = a.topp ? (a.p >= 1.0) : (int64_t(a.k) >= a.len);
    ri.target = a.topp ? 0.0 : double(a.k);
    a.info[row] = ri;
    a.ccnt[row] = 0;
  }
}

// level 1: coarse histogram of every entry; level 2: fine histogram of the crossing coarse bin,
// plus the bitmap of the row (entries of earlier coarse bins are selected).
template <int LEVEL>
__global__ __launch_bounds__(256) void k_long_hist(LongArgs a) {
  const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
  const int64_t row = int64_t(b) * a.Hq + h;
  if ((a.local_mask >> (h / a.G)) & 1) {
    // local heads select nothing themselves: their bitmap rows are zero
    if (LEVEL == 2) {
      const int64_t w0 = int64_t(blockIdx.x) * (kLongBlock / 32);
      for (int64_t w = w0 + tid; w < w0 + kLongBlock / 32 && w < a.words; w += 256) a.bits[row * a.words + w] = 0;
    }
    return;
  }
  const RowInfo ri = a.info[row];
  constexpr int NB = LEVEL == 1 ? kBins1 : kBins2;
  __shared__ double hm[NB];
  __shared__ uint32_t hc[NB];
  for (int i = tid; i < NB; i += 256) {
    hm[i] = 0.0;
    hc[i] = 0;
  }
  __syncthreads();
  const int64_t t0 = int64_t(blockIdx.x) * kLongBlock;
  const int64_t t1 = t0 + kLongBlock < a.len ? t0 + kLongBlock : a.len;
  const double* sr = a.s0 + row * a.len;
  for (int64_t base = t0; base < t0 + kLongBlock; base += 256) {
    const int64_t t = base + tid;
    bool sel = false;
    if (t < t1) {
      const double s = sr[t];
      int b1, b2;
      long_bins(s, ri, &b1, &b2);
      if (LEVEL == 1) {
        if (!ri.all) {
          atomicAdd(&hm[b1], long_weight(a, ri, s));
          atomicAdd(&hc[b1], 1u);
        }
      } else {
        sel = ri.all || b1 < ri.bin1;
        if (!ri.all && b1 == ri.bin1) {
          atomicAdd(&hm[b2], long_weight(a, ri, s));
          atomicAdd(&hc[b2], 1u);
        }
      }
    }
    if (LEVEL == 2 && base < a.len) {
      const uint64_t m = __ballot(sel);
      const int lane = tid & 63;
      const int64_t w = (base + (tid & ~63)) >> 5;
      if (lane == 0 && w < a.words) a.bits[row * a.words + w] = uint32_t(m);
      if (lane == 1 && w + 1 < a.words) a.bits[row * a.words + w + 1] = uint32_t(m >> 32);
    }
  }
  __syncthreads();
  if (ri.all) return;
  double* gm = LEVEL == 1 ? a.h1m + row * kBins1 : a.h2m + row * kBins2;
  uint32_t* gc = LEVEL == 1 ? a.h1c + row * kBins1 : a.h2c + row * kBins2;
  for (int i = tid; i < NB; i += 256) {
    if (hc[i]) {
      unsafeAtomicAdd(&gm[i], hm[i]);
      atomicAdd(&gc[i], hc[i]);
    }
  }
}

// Find the bin where the running weight crosses the target (one workgroup per row).
template <int LEVEL>
__global__ __launch_bounds__(kSelThreads) void k_long_find(LongArgs a) {
  const int b = blockIdx.y, h = blockIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  __shared__ double buf[kSelThreads];
  __shared__ int ibuf;
  RowInfo ri = a.info[row];
  if (ri.all) return;
  constexpr int NB = LEVEL == 1 ? kBins1 : kBins2;
  const double* gm = LEVEL == 1 ? a.h1m + row * kBins1 : a.h2m + row * kBins2;
  double base = 0.0;
  if (LEVEL == 1) {
    if (a.topp) {
      double Z;
      const int per = NB / kSelThreads;
      double local = 0.0;
      for (int i = threadIdx.x * per; i < threadIdx.x * per + per; ++i) local += gm[i];
      block_excl_scan(local, buf, &Z);
      ri.target = a.p * Z;
    }
  } else {
    base = ri.before1;
  }
  auto weight = [&](int i) { return gm[i]; };
  const int pos = block_first_crossing(NB, base, ri.target, weight, buf, &ibuf);
  // weight ahead of the crossing bin, in the same association as the crossing search
  double before;
  {
    const int per = (NB + kSelThreads - 1) / kSelThreads;
    const int i0 = threadIdx.x * per;
    double local = 0.0;
    for (int i = i0; i < min(NB, i0 + per); ++i) local += (pos >= 0 && i < pos) ? gm[i] : 0.0;
    double tot;
    block_excl_scan(local, buf, &tot);
    before = base + tot;
  }
  if (threadIdx.x == 0) {
    if (pos < 0) {
      // rounding left the target above the total weight: keep every entry
      ri.all = 1;
    } else if (LEVEL == 1) {
      ri.bin1 = pos;
      ri.before1 = before;
    } else {
      ri.bin2 = pos;
      ri.before2 = before;
    }
    a.info[row] = ri;
  }
}

// Entries of the crossing coarse bin: earlier fine bins are selected outright; the crossing fine
// bin's entries are gathered for the exact resolution.
__global__ __launch_bounds__(256) void k_long_collect(LongArgs a) {
  const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  const RowInfo ri = a.info[row];
  if (ri.all) return;
  const int64_t t0 = int64_t(blockIdx.x) * kLongBlock;
  const int64_t t1 = t0 + kLongBlock < a.len ? t0 + kLongBlock : a.len;
  const double* sr = a.s0 + row * a.len;
  for (int64_t t = t0 + tid; t < t1; t += 256) {
    const double s = sr[t];
    int b1, b2;
    long_bins(s, ri, &b1, &b2);
    if (b1 != ri.bin1) continue;
    if (b2 < ri.bin2) {
      atomicOr(&a.bits[row * a.words + (t >> 5)], 1u << (t & 31));
    } else if (b2 == ri.bin2) {
      const int pos = atomicAdd(&a.ccnt[row], 1);
      if (pos < kResolveCap) {
        a.ckey[row * kResolveCap + pos] = dkey(s);
        a.cidx[row * kResolveCap + pos] = int32_t(t);
      } else {
        atomicOr(&a.status[0], 1u);
      }
    }
  }
}

// Exact resolution of the crossing fine bin: sort its entries, walk the running weight from the
// weight of everything ahead of the bin, select up to the first crossing.
__global__ __launch_bounds__(kSelThreads) void k_long_resolve(LongArgs a) {
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  const RowInfo ri = a.info[row];
  if (ri.all) return;
  __shared__ uint64_t keys[kResolveCap];
  __shared__ int32_t idx[kResolveCap];
  __shared__ double buf[kSelThreads];
  __shared__ int ibuf;
  int n = a.ccnt[row];
  n = n < kResolveCap ? n : kResolveCap;
  int Lp = 2;
  while (Lp < n) Lp <<= 1;
  for (int i = tid; i < Lp; i += kSelThreads) {
    keys[i] = i < n ? a.ckey[row * kResolveCap + i] : 0ull;
    idx[i] = i < n ? a.cidx[row * kResolveCap + i] : 0x7FFFFFFF;
  }
  __syncthreads();
  bitonic_desc<int32_t>(keys, idx, Lp);
  auto weight = [&](int i) { return long_weight(a, ri, dkey_inv(keys[i])); };
  const int pos = block_first_crossing(n, ri.before2, ri.target, weight, buf, &ibuf);
  const int n_sel = pos < 0 ? n : pos + 1;
  for (int i = tid; i < n_sel; i += kSelThreads) {
    const int t = idx[i];
    atomicOr(&a.bits[row * a.words + (t >> 5)], 1u << (t & 31));
  }
}

// ---------------------------------------------------------------------------------------------
// GQA union and compaction: per (sequence, KV group) the OR of the group's per-head bitmaps plus
// forced sink / recent entries (scored groups) or the sink + window (local groups), then the set
// bits in ascending order. Ranges of 1024 words per workgroup; counts, then writes.
// ---------------------------------------------------------------------------------------------
constexpr int kUnionWordsPerBlock = 1024;

struct UnionArgs {
  const uint32_t* bits;
  uint32_t* ubits;
  int32_t* rcnt;
  int32_t* list;
  int32_t* cnt;
  int64_t words, n;
  int Hq, Hk, G, ranges;
  uint64_t local_mask;
  int keep_first, keep_last, sink, window;
};

__global__ __launch_bounds__(256) void k_union_count(UnionArgs a) {
  const int b = blockIdx.z, g = blockIdx.y, r = blockIdx.x, tid = threadIdx.x;
  const bool local = (a.local_mask >> g) & 1;
  const int64_t w0 = int64_t(r) * kUnionWordsPerBlock;
  const int64_t grp = int64_t(b) * a.Hk + g;
  int c = 0;
  for (int64_t w = w0 + tid; w < w0 + kUnionWordsPerBlock && w < a.words; w += 256) {
    uint32_t u;
    if (local) {
      u = edge_bits(w, a.n, a.sink, a.window);
    } else {
      u = edge_bits(w, a.n, a.keep_first, a.keep_last);
      for (int j = 0; j < a.G; ++j) u |= a.bits[(int64_t(b) * a.Hq + g * a.G + j) * a.words + w];
      if (w == a.words - 1 && (a.n & 31)) u &= (1u << (a.n & 31)) - 1u;
    }
    a.ubits[grp * a.words + w] = u;
    c += __popc(u);
  }
  for (int o = 32; o; o >>= 1) c += __shfl_xor(c, o);
  __shared__ int part[4];
  if ((tid & 63) == 0) part[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) a.rcnt[grp * a.ranges + r] = part[0] + part[1] + part[2] + part[3];
}

__global__ __launch_bounds__(256) void k_union_write(UnionArgs a) {
  const int b = blockIdx.z, g = blockIdx.y, r = blockIdx.x, tid = threadIdx.x;
  const int64_t grp = int64_t(b) * a.Hk + g;
  __shared__ int sbase;
  __shared__ int scan[256];
  if (tid == 0) {
    int s = 0;
    for (int i = 0; i < r; ++i) s += a.rcnt[grp * a.ranges + i];
    sbase = s;
  }
  // each thread owns 4 consecutive words
  const int64_t w0 = int64_t(r) * kUnionWordsPerBlock + tid * 4;
  uint32_t u[4];
  int c = 0;
  for (int i = 0; i < 4; ++i) {
    const int64_t w = w0 + i;
    u[i] = w < a.words ? a.ubits[grp * a.words + w] : 0u;
    c += __popc(u[i]);
  }
  scan[tid] = c;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  int pos = sbase + scan[tid] - c;
  int32_t* out = a.list + grp * a.n;
  for (int i = 0; i < 4; ++i) {
    uint32_t m = u[i];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      out[pos++] = int32_t((w0 + i) * 32 + bit);
    }
  }
  if (r == a.ranges - 1 && tid == 255) a.cnt[grp] = sbase + scan[255];
}

// ---------------------------------------------------------------------------------------------
// Gathered split-K attention. Workgroup = (split, KV group, sequence), 4 waves; each wave walks
// 32-token tiles of the split (raw tokens of the listed chunks, then their summary rows) with an
// online softmax, and the waves merge at the end into the split's partial (o, lse).
//
// Logits: MFMA with tokens as the 16-row M dimension and the group's heads as the N dimension
// (S^T = K Q^T); K fragments load straight from HBM in the A-operand layout, 16 bytes per lane.
// P V: MFMA with head slots as M, dims as N, tokens as K; P enters from the logit layout with no
// data movement. For bf16, P is split into hi = bf16(p) and lo = bf16(p - hi) rows (slots
// [0, G) and [G, 2G)), which restores fp32 accuracy of the probabilities; the two rows are added
// at the end. V tiles are staged in LDS (row-major, padded) and read per lane as the B operand.
// ---------------------------------------------------------------------------------------------
struct AttendArgs {
  const void* q;
  int64_t q_sb, q_sh;
  const void* k;
  const void* v;
  int64_t kv_sb, kv_sh, kv_st;
  const void* kg;
  const void* vg;
  int64_t g_sb, g_sh, g_st;
  const int32_t* list;
  const int32_t* cnt;
  float* po;
  float* pl;
  int64_t n_list;  // list row stride (entries)
  int G, Hq, Hk, chunk_shift, E, max_splits, attend_summary;
  float scale_log2;
};

constexpr int kMaxSplitEntries = 2048;

template <typename T, int D>
struct AttendLds {
  static constexpr int kRowWords = D * int(sizeof(T)) / 4 + 4;  // padded V row, 32-bit words
  static constexpr int kVtWords = kTile * kRowWords;             // one wave's V tile
  static constexpr int kMergeWords = 16 * D + 32;                // one wave's (acc, m, l)
  static constexpr int kWaveWords = kVtWords > kMergeWords ? kVtWords : kMergeWords;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void k_attend(AttendArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  using L = AttendLds<T, D>;
  __shared__ int32_t lst[kMaxSplitEntries];
  __shared__ uint32_t wlds[kWaves * L::kWaveWords];
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t grp = int64_t(b) * a.Hk + g;
  const int cnt = a.cnt[grp];
  const int e0 = s * a.E;
  if (e0 >= cnt) return;
  const int ne = min(a.E, cnt - e0);
  for (int i = threadIdx.x; i < ne; i += 256) lst[i] = a.list[grp * a.n_list + e0 + i];
  __syncthreads();

  const int cs = a.chunk_shift;
  const int C = 1 << cs;
  const int ntok = ne << cs;
  const int traw = (ntok + kTile - 1) / kTile;
  const int tsum = a.attend_summary ? (ne + kTile - 1) / kTile : 0;
  const int ntiles = traw + tsum;
  const int n = lane & 15, c = lane >> 4;
  const int G = a.G;
  const int hs = n < G ? n : (n < 2 * G ? n - G : -1);   // head of this lane's slot
  const bool lo_row = BF && n >= G && n < 2 * G;

  const T* qrow = reinterpret_cast<const T*>(a.q) + b * a.q_sb + int64_t(g * G + (hs < 0 ? 0 : hs)) * a.q_sh;
  const T* kraw = reinterpret_cast<const T*>(a.k) + b * a.kv_sb + int64_t(g) * a.kv_sh;
  const T* vraw = reinterpret_cast<const T*>(a.v) + b * a.kv_sb + int64_t(g) * a.kv_sh;
  const T* ksum = reinterpret_cast<const T*>(a.kg) + b * a.g_sb + int64_t(g) * a.g_sh;
  const T* vsum = reinterpret_cast<const T*>(a.vg) + b * a.g_sb + int64_t(g) * a.g_sh;
  uint32_t* vt = wlds + wave * L::kWaveWords;

  // query fragments (B operand of S^T = K Q^T)
  constexpr int QF = BF ? D / 32 : D / 4;
  uint4 qf[BF ? QF : 1];
  float qf32[BF ? 1 : D / 4];
  if constexpr (BF) {
#pragma unroll
    for (int j = 0; j < QF; ++j) qf[j] = hs >= 0 ? ld16(qrow + 32 * j + 8 * c) : make_uint4(0, 0, 0, 0);
  } else {
    // fp32: MFMA j, lane group c covers dim (D/4) c + j
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const uint4 v = hs >= 0 ? ld16(qrow + (D / 4) * c + 4 * j) : make_uint4(0, 0, 0, 0);
      const float* f = reinterpret_cast<const float*>(&v);
#pragma unroll
      for (int u = 0; u < 4; ++u) qf32[4 * j + u] = f[u];
    }
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = wave; t < ntiles; t += kWaves) {
    const bool sumt = t >= traw;
    const T* kb = sumt ? ksum : kraw;
    const T* vb = sumt ? vsum : vraw;
    const int64_t st = sumt ? a.g_st : a.kv_st;
    const int nv = sumt ? min(kTile, ne - (t - traw) * kTile) : min(kTile, ntok - t * kTile);
    auto rowof = [&](int x) -> int64_t {
      x = x < nv ? x : 0;  // padded positions read a valid row; their logits are masked
      if (sumt) return lst[(t - traw) * kTile + x];
      const int v = t * kTile + x;
      return (int64_t(lst[v >> cs]) << cs) | (v & (C - 1));
    };

    // ---- logits: S^T[token][slot]
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const T* kr = kb + rowof(16 * tb + n) * st;
      if constexpr (BF) {
        uint4 kf[QF];
#pragma unroll
        for (int j = 0; j < QF; ++j) kf[j] = ld16(kr + 32 * j + 8 * c);
#pragma unroll
        for (int j = 0; j < QF; ++j)
          sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[j]),
                                                              __builtin_bit_cast(bf16x8, qf[j]), sacc[tb], 0, 0, 0);
      } else {
        float kf[D / 4];
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const uint4 v = ld16(kr + (D / 4) * c + 4 * j);
          const float* f = reinterpret_cast<const float*>(&v);
#pragma unroll
          for (int u = 0; u < 4; ++u) kf[4 * j + u] = f[u];
        }
#pragma unroll
        for (int j = 0; j < D / 4; ++j)
          sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[j], qf32[j], sacc[tb], 0, 0, 0);
      }
    }

    // ---- V tile -> LDS, row-major [token][dim] with a 4-word pad per row
    {
      constexpr int EPV = 16 / int(sizeof(T));
      constexpr int PPR = D / EPV;                 // 16-byte pieces per row
      constexpr int PIECES = kTile * PPR / 64;     // per lane
#pragma unroll
      for (int kq = 0; kq < PIECES; ++kq) {
        const int pidx = kq * 64 + lane;
        const int x = pidx / PPR, cp = pidx - x * PPR;
        const uint4 v = ld16(vb + rowof(x) * st + cp * EPV);
        *reinterpret_cast<uint4*>(vt + x * L::kRowWords + cp * 4) = v;
      }
    }

    // ---- online softmax (base 2)
    float lg[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = 16 * tb + 4 * c + i;
        lg[tb * 4 + i] = x < nv ? sacc[tb][i] * a.scale_log2 : kNegInf;
      }
    float mt = lg[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, lg[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m_run, mt);
    const bool none = mn == kNegInf;
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
    float pr[8];
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = none ? 0.f : __builtin_amdgcn_exp2f(lg[i] - mn);
      ls += pr[i];
    }
    l_run = l_run * alpha + ls;
    m_run = mn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * c + i);
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) acc[nb][i] *= ai;
    }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- P V
    const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(vt);
    if constexpr (BF) {
      u16x8 pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t hi = f2bf(pr[e]);
        pa[e] = hs < 0 ? uint16_t(0) : (lo_row ? f2bf(pr[e] - bf2f(hi)) : hi);
      }
      // B operand slot e of lane group c = token (e < 4 ? 4c + e : 16 + 4c + e - 4)
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        u16x8 vbf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = (e < 4) ? 4 * c + e : 16 + 4 * c + (e - 4);
          vbf[e] = vt16[x * (2 * L::kRowWords) + 16 * nb + n];
        }
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                           __builtin_bit_cast(bf16x8, vbf), acc[nb], 0, 0, 0);
      }
    } else {
      const float* vtf = reinterpret_cast<const float*>(vt);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = hs >= 0 && n < G ? pr[tb * 4 + i] : 0.f;
          const int x = 16 * tb + 4 * c + i;
#pragma unroll
          for (int nb = 0; nb < D / 16; ++nb)
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, vtf[x * L::kRowWords + 16 * nb + n], acc[nb], 0, 0, 0);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the 4 waves
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();  // every wave is done with its V tile; reuse the LDS
  float* mw = reinterpret_cast<float*>(wlds + wave * L::kWaveWords);  // [16][D] acc, then m[16], l[16]
  const int nslots = BF ? 2 * G : G;
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 4 * c + i;
      if (slot < nslots) mw[slot * D + 16 * nb + n] = acc[nb][i];
    }
  if (c == 0 && n < G) {
    mw[16 * D + n] = m_run;
    mw[16 * D + 16 + n] = l_run;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < G * D; it += 256) {
    const int hh = it / D, dd = it - hh * D;
    float M = kNegInf;
    for (int w = 0; w < kWaves; ++w) {
      const float* ww = reinterpret_cast<const float*>(wlds + w * L::kWaveWords);
      M = fmaxf(M, ww[16 * D + hh]);
    }
    float Ls = 0.f, O = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float* ww = reinterpret_cast<const float*>(wlds + w * L::kWaveWords);
      const float mw_ = ww[16 * D + hh];
      if (mw_ == kNegInf) continue;
      const float f = __builtin_amdgcn_exp2f(mw_ - M);
      Ls += ww[16 * D + 16 + hh] * f;
      float o = ww[hh * D + dd];
      if (BF) o += ww[(hh + G) * D + dd];
      O += o * f;
    }
    const int64_t hrow = int64_t(b) * a.Hq + g * G + hh;
    a.po[(hrow * a.max_splits + s) * D + dd] = O / Ls;
    if (dd == 0) a.pl[hrow * a.max_splits + s] = (M + __log2f(Ls)) * 0.6931471805599453f;
  }
}

// LSE combine of the split partials into the final output (one workgroup per (sequence, head)).
template <int D>
__global__ __launch_bounds__(D) void k_combine(const float* __restrict__ po, const float* __restrict__ pl,
                                               const int32_t* __restrict__ cnt, int G, int Hq, int Hk, int E,
                                               int max_splits, float* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y, dd = threadIdx.x;
  const int64_t hrow = int64_t(b) * Hq + h;
  const int c = cnt[int64_t(b) * Hk + h / G];
  const int ns = (c + E - 1) / E;
  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pl[hrow * max_splits + s]);
  float Ls = 0.f, O = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = __expf(pl[hrow * max_splits + s] - M);
    Ls += w;
    O += w * po[(hrow * max_splits + s) * D + dd];
  }
  out[hrow * D + dd] = ns ? O / Ls : 0.f;
  if (dd == 0) lse[hrow] = ns ? M + __logf(Ls) : kNegInf;
}

template <typename T>
T* at(char* ws, size_t off) {
  return reinterpret_cast<T*>(ws + off);
}

LongArgs long_args(const Plan& p, char* ws) {
  const sd_config& c = p.cfg;
  LongArgs a;
  a.s0 = at<double>(ws, p.o_s0);
  a.len = p.len0;
  a.Hq = c.n_q_heads;
  a.G = p.G;
  a.local_mask = p.local_mask;
  a.topp = c.mode == SD_TOPP;
  a.k = c.top_k;
  a.p = c.top_p;
  a.scale = c.mode == SD_TOPP ? c.select_scale : 1.0;
  a.info = at<RowInfo>(ws, p.o_info);
  a.pmax = at<double>(ws, p.o_pmax);
  a.pmin = at<double>(ws, p.o_pmin);
  a.nblk = p.score_blocks0;
  a.h1m = at<double>(ws, p.o_h1m);
  a.h1c = at<uint32_t>(ws, p.o_h1c);
  a.h2m = at<double>(ws, p.o_h2m);
  a.h2c = at<uint32_t>(ws, p.o_h2c);
  a.ckey = at<uint64_t>(ws, p.o_ckey);
  a.cidx = at<int32_t>(ws, p.o_cidx);
  a.ccnt = at<int32_t>(ws, p.o_ccnt);
  a.bits = at<uint32_t>(ws, p.o_bits);
  a.words = p.words;
  a.status = at<uint32_t>(ws, p.o_status);
  return a;
}

template <typename T, int D>
int score_impl(const Plan& p, const sd_tensors& t, int level, char* ws, hipStream_t st) {
  const sd_config& c = p.cfg;
  const int B = c.batch, Hq = c.n_q_heads, Hk = c.n_kv_heads;
  uint32_t* status = at<uint32_t>(ws, p.o_status);
  if (c.route == SD_ROUTE_PROXY) {
    const int nb = (Hq * 16 + 255) / 256;
    hipLaunchKernelGGL((k_proxy_query<T, D>), dim3(nb, B), dim3(256), 0, st, static_cast<const T*>(t.q), t.q_sb,
                       t.q_sh, t.proj, p.G, Hq, p.local_mask, at<double>(ws, p.o_qp), status);
    hipLaunchKernelGGL(k_score_proxy, dim3(p.score_blocks0, Hk, B), dim3(256), 0, st,
                       static_cast<const uint16_t*>(t.kp), t.kp_sb, t.kp_sh, t.kp_st, at<double>(ws, p.o_qp),
                       p.G, Hq, c.n_ctx, p.local_mask, at<double>(ws, p.o_s0), at<double>(ws, p.o_pmax),
                       at<double>(ws, p.o_pmin), p.score_blocks0);
    return int(hipGetLastError());
  }
  if (c.mode == SD_HIER_TOPK && level == 1) {
    hipLaunchKernelGGL((k_score_rows<T, D>), dim3((p.len1 + 63) / 64, Hq, B), dim3(256), 0, st,
                       static_cast<const T*>(t.q), t.q_sb, t.q_sh, static_cast<const T*>(t.kg), t.g_sb, t.g_sh,
                       t.g_st, at<int32_t>(ws, p.o_cand), p.len1, p.M, p.G, Hq, p.local_mask, at<double>(ws, p.o_s1),
                       p.len1, static_cast<uint32_t*>(nullptr));
    return int(hipGetLastError());
  }
  const bool meta = c.mode == SD_HIER_TOPK;
  hipLaunchKernelGGL((k_score_rows<T, D>), dim3((p.len0 + 63) / 64, Hk, B), dim3(256), 0, st,
                     static_cast<const T*>(t.q), t.q_sb, t.q_sh, static_cast<const T*>(meta ? t.kmg : t.kg),
                     meta ? t.mg_sb : t.g_sb, meta ? t.mg_sh : t.g_sh, meta ? t.mg_st : t.g_st,
                     static_cast<const int32_t*>(nullptr), p.len0, p.len0, p.G, Hq, p.local_mask, at<double>(ws, p.o_s0),
                     p.len0, status);
  if (p.long0)
    hipLaunchKernelGGL(k_row_minmax, dim3(p.score_blocks0, Hq, B), dim3(256), 0, st, at<double>(ws, p.o_s0),
                       p.len0, p.G, Hq, p.local_mask, at<double>(ws, p.o_pmax), at<double>(ws, p.o_pmin),
                       p.score_blocks0);
  return int(hipGetLastError());
}

int union_impl(const Plan& p, char* ws, hipStream_t st) {
  const sd_config& c = p.cfg;
  UnionArgs u;
  u.bits = at<uint32_t>(ws, p.o_bits);
  u.ubits = at<uint32_t>(ws, p.o_ubits);
  u.rcnt = at<int32_t>(ws, p.o_rcnt);
  u.list = at<int32_t>(ws, p.o_list);
  u.cnt = at<int32_t>(ws, p.o_cnt);
  u.words = p.words;
  u.n = p.M;
  u.Hq = c.n_q_heads;
  u.Hk = c.n_kv_heads;
  u.G = p.G;
  u.ranges = p.ranges;
  u.local_mask = p.local_mask;
  u.keep_first = c.keep_first;
  u.keep_last = c.keep_last;
  u.sink = c.sink;
  u.window = c.window;
  const dim3 grid(p.ranges, c.n_kv_heads, c.batch);
  hipLaunchKernelGGL(k_union_count, grid, dim3(256), 0, st, u);
  hipLaunchKernelGGL(k_union_write, grid, dim3(256), 0, st, u);
  return int(hipGetLastError());
}

}  // namespace

int launch_score(const Plan& p, const sd_tensors& t, int level, char* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sd_config& c = p.cfg;
  if (c.kv_dtype == SD_BF16)
    return c.head_dim == 128 ? score_impl<uint16_t, 128>(p, t, level, ws, st)
                             : score_impl<uint16_t, 64>(p, t, level, ws, st);
  return c.head_dim == 128 ? score_impl<float, 128>(p, t, level, ws, st) : score_impl<float, 64>(p, t, level, ws, st);
}

int launch_select(const Plan& p, int level, char* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sd_config& c = p.cfg;
  const int B = c.batch, Hq = c.n_q_heads;
  const bool topp = c.mode == SD_TOPP;
  const bool hier = c.mode == SD_HIER_TOPK;
  if (hier && level == 0) {
    hipLaunchKernelGGL(k_select_small, dim3(Hq, B), dim3(kSelThreads), 0, st, at<double>(ws, p.o_s0), p.len0, Hq,
                       p.G, p.local_mask, 0, c.top_k_seg, 1.0, 1.0, 1, static_cast<const int32_t*>(nullptr),
                       at<int32_t>(ws, p.o_cand), c.seg_size, p.len1, at<uint32_t>(ws, p.o_bits), p.words);
    return int(hipGetLastError());
  }
  if (hier) {
    hipLaunchKernelGGL(k_select_small, dim3(Hq, B), dim3(kSelThreads), 0, st, at<double>(ws, p.o_s1), p.len1, Hq,
                       p.G, p.local_mask, 0, c.top_k, 1.0, 1.0, 2, at<int32_t>(ws, p.o_cand),
                       static_cast<int32_t*>(nullptr), c.seg_size, p.len1, at<uint32_t>(ws, p.o_bits), p.words);
  } else if (!p.long0) {
    hipLaunchKernelGGL(k_select_small, dim3(Hq, B), dim3(kSelThreads), 0, st, at<double>(ws, p.o_s0), p.len0, Hq,
                       p.G, p.local_mask, topp ? 1 : 0, c.top_k, c.top_p, c.select_scale, 0,
                       static_cast<const int32_t*>(nullptr), static_cast<int32_t*>(nullptr), 0, 0,
                       at<uint32_t>(ws, p.o_bits), p.words);
  } else {
    const LongArgs a = long_args(p, ws);
    const dim3 rows(Hq, B), blocks(p.long_blocks, Hq, B);
    hipLaunchKernelGGL(k_long_prep, rows, dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_long_hist<1>, blocks, dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_long_find<1>, rows, dim3(kSelThreads), 0, st, a);
    hipLaunchKernelGGL(k_long_hist<2>, blocks, dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_long_find<2>, rows, dim3(kSelThreads), 0, st, a);
    hipLaunchKernelGGL(k_long_collect, blocks, dim3(256), 0, st, a);
    hipLaunchKernelGGL(k_long_resolve, rows, dim3(kSelThreads), 0, st, a);
  }
  int e = int(hipGetLastError());
  if (e) return e;
  return union_impl(p, ws, st);
}

int launch_attend(const Plan& p, const sd_tensors& t, char* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sd_config& c = p.cfg;
  AttendArgs a;
  a.q = t.q;
  a.q_sb = t.q_sb;
  a.q_sh = t.q_sh;
  a.k = t.k;
  a.v = t.v;
  a.kv_sb = t.kv_sb;
  a.kv_sh = t.kv_sh;
  a.kv_st = t.kv_st;
  a.kg = c.attend_summary ? t.kg : t.k;
  a.vg = c.attend_summary ? t.vg : t.v;
  a.g_sb = t.g_sb;
  a.g_sh = t.g_sh;
  a.g_st = c.attend_summary ? t.g_st : t.kv_st;
  a.list = at<int32_t>(ws, p.o_list);
  a.cnt = at<int32_t>(ws, p.o_cnt);
  a.po = at<float>(ws, p.o_po);
  a.pl = at<float>(ws, p.o_pl);
  a.n_list = p.M;
  a.G = p.G;
  a.Hq = c.n_q_heads;
  a.Hk = c.n_kv_heads;
  int cs = 0;
  while ((1 << cs) < c.chunk_size) ++cs;
  a.chunk_shift = cs;
  a.E = p.split_entries;
  a.max_splits = p.max_splits;
  a.attend_summary = c.attend_summary;
  a.scale_log2 = c.softmax_scale * 1.4426950408889634f;
  const dim3 grid(p.max_splits, c.n_kv_heads, c.batch);
  if (c.kv_dtype == SD_BF16) {
    if (c.head_dim == 128)
      hipLaunchKernelGGL((k_attend<uint16_t, 128>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_attend<uint16_t, 64>), grid, dim3(256), 0, st, a);
  } else {
    if (c.head_dim == 128)
      hipLaunchKernelGGL((k_attend<float, 128>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_attend<float, 64>), grid, dim3(256), 0, st, a);
  }
  return int(hipGetLastError());
}

int launch_combine(const Plan& p, char* ws, float* out, float* lse, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sd_config& c = p.cfg;
  const dim3 grid(c.n_q_heads, c.batch);
  if (c.head_dim == 128)
    hipLaunchKernelGGL(k_combine<128>, grid, dim3(128), 0, st, at<float>(ws, p.o_po), at<float>(ws, p.o_pl),
                       at<int32_t>(ws, p.o_cnt), p.G, c.n_q_heads, c.n_kv_heads, p.split_entries, p.max_splits, out,
                       lse);
  else
    hipLaunchKernelGGL(k_combine<64>, grid, dim3(64), 0, st, at<float>(ws, p.o_po), at<float>(ws, p.o_pl),
                       at<int32_t>(ws, p.o_cnt), p.G, c.n_q_heads, c.n_kv_heads, p.split_entries, p.max_splits, out,
                       lse);
  return int(hipGetLastError());
}

const char* hip_error_string(int code) { return hipGetErrorString(static_cast<hipError_t>(code)); }

}  // namespace sd
