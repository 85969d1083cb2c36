// Selection kernels: per-head top-k / top-p / two-level, GQA union and compaction.
//
// Compiled with -ffp-contract=off: every fused multiply-add is an explicit fma(), so fp64 score
// arithmetic can be matched bit for bit by a sequential CPU evaluation.
#include "sd_device.h"

namespace sd {
namespace {
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

}  // namespace sd
