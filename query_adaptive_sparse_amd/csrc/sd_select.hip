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
template <typename Idx, int NT = kSelThreads>
__device__ void bitonic_desc(uint64_t* keys, Idx* idx, int Lp) {
  for (int kk = 2; kk <= Lp; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < Lp; i += NT) {
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
// Selection of rows up to kSmallRowMax entries, fused with the GQA union and the compaction.
// One 256-thread workgroup per (sequence, query head); the row lives in registers, at most
// kLaneEntries per lane:
//   1. fp64 scores, their range and, for top-p, the masses w = exp(scale*s - scale*smax) and Z
//      (fixed-order DPP reductions: every lane holds the same bits);
//   2. a 256-bin histogram of the weights (mass, or 1 for top-k) over the bins of (smax - s)
//      finds the bin where the running weight reaches the target (p*Z or k); if that bin holds
//      more than kCandCap entries a second 256-bin level splits it;
//   3. the crossing bin's entries are ranked in (score desc, index asc) order by counting and
//      their weights walked from the weight of everything ahead of the bin to the first crossing.
// Bins are monotone in the score, so every entry of an earlier bin precedes every entry of a
// later bin in the order: the result equals the sorted-prefix rule. A crossing bin still holding
// more than kCandCap entries after two levels (a mass of near-equal scores) falls back to a full
// sort of the row in LDS.
// The last workgroup of a group to finish (arrival counter; release / acquire fences at device
// scope) ORs the group's per-head bitmaps with the forced or local entries and writes the
// ascending list.
// kind 0: flat rows. kind 1: two-level, level 0 (kept segments -> ascending candidate chunk
// lists, no union). kind 2: two-level, level 1 (kept candidates -> chunk bitmaps -> union).
// ---------------------------------------------------------------------------------------------
constexpr int kNBin = 256;
constexpr int kCandCap = 256;
constexpr int kSelT = 256;                          // threads per head
constexpr int kSelW = kSelT / 64;                   // waves per head
constexpr int kLaneEntries = kSmallRowMax / kSelT;  // 8
constexpr int kUnionWordsMax = 4096;

struct GroupSelArgs {
  const double* s;
  int64_t len;  // row length (entries scored per head)
  int Hq, Hk, G;
  uint64_t local_mask;
  int topp, k;
  double p, scale;
  int kind;
  const int32_t* cand_in;  // kind 2: [B][Hq][len] chunk id of each candidate
  int32_t* cand_out;       // kind 1: [B][Hq][cand_len]
  int seg_size;
  int64_t cand_len;
  uint32_t* bits;  // per-head bitmaps [B][Hq][words]
  int64_t words;
  int32_t* list;      // [B][Hk][n_entries]
  int32_t* cnt;       // [B][Hk]
  int32_t* arrivals;  // [B][Hk], cleared by the score pass
  int64_t n_entries;
  int keep_first, keep_last, sink, window;
};

// Bin of a score: coarse bin of (smax - s) over the row's range, and its fine sub-bin.
__device__ __forceinline__ void bins_of(double s, double smax, double binscale, int* c1, int* c2) {
  double d = (smax - s) * binscale;
  d = d >= 0.0 ? (d < double(kNBin) ? d : double(kNBin)) : 0.0;
  int b = int(d);
  b = b < kNBin - 1 ? b : kNBin - 1;
  *c1 = b;
  int f = int((d - double(b)) * double(kNBin));
  *c2 = f < 0 ? 0 : (f < kNBin - 1 ? f : kNBin - 1);
}

__global__ __launch_bounds__(kSelT) void k_select_head(GroupSelArgs a) {
  __shared__ double hm[kNBin];
  __shared__ uint32_t hc[kNBin];
  __shared__ uint64_t ckey[kCandCap];
  __shared__ double cw[kCandCap];
  __shared__ double rw[kCandCap];
  __shared__ uint16_t cidx[kCandCap];
  __shared__ uint16_t ridx[kCandCap];
  __shared__ uint32_t selb[kSmallRowMax / 32];
  __shared__ uint32_t ubits[kUnionWordsMax];
  __shared__ uint64_t fkey[kSmallRowMax];  // whole-row fallback sort
  __shared__ uint16_t fidx[kSmallRowMax];
  __shared__ double wred[kSelW], wred2[kSelW];
  __shared__ int wcnt[kSelW];
  __shared__ double res_d;
  __shared__ int res_i, res_state, ncand, is_last;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.G, g = h / G;
  const int L = int(a.len);
  const bool local = (a.local_mask >> g) & 1;
  const int64_t row = int64_t(b) * a.Hq + h;
  const int words_row = (L + 31) / 32;

  for (int w = tid; w < words_row; w += kSelT) selb[w] = 0;
  for (int i = tid; i < kNBin; i += kSelT) {
    hm[i] = 0.0;
    hc[i] = 0;
  }
  if (tid == 0) ncand = 0;

  // ---- 1. scores (unconditional, clamped loads), range, weights, target
  double sv[kLaneEntries], wt[kLaneEntries];
  const int EPL = (L + kSelT - 1) / kSelT;
#pragma unroll
  for (int k = 0; k < kLaneEntries; ++k) {
    const int i = tid + kSelT * k;
    sv[k] = local ? 0.0 : a.s[row * a.len + (i < L ? i : L - 1)];
  }
  double smax = kNegInfD, smin = kPosInfD;
#pragma unroll
  for (int k = 0; k < kLaneEntries; ++k) {
    if (tid + kSelT * k < L) {
      smax = fmax(smax, sv[k]);
      smin = fmin(smin, sv[k]);
    }
  }
  smax = wave_max_dpp(smax);
  smin = wave_min_dpp(smin);
  if (lane == 0) {
    wred[wv] = smax;
    wred2[wv] = smin;
  }
  __syncthreads();
  smax = fmax(fmax(wred[0], wred[1]), fmax(wred[2], wred[3]));
  smin = fmin(fmin(wred2[0], wred2[1]), fmin(wred2[2], wred2[3]));
  __syncthreads();
  const bool all = a.topp ? (a.p >= 1.0) : (a.k >= L);
  const double ellmax = a.scale * smax;
  const double range = smax - smin;
  const double binscale = range > 0.0 ? double(kNBin) / range : 0.0;
  const bool work = !local && !all;
  double z = 0.0;
#pragma unroll
  for (int k = 0; k < kLaneEntries; ++k) {
    wt[k] = 0.0;
    if (work && k < EPL && tid + kSelT * k < L) {
      wt[k] = a.topp ? exp(a.scale * sv[k] - ellmax) : 1.0;
      z += wt[k];
    }
  }
  double target = double(a.k);
  if (a.topp) {
    z = wave_sum_dpp(z);
    if (lane == 0) wred[wv] = z;
    __syncthreads();
    target = a.p * ((wred[0] + wred[1]) + (wred[2] + wred[3]));
  }

  // ---- 2. histograms (two levels at most) and the crossing bin
  // state: 0 = next level, 1 / 2 = resolved at that level, 3 = fallback, 4 = every entry,
  // 5 = the whole crossing coarse bin, 6 = nothing to select (local head)
  int state = local ? 6 : (all ? 4 : 0);
  int b1 = 0, b2 = 0;
  double before = 0.0;
  for (int lv = 1; lv <= 2 && state == 0; ++lv) {
#pragma unroll
    for (int k = 0; k < kLaneEntries; ++k) {
      if (k < EPL && tid + kSelT * k < L) {
        int c1, c2;
        bins_of(sv[k], smax, binscale, &c1, &c2);
        if (lv == 2 && c1 != b1) continue;
        const int bin = lv == 1 ? c1 : c2;
        unsafeAtomicAdd(&hm[bin], wt[k]);
        atomicAdd(&hc[bin], 1u);
      }
    }
    __syncthreads();
    if (wv == 0) {
      double wl = 0.0;
      for (int j = 0; j < 4; ++j) wl += hm[4 * lane + j];
      const double incl = wave_scan_dpp(wl, lane);
      double c = before + (incl - wl);
      int hit = -1;
      double before_hit = 0.0;
      for (int j = 0; j < 4 && hit < 0; ++j) {
        const double cn = c + hm[4 * lane + j];
        if (cn >= target) {
          hit = 4 * lane + j;
          before_hit = c;
        }
        c = cn;
      }
      const uint64_t m = __ballot(hit >= 0);
      const int first = m ? __ffsll((unsigned long long)m) - 1 : 0;
      const int hb = __builtin_amdgcn_readlane(hit, first);  // first is wave-uniform
      const double bb = readlane_f64(before_hit, first);
      if (lane == 0) {
        if (!m) {
          // rounding left the target above the weight of the scanned bins: at level 1 every
          // entry is kept; at level 2 the whole crossing coarse bin is
          res_state = lv == 1 ? 4 : 5;
        } else {
          res_i = hb;
          res_d = bb;
          res_state = hc[hb] <= uint32_t(kCandCap) ? lv : (lv == 2 ? 3 : 0);
        }
      }
    }
    __syncthreads();
    state = res_state;
    if (state != 4 && state != 5) {
      if (lv == 1) b1 = res_i; else b2 = res_i;
      before = res_d;
    }
    if (state == 0) {
      for (int i = tid; i < kNBin; i += kSelT) {
        hm[i] = 0.0;
        hc[i] = 0;
      }
      __syncthreads();
    }
  }

  // ---- 3. mark entries ahead of the crossing bin (ballots), gather the crossing bin's entries
  const bool marking = state == 1 || state == 2 || state == 4 || state == 5;
#pragma unroll
  for (int k = 0; k < kLaneEntries; ++k) {
    if (k < EPL) {  // uniform across the workgroup
      const int i = tid + kSelT * k;
      bool sel = false, cand = false;
      if (marking && i < L) {
        sel = state == 4;
        if (state != 4) {
          int c1, c2;
          bins_of(sv[k], smax, binscale, &c1, &c2);
          if (state == 1) {
            sel = c1 < b1;
            cand = c1 == b1;
          } else {
            sel = c1 < b1 || (c1 == b1 && (state == 5 || c2 < b2));
            cand = state == 2 && c1 == b1 && c2 == b2;
          }
        }
      }
      const uint64_t ms = __ballot(sel);
      const int wbase = tid - lane + kSelT * k;  // first entry of this wave's 64
      if (lane == 0 && wbase < L) selb[wbase >> 5] = uint32_t(ms);
      if (lane == 1 && wbase + 32 < L) selb[(wbase >> 5) + 1] = uint32_t(ms >> 32);
      const uint64_t mc = __ballot(cand);
      if (mc) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&ncand, __popcll(mc));
        base = __builtin_amdgcn_readlane(base, 0);
        if (cand) {
          const int pos = base + __builtin_amdgcn_mbcnt_hi(uint32_t(mc >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mc), 0));
          ckey[pos] = dkey(sv[k]);
          cidx[pos] = uint16_t(i);
          cw[pos] = wt[k];
        }
      }
    }
  }
  __syncthreads();

  // ---- 4. order the candidates (ranks by counting) or, in the fallback, the whole row (sort),
  // then walk their weights from the weight ahead of them to the first crossing
  int n = 0;
  const double* wo = rw;         // weights in order
  const uint16_t* io = ridx;     // entries in order
  if (state == 1 || state == 2) {
    n = ncand;
    for (int c = tid; c < n; c += kSelT) {
      const uint64_t kc = ckey[c];
      const uint16_t ic = cidx[c];
      int r = 0;
      for (int d = 0; d < n; ++d) {
        const uint64_t kd = ckey[d];
        r += (kd > kc || (kd == kc && cidx[d] < ic)) ? 1 : 0;
      }
      rw[r] = cw[c];
      ridx[r] = ic;
    }
  } else if (state == 3) {
    n = L;
    int lp = 2;
    while (lp < L) lp <<= 1;
    for (int i = tid; i < lp; i += kSelT) {
      fkey[i] = i < L ? dkey(a.s[row * a.len + i]) : 0ull;
      fidx[i] = uint16_t(i < L ? i : 0xFFFF);
    }
    __syncthreads();
    bitonic_desc<uint16_t, kSelT>(fkey, fidx, lp);
    double* fw = reinterpret_cast<double*>(fkey);  // weights replace the keys in place
    for (int i = tid; i < L; i += kSelT) fw[i] = a.topp ? exp(a.scale * dkey_inv(fkey[i]) - ellmax) : 1.0;
    wo = fw;
    io = fidx;
    before = 0.0;
  }
  __syncthreads();
  if (n > 0) {
    const int per = (n + kSelT - 1) / kSelT;
    const int i0 = tid * per;
    double lw = 0.0;
    for (int i = i0; i < min(n, i0 + per); ++i) lw += wo[i];
    const double incl = wave_scan_dpp(lw, lane);
    if (lane == 63) wred[wv] = incl;
    __syncthreads();
    double c = before + incl - lw;
    for (int w = 0; w < wv; ++w) c += wred[w];
    int cross = 0x7FFFFFFF;
    for (int i = i0; i < min(n, i0 + per); ++i) {
      c += wo[i];
      if (c >= target) {
        cross = i + 1;
        break;
      }
    }
    cross = wave_min_i32_dpp(cross);
    if (lane == 0) wcnt[wv] = cross;
    __syncthreads();
    const int nsel = min(min(n, min(wcnt[0], wcnt[1])), min(wcnt[2], wcnt[3]));
    for (int i = tid; i < nsel; i += kSelT) {
      const int e = io[i];
      atomicOr(&selb[e >> 5], 1u << (e & 31));
    }
  }
  __syncthreads();

  // ---- 5. per-head outputs
  if (a.kind == 1) {
    // kept segments in ascending order -> candidate chunk lists (first wave)
    if (!local && wv == 0) {
      int base = 0;
      for (int w0 = 0; w0 < words_row; w0 += 64) {
        const int w = w0 + lane;
        const int pc = w < words_row ? __popc(selb[w]) : 0;
        const int incl = wave_scan_i32_dpp(pc, lane);
        int rank = base + incl - pc;
        if (w < words_row) {
          uint32_t m = selb[w];
          while (m) {
            const int bit = __ffs(m) - 1;
            m &= m - 1;
            const int seg = w * 32 + bit;
            for (int j = 0; j < a.seg_size; ++j)
              a.cand_out[row * a.cand_len + int64_t(rank) * a.seg_size + j] = seg * a.seg_size + j;
            ++rank;
          }
        }
        base += __builtin_amdgcn_readlane(incl, 63);
      }
    }
    return;
  }
  if (a.kind == 0) {
    for (int w = tid; w < a.words; w += kSelT) a.bits[row * a.words + w] = (!local && w < words_row) ? selb[w] : 0u;
  } else {
    for (int w = tid; w < a.words; w += kSelT) a.bits[row * a.words + w] = 0u;
    __syncthreads();  // the zeroing stores complete before the atomics below
    if (!local)
      for (int w = tid; w < words_row; w += kSelT) {
        uint32_t m = selb[w];
        while (m) {
          const int bit = __ffs(m) - 1;
          m &= m - 1;
          int e = a.cand_in[row * a.len + w * 32 + bit];
          e = e < 0 ? 0 : (e < int(a.n_entries) ? e : int(a.n_entries) - 1);
          atomicOr(&a.bits[row * a.words + (e >> 5)], 1u << (e & 31));
        }
      }
  }

  // ---- 6. the group's last workgroup builds the union and the ascending list
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  const int64_t grp = int64_t(b) * a.Hk + g;
  if (tid == 0) is_last = atomicAdd(&a.arrivals[grp], 1) == G - 1;
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int uwords = int((a.n_entries + 31) / 32);
  {
    const int64_t first = local ? a.sink : a.keep_first;
    const int64_t last = local ? a.window : a.keep_last;
    for (int w = tid; w < uwords; w += kSelT) {
      uint32_t u = edge_bits(w, a.n_entries, first, last);
      if (!local)
        for (int j = 0; j < G; ++j)
          u |= __builtin_nontemporal_load(&a.bits[(int64_t(b) * a.Hq + g * G + j) * a.words + w]);
      ubits[w] = u;
    }
  }
  if (tid == 0) a.arrivals[grp] = 0;
  __syncthreads();
  const int per = (uwords + kSelT - 1) / kSelT;  // <= 16
  const int w0 = tid * per;
  int pc = 0;
  for (int w = w0; w < min(uwords, w0 + per); ++w) pc += __popc(ubits[w]);
  const int incl = wave_scan_i32_dpp(pc, lane);
  if (lane == 63) wcnt[wv] = incl;
  __syncthreads();
  int pos = incl - pc;
  for (int w = 0; w < wv; ++w) pos += wcnt[w];
  int32_t* out = a.list + grp * a.n_entries;
  for (int w = w0; w < min(uwords, w0 + per); ++w) {
    uint32_t m = ubits[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      out[pos++] = w * 32 + bit;
    }
  }
  if (tid == kSelT - 1) a.cnt[grp] = pos;
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

GroupSelArgs group_args(const Plan& p, char* ws, int level) {
  const sd_config& c = p.cfg;
  const bool hier = c.mode == SD_HIER_TOPK;
  GroupSelArgs a;
  a.s = at<double>(ws, hier && level == 1 ? p.o_s1 : p.o_s0);
  a.len = hier && level == 1 ? p.len1 : p.len0;
  a.Hq = c.n_q_heads;
  a.Hk = c.n_kv_heads;
  a.G = p.G;
  a.local_mask = p.local_mask;
  a.topp = c.mode == SD_TOPP;
  a.k = hier && level == 0 ? c.top_k_seg : c.top_k;
  a.p = c.top_p;
  a.scale = c.mode == SD_TOPP ? c.select_scale : 1.0;
  a.kind = hier ? (level == 0 ? 1 : 2) : 0;
  a.cand_in = at<int32_t>(ws, p.o_cand);
  a.cand_out = at<int32_t>(ws, p.o_cand);
  a.seg_size = c.seg_size;
  a.cand_len = p.len1;
  a.bits = at<uint32_t>(ws, p.o_bits);
  a.words = p.words;
  a.list = at<int32_t>(ws, p.o_list);
  a.cnt = at<int32_t>(ws, p.o_cnt);
  a.arrivals = at<int32_t>(ws, p.o_arrive);
  a.n_entries = p.M;
  a.keep_first = c.keep_first;
  a.keep_last = c.keep_last;
  a.sink = c.sink;
  a.window = c.window;
  return a;
}

}  // namespace

int launch_select(const Plan& p, int level, char* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sd_config& c = p.cfg;
  const int B = c.batch, Hq = c.n_q_heads;
  if (c.mode == SD_HIER_TOPK || !p.long0) {
    // rows of at most kSmallRowMax entries: selection, union and compaction in one kernel
    hipLaunchKernelGGL(k_select_head, dim3(Hq, B), dim3(kSelT), 0, st, group_args(p, ws, level));
    return int(hipGetLastError());
  }
  const LongArgs a = long_args(p, ws);
  const dim3 rows(Hq, B), blocks(p.long_blocks, Hq, B);
  hipLaunchKernelGGL(k_long_prep, rows, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_long_hist<1>, blocks, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_long_find<1>, rows, dim3(kSelThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_hist<2>, blocks, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_long_find<2>, rows, dim3(kSelThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_collect, blocks, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_long_resolve, rows, dim3(kSelThreads), 0, st, a);
  int e = int(hipGetLastError());
  if (e) return e;
  return union_impl(p, ws, st);
}

}  // namespace sd
