// Selection kernels: per-head top-k / top-p / two-level, GQA union and compaction.
//
// Compiled with -ffp-contract=off: every fused multiply-add is an explicit fma(), so fp64 score
// arithmetic can be matched bit for bit by a sequential CPU evaluation.
#include "sd_device.h"
#include "long_rows.h"

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

// ---------------------------------------------------------------------------------------------
// Exact, order-independent histogram masses. A weight w in [0, 1] is held as two integers,
// hi = floor(w 2^39) and lo = floor((w 2^39 - hi) 2^40): w to a resolution of 2^-79 (exactly when
// w >= 2^-26; a smaller weight loses less than 2^-79). Integer addition is associative, so the
// bin sums that workgroups build with LDS atomics, and the slab partials summed afterwards, hold
// the same bits whatever order the entries arrive in. Up to 2^24 weights sum without overflow, so
// rows are limited to kMaxRowEntries
// (hi sums stay below 2^63, lo sums below 2^64); a sum's value is hi 2^-39 + lo 2^-79, rounded
// once per word when converted to fp64.
// ---------------------------------------------------------------------------------------------
constexpr int kFixLoBits = 40;
constexpr uint64_t kFixLoMask = (uint64_t(1) << kFixLoBits) - 1;
static_assert(kMaxRowEntries <= (int64_t(1) << 24), "fixed-point sums of a row must not overflow");
struct FixW {
  uint64_t hi, lo;
};
__device__ __forceinline__ FixW fix_of(double w) {
  const double x = w * 0x1p39;  // exact: a power-of-two scaling
  const double h = floor(x);
  const double f = floor((x - h) * 0x1p40);  // x - h and the scaling are exact
  // h and f are integers below 2^52: added to 2^52 they sit in the low mantissa bits
  constexpr uint64_t kMant = (uint64_t(1) << 52) - 1;
  return FixW{uint64_t(__double_as_longlong(h + 0x1p52)) & kMant, uint64_t(__double_as_longlong(f + 0x1p52)) & kMant};
}
__device__ __forceinline__ double fix_value(uint64_t hi, uint64_t lo) {
  hi += lo >> kFixLoBits;  // whole 2^-39 units of the low word
  lo &= kFixLoMask;
  return double(hi) * 0x1p-39 + double(lo) * 0x1p-79;
}
__device__ __forceinline__ void fix_add(unsigned long long* hi, unsigned long long* lo, double w) {
  const FixW f = fix_of(w);
  atomicAdd(hi, (unsigned long long)f.hi);
  atomicAdd(lo, (unsigned long long)f.lo);
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
// Selection of rows up to kSmallRowMax entries (the GQA union and the compaction follow in
// k_union_small). One 256-thread workgroup per (sequence, query head); the row lives in registers, at most
// kLaneEntries per lane:
//   1. fp64 scores, their range and, for top-p, the masses w = exp(scale*s - scale*smax) and Z
//      (fixed-order DPP reductions: every lane holds the same bits);
//   2. a 256-bin histogram of the weights (mass, or 1 for top-k) over the bins of (smax - s)
//      finds the bin where the running weight reaches the target (p*Z or k); if that bin holds
//      more than kRankDirect entries a second 256-bin level splits it;
//   3. the crossing bin's entries are ranked in (score desc, index asc) order by counting and
//      their weights walked from the weight of everything ahead of the bin to the first crossing.
// Bins are monotone in the score, so every entry of an earlier bin precedes every entry of a
// later bin in the order: the result equals the sorted-prefix rule. A crossing bin still holding
// more than kCandCap entries after two levels (a mass of near-equal scores) falls back to a full
// sort of the row in LDS. k_union_small then ORs each group's per-head bitmaps with the forced or
// local entries and writes the ascending list.
// kind 0: flat rows. kind 1: two-level, level 0 (kept segments -> ascending candidate chunk
// lists, no union). kind 2: two-level, level 1 (kept candidates -> chunk bitmaps -> union).
// ---------------------------------------------------------------------------------------------
constexpr int kNBin = 256;
constexpr int kCandCap = 256;
// A crossing coarse bin of more entries than this is split by the second level before ranking
// (ranking by counting costs n^2 LDS reads).
constexpr int kRankDirect = 16;
constexpr int kSelT = 256;                          // threads per head
// entry count of a short-row bin, kept in the high bits of its low mass word (a row of at most
// kSmallRowMax = 2^11 entries: low parts sum below 2^51, counts times 2^52 stay below 2^64)
constexpr int kCountShift = 52;
constexpr uint64_t kCountOne = uint64_t(1) << kCountShift;
static_assert(kSmallRowMax <= 2048, "short-row bin counts share the low mass word");
constexpr int kSelW = kSelT / 64;                   // waves per head
constexpr int kLaneEntries = kSmallRowMax / kSelT;  // 8
constexpr int kUnionWordsMax = 4096;

struct GroupSelArgs {
  const double* s;
  int64_t len;  // row length (entries scored per head)
  int Hq, Hk, G;
  uint64_t local_mask;
  int topp, k;
  const int32_t* kbudget;  // per-sequence top-k (coverage budget), or NULL: k
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
  // growing cache: tokens per sequence (device [B], or NULL: n_ctx); a flat row of sequence b holds
  // its complete chunks, ctx_len[b] >> chunk_shift of them
  const int32_t* ctx_len;
  int64_t n_ctx;
  int chunk_shift;
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
  // bin masses (exact fixed point, see fix_of): high words, and low words with the bin's entry
  // count in bits kCountShift and up (a row's low parts sum below 2^51)
  __shared__ unsigned long long hhi[kNBin];
  __shared__ unsigned long long hlo[kNBin];
  __shared__ uint64_t ckey[kCandCap];
  __shared__ double cw[kCandCap];
  __shared__ double rw[kCandCap];
  __shared__ uint16_t cidx[kCandCap];
  __shared__ uint16_t ridx[kCandCap];
  __shared__ uint32_t selb[kSmallRowMax / 32];
  __shared__ uint64_t fkey[kSmallRowMax];  // whole-row fallback sort
  __shared__ uint16_t fidx[kSmallRowMax];
  __shared__ double wred[kSelW], wred2[kSelW];
  __shared__ int wcnt[kSelW];
  __shared__ double res_d;
  __shared__ int res_i, res_state, ncand, nkept;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.G, g = h / G;
  // entries of this sequence's rows and of its union (the whole row without a growing cache)
  const int64_t n_ent = a.ctx_len ? (seq_tokens(a.ctx_len, b, a.n_ctx) >> a.chunk_shift) : a.n_entries;
  const int L = a.kind == 0 ? int(n_ent) : int(a.len);
  const bool local = (a.local_mask >> g) & 1;
  const int64_t row = int64_t(b) * a.Hq + h;
  const int words_row = (L + 31) / 32;

  for (int w = tid; w < kSmallRowMax / 32; w += kSelT) selb[w] = 0;
  for (int i = tid; i < kNBin; i += kSelT) {
    hhi[i] = 0;
    hlo[i] = 0;
  }
  if (tid == 0) ncand = 0;

  // ---- 1. scores (unconditional loads clamped to the row's capacity, so they do not wait for the
  // row's length; entries past it are never used), range, weights, target
  double sv[kLaneEntries], wt[kLaneEntries];
  const int EPL = (L + kSelT - 1) / kSelT;
  const int cap = int(a.len);
#pragma unroll
  for (int k = 0; k < kLaneEntries; ++k) {
    const int i = tid + kSelT * k;
    sv[k] = local ? 0.0 : a.s[row * a.len + (i < cap ? i : cap - 1)];
  }
  // candidate rows: the chunk id of each of the lane's entries, loaded with the scores (the bitmap
  // of the chosen chunks is built from them at the end)
  int32_t cid[kLaneEntries];
#pragma unroll
  for (int k = 0; k < kLaneEntries; ++k) {
    const int i = tid + kSelT * k;
    cid[k] = (a.kind == 2 && !local && k < EPL) ? a.cand_in[row * a.len + (i < cap ? i : cap - 1)] : 0;
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
  const int kk = a.kbudget ? a.kbudget[b] : a.k;
  const bool all = a.topp ? (a.p >= 1.0) : (kk >= L);
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
  double target = double(kk);
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
        if (a.topp) {
          const FixW f = fix_of(wt[k]);
          atomicAdd(&hhi[bin], (unsigned long long)f.hi);
          atomicAdd(&hlo[bin], (unsigned long long)(f.lo + kCountOne));
        } else {
          atomicAdd(&hlo[bin], (unsigned long long)kCountOne);  // unit weights: the mass is the count
        }
      }
    }
    __syncthreads();
    if (wv == 0) {
      double hm[4];
      for (int j = 0; j < 4; ++j) {
        const int bn = 4 * lane + j;
        hm[j] = a.topp ? fix_value(hhi[bn], hlo[bn] & (kCountOne - 1)) : double(hlo[bn] >> kCountShift);
      }
      double wl = 0.0;
      for (int j = 0; j < 4; ++j) wl += hm[j];
      const double incl = wave_scan_dpp(wl, lane);
      double c = before + (incl - wl);
      int hit = -1;
      double before_hit = 0.0;
      for (int j = 0; j < 4 && hit < 0; ++j) {
        const double cn = c + hm[j];
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
          const uint32_t n_hb = uint32_t(hlo[hb] >> kCountShift);
          res_state = n_hb <= uint32_t(lv == 1 ? kRankDirect : kCandCap) ? lv : (lv == 2 ? 3 : 0);
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
        hhi[i] = 0;
        hlo[i] = 0;
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
    // kept segments in ascending order, as a list in LDS (the fallback sort's index array is free
    // now), then their candidate chunk ids, written by every thread
    uint16_t* segs = fidx;
    if (wv == 0) {
      int base = 0;
      for (int w0 = 0; w0 < words_row; w0 += 64) {
        const int w = w0 + lane;
        uint32_t m = (!local && w < words_row) ? selb[w] : 0u;
        const int pc = __popc(m);
        const int incl = wave_scan_i32_dpp(pc, lane);
        int rank = base + incl - pc;
        while (m) {
          const int bit = __ffs(m) - 1;
          m &= m - 1;
          segs[rank++] = uint16_t(w * 32 + bit);
        }
        base += __builtin_amdgcn_readlane(incl, 63);
      }
      if (lane == 0) nkept = base;
    }
    __syncthreads();
    const int total = nkept * a.seg_size;
    int32_t* co = a.cand_out + row * a.cand_len;
    for (int e = tid; e < total; e += kSelT) {
      const int r = e / a.seg_size;
      co[e] = int(segs[r]) * a.seg_size + (e - r * a.seg_size);
    }
    return;
  }
  if (a.kind == 0) {
    for (int w = tid; w < a.words; w += kSelT) a.bits[row * a.words + w] = (!local && w < words_row) ? selb[w] : 0u;
  } else {
    // the chosen candidates' chunk ids as a bitmap over the chunks: built in LDS (the fallback
    // sort's key array is free now) and stored whole, or, past its size, cleared and set in place
    const bool in_lds = a.words <= int64_t(2 * kSmallRowMax);
    uint32_t* hb = in_lds ? reinterpret_cast<uint32_t*>(fkey) : a.bits + row * a.words;
    for (int w = tid; w < a.words; w += kSelT) hb[w] = 0u;
    __syncthreads();  // the zeroing stores complete before the atomics below
    if (!local)
#pragma unroll
      for (int k = 0; k < kLaneEntries; ++k) {
        const int i = tid + kSelT * k;
        if (k < EPL && i < L && ((selb[i >> 5] >> (i & 31)) & 1u)) {
          int e = cid[k];
          e = e < 0 ? 0 : (e < int(a.n_entries) ? e : int(a.n_entries) - 1);
          atomicOr(&hb[e >> 5], 1u << (e & 31));
        }
      }
    if (in_lds) {
      __syncthreads();
      for (int w = tid; w < a.words; w += kSelT) a.bits[row * a.words + w] = hb[w];
    }
  }
}

// GQA union and compaction of short rows, one workgroup per (sequence, KV group), launched after
// k_select_head: the OR of the group's per-head bitmaps with the forced entries (scored groups) or
// the sink + window (local groups), then its set bits in ascending order and their count. A launch
// of its own costs less than a last-arriving-workgroup hand-off inside k_select_head (device-scope
// release / acquire, then a wait for the group's slowest head): at 128K context score + select
// measured 25.8 us against 29.0 us with the hand-off (one box).
__global__ __launch_bounds__(kSelT) void k_union_small(GroupSelArgs a) {
  __shared__ uint32_t ubits[kUnionWordsMax];
  __shared__ int wcnt[kSelW];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = blockIdx.x, b = blockIdx.y;
  const int G = a.G;
  const bool local = (a.local_mask >> g) & 1;
  const int64_t n_ent = a.ctx_len ? (seq_tokens(a.ctx_len, b, a.n_ctx) >> a.chunk_shift) : a.n_entries;
  const int uwords = int((n_ent + 31) / 32);
  const int64_t first = local ? a.sink : a.keep_first;
  const int64_t last = local ? a.window : a.keep_last;
  for (int w = tid; w < uwords; w += kSelT) {
    uint32_t u = edge_bits(w, n_ent, first, last);
    if (!local)
      // the heads' words 8 at a time, every load of a block issued before the first is used
      // (heads past the group repeat its last head: the OR is unchanged)
      for (int j0 = 0; j0 < G; j0 += 8) {
        uint32_t v[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = j0 + jj < G ? j0 + jj : G - 1;
          v[jj] = a.bits[(int64_t(b) * a.Hq + g * G + j) * a.words + w];
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) u |= v[jj];
      }
    ubits[w] = u;
  }
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
  const int64_t grp = int64_t(b) * a.Hk + g;
  int32_t* out = a.list + grp * a.n_entries;
  if (uwords <= kSmallRowMax / 32) {
    // rows of at most kSmallRowMax entries: the list is expanded in LDS, then copied out with
    // coalesced stores
    __shared__ int32_t stage[kSmallRowMax];
    __shared__ int total;
    for (int w = w0; w < min(uwords, w0 + per); ++w) {
      uint32_t m = ubits[w];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        stage[pos++] = w * 32 + bit;
      }
    }
    if (tid == kSelT - 1) total = pos;
    __syncthreads();
    const int n = total;
    for (int i = tid; i < n; i += kSelT) out[i] = stage[i];
    if (tid == 0) a.cnt[grp] = n;
    return;
  }
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
// Selection of long rows (more than kSmallRowMax entries: token-level proxy rows, or fine chunk
// rows). The (score desc, index asc) order is resolved through a coarse histogram of the weights
// over the bins of (smax - s) on the row's score range, then the entries of the coarse bin where
// the running weight crosses the target. Weight = softmax mass exp(scale*s - scale*smax) for
// top-p, 1 for top-k. Bins are monotone in the score, so every entry of an earlier bin precedes
// every entry of a later one in the order. Histogram masses are exact fixed-point sums (fix_of),
// so they do not depend on the order of the atomic adds. Passes:
//   hist     per slab of kLongBlock entries: coarse bin of every entry (kept, 2 bytes), partial
//            coarse histogram (no atomics across workgroups);
//   sum      per row: bin totals (slab partials summed as integers), spread over many workgroups;
//   mark     per slab: Z, the target, the crossing coarse bin and the weight ahead of it (each
//            workgroup of the row scans the totals itself), bitmap words of the entries of
//            earlier coarse bins, the number of the
//            crossing bin's entries in the slab and (up to kResolveCap of them) their indices in
//            the slab's own region of the resolution buffer;
//   resolve  per row: when the crossing bin holds at most kResolveCap entries, they are split by a
//            sub-bin histogram of their interval; earlier sub-bins are selected, the crossing
//            sub-bin's entries are ranked and walked to the first crossing. A fuller crossing bin
//            (near-equal or tied scores) is narrowed by radix levels over the order keys, each
//            one more pass of the row, until its crossing part fits the buffer or is one key.
// ---------------------------------------------------------------------------------------------
struct LongArgs {
  const double* s0;
  int64_t len;
  int Hq, G;
  uint64_t local_mask;
  int topp, k;
  int ident;               // top-p of the values themselves (masses), not of exp weights
  int bitbins;             // values >= 0, binned by their bit patterns (see coarse_pos_of)
  const int32_t* kbudget;  // top-k per sequence (row / Hq), or NULL: k
  double p, scale;
  RowInfo* info;
  const double* pmax;  // [row][nblk] partial max / min of the scores
  const double* pmin;
  int nblk;
  int nb1;             // slabs per row
  unsigned long long* h1h;  // [row][kBins1] coarse histograms, summed over the row's slabs with
  unsigned long long* h1l;  //   integer atomics (zero before k_long_hist): fixed-point masses
  uint32_t* h1c;            //   (top-p) or entry counts (top-k)
  uint16_t* cbin;      // [row][cstride] coarse bin of every entry
  int64_t cstride;     // len rounded up to a multiple of 8 (16-byte aligned rows)
  int32_t* cidx;       // [row][slab][kResolveCap] indices of the crossing bin's entries ...
  uint64_t* ckey;      // ... and their order keys (dkey of the score)
  int32_t* ccnt;       // [row][slab] their counts (not capped)
  uint32_t* bits;
  int64_t words;
  uint32_t* status;
  // growing cache: tokens per sequence (device [B], or NULL: every row holds len entries); a row
  // of sequence b holds ctx_len[b] >> chunk_shift entries (row strides keep len)
  const int32_t* ctx_len;
  int64_t n_ctx;
  int chunk_shift;
};

// Entries of sequence b's rows.
__device__ __forceinline__ int64_t long_len(const LongArgs& a, int b) {
  return a.ctx_len ? (seq_tokens(a.ctx_len, b, a.n_ctx) >> a.chunk_shift) : a.len;
}

__device__ __forceinline__ double coarse_pos(double s, double smax, double binscale) {
  const double d = (smax - s) * binscale;
  return clamp0_f64(d, double(kBins1));  // NaN -> 0
}
// Bin axis of a long row. Default: linear in the score from the row max (kBins1 bins over the
// row's range), the right axis for exp weights. With bitbins (nonnegative values: importances,
// masses) the axis is the distance in IEEE bit patterns from the row max, 2^48 patterns per coarse
// bin: 16 bins per binade over 64 binades, everything smaller (zero included) in the last bin.
// Both are monotone non-increasing in the value, and every long-row kernel bins through here.
__device__ __forceinline__ double coarse_pos_of(const LongArgs& a, double s, double smax, double binscale) {
  if (a.bitbins) {
    const int64_t dv = __double_as_longlong(smax) - __double_as_longlong(s + 0.0);
    const double d = double(dv) * 0x1p-48;
    return d >= 0.0 ? (d < double(kBins1) ? d : double(kBins1)) : 0.0;
  }
  return coarse_pos(s, smax, binscale);
}
__device__ __forceinline__ int coarse_bin(double d) {
  const int c = int(d);
  return c < kBins1 - 1 ? c : kBins1 - 1;
}
// Exponent e with every value of a row whose maximum is smax below 2^e (0 when smax <= 0): the
// masses of an `ident` row are held as value 2^-e, weights in [0, 1) as the fixed-point sums need.
// A power-of-two scaling is exact and keeps every comparison of sums with the target.
__device__ __forceinline__ int ident_exp(double smax) {
  if (!(smax > 0.0)) return 0;
  int e;
  frexp(smax, &e);  // smax = f 2^e, f in [0.5, 1)
  return e;
}
// Softmax weights of a long top-p row, exp(x) with x = scale s - scale smax <= 0. Let dx =
// scale / binscale be the coarse bin width in logits. An entry of coarse bin c has r = x + c dx in
// (-dx, 0] (up to rounding), so exp(x) = exp(-c dx) exp(r): exp at the bin's edge (one table entry
// per bin) times a degree-9 Taylor polynomial of r, whose truncation error is below
// dx^10 / 10! < 2^-61 when dx <= 1/16. Rows with wider bins take exp itself. Every kernel of the
// row weighs an entry through here (the histogram through a table of the same edge values), so the
// fixed-point sums of every pass agree bit for bit.
constexpr double kTaylorMaxDx = 0.0625;
__device__ __forceinline__ bool taylor_row(const LongArgs& a, double binscale) {
  return a.topp && !a.ident && !a.bitbins && binscale > 0.0 && a.scale / binscale <= kTaylorMaxDx;
}
__device__ __forceinline__ double bin_edge_exp(const LongArgs& a, double binscale, int c) {
  return exp(-double(c) * (a.scale / binscale));
}
// Taylor coefficients 1/9!, 1/8!, ..., 1/1!, 1/0! (Horner order). A kernel that evaluates many
// weights first moves them into scalar registers (taylor_sgpr), so that the fma operands need no
// per-entry copies.
struct TaylorC {
  double c[10];
};
__device__ __forceinline__ TaylorC taylor_consts() {
  return TaylorC{{1.0 / 362880.0, 1.0 / 40320.0, 1.0 / 5040.0, 1.0 / 720.0, 1.0 / 120.0, 1.0 / 24.0, 1.0 / 6.0, 0.5,
                  1.0, 1.0}};
}
__device__ __forceinline__ TaylorC taylor_sgpr() {
  TaylorC t = taylor_consts();
#pragma unroll
  for (int i = 0; i < 10; ++i) asm volatile("" : "+s"(t.c[i]));  // opaque: kept in scalar registers
  return t;
}
__device__ __forceinline__ double exp_in_bin(double x, int c, double dx, double edge, const TaylorC& tc) {
  const double r = x + double(c) * dx;
  double e = tc.c[0];
#pragma unroll
  for (int i = 1; i < 10; ++i) e = fma(e, r, tc.c[i]);
  // into [0, 1]: r may round a hair above 0 in bin 0, and a NaN weight counts as 0
  return clamp01_f64(edge * e);
}
// the weight of a top-p row without the bin tables: masses, or exp itself
__device__ __forceinline__ double plain_weight(const LongArgs& a, double smax, int wexp, double s) {
  return max_f64(a.ident ? ldexp(s, -wexp) : exp(a.scale * s - a.scale * smax), 0.0);  // NaN -> 0
}
__device__ __forceinline__ double long_weight(const LongArgs& a, double smax, double binscale, int wexp,
                                              double s) {
  if (!a.topp) return 1.0;
  if (taylor_row(a, binscale)) {
    const int c = coarse_bin(coarse_pos(s, smax, binscale));
    return exp_in_bin(a.scale * s - a.scale * smax, c, a.scale / binscale, bin_edge_exp(a, binscale, c),
                      taylor_consts());
  }
  return plain_weight(a, smax, wexp, s);
}
__device__ __forceinline__ int long_k(const LongArgs& a, int b) { return a.kbudget ? a.kbudget[b] : a.k; }

// Inclusive scan of one double per thread over an NT-thread workgroup, in thread order; `wtot`
// holds NT/64 doubles of LDS. Returns the inclusive value; *total = the workgroup's sum.
template <int NT = 256>
__device__ __forceinline__ double block_scan(double v, double* wtot, double* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const double incl = wave_scan_dpp(v, lane);
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wv; ++w) before += wtot[w];
  double tot = 0.0;
  for (int w = 0; w < NT / 64; ++w) tot += wtot[w];
  *total = tot;
  __syncthreads();
  return before + incl;
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

constexpr int kLongThreads = 1024;
constexpr int kHistThreads = 512;  // (1024 would cap the registers at 128 and spill)
__global__ __launch_bounds__(kHistThreads) void k_long_hist(LongArgs a) {
  constexpr int NT = kHistThreads;
  const int b = blockIdx.z, h = blockIdx.y, slab = blockIdx.x, tid = threadIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  __shared__ unsigned long long hh[kBins1], hl[kBins1];
  __shared__ uint32_t hc[kBins1];
  __shared__ double rmax[NT / 64], rmin[NT / 64];
  __shared__ double ebin[kBins1];
  for (int i = tid; i < kBins1; i += NT) {
    hh[i] = 0;
    hl[i] = 0;
    hc[i] = 0;
  }
  // the row's score range from the score pass's partials (every workgroup gets the same bits)
  double mx = kNegInfD, mn = kPosInfD;
  for (int i = tid; i < a.nblk; i += NT) {
    mx = fmax(mx, a.pmax[row * a.nblk + i]);
    mn = fmin(mn, a.pmin[row * a.nblk + i]);
  }
  mx = wave_max_dpp(mx);
  mn = wave_min_dpp(mn);
  if ((tid & 63) == 0) {
    rmax[tid >> 6] = mx;
    rmin[tid >> 6] = mn;
  }
  __syncthreads();
  double smax = rmax[0], smin = rmin[0];
  for (int w = 1; w < NT / 64; ++w) {
    smax = fmax(smax, rmax[w]);
    smin = fmin(smin, rmin[w]);
  }
  const double range = smax - smin;
  const double binscale = range > 0.0 ? double(kBins1) / range : 0.0;
  const int wexp = a.ident ? ident_exp(smax) : 0;
  const int64_t len = long_len(a, b);
  const bool all = len == 0 || (a.topp ? (a.p >= 1.0) : (int64_t(long_k(a, b)) >= len));
  // softmax weights by bin (long_weight): the bins' edge values in LDS
  const bool taylor = taylor_row(a, binscale);
  const double dx = taylor ? a.scale / binscale : 0.0;
  if (taylor)
    for (int i = tid; i < kBins1; i += NT) ebin[i] = bin_edge_exp(a, binscale, i);
  __syncthreads();
  if (slab == 0 && tid == 0) {
    RowInfo ri = {};
    ri.smax = smax;
    ri.smin = smin;
    ri.binscale = binscale;
    ri.all = all;
    ri.wexp = wexp;
    a.info[row] = ri;
  }
  const int64_t t0 = int64_t(slab) * kLongBlock;
  if (all || t0 >= len) return;  // slabs past the row's entries hold nothing (the bin sums skip them)
  const int64_t t1 = t0 + kLongBlock < len ? t0 + kLongBlock : len;
  const double* sr = a.s0 + row * a.len;
  uint16_t* br = a.cbin + row * a.cstride;
  // kLongBlock / (8 NT) batches of 8 entries per thread; the next batch's loads are issued before
  // the current batch is binned (clamped, so every load is unconditional). Two layouts of a batch:
  // strided (entry k of lane tid at tid + NT k: 8-byte loads, 2-byte bin stores), or, when the row
  // length is a multiple of 8 (every 8-entry piece 64-byte aligned and inside the row), 8
  // consecutive entries per lane (16-byte loads and one 16-byte store of the 8 bins).
  constexpr int kIters = kLongBlock / (NT * 8);
  static_assert(kIters % 2 == 0, "batches go in pairs");
  double sv[2][8];
  auto bin_all = [&](auto taylor_tag, auto vec_tag) {
    constexpr bool kTaylor = decltype(taylor_tag)::value;
    constexpr bool kVec = decltype(vec_tag)::value;
    const TaylorC tc = taylor_sgpr();
    auto entry = [&](int it, int k) -> int64_t {
      return kVec ? t0 + 8 * (int64_t(tid) + int64_t(NT) * it) + k : t0 + int64_t(it) * (NT * 8) + tid + NT * k;
    };
    auto load = [&](double* dst, int it) {
      if (kVec) {
        int64_t e = entry(it, 0);
        const int64_t last = (t1 - 1) & ~int64_t(7);
        e = e < last ? e : last;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const double2 x = *reinterpret_cast<const double2*>(sr + e + 2 * k);
          dst[2 * k] = x.x;
          dst[2 * k + 1] = x.y;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int64_t t = entry(it, k);
          dst[k] = sr[t < t1 ? t : t1 - 1];
        }
      }
    };
    auto bin8 = [&](const double* vals, int it) {
      if (kVec && entry(it, 0) >= t1) return;
      uint16_t cb[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t t = entry(it, k);
        const double v = vals[k];
        // (Taylor rows are never bitbins rows)
        const int c = coarse_bin(kTaylor ? coarse_pos(v, smax, binscale) : coarse_pos_of(a, v, smax, binscale));
        cb[k] = uint16_t(c);
        if (t < t1) {
          if (!kVec) br[t] = uint16_t(c);
          if (a.topp) {
            const double w = kTaylor ? exp_in_bin(a.scale * v - a.scale * smax, c, dx, ebin[c], tc)
                                     : plain_weight(a, smax, wexp, v);
            fix_add(&hh[c], &hl[c], w);
          } else {
            atomicAdd(&hc[c], 1u);
          }
        }
      }
      if (kVec) {  // bins past the row's entries are written too (inside the row; never read as entries)
        uint4 pk;
        pk.x = uint32_t(cb[0]) | (uint32_t(cb[1]) << 16);
        pk.y = uint32_t(cb[2]) | (uint32_t(cb[3]) << 16);
        pk.z = uint32_t(cb[4]) | (uint32_t(cb[5]) << 16);
        pk.w = uint32_t(cb[6]) | (uint32_t(cb[7]) << 16);
        *reinterpret_cast<uint4*>(br + entry(it, 0)) = pk;
      }
    };
    load(sv[0], 0);
    for (int it = 0; it < kIters; it += 2) {
      load(sv[1], it + 1);
      bin8(sv[0], it);
      if (it + 2 < kIters) load(sv[0], it + 2);
      bin8(sv[1], it + 1);
    }
  };
  const bool vec = (a.len & 7) == 0 && (a.cstride & 7) == 0;
  if (taylor) {
    if (vec)
      bin_all(BoolTag<true>{}, BoolTag<true>{});
    else
      bin_all(BoolTag<true>{}, BoolTag<false>{});
  } else {
    if (vec)
      bin_all(BoolTag<false>{}, BoolTag<true>{});
    else
      bin_all(BoolTag<false>{}, BoolTag<false>{});
  }
  __syncthreads();
  // the slab's histogram into the row's totals (integer sums: the same bits in any order)
  const int64_t o = row * kBins1;
  for (int i = tid; i < kBins1; i += NT) {
    if (a.topp) {
      if (hh[i]) atomicAdd(&a.h1h[o + i], hh[i]);
      if (hl[i]) atomicAdd(&a.h1l[o + i], hl[i]);
    } else {
      if (hc[i]) atomicAdd(&a.h1c[o + i], hc[i]);
    }
  }
}

// Clears a row's coarse bin totals before k_long_hist adds into them (the kernel ahead of the
// histogram does it: k_long_zero, or the proxy query kernel on the token-row path).
__global__ __launch_bounds__(256) void k_long_zero(LongArgs a) {
  const int64_t row = int64_t(blockIdx.y) * a.Hq + blockIdx.x;
  zero_long_totals(a.h1h, a.h1l, a.h1c, row, threadIdx.x, 256);
}

// Per slab: the crossing coarse bin of the row (a scan of the bin totals that every workgroup of
// the row repeats bit for bit: Z, the target, the first bin where the running weight reaches it
// and the weight ahead of it; slab 0's workgroup records them for the resolution), the row's
// bitmap (entries of coarse bins ahead of the crossing bin, or every entry when the whole row is
// kept; zero for local heads), the number of the crossing bin's entries in
// the slab and, up to kResolveCap of them, their indices in the slab's region of the resolution
// buffer. Each lane takes 8 consecutive entries (one 16-byte load of their bins, all of a slab's
// loads issued at once) and writes their 8 bits as one byte of the bitmap.
__global__ __launch_bounds__(kLongThreads) void k_long_mark(LongArgs a) {
  constexpr int NT = kLongThreads;
  const int b = blockIdx.z, h = blockIdx.y, slab = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row = int64_t(b) * a.Hq + h;
  const int64_t t0 = int64_t(slab) * kLongBlock;
  const int64_t t1c = t0 + kLongBlock < a.len ? t0 + kLongBlock : a.len;  // the slab in the row
  const bool local = (a.local_mask >> (h / a.G)) & 1;
  uint32_t* bw = a.bits + row * a.words;
  static_assert(NT == kBins1, "one lane per coarse bin in the crossing scan");
  const uint16_t* br = a.cbin + row * a.cstride;
  constexpr int kVec = kLongBlock / (NT * 8);  // 16-byte pieces per lane
  // every load of the prologue goes out in one round, before the step's row length and the row's
  // state are known: piece v of lane tid covers entries t0 + 8 * (tid + NT v) .. + 7 (pieces past
  // the slab's capacity load its last piece again: rows are padded to a multiple of 8 entries;
  // entries past the row's length are masked below), and lane tid's coarse bin total
  uint4 pc[kVec];
  unsigned long long th = 0, tl = 0;
  uint32_t tcount = 0;
  if (!local) {
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      int64_t e = t0 + 8 * (int64_t(tid) + NT * v);
      const int64_t last = (t1c - 1) & ~int64_t(7);
      e = e < last ? e : last;
      pc[v] = ld16(br + e);
    }
    const int64_t o = row * kBins1 + tid;
    if (a.topp) {
      th = a.h1h[o];
      tl = a.h1l[o];
    } else {
      tcount = a.h1c[o];
    }
  }
  const int all0 = local ? 0 : a.info[row].all;
  const int64_t len = long_len(a, b);
  const int64_t t1 = t1c < len ? t1c : len;                              // its entries
  if (local || t1 <= t0) {
    for (int64_t w = (t0 >> 5) + tid; w < ((t1c + 31) >> 5); w += NT) bw[w] = 0u;
    if (tid == 0 && t1 <= t0 && !local) a.ccnt[row * a.nb1 + slab] = 0;
    return;
  }
  __shared__ int scnt, hit_bin;
  __shared__ double btot[NT / 64], hit_before;
  if (tid == 0) {
    scnt = 0;
    hit_bin = 0x7FFFFFFF;
  }
  __syncthreads();
  uint8_t* bb = reinterpret_cast<uint8_t*>(bw);
  int32_t* out = a.cidx + (row * a.nb1 + slab) * kResolveCap;
  uint64_t* outk = a.ckey + (row * a.nb1 + slab) * kResolveCap;
  __shared__ int32_t cst[kResolveCap];  // the crossing bin's entries, staged
  bool all = all0;
  int bin1 = 0;
  if (!all0) {
    const double m = a.topp ? fix_value(th, tl) : double(tcount);
    double Z;
    const double incl = block_scan<NT>(m, btot, &Z);
    const double target = a.topp ? a.p * Z : double(long_k(a, b));
    const double excl = incl - m;
    const unsigned long long reach = __ballot(excl + m >= target);  // bins in lane order
    if (reach && lane == __ffsll(reach) - 1) atomicMin(&hit_bin, tid);
    __syncthreads();
    bin1 = hit_bin;
    if (bin1 == tid) hit_before = excl;
    __syncthreads();
    all = bin1 == 0x7FFFFFFF;  // rounding left the target above the total weight: keep every entry
    if (slab == 0 && tid == 0) {
      RowInfo* ri = a.info + row;
      if (all) {
        ri->all = 1;
      } else {
        ri->bin1 = bin1;
        ri->before1 = hit_before;
        ri->target = target;
      }
    }
  }
  const bool gather = !all;
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    const int64_t e0 = t0 + 8 * (int64_t(tid) + NT * v);
    const uint16_t* cb = reinterpret_cast<const uint16_t*>(&pc[v]);
    uint32_t sel = 0, cand = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool valid = e0 + u < t1;
      sel |= (valid && (all || cb[u] < bin1)) ? (1u << u) : 0u;
      cand |= (gather && valid && cb[u] == bin1) ? (1u << u) : 0u;
    }
    if (e0 < ((t1c + 31) & ~int64_t(31))) bb[e0 >> 3] = uint8_t(sel);  // whole words, zero past the entries
    const int nc = __popc(cand);
    const int incl = wave_scan_i32_dpp(nc, lane);
    const int wtot = __builtin_amdgcn_readlane(incl, 63);
    if (wtot) {
      int p0 = 0;
      if (lane == 0) p0 = atomicAdd(&scnt, wtot);
      p0 = __builtin_amdgcn_readlane(p0, 0);
      int pos = p0 + incl - nc;
      while (cand) {
        const int u = __ffs(cand) - 1;
        cand &= cand - 1;
        if (pos < kResolveCap) cst[pos] = int32_t(e0 + u);
        ++pos;
      }
    }
  }
  __syncthreads();
  // the slab's crossing-bin entries with their order keys (one round of score loads)
  const int nst = scnt < kResolveCap ? scnt : kResolveCap;
  for (int i = tid; i < nst; i += NT) {
    const int32_t t = cst[i];
    out[i] = t;
    outk[i] = dkey(a.s0[row * a.len + t]);
  }
  if (tid == 0) a.ccnt[row * a.nb1 + slab] = scnt;
}

// Exact resolution of the crossing coarse bin. When its entries fit the resolution buffer they
// span one interval of the bin axis; a kSub-bin histogram of that interval (monotone in the score)
// finds the sub-bin where the running weight, started at the weight ahead of the interval, crosses
// the target. Entries of earlier sub-bins are selected; the crossing sub-bin's entries are ranked
// by counting in (score desc, index asc) order and walked to the first crossing. A crossing
// sub-bin of more than kSubCap entries is resolved by sorting every gathered entry instead.
// A crossing coarse bin with more entries than the buffer goes to resolve_radix.
constexpr int kSub = 1024;
constexpr int kSubCap = 256;
constexpr int kResolveThreads = 512;
// radix levels of an overfull crossing bin: kRadixBits bits of the order key per level (the
// level histograms use the sub-bin arrays)
constexpr int kRadixBits = 10;
constexpr int kRadixBins = 1 << kRadixBits;
static_assert(kRadixBins <= kSub, "radix levels reuse the sub-bin histogram");

struct ResolveLds {
  uint64_t* keys;  // [kResolveCap] gather buffer (order keys) ...
  int32_t* idx;    // ... and entry indices
  unsigned long long* hh;  // [kSub] histogram: fixed-point masses (top-p) ...
  unsigned long long* hl;
  uint32_t* hc;            // ... and entry counts
  double* wtot;    // [kResolveThreads / 64]
  double* buf;     // [kSelThreads] (block_first_crossing)
  int* ibuf;
  int* nx;
  int* hit;
  double* hit_before;
  uint64_t* kred;  // [2 * kResolveThreads / 64] key min / max per wave
};

__device__ __forceinline__ void set_bit(uint32_t* bw, int64_t t) { atomicOr(&bw[t >> 5], 1u << (t & 31)); }

// Narrows a crossing coarse bin of `cnt` (> kResolveCap) entries. Its entries occupy one interval
// [klo, khi] of order keys (dkey: a larger key comes earlier in the order). A level histograms the
// interval's entries by (khi - key) >> shift over kRadixBins bins (exact fixed-point masses and
// counts, one pass of the row), finds the bin where the running weight -- started at the weight
// of everything ahead of the interval -- reaches the target, and narrows the interval to that bin.
// Every level resolves kRadixBits bits of the key, so a few levels reach an interval of one key.
// The loop ends when the interval holds at most kResolveCap entries (gathered, sorted in (score
// desc, index asc) order and walked to the first crossing) or a single key (exact ties, equal
// weights: the lowest indices up to the crossing). Entries of the coarse bin ahead of the final
// interval are selected in the last pass. Exact for every input.
template <int NT>
__device__ void resolve_radix(const LongArgs& a, const RowInfo& ri, int64_t row, int64_t len, int64_t cnt,
                              const ResolveLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const double* sr = a.s0 + row * a.len;
  const uint16_t* br = a.cbin + row * a.cstride;
  uint32_t* bw = a.bits + row * a.words;
  const int wexp = ri.wexp;
  auto weight = [&](uint64_t k) { return long_weight(a, ri.smax, ri.binscale, wexp, dkey_inv(k)); };
  // key interval of the bin's entries
  uint64_t kmn = ~0ull, kmx = 0ull;
  for (int64_t t = tid; t < len; t += NT)
    if (br[t] == ri.bin1) {
      const uint64_t k = dkey(sr[t]);
      kmn = k < kmn ? k : kmn;
      kmx = k > kmx ? k : kmx;
    }
  for (int o = 32; o; o >>= 1) {
    const uint64_t x = __shfl_xor(kmn, o), y = __shfl_xor(kmx, o);
    kmn = x < kmn ? x : kmn;
    kmx = y > kmx ? y : kmx;
  }
  if (lane == 0) {
    L.kred[wv] = kmn;
    L.kred[NT / 64 + wv] = kmx;
  }
  __syncthreads();
  uint64_t klo = L.kred[0], khi = L.kred[NT / 64];
  for (int w = 1; w < NT / 64; ++w) {
    klo = L.kred[w] < klo ? L.kred[w] : klo;
    khi = L.kred[NT / 64 + w] > khi ? L.kred[NT / 64 + w] : khi;
  }
  double before = ri.before1;
  for (;;) {
    const uint64_t span = khi - klo;
    if (span == 0 || cnt <= kResolveCap) break;
    const int nbits = 64 - __clzll((long long)span);
    const int shift = nbits > kRadixBits ? nbits - kRadixBits : 0;  // (span >> shift) < kRadixBins
    __syncthreads();
    for (int i = tid; i < kRadixBins; i += NT) {
      L.hh[i] = 0;
      L.hl[i] = 0;
      L.hc[i] = 0;
    }
    if (tid == 0) *L.hit = 0x7FFFFFFF;
    __syncthreads();
    for (int64_t t = tid; t < len; t += NT)
      if (br[t] == ri.bin1) {
        const uint64_t k = dkey(sr[t]);
        if (k >= klo && k <= khi) {
          const int j = int((khi - k) >> shift);
          atomicAdd(&L.hc[j], 1u);
          if (a.topp) fix_add(&L.hh[j], &L.hl[j], weight(k));
        }
      }
    __syncthreads();
    constexpr int PER = kRadixBins / NT;
    double m[PER];
    double local = 0.0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = PER * tid + u;
      m[u] = a.topp ? fix_value(L.hh[j], L.hl[j]) : double(L.hc[j]);
      local += m[u];
    }
    double tot;
    const double incl = block_scan<NT>(local, L.wtot, &tot);
    double c = before + (incl - local);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const double cn = c + m[u];
      if (cn >= ri.target) {
        atomicMin(L.hit, PER * tid + u);
        break;
      }
      c = cn;
    }
    __syncthreads();
    const int jc = *L.hit;
    if (jc == 0x7FFFFFFF) {
      // rounding left the target beyond the interval's weight: every entry of the interval is kept
      for (int64_t t = tid; t < len; t += NT)
        if (br[t] == ri.bin1 && dkey(sr[t]) >= klo) set_bit(bw, t);
      return;
    }
    if (jc / PER == tid) {
      double cb = before + (incl - local);
      for (int u = 0; u < jc - PER * tid; ++u) cb += m[u];
      *L.hit_before = cb;
    }
    __syncthreads();
    before = *L.hit_before;
    cnt = L.hc[jc];
    const uint64_t nhi = khi - (uint64_t(jc) << shift);
    const uint64_t wdt = (uint64_t(1) << shift) - 1;
    klo = nhi - klo >= wdt ? nhi - wdt : klo;
    khi = nhi;
  }
  __syncthreads();
  if (cnt <= kResolveCap) {
    // gather the interval's entries, select the ones ahead of it, sort and walk
    if (tid == 0) *L.nx = 0;
    __syncthreads();
    for (int64_t t = tid; t < len; t += NT)
      if (br[t] == ri.bin1) {
        const uint64_t k = dkey(sr[t]);
        if (k > khi) {
          set_bit(bw, t);
        } else if (k >= klo) {
          const int q = atomicAdd(L.nx, 1);
          if (q < kResolveCap) {
            L.keys[q] = k;
            L.idx[q] = int32_t(t);
          }
        }
      }
    __syncthreads();
    // the gathered entries are exactly the level's crossing bin (cnt of them)
    if (tid == 0 && *L.nx != int(cnt)) atomicOr(&a.status[0], 2u);
    const int n = *L.nx < kResolveCap ? *L.nx : kResolveCap;
    if (n == 0) return;
    int Lp = 2;
    while (Lp < n) Lp <<= 1;
    for (int i = n + tid; i < Lp; i += NT) {
      L.keys[i] = 0ull;
      L.idx[i] = 0x7FFFFFFF;
    }
    __syncthreads();
    bitonic_desc<int32_t, NT>(L.keys, L.idx, Lp);
    auto wsorted = [&](int i) { return weight(L.keys[i]); };
    const int pos = block_first_crossing(n, before, ri.target, wsorted, L.buf, L.ibuf);
    const int n_sel = pos < 0 ? n : pos + 1;
    for (int i = tid; i < n_sel; i += NT) set_bit(bw, L.idx[i]);
    return;
  }
  // one key: equal weights, the lowest indices up to the crossing. Entries are taken in contiguous
  // per-thread index ranges, so a thread-order scan of their counts ranks them by index.
  const double wt = weight(khi);
  auto same = [&](int) { return wt; };
  const int pos = block_first_crossing(int(cnt), before, ri.target, same, L.buf, L.ibuf);
  const int take = pos < 0 ? int(cnt) : pos + 1;
  const int64_t per = (len + NT - 1) / NT;
  const int64_t r0 = int64_t(tid) * per, r1 = r0 + per < len ? r0 + per : len;
  int mine = 0;
  for (int64_t t = r0; t < r1; ++t)
    if (br[t] == ri.bin1 && dkey(sr[t]) == khi) ++mine;
  double tot;
  int rank = int(block_scan<NT>(double(mine), L.wtot, &tot)) - mine;
  for (int64_t t = r0; t < r1; ++t)
    if (br[t] == ri.bin1) {
      const uint64_t k = dkey(sr[t]);
      if (k > khi) {
        set_bit(bw, t);
      } else if (k == khi) {
        if (rank < take) set_bit(bw, t);
        ++rank;
      }
    }
}

__global__ __launch_bounds__(kResolveThreads) void k_long_resolve(LongArgs a) {
  constexpr int NT = kResolveThreads;
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  // the slabs' crossing-bin counts are loaded with the row's state and length (slabs past the
  // step's length hold a count of 0, written by the marking pass)
  const int per = (a.nb1 + kResolveThreads - 1) / kResolveThreads;  // slabs per thread
  double local = 0.0;
  for (int s = tid * per; s < min(a.nb1, tid * per + per); ++s) local += double(a.ccnt[row * a.nb1 + s]);
  const RowInfo ri = a.info[row];
  if (ri.all) return;
  __shared__ uint64_t keys[kResolveCap];
  __shared__ int32_t idx[kResolveCap];
  __shared__ uint16_t sub[kResolveCap];
  __shared__ unsigned long long hh[kSub], hl[kSub];
  __shared__ uint32_t hc[kSub];
  __shared__ uint64_t xkey[kSubCap];
  __shared__ int32_t xidx[kSubCap];
  __shared__ double xw[kSubCap];
  __shared__ int32_t ridx[kSubCap];
  __shared__ double wtot[NT / 64];
  __shared__ double buf[kSelThreads];
  __shared__ uint64_t kred[2 * NT / 64];
  __shared__ int soff[NT + 1];
  __shared__ int hit_bin, nx, ibuf;
  __shared__ double hit_before;
  uint32_t* bw = a.bits + row * a.words;
  const int wexp = ri.wexp;
  const int64_t len = long_len(a, b);
  const int nb = a.nb1;
  // ---- the crossing bin's entry count over the slabs (slab s owns soff[s] .. soff[s+1] of the
  // gathered entries when they fit the buffer)
  const int nthr = (nb + per - 1) / per;  // threads holding slabs
  double tot;
  const double incl = block_scan<NT>(local, wtot, &tot);
  if (tot > double(kResolveCap)) {
    const ResolveLds L{keys, idx, hh, hl, hc, wtot, buf, &ibuf, &nx, &hit_bin, &hit_before, kred};
    resolve_radix<NT>(a, ri, row, len, int64_t(tot), L);
    return;
  }
  // soff holds the first position of every thread's first slab; slabs inside a thread's range
  // are walked in order below
  soff[tid] = int(incl - local);
  if (tid == NT - 1) soff[NT] = int(tot);
  __syncthreads();
  const int n = int(tot);
  if (n == 0) return;
  {
    constexpr int PER = kResolveCap / NT;
    int32_t tv[PER];
    uint64_t kv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + NT * k;
      const int j = i < n ? i : n - 1;
      // owner thread range: last thread u with soff[u] <= j (threads past nthr hold no slab)
      int lo = 0, hi = nthr;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (soff[mid] <= j) lo = mid; else hi = mid;
      }
      int s = lo * per, off = j - soff[lo];
      // with one slab per thread, soff[lo + 1] - soff[lo] is that slab's count, so j lies in slab
      // lo and no count needs reading
      while (per > 1 && s + 1 < nb && off >= a.ccnt[row * a.nb1 + s]) {  // at most `per` steps
        off -= a.ccnt[row * a.nb1 + s];
        ++s;
      }
      tv[k] = a.cidx[(row * a.nb1 + s) * kResolveCap + off];
      kv[k] = a.ckey[(row * a.nb1 + s) * kResolveCap + off];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + NT * k;
      if (i < n) {
        keys[i] = kv[k];
        idx[i] = tv[k];
      }
    }
  }
  const double before = ri.before1;
  const double dlo = double(ri.bin1);
  // every gathered entry lies in the crossing coarse bin, so its weight (long_weight) takes that
  // bin's edge value, computed once
  const bool ty = taylor_row(a, ri.binscale);
  const double dx1 = ty ? a.scale / ri.binscale : 0.0;
  const double edge1 = ty ? bin_edge_exp(a, ri.binscale, ri.bin1) : 0.0;
  const TaylorC tc = taylor_sgpr();
  auto wt = [&](double s) {
    if (!a.topp) return 1.0;
    return ty ? exp_in_bin(a.scale * s - a.scale * ri.smax, ri.bin1, dx1, edge1, tc) : plain_weight(a, ri.smax, wexp, s);
  };
  const double sscale = double(kSub);
  // ---- sub-bin histogram of the gathered entries
  for (int i = tid; i < kSub; i += NT) {
    hh[i] = 0;
    hl[i] = 0;
    hc[i] = 0;
  }
  if (tid == 0) {
    nx = 0;
    hit_bin = 0x7FFFFFFF;
  }
  __syncthreads();
  for (int i = tid; i < n; i += NT) {
    const double s = dkey_inv(keys[i]);
    const double x = (coarse_pos_of(a, s, ri.smax, ri.binscale) - dlo) * sscale;
    int sb = x >= 0.0 ? (x < double(kSub) ? int(x) : kSub - 1) : 0;
    sb = sb < kSub - 1 ? sb : kSub - 1;
    sub[i] = uint16_t(sb);
    atomicAdd(&hc[sb], 1u);
    if (a.topp) fix_add(&hh[sb], &hl[sb], wt(s));
  }
  __syncthreads();
  constexpr int SPER = kSub / NT;
  double m[SPER];
  double lsum = 0.0;
#pragma unroll
  for (int j = 0; j < SPER; ++j) {
    const int bj = SPER * tid + j;
    m[j] = a.topp ? fix_value(hh[bj], hl[bj]) : double(hc[bj]);
    lsum += m[j];
  }
  double stot;
  const double sincl = block_scan<NT>(lsum, wtot, &stot);
  double c = before + (sincl - lsum);
  const double c0 = c;
#pragma unroll
  for (int j = 0; j < SPER; ++j) {
    const double cn = c + m[j];
    if (cn >= ri.target) {
      atomicMin(&hit_bin, SPER * tid + j);
      break;
    }
    c = cn;
  }
  __syncthreads();
  const int hb = hit_bin;
  if (hb != 0x7FFFFFFF && hb / SPER == tid) {
    double cb = c0;
    for (int j = 0; j < hb - SPER * tid; ++j) cb += m[j];
    hit_before = cb;
  }
  __syncthreads();
  if (hb == 0x7FFFFFFF) {
    // rounding: the target lies beyond the gathered entries; keep all of them
    for (int i = tid; i < n; i += NT) set_bit(bw, idx[i]);
    return;
  }
  if (hc[hb] <= uint32_t(kSubCap)) {
    for (int i = tid; i < n; i += NT) {
      const int sb = sub[i];
      if (sb < hb) {
        set_bit(bw, idx[i]);
      } else if (sb == hb) {
        const int q = atomicAdd(&nx, 1);
        xkey[q] = keys[i];
        xidx[q] = idx[i];
      }
    }
    __syncthreads();
    const int nc = nx;
    for (int q = tid; q < nc; q += NT) {
      const uint64_t kq = xkey[q];
      const int32_t iq = xidx[q];
      int r = 0;
      for (int u = 0; u < nc; ++u) {
        const uint64_t ku = xkey[u];
        r += (ku > kq || (ku == kq && xidx[u] < iq)) ? 1 : 0;
      }
      xw[r] = wt(dkey_inv(kq));
      ridx[r] = iq;
    }
    __syncthreads();
    // the first rank where the running weight reaches the target (a block scan, not a walk)
    static_assert(NT == kSelThreads, "block_first_crossing spans the workgroup");
    const int pos = block_first_crossing(nc, hit_before, ri.target, [&](int r) { return xw[r]; }, buf, &ibuf);
    const int ns = pos < 0 ? nc : pos + 1;
    for (int r = tid; r < ns; r += NT) set_bit(bw, ridx[r]);
    return;
  }
  // near-equal scores fill the crossing sub-bin: sort every gathered entry and walk them all
  int Lp = 2;
  while (Lp < n) Lp <<= 1;
  for (int i = n + tid; i < Lp; i += NT) {
    keys[i] = 0ull;
    idx[i] = 0x7FFFFFFF;
  }
  __syncthreads();
  bitonic_desc<int32_t, NT>(keys, idx, Lp);
  auto weight = [&](int i) { return wt(dkey_inv(keys[i])); };
  const int pos = block_first_crossing(n, before, ri.target, weight, buf, &ibuf);
  const int n_sel = pos < 0 ? n : pos + 1;
  for (int i = tid; i < n_sel; i += NT) set_bit(bw, idx[i]);
}

// ---------------------------------------------------------------------------------------------
// Coverage budget (dynamic token coverage, decode form): per sequence, every scored head's softmax
// of select_scale * s over its row, summed per entry (the column sums of the proxy attention map);
// the entries in ascending importance; the shortest ascending prefix whose mass exceeds tau x the
// total is cut; budget = max(1, entries - cut), used by every head of the sequence as its top-k.
// Four short launches, each spread over many workgroups:
//   k_cov_mass        per (head, sequence): the head's softmax masses (zero for a local head);
//   k_cov_importance  per (slice, sequence): the masses summed per entry in head order;
//   k_cov_rank        per (slice, sequence): each entry's ascending rank, counted against every
//                     entry of the sequence (ties by index), and its importance scattered to
//                     that sorted position;
//   k_cov_budget      per sequence: the running sum in sorted order and the first crossing.
// Rows of at most kSmallRowMax entries.
// ---------------------------------------------------------------------------------------------
struct CoverageArgs {
  const double* s;
  int64_t len;
  int Hq, G;
  uint64_t local_mask;
  double scale, tau;
  double* mass;    // [B][Hq][len]
  double* imp;     // [B][len]
  double* sorted;  // [B][len] importance in ascending order
  int32_t* budget; // [B]
  // growing cache: sequence b's rows hold ctx_len[b] >> chunk_shift entries (NULL: len)
  const int32_t* ctx_len;
  int64_t n_ctx;
  int chunk_shift;
};

// Entries of sequence b's coverage rows.
__device__ __forceinline__ int cov_len(const CoverageArgs& a, int b) {
  return int(a.ctx_len ? (seq_tokens(a.ctx_len, b, a.n_ctx) >> a.chunk_shift) : a.len);
}

constexpr int kCovThreads = 256;
constexpr int kCovRankEntries = 32;   // entries ranked per workgroup
constexpr int kCovRankPerThread = 4;  // entries per thread (each key read serves all of them)

__global__ __launch_bounds__(kCovThreads) void k_cov_mass(CoverageArgs a) {
  constexpr int NT = kCovThreads, PT = kSmallRowMax / NT;
  __shared__ double wred[NT / 64];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L = cov_len(a, b);
  const int64_t row = int64_t(b) * a.Hq + h;
  double* mr = a.mass + row * a.len;
  if ((a.local_mask >> (h / a.G)) & 1) {
    // a local head scores nothing: zero masses keep the per-entry sum branch-free and exact
    for (int m = tid; m < L; m += NT) mr[m] = 0.0;
    return;
  }
  const double* sr = a.s + row * a.len;
  double v[PT];
  double mx = kNegInfD;
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int m = tid + NT * k;
    v[k] = m < L ? sr[m] : kNegInfD;
    mx = fmax(mx, v[k]);
  }
  mx = wave_max_dpp(mx);
  if (lane == 0) wred[wv] = mx;
  __syncthreads();
  mx = fmax(fmax(wred[0], wred[1]), fmax(wred[2], wred[3]));
  __syncthreads();
  double z = 0.0;
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    v[k] = tid + NT * k < L ? exp(a.scale * v[k] - a.scale * mx) : 0.0;
    z += v[k];
  }
  z = wave_sum_dpp(z);
  if (lane == 0) wred[wv] = z;
  __syncthreads();
  z = (wred[0] + wred[1]) + (wred[2] + wred[3]);
#pragma unroll
  for (int k = 0; k < PT; ++k)
    if (tid + NT * k < L) mr[tid + NT * k] = v[k] / z;
}

__global__ __launch_bounds__(kCovThreads) void k_cov_importance(CoverageArgs a) {
  const int b = blockIdx.y, m = blockIdx.x * kCovThreads + threadIdx.x;
  if (m >= cov_len(a, b)) return;
  const double* mb = a.mass + int64_t(b) * a.Hq * a.len + m;
  double imp = 0.0;
#pragma unroll 8
  for (int h = 0; h < a.Hq; ++h) imp += mb[int64_t(h) * a.len];
  a.imp[int64_t(b) * a.len + m] = imp;
}

__global__ __launch_bounds__(kCovThreads) void k_cov_rank(CoverageArgs a) {
  constexpr int NT = kCovThreads, E = kCovRankEntries, EPT = kCovRankPerThread;
  constexpr int EG = E / EPT, S = NT / EG;  // entry groups, key slices
  __shared__ uint64_t keys[kSmallRowMax];
  __shared__ int part[S][E];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int L = cov_len(a, b);
  const double* ib = a.imp + int64_t(b) * a.len;
  for (int j = tid; j < L; j += NT) keys[j] = dkey(ib[j]);
  __syncthreads();
  // thread: entries e0 + EG i (i < EPT) against keys slice, slice + S, ... (consecutive slices
  // of a wave read consecutive keys)
  const int eg = tid % EG, slice = tid / EG;
  const int e0 = blockIdx.x * E + eg;
  uint64_t ke[EPT];
  int cnt[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = e0 + EG * i;
    ke[i] = e < L ? keys[e] : 0ull;
    cnt[i] = 0;
  }
#pragma unroll 4
  for (int j = slice; j < L; j += S) {
    const uint64_t kj = keys[j];
#pragma unroll
    for (int i = 0; i < EPT; ++i) cnt[i] += (kj < ke[i]) | ((kj == ke[i]) & (j < e0 + EG * i));
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) part[slice][eg + EG * i] = cnt[i];
  __syncthreads();
  const int e = blockIdx.x * E + tid;
  if (tid < E && e < L) {
    int r = 0;
#pragma unroll 8
    for (int q = 0; q < S; ++q) r += part[q][tid];
    a.sorted[int64_t(b) * a.len + r] = ib[e];
  }
}

constexpr int kCovBudgetThreads = 1024;
__global__ __launch_bounds__(kCovBudgetThreads) void k_cov_budget(CoverageArgs a) {
  constexpr int NT = kCovBudgetThreads, PT = kSmallRowMax / NT;
  __shared__ double wtot[NT / 64];
  __shared__ int hit;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = cov_len(a, b);
  const double* sb = a.sorted + int64_t(b) * a.len;
  double w[PT];
  double local = 0.0;
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int i = PT * tid + k;
    w[k] = i < L ? sb[i] : 0.0;
    local += w[k];
  }
  if (tid == 0) hit = 0x7FFFFFFF;
  double total;
  const double incl = block_scan<NT>(local, wtot, &total);
  const double thr = a.tau * total;
  double c = incl - local;
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    c += w[k];
    if (PT * tid + k < L && c > thr) {
      atomicMin(&hit, PT * tid + k);
      break;
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int removed = hit == 0x7FFFFFFF ? L : hit + 1;
    a.budget[b] = L - removed > 1 ? L - removed : 1;
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
  // growing cache: sequence b's union covers ctx_len[b] >> chunk_shift entries (NULL: n)
  const int32_t* ctx_len;
  int64_t n_ctx;
  int chunk_shift;
};

// Per range of kUnionWordsPerBlock words: the union words (OR of the group's per-head words and
// the forced / local edge bits) and their popcount. Every load is issued first.
__global__ __launch_bounds__(256) void k_union_count(UnionArgs a) {
  const int b = blockIdx.z, g = blockIdx.y, r = blockIdx.x, tid = threadIdx.x;
  const bool local = (a.local_mask >> g) & 1;
  const int64_t w0 = int64_t(r) * kUnionWordsPerBlock;
  const int64_t grp = int64_t(b) * a.Hk + g;
  constexpr int PER = kUnionWordsPerBlock / 256;
  uint32_t u[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) u[i] = 0u;
  if (!local) {
    // the group's heads four at a time, every load of a block issued before the first is used
    // (heads past the group repeat its last head: the OR is unchanged)
    for (int j0 = 0; j0 < a.G; j0 += 4) {
      uint32_t v[4][PER];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = j0 + jj < a.G ? j0 + jj : a.G - 1;
        const uint32_t* src = a.bits + (int64_t(b) * a.Hq + g * a.G + j) * a.words;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int64_t w = w0 + tid + 256 * i;
          v[jj][i] = src[w < a.words ? w : a.words - 1];
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int i = 0; i < PER; ++i) u[i] |= v[jj][i];
    }
  }
  int c = 0;
  const int64_t n = a.ctx_len ? (seq_tokens(a.ctx_len, b, a.n_ctx) >> a.chunk_shift) : a.n;  // entries
  const int64_t nw = (n + 31) >> 5;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t w = w0 + tid + 256 * i;
    if (w < a.words) {
      uint32_t x = local ? edge_bits(w, n, a.sink, a.window) : (u[i] | edge_bits(w, n, a.keep_first, a.keep_last));
      if (w >= nw) x = 0u;
      if (w == nw - 1 && (n & 31)) x &= (1u << (n & 31)) - 1u;
      a.ubits[grp * a.words + w] = x;
      c += __popc(x);
    }
  }
  c = wave_sum_i32_dpp(c);
  __shared__ int part[4];
  if ((tid & 63) == 0) part[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) a.rcnt[grp * a.ranges + r] = part[0] + part[1] + part[2] + part[3];
}

// Per range: the set bits of the union words in ascending order, after the earlier ranges'
// entries. Wave w takes words [256 w, 256 w + 256) of the range in 4 rounds of 64 (one word per
// lane); a round's entries are expanded into LDS and copied out with coalesced stores.
__global__ __launch_bounds__(256) void k_union_write(UnionArgs a) {
  const int b = blockIdx.z, g = blockIdx.y, r = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t grp = int64_t(b) * a.Hk + g;
  constexpr int ROUNDS = kUnionWordsPerBlock / 256;
  __shared__ int wpart[4], wtot[4];
  __shared__ int32_t stage[4][64 * 32];
  const int64_t wbase = int64_t(r) * kUnionWordsPerBlock + wave * (64 * ROUNDS);
  uint32_t u[ROUNDS];
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int64_t w = wbase + 64 * i + lane;
    u[i] = w < a.words ? a.ubits[grp * a.words + w] : 0u;
  }
  // counts of the earlier ranges, summed by the whole workgroup
  int s = 0;
  for (int i = tid; i < r; i += 256) s += a.rcnt[grp * a.ranges + i];
  s = wave_sum_i32_dpp(s);
  int mine = 0;
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) mine += __popc(u[i]);
  mine = wave_sum_i32_dpp(mine);
  if (lane == 0) {
    wpart[wave] = s;
    wtot[wave] = mine;
  }
  __syncthreads();
  int pos = wpart[0] + wpart[1] + wpart[2] + wpart[3];
  for (int w = 0; w < wave; ++w) pos += wtot[w];
  int32_t* out = a.list + grp * a.n;
  int32_t* st = stage[wave];
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int c = __popc(u[i]);
    const int incl = wave_scan_i32_dpp(c, lane);
    const int n = __builtin_amdgcn_readlane(incl, 63);
    int o = incl - c;
    uint32_t m = u[i];
    const int32_t wi = int32_t((wbase + 64 * i + lane) * 32);
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      st[o++] = wi + bit;
    }
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < n; e += 64) out[pos + e] = st[e];
    __builtin_amdgcn_wave_barrier();
    pos += n;
  }
  if (r == a.ranges - 1 && wave == 3 && lane == 0) a.cnt[grp] = pos;
}

LongArgs long_args(const Plan& p, char* ws) {
  const sd_config& c = p.cfg;
  LongArgs a;
  a.bitbins = 0;
  a.s0 = at<double>(ws, p.o_s0);
  a.len = p.len0;
  a.Hq = c.n_q_heads;
  a.G = p.G;
  a.local_mask = p.local_mask;
  a.topp = c.mode == SD_TOPP;
  a.k = c.top_k;
  a.ident = 0;
  a.kbudget = nullptr;
  a.p = c.top_p;
  a.scale = c.mode == SD_TOPP ? c.select_scale : 1.0;
  a.info = at<RowInfo>(ws, p.o_info);
  a.pmax = at<double>(ws, p.o_pmax);
  a.pmin = at<double>(ws, p.o_pmin);
  a.nblk = p.score_blocks0;
  a.nb1 = p.long_blocks;
  a.h1h = at<unsigned long long>(ws, p.o_h1h);
  a.h1l = at<unsigned long long>(ws, p.o_h1l);
  a.h1c = at<uint32_t>(ws, p.o_h1c);
  a.cbin = at<uint16_t>(ws, p.o_cbin);
  a.cstride = (p.len0 + 7) & ~int64_t(7);
  a.cidx = at<int32_t>(ws, p.o_cidx);
  a.ckey = at<uint64_t>(ws, p.o_ckey);
  a.ccnt = at<int32_t>(ws, p.o_ccnt);
  a.bits = at<uint32_t>(ws, p.o_bits);
  a.words = p.words;
  a.status = at<uint32_t>(ws, p.o_status);
  a.ctx_len = at<int32_t>(ws, p.o_ctx);
  a.n_ctx = c.n_ctx;
  a.chunk_shift = p.chunk_shift;
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
  u.ctx_len = at<int32_t>(ws, p.o_ctx);
  u.n_ctx = c.n_ctx;
  u.chunk_shift = p.chunk_shift;
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
  a.kbudget = c.mode == SD_COVERAGE ? at<int32_t>(ws, p.o_budget) : nullptr;
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
  a.ctx_len = at<int32_t>(ws, p.o_ctx);
  a.n_ctx = c.n_ctx;
  a.chunk_shift = p.chunk_shift;
  return a;
}

}  // namespace

int launch_select(const Plan& p, int level, char* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sd_config& c = p.cfg;
  const int B = c.batch, Hq = c.n_q_heads;
  if (c.mode == SD_COVERAGE && p.n_scored > 0) {
    CoverageArgs ca;
    ca.s = at<double>(ws, p.o_s0);
    ca.len = p.len0;
    ca.Hq = Hq;
    ca.G = p.G;
    ca.local_mask = p.local_mask;
    ca.scale = c.select_scale;
    ca.tau = c.tau;
    ca.mass = at<double>(ws, p.o_cmass);
    ca.imp = at<double>(ws, p.o_cimp);
    ca.sorted = at<double>(ws, p.o_csort);
    ca.budget = at<int32_t>(ws, p.o_budget);
    ca.ctx_len = at<int32_t>(ws, p.o_ctx);
    ca.n_ctx = c.n_ctx;
    ca.chunk_shift = p.chunk_shift;
    const int L = int(p.len0);
    hipLaunchKernelGGL(k_cov_mass, dim3(Hq, B), dim3(kCovThreads), 0, st, ca);
    hipLaunchKernelGGL(k_cov_importance, dim3((L + kCovThreads - 1) / kCovThreads, B), dim3(kCovThreads), 0, st, ca);
    hipLaunchKernelGGL(k_cov_rank, dim3((L + kCovRankEntries - 1) / kCovRankEntries, B), dim3(kCovThreads), 0, st, ca);
    hipLaunchKernelGGL(k_cov_budget, dim3(B), dim3(kCovBudgetThreads), 0, st, ca);
  }
  if (c.mode == SD_HIER_TOPK || !p.long0) {
    // rows of at most kSmallRowMax entries: per-head selection, then (after the last level) the
    // group union and compaction
    const GroupSelArgs ga = group_args(p, ws, level);
    hipLaunchKernelGGL(k_select_head, dim3(Hq, B), dim3(kSelT), 0, st, ga);
    if (ga.kind != 1) hipLaunchKernelGGL(k_union_small, dim3(c.n_kv_heads, B), dim3(kSelT), 0, st, ga);
    return int(hipGetLastError());
  }
  const LongArgs a = long_args(p, ws);
  const dim3 rows(Hq, B), blocks(p.long_blocks, Hq, B);
  // the proxy query kernel has cleared the bin totals on the token-row path
  if (c.route != SD_ROUTE_PROXY) hipLaunchKernelGGL(k_long_zero, rows, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_long_hist, blocks, dim3(kHistThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_mark, blocks, dim3(kLongThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_resolve, rows, dim3(kResolveThreads), 0, st, a);
  int e = int(hipGetLastError());
  if (e) return e;
  return union_impl(p, ws, st);
}

// ---- long-row selection over caller-given rows (the prefill path's budget and per-head top-k)
namespace {
struct LongScratch {
  size_t info, h1h, h1l, h1c, cbin, cidx, ckey, ccnt, total;
};
LongScratch long_scratch_layout(int64_t rows, int64_t len) {
  const int64_t nb1 = (len + kLongBlock - 1) / kLongBlock;
  LongScratch l;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + (bytes > 0 ? bytes : 1) + 255) & ~size_t(255);
    return o;
  };
  l.info = take(size_t(rows) * sizeof(RowInfo));
  l.h1h = take(size_t(rows * kBins1) * 8);
  l.h1l = take(size_t(rows * kBins1) * 8);
  l.h1c = take(size_t(rows * kBins1) * 4);
  l.cbin = take(size_t(rows * ((len + 7) & ~int64_t(7))) * 2);
  l.cidx = take(size_t(rows * nb1 * kResolveCap) * 4);
  l.ckey = take(size_t(rows * nb1 * kResolveCap) * 8);
  l.ccnt = take(size_t(rows * nb1) * 4);
  l.total = off;
  return l;
}
}  // namespace

size_t long_rows_scratch(int64_t rows, int64_t len) { return long_scratch_layout(rows, len).total; }

int launch_long_rows(const LongRows& r, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const LongScratch l = long_scratch_layout(int64_t(r.B) * r.H, r.len);
  LongArgs a;
  a.s0 = r.s;
  a.len = r.len;
  a.Hq = r.H;
  a.G = 1;
  a.local_mask = 0;
  a.topp = r.topp;
  a.k = r.k;
  a.ident = r.ident;
  a.bitbins = r.bitbins;
  a.kbudget = r.kbudget;
  a.p = r.p;
  a.scale = r.scale;
  a.info = reinterpret_cast<RowInfo*>(r.scratch + l.info);
  a.pmax = r.pmax;
  a.pmin = r.pmin;
  a.nblk = r.nblk;
  a.nb1 = int((r.len + kLongBlock - 1) / kLongBlock);
  a.h1h = reinterpret_cast<unsigned long long*>(r.scratch + l.h1h);
  a.h1l = reinterpret_cast<unsigned long long*>(r.scratch + l.h1l);
  a.h1c = reinterpret_cast<uint32_t*>(r.scratch + l.h1c);
  a.cbin = reinterpret_cast<uint16_t*>(r.scratch + l.cbin);
  a.cstride = (r.len + 7) & ~int64_t(7);
  a.cidx = reinterpret_cast<int32_t*>(r.scratch + l.cidx);
  a.ckey = reinterpret_cast<uint64_t*>(r.scratch + l.ckey);
  a.ccnt = reinterpret_cast<int32_t*>(r.scratch + l.ccnt);
  a.bits = r.bits;
  a.words = r.words;
  a.status = r.status;
  a.ctx_len = nullptr;  // caller-given rows are whole
  a.n_ctx = r.len;
  a.chunk_shift = 0;
  const dim3 rows(r.H, r.B), blocks(a.nb1, r.H, r.B);
  hipLaunchKernelGGL(k_long_zero, rows, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_long_hist, blocks, dim3(kHistThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_mark, blocks, dim3(kLongThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_resolve, rows, dim3(kResolveThreads), 0, st, a);
  return int(hipGetLastError());
}

}  // namespace sd
