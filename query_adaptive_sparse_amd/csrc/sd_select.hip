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
//      more than kRankDirect entries a second 256-bin level splits it;
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
// A crossing coarse bin of more entries than this is split by the second level before ranking
// (ranking by counting costs n^2 LDS reads).
constexpr int kRankDirect = 16;
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
          res_state = hc[hb] <= uint32_t(lv == 1 ? kRankDirect : kCandCap) ? lv : (lv == 2 ? 3 : 0);
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
        // the heads' words 8 at a time, every load of a block issued before the first is used
        // (heads past the group repeat its last head: the OR is unchanged)
        for (int j0 = 0; j0 < G; j0 += 8) {
          uint32_t v[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int j = j0 + jj < G ? j0 + jj : G - 1;
            v[jj] = __builtin_nontemporal_load(&a.bits[(int64_t(b) * a.Hq + g * G + j) * a.words + w]);
          }
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) u |= v[jj];
        }
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
// Selection of long rows (more than kSmallRowMax entries: token-level proxy rows, or fine chunk
// rows). The (score desc, index asc) order is resolved through a coarse histogram of the weights
// over the bins of (smax - s) on the row's score range, then the entries of the coarse bin where
// the running weight crosses the target. Weight = softmax mass exp(scale*s - scale*smax) for
// top-p, 1 for top-k. Bins are monotone in the score, so every entry of an earlier bin precedes
// every entry of a later one in the order. Passes:
//   hist     per slab of kLongBlock entries: coarse bin of every entry (kept, 2 bytes), partial
//            coarse histogram (no atomics across workgroups);
//   find1    per row: bin totals (slab partials in slab order), Z and the target, the crossing
//            coarse bin and the weight ahead of it;
//   mark     per slab: bitmap words of the entries of earlier coarse bins, and the indices of the
//            crossing bin's entries in the slab's own region of the resolution buffer;
//   resolve  per row: the crossing bin's entries split by a sub-bin histogram of their interval;
//            earlier sub-bins are selected, the crossing sub-bin's entries are ranked and walked to
//            the first crossing.
// A crossing coarse bin of more than kResolveCap entries (heavily tied scores) is split inside the
// resolve workgroup by a fine histogram over one more pass of the row (slow, and only then).
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
  double* h1m;         // [row][slab][kBins1] partial coarse histograms
  uint32_t* h1c;
  uint16_t* cbin;      // [row][cstride] coarse bin of every entry
  int64_t cstride;     // len rounded up to a multiple of 8 (16-byte aligned rows)
  int32_t* cidx;       // [row][slab][kResolveCap] indices of the crossing bin's entries
  int32_t* ccnt;       // [row][slab] their counts
  uint32_t* bits;
  int64_t words;
  uint32_t* status;
};

__device__ __forceinline__ double coarse_pos(double s, double smax, double binscale) {
  const double d = (smax - s) * binscale;
  return d >= 0.0 ? (d < double(kBins1) ? d : double(kBins1)) : 0.0;  // NaN -> 0
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
__device__ __forceinline__ int fine_bin(double d, int c1) {
  const int c2 = int((d - double(c1)) * double(kBins2));
  return c2 < 0 ? 0 : (c2 < kBins2 - 1 ? c2 : kBins2 - 1);
}
__device__ __forceinline__ double long_weight(const LongArgs& a, double smax, double s) {
  return a.topp ? (a.ident ? s : exp(a.scale * s - a.scale * smax)) : 1.0;
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

constexpr int kLongThreads = 1024;
__global__ __launch_bounds__(kLongThreads) void k_long_hist(LongArgs a) {
  constexpr int NT = kLongThreads;
  const int b = blockIdx.z, h = blockIdx.y, slab = blockIdx.x, tid = threadIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  __shared__ double hm[kBins1];
  __shared__ uint32_t hc[kBins1];
  __shared__ double rmax[NT / 64], rmin[NT / 64];
  for (int i = tid; i < kBins1; i += NT) {
    hm[i] = 0.0;
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
  const bool all = a.topp ? (a.p >= 1.0) : (int64_t(long_k(a, b)) >= a.len);
  if (slab == 0 && tid == 0) {
    RowInfo ri = {};
    ri.smax = smax;
    ri.smin = smin;
    ri.binscale = binscale;
    ri.all = all;
    a.info[row] = ri;
  }
  if (all) return;
  const int64_t t0 = int64_t(slab) * kLongBlock;
  const int64_t t1 = t0 + kLongBlock < a.len ? t0 + kLongBlock : a.len;
  const double* sr = a.s0 + row * a.len;
  uint16_t* br = a.cbin + row * a.cstride;
  // kLongBlock / (8 NT) batches of 8 entries per thread; the next batch's loads are issued before
  // the current batch is binned (clamped, so every load is unconditional)
  constexpr int kIters = kLongBlock / (NT * 8);
  double sv[2][8];
  auto load = [&](double* dst, int it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t t = t0 + int64_t(it) * (NT * 8) + tid + NT * k;
      dst[k] = sr[t < t1 ? t : t1 - 1];
    }
  };
  load(sv[0], 0);
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    if (it + 1 < kIters) load(sv[(it + 1) & 1], it + 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t t = t0 + int64_t(it) * (NT * 8) + tid + NT * k;
      if (t < t1) {
        const double v = sv[it & 1][k];
        const int c = coarse_bin(coarse_pos_of(a, v, smax, binscale));
        br[t] = uint16_t(c);
        unsafeAtomicAdd(&hm[c], long_weight(a, smax, v));
        atomicAdd(&hc[c], 1u);
      }
    }
  }
  __syncthreads();
  const int64_t o = (row * a.nb1 + slab) * kBins1;
  for (int i = tid; i < kBins1; i += NT) {
    a.h1m[o + i] = hm[i];
    a.h1c[o + i] = hc[i];
  }
}

// Per row: coarse bin totals (slab partials summed in slab order), Z and the target, the crossing
// coarse bin, the weight ahead of it, and whether its entries fit the resolution buffer.
constexpr int kFindThreads = kBins1;
__global__ __launch_bounds__(kFindThreads) void k_long_find1(LongArgs a) {
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  __shared__ double wtot[kFindThreads / 64];
  __shared__ int hit_bin;
  __shared__ double hit_before;
  __shared__ uint32_t hit_count;
  RowInfo ri = a.info[row];
  if (ri.all) return;
  double m = 0.0;
  uint32_t cn = 0;
  const int64_t o = row * a.nb1 * kBins1 + tid;
#pragma unroll 16
  for (int sl = 0; sl < a.nb1; ++sl) {
    m += a.h1m[o + int64_t(sl) * kBins1];
    cn += a.h1c[o + int64_t(sl) * kBins1];
  }
  double Z;
  const double incl = block_scan<kFindThreads>(m, wtot, &Z);
  const double target = a.topp ? a.p * Z : double(long_k(a, b));
  if (tid == 0) hit_bin = 0x7FFFFFFF;
  __syncthreads();
  const double excl = incl - m;
  if (excl + m >= target) atomicMin(&hit_bin, tid);
  __syncthreads();
  const int bin1 = hit_bin;
  if (bin1 == tid) {
    hit_before = excl;
    hit_count = cn;
  }
  __syncthreads();
  if (tid == 0) {
    if (bin1 == 0x7FFFFFFF) {
      ri.all = 1;  // rounding left the target above the total weight: keep every entry
    } else {
      ri.bin1 = bin1;
      ri.before1 = hit_before;
      ri.target = target;
      ri.gather = hit_count <= uint32_t(kResolveCap);
    }
    a.info[row] = ri;
  }
}

// Per slab: the row's bitmap (entries of coarse bins ahead of the crossing bin, or every entry
// when the whole row is kept; zero for local heads) and, in gather mode, the indices of the
// crossing bin's entries in the slab's region of the resolution buffer. Each lane takes 8
// consecutive entries (one 16-byte load of their bins, all of a slab's loads issued at once) and
// writes their 8 bits as one byte of the bitmap.
__global__ __launch_bounds__(kLongThreads) void k_long_mark(LongArgs a) {
  constexpr int NT = kLongThreads;
  const int b = blockIdx.z, h = blockIdx.y, slab = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row = int64_t(b) * a.Hq + h;
  const int64_t t0 = int64_t(slab) * kLongBlock;
  const int64_t t1 = t0 + kLongBlock < a.len ? t0 + kLongBlock : a.len;
  uint32_t* bw = a.bits + row * a.words;
  if ((a.local_mask >> (h / a.G)) & 1) {
    for (int64_t w = (t0 >> 5) + tid; w < ((t1 + 31) >> 5); w += NT) bw[w] = 0u;
    return;
  }
  __shared__ int scnt;
  if (tid == 0) scnt = 0;
  __syncthreads();
  const RowInfo ri = a.info[row];
  const bool gather = !ri.all && ri.gather;
  const uint16_t* br = a.cbin + row * a.cstride;
  uint8_t* bb = reinterpret_cast<uint8_t*>(bw);
  int32_t* out = a.cidx + (row * a.nb1 + slab) * kResolveCap;
  constexpr int kVec = kLongBlock / (NT * 8);  // 16-byte pieces per lane
  // piece v of lane tid covers entries t0 + 8 * (tid + NT v) .. + 7; pieces past the slab load
  // the slab's last piece again (rows are padded to a multiple of 8 entries) and are masked
  uint4 pc[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    int64_t e = t0 + 8 * (int64_t(tid) + NT * v);
    const int64_t last = (t1 - 1) & ~int64_t(7);
    e = e < last ? e : last;
    pc[v] = ri.all ? make_uint4(0, 0, 0, 0) : ld16(br + e);
  }
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    const int64_t e0 = t0 + 8 * (int64_t(tid) + NT * v);
    const uint16_t* cb = reinterpret_cast<const uint16_t*>(&pc[v]);
    uint32_t sel = 0, cand = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool valid = e0 + u < t1;
      sel |= (valid && (ri.all || cb[u] < ri.bin1)) ? (1u << u) : 0u;
      cand |= (gather && valid && cb[u] == ri.bin1) ? (1u << u) : 0u;
    }
    if (e0 < ((t1 + 31) & ~int64_t(31))) bb[e0 >> 3] = uint8_t(sel);  // whole words, zero past the row
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
        if (pos < kResolveCap) out[pos] = int32_t(e0 + u);
        ++pos;
      }
    }
  }
  __syncthreads();
  if (tid == 0) a.ccnt[row * a.nb1 + slab] = scnt < kResolveCap ? scnt : kResolveCap;
}

// Exact resolution of the crossing bin's entries. They span one interval of the bin axis; a
// kSub-bin histogram of that interval (monotone in the score) finds the sub-bin where the running
// weight, started at the weight ahead of the interval, crosses the target. Entries of earlier
// sub-bins are selected; the crossing sub-bin's entries are ranked by counting in (score desc,
// index asc) order and walked to the first crossing. A crossing sub-bin of more than kSubCap
// entries is resolved by sorting every gathered entry instead.
constexpr int kSub = 1024;
constexpr int kSubCap = 256;
constexpr int kResolveThreads = 512;

__global__ __launch_bounds__(kResolveThreads) void k_long_resolve(LongArgs a) {
  constexpr int NT = kResolveThreads;
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  if ((a.local_mask >> (h / a.G)) & 1) return;
  const int64_t row = int64_t(b) * a.Hq + h;
  const RowInfo ri = a.info[row];
  if (ri.all) return;
  __shared__ uint64_t keys[kResolveCap];
  __shared__ int32_t idx[kResolveCap];
  __shared__ uint16_t sub[kResolveCap];
  __shared__ double hm[kSub];
  __shared__ uint32_t hc[kSub];
  __shared__ uint64_t xkey[kSubCap];
  __shared__ int32_t xidx[kSubCap];
  __shared__ double xw[kSubCap];
  __shared__ int32_t ridx[kSubCap];
  __shared__ double wtot[NT / 64];
  __shared__ double buf[kSelThreads];
  __shared__ int soff[NT + 1];
  __shared__ int hit_bin, nx, ibuf;
  __shared__ double hit_before;
  const double* sr = a.s0 + row * a.len;
  uint32_t* bw = a.bits + row * a.words;
  int n;
  double before, dlo, sscale;
  if (ri.gather) {
    // ---- the crossing bin's entries, slab after slab (slab s owns soff[s] .. soff[s+1])
    const int per = (a.nb1 + NT - 1) / NT;  // slabs per thread
    double local = 0.0;
    for (int s = tid * per; s < min(a.nb1, tid * per + per); ++s) local += double(a.ccnt[row * a.nb1 + s]);
    double tot;
    const double incl = block_scan<NT>(local, wtot, &tot);
    // soff holds the first position of every thread's first slab; slabs inside a thread's range
    // are walked in order below
    soff[tid] = int(incl - local);
    if (tid == NT - 1) soff[NT] = int(tot);
    __syncthreads();
    n = int(tot) < kResolveCap ? int(tot) : kResolveCap;
    if (n == 0) return;
    constexpr int PER = kResolveCap / NT;
    int32_t tv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + NT * k;
      const int j = i < n ? i : n - 1;
      // owner thread range: last thread u with soff[u] <= j
      int lo = 0, hi = NT;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (soff[mid] <= j) lo = mid; else hi = mid;
      }
      int s = lo * per, off = j - soff[lo];
      // with one slab per thread, soff[lo + 1] - soff[lo] is that slab's count, so j lies in slab
      // lo and no count needs reading
      while (per > 1 && s + 1 < a.nb1 && off >= a.ccnt[row * a.nb1 + s]) {  // at most `per` steps
        off -= a.ccnt[row * a.nb1 + s];
        ++s;
      }
      tv[k] = a.cidx[(row * a.nb1 + s) * kResolveCap + off];
    }
    double sv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) sv[k] = sr[tv[k]];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + NT * k;
      if (i < n) {
        keys[i] = dkey(sv[k]);
        idx[i] = tv[k];
      }
    }
    before = ri.before1;
    dlo = double(ri.bin1);
    sscale = double(kSub);
  } else {
    // ---- crossing coarse bin too full: fine histogram of its entries over one pass of the row
    double* fm = reinterpret_cast<double*>(keys);    // kBins2 doubles
    uint32_t* fc = reinterpret_cast<uint32_t*>(idx);  // kBins2 counts
    for (int i = tid; i < kBins2; i += NT) {
      fm[i] = 0.0;
      fc[i] = 0;
    }
    if (tid == 0) {
      nx = 0;
      hit_bin = 0x7FFFFFFF;
    }
    __syncthreads();
    const uint16_t* br = a.cbin + row * a.cstride;
    for (int64_t t = tid; t < a.len; t += NT) {
      if (br[t] == ri.bin1) {
        const double s = sr[t];
        const int f = fine_bin(coarse_pos_of(a, s, ri.smax, ri.binscale), ri.bin1);
        unsafeAtomicAdd(&fm[f], long_weight(a, ri.smax, s));
        atomicAdd(&fc[f], 1u);
      }
    }
    __syncthreads();
    constexpr int FPER = kBins2 / NT;
    double m[FPER];
    double local = 0.0;
#pragma unroll
    for (int j = 0; j < FPER; ++j) {
      m[j] = fm[FPER * tid + j];
      local += m[j];
    }
    double tot;
    const double incl = block_scan<NT>(local, wtot, &tot);
    double c = ri.before1 + (incl - local);
    const double c0 = c;
#pragma unroll
    for (int j = 0; j < FPER; ++j) {
      const double cn = c + m[j];
      if (cn >= ri.target) {
        atomicMin(&hit_bin, FPER * tid + j);
        break;
      }
      c = cn;
    }
    __syncthreads();
    const int bin2 = hit_bin == 0x7FFFFFFF ? kBins2 : hit_bin;  // none: keep the whole coarse bin
    if (bin2 < kBins2 && bin2 / FPER == tid) {
      double cb = c0;
      for (int j = 0; j < bin2 - FPER * tid; ++j) cb += m[j];
      hit_before = cb;
    }
    __syncthreads();
    const uint32_t cnt2 = bin2 < kBins2 ? fc[bin2] : 0u;
    if (cnt2 > uint32_t(kResolveCap)) {
      // The crossing fine bin holds more entries than the buffer. Resolvable here when they all
      // carry one score (exact ties): their order is then the index order and their weights are
      // equal. Entries are taken in contiguous per-thread index ranges, so a thread-order scan of
      // their counts ranks them by index.
      __shared__ double tmin[NT / 64], tmax[NT / 64];
      const int64_t per = (a.len + NT - 1) / NT;
      const int64_t r0 = int64_t(tid) * per, r1 = r0 + per < a.len ? r0 + per : a.len;
      double lo = kPosInfD, hi = kNegInfD;
      int mine = 0;
      for (int64_t t = r0; t < r1; ++t) {
        if (br[t] == ri.bin1) {
          const double sc = sr[t];
          const int f = fine_bin(coarse_pos_of(a, sc, ri.smax, ri.binscale), ri.bin1);
          if (f < bin2) {
            atomicOr(&bw[t >> 5], 1u << (t & 31));
          } else if (f == bin2) {
            lo = fmin(lo, sc);
            hi = fmax(hi, sc);
            ++mine;
          }
        }
      }
      lo = wave_min_dpp(lo);
      hi = wave_max_dpp(hi);
      if ((tid & 63) == 0) {
        tmin[tid >> 6] = lo;
        tmax[tid >> 6] = hi;
      }
      __syncthreads();
      for (int w = 0; w < NT / 64; ++w) {
        lo = fmin(lo, tmin[w]);
        hi = fmax(hi, tmax[w]);
      }
      if (lo != hi) {  // near-equal but distinct scores beyond the buffer: not resolved
        if (tid == 0) atomicOr(&a.status[0], 1u);
        return;
      }
      const double wt = long_weight(a, ri.smax, lo);
      auto same = [&](int) { return wt; };
      const int pos = block_first_crossing(int(cnt2), hit_before, ri.target, same, buf, &ibuf);
      const int take = pos < 0 ? int(cnt2) : pos + 1;
      double tot;
      const int rank0 = int(block_scan<NT>(double(mine), wtot, &tot)) - mine;
      int rank = rank0;
      for (int64_t t = r0; t < r1 && rank < take; ++t) {
        if (br[t] == ri.bin1 && fine_bin(coarse_pos_of(a, sr[t], ri.smax, ri.binscale), ri.bin1) == bin2) {
          atomicOr(&bw[t >> 5], 1u << (t & 31));
          ++rank;
        }
      }
      return;
    }
    // the fine histogram is dead from here: keys / idx take the candidates
    for (int64_t t = tid; t < a.len; t += NT) {
      if (br[t] == ri.bin1) {
        const double s = sr[t];
        const int f = fine_bin(coarse_pos_of(a, s, ri.smax, ri.binscale), ri.bin1);
        if (f < bin2) {
          atomicOr(&bw[t >> 5], 1u << (t & 31));
        } else if (f == bin2) {
          const int q = atomicAdd(&nx, 1);
          if (q < kResolveCap) {
            keys[q] = dkey(s);
            idx[q] = int32_t(t);
          } else {
            atomicOr(&a.status[0], 1u);
          }
        }
      }
    }
    __syncthreads();
    n = nx < kResolveCap ? nx : kResolveCap;
    if (n == 0) return;
    before = hit_before;
    dlo = double(ri.bin1) + double(bin2) / double(kBins2);
    sscale = double(kSub) * double(kBins2);
  }
  // ---- sub-bin histogram of the gathered entries
  for (int i = tid; i < kSub; i += NT) {
    hm[i] = 0.0;
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
    unsafeAtomicAdd(&hm[sb], long_weight(a, ri.smax, s));
    atomicAdd(&hc[sb], 1u);
  }
  __syncthreads();
  constexpr int SPER = kSub / NT;
  double m[SPER];
  double local = 0.0;
#pragma unroll
  for (int j = 0; j < SPER; ++j) {
    m[j] = hm[SPER * tid + j];
    local += m[j];
  }
  double tot;
  const double incl = block_scan<NT>(local, wtot, &tot);
  double c = before + (incl - local);
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
    for (int i = tid; i < n; i += NT) atomicOr(&bw[idx[i] >> 5], 1u << (idx[i] & 31));
    return;
  }
  if (hc[hb] <= uint32_t(kSubCap)) {
    for (int i = tid; i < n; i += NT) {
      const int sb = sub[i];
      if (sb < hb) {
        atomicOr(&bw[idx[i] >> 5], 1u << (idx[i] & 31));
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
      xw[r] = long_weight(a, ri.smax, dkey_inv(kq));
      ridx[r] = iq;
    }
    __syncthreads();
    if (tid == 0) {
      double cw = hit_before;
      int ns = nc;
      for (int r = 0; r < nc; ++r) {
        cw += xw[r];
        if (cw >= ri.target) {
          ns = r + 1;
          break;
        }
      }
      ibuf = ns;
    }
    __syncthreads();
    for (int r = tid; r < ibuf; r += NT) atomicOr(&bw[ridx[r] >> 5], 1u << (ridx[r] & 31));
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
  auto weight = [&](int i) { return long_weight(a, ri.smax, dkey_inv(keys[i])); };
  const int pos = block_first_crossing(n, before, ri.target, weight, buf, &ibuf);
  const int n_sel = pos < 0 ? n : pos + 1;
  for (int i = tid; i < n_sel; i += NT) atomicOr(&bw[idx[i] >> 5], 1u << (idx[i] & 31));
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
};

constexpr int kCovThreads = 256;
constexpr int kCovRankEntries = 32;   // entries ranked per workgroup
constexpr int kCovRankPerThread = 4;  // entries per thread (each key read serves all of them)

__global__ __launch_bounds__(kCovThreads) void k_cov_mass(CoverageArgs a) {
  constexpr int NT = kCovThreads, PT = kSmallRowMax / NT;
  __shared__ double wred[NT / 64];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L = int(a.len);
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
  if (m >= a.len) return;
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
  const int L = int(a.len);
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
  const int L = int(a.len);
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
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t w = w0 + tid + 256 * i;
    if (w < a.words) {
      uint32_t x = local ? edge_bits(w, a.n, a.sink, a.window) : (u[i] | edge_bits(w, a.n, a.keep_first, a.keep_last));
      if (w == a.words - 1 && (a.n & 31)) x &= (1u << (a.n & 31)) - 1u;
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
  a.h1m = at<double>(ws, p.o_h1m);
  a.h1c = at<uint32_t>(ws, p.o_h1c);
  a.cbin = at<uint16_t>(ws, p.o_cbin);
  a.cstride = (p.len0 + 7) & ~int64_t(7);
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
    const int L = int(p.len0);
    hipLaunchKernelGGL(k_cov_mass, dim3(Hq, B), dim3(kCovThreads), 0, st, ca);
    hipLaunchKernelGGL(k_cov_importance, dim3((L + kCovThreads - 1) / kCovThreads, B), dim3(kCovThreads), 0, st, ca);
    hipLaunchKernelGGL(k_cov_rank, dim3((L + kCovRankEntries - 1) / kCovRankEntries, B), dim3(kCovThreads), 0, st, ca);
    hipLaunchKernelGGL(k_cov_budget, dim3(B), dim3(kCovBudgetThreads), 0, st, ca);
  }
  if (c.mode == SD_HIER_TOPK || !p.long0) {
    // rows of at most kSmallRowMax entries: selection, union and compaction in one kernel
    hipLaunchKernelGGL(k_select_head, dim3(Hq, B), dim3(kSelT), 0, st, group_args(p, ws, level));
    return int(hipGetLastError());
  }
  const LongArgs a = long_args(p, ws);
  const dim3 rows(Hq, B), blocks(p.long_blocks, Hq, B);
  hipLaunchKernelGGL(k_long_hist, blocks, dim3(kLongThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_find1, rows, dim3(kFindThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_mark, blocks, dim3(kLongThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_resolve, rows, dim3(kResolveThreads), 0, st, a);
  int e = int(hipGetLastError());
  if (e) return e;
  return union_impl(p, ws, st);
}

// ---- long-row selection over caller-given rows (the prefill path's budget and per-head top-k)
namespace {
struct LongScratch {
  size_t info, h1m, h1c, cbin, cidx, ccnt, total;
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
  l.h1m = take(size_t(rows * nb1 * kBins1) * 8);
  l.h1c = take(size_t(rows * nb1 * kBins1) * 4);
  l.cbin = take(size_t(rows * ((len + 7) & ~int64_t(7))) * 2);
  l.cidx = take(size_t(rows * nb1 * kResolveCap) * 4);
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
  a.h1m = reinterpret_cast<double*>(r.scratch + l.h1m);
  a.h1c = reinterpret_cast<uint32_t*>(r.scratch + l.h1c);
  a.cbin = reinterpret_cast<uint16_t*>(r.scratch + l.cbin);
  a.cstride = (r.len + 7) & ~int64_t(7);
  a.cidx = reinterpret_cast<int32_t*>(r.scratch + l.cidx);
  a.ccnt = reinterpret_cast<int32_t*>(r.scratch + l.ccnt);
  a.bits = r.bits;
  a.words = r.words;
  a.status = r.status;
  const dim3 rows(r.H, r.B), blocks(a.nb1, r.H, r.B);
  hipLaunchKernelGGL(k_long_hist, blocks, dim3(kLongThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_find1, rows, dim3(kFindThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_mark, blocks, dim3(kLongThreads), 0, st, a);
  hipLaunchKernelGGL(k_long_resolve, rows, dim3(kResolveThreads), 0, st, a);
  return int(hipGetLastError());
}

}  // namespace sd
