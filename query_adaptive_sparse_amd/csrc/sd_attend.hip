// Gathered split-K attention and the log-sum-exp combine.
//
// Work decomposition. Every (sequence, KV group) -- a "group" -- owns an ascending list of
// selected entries (chunks, or tokens). Its hybrid context is cut into 16-token tiles: raw tiles
// (the listed chunks' tokens, in list order) then summary tiles (the listed chunks' summary rows).
// The tiles of all groups, concatenated in group order, are split into contiguous,
// equal slices -- one per persistent workgroup (attend_blocks of them) -- so every workgroup streams the same number of
// bytes whatever the per-group list lengths are. Inside a workgroup the 4 waves take alternate
// tiles, each with its own online softmax, and merge in LDS whenever the slice leaves a group:
// one partial (o, lse) per (workgroup, group), written to pool slot (workgroup + group).
//
// Per tile and wave: q.K^T on MFMA with tokens as M and the group's heads as N (K fragments load
// straight from HBM in the A-operand layout), online softmax in base 2, then P.V on MFMA with head
// slots as M. P arrives from the logit layout with no data movement; for bf16 it is split into
// hi = bf16(p) (slots [0, G)) and lo = bf16(p - hi) (slots [G, 2G)) rows, which keeps fp32
// accuracy. V goes through LDS (row-major, padded rows) to reach the B-operand layout. The next
// tile's K and V loads are issued before the current tile is computed (a ring of register stages).
// K and V rows are read exactly once per call, so their loads are marked non-temporal: without
// the hint they evict each other in the per-XCD L2s and some XCDs stream 10-20% slower than others,
// which leaves the whole chip waiting on the slowest one at the end of the launch.
#include "sd_device.h"

namespace sd {
namespace {

struct AttendArgs {
  const void* q;
  QRows qm;
  const void* k;
  const void* v;
  int64_t kv_sb, kv_sh, kv_st;
  const void* kg;
  const void* vg;
  int64_t g_sb, g_sh, g_st;
  const int32_t* list;
  const int32_t* cnt;
  int32_t* gpre_out;  // [n_groups + 1] tile prefix over groups, for the combine
  float* po;          // [attend_blocks + n_groups][G][D] partial outputs
  float* pl;          // [attend_blocks + n_groups][G] partial lse (natural log)
  int64_t n_list;     // list row stride (entries) = entries per row (M)
  int n_groups, Hk, Hq, G, chunk_shift;
  int attend_summary;  // 0 none, 1 the listed chunks' summaries, 2 every chunk's
  // bf16 P.V: with at most 8 query rows per group, the hi and lo halves of P share one MFMA in
  // rows [0, G) and [G, 2G); with more rows they go through two MFMAs into one accumulator
  // (the kernel's SPLIT instance)
  int pv_split;
  float scale_log2;
  // per-head masks (variant): head h sees only its own entries plus the forced ones
  int head_masks;
  const uint32_t* bits;  // per-head bitmaps [B][Hq][words]
  int64_t words;
  int keep_first, keep_last;
  uint64_t local_mask;
  // growing cache: the step's tokens per sequence (workspace copy [B]) and the capacity
  const int32_t* ctx_len;
  int64_t n_ctx;
};

template <typename T, int D>
struct Cfg {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int EPV = 16 / int(sizeof(T));   // elements per 16-byte piece
  static constexpr int PPR = D / EPV;               // 16-byte pieces per row
  static constexpr int VPL = kTile * PPR / 64;      // V pieces per lane per tile
  static constexpr int KQ = BF ? D / 32 : D / 16;   // K pieces per lane per tile
  static constexpr int QF = BF ? D / 32 : D / 4;    // query fragment registers
  static constexpr int kRowWords = D * int(sizeof(T)) / 4 + 4;  // padded LDS V row (32-bit words)
  static constexpr int kVtWords = kTile * kRowWords;
  static constexpr int kMergeWords = 16 * D + 32;
  static constexpr int kWaveWords = kVtWords > kMergeWords ? kVtWords : kMergeWords;
  // register stages of the load pipeline: about 8 KB of K / V in flight per wave beyond the tile
  // being computed. With non-temporal loads, deeper rings measured slower on MI355X (more requests
  // queued per wave, same bandwidth): 2 stages for 8 KB tiles (bf16, d = 128), 3 for 4 KB tiles.
  static constexpr int kTileBytes = 2 * kTile * D * int(sizeof(T));
  static constexpr int NS = 1 + (8192 / kTileBytes > 1 ? 8192 / kTileBytes : 1);
};

template <typename T, int D>
struct TileRegs {
  uint4 k[Cfg<T, D>::KQ];
  uint4 v[Cfg<T, D>::VPL];
};

// Per-wave running state of one group.
template <int D>
struct SoftmaxState {
  float m, l;
  f32x4 acc[D / 16];
};

constexpr int kListLds = 4096;
// Cost of starting a segment (a group's raw tiles, or its summary tiles) in tiles of streaming:
// the load ring refills and the query and list slice are reloaded. Each segment start counts as
// this many extra tiles when the tile sequence is cut into equal slices, so a slice that starts a
// segment carries fewer tiles (workgroups whose slice crossed a group boundary measured ~7 us
// slower at 128K context without it).
constexpr int kSegmentCost = 16;

// A group's cache at this step: its complete chunks (the selection entries, each with a summary
// row) and the raw tokens of its incomplete last chunk, which every head attends unselected.
struct GroupCache {
  int64_t M;   // complete chunks (entries)
  int tail;    // tokens of the incomplete last chunk (0 for token rows)
};
__device__ __forceinline__ GroupCache group_cache(const AttendArgs& a, int gid) {
  const int64_t n = seq_tokens(a.ctx_len, gid / a.Hk, a.n_ctx);
  const int64_t M = n >> a.chunk_shift;
  return GroupCache{M, int(n - (M << a.chunk_shift))};
}

// Extent of a group in the sliced sequence: [kSegmentCost virtual tiles, raw tiles (the listed
// chunks' tokens), tail tiles (the incomplete chunk's tokens), kSegmentCost virtual tiles, summary
// tiles]; an empty group has none.
__device__ __forceinline__ int summary_tiles(int cnt, int attend_summary, int64_t M) {
  return attend_summary == 2 ? int((M + kTile - 1) / kTile) : (attend_summary ? (cnt + kTile - 1) / kTile : 0);
}
__device__ __forceinline__ int group_extent(int cnt, int cs, int attend_summary, const GroupCache& gc) {
  cnt = cnt > 0 ? cnt : 0;
  if (cnt == 0 && gc.tail == 0) return 0;
  const int traw = ((cnt << cs) + kTile - 1) / kTile;
  const int ttail = (gc.tail + kTile - 1) / kTile;
  const int tsum = summary_tiles(cnt, attend_summary, gc.M);
  return kSegmentCost + traw + ttail + (tsum ? kSegmentCost + tsum : 0);
}

// How the rows of a run of tiles are found: the listed chunks' tokens (list entry, token in the
// chunk), the listed chunks' summary rows (list entry), or consecutive rows from a base (every
// chunk's summary, or the incomplete chunk's tokens).
enum RowKind { kRawRows = 0, kListedRows = 1, kDirectRows = 2 };

// Heads of group `gid` whose own selection holds entry e (bit j = head j of the group): every head
// for a forced entry or a local group.
__device__ __forceinline__ uint32_t head_mask_of(const AttendArgs& a, int gid, int e, int64_t M) {
  const int b = gid / a.Hk, g = gid - b * a.Hk;
  if (((a.local_mask >> g) & 1) || e < a.keep_first || int64_t(e) >= M - a.keep_last) return 0xFFFFu;
  uint32_t m = 0;
  for (int j = 0; j < a.G; ++j) {
    const uint32_t w = a.bits[(int64_t(b) * a.Hq + g * a.G + j) * a.words + (e >> 5)];
    m |= ((w >> (e & 31)) & 1u) << j;
  }
  return m;
}

template <typename T, int D, bool SPLIT>
struct Attender {
  using CF = Cfg<T, D>;
  const AttendArgs& a;
  const int lane, wave, n, c;
  const int32_t* lst;   // LDS list slice
  const uint16_t* lmask; // LDS head masks of the slice's entries (per-head-mask variant)
  uint32_t* vt;         // this wave's LDS region
  // current group
  int gid, G, hs;
  bool lo_row;
  const T* kb;
  const T* vb;
  int64_t st;
  // query fragments
  uint4 qf[CF::BF ? CF::QF : 1];
  float qf32[CF::BF ? 1 : CF::QF];

  __device__ Attender(const AttendArgs& args, const int32_t* l, const uint16_t* lm, uint32_t* v)
      : a(args), lane(threadIdx.x & 63), wave(threadIdx.x >> 6), n(lane & 15), c(lane >> 4), lst(l), lmask(lm),
        vt(v) {}

  __device__ void load_query(int group) {
    gid = group;
    G = a.G;
    hs = n < G ? n : (!SPLIT && n < 2 * G ? n - G : -1);
    lo_row = CF::BF && !SPLIT && n >= G && n < 2 * G;
    const int b = group / a.Hk, g = group - b * a.Hk;
    const T* qrow = reinterpret_cast<const T*>(a.q) + q_offset(a.qm, b, g * G + (hs < 0 ? 0 : hs));
    if constexpr (CF::BF) {
#pragma unroll
      for (int j = 0; j < CF::QF; ++j) qf[j] = hs >= 0 ? ld16(qrow + 32 * j + 8 * c) : make_uint4(0, 0, 0, 0);
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
  }

  // Base pointers of the raw (summary = false) or summary (true) rows of the current group,
  // starting at row `row0`.
  __device__ void set_kind(bool summary, int64_t row0 = 0) {
    const int b = gid / a.Hk, g = gid - b * a.Hk;
    if (summary) {
      kb = reinterpret_cast<const T*>(a.kg) + b * a.g_sb + int64_t(g) * a.g_sh + row0 * a.g_st;
      vb = reinterpret_cast<const T*>(a.vg) + b * a.g_sb + int64_t(g) * a.g_sh + row0 * a.g_st;
      st = a.g_st;
    } else {
      kb = reinterpret_cast<const T*>(a.k) + b * a.kv_sb + int64_t(g) * a.kv_sh + row0 * a.kv_st;
      vb = reinterpret_cast<const T*>(a.v) + b * a.kv_sb + int64_t(g) * a.kv_sh + row0 * a.kv_st;
      st = a.kv_st;
    }
  }

  // Row of token x of a tile: raw tiles, token v = first + x of the listed chunks' token sequence;
  // listed summary tiles, list entry first + x; direct tiles, row first + x from the base. `e0` is
  // the first list entry held in the LDS slice.
  __device__ __forceinline__ int64_t row_of(int kind, int first, int x, int nv, int e0) const {
    x = x < nv ? x : 0;  // padded positions read a valid row; their logits are masked
    if (kind == kDirectRows) return first + x;
    if (kind == kListedRows) return lst[first + x - e0];
    const int cs = a.chunk_shift;
    const int v = first + x;
    return (int64_t(lst[(v >> cs) - e0]) << cs) | (v & ((1 << cs) - 1));
  }

  __device__ __forceinline__ void issue(TileRegs<T, D>& r, int kind, int first, int nv, int e0) const {
    const T* kr = kb + row_of(kind, first, n, nv, e0) * st;
#pragma unroll
    for (int q = 0; q < CF::KQ; ++q) r.k[q] = ld16_stream(kr + (CF::BF ? 32 * q + 8 * c : (D / 4) * c + 4 * q));
#pragma unroll
    for (int kq = 0; kq < CF::VPL; ++kq) {
      const int pidx = kq * 64 + lane;
      const int x = pidx / CF::PPR, cp = pidx - x * CF::PPR;
      r.v[kq] = ld16_stream(vb + row_of(kind, first, x, nv, e0) * st + cp * CF::EPV);
    }
  }

  __device__ __forceinline__ void compute(const TileRegs<T, D>& r, int nv, SoftmaxState<D>& s, int kind,
                                          int first, int e0) {
    // ---- logits: S^T[token][slot]; lane (n, c) gets tokens 4c + i of head slot n
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (CF::BF) {
#pragma unroll
      for (int j = 0; j < CF::QF; ++j)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[j]),
                                                        __builtin_bit_cast(bf16x8, qf[j]), sacc, 0, 0, 0);
    } else {
#pragma unroll
      for (int q = 0; q < CF::KQ; ++q) {
        const float* f = reinterpret_cast<const float*>(&r.k[q]);
#pragma unroll
        for (int u = 0; u < 4; ++u) sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(f[u], qf32[4 * q + u], sacc, 0, 0, 0);
      }
    }
    // ---- V tile -> LDS, row-major with a 4-word pad per row
#pragma unroll
    for (int kq = 0; kq < CF::VPL; ++kq) {
      const int pidx = kq * 64 + lane;
      const int x = pidx / CF::PPR, cp = pidx - x * CF::PPR;
      *reinterpret_cast<uint4*>(vt + x * CF::kRowWords + cp * 4) = r.v[kq];
    }
    // ---- online softmax (base 2)
    float lg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[i] = 4 * c + i < nv ? sacc[i] * a.scale_log2 : kNegInf;
    if (a.head_masks && kind != kDirectRows && hs >= 0) {
      // per-head masks: a token whose entry is outside this head's own set is not attended (direct
      // rows -- every chunk's summary, the incomplete chunk's tokens -- are seen by every head)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = 4 * c + i < nv ? 4 * c + i : 0;
        const int ei = kind == kListedRows ? first + x - e0 : ((first + x) >> a.chunk_shift) - e0;
        if (!((lmask[ei] >> hs) & 1)) lg[i] = kNegInf;
      }
    }
    float mt = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(s.m, mt);
    const bool none = mn == kNegInf;
    // rescale only when some head's running max grew (rare after the first tiles)
    if (__ballot(mn > s.m)) {
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(s.m - mn);
      s.l *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * c + i);
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) s.acc[nb][i] *= ai;
      }
      s.m = mn;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = none ? 0.f : __builtin_amdgcn_exp2f(lg[i] - mn);
      s.l += pr[i];
    }
    // LDS operations of one wave complete in order: the V tile written above is visible to the
    // reads below without a wait; the barrier only keeps the compiler from reordering them.
    __builtin_amdgcn_wave_barrier();
    // ---- P V: P is the A operand (row = head slot, k = tokens 4c .. 4c+3), V the B operand
    if constexpr (CF::BF) {
      const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(vt);
      u16x4 pa, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t hi = f2bf(pr[i]);
        const uint16_t lo = f2bf(pr[i] - bf2f(hi));
        pa[i] = hs < 0 ? uint16_t(0) : (lo_row ? lo : hi);
        pl[i] = hs < 0 ? uint16_t(0) : lo;
      }
      if constexpr (!SPLIT) {
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          u16x4 vbf;
#pragma unroll
          for (int i = 0; i < 4; ++i) vbf[i] = vt16[(4 * c + i) * (2 * CF::kRowWords) + 16 * nb + n];
          s.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, pa),
                                                                 __builtin_bit_cast(bf16x4, vbf), s.acc[nb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          u16x4 vbf;
#pragma unroll
          for (int i = 0; i < 4; ++i) vbf[i] = vt16[(4 * c + i) * (2 * CF::kRowWords) + 16 * nb + n];
          s.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, pa),
                                                                 __builtin_bit_cast(bf16x4, vbf), s.acc[nb], 0, 0, 0);
          s.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, pl),
                                                                 __builtin_bit_cast(bf16x4, vbf), s.acc[nb], 0, 0, 0);
        }
      }
    } else {
      const float* vtf = reinterpret_cast<const float*>(vt);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = hs >= 0 ? pr[i] : 0.f;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb)
          s.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv, vtf[(4 * c + i) * CF::kRowWords + 16 * nb + n], s.acc[nb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // This wave's tiles of [u0, u1) (alternating with the other waves) through an NS-stage register
  // ring: the loads of the next NS - 1 tiles are in flight while a tile is computed. Tile u starts
  // at position kTile*u of the run's rows (see row_of); `limit` = rows in the run.
  __device__ void run(int kind, int u0, int u1, int limit, int e0, SoftmaxState<D>& s) {
    constexpr int NS = CF::NS;
    const int first = u0 + wave;
    if (first >= u1) return;
    const int nt = (u1 - first + kWaves - 1) / kWaves;  // this wave's tiles
    TileRegs<T, D> R[NS];
    auto tile = [&](int k) { return first + k * kWaves; };
    auto nv_of = [&](int t) { return min(kTile, limit - t * kTile); };
    // Loads are issued unconditionally (past the end they repeat the wave's last tile, which is
    // still cached), so the compiler can count the loads in flight exactly and wait only for the
    // stage being computed.
    auto clamp = [&](int k) { return tile(k < nt ? k : nt - 1); };
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) issue(R[k], kind, clamp(k) * kTile, nv_of(clamp(k)), e0);
    for (int k0 = 0; k0 < nt; k0 += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int k = k0 + j;
        const int kn = k + NS - 1;
        issue(R[(j + NS - 1) % NS], kind, clamp(kn) * kTile, nv_of(clamp(kn)), e0);
        if (k < nt) compute(R[j], nv_of(tile(k)), s, kind, tile(k) * kTile, e0);
      }
    }
  }
};

template <typename T, int D, bool SPLIT>
__global__ __launch_bounds__(256, 2) void k_attend(AttendArgs a) {
  using CF = Cfg<T, D>;
  __shared__ int32_t gpre[kMaxGroups + 1];
  __shared__ int32_t lst[kListLds];
  __shared__ uint16_t lmask[kListLds];
  __shared__ uint32_t wlds[kWaves * CF::kWaveWords];
  __shared__ int32_t sbuf[kWaves];
  const int tid = threadIdx.x;
  const int NG = a.n_groups;
  const int cs = a.chunk_shift;

  // ---- extent of every group (tiles plus segment costs), exclusive prefix in gpre[0..NG]
  {
    const int per = (NG + 255) / 256;
    const int g0 = tid * per;
    int sum = 0;
    for (int gg = g0; gg < min(NG, g0 + per); ++gg) {
      sum += group_extent(a.cnt[gg], cs, a.attend_summary, group_cache(a, gg));
    }
    // inclusive scan over the 256 threads in thread order: DPP within each wave, then the
    // earlier waves' totals (one barrier)
    const int incl = wave_scan_i32_dpp(sum, tid & 63);
    if ((tid & 63) == 63) sbuf[tid >> 6] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < (tid >> 6); ++w) run += sbuf[w];
    for (int gg = g0; gg < min(NG, g0 + per); ++gg) {
      gpre[gg] = run;
      run += group_extent(a.cnt[gg], cs, a.attend_summary, group_cache(a, gg));
    }
    if (tid == 255) gpre[NG] = run;  // the last thread's running sum is the total
    __syncthreads();
  }
  const int total = gpre[NG];
  if (blockIdx.x == 0)
    for (int i = tid; i <= NG; i += 256) a.gpre_out[i] = gpre[i];
  const int NB = gridDim.x;
  const int b0 = int((int64_t(blockIdx.x) * total) / NB);
  const int b1 = int((int64_t(blockIdx.x + 1) * total) / NB);
  if (b0 >= b1) return;

  // first group containing tile b0: last gi with gpre[gi] <= b0
  int lo = 0, hi = NG;  // invariant: gpre[lo] <= b0 < gpre[hi] (gpre[NG] = total > b0)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (gpre[mid] <= b0) lo = mid; else hi = mid;
  }

  const int wave = tid >> 6;
  uint32_t* vt = wlds + wave * CF::kWaveWords;
  Attender<T, D, SPLIT> at(a, lst, lmask, vt);
  const int lane = tid & 63, n = lane & 15, c = lane >> 4;
  // a piece of the list (ne <= kListLds entries) into LDS, in rounds of 8 entries per thread
  // whose loads (from clamped indices) are all issued before the first is stored: a piece costs
  // at most kListLds / 2048 memory round trips, not one per 256 entries
  auto load_list = [&](const int32_t* src, int ne, int gid, int64_t M) {
    constexpr int kPer = 8;
    for (int r0 = 0; r0 < ne; r0 += 256 * kPer) {
      int32_t ev[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = r0 + tid + 256 * k;
        ev[k] = src[i < ne ? i : ne - 1];
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = r0 + tid + 256 * k;
        if (i < ne) {
          lst[i] = ev[k];
          if (a.head_masks) lmask[i] = uint16_t(head_mask_of(a, gid, ev[k], M));
        }
      }
    }
  };

  for (int gi = lo; gi < NG && gpre[gi] < b1; ++gi) {
    const int s0 = max(b0, gpre[gi]) - gpre[gi];
    const int s1 = min(b1, gpre[gi + 1]) - gpre[gi];
    if (s0 >= s1) continue;
    const int cnt = a.cnt[gi];
    const GroupCache gc = group_cache(a, gi);
    const int ntok = cnt << cs;  // the listed chunks' tokens
    const int traw = (ntok + kTile - 1) / kTile;
    const int ttail = (gc.tail + kTile - 1) / kTile;
    at.load_query(gi);
    SoftmaxState<D> st;
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int32_t* glist = a.list + int64_t(gi) * a.n_list;

    // raw tiles [r0, r1) (the group's extent puts them at [kSegmentCost, kSegmentCost + traw)), in
    // pieces whose list entries fit the LDS buffer
    {
      const int r0 = max(s0, kSegmentCost) - kSegmentCost, r1 = min(s1, kSegmentCost + traw) - kSegmentCost;
      // a piece of u tiles spans at most (u * kTile) / C + 2 list entries
      const int64_t tps = (int64_t(kListLds - 2) << cs) / kTile;
      const int tiles_per_slice = int(tps < 1 ? 1 : (tps > (1 << 30) ? (1 << 30) : tps));
      at.set_kind(false);
      for (int u0 = r0; u0 < r1; u0 += tiles_per_slice) {
        const int u1 = min(r1, u0 + tiles_per_slice);
        const int e0 = (u0 * kTile) >> cs;
        const int e1 = min(cnt, ((u1 * kTile - 1) >> cs) + 1);
        __syncthreads();
        load_list(glist + e0, e1 - e0, gi, gc.M);
        __syncthreads();
        at.run(kRawRows, u0, u1, ntok, e0, st);
      }
    }
    // tail tiles [t0, t1) (at [kSegmentCost + traw, kSegmentCost + traw + ttail)): the incomplete
    // chunk's tokens, consecutive rows from its first token
    if (gc.tail) {
      const int base = kSegmentCost + traw;
      const int t0 = max(s0, base) - base, t1 = min(s1 - base, ttail);
      if (t0 < t1) {
        at.set_kind(false, gc.M << cs);
        at.run(kDirectRows, t0, t1, gc.tail, 0, st);
      }
    }
    // summary tiles [q0, q1) (at [2 kSegmentCost + traw + ttail, extent) of the group's extent): the
    // listed chunks' summary rows, or (attend_summary 2) every chunk's, addressed directly
    if (a.attend_summary) {
      const int tsum = summary_tiles(cnt, a.attend_summary, gc.M);
      const int nsum = a.attend_summary == 2 ? int(gc.M) : cnt;
      const int base = 2 * kSegmentCost + traw + ttail;
      const int q0 = max(s0, base) - base, q1 = min(s1 - base, tsum);
      at.set_kind(true);
      const int tiles_per_slice = a.attend_summary == 2 ? (1 << 30) : kListLds / kTile;
      for (int u0 = q0; u0 < q1; u0 += tiles_per_slice) {
        const int u1 = min(q1, u0 + tiles_per_slice);
        const int e0 = u0 * kTile;
        if (a.attend_summary == 1) {
          const int e1 = min(cnt, u1 * kTile);
          __syncthreads();
          load_list(glist + e0, e1 - e0, gi, gc.M);
          __syncthreads();
        }
        at.run(a.attend_summary == 2 ? kDirectRows : kListedRows, u0, u1, nsum, e0, st);
      }
    }

    // ---- merge the 4 waves into partial slot (workgroup + group)
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    __syncthreads();  // every wave is done with its V tile; reuse the LDS regions
    float* mw = reinterpret_cast<float*>(vt);  // [16][D] acc rows, then m[16], l[16]
    const int G = a.G;
    const bool lo_rows = CF::BF && !SPLIT;
    const int nslots = lo_rows ? 2 * G : G;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 4 * c + i;
        if (slot < nslots) mw[slot * D + 16 * nb + n] = st.acc[nb][i];
      }
    if (c == 0 && n < G) {
      mw[16 * D + n] = st.m;
      mw[16 * D + 16 + n] = st.l;
    }
    __syncthreads();
    const int64_t slot = int64_t(blockIdx.x) + gi;
    for (int it = tid; it < G * D; it += 256) {
      const int hh = it / D, dd = it - hh * D;
      float M = kNegInf;
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, reinterpret_cast<const float*>(wlds + w * CF::kWaveWords)[16 * D + hh]);
      float Ls = 0.f, O = 0.f;
      for (int w = 0; w < kWaves; ++w) {
        const float* ww = reinterpret_cast<const float*>(wlds + w * CF::kWaveWords);
        const float mw_ = ww[16 * D + hh];
        if (mw_ == kNegInf) continue;
        const float f = __builtin_amdgcn_exp2f(mw_ - M);
        Ls += ww[16 * D + 16 + hh] * f;
        float o = ww[hh * D + dd];
        if (lo_rows) o += ww[(hh + G) * D + dd];
        O += o * f;
      }
      a.po[(slot * G + hh) * D + dd] = Ls > 0.f ? O / Ls : 0.f;  // no tiles of the group: empty partial
      if (dd == 0) a.pl[slot * G + hh] = (M + __log2f(Ls)) * 0.6931471805599453f;
    }
    __syncthreads();
  }
}

// floor(a / b) for 0 <= a, 0 < b, both below 2^53: the fp64 quotient truncated is within one of
// it, and one exact integer step corrects it (a 64-bit integer division is a long software
// sequence on the GPU)
__device__ __forceinline__ int64_t div_floor(int64_t a, int64_t b) {
  int64_t q = int64_t(double(a) / double(b));
  if (q * b > a)
    --q;
  else if ((q + 1) * b <= a)
    ++q;
  return q;
}

// LSE combine. One workgroup of NT threads per (sequence, query row): the partials of the head's
// group are the pool slots (k + group) of the persistent workgroups k whose tile slice meets the
// group. Thread j holds partial j's lse; each thread accumulates one output dimension over a fixed
// subset of the partials (j = grp, grp + NGRP, ...), kCombinePrefetch loads at a time, and the
// first of those rounds is issued with the lse loads, before the max is known. Beyond NT partials
// the rest is taken in further rounds. Summation order is fixed: the result is deterministic. NT
// is 256 when groups have few partials (many groups share the persistent workgroups), else 1024.
constexpr int kCombinePrefetch = 12;

template <int D, int NT>
__global__ __launch_bounds__(NT) void k_combine(const float* __restrict__ po, const float* __restrict__ pl,
                                                const int32_t* __restrict__ gpre, int n_groups, int nb_attend,
                                                int G, int Hq, int Hk, int Gq, float* __restrict__ out,
                                                float* __restrict__ lse) {
  constexpr int NW = NT / 64;
  constexpr int NGRP = NT / D;  // thread groups, each covering all D dims
  constexpr int U = kCombinePrefetch;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int gid = b * Hk + h / G, hh = h % G;
  // query row h = g G + t Gq + j (token t, head g Gq + j) -> output row [b][t][g Gq + j]
  int64_t hrow = int64_t(b) * Hq + h;
  if (G != Gq) {
    const int tq = hh / Gq, HqU = Hq / (G / Gq);
    hrow = (int64_t(b) * (G / Gq) + tq) * HqU + (h / G) * Gq + (hh - tq * Gq);
  }
  const int64_t T = gpre[n_groups];
  const int64_t t0 = gpre[gid], t1 = gpre[gid + 1];
  __shared__ float red[NW], red2[NW];
  __shared__ float wj[NT];
  __shared__ float part[NGRP][D];
  if (t0 == t1) {
    for (int d = tid; d < D; d += NT) out[hrow * D + d] = 0.f;
    if (tid == 0) lse[hrow] = kNegInf;
    return;
  }
  const int64_t NB = nb_attend;
  const int k0 = int(div_floor((t0 + 1) * NB - 1, T));
  const int nt = int(div_floor(t1 * NB - 1, T)) - k0 + 1;
  // with at least one tile per workgroup every slice is non-empty
  const bool all_live = T >= NB;
  auto live = [&](int k) { return all_live || div_floor(int64_t(k) * T, NB) < div_floor(int64_t(k + 1) * T, NB); };
  auto lse_of = [&](int j) { return live(k0 + j) ? pl[(int64_t(k0 + j) + gid) * G + hh] : kNegInf; };
  auto prow = [&](int j) { return po + ((int64_t(k0 + j) + gid) * G + hh) * D; };
  const int grp = tid / D, d = tid - grp * D;
  // an empty slice's slot is never written: it is read, but its weight is 0 and it is skipped
  float v[U];
  auto load_round = [&](int c0, int jb, int n) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + NGRP * u;
      v[u] = j < n ? prow(c0 + j)[d] : 0.f;
    }
  };
  const float lv = tid < nt ? lse_of(tid) : kNegInf;
  load_round(0, grp, min(NT, nt));
  float M = lv;
  for (int j = tid + NT; j < nt; j += NT) M = fmaxf(M, lse_of(j));
  for (int o = 32; o; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = red[0];
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
  float acc = 0.f, wsum = 0.f;
  for (int c0 = 0; c0 < nt; c0 += NT) {
    const int n = min(NT, nt - c0);
    __syncthreads();  // the previous round's weights are consumed
    float w = 0.f;
    if (tid < n) {
      const float l = c0 == 0 ? lv : lse_of(c0 + tid);
      w = live(k0 + c0 + tid) ? __expf(l - M) : 0.f;
      wj[tid] = w;
    }
    wsum += w;
    __syncthreads();
    for (int jb = grp; jb < n; jb += NGRP * U) {
      if (c0 > 0 || jb > grp) load_round(c0, jb, n);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = jb + NGRP * u;
        if (j < n) {
          const float wu = wj[j];
          acc += wu != 0.f ? wu * v[u] : 0.f;
        }
      }
    }
  }
  part[grp][d] = acc;
  for (int o = 32; o; o >>= 1) wsum += __shfl_xor(wsum, o);
  if (lane == 0) red2[wave] = wsum;
  __syncthreads();
  float L = red2[0];
  for (int w = 1; w < NW; ++w) L += red2[w];
  for (int e = tid; e < D; e += NT) {
    float o = 0.f;
    for (int g2 = 0; g2 < NGRP; ++g2) o += part[g2][e];
    out[hrow * D + e] = o / L;
  }
  if (tid == 0) lse[hrow] = M + __logf(L);
}

}  // namespace

int launch_attend(const Plan& p, const sd_tensors& t, char* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sd_config& c = p.cfg;
  AttendArgs a;
  a.q = t.q;
  a.qm = QRows{t.q_sb, t.q_st, t.q_sh, p.G, p.Gq};
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
  a.gpre_out = at<int32_t>(ws, p.o_gpre);
  a.po = at<float>(ws, p.o_po);
  a.pl = at<float>(ws, p.o_pl);
  a.n_list = p.M;
  a.n_groups = c.batch * c.n_kv_heads;
  a.Hk = c.n_kv_heads;
  a.Hq = c.n_q_heads;
  a.G = p.G;
  int cs = 0;
  while ((1 << cs) < c.chunk_size) ++cs;
  a.chunk_shift = cs;
  a.attend_summary = c.attend_summary;
  a.pv_split = c.kv_dtype == SD_BF16 && 2 * p.G > 16;
  a.scale_log2 = c.softmax_scale * 1.4426950408889634f;
  a.head_masks = c.head_masks;
  a.bits = at<uint32_t>(ws, p.o_bits);
  a.words = p.words;
  a.keep_first = c.keep_first;
  a.keep_last = c.keep_last;
  a.local_mask = p.local_mask;
  a.ctx_len = at<int32_t>(ws, p.o_ctx);
  a.n_ctx = c.n_ctx;
  const dim3 grid(p.attend_blocks);
  if (c.kv_dtype == SD_BF16) {
    if (c.head_dim == 128) {
      if (a.pv_split)
        hipLaunchKernelGGL((k_attend<uint16_t, 128, true>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((k_attend<uint16_t, 128, false>), grid, dim3(256), 0, st, a);
    } else {
      if (a.pv_split)
        hipLaunchKernelGGL((k_attend<uint16_t, 64, true>), grid, dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((k_attend<uint16_t, 64, false>), grid, dim3(256), 0, st, a);
    }
  } else {
    if (c.head_dim == 128)
      hipLaunchKernelGGL((k_attend<float, 128, false>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_attend<float, 64, false>), grid, dim3(256), 0, st, a);
  }
  return int(hipGetLastError());
}

int launch_combine(const Plan& p, char* ws, float* out, float* lse, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sd_config& c = p.cfg;
  const dim3 grid(c.n_q_heads, c.batch);
  const int NG = c.batch * c.n_kv_heads;
  // partials per group: about attend_blocks / groups + 1
  const bool few = int64_t(p.attend_blocks) <= int64_t(16) * NG;
#define SD_COMBINE(D, NT)                                                                                   \
  hipLaunchKernelGGL((k_combine<D, NT>), grid, dim3(NT), 0, st, at<float>(ws, p.o_po), at<float>(ws, p.o_pl), \
                     at<int32_t>(ws, p.o_gpre), NG, p.attend_blocks, p.G, c.n_q_heads, c.n_kv_heads, p.Gq, out, lse)
  if (c.head_dim == 128) {
    if (few) SD_COMBINE(128, 256); else SD_COMBINE(128, 1024);
  } else {
    if (few) SD_COMBINE(64, 256); else SD_COMBINE(64, 1024);
  }
#undef SD_COMBINE
  return int(hipGetLastError());
}

const char* hip_error_string(int code) { return hipGetErrorString(static_cast<hipError_t>(code)); }

}  // namespace sd
