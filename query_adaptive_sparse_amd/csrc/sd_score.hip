// Score kernels: summary / meta-summary / candidate rows, proxy query and proxy scores.
//
// Compiled with -ffp-contract=off: every fused multiply-add is an explicit fma(), so fp64 score
// arithmetic can be matched bit for bit by a sequential CPU evaluation.
#include "sd_device.h"

namespace sd {
namespace {
// ---------------------------------------------------------------------------------------------
// Scores. A workgroup scores 64 RPT summary rows (or candidate rows) for the query rows ("slots")
// of one KV group: it stages the slots' queries in LDS as fp64 (exact) and the key rows in LDS
// (each wave its own rows, one coalesced pass), then 4 lanes share RPT rows and each runs the dot
// products of HPT slots with each of its RPT rows, one fp64 fma per dimension in index order. A
// product of two bf16 or two fp32 values is exact in fp64, so fma(q, k, acc) equals the CPU's
// acc + q*k step for step. A lane converts each key element once for its HPT chains, and each
// query value it reads from LDS serves its RPT rows: the LDS reads of the queries, not HBM, bound
// this kernel, so RPT = 2 halves them per row when there are rows enough for two workgroups per CU
// at that size (else RPT = 1, for more workgroups). The HPT x RPT independent chains hide the fma
// latency.
// Block (0, 0, 0) also clears the device status words and the per-group arrival counters of the
// selection.
// ---------------------------------------------------------------------------------------------
template <typename T, int D, int HPT, int RPT>
__global__ __launch_bounds__(256) void k_score_rows(const T* __restrict__ q, QRows qm,
                                                    const T* __restrict__ keys, int64_t k_sb, int64_t k_sh,
                                                    int64_t k_st, const int32_t* __restrict__ cand,
                                                    int64_t n_rows, int64_t n_keys, int G, int Hq,
                                                    uint64_t local_mask, double* __restrict__ out, int64_t out_len,
                                                    uint32_t* __restrict__ status, int32_t* __restrict__ arrivals,
                                                    int n_groups, StepLens lens) {
  constexpr int kScoreRows = 64 * RPT;
  constexpr int EPV = 16 / int(sizeof(T));
  constexpr int PPR = D / EPV;                          // 16-byte pieces per row
  constexpr int QW = D + 2;                             // padded fp64 query row
  constexpr int KW = (D * int(sizeof(T)) + 16) / 16;    // padded key row, in 16-byte pieces
  __shared__ double qs[kMaxGroup * QW];
  __shared__ uint4 ks[kScoreRows * KW];
  const int b = blockIdx.z, y = blockIdx.y, tid = threadIdx.x;
  if (status && blockIdx.x == 0 && y == 0 && b == 0) {
    if (tid < 16) status[tid] = 0;
    for (int i = tid; i < n_groups; i += 256) arrivals[i] = 0;
    lens.publish(tid, 256);
  }
  const int g = cand ? y / G : y;
  if ((local_mask >> g) & 1) return;
  const int h0 = cand ? y : y * G;
  const int nh = cand ? 1 : G;
  const int64_t r0 = int64_t(blockIdx.x) * kScoreRows;
  // rows of this sequence: its complete chunks when the cache grows (candidate rows: all)
  const int64_t rows_b = cand ? n_rows : lens.entries(b, n_rows);
  if (r0 >= rows_b) return;
  // the slots' query elements (4 HPT slots at most: one unrolled round of loads from clamped rows),
  // then the key rows of this workgroup, 16 bytes per thread per step (rows past the end repeat
  // the last); the queries are staged in LDS while the key loads are in flight
  constexpr int QPT = 4 * HPT * D / 256;
  T qv[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + 256 * k, j = i / D, dd = i - j * D;
    qv[k] = q[q_offset(qm, b, h0 + (j < nh ? j : nh - 1)) + dd];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the key loads
  // lane l of wave w scores rows 16 w + l / 4 + 64 i (i < RPT); the wave loads exactly those rows,
  // so that it can start on them as soon as its own loads arrive, with no workgroup barrier between
  // the loads and the arithmetic
  constexpr int WROWS = 16 * RPT;
  constexpr int KPT = WROWS * PPR / 64;
  uint4 kreg[KPT];
  const T* kbase = keys + b * k_sb + int64_t(g) * k_sh;
  const int wv = tid >> 6, ln = tid & 63;
  auto piece_local = [&](int k) {  // row in the workgroup
    const int e = (ln + 64 * k) / PPR;
    return 16 * wv + 64 * (e >> 4) + (e & 15);
  };
  auto piece_col = [&](int k) { return (ln + 64 * k) % PPR; };
  auto piece_row = [&](int k) {
    const int r = piece_local(k);
    return int32_t(r0 + r < n_rows ? r0 + r : n_rows - 1);
  };
  if (cand) {
    // candidate rows: every chunk id is looked up first, then every key piece loaded
    const int32_t* cr = cand + (int64_t(b) * Hq + h0) * out_len;
    int32_t src[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) src[k] = cr[piece_row(k)];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int64_t sk = src[k] < 0 ? 0 : (src[k] < n_keys ? src[k] : n_keys - 1);
      kreg[k] = ld16(kbase + sk * k_st + piece_col(k) * EPV);
    }
  } else {
#pragma unroll
    for (int k = 0; k < KPT; ++k) kreg[k] = ld16(kbase + int64_t(piece_row(k)) * k_st + piece_col(k) * EPV);
  }
  __builtin_amdgcn_sched_barrier(0);  // every key load is issued before the queries are staged
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + 256 * k, j = i / D, dd = i - j * D;
    if (j < nh) qs[j * QW + dd] = double(elem_f32<T>(&qv[k]));
  }
  __syncthreads();  // the queries are staged (the key loads are still in flight)
#pragma unroll
  for (int k = 0; k < KPT; ++k) ks[piece_local(k) * KW + piece_col(k)] = kreg[k];
  // the wave reads only the rows it wrote: its LDS accesses are done in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int r = tid >> 2, j0 = (tid & 3) * HPT;
  if (r0 + r >= rows_b || j0 >= nh) return;  // row r + 64 i is then past the end as well
  double acc[RPT][HPT];
  const double* qrow[HPT];
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    qrow[u] = qs + min(j0 + u, nh - 1) * QW;  // slots past the group read a valid row; not stored
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc[i][u] = 0.0;
  }
#pragma unroll 2
  for (int pc = 0; pc < PPR; ++pc) {
    double kd[RPT][EPV];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const uint4 piece = ks[(r + 64 * i) * KW + pc];
      const T* e = reinterpret_cast<const T*>(&piece);
#pragma unroll
      for (int x = 0; x < EPV; ++x) kd[i][x] = double(elem_f32<T>(e + x));
    }
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
#pragma unroll
      for (int x = 0; x < EPV; x += 2) {
        const double2 q2 = *reinterpret_cast<const double2*>(qrow[u] + pc * EPV + x);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          acc[i][u] = fma(q2.x, kd[i][x], acc[i][u]);
          acc[i][u] = fma(q2.y, kd[i][x + 1], acc[i][u]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int64_t row = r0 + r + 64 * i;
    if (row < rows_b)
#pragma unroll
      for (int u = 0; u < HPT; ++u)
        if (j0 + u < nh) out[(int64_t(b) * Hq + h0 + j0 + u) * out_len + row] = acc[i][u];
  }
}

// Projected query q_p = q P (d -> 16) per head, fp64, one fma chain in index order per output. A
// bf16 or fp32 query element times an fp32 projection entry is exact in fp64, so every step rounds
// only the sum, as the sequential CPU evaluation does. One workgroup per (KV group, sequence): the
// group's projection and its heads' queries are staged in LDS with one round of coalesced loads,
// then one lane per (head, proxy dim) runs the chain. Local groups get zeros. Workgroup (0, 0)
// also clears the status words and the per-group arrival counters and publishes the step's cache
// lengths; when the token rows take the long-row path (tot_h not NULL), each workgroup clears its
// heads' coarse bin totals for the histogram pass.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_proxy_query(const T* __restrict__ q, QRows qm,
                                                     const float* __restrict__ proj, int G, int Hq,
                                                     uint64_t local_mask, double* __restrict__ qp,
                                                     uint32_t* __restrict__ status, int32_t* __restrict__ arrivals,
                                                     int n_groups, StepLens lens, unsigned long long* __restrict__ tot_h,
                                                     unsigned long long* __restrict__ tot_l, uint32_t* __restrict__ tot_c) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  if (g == 0 && b == 0) {
    if (tid < 16) status[tid] = 0;
    for (int i = tid; i < n_groups; i += 256) arrivals[i] = 0;
    lens.publish(tid, 256);
  }
  if (tot_h)
    for (int j = 0; j < G; ++j) zero_long_totals(tot_h, tot_l, tot_c, int64_t(b) * Hq + g * G + j, tid, 256);
  double* out = qp + (int64_t(b) * Hq + int64_t(g) * G) * 16;
  if ((local_mask >> g) & 1) {
    for (int o = tid; o < G * 16; o += 256) out[o] = 0.0;
    return;
  }
  __shared__ float Ps[D * 16];
  __shared__ float Qs[kMaxProxyGroup * D];
  constexpr int PPT = D * 16 / 256;  // projection entries per thread
  static_assert(PPT * 256 == D * 16, "256 threads cover the projection");
  const float* P = proj + int64_t(g) * D * 16;
  float pv[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) pv[k] = P[tid + 256 * k];
  for (int i = tid; i < G * D; i += 256) {
    const int hh = i / D;
    Qs[i] = elem_f32<T>(q + q_offset(qm, b, g * G + hh) + (i - hh * D));
  }
#pragma unroll
  for (int k = 0; k < PPT; ++k) Ps[tid + 256 * k] = pv[k];
  __syncthreads();
  for (int o = tid; o < G * 16; o += 256) {
    const int hh = o >> 4, j = o & 15;
    double acc = 0.0;
#pragma unroll 16
    for (int i = 0; i < D; ++i) acc = fma(double(Qs[hh * D + i]), double(Ps[i * 16 + j]), acc);
    out[o] = acc;
  }
}

// Proxy scores s_t = q_p . k_p[t] over the 16 proxy dims, separate multiply and add in index
// order (q_p has 53 significant bits, so the products round). q_p comes from k_proxy_query, which
// runs first in the step. One 256-thread workgroup per kMinMaxBlock tokens of one scored KV group;
// each thread takes kProxyTok tokens 256 apart, two at a time: the next pair's keys are loaded
// while the current pair is scored. A pair's keys are converted to fp64 once and scored against
// every head of the group, two heads at a time: their q_p values are the same for every lane, so
// they are read with uniform loads into scalar registers (q_p is read-only here and the outputs are
// distinct restrict pointers, which lets the compiler use scalar loads). The workgroup writes its
// max and min per head. GM bounds the group size (registers for the running max / min).
struct ProxyArgs {
  const uint16_t* kp;
  int64_t kp_sb, kp_sh, kp_st;
  int G, Hq;
  int64_t N;
  int nblk;
  StepLens lens;
  int8_t scored[kMaxKvHeads];  // blockIdx.y -> KV group
};

constexpr int kProxyThreads = 256;
constexpr int kProxyTok = kMinMaxBlock / kProxyThreads;  // tokens per thread
static_assert(kProxyTok % 2 == 0, "tokens go in pairs");

template <int GM>
__global__ __launch_bounds__(kProxyThreads) void k_score_proxy(ProxyArgs a, const double* __restrict__ qp,
                                                               double* __restrict__ s0, double* __restrict__ pmax,
                                                               double* __restrict__ pmin) {
  constexpr int NT = kProxyThreads, NW = NT / 64;
  const int b = blockIdx.z, g = a.scored[blockIdx.y], tid = threadIdx.x;
  const int G = a.G;
  __shared__ double rmax[GM][NW], rmin[GM][NW];
  const int64_t n_b = a.lens.entries(b, a.N);  // this sequence's tokens
  const int64_t t0 = int64_t(blockIdx.x) * kMinMaxBlock + tid;
  const uint16_t* kb = a.kp + b * a.kp_sb + int64_t(g) * a.kp_sh;
  const int64_t row0 = int64_t(b) * a.Hq + g * G;
  auto load_pair = [&](uint4 (&dst)[2][2], int pr) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      int64_t t = t0 + int64_t(NT) * (2 * pr + k);
      t = t < a.N ? t : a.N - 1;
      dst[k][0] = ld16(kb + t * a.kp_st);
      dst[k][1] = ld16(kb + t * a.kp_st + 8);
    }
  };
  double mx[GM], mn[GM];
#pragma unroll
  for (int j = 0; j < GM; ++j) {
    mx[j] = kNegInfD;
    mn[j] = kPosInfD;
  }
  uint4 raw[2][2][2];
  load_pair(raw[0], 0);
#pragma unroll
  for (int pr = 0; pr < kProxyTok / 2; ++pr) {
    if (pr + 1 < kProxyTok / 2) load_pair(raw[(pr + 1) & 1], pr + 1);
    double kd[2][16];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&raw[pr & 1][k][0]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        kd[k][2 * u] = double(float(__builtin_bit_cast(_Float16, uint16_t(w[u] & 0xffffu))));
        kd[k][2 * u + 1] = double(float(__builtin_bit_cast(_Float16, uint16_t(w[u] >> 16))));
      }
    }
#pragma unroll
    for (int h0 = 0; h0 < GM; h0 += 2) {
      if (h0 < G) {
        double q0[16], q1[16];
        const double* qr0 = qp + (row0 + h0) * 16;
        const double* qr1 = qp + (row0 + (h0 + 1 < G ? h0 + 1 : h0)) * 16;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          q0[u] = qr0[u];
          q1[u] = qr1[u];
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int64_t t = t0 + int64_t(NT) * (2 * pr + k);
          double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            acc0 = acc0 + q0[u] * kd[k][u];
            acc1 = acc1 + q1[u] * kd[k][u];
          }
          if (t < n_b) {
            s0[(row0 + h0) * a.N + t] = acc0;
            mx[h0] = max_f64(mx[h0], acc0);
            mn[h0] = min_f64(mn[h0], acc0);
            if (h0 + 1 < G) {
              s0[(row0 + h0 + 1) * a.N + t] = acc1;
              mx[h0 + 1] = max_f64(mx[h0 + 1], acc1);
              mn[h0 + 1] = min_f64(mn[h0 + 1], acc1);
            }
          }
        }
      }
    }
  }
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int j = 0; j < GM; ++j) {
    if (j < G) {
      const double wx = wave_max_dpp(mx[j]), wn = wave_min_dpp(mn[j]);
      if (lane == 0) {
        rmax[j][wave] = wx;
        rmin[j][wave] = wn;
      }
    }
  }
  __syncthreads();
  if (tid < G) {
    double x = rmax[tid][0], y = rmin[tid][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      x = fmax(x, rmax[tid][w]);
      y = fmin(y, rmin[tid][w]);
    }
    pmax[(row0 + tid) * a.nblk + blockIdx.x] = x;
    pmin[(row0 + tid) * a.nblk + blockIdx.x] = y;
  }
}

// Max / min of each kMinMaxBlock entries of score rows that take the long-row path on summary
// routing (8 entries per thread, loads issued first).
__global__ __launch_bounds__(256) void k_row_minmax(const double* __restrict__ s0, int64_t len, int G, int Hq,
                                                    uint64_t local_mask, double* __restrict__ pmax,
                                                    double* __restrict__ pmin, int nblk, StepLens lens) {
  const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
  if ((local_mask >> (h / G)) & 1) return;
  const int64_t len_b = lens.entries(b, len);  // entries of this sequence's rows (stride: len)
  __shared__ double rmax[4], rmin[4];
  const int64_t row = int64_t(b) * Hq + h;
  const int64_t t0 = int64_t(blockIdx.x) * kMinMaxBlock;
  double v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t t = t0 + tid + 256 * k;
    v[k] = s0[row * len + (t < len ? t : len - 1)];
  }
  double mx = kNegInfD, mn = kPosInfD;  // a block past the entries keeps the identities
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (t0 + tid + 256 * k < len_b) {
      mx = fmax(mx, v[k]);
      mn = fmin(mn, v[k]);
    }
  }
  mx = wave_max_dpp(mx);
  mn = wave_min_dpp(mn);
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

template <typename T, int D>
int score_impl(const Plan& p, const sd_tensors& t, int level, char* ws, hipStream_t st) {
  const sd_config& c = p.cfg;
  const int B = c.batch, Hq = c.n_q_heads, Hk = c.n_kv_heads;
  uint32_t* status = at<uint32_t>(ws, p.o_status);
  const QRows qm{t.q_sb, t.q_st, t.q_sh, p.G, p.Gq};
  // the step's cache lengths: read from the caller's array, published into the workspace by the
  // first kernel of the step (level 0)
  const StepLens lens{t.ctx_len, level == 0 ? at<int32_t>(ws, p.o_ctx) : nullptr, B, c.n_ctx, p.chunk_shift};
  if (c.route == SD_ROUTE_PROXY) {
    // the projected queries (this launch also clears the status words and counters and publishes
    // the step's lengths), then the proxy scores of the scored groups
    hipLaunchKernelGGL((k_proxy_query<T, D>), dim3(Hk, B), dim3(256), 0, st, static_cast<const T*>(t.q), qm,
                       t.proj, p.G, Hq, p.local_mask, at<double>(ws, p.o_qp), status,
                       at<int32_t>(ws, p.o_arrive), p.n_arrive, lens,
                       p.long0 ? at<unsigned long long>(ws, p.o_h1h) : nullptr,
                       p.long0 ? at<unsigned long long>(ws, p.o_h1l) : nullptr,
                       p.long0 ? at<uint32_t>(ws, p.o_h1c) : nullptr);
    if (p.n_scored > 0) {
      ProxyArgs pa;
      pa.kp = static_cast<const uint16_t*>(t.kp);
      pa.kp_sb = t.kp_sb;
      pa.kp_sh = t.kp_sh;
      pa.kp_st = t.kp_st;
      pa.G = p.G;
      pa.Hq = Hq;
      pa.N = c.n_ctx;
      pa.nblk = p.score_blocks0;
      pa.lens = StepLens{t.ctx_len, nullptr, B, c.n_ctx, p.chunk_shift};
      for (int i = 0; i < kMaxKvHeads; ++i) pa.scored[i] = i < p.n_scored ? p.scored[i] : 0;
      const double* qpw = at<double>(ws, p.o_qp);
      double *s0 = at<double>(ws, p.o_s0), *pmx = at<double>(ws, p.o_pmax), *pmn = at<double>(ws, p.o_pmin);
      const dim3 grid(p.score_blocks0, p.n_scored, B), blk(kProxyThreads);
      if (p.G <= 2)
        hipLaunchKernelGGL(k_score_proxy<2>, grid, blk, 0, st, pa, qpw, s0, pmx, pmn);
      else if (p.G <= 4)
        hipLaunchKernelGGL(k_score_proxy<4>, grid, blk, 0, st, pa, qpw, s0, pmx, pmn);
      else
        hipLaunchKernelGGL(k_score_proxy<kMaxProxyGroup>, grid, blk, 0, st, pa, qpw, s0, pmx, pmn);
    }
    return int(hipGetLastError());
  }
  // rows per lane: 2 when that still gives two workgroups of 128 rows per CU of a 256-CU MI355X
  auto rpt_of = [&](int64_t rows, int64_t wgs_per_row_set) {
    return (rows + 127) / 128 * wgs_per_row_set >= 512 ? 2 : 1;
  };
  if (c.mode == SD_HIER_TOPK && level == 1) {
    const int rpt = rpt_of(p.len1, int64_t(Hq) * B);
#define SD_SCORE_CAND(RPT)                                                                                     \
  hipLaunchKernelGGL((k_score_rows<T, D, 1, RPT>), dim3((p.len1 + 64 * RPT - 1) / (64 * RPT), Hq, B), dim3(256), 0, \
                     st, static_cast<const T*>(t.q), qm, static_cast<const T*>(t.kg), t.g_sb, t.g_sh, t.g_st,       \
                     at<int32_t>(ws, p.o_cand), p.len1, p.M, p.G, Hq, p.local_mask, at<double>(ws, p.o_s1), p.len1, \
                     static_cast<uint32_t*>(nullptr), static_cast<int32_t*>(nullptr), 0, lens)
    if (rpt == 2)
      SD_SCORE_CAND(2);
    else
      SD_SCORE_CAND(1);
#undef SD_SCORE_CAND
    return int(hipGetLastError());
  }
  const bool meta = c.mode == SD_HIER_TOPK;
  // query slots per lane (4 lanes per row): 1 up to 4 query rows per group, 2 up to 8, 4 up to 16
  const int hpt = p.G <= 4 ? 1 : (p.G <= 8 ? 2 : 4);
  const int rpt = rpt_of(p.len0, int64_t(Hk) * B);
  const T* keys = static_cast<const T*>(meta ? t.kmg : t.kg);
  const int64_t ksb = meta ? t.mg_sb : t.g_sb, ksh = meta ? t.mg_sh : t.g_sh, kst = meta ? t.mg_st : t.g_st;
#define SD_SCORE_ROWS(HPT, RPT)                                                                                    \
  hipLaunchKernelGGL((k_score_rows<T, D, HPT, RPT>), dim3((p.len0 + 64 * RPT - 1) / (64 * RPT), Hk, B), dim3(256), 0, \
                     st, static_cast<const T*>(t.q), qm, keys, ksb, ksh, kst, static_cast<const int32_t*>(nullptr),   \
                     p.len0, p.len0, p.G, Hq, p.local_mask, at<double>(ws, p.o_s0), p.len0, status,                   \
                     at<int32_t>(ws, p.o_arrive), p.n_arrive, lens)
  if (rpt == 2) {
    if (hpt == 1)
      SD_SCORE_ROWS(1, 2);
    else if (hpt == 2)
      SD_SCORE_ROWS(2, 2);
    else
      SD_SCORE_ROWS(4, 2);
  } else {
    if (hpt == 1)
      SD_SCORE_ROWS(1, 1);
    else if (hpt == 2)
      SD_SCORE_ROWS(2, 1);
    else
      SD_SCORE_ROWS(4, 1);
  }
#undef SD_SCORE_ROWS
  if (p.long0)
    hipLaunchKernelGGL(k_row_minmax, dim3(p.score_blocks0, Hq, B), dim3(256), 0, st, at<double>(ws, p.o_s0),
                       p.len0, p.G, Hq, p.local_mask, at<double>(ws, p.o_pmax), at<double>(ws, p.o_pmin),
                       p.score_blocks0, lens);
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

}  // namespace sd
