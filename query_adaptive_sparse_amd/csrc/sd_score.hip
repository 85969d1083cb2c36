// Score kernels: summary / meta-summary / candidate rows, proxy query and proxy scores.
//
// Compiled with -ffp-contract=off: every fused multiply-add is an explicit fma(), so fp64 score
// arithmetic can be matched bit for bit by a sequential CPU evaluation.
#include "sd_device.h"

namespace sd {
namespace {
// ---------------------------------------------------------------------------------------------
// Scores. A workgroup scores kScoreRows summary rows (or candidate rows) for the query rows
// ("slots") of one KV group: it stages the slots' queries in LDS as fp64 (exact) and the key rows
// in LDS (one coalesced pass), then 4 lanes share a row and each runs HPT slots' dot products,
// one fp64 fma per dimension in index order. A product of two bf16 or two fp32 values is exact in
// fp64, so fma(q, k, acc) equals the CPU's acc + q*k step for step. A lane converts each key
// element once for its HPT independent chains, which also hides the fma latency.
// Block (0, 0, 0) also clears the device status words and the per-group arrival counters of the
// selection.
// ---------------------------------------------------------------------------------------------
constexpr int kScoreRows = 64;

template <typename T, int D, int HPT>
__global__ __launch_bounds__(256) void k_score_rows(const T* __restrict__ q, QRows qm,
                                                    const T* __restrict__ keys, int64_t k_sb, int64_t k_sh,
                                                    int64_t k_st, const int32_t* __restrict__ cand,
                                                    int64_t n_rows, int64_t n_keys, int G, int Hq,
                                                    uint64_t local_mask, double* __restrict__ out, int64_t out_len,
                                                    uint32_t* __restrict__ status, int32_t* __restrict__ arrivals,
                                                    int n_groups) {
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
  }
  const int g = cand ? y / G : y;
  if ((local_mask >> g) & 1) return;
  const int h0 = cand ? y : y * G;
  const int nh = cand ? 1 : G;
  const int64_t r0 = int64_t(blockIdx.x) * kScoreRows;
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
  constexpr int KPT = kScoreRows * PPR / 256;
  uint4 kreg[KPT];
  const T* kbase = keys + b * k_sb + int64_t(g) * k_sh;
  auto piece_row = [&](int k) {
    const int r = (tid + 256 * k) / PPR;
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
      kreg[k] = ld16(kbase + sk * k_st + ((tid + 256 * k) % PPR) * EPV);
    }
  } else {
#pragma unroll
    for (int k = 0; k < KPT; ++k) kreg[k] = ld16(kbase + int64_t(piece_row(k)) * k_st + ((tid + 256 * k) % PPR) * EPV);
  }
  __builtin_amdgcn_sched_barrier(0);  // every key load is issued before the queries are staged
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + 256 * k, j = i / D, dd = i - j * D;
    if (j < nh) qs[j * QW + dd] = double(elem_f32<T>(&qv[k]));
  }
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = tid + 256 * k, r = i / PPR, pc = i - r * PPR;
    ks[r * KW + pc] = kreg[k];
  }
  __syncthreads();
  const int r = tid >> 2, j0 = (tid & 3) * HPT;
  const int64_t row = r0 + r;
  if (row >= n_rows || j0 >= nh) return;
  const uint4* kr = ks + r * KW;
  double acc[HPT];
  const double* qrow[HPT];
#pragma unroll
  for (int u = 0; u < HPT; ++u) {
    acc[u] = 0.0;
    qrow[u] = qs + min(j0 + u, nh - 1) * QW;  // slots past the group read a valid row; not stored
  }
#pragma unroll 2
  for (int pc = 0; pc < PPR; ++pc) {
    const uint4 piece = kr[pc];
    const T* e = reinterpret_cast<const T*>(&piece);
    double kd[EPV];
#pragma unroll
    for (int x = 0; x < EPV; ++x) kd[x] = double(elem_f32<T>(e + x));
#pragma unroll
    for (int u = 0; u < HPT; ++u) {
#pragma unroll
      for (int x = 0; x < EPV; x += 2) {
        const double2 q2 = *reinterpret_cast<const double2*>(qrow[u] + pc * EPV + x);
        acc[u] = fma(q2.x, kd[x], acc[u]);
        acc[u] = fma(q2.y, kd[x + 1], acc[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < HPT; ++u)
    if (j0 + u < nh) out[(int64_t(b) * Hq + h0 + j0 + u) * out_len + row] = acc[u];
}

// Projected query q_p = q P (d -> 16) per scored head, fp64, index order. A bf16 or fp32 query
// times an fp32 projection entry is exact in fp64.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_proxy_query(const T* __restrict__ q, QRows qm,
                                                     const float* __restrict__ proj, int G, int Hq,
                                                     uint64_t local_mask, double* __restrict__ qp,
                                                     uint32_t* __restrict__ status, int32_t* __restrict__ arrivals,
                                                     int n_groups) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && b == 0) {
    if (threadIdx.x < 16) status[threadIdx.x] = 0;
    for (int i = threadIdx.x; i < n_groups; i += 256) arrivals[i] = 0;
  }
  const int h = t >> 4, j = t & 15;
  if (h >= Hq) return;
  const int g = h / G;
  double acc = 0.0;
  if (!((local_mask >> g) & 1)) {
    const float* P = proj + int64_t(g) * D * 16;
    const T* qh = q + q_offset(qm, b, h);
    for (int i = 0; i < D; ++i) acc = fma(double(elem_f32<T>(qh + i)), double(P[i * 16 + j]), acc);
  }
  qp[(int64_t(b) * Hq + h) * 16 + j] = acc;
}

// Proxy scores s_t = q_p . k_p[t] over the 16 proxy dims, separate multiply and add in index
// order (q_p has 53 significant bits, so the products round). One 512-thread workgroup per
// kMinMaxBlock tokens of one scored KV group; each thread takes 4 tokens 512 apart, and the group's
// G heads share each token's proxy key. The workgroup projects the group's queries itself (q_p =
// q P, fp64 in index order, the same arithmetic as k_proxy_query) while the key loads are in
// flight, and writes its max and min per head.
// Workgroup (0, 0, 0) clears the status words and the per-group arrival counters.
struct ProxyArgs {
  const uint16_t* kp;
  int64_t kp_sb, kp_sh, kp_st;
  const void* q;
  QRows qm;
  const float* proj;
  int G, Hq;
  int64_t N;
  double* s0;
  double* pmax;
  double* pmin;
  int nblk;
  uint32_t* status;
  int32_t* arrivals;
  int n_groups;
  int8_t scored[kMaxKvHeads];  // blockIdx.y -> KV group
};

template <typename T, int D>
__global__ __launch_bounds__(512) void k_score_proxy(ProxyArgs a) {
  const int b = blockIdx.z, g = a.scored[blockIdx.y], tid = threadIdx.x;
  const int G = a.G;
  __shared__ double qs[kMaxProxyGroup][16];
  __shared__ double rmax[kMaxProxyGroup][8], rmin[kMaxProxyGroup][8];
  if (blockIdx.x == 0 && blockIdx.y == 0 && b == 0) {
    if (tid < 16) a.status[tid] = 0;
    for (int i = tid; i < a.n_groups; i += 512) a.arrivals[i] = 0;
  }
  // The group's projection and queries are loaded first (one unrolled round into registers, from
  // clamped rows, so every load is issued before any is used), then the tokens' proxy keys; the
  // projection is staged in LDS and q_p = q P computed (one thread per (head, proxy dim), the
  // index-order fma chain) while the key loads are still in flight.
  __shared__ float Ps[D * 16];
  __shared__ float Qs[kMaxProxyGroup][D];
  constexpr int PPT = D * 16 / 512;              // projection entries per thread
  constexpr int QPT = kMaxProxyGroup * D / 512;  // query slots per thread
  static_assert(PPT * 512 == D * 16 && QPT * 512 == kMaxProxyGroup * D, "512 threads cover P and q");
  const float* P = a.proj + int64_t(g) * D * 16;
  float pv[PPT];
  T qv[QPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) pv[k] = P[tid + 512 * k];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + 512 * k, hh = i / D, e = i - hh * D;
    qv[k] = static_cast<const T*>(a.q)[q_offset(a.qm, b, g * G + (hh < G ? hh : G - 1)) + e];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the key loads
  const int64_t t0 = int64_t(blockIdx.x) * kMinMaxBlock;
  const uint16_t* kb = a.kp + b * a.kp_sb + int64_t(g) * a.kp_sh;
  constexpr int TPT = kMinMaxBlock / 512;  // tokens per thread (512 threads)
  uint4 raw[TPT][2];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    int64_t t = t0 + tid + 512 * k;
    t = t < a.N ? t : a.N - 1;
    raw[k][0] = ld16(kb + t * a.kp_st);
    raw[k][1] = ld16(kb + t * a.kp_st + 8);
  }
  __builtin_amdgcn_sched_barrier(0);  // every key load is issued before P and q are staged
#pragma unroll
  for (int k = 0; k < PPT; ++k) Ps[tid + 512 * k] = pv[k];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + 512 * k, hh = i / D, e = i - hh * D;
    if (hh < G) Qs[hh][e] = elem_f32<T>(&qv[k]);
  }
  __syncthreads();
  if (tid < G * 16) {
    const int hh = tid >> 4, j = tid & 15;
    double acc = 0.0;
#pragma unroll 16
    for (int i = 0; i < D; ++i) acc = fma(double(Qs[hh][i]), double(Ps[i * 16 + j]), acc);
    qs[hh][j] = acc;
  }
  __syncthreads();
  double mx[kMaxProxyGroup], mn[kMaxProxyGroup];
#pragma unroll
  for (int j = 0; j < kMaxProxyGroup; ++j) {
    mx[j] = kNegInfD;
    mn[j] = kPosInfD;
  }
  const int64_t row0 = int64_t(b) * a.Hq + g * G;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int64_t t = t0 + tid + 512 * k;
    const bool valid = t < a.N;
    double kd[16];
    const _Float16* h0 = reinterpret_cast<const _Float16*>(&raw[k][0]);
    const _Float16* h1 = reinterpret_cast<const _Float16*>(&raw[k][1]);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      kd[u] = double(float(h0[u]));
      kd[u + 8] = double(float(h1[u]));
    }
#pragma unroll
    for (int j = 0; j < kMaxProxyGroup; ++j) {
      if (j < G) {
        double acc = 0.0;
#pragma unroll
        for (int u = 0; u < 16; ++u) acc = acc + qs[j][u] * kd[u];
        if (valid) {
          a.s0[(row0 + j) * a.N + t] = acc;
          mx[j] = fmax(mx[j], acc);
          mn[j] = fmin(mn[j], acc);
        }
      }
    }
  }
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int j = 0; j < kMaxProxyGroup; ++j) {
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
    for (int w = 1; w < 8; ++w) {
      x = fmax(x, rmax[tid][w]);
      y = fmin(y, rmin[tid][w]);
    }
    a.pmax[(row0 + tid) * a.nblk + blockIdx.x] = x;
    a.pmin[(row0 + tid) * a.nblk + blockIdx.x] = y;
  }
}

// Max / min of each kMinMaxBlock entries of score rows that take the long-row path on summary
// routing (8 entries per thread, loads issued first).
__global__ __launch_bounds__(256) void k_row_minmax(const double* __restrict__ s0, int64_t len, int G, int Hq,
                                                    uint64_t local_mask, double* __restrict__ pmax,
                                                    double* __restrict__ pmin, int nblk) {
  const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
  if ((local_mask >> (h / G)) & 1) return;
  __shared__ double rmax[4], rmin[4];
  const int64_t row = int64_t(b) * Hq + h;
  const int64_t t0 = int64_t(blockIdx.x) * kMinMaxBlock;
  double v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t t = t0 + tid + 256 * k;
    v[k] = s0[row * len + (t < len ? t : len - 1)];
  }
  double mx = kNegInfD, mn = kPosInfD;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (t0 + tid + 256 * k < len) {
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
  if (c.route == SD_ROUTE_PROXY) {
    if (p.n_scored == 0) {  // every group is local: only the status words and counters need clearing
      const int nb = (Hq * 16 + 255) / 256;
      hipLaunchKernelGGL((k_proxy_query<T, D>), dim3(nb, B), dim3(256), 0, st, static_cast<const T*>(t.q), qm,
                         t.proj, p.G, Hq, p.local_mask, at<double>(ws, p.o_qp), status,
                         at<int32_t>(ws, p.o_arrive), p.n_arrive);
    } else {
      ProxyArgs pa;
      pa.kp = static_cast<const uint16_t*>(t.kp);
      pa.kp_sb = t.kp_sb;
      pa.kp_sh = t.kp_sh;
      pa.kp_st = t.kp_st;
      pa.q = t.q;
      pa.qm = qm;
      pa.proj = t.proj;
      pa.G = p.G;
      pa.Hq = Hq;
      pa.N = c.n_ctx;
      pa.s0 = at<double>(ws, p.o_s0);
      pa.pmax = at<double>(ws, p.o_pmax);
      pa.pmin = at<double>(ws, p.o_pmin);
      pa.nblk = p.score_blocks0;
      pa.status = status;
      pa.arrivals = at<int32_t>(ws, p.o_arrive);
      pa.n_groups = p.n_arrive;
      for (int i = 0; i < kMaxKvHeads; ++i) pa.scored[i] = i < p.n_scored ? p.scored[i] : 0;
      hipLaunchKernelGGL((k_score_proxy<T, D>), dim3(p.score_blocks0, p.n_scored, B), dim3(512), 0, st, pa);
    }
    return int(hipGetLastError());
  }
  if (c.mode == SD_HIER_TOPK && level == 1) {
    hipLaunchKernelGGL((k_score_rows<T, D, 1>), dim3((p.len1 + kScoreRows - 1) / kScoreRows, Hq, B), dim3(256), 0, st,
                       static_cast<const T*>(t.q), qm, static_cast<const T*>(t.kg), t.g_sb, t.g_sh,
                       t.g_st, at<int32_t>(ws, p.o_cand), p.len1, p.M, p.G, Hq, p.local_mask, at<double>(ws, p.o_s1),
                       p.len1, static_cast<uint32_t*>(nullptr), static_cast<int32_t*>(nullptr), 0);
    return int(hipGetLastError());
  }
  const bool meta = c.mode == SD_HIER_TOPK;
  // query slots per lane (4 lanes per row): 1 up to 4 query rows per group, 2 up to 8, 4 up to 16
  const int hpt = p.G <= 4 ? 1 : (p.G <= 8 ? 2 : 4);
  const dim3 grid((p.len0 + kScoreRows - 1) / kScoreRows, Hk, B);
  const T* keys = static_cast<const T*>(meta ? t.kmg : t.kg);
  const int64_t ksb = meta ? t.mg_sb : t.g_sb, ksh = meta ? t.mg_sh : t.g_sh, kst = meta ? t.mg_st : t.g_st;
#define SD_SCORE_ROWS(HPT)                                                                                       \
  hipLaunchKernelGGL((k_score_rows<T, D, HPT>), grid, dim3(256), 0, st, static_cast<const T*>(t.q), qm, keys, ksb, \
                     ksh, kst, static_cast<const int32_t*>(nullptr), p.len0, p.len0, p.G, Hq, p.local_mask,          \
                     at<double>(ws, p.o_s0), p.len0, status, at<int32_t>(ws, p.o_arrive), p.n_arrive)
  if (hpt == 1)
    SD_SCORE_ROWS(1);
  else if (hpt == 2)
    SD_SCORE_ROWS(2);
  else
    SD_SCORE_ROWS(4);
#undef SD_SCORE_ROWS
  if (p.long0)
    hipLaunchKernelGGL(k_row_minmax, dim3(p.score_blocks0, Hq, B), dim3(256), 0, st, at<double>(ws, p.o_s0),
                       p.len0, p.G, Hq, p.local_mask, at<double>(ws, p.o_pmax), at<double>(ws, p.o_pmin),
                       p.score_blocks0);
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
