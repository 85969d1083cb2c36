// Token-Sparse prefill: dynamic token coverage selection, then compressed causal attention over
// each head's kept tokens, scattered back into the sequence-length output.
//
// Selection (fp64, matching a sequential CPU evaluation up to the order of the softmax sums):
//   k_pf_scores      proxy scores s[key][q] = q . k of the W window queries against 4 blocks of 64
//                    keys per workgroup (the next block's keys load during a block's MFMAs), on
//                    the fp64 MFMA (16 keys x 16 queries x 4 dimensions per instruction; chained
//                    over the dimensions in index order, each output is the sequential fma chain
//                    of the dot product); per key block and query, the max m_b over the visible
//                    keys and z_b, the sum of exp(scale (s - m_b)) over them;
//   k_pf_rowmax      every window query's max over its visible keys;
//   k_pf_zslab       per 2048-key slab and query, the sum over the slab's blocks, in order, of
//                    z_b exp(scale (m_b - max)): the slab's sum of exp(scale (s - max));
//   k_pf_importance  per key, the sum over the window queries (in order) of the query's softmax
//                    probability of that key, and the slab's max / min of it;
//   k_pf_global      per key, the sparse heads' importances summed in head order;
//   long-row pass    top-p of the global importance with the values as masses, p = 1 - tau;
//   k_pf_budget      budget = (that count) - 1, at least 1: the tokens left after cutting the
//                    ascending tail whose mass exceeds tau of the total;
//   long-row pass    every head's top-budget tokens by its own importance;
//   k_pf_lists       each head's bitmap as an ascending position list (a full-attention head:
//                    every position).
// Attention:
//   k_pf_vmax        each KV head's max |v| (per slab);
//   k_pf_gather      compression: every head's K and V rows at its kept positions, in list order,
//                    into contiguous per-head sequences (padded with zero rows to a whole step), V
//                    converted to fp16 under the head's power-of-two scale;
//   k_pf_attend      128 compact queries per workgroup (32 per wave), heaviest blocks first; the
//                    workgroup stages 64 gathered keys' K and V rows per step in LDS (K pieces
//                    XOR-swizzled per row, V rows padded for transpose reads), each wave runs q.K^T
//                    on the bf16 MFMA, the causal mask in compact order, an online softmax whose
//                    reference moves only when a logit exceeds it by 2^8, and P.V on the fp16
//                    MFMA (P rounded to fp16 and the normaliser summed from the same rounded
//                    values, V converted at the gather), then writes its rows;
//                    the workgroups past a head's query blocks write the zero rows of the
//                    positions it did not keep.
#include "sd_device.h"
#include "sp_internal.h"
#include "sd_exp.h"

namespace sd {
namespace {

using f64x4 = __attribute__((ext_vector_type(4))) double;

// ---------------------------------------------------------------------------------------------
// Proxy scores on the fp64 MFMA. Layout of v_mfma_f64_16x16x4f64 (lane l): A element
// [row l % 16][k l / 16], B element [k l / 16][col l % 16], accumulator element v at
// [row l / 16 + 4 v][col l % 16]. Rows are keys, columns window queries, k the dimensions.
// ---------------------------------------------------------------------------------------------
struct PfScoreArgs {
  const uint16_t* q;
  int64_t q_sb, q_sh, q_st;
  const uint16_t* k;
  int64_t kv_sb, kv_sh, kv_st;
  int64_t L;
  int W, Hq, G, nkb;
  double* S;       // [B][Hq][L][W] scores, key-major
  double* pmq;     // [B][Hq][nkb][W] each query's max over the block's visible keys
  double* zb;      // [B][Hq][nkb][W] each query's sum of exp(scale (s - that max)) over them
  double scale;
  uint32_t* status;
};

constexpr int kD = 128;
constexpr int kKRow = kD + 8;  // padded bf16 row in LDS (elements)

// 2^(j/64) for exp_nonpos, copied into LDS by the kernels that use it
__constant__ double kExp2Tab[64] = {SD_EXP2_64_TABLE};
__device__ __forceinline__ void load_exp_table(double* etab, int tid, int nt) {
  for (int i = tid; i < 64; i += nt) etab[i] = kExp2Tab[i];
}

constexpr int kPfScoreBlocks = 4;  // key blocks per proxy-score workgroup (the window queries load once)

__global__ __launch_bounds__(256) void k_pf_scores(PfScoreArgs a) {
  __shared__ uint16_t qs[kPfMaxWindow * kKRow];
  __shared__ uint16_t ks[kPfKeyBlock * kKRow];
  __shared__ double wmax[4][kPfMaxWindow], wz[4][kPfMaxWindow];
  __shared__ double etab[64];
  load_exp_table(etab, threadIdx.x, 256);  // read after the loop's first barrier
  const ExpC ec = exp_consts();
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, n = lane & 15, c = lane >> 4;
  if (a.status && blockIdx.x == 0 && h == 0 && b == 0 && tid < 16) a.status[tid] = 0;
  const int g = h / a.G;
  const int64_t qpos0 = a.L - a.W;
  const int kbA = blockIdx.x * kPfScoreBlocks;
  const int kbB = kbA + kPfScoreBlocks < a.nkb ? kbA + kPfScoreBlocks : a.nkb;
  // window queries (rows past W are zero) -> LDS, once
  for (int i = tid; i < kPfMaxWindow * (kD / 8); i += 256) {
    const int r = i / (kD / 8), pc = i - r * (kD / 8);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < a.W) v = ld16(a.q + b * a.q_sb + h * a.q_sh + (qpos0 + r) * a.q_st + pc * 8);
    *reinterpret_cast<uint4*>(qs + r * kKRow + pc * 8) = v;
  }
  // a key block's rows (past L: the last key), 4 pieces per thread: registers, then LDS
  constexpr int kKPer = kPfKeyBlock * (kD / 8) / 256;
  uint4 rk[kKPer];
  auto load = [&](int kb) {
#pragma unroll
    for (int u = 0; u < kKPer; ++u) {
      const int i = tid + 256 * u, r = i / (kD / 8), pc = i - r * (kD / 8);
      const int64_t key0 = int64_t(kb) * kPfKeyBlock;
      const int64_t key = key0 + r < a.L ? key0 + r : a.L - 1;
      rk[u] = ld16(a.k + b * a.kv_sb + g * a.kv_sh + key * a.kv_st + pc * 8);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < kKPer; ++u) {
      const int i = tid + 256 * u, r = i / (kD / 8), pc = i - r * (kD / 8);
      *reinterpret_cast<uint4*>(ks + r * kKRow + pc * 8) = rk[u];
    }
  };
  load(kbA);
  store();
  for (int kb = kbA; kb < kbB; ++kb) {
    __syncthreads();  // the block's keys (and the queries) are in LDS
    if (kb + 1 < kbB) load(kb + 1);  // in flight during the block's MFMAs
    const int64_t key0 = int64_t(kb) * kPfKeyBlock;
    // wave: keys 16 wave .. + 15 of the block against the 4 query tiles
    f64x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};
    const uint16_t* kr = ks + (16 * wave + n) * kKRow + c;
#pragma unroll 4
    for (int s = 0; s < kD / 4; ++s) {
      const double av = double(bf2f(kr[4 * s]));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const double bv = double(bf2f(qs[(16 * t + n) * kKRow + 4 * s + c]));
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[t], 0, 0, 0);
      }
    }
    // scores out (key-major, W per key) and each query's max over the visible keys of the wave
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int qi = 16 * t + n;
      double m = kNegInfD;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t key = key0 + 16 * wave + c + 4 * v;
        if (key < a.L && qi < a.W) {
          a.S[((int64_t(b) * a.Hq + h) * a.L + key) * a.W + qi] = acc[t][v];
          if (key <= qpos0 + qi) m = fmax(m, acc[t][v]);
        }
      }
      m = fmax(m, __shfl_xor(m, 16));
      m = fmax(m, __shfl_xor(m, 32));
      if (c == 0) wmax[wave][qi] = m;
    }
    __syncthreads();  // every wave is done with ks and has its maxima in wmax
    // each query's block max m (the waves' maxima), then its sum over the wave's visible keys of
    // exp(scale s - scale m): keys c, c + 4, c + 8, c + 12 of the lane, then the lane groups
    // (the same sum in every lane), then the waves in order
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int qi = 16 * t + n;
      const double sm = a.scale * fmax(fmax(wmax[0][qi], wmax[1][qi]), fmax(wmax[2][qi], wmax[3][qi]));
      double z = 0.0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t key = key0 + 16 * wave + c + 4 * v;
        if (key < a.L && qi < a.W && key <= qpos0 + qi) z += exp_nonpos(a.scale * acc[t][v] - sm, etab, ec);
      }
      z += __shfl_xor(z, 16);
      z += __shfl_xor(z, 32);
      if (c == 0) wz[wave][qi] = z;
    }
    if (kb + 1 < kbB) store();
    __syncthreads();  // every wave's sums are in wz
    if (tid < a.W) {
      const int64_t o = ((int64_t(b) * a.Hq + h) * a.nkb + kb) * a.W + tid;
      a.pmq[o] = fmax(fmax(wmax[0][tid], wmax[1][tid]), fmax(wmax[2][tid], wmax[3][tid]));
      a.zb[o] = ((wz[0][tid] + wz[1][tid]) + wz[2][tid]) + wz[3][tid];
    }
  }
}

// Every window query's max over its visible keys: the block maxima, 16 parts of the blocks per
// query with 8 loads in flight per thread (max is exact, so the order does not matter).
__global__ __launch_bounds__(1024) void k_pf_rowmax(const double* __restrict__ pmq, int nkb, int W, double* __restrict__ M) {
  const int h = blockIdx.x, b = blockIdx.y, Hq = gridDim.x, tid = threadIdx.x;
  __shared__ double red[16][kPfMaxWindow];
  const int qi = tid & 63, part = tid >> 6;
  double m = kNegInfD;
  if (qi < W) {
    const double* pq = pmq + (int64_t(b) * Hq + h) * nkb * W + qi;
    int kb = part;
    for (; kb + 16 * 7 < nkb; kb += 16 * 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pq[int64_t(kb + 16 * u) * W];
#pragma unroll
      for (int u = 0; u < 8; ++u) m = fmax(m, v[u]);
    }
    for (; kb < nkb; kb += 16) m = fmax(m, pq[int64_t(kb) * W]);
  }
  red[part][qi] = m;
  __syncthreads();
  if (tid < W) {
    double r = red[0][tid];
    for (int p = 1; p < 16; ++p) r = fmax(r, red[p][tid]);
    M[(int64_t(b) * Hq + h) * W + tid] = r;
  }
}

struct PfImpArgs {
  const double* S;
  const double* M;   // [B][Hq][W]
  double* zq;        // [B][Hq][nslab][W]
  double* imp;       // [B][Hq][L]
  double* pmax;      // [B][Hq][nslab]
  double* pmin;
  int64_t L;
  int W, Hq, nslab;
  double scale;
};

// Per slab and window query: the sum over the slab's key blocks, in order, of
// z_b exp(scale m_b - scale max), z_b the block's sum of exp(scale s - scale m_b) over the query's
// visible keys and m_b their max (a block with none has z_b = 0 and m_b = -inf and adds 0). Each
// term is the block's sum of exp(scale s - scale max) up to the rounding of the two factors.
__global__ __launch_bounds__(kPfMaxWindow) void k_pf_zslab(PfImpArgs a, const double* __restrict__ pmq,
                                                           const double* __restrict__ zb, int nkb) {
  constexpr int kBlocks = kPfSlab / kPfKeyBlock;  // key blocks per slab
  static_assert(kPfSlab % kPfKeyBlock == 0, "slabs are whole key blocks");
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z, qi = threadIdx.x;
  __shared__ double etab[64];
  load_exp_table(etab, qi, kPfMaxWindow);
  __syncthreads();
  if (qi >= a.W) return;
  const ExpC ec = exp_consts();
  const int64_t row = int64_t(b) * a.Hq + h;
  const double mq = a.scale * a.M[row * a.W + qi];
  const int kb0 = sl * kBlocks;
  double zv[kBlocks], mv[kBlocks];
#pragma unroll
  for (int u = 0; u < kBlocks; ++u) {
    const int kb = kb0 + u < nkb ? kb0 + u : nkb - 1;
    zv[u] = zb[(row * nkb + kb) * a.W + qi];
    mv[u] = pmq[(row * nkb + kb) * a.W + qi];
  }
  double z = 0.0;
#pragma unroll
  for (int u = 0; u < kBlocks; ++u)
    if (kb0 + u < nkb && zv[u] > 0.0) z += zv[u] * exp_nonpos(a.scale * mv[u] - mq, etab, ec);
  a.zq[(row * a.nslab + sl) * a.W + qi] = z;
}

// Per key of the slab: importance = sum over the window queries, in order, of
// exp(scale s - scale max_q) x (1 / Z_q) (Z_q: the slab partials summed in slab order; the product
// with the reciprocal is within an ulp of the quotient); and the slab's max / min of the importance.
__global__ __launch_bounds__(256) void k_pf_importance(PfImpArgs a) {
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ double zs[kPfMaxWindow], ms[kPfMaxWindow];  // 1 / Z_q, scale x max_q
  __shared__ double rmax[4], rmin[4];
  __shared__ double etab[64];
  load_exp_table(etab, tid, 256);
  const ExpC ec = exp_consts();
  const int64_t row = int64_t(b) * a.Hq + h;
  if (tid < a.W) {
    double z = 0.0;
    for (int s = 0; s < a.nslab; ++s) z += a.zq[(row * a.nslab + s) * a.W + tid];
    zs[tid] = 1.0 / z;
    ms[tid] = a.scale * a.M[row * a.W + tid];
  }
  __syncthreads();
  const int64_t j0 = int64_t(sl) * kPfSlab, j1 = j0 + kPfSlab < a.L ? j0 + kPfSlab : a.L;
  double mx = kNegInfD, mn = kPosInfD;
  for (int64_t j = j0 + tid; j < j1; j += 256) {
    const double* sp = a.S + (row * a.L + j) * a.W;
    const int64_t q0 = j - (a.L - a.W);  // first window query that sees key j
    const int qa = q0 > 0 ? int(q0) : 0;
    double v = 0.0;
    if (qa == 0 && (a.W & 7) == 0) {
      // every query sees the key: 8 scores per step, loaded together
      for (int q8 = 0; q8 < a.W; q8 += 8) {
        double sv[8];
#pragma unroll
        for (int u = 0; u < 8; u += 2) {
          const double2 d2 = *reinterpret_cast<const double2*>(sp + q8 + u);
          sv[u] = d2.x;
          sv[u + 1] = d2.y;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) v += exp_nonpos(a.scale * sv[u] - ms[q8 + u], etab, ec) * zs[q8 + u];
      }
    } else {
      for (int qi = qa; qi < a.W; ++qi) v += exp_nonpos(a.scale * sp[qi] - ms[qi], etab, ec) * zs[qi];
    }
    a.imp[row * a.L + j] = v;
    mx = fmax(mx, v);
    mn = fmin(mn, v);
  }
  mx = wave_max_dpp(mx);
  mn = wave_min_dpp(mn);
  if (lane == 0) {
    rmax[wave] = mx;
    rmin[wave] = mn;
  }
  __syncthreads();
  if (tid == 0) {
    a.pmax[row * a.nslab + sl] = fmax(fmax(rmax[0], rmax[1]), fmax(rmax[2], rmax[3]));
    a.pmin[row * a.nslab + sl] = fmin(fmin(rmin[0], rmin[1]), fmin(rmin[2], rmin[3]));
  }
}

// Per key: the heads' importances summed in head order; and the slab's max / min.
__global__ __launch_bounds__(256) void k_pf_global(const double* __restrict__ imp, const int8_t* __restrict__ mode,
                                                   int Hq, int64_t L, int nslab, double* __restrict__ gimp,
                                                   double* __restrict__ gpmax, double* __restrict__ gpmin) {
  const int sl = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ double rmax[4], rmin[4];
  const int64_t j0 = int64_t(sl) * kPfSlab, j1 = j0 + kPfSlab < L ? j0 + kPfSlab : L;
  double mx = kNegInfD, mn = kPosInfD;
  for (int64_t j = j0 + tid; j < j1; j += 256) {
    double v = 0.0;
    for (int h = 0; h < Hq; ++h)
      if (!mode || !mode[h]) v += imp[(int64_t(b) * Hq + h) * L + j];  // sparse heads only
    gimp[int64_t(b) * L + j] = v;
    mx = fmax(mx, v);
    mn = fmin(mn, v);
  }
  mx = wave_max_dpp(mx);
  mn = wave_min_dpp(mn);
  if (lane == 0) {
    rmax[wave] = mx;
    rmin[wave] = mn;
  }
  __syncthreads();
  if (tid == 0) {
    gpmax[int64_t(b) * nslab + sl] = fmax(fmax(rmax[0], rmax[1]), fmax(rmax[2], rmax[3]));
    gpmin[int64_t(b) * nslab + sl] = fmin(fmin(rmin[0], rmin[1]), fmin(rmin[2], rmin[3]));
  }
}

// budget[b] = max(1, |top-p set of the global importance| - 1).
__global__ __launch_bounds__(1024) void k_pf_budget(const uint32_t* __restrict__ bbits, int64_t words,
                                                    int32_t* __restrict__ budget) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int red[16];
  int cnt = 0;
  for (int64_t w = tid; w < words; w += 1024) cnt += __popc(bbits[int64_t(b) * words + w]);
  cnt = wave_sum_i32_dpp(cnt);
  if (lane == 0) red[wave] = cnt;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < 16; ++w) t += red[w];
    budget[b] = t - 1 > 1 ? t - 1 : 1;
  }
}

// Each head's bitmap as an ascending position list (one workgroup per head).
__global__ __launch_bounds__(1024) void k_pf_lists(uint32_t* __restrict__ bits, const int8_t* __restrict__ mode,
                                                   int64_t words, int64_t L, int32_t* __restrict__ list) {
  const int h = blockIdx.x, b = blockIdx.y, Hq = gridDim.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int wtot[16];
  const int64_t row = int64_t(b) * Hq + h;
  uint32_t* bw = bits + row * words;
  int32_t* out = list + row * L;
  if (mode && mode[h]) {
    // a full-attention head keeps every position
    for (int64_t w = tid; w < words; w += 1024) {
      const int64_t left = L - w * 32;
      bw[w] = left >= 32 ? 0xffffffffu : (1u << left) - 1u;
    }
    for (int64_t j = tid; j < L; j += 1024) out[j] = int32_t(j);
    return;
  }
  const int64_t per = (words + 1023) / 1024;
  const int64_t w0 = tid * per, w1 = w0 + per < words ? w0 + per : words;
  int pc = 0;
  for (int64_t w = w0; w < w1; ++w) pc += __popc(bw[w]);
  const int incl = wave_scan_i32_dpp(pc, lane);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int pos = incl - pc;
  for (int w = 0; w < wave; ++w) pos += wtot[w];
  for (int64_t w = w0; w < w1; ++w) {
    uint32_t m = bw[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      out[pos++] = int32_t(w * 32 + bit);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Compressed causal attention. A workgroup owns 128 compact queries (wave w: queries
// 128 qb + 32 w + 16 t + n for its two query tiles t); per step it stages 64 compact keys' K and V
// rows in LDS and every wave computes its 32 x 64 logits (each K fragment read serves both query
// tiles), one online-softmax update per tile and step, and P.V (each V operand read serves both
// query tiles and both halves of P).
// ---------------------------------------------------------------------------------------------
struct PfAttnArgs {
  const uint16_t* q;
  int64_t q_sb, q_sh, q_st;
  const uint16_t* k;
  const uint16_t* v;
  int64_t kv_sb, kv_sh, kv_st;
  const int32_t* list;    // [B][Hq][L]
  const int32_t* budget;  // [B]
  const int8_t* mode;     // [Hq] 1 = full-attention head (keeps every position), or null
  uint16_t* kc;           // gathered K rows [B][Hq][Lpad][d], bf16
  uint16_t* vc;           // gathered V rows [B][Hq][Lpad][d], fp16 scaled by 2^-vexp[b][h]
  float* vmaxp;           // [B][Hkv][nslab] max |v| per slab
  int32_t* vexp;          // [B][Hq]
  int nslab, Hkv;
  const uint32_t* bits;   // kept positions [B][Hq][words]
  int64_t words;
  float* out;             // [B][Hq][L][d]
  int64_t L, Lpad;
  int Hq, G;
  float scale_log2;
};

// max |v| over a slab of kPfSlab rows of one KV head (one workgroup per slab).
__global__ __launch_bounds__(256) void k_pf_vmax(PfAttnArgs a) {
  const int sl = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  __shared__ float red[4];
  const int64_t j0 = int64_t(sl) * kPfSlab, j1 = j0 + kPfSlab < a.L ? j0 + kPfSlab : a.L;
  const uint16_t* vb = a.v + b * a.kv_sb + g * a.kv_sh;
  uint32_t mx = 0;  // |v| as bits: monotone for nonnegative floats
  for (int64_t i = j0 * (kD / 8) + tid; i < j1 * (kD / 8); i += 256) {
    const int64_t r = i / (kD / 8), pc = i - r * (kD / 8);
    const uint4 w = ld16_stream(vb + r * a.kv_st + pc * 8);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) mx = max(mx, max((u[k] << 16) & 0x7fff0000u, u[k] & 0x7fff0000u));
  }
#pragma unroll
  for (int o = 32; o; o >>= 1) mx = max(mx, uint32_t(__shfl_xor(int(mx), o)));
  if ((tid & 63) == 0) red[tid >> 6] = __uint_as_float(mx);
  __syncthreads();
  if (tid == 0) a.vmaxp[(int64_t(b) * a.Hkv + g) * a.nslab + sl] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Compression: every head's K and V rows at its kept positions, in list order, into contiguous
// per-head sequences; rows from the budget up to the next multiple of kPfKeyTile are zero (their
// logits are masked, and zero values keep their products finite). K stays bf16; V becomes fp16
// scaled by 2^-e with e = (exponent of the KV head's max |v|) - 15, so the largest value lands in
// [2^14, 2^15): every bf16 value of magnitude down to 2^-29 of the max converts exactly, smaller ones
// round to the fp16 grid (absolute error below 2^-39 of the max). One workgroup per 64 rows.
__device__ __forceinline__ int pf_vexp(const PfAttnArgs& a, int b, int g) {
  const float* vm = a.vmaxp + (int64_t(b) * a.Hkv + g) * a.nslab;
  float m = 0.f;
  for (int s = 0; s < a.nslab; ++s) m = fmaxf(m, vm[s]);
  int e = 0;
  if (m > 0.f && m <= 3.4028235e38f) {  // every finite max (inputs are finite)
    frexpf(m, &e);  // m = f 2^e, f in [0.5, 1)
    e -= 15;
    // 2^-e and 2^e stay finite fp32 values: a head whose max |v| is below 2^-111 is scaled by
    // 2^126 only (its values then fill less of the fp16 range; each keeps an absolute error of
    // at most 2^-151)
    e = e > -126 ? e : -126;
  }
  return e;
}

__global__ __launch_bounds__(256) void k_pf_gather(PfAttnArgs a) {
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int Li = int(a.L);
  const int kk = a.mode && a.mode[h] ? Li : min(max(a.budget[b], 1), Li);
  const int r0 = blockIdx.x * kPfKeyTile;
  if (r0 >= kk) return;
  const int g = h / a.G;
  const int32_t* lst = a.list + (int64_t(b) * a.Hq + h) * a.L;
  const int64_t head = (int64_t(b) * a.Hq + h) * a.Lpad;
  const int pc = tid & 15;
  uint4 kv[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + (tid >> 4) + 16 * i;
    if (r < kk) {
      const int64_t pos = min(max(lst[r], 0), Li - 1);
      const int64_t src = b * a.kv_sb + g * a.kv_sh + pos * a.kv_st + pc * 8;
      kv[0][i] = ld16_stream(a.k + src);
      kv[1][i] = ld16_stream(a.v + src);
    } else {
      kv[0][i] = kv[1][i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const int e = pf_vexp(a, b, g);
  if (blockIdx.x == 0 && tid == 0) a.vexp[int64_t(b) * a.Hq + h] = e;
  const float sc = ldexpf(1.f, -e);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t dst = (head + r0 + (tid >> 4) + 16 * i) * kD + pc * 8;
    *reinterpret_cast<uint4*>(a.kc + dst) = kv[0][i];
    const uint32_t u[4] = {kv[1][i].x, kv[1][i].y, kv[1][i].z, kv[1][i].w};
    uint32_t hw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      h2 hv;
      hv[0] = (_Float16)(__uint_as_float(u[k] << 16) * sc);
      hv[1] = (_Float16)(__uint_as_float(u[k] & 0xffff0000u) * sc);
      hw[k] = __builtin_bit_cast(uint32_t, hv);
    }
    *reinterpret_cast<uint4*>(a.vc + dst) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  }
}

constexpr int kPPR = kD / 8;   // 16-byte pieces per row
constexpr int kKeyTile = kPfKeyTile;  // compact keys staged per step
constexpr int kQTiles = 2;     // 16-query tiles per wave
constexpr float kPfLazy = 8.f; // log2 headroom of the lazily moved softmax reference
// V rows are staged as they are (key-major), pitch 72 words: the B operand of P.V (4 consecutive
// keys of one dimension) is one LDS transpose read. ds_read_b64_tr_b16 works on groups of 16
// lanes: lane i of a group receives element i % 4 of the 8 bytes addressed by the group's lanes
// i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12. So lane j of group c addresses key 4 c + j / 4 of the
// sub-tile, dimensions 16 nb + 4 (j % 4) .. + 3, and lane n then holds V[4 c + 0..3][16 nb + n].
// With a pitch of 8 (mod 64) words the 16 addresses of a group, and those of its neighbour group,
// fall in distinct banks.
constexpr int kVPitchW = kD / 2 + 8;  // 32-bit words per staged V row

__device__ __forceinline__ int pf_kswz(int x) { return x & 15; }

constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfPieces = kKeyTile * kPPR / kPfThreads;  // 16-byte K (and V) pieces per thread per step
static_assert(kPfPieces * kPfThreads == kKeyTile * kPPR, "the threads cover a step's pieces");

__global__ __launch_bounds__(kPfThreads, 2) void k_pf_attend(PfAttnArgs a) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  __shared__ uint4 kstb[2][kKeyTile * kPPR];
  __shared__ uint32_t vstb[2][kKeyTile * kVPitchW];
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, n = lane & 15, c = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Li = int(a.L);
  const int kk = a.mode && a.mode[h] ? Li : min(max(a.budget[b], 1), Li);
  const int nqb = (kk + kPfQueryBlock - 1) / kPfQueryBlock;
  if (int(blockIdx.x) >= nqb) {
    // decompression: the workgroups past the head's query blocks (at least one per head, by the
    // launch) write the zero rows of the positions the head did not keep, kZr rows of 32 x 16
    // bytes at a time, 8 times per pass, while the attention blocks run
    constexpr int kZr = kPfThreads / 32;
    const int nz = int(gridDim.x) - nqb, z = int(blockIdx.x) - nqb;
    const int per = ((Li + nz - 1) / nz + 7) & ~7;
    const int j1 = min(Li, (z + 1) * per);
    const uint32_t* hb = a.bits + (int64_t(b) * a.Hq + h) * a.words;
    float* ob = a.out + (int64_t(b) * a.Hq + h) * a.L * kD + (tid & 31) * 4;
    typedef float f4v __attribute__((ext_vector_type(4)));
    for (int j0 = z * per + (tid >> 5); j0 < j1; j0 += 8 * kZr) {
      uint32_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + kZr * u;
        const uint32_t wj = hb[min(j, j1 - 1) >> 5] >> (j & 31);  // j0 < j1: an in-range word
        w[u] = j < j1 ? wj : 1u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (!(w[u] & 1u))
          __builtin_nontemporal_store(f4v{0.f, 0.f, 0.f, 0.f},
                                      reinterpret_cast<f4v*>(ob + int64_t(j0 + kZr * u) * kD));
    }
    return;
  }
  const int qb = nqb - 1 - int(blockIdx.x);  // heaviest (longest causal range) first
  const int32_t* lst = a.list + (int64_t(b) * a.Hq + h) * a.L;
  // list entries are positions in [0, L); clamped so that no list entry can ever address outside
  // the tensors
  auto pos_of = [&](int i) { return int64_t(min(max(lst[i], 0), Li - 1)); };
  const int q0w = qb * kPfQueryBlock + 32 * wave;  // first query of this wave
  // query fragments (B operand of q.K^T: query n, dimensions 32 j + 8 c .. + 7) per query tile
  uint4 qf[kQTiles][kD / 32];
#pragma unroll
  for (int t = 0; t < kQTiles; ++t) {
    const int qi = q0w + 16 * t + n;
    const int64_t qrow = pos_of(qi < kk ? qi : kk - 1);
#pragma unroll
    for (int j = 0; j < kD / 32; ++j) qf[t][j] = ld16(a.q + b * a.q_sb + h * a.q_sh + qrow * a.q_st + 32 * j + 8 * c);
  }
  // running reference of every query column in log2 units (scale_log2 x raw logit); it is moved
  // only when a logit exceeds it by more than kPfLazy, so the probabilities stay below 2^kPfLazy
  // the normaliser of query row 4 c + i of tile t sits in accl[t][i] of every lane of group c: it
  // is a P.V product against a block of ones, so it sums exactly the fp16 weights that multiply V
  float m[kQTiles];
  f32x4 accl[kQTiles];
  f32x4 acc[kQTiles][kD / 16];
#pragma unroll
  for (int t = 0; t < kQTiles; ++t) {
    m[t] = kNegInf;
    accl[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < kD / 16; ++nb) acc[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // keys of step kt: gathered rows kKeyTile kt + x; thread pieces tid + kPfThreads i (row x =
  // tid / 16 + (kPfThreads / 16) i, 16-byte piece pc = tid % 16 of it). LDS holds steps kt (being computed) and kt + 1
  // (written at the start of step kt); one register stage holds the loads of step kt + 2 in flight
  // for a whole step. One barrier per step.
  const int pc = tid & 15, x0 = tid >> 4;
  const int64_t head = (int64_t(b) * a.Hq + h) * a.Lpad * kD;
  const uint16_t* kthr = a.kc + head + x0 * kD + pc * 8;
  const uint16_t* vthr = a.vc + head + x0 * kD + pc * 8;
  constexpr int kRowStep = kPfThreads / 16;
  uint4 rk[kPfPieces], rv[kPfPieces];
  auto stage = [&](int sbuf) {
#pragma unroll
    for (int i = 0; i < kPfPieces; ++i) {
      const int x = x0 + kRowStep * i;
      kstb[sbuf][x * kPPR + (pc ^ pf_kswz(x))] = rk[i];
      *reinterpret_cast<uint4*>(vstb[sbuf] + x * kVPitchW + pc * 4) = rv[i];
    }
  };
  const int nkt = (min(kk, (qb + 1) * kPfQueryBlock) + kKeyTile - 1) / kKeyTile;  // causal key tiles
  auto issue = [&](int kt) {
    kt = kt < nkt ? kt : nkt - 1;  // past the end: the last step again (still cached)
    const int64_t o = int64_t(kt) * kKeyTile * kD;
#pragma unroll
    for (int i = 0; i < kPfPieces; ++i) {
      rk[i] = ld16(kthr + o + kRowStep * i * kD);
      rv[i] = ld16(vthr + o + kRowStep * i * kD);
    }
  };
  issue(0);
  stage(0);
  issue(1);
  // let step 1's loads land before the loop: the loop head then sees only the loads in flight at
  // its back edge, and waits for none of them before the barrier
  __builtin_amdgcn_s_waitcnt(0);
  const float cs = a.scale_log2;
  // one step; sb = kt % 2 is a constant at each call site
  auto step = [&](const int sb, const int kt) {
    // step kt's tiles (buffer sb) are complete, and every wave is done with step kt - 1, whose
    // buffer now takes step kt + 1; the registers then load step kt + 2
    __syncthreads();
    stage(sb ^ 1);
    issue(kt + 2);
    const uint4* kst = kstb[sb];
    const uint32_t* vst = vstb[sb];
    const int kc0 = kt * kKeyTile;
    if (kc0 > q0w + 31) return;  // every key of the step is after every query of this wave
    // ---- logits: S^T[key 16 st + 4 c + i][query 16 t + n]
    f32x4 sacc[kQTiles][kKeyTile / 16];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int st = 0; st < kKeyTile / 16; ++st) {
      const int x = 16 * st + n;
      uint4 kf[kD / 32];
#pragma unroll
      for (int j = 0; j < kD / 32; ++j) kf[j] = kst[x * kPPR + ((4 * j + c) ^ pf_kswz(x))];
#pragma unroll
      for (int t = 0; t < kQTiles; ++t) {
        f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kD / 32; ++j)
          s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[j]),
                                                        __builtin_bit_cast(bf16x8, qf[t][j]), s4, 0, 0, 0);
        sacc[t][st] = s4;
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // the causal / budget mask is needed only where the step reaches this wave's queries or the
    // end of the compact sequence (a wave-uniform test)
    if (kc0 + kKeyTile - 1 > q0w || kc0 + kKeyTile > kk) {
#pragma unroll
      for (int t = 0; t < kQTiles; ++t) {
        const int qi = q0w + 16 * t + n;
#pragma unroll
        for (int st = 0; st < kKeyTile / 16; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kc = kc0 + 16 * st + 4 * c + i;
            sacc[t][st][i] = (kc <= qi && kc < kk) ? sacc[t][st][i] : kNegInf;
          }
      }
    }
    // both tiles' column maxima, then one wave-uniform test for the rare move of a reference
    float mt[kQTiles];
#pragma unroll
    for (int t = 0; t < kQTiles; ++t) {
      mt[t] = kNegInf;
#pragma unroll
      for (int st = 0; st < kKeyTile / 16; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt[t] = fmaxf(mt[t], sacc[t][st][i]);
      mt[t] = fmaxf(mt[t], __shfl_xor(mt[t], 16));
      mt[t] = fmaxf(mt[t], __shfl_xor(mt[t], 32));
      mt[t] *= cs;  // scale > 0: the scaled maximum is the maximum of the scaled logits
    }
    if (__ballot(mt[0] > m[0] + kPfLazy || mt[1] > m[1] + kPfLazy)) {
#pragma unroll
      for (int t = 0; t < kQTiles; ++t) {
        const float mn = fmaxf(m[t], mt[t]);
        const float alpha = mn == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m[t] - mn);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * c + i);
          accl[t][i] *= ai;
#pragma unroll
          for (int nb = 0; nb < kD / 16; ++nb) acc[t][nb][i] *= ai;
        }
        m[t] = mn;
      }
    }
    // P in fp16 (rounded to nearest even; the probabilities are below 2^8 by the lazy reference);
    // the normaliser is summed from the same rounded values (accl), so the output is the exact
    // softmax average under logits moved by at most 2^-11 (the weights multiplying V and those
    // dividing agree). ph[t][st][u]: keys 16 st + 4 c + 2 u, + 1 of query 16 t + n, packed
    uint32_t ph[kQTiles][kKeyTile / 16][2];
#pragma unroll
    for (int t = 0; t < kQTiles; ++t) {
      // a column whose reference is still -inf has seen masked logits only: exponent -inf
      const float nm = m[t] == kNegInf ? 0.f : -m[t];
#pragma unroll
      for (int st = 0; st < kKeyTile / 16; ++st) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][st][i], cs, nm));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          typedef _Float16 h2 __attribute__((ext_vector_type(2)));
          h2 hv;
          hv[0] = (_Float16)pr[2 * u];
          hv[1] = (_Float16)pr[2 * u + 1];
          ph[t][st][u] = __builtin_bit_cast(uint32_t, hv);
        }
      }
    }
    // ---- P.V on fp16 K = 32 MFMAs over sub-tile pairs (2 sp, 2 sp + 1): k-slots 8 c .. 8 c + 3 are
    // keys 4 c .. 4 c + 3 of the first sub-tile, 8 c + 4 .. 8 c + 7 the same keys of the second; A = P
    // of query 16 t + n, B = the scaled fp16 V by transpose reads
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int sp = 0; sp < kKeyTile / 32; ++sp) {
      const uint32_t* vr0 = vst + (32 * sp + 4 * c + (n >> 2)) * kVPitchW + 2 * (n & 3);
      const uint32_t* vr1 = vr0 + 16 * kVPitchW;
      const f16x8 ones = f16x8{1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
      for (int t = 0; t < kQTiles; ++t) {
        const uint4 ah = make_uint4(ph[t][2 * sp][0], ph[t][2 * sp][1], ph[t][2 * sp + 1][0], ph[t][2 * sp + 1][1]);
        accl[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ah), ones, accl[t], 0, 0, 0);
      }
#pragma unroll
      for (int nb = 0; nb < kD / 16; ++nb) {
        const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                        (__attribute__((address_space(3))) v4s*)(vr0 + 8 * nb)));
        const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                        (__attribute__((address_space(3))) v4s*)(vr1 + 8 * nb)));
        const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
        for (int t = 0; t < kQTiles; ++t) {
          const uint4 ah = make_uint4(ph[t][2 * sp][0], ph[t][2 * sp][1], ph[t][2 * sp + 1][0], ph[t][2 * sp + 1][1]);
          acc[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ah), bop, acc[t][nb], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  for (int kt = 0;;) {
    step(0, kt);
    if (++kt >= nkt) break;
    step(1, kt);
    if (++kt >= nkt) break;
  }
  const float vscale = ldexpf(1.f, a.vexp[int64_t(b) * a.Hq + h]);  // undo the V scaling
  // acc[t][nb][i]: query 16 t + 4 c + i of the wave, dimension 16 nb + n; accl[t][i]: its normaliser
#pragma unroll
  for (int t = 0; t < kQTiles; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = accl[t][i];
      const int qo = q0w + 16 * t + 4 * c + i;
      if (qo < kk) {
        float* orow = a.out + ((int64_t(b) * a.Hq + h) * a.L + pos_of(qo)) * kD;
#pragma unroll
        for (int nb = 0; nb < kD / 16; ++nb) orow[16 * nb + n] = acc[t][nb][i] / li * vscale;
      }
    }
  }
}

}  // namespace

int launch_prefill_select(const PrefillPlan& p, const sp_tensors& t, char* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sp_config& c = p.cfg;
  const int B = c.batch, Hq = c.n_q_heads, W = c.window;
  uint32_t* status = at<uint32_t>(ws, p.o_status);
  PfScoreArgs s;
  s.q = static_cast<const uint16_t*>(t.q);
  s.q_sb = t.q_sb;
  s.q_sh = t.q_sh;
  s.q_st = t.q_st;
  s.k = static_cast<const uint16_t*>(t.k);
  s.kv_sb = t.kv_sb;
  s.kv_sh = t.kv_sh;
  s.kv_st = t.kv_st;
  s.L = p.L;
  s.W = W;
  s.Hq = Hq;
  s.G = p.G;
  s.nkb = p.nkb;
  s.S = at<double>(ws, p.o_S);
  s.pmq = at<double>(ws, p.o_pmq);
  s.zb = at<double>(ws, p.o_zb);
  s.scale = c.softmax_scale;
  s.status = status;
  hipLaunchKernelGGL(k_pf_scores, dim3((p.nkb + kPfScoreBlocks - 1) / kPfScoreBlocks, Hq, B), dim3(256), 0, st, s);
  hipLaunchKernelGGL(k_pf_rowmax, dim3(Hq, B), dim3(1024), 0, st, at<double>(ws, p.o_pmq), p.nkb, W, at<double>(ws, p.o_M));
  PfImpArgs ia;
  ia.S = at<double>(ws, p.o_S);
  ia.M = at<double>(ws, p.o_M);
  ia.zq = at<double>(ws, p.o_zq);
  ia.imp = at<double>(ws, p.o_imp);
  ia.pmax = at<double>(ws, p.o_pmax);
  ia.pmin = at<double>(ws, p.o_pmin);
  ia.L = p.L;
  ia.W = W;
  ia.Hq = Hq;
  ia.nslab = p.nslab;
  ia.scale = c.softmax_scale;
  hipLaunchKernelGGL(k_pf_zslab, dim3(p.nslab, Hq, B), dim3(kPfMaxWindow), 0, st, ia,
                     static_cast<const double*>(at<double>(ws, p.o_pmq)), static_cast<const double*>(at<double>(ws, p.o_zb)),
                     p.nkb);
  hipLaunchKernelGGL(k_pf_importance, dim3(p.nslab, Hq, B), dim3(256), 0, st, ia);
  hipLaunchKernelGGL(k_pf_global, dim3(p.nslab, B), dim3(256), 0, st, at<double>(ws, p.o_imp), t.head_mode, Hq, p.L,
                     p.nslab,
                     at<double>(ws, p.o_gimp), at<double>(ws, p.o_gpmax), at<double>(ws, p.o_gpmin));
  int e = int(hipGetLastError());
  if (e) return e;
  // budget: top-p of the global importance as masses, p = 1 - tau
  LongRows r;
  r.s = at<double>(ws, p.o_gimp);
  r.len = p.L;
  r.B = B;
  r.H = 1;
  r.topp = 1;
  r.ident = 1;
  r.bitbins = 1;  // importances are >= 0 and span many binades
  r.k = 0;
  r.kbudget = nullptr;
  r.p = 1.0 - c.tau;
  r.scale = 1.0;
  r.pmax = at<double>(ws, p.o_gpmax);
  r.pmin = at<double>(ws, p.o_gpmin);
  r.nblk = p.nslab;
  r.scratch = ws + p.o_long;
  r.bits = at<uint32_t>(ws, p.o_bbits);
  r.words = p.words;
  r.status = status;
  e = launch_long_rows(r, stream);
  if (e) return e;
  hipLaunchKernelGGL(k_pf_budget, dim3(B), dim3(1024), 0, st, at<uint32_t>(ws, p.o_bbits), p.words,
                     at<int32_t>(ws, p.o_budget));
  // every head's top-budget tokens
  r.s = at<double>(ws, p.o_imp);
  r.H = Hq;
  r.topp = 0;
  r.ident = 0;
  r.kbudget = at<int32_t>(ws, p.o_budget);
  r.p = 1.0;
  r.pmax = at<double>(ws, p.o_pmax);
  r.pmin = at<double>(ws, p.o_pmin);
  r.bits = at<uint32_t>(ws, p.o_bits);
  e = launch_long_rows(r, stream);
  if (e) return e;
  hipLaunchKernelGGL(k_pf_lists, dim3(Hq, B), dim3(1024), 0, st, at<uint32_t>(ws, p.o_bits), t.head_mode, p.words,
                     p.L, at<int32_t>(ws, p.o_list));
  return int(hipGetLastError());
}

int launch_prefill_attend(const PrefillPlan& p, const sp_tensors& t, char* ws, float* out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const sp_config& c = p.cfg;
  const int B = c.batch, Hq = c.n_q_heads;
  PfAttnArgs a;
  a.q = static_cast<const uint16_t*>(t.q);
  a.q_sb = t.q_sb;
  a.q_sh = t.q_sh;
  a.q_st = t.q_st;
  a.k = static_cast<const uint16_t*>(t.k);
  a.v = static_cast<const uint16_t*>(t.v);
  a.kv_sb = t.kv_sb;
  a.kv_sh = t.kv_sh;
  a.kv_st = t.kv_st;
  a.list = at<int32_t>(ws, p.o_list);
  a.budget = at<int32_t>(ws, p.o_budget);
  a.mode = t.head_mode;
  a.bits = at<uint32_t>(ws, p.o_bits);
  a.words = p.words;
  a.vmaxp = at<float>(ws, p.o_vmaxp);
  a.vexp = at<int32_t>(ws, p.o_vexp);
  a.nslab = p.nslab;
  a.Hkv = c.n_kv_heads;
  a.kc = at<uint16_t>(ws, p.o_kvc);
  a.vc = a.kc + size_t(B) * Hq * p.Lpad * kD;
  a.out = out;
  a.L = p.L;
  a.Lpad = p.Lpad;
  a.Hq = Hq;
  a.G = p.G;
  a.scale_log2 = float(c.softmax_scale * 1.4426950408889634);
  const int nqb = int((p.L + kPfQueryBlock - 1) / kPfQueryBlock);
  hipLaunchKernelGGL(k_pf_vmax, dim3(p.nslab, c.n_kv_heads, B), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_pf_gather, dim3(int(p.Lpad / kKeyTile), Hq, B), dim3(256), 0, st, a);
  // query blocks for a budget up to L, and at least one zero-row block per head past them
  hipLaunchKernelGGL(k_pf_attend, dim3(nqb + int((p.L + 1023) / 1024), Hq, B), dim3(kPfThreads), 0, st, a);
  return int(hipGetLastError());
}

}  // namespace sd
