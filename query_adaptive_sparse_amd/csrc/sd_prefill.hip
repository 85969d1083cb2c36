// Token-Sparse prefill: dynamic token coverage selection, then compressed causal attention over
// each head's kept tokens, scattered back into the sequence-length output.
//
// Selection (fp64, matching a sequential CPU evaluation up to the order of the softmax sums):
//   k_pf_scores      proxy scores s[key][q] = q . k of the W window queries against 64 keys per
//                    workgroup, on the fp64 MFMA (16 keys x 16 queries x 4 dimensions per
//                    instruction; chained over the dimensions in index order, each output is the
//                    sequential fma chain of the dot product), and each query's max per key block;
//   k_pf_rowmax      every window query's max over its visible keys;
//   k_pf_zpart       per 2048-key slab and query, the sum of exp(scale (s - max)) over the slab;
//   k_pf_importance  per key, the sum over the window queries (in order) of the query's softmax
//                    probability of that key, and the slab's max / min of it;
//   k_pf_global      per key, the heads' importances summed in head order;
//   long-row pass    top-p of the global importance with the values as masses, p = 1 - tau;
//   k_pf_budget      budget = (that count) - 1, at least 1: the tokens left after cutting the
//                    ascending tail whose mass exceeds tau of the total;
//   long-row pass    every head's top-budget tokens by its own importance;
//   k_pf_lists       each head's bitmap as an ascending position list.
// Attention:
//   k_pf_attend      64 compact queries per workgroup (16 per wave), heaviest blocks first; the
//                    workgroup gathers 64 compact keys' K and V rows per step into LDS (K pieces
//                    XOR-swizzled per row, V rows padded), each wave runs q.K^T on the bf16 MFMA,
//                    the causal mask in compact order, an online softmax and P.V (hi and lo
//                    halves of P on two MFMAs), then writes its rows to their positions;
//   k_pf_zero        positions a head did not keep get zero rows.
#include "sd_device.h"

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
  uint32_t* status;
};

constexpr int kD = 128;
constexpr int kKRow = kD + 8;  // padded bf16 row in LDS (elements)

__global__ __launch_bounds__(256) void k_pf_scores(PfScoreArgs a) {
  __shared__ uint16_t qs[kPfMaxWindow * kKRow];
  __shared__ uint16_t ks[kPfKeyBlock * kKRow];
  __shared__ double wmax[4][kPfMaxWindow];
  const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, n = lane & 15, c = lane >> 4;
  if (a.status && kb == 0 && h == 0 && b == 0 && tid < 16) a.status[tid] = 0;
  const int g = h / a.G;
  const int64_t key0 = int64_t(kb) * kPfKeyBlock;
  const int64_t qpos0 = a.L - a.W;
  // window queries (rows past W are zero) and the block's keys (past L: the last key) -> LDS
  for (int i = tid; i < kPfMaxWindow * (kD / 8); i += 256) {
    const int r = i / (kD / 8), pc = i - r * (kD / 8);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < a.W) v = ld16(a.q + b * a.q_sb + h * a.q_sh + (qpos0 + r) * a.q_st + pc * 8);
    *reinterpret_cast<uint4*>(qs + r * kKRow + pc * 8) = v;
  }
  for (int i = tid; i < kPfKeyBlock * (kD / 8); i += 256) {
    const int r = i / (kD / 8), pc = i - r * (kD / 8);
    const int64_t key = key0 + r < a.L ? key0 + r : a.L - 1;
    *reinterpret_cast<uint4*>(ks + r * kKRow + pc * 8) =
        ld16(a.k + b * a.kv_sb + g * a.kv_sh + key * a.kv_st + pc * 8);
  }
  __syncthreads();
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
  __syncthreads();
  if (tid < a.W)
    a.pmq[((int64_t(b) * a.Hq + h) * a.nkb + kb) * a.W + tid] =
        fmax(fmax(wmax[0][tid], wmax[1][tid]), fmax(wmax[2][tid], wmax[3][tid]));
}

// Every window query's max over its visible keys (the block maxima reduced in block order).
__global__ __launch_bounds__(256) void k_pf_rowmax(const double* __restrict__ pmq, int nkb, int W, double* __restrict__ M) {
  const int h = blockIdx.x, b = blockIdx.y, Hq = gridDim.x, tid = threadIdx.x;
  __shared__ double red[4][kPfMaxWindow];
  const int qi = tid & 63, part = tid >> 6;
  double m = kNegInfD;
  if (qi < W)
    for (int kb = part; kb < nkb; kb += 4) m = fmax(m, pmq[((int64_t(b) * Hq + h) * nkb + kb) * W + qi]);
  red[part][qi] = m;
  __syncthreads();
  if (tid < W) M[(int64_t(b) * Hq + h) * W + tid] = fmax(fmax(red[0][tid], red[1][tid]), fmax(red[2][tid], red[3][tid]));
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

// Per slab and window query: the sum over the slab's visible keys of exp(scale s - scale max), keys
// in order within each of the 4 waves (a quarter of the slab each), the waves in order.
__global__ __launch_bounds__(256) void k_pf_zpart(PfImpArgs a) {
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int qi = tid & 63, wave = tid >> 6;
  __shared__ double red[4][kPfMaxWindow];
  const int64_t row = int64_t(b) * a.Hq + h;
  const int64_t j0 = int64_t(sl) * kPfSlab, j1 = j0 + kPfSlab < a.L ? j0 + kPfSlab : a.L;
  const int64_t per = (j1 - j0 + 3) / 4;
  const int64_t ja = j0 + wave * per, jb = ja + per < j1 ? ja + per : j1;
  double z = 0.0;
  if (qi < a.W) {
    const double mq = a.scale * a.M[row * a.W + qi];
    const int64_t vis = a.L - a.W + qi;  // last visible key
    const double* sp = a.S + row * a.L * a.W + qi;
    for (int64_t j = ja; j < jb && j <= vis; ++j) z += exp(a.scale * sp[j * a.W] - mq);
  }
  red[wave][qi] = z;
  __syncthreads();
  if (tid < a.W) a.zq[(row * a.nslab + sl) * a.W + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

// Per key of the slab: importance = sum over the window queries, in order, of
// exp(scale s - scale max_q) / Z_q (Z_q: the slab partials summed in slab order); and the slab's
// max / min of the importance.
__global__ __launch_bounds__(256) void k_pf_importance(PfImpArgs a) {
  const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ double zs[kPfMaxWindow], ms[kPfMaxWindow];
  __shared__ double rmax[4], rmin[4];
  const int64_t row = int64_t(b) * a.Hq + h;
  if (tid < a.W) {
    double z = 0.0;
    for (int s = 0; s < a.nslab; ++s) z += a.zq[(row * a.nslab + s) * a.W + tid];
    zs[tid] = z;
    ms[tid] = a.scale * a.M[row * a.W + tid];
  }
  __syncthreads();
  const int64_t j0 = int64_t(sl) * kPfSlab, j1 = j0 + kPfSlab < a.L ? j0 + kPfSlab : a.L;
  double mx = kNegInfD, mn = kPosInfD;
  for (int64_t j = j0 + tid; j < j1; j += 256) {
    const double* sp = a.S + (row * a.L + j) * a.W;
    const int64_t q0 = j - (a.L - a.W);  // first window query that sees key j
    double v = 0.0;
    for (int qi = q0 > 0 ? int(q0) : 0; qi < a.W; ++qi) v += exp(a.scale * sp[qi] - ms[qi]) / zs[qi];
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
__global__ __launch_bounds__(256) void k_pf_global(const double* __restrict__ imp, int Hq, int64_t L, int nslab,
                                                   double* __restrict__ gimp, double* __restrict__ gpmax,
                                                   double* __restrict__ gpmin) {
  const int sl = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ double rmax[4], rmin[4];
  const int64_t j0 = int64_t(sl) * kPfSlab, j1 = j0 + kPfSlab < L ? j0 + kPfSlab : L;
  double mx = kNegInfD, mn = kPosInfD;
  for (int64_t j = j0 + tid; j < j1; j += 256) {
    double v = 0.0;
    for (int h = 0; h < Hq; ++h) v += imp[(int64_t(b) * Hq + h) * L + j];
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
__global__ __launch_bounds__(1024) void k_pf_lists(const uint32_t* __restrict__ bits, int64_t words,
                                                   int64_t L, int32_t* __restrict__ list) {
  const int h = blockIdx.x, b = blockIdx.y, Hq = gridDim.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int wtot[16];
  const int64_t row = int64_t(b) * Hq + h;
  const uint32_t* bw = bits + row * words;
  int32_t* out = list + row * L;
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
// Compressed causal attention. Wave w of query block qb owns compact queries
// 64 qb + 16 w + n (n = lane % 16); per step the workgroup holds 64 compact keys in LDS.
// ---------------------------------------------------------------------------------------------
struct PfAttnArgs {
  const uint16_t* q;
  int64_t q_sb, q_sh, q_st;
  const uint16_t* k;
  const uint16_t* v;
  int64_t kv_sb, kv_sh, kv_st;
  const int32_t* list;    // [B][Hq][L]
  const int32_t* budget;  // [B]
  float* out;             // [B][Hq][L][d]
  int64_t L;
  int Hq, G;
  float scale_log2;
};

constexpr int kPPR = kD / 8;        // 16-byte pieces per row
constexpr int kVRowW = kD / 2 + 4;  // padded V row in LDS (32-bit words)

__device__ __forceinline__ int pf_kswz(int x) { return x & 15; }

__global__ __launch_bounds__(256, 2) void k_pf_attend(PfAttnArgs a) {
  __shared__ uint4 kst[kPfQueryBlock * kPPR];
  __shared__ uint32_t vst[kPfQueryBlock * kVRowW];
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, n = lane & 15, c = lane >> 4;
  const int kk = min(max(a.budget[b], 1), int(a.L));
  const int nqb = (kk + kPfQueryBlock - 1) / kPfQueryBlock;
  if (int(blockIdx.x) >= nqb) return;
  const int qb = nqb - 1 - int(blockIdx.x);  // heaviest (longest causal range) first
  const int g = h / a.G;
  const int32_t* lst = a.list + (int64_t(b) * a.Hq + h) * a.L;
  // list entries are positions in [0, L); clamped so that an incomplete selection row (status
  // flag raised) can never address outside the tensors
  auto pos_of = [&](int i) {
    const int v = lst[i];
    return int64_t(v < 0 ? 0 : (v < a.L ? v : a.L - 1));
  };
  const uint16_t* kbase = a.k + b * a.kv_sb + g * a.kv_sh;
  const uint16_t* vbase = a.v + b * a.kv_sb + g * a.kv_sh;
  // this lane's query (B operand of q.K^T: query n, dimensions 32 j + 8 c .. + 7)
  const int qi = qb * kPfQueryBlock + 16 * wave + n;
  const int64_t qrow = pos_of(qi < kk ? qi : kk - 1);
  uint4 qf[kD / 32];
#pragma unroll
  for (int j = 0; j < kD / 32; ++j) qf[j] = ld16(a.q + b * a.q_sb + h * a.q_sh + int64_t(qrow) * a.q_st + 32 * j + 8 * c);
  float m = kNegInf, l = 0.f;
  f32x4 acc[kD / 16];
#pragma unroll
  for (int nb = 0; nb < kD / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // keys of step kt: compact 64 kt + x; thread pieces tid + 256 i (row x = piece / 16)
  uint4 rk[4], rv[4];
  auto issue = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pcs = tid + 256 * i, x = pcs >> 4, pc = pcs & 15;
      const int kc = kt * kPfQueryBlock + x;
      const int64_t row = pos_of(kc < kk ? kc : kk - 1);
      rk[i] = ld16_stream(kbase + row * a.kv_st + pc * 8);
      rv[i] = ld16_stream(vbase + row * a.kv_st + pc * 8);
    }
  };
  issue(0);
  for (int kt = 0; kt <= qb; ++kt) {
    __syncthreads();  // every wave is done with the previous step's tiles
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pcs = tid + 256 * i, x = pcs >> 4, pc = pcs & 15;
      kst[x * kPPR + (pc ^ pf_kswz(x))] = rk[i];
      *reinterpret_cast<uint4*>(vst + x * kVRowW + pc * 4) = rv[i];
    }
    __syncthreads();
    if (kt < qb) issue(kt + 1);
#pragma unroll 1
    for (int st = 0; st < kPfQueryBlock / 16; ++st) {
      const int kc0 = kt * kPfQueryBlock + 16 * st;  // first compact key of the sub-tile
      if (kc0 > qb * kPfQueryBlock + 16 * wave + 15) break;  // past every query of this wave
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
      const int x = 16 * st + n;
#pragma unroll
      for (int j = 0; j < kD / 32; ++j)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kst[x * kPPR + ((4 * j + c) ^ pf_kswz(x))]),
                                                        __builtin_bit_cast(bf16x8, qf[j]), sacc, 0, 0, 0);
      // logits S^T[key 4c + i][query n]; causal in compact order and inside the budget
      float lg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kc = kc0 + 4 * c + i;
        lg[i] = (kc <= qi && kc < kk) ? sacc[i] * a.scale_log2 : kNegInf;
      }
      float mt = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      const bool none = mn == kNegInf;
      if (__ballot(mn > m)) {
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * c + i);
#pragma unroll
          for (int nb = 0; nb < kD / 16; ++nb) acc[nb][i] *= ai;
        }
        m = mn;
      }
      u16x4 ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = none ? 0.f : __builtin_amdgcn_exp2f(lg[i] - mn);
        l += pr;
        const uint16_t hi = f2bf(pr);
        ph[i] = hi;
        pl[i] = f2bf(pr - bf2f(hi));
      }
      const uint16_t* v16 = reinterpret_cast<const uint16_t*>(vst);
#pragma unroll
      for (int nb = 0; nb < kD / 16; ++nb) {
        u16x4 vb;
#pragma unroll
        for (int i = 0; i < 4; ++i) vb[i] = v16[(16 * st + 4 * c + i) * (2 * kVRowW) + 16 * nb + n];
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, ph),
                                                             __builtin_bit_cast(bf16x4, vb), acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, pl),
                                                             __builtin_bit_cast(bf16x4, vb), acc[nb], 0, 0, 0);
      }
    }
  }
  // normaliser of every query column (the 4 lane groups hold partial sums of the same column)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  // acc[nb][i]: query 16 wave + 4c + i (of the block), dimension 16 nb + n
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float li = __shfl(l, 4 * c + i);
    const int qo = qb * kPfQueryBlock + 16 * wave + 4 * c + i;
    if (qo < kk) {
      float* orow = a.out + ((int64_t(b) * a.Hq + h) * a.L + pos_of(qo)) * kD;
#pragma unroll
      for (int nb = 0; nb < kD / 16; ++nb) orow[16 * nb + n] = acc[nb][i] / li;
    }
  }
}

// Zero rows at the positions a head did not keep (one thread per position).
__global__ __launch_bounds__(256) void k_pf_zero(const uint32_t* __restrict__ bits, int64_t words, int64_t L,
                                                 float* __restrict__ out) {
  const int h = blockIdx.y, b = blockIdx.z, Hq = gridDim.y;
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j >= L) return;
  const int64_t row = int64_t(b) * Hq + h;
  if ((bits[row * words + (j >> 5)] >> (j & 31)) & 1u) return;
  float4* o = reinterpret_cast<float4*>(out + (row * L + j) * kD);
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
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
  s.status = status;
  hipLaunchKernelGGL(k_pf_scores, dim3(p.nkb, Hq, B), dim3(256), 0, st, s);
  hipLaunchKernelGGL(k_pf_rowmax, dim3(Hq, B), dim3(256), 0, st, at<double>(ws, p.o_pmq), p.nkb, W, at<double>(ws, p.o_M));
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
  hipLaunchKernelGGL(k_pf_zpart, dim3(p.nslab, Hq, B), dim3(256), 0, st, ia);
  hipLaunchKernelGGL(k_pf_importance, dim3(p.nslab, Hq, B), dim3(256), 0, st, ia);
  hipLaunchKernelGGL(k_pf_global, dim3(p.nslab, B), dim3(256), 0, st, at<double>(ws, p.o_imp), Hq, p.L, p.nslab,
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
  hipLaunchKernelGGL(k_pf_lists, dim3(Hq, B), dim3(1024), 0, st, at<uint32_t>(ws, p.o_bits), p.words, p.L,
                     at<int32_t>(ws, p.o_list));
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
  a.out = out;
  a.L = p.L;
  a.Hq = Hq;
  a.G = p.G;
  a.scale_log2 = float(c.softmax_scale * 1.4426950408889634);
  const int nqb = int((p.L + kPfQueryBlock - 1) / kPfQueryBlock);
  hipLaunchKernelGGL(k_pf_zero, dim3(int((p.L + 255) / 256), Hq, B), dim3(256), 0, st, at<uint32_t>(ws, p.o_bits),
                     p.words, p.L, out);
  hipLaunchKernelGGL(k_pf_attend, dim3(nqb, Hq, B), dim3(256), 0, st, a);
  return int(hipGetLastError());
}

}  // namespace sd
