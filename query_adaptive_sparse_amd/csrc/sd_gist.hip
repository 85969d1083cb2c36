// Gist-masked (SSA) block-sparse prefill attention: the review of "Simplified Sparse Attention"
// (aitrends.kr, article 69798), sections on the method and technical details (a gist token after
// every chunk; the gist causal mask) and contributions (key-column permutation, block skipping).
//
// Queries come in blocks of 128 of one kind: raw tokens t0 .. t0 + 127, or gists m0 .. m0 + 127.
// After the key-column permutation [gists | raw tokens], a block's visible keys are
//   segment A: gists 0 .. (raw: chunk of its last token - 1; gist: its last gist), and
//   segment B: raw tokens from the start of its first query's chunk (raw) / first gist's chunk
//              (gist) to its last query (raw) / the end of its last gist's chunk (gist),
// so a block visits ceil(|A| / 64) + ceil(|B| / 64) key tiles and skips every other block of the
// mask. Two passes first write every KV head's values as fp16 under a power-of-two scale (the
// max |v| of the head's gist and raw rows, then the scaled copy, gists first) into the workspace.
// Per 64-key step the workgroup stages the tile's K rows (bf16) and V rows (fp16 copy) in LDS (K
// pieces XOR-swizzled, V rows padded for transpose reads); each wave runs q.K^T for its 32 queries
// on the bf16 MFMA, masks where the step reaches a mask boundary, updates an online softmax whose
// reference moves only when a logit exceeds it by 2^8, and accumulates P.V on the fp16 MFMA (K = 32)
// with P rounded to fp16; the normaliser is the same P against a block of ones on the MFMA, so the
// weights multiplying V and those dividing agree. Within a segment, element visibility:
//   raw query t (chunk start s = t - t % C):  gist j < t / C;  raw k in [s, t]
//   gist query m:                             gist j <= m;     raw k in [m C, m C + C)
#include "sd_device.h"
#include "gp_internal.h"

namespace sd {
namespace {

constexpr int kD = 128;         // head dimension
constexpr int kQB = 128;        // queries per workgroup (32 per wave)
constexpr int kPPR = kD / 8;    // 16-byte pieces per row
constexpr int kKeyTile = 64;    // keys staged per step
constexpr int kQTiles = 2;      // 16-query tiles per wave
constexpr float kLazy = 8.f;    // log2 headroom of the lazily moved softmax reference
constexpr int kVPitchW = kD / 2 + 8;  // 32-bit words per staged V row (transpose reads, no bank clash)

struct GpArgs {
  const uint16_t* vc;    // fp16 scaled values [B][Hkv][R][d]: gist rows, then raw rows
  const int32_t* vexp;   // the scale exponent per KV head: vc = v 2^-vexp
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* qg;
  const uint16_t* kg;
  const uint16_t* vg;
  int64_t q_sb, q_sh, q_st, kv_sb, kv_sh, kv_st;
  int64_t qg_sb, qg_sh, qg_st, kvg_sb, kvg_sh, kvg_st;
  float* out;       // [B][Hq][N][d]
  float* out_gist;  // [B][Hq][M][d]
  int N, M, C, Hq, Hkv, G;
  int64_t R;        // M + N
  int nrb, ngb;     // raw and gist query blocks
  float scale_log2;
};

// max |v| over a slab of kGpSlab rows of one KV head's [gists | raw] rows (one workgroup per slab,
// every load of a thread issued before the first is used)
__global__ __launch_bounds__(256) void k_gp_vmax(GpArgs a, float* __restrict__ vmaxp, int nslab) {
  constexpr int kPer = kGpSlab * 16 / 256;  // 16-byte pieces per thread
  const int sl = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  __shared__ float red[4];
  const int64_t j0 = int64_t(sl) * kGpSlab;
  uint4 w[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t i = j0 * 16 + tid + 256 * k;
    const int64_t r = min(i >> 4, a.R - 1);  // rows past the end repeat the last (max unchanged)
    const uint16_t* src = r < a.M ? a.vg + b * a.kvg_sb + g * a.kvg_sh + r * a.kvg_st
                                  : a.v + b * a.kv_sb + g * a.kv_sh + (r - a.M) * a.kv_st;
    w[k] = ld16_stream(src + (i & 15) * 8);
  }
  uint32_t mx = 0;  // |v| as bits: monotone for nonnegative floats
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t u[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = max(mx, max((u[e] << 16) & 0x7fff0000u, u[e] & 0x7fff0000u));
  }
#pragma unroll
  for (int o = 32; o; o >>= 1) mx = max(mx, uint32_t(__shfl_xor(int(mx), o)));
  if ((tid & 63) == 0) red[tid >> 6] = __uint_as_float(mx);
  __syncthreads();
  if (tid == 0) vmaxp[(int64_t(b) * a.Hkv + g) * nslab + sl] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// The scaled fp16 copy of 64 rows of one KV head: scale 2^-e with e = (exponent of the head's max
// |v|) - 15, so the largest value lands in [2^14, 2^15): every bf16 value of magnitude down to 2^-29
// of the max converts exactly, smaller ones round to the fp16 grid (absolute error below 2^-39 of
// the max). e is clamped so that 2^-e and 2^e stay finite fp32 values.
__global__ __launch_bounds__(256) void k_gp_vconv(GpArgs a, const float* __restrict__ vmaxp, int nslab,
                                                  int32_t* __restrict__ vexp, uint16_t* __restrict__ vc) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t head = int64_t(b) * a.Hkv + g;
  const int64_t r0 = int64_t(blockIdx.x) * 64;
  const int pc = tid & 15;
  uint4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = min(r0 + (tid >> 4) + 16 * i, a.R - 1);
    const uint16_t* src = r < a.M ? a.vg + b * a.kvg_sb + g * a.kvg_sh + r * a.kvg_st
                                  : a.v + b * a.kv_sb + g * a.kv_sh + (r - a.M) * a.kv_st;
    w[i] = ld16_stream(src + pc * 8);
  }
  // the head's max |v| from its slab partials, reduced by the workgroup
  __shared__ float red[4];
  float m = 0.f;
  for (int s = tid; s < nslab; s += 256) m = fmaxf(m, vmaxp[head * nslab + s]);
#pragma unroll
  for (int o = 32; o; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (m > 0.f && m <= 3.4028235e38f) {  // every finite max (inputs are finite)
    frexpf(m, &e);                       // m = f 2^e, f in [0.5, 1)
    e -= 15;
    e = e > -126 ? e : -126;
  }
  if (blockIdx.x == 0 && tid == 0) vexp[head] = e;
  const float sc = ldexpf(1.f, -e);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + (tid >> 4) + 16 * i;
    if (r >= a.R) continue;
    const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
    uint32_t hw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      h2 hv;
      hv[0] = (_Float16)(__uint_as_float(u[k] << 16) * sc);
      hv[1] = (_Float16)(__uint_as_float(u[k] & 0xffff0000u) * sc);
      hw[k] = __builtin_bit_cast(uint32_t, hv);
    }
    *reinterpret_cast<uint4*>(vc + (head * a.R + r) * kD + pc * 8) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  }
}


__global__ __launch_bounds__(256, 2) void k_gp_attend(GpArgs a) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  __shared__ uint4 kstb[2][kKeyTile * kPPR];
  __shared__ uint32_t vstb[2][kKeyTile * kVPitchW];
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, n = lane & 15, c = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = h / a.G, C = a.C;
  // heaviest blocks first: the gist blocks (their raw segment spans 128 chunks), last to first,
  // then the raw blocks, last to first
  const bool gist = int(blockIdx.x) < a.ngb;
  const int qblk = gist ? a.ngb - 1 - int(blockIdx.x) : a.nrb - 1 - (int(blockIdx.x) - a.ngb);
  const int nq = gist ? a.M : a.N;            // queries of this kind
  const int q0 = qblk * kQB;
  const int qlast = min(q0 + kQB, nq) - 1;
  // segment A: gist keys [0, na_keys); segment B: raw keys [kb0, kb1)
  const int na_keys = gist ? qlast + 1 : qlast / C;
  const int kb0 = gist ? q0 * C : q0 - q0 % C;
  const int kb1 = gist ? (qlast + 1) * C : qlast + 1;
  const int nA = (na_keys + kKeyTile - 1) / kKeyTile;
  const int nst = nA + (kb1 - kb0 + kKeyTile - 1) / kKeyTile;
  const int q0w = q0 + 32 * wave;              // first query of this wave
  const bool wave_empty = q0w >= nq;           // a wave past the last query only stages tiles
  const int q0v = min(q0w, nq - 1);
  const int qmaxw = min(q0w + 31, nq - 1);
  // query fragments (B operand of q.K^T: query n, dimensions 32 j + 8 c .. + 7) per query tile, and
  // each lane's visibility bounds for its query columns n of the two tiles
  uint4 qf[kQTiles][kD / 32];
  int abound[kQTiles], blo[kQTiles], bhi[kQTiles];
#pragma unroll
  for (int t = 0; t < kQTiles; ++t) {
    const int qi = q0w + 16 * t + n;
    const int qc = min(qi, nq - 1);
    const uint16_t* qrow = gist ? a.qg + b * a.qg_sb + h * a.qg_sh + qc * a.qg_st
                                : a.q + b * a.q_sb + h * a.q_sh + qc * a.q_st;
#pragma unroll
    for (int j = 0; j < kD / 32; ++j) qf[t][j] = ld16(qrow + 32 * j + 8 * c);
    abound[t] = gist ? qc + 1 : qc / C;        // gist keys j < abound
    blo[t] = gist ? qc * C : qc - qc % C;      // raw keys blo <= k < bhi
    bhi[t] = gist ? qc * C + C : qc + 1;
    if (qi >= nq) abound[t] = bhi[t] = 0;      // padding column: sees nothing
  }
  // the wave's union of visible keys per segment, for skipping whole steps
  const int wa_hi = gist ? qmaxw + 1 : qmaxw / C;
  const int wb_lo = gist ? q0v * C : q0v - q0v % C;
  const int wb_hi = gist ? (qmaxw + 1) * C : qmaxw + 1;
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
  // staging: thread pieces tid + 256 i (row x = tid / 16 + 16 i, 16-byte piece pc = tid % 16)
  const int pc = tid & 15, x0 = tid >> 4;
  const uint16_t* kga = a.kg + b * a.kvg_sb + g * a.kvg_sh + pc * 8;
  const uint16_t* kra = a.k + b * a.kv_sb + g * a.kv_sh + pc * 8;
  const uint16_t* vca = a.vc + (int64_t(b) * a.Hkv + g) * a.R * kD + pc * 8;  // gist rows, then raw
  uint4 rk[4], rv[4];
  auto stage = [&](int sbuf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = x0 + 16 * i;
      kstb[sbuf][x * kPPR + (pc ^ (x & 15))] = rk[i];
      *reinterpret_cast<uint4*>(vstb[sbuf] + x * kVPitchW + pc * 4) = rv[i];
    }
  };
  // rows past a segment's end are clamped to the tensor's last row (finite values, masked)
  auto issue = [&](int s) {
    s = s < nst ? s : nst - 1;  // past the end: the last step again (still cached)
    if (s < nA) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = min(s * kKeyTile + x0 + 16 * i, a.M - 1);
        rk[i] = ld16(kga + r * a.kvg_st);
        rv[i] = ld16(vca + r * kD);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = min(kb0 + (s - nA) * kKeyTile + x0 + 16 * i, a.N - 1);
        rk[i] = ld16(kra + r * a.kv_st);
        rv[i] = ld16(vca + (a.M + r) * kD);
      }
    }
  };
  issue(0);
  stage(0);
  issue(1);
  // let step 1's loads land before the loop: the loop head then sees only the loads in flight at
  // its back edge
  __builtin_amdgcn_s_waitcnt(0);
  const float cs = a.scale_log2;
  // one step; sb = s % 2 is a constant at each call site
  auto step = [&](const int sb, const int s) {
    // step s's tiles (buffer sb) are complete, and every wave is done with step s - 1, whose
    // buffer now takes step s + 1; the registers then load step s + 2
    __syncthreads();
    stage(sb ^ 1);
    issue(s + 2);
    const uint4* kst = kstb[sb];
    const uint32_t* vst = vstb[sb];
    const bool segA = s < nA;
    const int k0 = segA ? s * kKeyTile : kb0 + (s - nA) * kKeyTile;  // first key of the step
    // skip a step none of whose keys this wave's queries see
    if (wave_empty || (segA ? k0 >= wa_hi : (k0 >= wb_hi || k0 + kKeyTile <= wb_lo))) return;
    // ---- logits: S^T[key 16 st + 4 c + i][query 16 t + n]
    f32x4 sacc[kQTiles][kKeyTile / 16];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int st = 0; st < kKeyTile / 16; ++st) {
      const int x = 16 * st + n;
      uint4 kf[kD / 32];
#pragma unroll
      for (int j = 0; j < kD / 32; ++j) kf[j] = kst[x * kPPR + ((4 * j + c) ^ (x & 15))];
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
    // mask: segment A where the step reaches the smallest bound of the wave's queries; segment B
    // always (chunk-diagonal blocks). Wave-uniform tests.
    if (segA ? k0 + kKeyTile > (gist ? q0v + 1 : q0v / C) : true) {
#pragma unroll
      for (int t = 0; t < kQTiles; ++t)
#pragma unroll
        for (int st = 0; st < kKeyTile / 16; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kx = k0 + 16 * st + 4 * c + i;
            const bool vis = segA ? kx < abound[t] : (kx >= blo[t] && kx < bhi[t]);
            sacc[t][st][i] = vis ? sacc[t][st][i] : kNegInf;
          }
    }
    // P in fp16 (rounded to nearest even; below 2^8 by the lazy reference). ph[t][st][u]: keys
    // 16 st + 4 c + 2 u, + 1 of query 16 t + n, packed
    uint32_t ph[kQTiles][kKeyTile / 16][2];
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
    if (__ballot(mt[0] > m[0] + kLazy || mt[1] > m[1] + kLazy)) {
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
    // keys 4 c .. 4 c + 3 of the first sub-tile, 8 c + 4 .. 8 c + 7 the same keys of the second. The
    // V operand is one ds_read_b64_tr_b16 per sub-tile: lane i of a 16-lane group receives element
    // i % 4 of the 8-byte words addressed by lanes i / 4, + 4, + 8, + 12 of its group
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
  for (int s = 0;;) {
    step(0, s);
    if (++s >= nst) break;
    step(1, s);
    if (++s >= nst) break;
  }
  // acc[t][nb][i]: query 16 t + 4 c + i of the wave, dimension 16 nb + n; accl[t][i]: its normaliser
  float* obase = gist ? a.out_gist + (int64_t(b) * a.Hq + h) * a.M * kD : a.out + (int64_t(b) * a.Hq + h) * a.N * kD;
  const float vscale = ldexpf(1.f, a.vexp[int64_t(b) * a.Hkv + g]);  // undo the V scaling
#pragma unroll
  for (int t = 0; t < kQTiles; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = accl[t][i];
      const int qo = q0w + 16 * t + 4 * c + i;
      if (qo < nq) {
        float* orow = obase + int64_t(qo) * kD;
#pragma unroll
        for (int nb = 0; nb < kD / 16; ++nb) orow[16 * nb + n] = acc[t][nb][i] / li * vscale;
      }
    }
  }
}

}  // namespace

int launch_gist_prefill(const GistPlan& p, const gp_tensors& t, char* ws, float* out, float* out_gist, void* stream) {
  const gp_config& c = p.cfg;
  hipStream_t st = static_cast<hipStream_t>(stream);
  GpArgs a;
  float* vmaxp = reinterpret_cast<float*>(ws + p.o_vmaxp);
  int32_t* vexp = reinterpret_cast<int32_t*>(ws + p.o_vexp);
  uint16_t* vc = reinterpret_cast<uint16_t*>(ws + p.o_vc);
  a.vc = vc;
  a.vexp = vexp;
  a.q = static_cast<const uint16_t*>(t.q);
  a.k = static_cast<const uint16_t*>(t.k);
  a.v = static_cast<const uint16_t*>(t.v);
  a.qg = static_cast<const uint16_t*>(t.qg);
  a.kg = static_cast<const uint16_t*>(t.kg);
  a.vg = static_cast<const uint16_t*>(t.vg);
  a.q_sb = t.q_sb;
  a.q_sh = t.q_sh;
  a.q_st = t.q_st;
  a.kv_sb = t.kv_sb;
  a.kv_sh = t.kv_sh;
  a.kv_st = t.kv_st;
  a.qg_sb = t.qg_sb;
  a.qg_sh = t.qg_sh;
  a.qg_st = t.qg_st;
  a.kvg_sb = t.kvg_sb;
  a.kvg_sh = t.kvg_sh;
  a.kvg_st = t.kvg_st;
  a.out = out;
  a.out_gist = out_gist;
  a.N = int(c.n_tokens);
  a.M = p.M;
  a.C = c.chunk_size;
  a.Hq = c.n_q_heads;
  a.Hkv = c.n_kv_heads;
  a.G = p.G;
  a.R = p.R;
  a.nrb = (a.N + kQB - 1) / kQB;
  a.ngb = (a.M + kQB - 1) / kQB;
  a.scale_log2 = float(c.softmax_scale * 1.4426950408889634);
  hipLaunchKernelGGL(k_gp_vmax, dim3(p.nslab, c.n_kv_heads, c.batch), dim3(256), 0, st, a, vmaxp, p.nslab);
  hipLaunchKernelGGL(k_gp_vconv, dim3(unsigned((p.R + 63) / 64), c.n_kv_heads, c.batch), dim3(256), 0, st, a,
                     static_cast<const float*>(vmaxp), p.nslab, vexp, vc);
  hipLaunchKernelGGL(k_gp_attend, dim3(a.nrb + a.ngb, c.n_q_heads, c.batch), dim3(256), 0, st, a);
  return int(hipGetLastError());
}

}  // namespace sd
