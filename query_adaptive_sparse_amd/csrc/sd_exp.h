// exp(x) for x <= 0 in fp64, for the prefill's proxy softmax sums: the library exp spends about
// 21 fp64 and 25 other vector instructions per call on gfx950, this one 11 fp64 ones and an LDS read.
//   exp(x) = 2^k 2^(j/64) exp(r),  n = rint(64 x / ln 2) = 64 k + j (0 <= j < 64),
//   r = x - n ln2/64, |r| <= ln2/128, with ln2/64 in two parts (n times the 36-bit high part is
//   exact for |n| < 2^17), and exp(r) by its Taylor polynomial of degree 5 (truncation below
//   r^6/720 < 3.5e-17 relative); the result is 2^(j/64) (1 + q), q = exp(r) - 1, in one fma. The
//   table holds 2^(j/64) correctly rounded (written by gen_exp_table.py). About 1 ulp from exp (a
//   host build of this code is checked against numpy's exp); 0 below about -745 (arguments are
//   clamped to -1100, NaN included).
#pragma once

#define SD_EXP2_64_TABLE \
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0, \
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0, \
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0, \
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0, \
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0, \
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0, \
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0, \
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0, \
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0, \
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0, \
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0, \
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0, \
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0, \
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0, \
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0, \
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0

namespace sd {

struct ExpC {
  double inv, hi, lo, c3, c4, c5;
};
__host__ __device__ inline ExpC exp_consts() {
  return ExpC{0x1.71547652b82fep+6,   // 64 / ln 2
              0x1.62e42fefa0000p-7,   // ln 2 / 64, high 36 bits
              0x1.cf79abc9e3b3ap-46,  // ln 2 / 64 - high part
              1.0 / 6.0, 1.0 / 24.0, 1.0 / 120.0};
}

// tab: the 64 values of SD_EXP2_64_TABLE (LDS on the device)
__host__ __device__ inline double exp_nonpos(double x, const double* tab, const ExpC& c) {
  x = x > -1100.0 ? x : -1100.0;
  const double nd = rint(x * c.inv);
  const int n = int(nd);
  const double r = fma(-nd, c.lo, fma(-nd, c.hi, x));
  // q = exp(r) - 1 (small: its rounding barely reaches the result), then t + t q in one rounding
  double p = fma(r, c.c5, c.c4);
  p = fma(p, r, c.c3);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  const double q = p * r;
  const double t = tab[n & 63];
  return ldexp(fma(t, q, t), n >> 6);
}

}  // namespace sd
