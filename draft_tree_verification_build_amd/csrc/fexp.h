// exp(d) for d <= 0 in float64, table-driven (P. T. P. Tang, "Table-driven implementation
// of the exponential function in IEEE floating-point arithmetic", ACM TOMS 15(2), 1989).
//
// d = (64 M + j) ln2/64 + r with |r| <= ln2/128; exp(d) = 2^M * 2^(j/64) * p(r), where p is
// the degree-5 Taylor polynomial of exp (truncation error below 4e-17 relative on that
// interval) and 2^(j/64) comes from a 64-entry table. ln2/64 is split in two parts so that
// k * L1 is exact for every |k| < 2^17. Accuracy: about 1 ulp, in about ten float64
// operations and one shared-memory read.
#pragma once

#include <hip/hip_runtime.h>

namespace dtv {

// 2^(j/64), j = 0..63, each rounded to the nearest double.
__constant__ double kExp2_64[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

// Copies the table into shared memory (call from every thread, then __syncthreads()).
__device__ __forceinline__ void exp_table_load(double* t) {
  for (int j = threadIdx.x; j < 64; j += blockDim.x) t[j] = kExp2_64[j];
}

// exp(d) for d <= 0 (d = -inf or NaN gives 0). `t` is the shared-memory copy of kExp2_64.
// Branch-free, so that a caller's unrolled loop keeps all its table reads in flight.
__device__ __forceinline__ double exp_nonpos(double d, const double* t) {
  const bool under = !(d >= -745.0);
  const double dc = under ? -745.0 : d;
  const double kInv = 0x1.71547652b82fep+6;   // 64 / ln2
  const double kL1 = 0x1.62e42fefa0000p-7;    // ln2/64, leading 36 bits
  const double kL2 = 0x1.cf79abc9e3b3ap-46;   // ln2/64 - kL1
  const double k = rint(dc * kInv);
  const int n = static_cast<int>(k);
  const double r = fma(-k, kL2, fma(-k, kL1, dc));
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(r, p, 1.0 / 6.0);
  p = fma(r, p, 0.5);
  p = fma(r, p, 1.0);
  p = fma(r, p, 1.0);
  const double e = ldexp(t[n & 63] * p, n >> 6);
  return under ? 0.0 : e;
}

// sum_j exp(x[j] - m) for x[j] <= m, each term as in exp_nonpos except for how the
// reduction is rounded: k = rint(d * 64/ln2) is read off fma(d, 64/ln2, 1.5 * 2^52), whose
// low 32 bits hold k in two's complement, and d is clamped at -745 instead of selecting 0
// (a term of exp(-745) < 2^-1074 is below every sum, which is at least 1). Entries of -inf
// contribute that negligible term. Groups of G terms are written in three passes
// (reductions, table reads, scaling) so that the group's table reads are in flight
// together; G bounds the extra registers.
template <int N, int G = 8>
__device__ __forceinline__ double exp_nonpos_sum(const float (&x)[N], double m, const double* t) {
  static_assert(N % G == 0, "N must be a multiple of G");
  const double kInv = 0x1.71547652b82fep+6;
  const double kL1 = 0x1.62e42fefa0000p-7;
  const double kL2 = 0x1.cf79abc9e3b3ap-46;
  const double kShift = 0x1.8p52;
  double s = 0.0;
#pragma unroll
  for (int g0 = 0; g0 < N; g0 += G) {
    double p[G];
    int n[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const double dc = fmax(static_cast<double>(x[g0 + j]) - m, -745.0);
      const double kp = fma(dc, kInv, kShift);
      n[j] = __double2loint(kp);
      const double k = kp - kShift;
      const double r = fma(-k, kL2, fma(-k, kL1, dc));
      double q = fma(r, 1.0 / 120.0, 1.0 / 24.0);
      q = fma(r, q, 1.0 / 6.0);
      q = fma(r, q, 0.5);
      q = fma(r, q, 1.0);
      p[j] = fma(r, q, 1.0);
    }
    double tv[G];
#pragma unroll
    for (int j = 0; j < G; ++j) tv[j] = t[n[j] & 63];
#pragma unroll
    for (int j = 0; j < G; ++j) s += ldexp(tv[j] * p[j], n[j] >> 6);
  }
  return s;
}

}  // namespace dtv
