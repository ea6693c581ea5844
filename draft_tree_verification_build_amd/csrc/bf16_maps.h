// Integer maps and compile-time tables for bf16 logit rows. Plain C++17 constexpr (no HIP
// headers), so the same definitions serve the kernels and a host-side check.
//
// Order keys: the 16-bit key of a bf16 pattern b is 0x8000 + x, where x is the signed
// magnitude of b read as a two's complement integer (+m for a positive pattern, -m for a
// negative one, m = b & 0x7FFF). Keys are monotone in the value, -0 and +0 share a key, and
// every pattern has a key in 1..0xFFFF, so 0 is free to mark padding past a row's end.
//
// Exponentials: entry 2r + s of the table holds exp(v) for the bf16 value v whose magnitude
// bits are kExpBf16Lo + r and whose sign is s, for every value 2^-16 <= |v| < 2^8. Then a
// pair of 1.0 (r = kExpBf16Mags, where out-of-range magnitudes are sent: exp of a tiny value,
// to be corrected) and a pair of 0.0 (r = kExpBf16Mags + 1, for padding). Each
// entry is evaluated at compile time by Tang's table-driven method (P. T. P. Tang, ACM TOMS
// 15(2), 1989): v = (64 M + j) ln2/64 + r, exp(v) = 2^M 2^(j/64) (1 + q(r)), with q the
// degree-5 Taylor polynomial of exp(r) - 1 (truncation below 4e-17 relative for
// |r| <= ln2/128), added to 2^(j/64) last so that an entry is within about 1 ulp.
#pragma once

#include <stdint.h>

namespace dtv {

constexpr uint32_t bf16_order_key(uint32_t b) {
  const uint32_t m = b & 0x7FFFu;
  return (b & 0x8000u) ? 0x8000u - m : 0x8000u + m;
}

// Inverse of bf16_order_key for keys 1..0xFFFF (key 0x8000 gives +0).
constexpr uint32_t bf16_key_bits(uint32_t k) { return k >= 0x8000u ? k - 0x8000u : (0x8000u | (0x8000u - k)); }

// 2^(j/64), j = 0..63, each rounded to the nearest double.
struct Exp2Table {
  double v[64];
};
constexpr Exp2Table kExp2Tab = {{
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
}};

constexpr uint32_t kExpBf16Lo = 0x3780u;          // magnitude bits of 2^-16
constexpr uint32_t kExpBf16Mags = 24u * 128u;     // magnitudes 2^-16 .. 2^8 (exclusive)
constexpr int kExpBf16Entries = 2 * kExpBf16Mags + 4;

struct ExpBf16Table {
  double v[kExpBf16Entries];
};

// v * 2^e, exact while the result is a normal double.
constexpr double cx_scale2(double v, int e) {
  double p = 1.0, b = e >= 0 ? 2.0 : 0.5;
  for (int n = e >= 0 ? e : -e; n != 0; n >>= 1) {
    if (n & 1) p *= b;
    b *= b;
  }
  return v * p;
}

// exp(x) for |x| < 700, Tang's reduction with ln2/64 in two parts (k * L1 is exact for
// |k| < 2^17).
constexpr double cx_exp(double x) {
  const double kInv = 0x1.71547652b82fep+6;   // 64 / ln2
  const double kL1 = 0x1.62e42fefa0000p-7;
  const double kL2 = 0x1.cf79abc9e3b3ap-46;
  const double xk = x * kInv;
  const long long k = static_cast<long long>(xk >= 0.0 ? xk + 0.5 : xk - 0.5);
  const double kd = static_cast<double>(k);
  const double r = (x - kd * kL1) - kd * kL2;
  // q = exp(r) - 1, so that the table value takes one rounding at the end: T + T q
  double q = r * (1.0 / 120.0) + 1.0 / 24.0;
  q = r * q + 1.0 / 6.0;
  q = r * q + 0.5;
  q = r * q + 1.0;
  q = r * q;
  const long long j = k & 63;
  const long long m = (k - j) / 64;
  const double t = kExp2Tab.v[j];
  return cx_scale2(t + t * q, static_cast<int>(m));
}

// The bf16 value of magnitude bits mb (a normal number), as a double.
constexpr double bf16_magnitude(uint32_t mb) {
  return cx_scale2(static_cast<double>(128u + (mb & 127u)), static_cast<int>(mb >> 7) - 127 - 7);
}

constexpr ExpBf16Table make_exp_bf16_table() {
  ExpBf16Table t{};
  for (uint32_t r = 0; r < kExpBf16Mags; ++r) {
    const double v = bf16_magnitude(kExpBf16Lo + r);
    t.v[2 * r] = cx_exp(v);
    t.v[2 * r + 1] = cx_exp(-v);
  }
  t.v[2 * kExpBf16Mags] = 1.0;
  t.v[2 * kExpBf16Mags + 1] = 1.0;
  t.v[2 * kExpBf16Mags + 2] = 0.0;
  t.v[2 * kExpBf16Mags + 3] = 0.0;
  return t;
}

constexpr ExpBf16Table kExpBf16Tab = make_exp_bf16_table();

}  // namespace dtv
