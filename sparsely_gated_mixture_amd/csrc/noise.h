// Counter-based Gaussian noise of the noisy gate, shared by the router and the
// backward pass (the same sample must be redrawn there).
//
// The pages ask for a fresh N(0, 1) sample per expert component ("Outrageously
// Large Neural Networks" summary, section 3.4, "Noisy Top-K Gating", Step 1);
// the sample for token t and experts 4q .. 4q+3 is Philox4x64-10 at counter
// (t, q, 0, 0) under key (seed, key1), fed through Box-Muller in fp64.
#pragma once

#include <stdint.h>

namespace moe {

// Salmon et al., SC'11: ten rounds; each round multiplies counter words 0 and 2
// by the two published constants (full 128-bit products), mixes in the key and
// permutes; the key advances by the published Weyl increments between rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t& c0, uint64_t& c1, uint64_t& c2,
                                              uint64_t& c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
}

// sin(2 pi u) and cos(2 pi u) in fp64 for u = m 2^-53 in [0, 1). The argument needs no
// general range reduction: 4u is exact, q = the nearest integer (the quadrant) and r = 4u - q
// in [-1/2, 1/2] are exact, and x = r pi/2 (pi/2 split in two parts) lies in [-pi/4, pi/4],
// where the Taylor series of sin to x^17 and of cos to x^18 leave a remainder below 1e-19.
__device__ __forceinline__ void sincos_2pi(double u, double& s, double& c) {
  const double u4 = u * 4.0;
  const double q = rint(u4);
  const double r = u4 - q;
  const double x = fma(r, 1.5707963267948966, r * 6.123233995736766e-17);
  const double x2 = x * x;
  double ps = -1.0 / 355687428096000.0;  // -1/17!
  ps = fma(ps, x2, 1.0 / 1307674368000.0);
  ps = fma(ps, x2, -1.0 / 6227020800.0);
  ps = fma(ps, x2, 1.0 / 39916800.0);
  ps = fma(ps, x2, -1.0 / 362880.0);
  ps = fma(ps, x2, 1.0 / 5040.0);
  ps = fma(ps, x2, -1.0 / 120.0);
  ps = fma(ps, x2, 1.0 / 6.0);
  const double sx = fma(-x * x2, ps, x);
  double pc = 1.0 / 6402373705728000.0;  // 1/18!
  pc = fma(pc, x2, -1.0 / 20922789888000.0);
  pc = fma(pc, x2, 1.0 / 87178291200.0);
  pc = fma(pc, x2, -1.0 / 479001600.0);
  pc = fma(pc, x2, 1.0 / 3628800.0);
  pc = fma(pc, x2, -1.0 / 40320.0);
  pc = fma(pc, x2, 1.0 / 720.0);
  pc = fma(pc, x2, -1.0 / 24.0);
  pc = fma(pc, x2, 0.5);
  const double cx = fma(-x2, pc, 1.0);
  // angle = q pi/2 + x: an odd quadrant swaps sin and cos; sin changes sign in quadrants 2
  // and 3, cos in quadrants 1 and 2 (sign-bit flips, no branches)
  const int qi = static_cast<int>(q) & 3;
  const bool odd = (qi & 1) != 0;
  const double sa = odd ? cx : sx, ca = odd ? sx : cx;
  const uint64_t fs = static_cast<uint64_t>(qi & 2) << 62, fc = static_cast<uint64_t>((qi + 1) & 2) << 62;
  s = __longlong_as_double(static_cast<long long>(static_cast<uint64_t>(__double_as_longlong(sa)) ^ fs));
  c = __longlong_as_double(static_cast<long long>(static_cast<uint64_t>(__double_as_longlong(ca)) ^ fc));
}

// log(n 2^-53) in fp64 for an integer n in [1, 2^53]: n = 2^e m with m in [sqrt(1/2),
// sqrt(2)) (exact), and log m = 2 atanh(s) with s = (m - 1) / (m + 1), |s| < 0.1716: the
// odd series of atanh to s^23 leaves a remainder below 1e-19; ln 2 in two parts.
__device__ __forceinline__ double log_u53(uint64_t n) {
  int e = 63 - __builtin_clzll(n);
  double m = static_cast<double>(n) * __builtin_ldexp(1.0, -e);
  if (m > 1.4142135623730951) {
    m *= 0.5;
    ++e;
  }
  const double sv = (m - 1.0) / (m + 1.0);
  const double s2 = sv * sv;
  double p = 1.0 / 23.0;
  p = fma(p, s2, 1.0 / 21.0);
  p = fma(p, s2, 1.0 / 19.0);
  p = fma(p, s2, 1.0 / 17.0);
  p = fma(p, s2, 1.0 / 15.0);
  p = fma(p, s2, 1.0 / 13.0);
  p = fma(p, s2, 1.0 / 11.0);
  p = fma(p, s2, 1.0 / 9.0);
  p = fma(p, s2, 1.0 / 7.0);
  p = fma(p, s2, 1.0 / 5.0);
  p = fma(p, s2, 1.0 / 3.0);
  const double lm = fma(2.0 * sv * s2, p, 2.0 * sv);
  const double k = static_cast<double>(e - 53);
  return fma(k, 0.6931471805599453, fma(k, 2.3190468138462996e-17, lm));
}

// Box and Muller (1958): two independent N(0,1) from two uniforms, in fp64, each rounded
// once to fp32. u1 = (a / 2^11 + 1) 2^-53 in (0,1], u2 = (b / 2^11) 2^-53 in [0,1).
__device__ __forceinline__ void box_muller(uint64_t a, uint64_t b, float& g0, float& g1) {
  const double rho = sqrt(-2.0 * log_u53((a >> 11) + 1));
  double s, c;
  sincos_2pi(static_cast<double>(b >> 11) * 0x1p-53, s, c);
  g0 = static_cast<float>(rho * c);
  g1 = static_cast<float>(rho * s);
}

// eps for experts 4q .. 4q+3 of token t; key (seed, key1).
__device__ __forceinline__ void noise4(uint64_t seed, uint64_t key1, int t, int q, float g[4]) {
  uint64_t c0 = static_cast<uint64_t>(t), c1 = static_cast<uint64_t>(q), c2 = 0, c3 = 0;
  philox4x64_10(c0, c1, c2, c3, seed, key1);
  box_muller(c0, c1, g[0], g[1]);
  box_muller(c2, c3, g[2], g[3]);
}

}  // namespace moe
