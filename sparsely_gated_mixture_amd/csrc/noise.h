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

// Box and Muller (1958): two independent N(0,1) from two uniforms, in fp64,
// each rounded once to fp32. u1 in (0,1], u2 in [0,1).
__device__ __forceinline__ void box_muller(uint64_t a, uint64_t b, float& g0, float& g1) {
  const double u1 = (static_cast<double>(a >> 11) + 1.0) * 0x1p-53;
  const double u2 = static_cast<double>(b >> 11) * 0x1p-53;
  const double rho = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586 * u2;
  double s, c;
  sincos(th, &s, &c);
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
