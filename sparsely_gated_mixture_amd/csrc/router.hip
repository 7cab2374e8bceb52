// Router: gate GEMM + noise + KeepTopK + softmax, one fused kernel.
//
// Noisy top-k gating: "Outrageously Large Neural Networks" summary, section
// 3.4, "Noisy Top-K Gating" Steps 1-3 (clean = X.Wg, std = Softplus(X.Wnoise),
// H = clean + N(0,1) * std, keep the k largest, softmax over the kept ones).
// Switch top-1: "Switch Transformer" explainer, "Implementation" steps 1-2
// (fp32 softmax over all experts, argmax first on ties, gate = that
// probability).
//
// Layout and work split
//   * The router weights are re-laid out per call (router_pack) into MFMA
//     fragment order: for every 32-column block and 16-deep (bf16) or 8-deep
//     (fp32) k-step, the 64 lanes' 16-byte operands are contiguous, so a wave
//     reads its B operand with one coalesced 1 KB load straight from L2.
//     Column blocks alternate clean / noise (2j: Wg experts 32j.., 2j+1: Wnoise
//     for the same experts), so a lane holds clean and raw of the same
//     (token, expert) in the same accumulator slot.
//   * bf16 X: each fp32 weight is split exactly into three bf16 pieces
//     (hi + mid + lo); X is exactly bf16, so every product is exact in fp32 and
//     three bf16 MFMAs accumulate the fp32 dot product. fp32 X: fp32 MFMA.
//   * A block owns 64 token rows and walks the experts in passes of 128 (one
//     32-expert block per wave). Per pass the X rows stream through LDS in
//     64-byte... 128-byte-wide k stages (double buffered), the accumulators go
//     through LDS to an epilogue that computes softplus, the Philox noise and
//     H, stores clean / std, and merges the pass's H values into a running
//     top-(k+1) list per row with wavefront arg-max rounds.
#include "common.h"

namespace moe {
namespace {

constexpr int kRows = 64;          // token rows per block
constexpr int kThreads = 256;      // 4 waves
constexpr int kExpPass = 128;      // experts per pass (32 per wave)
constexpr int kStageBytes = 128;   // bytes of one X row per k stage
constexpr int kAStride = 144;      // padded LDS row stride (bytes)
constexpr int kCStride = kExpPass + 4;
constexpr int kList = MOE_MAX_K + 1;
constexpr int kNone = 0x7fffffff;  // index of an empty / taken candidate

struct RouterArgs {
  const void* X;
  const uint4* wfrag;  // fragment-ordered router weights (workspace)
  const float* bias;
  const float* eps;
  int32_t* ids;
  float* gates;
  float* clean;
  float* std_out;
  float* row_stats;
  int* nonfinite;
  uint64_t seed;
  int T, D, E, k;
  int NB;      // 32-column blocks in wfrag (per piece)
  int KS;      // k-steps in wfrag (per column block)
  int use_noise;
  int switch_gate;
};

// ------------------------------------------------------------------ Philox4x64-10 + Box-Muller
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

// eps for experts 4q .. 4q+3 of token t.
__device__ __forceinline__ void noise4(uint64_t seed, int t, int q, float g[4]) {
  uint64_t c0 = static_cast<uint64_t>(t), c1 = static_cast<uint64_t>(q), c2 = 0, c3 = 0;
  philox4x64_10(c0, c1, c2, c3, seed, 0);
  box_muller(c0, c1, g[0], g[1]);
  box_muller(c2, c3, g[2], g[3]);
}

__device__ __forceinline__ float softplus(float z) {
  return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

// (value descending, index ascending) total order.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(i, off);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ------------------------------------------------------------------ weight re-layout
// One thread per (column block nb, k-step ks, lane). Column n of block nb is
// expert 32*(nb/2) + lane%32 of Wg (nb even) or Wnoise (nb odd) with noise,
// else expert 32*nb + lane%32 of Wg. k = ks*2V + (lane/32)*V + i. Zero padded.
template <bool kBf16>
__global__ void router_pack(const float* __restrict__ Wg, const float* __restrict__ Wn,
                            int D, int E, int with_noise, int NB, int KS,
                            uint4* __restrict__ out) {
  constexpr int V = kBf16 ? 8 : 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(NB) * KS * kWave;
  if (idx >= total) return;
  const int lane = static_cast<int>(idx % kWave);
  const int ks = static_cast<int>((idx / kWave) % KS);
  const int nb = static_cast<int>(idx / (static_cast<int64_t>(kWave) * KS));
  const int eb = with_noise ? (nb >> 1) : nb;
  const float* W = (with_noise && (nb & 1)) ? Wn : Wg;
  const int e = eb * 32 + (lane & 31);
  const int k0 = ks * 2 * V + (lane >> 5) * V;
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int kk = k0 + i;
    v[i] = (e < E && kk < D) ? W[static_cast<int64_t>(kk) * E + e] : 0.f;
  }
  const int64_t slot = (static_cast<int64_t>(nb) * KS + ks) * kWave + lane;
  if constexpr (kBf16) {
    uint16_t hi[8], mid[8], lo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hi[i] = f32_to_bf16(v[i]);
      const float r1 = v[i] - bf16_to_f32(hi[i]);
      mid[i] = f32_to_bf16(r1);
      const float r2 = r1 - bf16_to_f32(mid[i]);
      lo[i] = f32_to_bf16(r2);
    }
    const int64_t piece = static_cast<int64_t>(NB) * KS * kWave;
    out[slot] = *reinterpret_cast<const uint4*>(hi);
    out[slot + piece] = *reinterpret_cast<const uint4*>(mid);
    out[slot + 2 * piece] = *reinterpret_cast<const uint4*>(lo);
  } else {
    out[slot] = *reinterpret_cast<const uint4*>(v);
  }
}

// ------------------------------------------------------------------ fused router
template <typename XT>
__global__ __launch_bounds__(kThreads) void router_kernel(RouterArgs a) {
  constexpr bool kBf16 = sizeof(XT) == 2;
  constexpr int V = Elem<XT>::kVec;
  constexpr int kPieces = kBf16 ? 3 : 1;
  constexpr int kStageElems = kStageBytes / static_cast<int>(sizeof(XT));

  __shared__ __align__(16) unsigned char sA[2][kRows * kAStride];
  __shared__ __align__(16) float sC[2][kRows][kCStride];
  __shared__ float sLv[kRows][kList];
  __shared__ int sLi[kRows][kList];
  __shared__ float sM[kRows], sS[kRows];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * kRows;
  const int T = a.T, D = a.D, E = a.E, K = a.k + 1;
  const int ncol = a.use_noise ? 2 : 1;   // column blocks per expert block
  const int EB = (E + 31) / 32;           // expert blocks
  const int npass = (EB + 3) / 4;
  const int kstages = a.KS / 4;           // 4 k-steps per stage
  const int64_t piece_stride = static_cast<int64_t>(a.NB) * a.KS * kWave;
  const XT* X = static_cast<const XT*>(a.X);
  const bool vec_ok = (D % V) == 0;
  const bool check = a.nonfinite != nullptr;

  for (int r = tid; r < kRows; r += kThreads) {
    sM[r] = -INFINITY;
    sS[r] = 0.f;
  }

  // X stage loader: 64 rows x 128 B = 512 16-byte chunks, 2 per thread.
  auto load_stage = [&](int st, uint4 regs[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 3, seg = c & 7;
      const int t = min(row0 + r, T - 1);
      regs[i] = load_row16<XT>(X + static_cast<int64_t>(t) * D, st * kStageElems + seg * V, D, vec_ok);
    }
  };
  auto store_stage = [&](int buf, const uint4 regs[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 3, seg = c & 7;
      *reinterpret_cast<uint4*>(&sA[buf][r * kAStride + seg * 16]) = regs[i];
    }
  };

  for (int pass = 0; pass < npass; ++pass) {
    const int eb = pass * 4 + wave;
    const bool active = eb < EB;
    f32x16 acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][c][i] = 0.f;

    uint4 regs[2];
    load_stage(0, regs);
    __syncthreads();  // previous pass finished with sA / sC
    store_stage(0, regs);
    __syncthreads();
    for (int st = 0; st < kstages; ++st) {
      const int buf = st & 1;
      if (st + 1 < kstages) load_stage(st + 1, regs);
      if (active) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kg = st * 4 + ks;
          uint4 af[2];
#pragma unroll
          for (int m = 0; m < 2; ++m)
            af[m] = *reinterpret_cast<const uint4*>(
                &sA[buf][(m * 32 + (lane & 31)) * kAStride + ks * 32 + (lane >> 5) * 16]);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            if (c < ncol) {
              const int nb = eb * ncol + c;
              const int64_t slot = (static_cast<int64_t>(nb) * a.KS + kg) * kWave + lane;
#pragma unroll
              for (int pc = 0; pc < kPieces; ++pc) {
                const uint4 bf = a.wfrag[slot + pc * piece_stride];
#pragma unroll
                for (int m = 0; m < 2; ++m) acc[m][c] = mfma_step<XT>(af[m], bf, acc[m][c]);
              }
            }
          }
        }
      }
      if (st + 1 < kstages) store_stage(buf ^ 1, regs);
      __syncthreads();
    }

    // accumulators -> LDS (row, expert-in-pass)
    if (active) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (c < ncol) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              sC[c][m * 32 + acc_row(lane, i)][wave * 32 + (lane & 31)] = acc[m][c][i];
        }
      }
    }
    __syncthreads();

    // epilogue: (row, 4 experts) items -> clean, std, eps, H
    for (int it = tid; it < kRows * (kExpPass / 4); it += kThreads) {
      const int r = it >> 5, g = it & 31;
      const int t = row0 + r;
      const int e0 = pass * kExpPass + 4 * g;
      if (t >= T || e0 >= E) continue;
      float cl[4], sd[4] = {0.f, 0.f, 0.f, 0.f}, ep[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cl[i] = sC[0][r][4 * g + i];
        if (a.bias && e0 + i < E) cl[i] += a.bias[e0 + i];
      }
      const int64_t base = static_cast<int64_t>(t) * E + e0;
      const bool full4 = (E % 4 == 0);
      bool bad = false;
      if (a.use_noise) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float raw = sC[1][r][4 * g + i];
          bad |= !isfinite(raw);
          sd[i] = softplus(raw);
        }
        if (a.eps) {
#pragma unroll
          for (int i = 0; i < 4; ++i) ep[i] = (e0 + i < E) ? a.eps[base + i] : 0.f;
        } else {
          noise4(a.seed, t, e0 >> 2, ep);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) bad |= !isfinite(cl[i]);
      if (check) note_nonfinite(a.nonfinite, bad);
      if (full4) {
        *reinterpret_cast<float4*>(a.clean + base) = make_float4(cl[0], cl[1], cl[2], cl[3]);
        if (a.use_noise)
          *reinterpret_cast<float4*>(a.std_out + base) = make_float4(sd[0], sd[1], sd[2], sd[3]);
      } else {
        for (int i = 0; i < 4 && e0 + i < E; ++i) {
          a.clean[base + i] = cl[i];
          if (a.use_noise) a.std_out[base + i] = sd[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sC[0][r][4 * g + i] = a.use_noise ? fmaf(sd[i], ep[i], cl[i]) : cl[i];
    }
    __syncthreads();

    // merge this pass's scores into each row's running top-(k+1) list
    for (int rr = 0; rr < kRows / 4; ++rr) {
      const int r = wave * (kRows / 4) + rr;
      if (row0 + r >= T) break;
      float v[3];
      int ix[3];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = pass * kExpPass + lane + 64 * h;
        const float s = sC[0][r][lane + 64 * h];
        const bool ok = e < E && !isnan(s);
        v[h] = ok ? s : -INFINITY;
        ix[h] = ok ? e : kNone;
      }
      if (pass > 0 && lane < K) {
        v[2] = sLv[r][lane];
        ix[2] = sLi[r][lane];
      } else {
        v[2] = -INFINITY;
        ix[2] = kNone;
      }
      if (a.switch_gate) {  // online softmax statistics of the row
        const float cm = wave_max(fmaxf(v[0], v[1]));
        const float cs = wave_sum((ix[0] != kNone ? expf(v[0] - cm) : 0.f) +
                                  (ix[1] != kNone ? expf(v[1] - cm) : 0.f));
        if (lane == 0) {
          const float m0 = sM[r], s0 = sS[r];
          const float mn = fmaxf(m0, cm);
          sS[r] = (m0 == -INFINITY ? 0.f : s0 * expf(m0 - mn)) + cs * expf(cm - mn);
          sM[r] = mn;
        }
      }
      float keep_v = -INFINITY;
      int keep_i = kNone;
      for (int s = 0; s < K; ++s) {
        int bsel = 0;
        if (better(v[1], ix[1], v[bsel], ix[bsel])) bsel = 1;
        if (better(v[2], ix[2], v[bsel], ix[bsel])) bsel = 2;
        float bv = v[bsel];
        int bi = ix[bsel];
        wave_argmax(bv, bi);
        if (bi != kNone) {
#pragma unroll
          for (int h = 0; h < 3; ++h)
            if (ix[h] == bi) {
              v[h] = -INFINITY;
              ix[h] = kNone;
            }
        }
        if (lane == s) {
          keep_v = bv;
          keep_i = bi;
        }
      }
      if (lane < K) {
        sLv[r][lane] = keep_v;
        sLi[r][lane] = keep_i;
      }
    }
    __syncthreads();
  }

  // final outputs per row
  for (int rr = 0; rr < kRows / 4; ++rr) {
    const int r = wave * (kRows / 4) + rr;
    const int t = row0 + r;
    if (t >= T) break;
    const int k = a.k;
    const float v0 = sLv[r][0];
    const float vj = lane < k ? sLv[r][lane] : -INFINITY;
    float g;
    if (a.switch_gate) {
      g = expf(vj - sM[r]) / sS[r];
    } else {
      const float ej = lane < k ? expf(vj - v0) : 0.f;
      g = ej / wave_sum(ej);
    }
    if (lane < k) {
      a.ids[static_cast<int64_t>(t) * k + lane] = sLi[r][lane];
      a.gates[static_cast<int64_t>(t) * k + lane] = g;
    }
    if (a.row_stats && lane == 0) {
      a.row_stats[2 * static_cast<int64_t>(t)] = sLv[r][k - 1];
      a.row_stats[2 * static_cast<int64_t>(t) + 1] = sLv[r][k];
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ host side
static int router_ks(const Dims& d) {
  const int stage = d.dtype == MOE_BF16 ? 64 : 32;  // elements per 128-byte stage
  return ceil_div(d.D, stage) * 4;
}
static int router_nb(const Dims& d) {
  const bool noise = d.gating == MOE_GATE_NOISY_TOPK && d.noise;
  return ceil_div(d.E, 32) * (noise ? 2 : 1);
}

size_t route_workspace(const Dims& d) {
  const size_t pieces = d.dtype == MOE_BF16 ? 3 : 1;
  return align256(pieces * router_nb(d) * static_cast<size_t>(router_ks(d)) * kWave * 16);
}

moe_status route_launch(const Dims& d, const moe_problem* p, const void* X, const float* Wg,
                        const float* Wnoise, const float* bias, const float* eps, int32_t* ids,
                        float* gates, float* clean, float* noise_std, float* row_stats,
                        void* ws, int* nonfinite, hipStream_t stream) {
  const bool noise = d.gating == MOE_GATE_NOISY_TOPK && d.noise;
  const int NB = router_nb(d), KS = router_ks(d);
  uint4* wfrag = static_cast<uint4*>(ws);
  const int64_t items = static_cast<int64_t>(NB) * KS * kWave;
  const int pb = 256;
  const int pgrid = static_cast<int>(ceil_div64(items, pb));
  if (d.dtype == MOE_BF16)
    router_pack<true><<<pgrid, pb, 0, stream>>>(Wg, noise ? Wnoise : nullptr, d.D, d.E, noise, NB, KS, wfrag);
  else
    router_pack<false><<<pgrid, pb, 0, stream>>>(Wg, noise ? Wnoise : nullptr, d.D, d.E, noise, NB, KS, wfrag);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;

  RouterArgs a;
  a.X = X;
  a.wfrag = wfrag;
  a.bias = bias;
  a.eps = noise ? eps : nullptr;
  a.ids = ids;
  a.gates = gates;
  a.clean = clean;
  a.std_out = noise ? noise_std : nullptr;
  a.row_stats = row_stats;
  a.nonfinite = nonfinite;
  a.seed = p->seed;
  a.T = d.T;
  a.D = d.D;
  a.E = d.E;
  a.k = d.k;
  a.NB = NB;
  a.KS = KS;
  a.use_noise = noise ? 1 : 0;
  a.switch_gate = d.gating == MOE_GATE_SWITCH_TOP1 ? 1 : 0;
  const int grid = ceil_div(d.T, kRows);
  if (d.dtype == MOE_BF16)
    router_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(a);
  else
    router_kernel<float><<<grid, kThreads, 0, stream>>>(a);
  return launch_status();
}

}  // namespace moe
