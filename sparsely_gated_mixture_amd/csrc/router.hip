// Router: gate GEMM + noise + KeepTopK + softmax.
//
// Noisy top-k gating: "Outrageously Large Neural Networks" summary, section
// 3.4, "Noisy Top-K Gating" Steps 1-3 (clean = X.Wg, std = Softplus(X.Wnoise),
// H = clean + N(0,1) * std, keep the k largest, softmax over the kept ones).
// Switch top-1: "Switch Transformer" explainer, "Implementation" steps 1-2
// (fp32 softmax over all experts, argmax first on ties, gate = that
// probability).
//
// Three launches:
//   router_pack    re-lays Wg / Wnoise into MFMA fragment order (per call; a
//                  few microseconds). Column blocks alternate clean / noise
//                  for the same 32 experts, so a wave's two accumulators hold
//                  clean and raw of the same (token, expert). For bf16 X each
//                  fp32 weight is split exactly into three bf16 pieces
//                  (hi + mid + lo): X is exactly bf16, every product is exact
//                  in fp32, and three bf16 MFMAs accumulate the fp32 dot
//                  product. fp32 X uses fp32 MFMA.
//   router_gemm    128 tokens x 256 weight columns per block, the grouped
//                  GEMM's pipeline (X through double-buffered LDS, B fragments
//                  streamed into registers). Epilogue through a wave-private
//                  LDS tile: per (token, 4 experts) one Philox call gives the
//                  four noise samples; writes clean, std and the score H.
//   router_select  8-64 lanes per token row: per-lane sorted top-K lists
//                  (K = next power of two >= k+1) merged by a bitonic
//                  butterfly; writes ids, gates, row_stats. Switch also sums
//                  exp(logit - max) for its gate.
#include <algorithm>

#include "common.h"
#include "noise.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 256;          // weight columns per block (8 blocks of 32)
constexpr int kAStride = 144;     // padded LDS row stride (bytes)
constexpr int kTS = 36;           // epilogue tile row stride (floats)
constexpr int kXcds = 8;
constexpr int kNone = 0x7fffffff; // index of an empty / taken candidate

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mma<uint16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mma<float>(u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s]), __uint_as_float(b[s]), c, 0, 0, 0);
  return c;
}

struct GemmArgs {
  const void* X;
  const u32x4* wfrag;  // fragment-ordered router weights (workspace)
  const float* bias;
  const float* eps;
  float* clean;
  float* std_out;
  float* H;            // noisy scores (workspace); unused without noise
  int* nonfinite;
  uint64_t seed;
  int T, D, E;
  int NB;              // 32-column blocks in wfrag (per piece)
  int KS;              // k-steps per column block (multiple of 4)
  int use_noise;
  int vec_out;         // E % 4 == 0 and the outputs 16-byte aligned: float4 stores
  // grouped mode (secondary gates of a hierarchical MoE): rows offsets goff[g] ..
  // goff[g+1]-1 belong to group g, hold token row_token[r], use group g's weights
  // (wfrag + g * wgroup) and draw noise from key (seed, 1 + g)
  const int32_t* goff;
  const int32_t* row_token;
  int G;
  int64_t wgroup;
};

struct SelectArgs {
  const float* score;  // H (noisy) or clean
  int32_t* ids;
  float* gates;
  float* row_stats;
  int T, E, k, switch_gate;
  int vec;             // E % 4 == 0 and score 16-byte aligned: float4 reads
};
// softplus(z) = max(z, 0) + log1p(e^-|z|) with the hardware base-2 exponential and logarithm
// (about 1 ulp each) in place of the library's expf / log1pf: u = e^-|z|, w = 1 + u rounded,
// and log1p(u) = ln w - ((w - 1) - u) / w, where the second term is the rounding error of
// 1 + u (w - 1 is exact), so small u keeps its full precision (for u below half an ulp of 1,
// w = 1 and the result is u). Over |z| <= 40 the largest absolute error equals the library
// form's (4.8e-7, the rounding of the result near 40); the relative error stays below 2e-6
// where softplus is tiny (the rounding of |z| log2 e in the exponent), which moves the
// scores H = clean + eps * softplus by far less than their own rounding.
__device__ __forceinline__ float softplus(float z) {
  const float u = __builtin_amdgcn_exp2f(-fabsf(z) * 1.44269504088896341f);
  const float w = 1.f + u;
  const float lw = __builtin_amdgcn_logf(w) * 0.693147180559945309f;
  return fmaxf(z, 0.f) + (lw - ((w - 1.f) - u) * __builtin_amdgcn_rcpf(w));
}

// (value descending, index ascending) total order.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// ------------------------------------------------------------------ weight re-layout
// One thread per (column block nb, k-step ks, lane). Column n of block nb is
// expert 32*(nb/2) + lane%32 of Wg (nb even) or Wnoise (nb odd) with noise,
// else expert 32*nb + lane%32 of Wg. k = ks*2V + (lane/32)*V + i. Zero padded.
// blockIdx.y selects a gate of a stack (weights wstride floats apart, packed outputs
// ostride uint4 apart): the secondary gates of a hierarchical MoE.
template <bool kBf16>
__global__ void router_pack(const float* __restrict__ Wg, const float* __restrict__ Wn,
                            int D, int E, int with_noise, int NB, int KS,
                            uint4* __restrict__ out, int64_t wstride, int64_t ostride) {
  constexpr int V = kBf16 ? 8 : 4;
  Wg += blockIdx.y * wstride;
  if (Wn) Wn += blockIdx.y * wstride;
  out += blockIdx.y * ostride;
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

// ------------------------------------------------------------------ router GEMM + epilogue
// BM token rows per block (128, or 64 / 32 when T is small). kGrouped: rows grouped by
// gate (tile table from goff in dynamic LDS, G + 1 ints).
// kNoiseWaves (noise drawn here, 128-row tiles, not grouped): the block has 8 waves. Waves
// 0-3 compute the tile as in the 4-wave form; wave 4 + w shares a SIMD with wave w and, while
// wave w runs its MFMAs, draws the Gaussian noise its epilogue will need into an LDS tile, in
// the order that epilogue reads it (one (token, 4 experts) group a lane per k-stage at
// D = 1024). The noise is then vector-ALU work of a second wave beside the MFMAs instead of
// work after them: on this chip the two overlap when they come from different waves.
constexpr int kNoiseGroups = 16;  // noise groups a lane of a noise wave draws per tile
template <typename XT, bool kFullK, int BM, bool kGrouped, bool kNoiseWaves = false>
__global__ __launch_bounds__(kNoiseWaves ? 2 * kThreads : kThreads, kNoiseWaves ? 1 : 2)
void router_gemm(GemmArgs a) {
  static_assert(!kNoiseWaves || (BM == 128 && !kGrouped), "noise waves: 128-row tiles, flat gate");
  constexpr int V = Elem<XT>::kVec;
  constexpr int kPieces = sizeof(XT) == 2 ? 3 : 1;
  constexpr int kStageElems = 128 / static_cast<int>(sizeof(XT));
  constexpr int MB = BM / 32;
  constexpr int kChunks = BM * 8 / kThreads;
  // one A stage buffer; the two together also hold the epilogue tiles [4 waves][2][32][kTS]
  constexpr int kEpiHalf = (kThreads / 64) * 2 * 32 * kTS * 4 / 2;
  constexpr int kStage = BM * kAStride > kEpiHalf ? BM * kAStride : kEpiHalf;

  __shared__ __align__(16) unsigned char sA[2][kStage];
  extern __shared__ int sCum[];  // grouped: G + 1 running row-tile counts
  // noise tile: [MFMA wave w][32-row block m][pass h][lane] float4, the epilogue's order
  __shared__ __align__(16) float4 sE[kNoiseWaves ? (kThreads / 64) * MB * 4 * 64 : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int T = a.T, D = a.D, E = a.E;
  const int ntiles = (a.NB + 7) / 8;
  int g = 0, m_tile, n_tile, r0, rows;
  if constexpr (kGrouped) {
    const int G = a.G;
    const int per = (G + kThreads - 1) / kThreads;
    const int g0 = tid * per, g1 = min(G, g0 + per);
    int s = 0;
    for (int q = g0; q < g1; ++q) s += (a.goff[q + 1] - a.goff[q] + BM - 1) / BM;
    int excl;
    __shared__ int wt[kThreads / 64];
    const int tot = block_exclusive_scan<kThreads>(s, &excl, wt);
    for (int q = g0; q < g1; ++q) {
      sCum[q] = excl;
      excl += (a.goff[q + 1] - a.goff[q] + BM - 1) / BM;
    }
    if (tid == 0) sCum[G] = tot;
    __syncthreads();
    const int total = sCum[G] * ntiles;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int local = blockIdx.x / kXcds;
    if (local >= per_xcd) return;
    const int logical = (blockIdx.x % kXcds) * per_xcd + local;
    if (logical >= total) return;
    const int q = logical / ntiles;  // group-major, then column tile, then row tile
    int lo = 0, hi = G;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sCum[mid] > q) hi = mid; else lo = mid + 1;
    }
    g = lo - 1;
    const int mt = sCum[g + 1] - sCum[g];
    const int loc = logical - sCum[g] * ntiles;
    n_tile = loc / mt;
    m_tile = loc - n_tile * mt;
    r0 = a.goff[g] + m_tile * BM;
    rows = min(BM, a.goff[g + 1] - r0);
  } else {
    const int mtiles = (T + BM - 1) / BM;
    const int total = mtiles * ntiles;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int local = blockIdx.x / kXcds;
    if (local >= per_xcd) return;
    const int logical = (blockIdx.x % kXcds) * per_xcd + local;
    if (logical >= total) return;
    m_tile = logical / ntiles;
    n_tile = logical - m_tile * ntiles;
    r0 = m_tile * BM;
    rows = min(BM, T - r0);
  }
  const int nst = a.KS / 4;

  if constexpr (kNoiseWaves) {
    if (wave >= kThreads / 64) {
      // noise wave: the groups MFMA wave w = wave - 4 reads in its epilogue (32 experts of
      // block n_tile * 4 + w, 128 rows), spread over the k-stages, one barrier a stage as
      // the MFMA waves have (their prologue's and every stage's)
      const int w = wave - kThreads / 64;
      const int eb = n_tile * 4 + w;
      auto draw = [&](int gi) {  // gi = 4 m + h
        const int m = gi >> 2, h = gi & 3;
        const int it = lane + 64 * h;
        const int row = it >> 3, g4 = it & 7;
        const int e0 = eb * 32 + 4 * g4;
        if (m * 32 + row >= rows || e0 >= E) return;
        float ep[4];
        noise4(a.seed, 0, r0 + m * 32 + row, e0 >> 2, ep);
        sE[((w * MB + m) * 4 + h) * 64 + lane] = make_float4(ep[0], ep[1], ep[2], ep[3]);
      };
      __syncthreads();
      for (int st = 0; st < nst; ++st) {
        for (int gi = st * kNoiseGroups / nst; gi < (st + 1) * kNoiseGroups / nst; ++gi) draw(gi);
        __syncthreads();
      }
      return;
    }
  }

  const XT* X = static_cast<const XT*>(a.X);
  const int aseg = tid & 7, arow0 = tid >> 3;
  const bool vec_ok = (D % V) == 0;
  u32x4 areg[kChunks];
  int64_t asrc[kChunks];  // X row of each chunk (the row's token when grouped)
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int r = r0 + min(arow0 + i * (kThreads / 8), rows - 1);
    asrc[i] = static_cast<int64_t>(kGrouped ? a.row_token[r] : r) * D;
  }
  auto load_a = [&](int st) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const XT* row = X + asrc[i];
      if constexpr (kFullK) {
        areg[i] = *reinterpret_cast<const u32x4*>(row + st * kStageElems + aseg * V);
      } else {
        const uint4 v = load_row16<XT>(row, st * kStageElems + aseg * V, D, vec_ok);
        areg[i] = u32x4{v.x, v.y, v.z, v.w};
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      *reinterpret_cast<u32x4*>(&sA[buf][(arow0 + i * (kThreads / 8)) * kAStride + aseg * 16]) = areg[i];
  };

  // wave's two column blocks (clean, raw of one 32-expert block with noise; two clean
  // blocks without); blocks past NB read a valid block and are never stored
  const int cb0 = n_tile * 8 + wave * 2;
  const int64_t piece = static_cast<int64_t>(a.NB) * a.KS * kWave;
  const u32x4* wf = a.wfrag + (kGrouped ? g * a.wgroup : 0);
  const u32x4* W0 = wf + static_cast<int64_t>(min(cb0, a.NB - 1)) * a.KS * kWave + lane;
  const u32x4* W1 = wf + static_cast<int64_t>(min(cb0 + 1, a.NB - 1)) * a.KS * kWave + lane;

  f32x16 acc[MB][2];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][j][i] = 0.f;

  const int arow = (lane & 31) * kAStride + (lane >> 5) * 16;
  // B ring: two k-steps ahead
  u32x4 bq[2][kPieces][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      bq[s][p][0] = W0[p * piece + s * kWave];
      bq[s][p][1] = W1[p * piece + s * kWave];
    }
  load_a(0);
  store_a(0);
  __syncthreads();

  const int nks = a.KS;
  u32x4 af[2][MB];
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    load_a(min(st + 1, nst - 1));
#pragma unroll
    for (int m = 0; m < MB; ++m)
      af[0][m] = *reinterpret_cast<const u32x4*>(&sA[buf][m * 32 * kAStride + arow]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
          af[(ks + 1) & 1][m] =
              *reinterpret_cast<const u32x4*>(&sA[buf][m * 32 * kAStride + (ks + 1) * 32 + arow]);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int p = 0; p < kPieces; ++p)
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          acc[m][0] = mma<XT>(af[ks & 1][m], bq[ks & 1][p][0], acc[m][0]);
          acc[m][1] = mma<XT>(af[ks & 1][m], bq[ks & 1][p][1], acc[m][1]);
        }
      __builtin_amdgcn_s_setprio(0);
      const int64_t kn = static_cast<int64_t>(min(st * 4 + ks + 2, nks - 1)) * kWave;
#pragma unroll
      for (int p = 0; p < kPieces; ++p) {
        bq[ks & 1][p][0] = W0[p * piece + kn];
        bq[ks & 1][p][1] = W1[p * piece + kn];
      }
    }
    store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue, one 32-row block at a time through a wave-private LDS tile [2][32][kTS]
  float* Ts = reinterpret_cast<float*>(&sA[0][0]) + wave * (2 * 32 * kTS);
  const bool check = a.nonfinite != nullptr;
  const bool full4 = a.vec_out != 0;
  const uint64_t key1 = kGrouped ? static_cast<uint64_t>(1 + g) : 0;
  bool bad = false;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) Ts[(c * 32 + acc_row(lane, i)) * kTS + (lane & 31)] = acc[m][c][i];
    if (a.use_noise) {
      // experts of this wave: one 32-expert block, clean in Ts[0], raw in Ts[1]
      const int eb = n_tile * 4 + wave;
#pragma unroll 1
      for (int h = 0; h < 4; ++h) {
        const int it = lane + 64 * h;
        const int row = it >> 3, g4 = it & 7;
        const int t = r0 + m * 32 + row;
        const int e0 = eb * 32 + 4 * g4;
        if (m * 32 + row >= rows || e0 >= E) continue;
        float cl[4], sd[4], ep[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cl[i] = Ts[row * kTS + 4 * g4 + i];
          if (a.bias && e0 + i < E) cl[i] += a.bias[e0 + i];
          const float raw = Ts[(32 + row) * kTS + 4 * g4 + i];
          bad |= (e0 + i < E) && !(isfinite(raw) && isfinite(cl[i]));
          sd[i] = softplus(raw);
        }
        const int64_t base = static_cast<int64_t>(t) * E + e0;
        if constexpr (kNoiseWaves) {
          const float4 e4 = sE[((wave * MB + m) * 4 + h) * 64 + lane];
          ep[0] = e4.x;
          ep[1] = e4.y;
          ep[2] = e4.z;
          ep[3] = e4.w;
        } else if (a.eps) {
#pragma unroll
          for (int i = 0; i < 4; ++i) ep[i] = (e0 + i < E) ? a.eps[base + i] : 0.f;
        } else {
          noise4(a.seed, key1, kGrouped ? a.row_token[t] : t, e0 >> 2, ep);
        }
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = fmaf(sd[i], ep[i], cl[i]);
        if (full4) {
          *reinterpret_cast<float4*>(a.clean + base) = make_float4(cl[0], cl[1], cl[2], cl[3]);
          *reinterpret_cast<float4*>(a.std_out + base) = make_float4(sd[0], sd[1], sd[2], sd[3]);
          *reinterpret_cast<float4*>(a.H + base) = make_float4(hv[0], hv[1], hv[2], hv[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (e0 + i < E) {
              a.clean[base + i] = cl[i];
              a.std_out[base + i] = sd[i];
              a.H[base + i] = hv[i];
            }
        }
      }
    } else {
      // experts of this wave: two consecutive 32-expert blocks, both clean
#pragma unroll 1
      for (int h = 0; h < 8; ++h) {
        const int it = lane + 64 * h;
        const int row = it >> 4, g = it & 15;
        const int c = g >> 3, g4 = g & 7;
        const int t = r0 + m * 32 + row;
        const int e0 = (cb0 + c) * 32 + 4 * g4;
        if (m * 32 + row >= rows || e0 >= E) continue;
        float cl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cl[i] = Ts[(c * 32 + row) * kTS + 4 * g4 + i];
          if (a.bias && e0 + i < E) cl[i] += a.bias[e0 + i];
          bad |= (e0 + i < E) && !isfinite(cl[i]);
        }
        const int64_t base = static_cast<int64_t>(t) * E + e0;
        if (full4) {
          *reinterpret_cast<float4*>(a.clean + base) = make_float4(cl[0], cl[1], cl[2], cl[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (e0 + i < E) a.clean[base + i] = cl[i];
        }
      }
    }
  }
  if (check) note_nonfinite(a.nonfinite, bad);
}

// ------------------------------------------------------------------ row selection
// Candidates compare by (score descending, index ascending): a total order, so the
// selected set and its order are unique. NaN scores never win.
template <int KL>
__device__ __forceinline__ void list_insert(float (&v)[KL], int (&ix)[KL], float x, int i) {
  if (!better(x, i, v[KL - 1], ix[KL - 1])) return;
  v[KL - 1] = x;
  ix[KL - 1] = i;
#pragma unroll
  for (int j = KL - 1; j > 0; --j) {
    if (better(v[j], ix[j], v[j - 1], ix[j - 1])) {
      const float tv = v[j];
      v[j] = v[j - 1];
      v[j - 1] = tv;
      const int ti = ix[j];
      ix[j] = ix[j - 1];
      ix[j - 1] = ti;
    }
  }
}

// Merge the sorted list with the partner lane's (xor off): the elementwise best of
// a[j] and b[KL-1-j] is the top KL of the union as a bitonic sequence, which a
// bitonic network then sorts.
template <int KL>
__device__ __forceinline__ void list_merge(float (&v)[KL], int (&ix)[KL], int off) {
  float pv[KL];
  int pi[KL];
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    pv[j] = __shfl_xor(v[j], off);
    pi[j] = __shfl_xor(ix[j], off);
  }
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    const float bv = pv[KL - 1 - j];
    const int bi = pi[KL - 1 - j];
    if (better(bv, bi, v[j], ix[j])) {
      v[j] = bv;
      ix[j] = bi;
    }
  }
#pragma unroll
  for (int w = KL / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int j = 0; j < KL; ++j)
      if ((j & w) == 0 && better(v[j + w], ix[j + w], v[j], ix[j])) {
        const float tv = v[j];
        v[j] = v[j + w];
        v[j + w] = tv;
        const int ti = ix[j];
        ix[j] = ix[j + w];
        ix[j + w] = ti;
      }
}

// LPR lanes per token row (a power of two, 8..64, within one wave).
template <int KL, int LPR>
__global__ __launch_bounds__(kThreads) void router_select(SelectArgs a) {
  const int tid = threadIdx.x;
  const int sub = tid & (LPR - 1);               // lane within the row group
  const int t = blockIdx.x * (kThreads / LPR) + tid / LPR;
  const bool live = t < a.T;
  const int E = a.E, k = a.k;
  const float* row = a.score + static_cast<int64_t>(live ? t : 0) * E;
  float v[KL];
  int ix[KL];
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    v[j] = -INFINITY;
    ix[j] = kNone;
  }
  if (live) {
    if (a.vec) {
      // lane sub reads 16 bytes at 4*sub (+ 4*LPR): the row group reads 16*LPR contiguous
      // bytes per load
      for (int e0 = 4 * sub; e0 < E; e0 += 8 * LPR) {
        const float4 x0 = *reinterpret_cast<const float4*>(row + e0);
        const bool two = e0 + 4 * LPR < E;
        const float4 x1 = two ? *reinterpret_cast<const float4*>(row + e0 + 4 * LPR)
                              : make_float4(NAN, NAN, NAN, NAN);
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (!isnan(xs[i])) list_insert<KL>(v, ix, xs[i], e0 + (i & 3) + 4 * LPR * (i >> 2));
      }
    } else {
      for (int e = sub; e < E; e += LPR) {
        const float x = row[e];
        if (!isnan(x)) list_insert<KL>(v, ix, x, e);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) list_merge<KL>(v, ix, off);
  // every lane of the group now holds the row's top KL
  float gsum = 0.f;
  if (a.switch_gate) {
    float s = 0.f;
    if (live)
      for (int e = sub; e < E; e += LPR) {
        const float x = row[e];
        if (!isnan(x)) s += expf(x - v[0]);
      }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
    gsum = s;
  } else {
#pragma unroll
    for (int j = 0; j < KL; ++j)
      if (j < k) gsum += expf(v[j] - v[0]);
  }
  if (!live) return;
  const int64_t o = static_cast<int64_t>(t) * k;
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    if (j < k && (j & (LPR - 1)) == sub) {
      a.ids[o + j] = ix[j];
      a.gates[o + j] = a.switch_gate ? expf(v[j] - v[0]) / gsum : expf(v[j] - v[0]) / gsum;
    }
  }
  if (a.row_stats && sub == 0) {
    float vk = v[0], vk1 = -INFINITY;
#pragma unroll
    for (int j = 0; j < KL; ++j) {
      if (j == k - 1) vk = v[j];
      if (j == k) vk1 = v[j];
    }
    a.row_stats[2 * static_cast<int64_t>(t)] = vk;
    a.row_stats[2 * static_cast<int64_t>(t) + 1] = vk1;
  }
}

}  // namespace

// ------------------------------------------------------------------ host side
static int router_ks(const Dims& d) {
  const int stage = d.dtype == MOE_BF16 ? 64 : 32;  // elements per 128-byte stage
  return ceil_div(d.D, stage) * 4;
}
static bool router_noise(const Dims& d) { return d.gating == MOE_GATE_NOISY_TOPK && d.noise; }
static int router_nb(const Dims& d) { return ceil_div(d.E, 32) * (router_noise(d) ? 2 : 1); }
static size_t router_wbytes(const Dims& d) {
  const size_t pieces = d.dtype == MOE_BF16 ? 3 : 1;
  return align256(pieces * router_nb(d) * static_cast<size_t>(router_ks(d)) * kWave * 16);
}

// 128-row tiles, or 64 / 32 while that leaves fewer than 512 blocks
static int router_bm(int64_t rows, int NB) {
  int bm = 128;
  while (bm > 32 && ceil_div64(rows, bm) * ceil_div(NB, 8) < 512) bm >>= 1;
  return bm;
}
static int vec_outputs(int E, const float* a, const float* b, const float* c) {
  const uintptr_t m = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                      reinterpret_cast<uintptr_t>(c);
  return (E % 4 == 0 && m % 16 == 0) ? 1 : 0;
}

size_t route_workspace(const Dims& d) {
  size_t b = router_wbytes(d);
  if (router_noise(d)) b += align256(static_cast<size_t>(d.T) * d.E * sizeof(float));
  return b;
}

// The noisy scores H [T,E] that the selection used: after the packed weights in the route
// workspace (NULL without noise).
const float* route_scores(const Dims& d, const void* ws) {
  if (!router_noise(d) || !ws) return nullptr;
  return reinterpret_cast<const float*>(static_cast<const char*>(ws) + router_wbytes(d));
}

template <typename XT, bool kFullK, bool kGrouped>
static void router_gemm_bm(int bm, int grid, const GemmArgs& g, hipStream_t stream) {
  const size_t lds = kGrouped ? (static_cast<size_t>(g.G) + 1) * sizeof(int) : 0;
  // the noise drawn here over 128-row tiles: the 8-wave form (noise waves beside the MFMAs)
  if constexpr (!kGrouped) {
    if (bm == 128 && g.use_noise && !g.eps) {
      router_gemm<XT, kFullK, 128, false, true><<<grid, 2 * kThreads, 0, stream>>>(g);
      return;
    }
  }
  if (bm == 128) router_gemm<XT, kFullK, 128, kGrouped><<<grid, kThreads, lds, stream>>>(g);
  else if (bm == 64) router_gemm<XT, kFullK, 64, kGrouped><<<grid, kThreads, lds, stream>>>(g);
  else router_gemm<XT, kFullK, 32, kGrouped><<<grid, kThreads, lds, stream>>>(g);
}
template <bool kGrouped>
static void router_gemm_launch(const Dims& d, int bm, int grid, const GemmArgs& g, hipStream_t stream) {
  const bool full = d.D % (d.dtype == MOE_BF16 ? 64 : 32) == 0;
  if (d.dtype == MOE_BF16) {
    if (full) router_gemm_bm<uint16_t, true, kGrouped>(bm, grid, g, stream);
    else router_gemm_bm<uint16_t, false, kGrouped>(bm, grid, g, stream);
  } else {
    if (full) router_gemm_bm<float, true, kGrouped>(bm, grid, g, stream);
    else router_gemm_bm<float, false, kGrouped>(bm, grid, g, stream);
  }
}

template <int KL>
static void select_lpr(int lpr, const SelectArgs& sa, hipStream_t stream) {
  const int T = sa.T;
  switch (lpr) {
    case 8: router_select<KL, 8><<<ceil_div(T, kThreads / 8), kThreads, 0, stream>>>(sa); break;
    case 16: router_select<KL, 16><<<ceil_div(T, kThreads / 16), kThreads, 0, stream>>>(sa); break;
    case 32: router_select<KL, 32><<<ceil_div(T, kThreads / 32), kThreads, 0, stream>>>(sa); break;
    default: router_select<KL, 64><<<ceil_div(T, kThreads / 64), kThreads, 0, stream>>>(sa); break;
  }
}
static void select_launch(int kl, int lpr, const SelectArgs& sa, hipStream_t stream) {
  switch (kl) {
    case 2: select_lpr<2>(lpr, sa, stream); break;
    case 4: select_lpr<4>(lpr, sa, stream); break;
    case 8: select_lpr<8>(lpr, sa, stream); break;
    default: select_lpr<16>(lpr, sa, stream); break;
  }
}

// Top-k of every score row: ids, gates, row_stats (v_k, v_{k+1}).
static void select_rows(const float* score, int T, int E, int k, bool switch_gate, int32_t* ids,
                        float* gates, float* row_stats, hipStream_t stream) {
  SelectArgs sa;
  sa.score = score;
  sa.ids = ids;
  sa.gates = gates;
  sa.row_stats = row_stats;
  sa.T = T;
  sa.E = E;
  sa.k = k;
  sa.switch_gate = switch_gate ? 1 : 0;
  sa.vec = (E % 4 == 0 && reinterpret_cast<uintptr_t>(score) % 16 == 0) ? 1 : 0;
  // lanes per row: 8, doubled (up to 64) while the grid would hold fewer than 64K threads and
  // each lane would still see at least 16 scores
  int lpr = 8;
  while (lpr < 64 && static_cast<int64_t>(T) * lpr < 65536 && E >= 32 * lpr) lpr <<= 1;
  const int need = k + 1;
  const int kl = need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
  select_launch(kl, lpr, sa, stream);
}

// Router weights packed, then the GEMM with its epilogue: clean (+ std and H with noise).
static moe_status router_scores(const Dims& d, uint64_t seed, const void* X, const float* Wg,
                                const float* Wnoise, const float* bias, const float* eps,
                                float* clean, float* noise_std, void* ws, int* nonfinite,
                                hipStream_t stream) {
  const bool noise = router_noise(d);
  const int NB = router_nb(d), KS = router_ks(d);
  uint4* wfrag = static_cast<uint4*>(ws);
  float* H = noise ? reinterpret_cast<float*>(static_cast<char*>(ws) + router_wbytes(d)) : nullptr;
  const int64_t items = static_cast<int64_t>(NB) * KS * kWave;
  const int pgrid = static_cast<int>(ceil_div64(items, 256));
  if (d.dtype == MOE_BF16)
    router_pack<true><<<pgrid, 256, 0, stream>>>(Wg, noise ? Wnoise : nullptr, d.D, d.E, noise, NB, KS, wfrag, 0, 0);
  else
    router_pack<false><<<pgrid, 256, 0, stream>>>(Wg, noise ? Wnoise : nullptr, d.D, d.E, noise, NB, KS, wfrag, 0, 0);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;

  GemmArgs g;
  g.X = X;
  g.wfrag = reinterpret_cast<const u32x4*>(wfrag);
  g.bias = bias;
  g.eps = noise ? eps : nullptr;
  g.clean = clean;
  g.std_out = noise ? noise_std : nullptr;
  g.H = H;
  g.nonfinite = nonfinite;
  g.seed = seed;
  g.T = d.T;
  g.D = d.D;
  g.E = d.E;
  g.NB = NB;
  g.KS = KS;
  g.use_noise = noise ? 1 : 0;
  g.vec_out = vec_outputs(d.E, clean, noise ? noise_std : nullptr, H);
  g.goff = nullptr;
  g.row_token = nullptr;
  g.G = 0;
  g.wgroup = 0;
  const int bm = router_bm(d.T, NB);
  const int64_t tiles = static_cast<int64_t>(ceil_div(d.T, bm)) * ceil_div(NB, 8);
  const int grid = static_cast<int>(ceil_div64(tiles, kXcds) * kXcds);
  router_gemm_launch<false>(d, bm, grid, g, stream);
  return launch_status();
}

moe_status route_launch(const Dims& d, const moe_problem* p, const void* X, const float* Wg,
                        const float* Wnoise, const float* bias, const float* eps, int32_t* ids,
                        float* gates, float* clean, float* noise_std, float* row_stats,
                        void* ws, int* nonfinite, hipStream_t stream) {
  const moe_status s = router_scores(d, p->seed, X, Wg, Wnoise, bias, eps, clean, noise_std, ws,
                                     nonfinite, stream);
  if (s != MOE_OK) return s;
  const bool noise = router_noise(d);
  float* H = noise ? reinterpret_cast<float*>(static_cast<char*>(ws) + router_wbytes(d)) : nullptr;
  select_rows(noise ? H : clean, d.T, d.E, d.k, d.gating == MOE_GATE_SWITCH_TOP1, ids, gates,
              row_stats, stream);
  return launch_status();
}

// clean = X . Wg (+ bias) only (no noise, no selection); workspace router_wbytes(d).
size_t router_clean_workspace(const Dims& d) {
  Dims dn = d;
  dn.noise = 0;
  return router_wbytes(dn);
}
moe_status router_clean_launch(const Dims& d, const void* X, const float* Wg, const float* bias,
                               float* clean, void* ws, int* nonfinite, hipStream_t stream) {
  Dims dn = d;
  dn.noise = 0;
  return router_scores(dn, 0, X, Wg, nullptr, bias, nullptr, clean, nullptr, ws, nonfinite, stream);
}

// ------------------------------------------------------------------ grouped gates
// Secondary gates of a hierarchical MoE. ds: T = R rows (grouped by gate through goff),
// D, E = experts per group, k = kept per group. Weights [G][D][E] (Wsg, Wsn).
static int64_t group_pack_stride(const Dims& ds) {  // uint4 per group in the packed stack
  const int pieces = ds.dtype == MOE_BF16 ? 3 : 1;
  return static_cast<int64_t>(pieces) * router_nb(ds) * router_ks(ds) * kWave;
}

size_t route_groups_workspace(const Dims& ds, int G) {
  size_t b = align256(static_cast<size_t>(G) * group_pack_stride(ds) * 16);
  if (router_noise(ds)) b += align256(static_cast<size_t>(ds.T) * ds.E * sizeof(float));
  return b;
}

moe_status route_groups_launch(const Dims& ds, int G, uint64_t seed, const void* X,
                               const int32_t* goff, const int32_t* row_token, const float* Wsg,
                               const float* Wsn, int32_t* ids, float* gates, float* clean,
                               float* noise_std, float* row_stats, void* ws, int* nonfinite,
                               hipStream_t stream) {
  const bool noise = router_noise(ds);
  const int NB = router_nb(ds), KS = router_ks(ds);
  const int64_t gstride = group_pack_stride(ds);
  uint4* wfrag = static_cast<uint4*>(ws);
  float* H = noise ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                              align256(static_cast<size_t>(G) * gstride * 16))
                   : nullptr;
  const int64_t items = static_cast<int64_t>(NB) * KS * kWave;
  const dim3 pgrid(static_cast<unsigned>(ceil_div64(items, 256)), static_cast<unsigned>(G));
  const int64_t wstride = static_cast<int64_t>(ds.D) * ds.E;
  if (ds.dtype == MOE_BF16)
    router_pack<true><<<pgrid, 256, 0, stream>>>(Wsg, noise ? Wsn : nullptr, ds.D, ds.E, noise, NB,
                                                 KS, wfrag, wstride, gstride);
  else
    router_pack<false><<<pgrid, 256, 0, stream>>>(Wsg, noise ? Wsn : nullptr, ds.D, ds.E, noise, NB,
                                                  KS, wfrag, wstride, gstride);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;

  GemmArgs g;
  g.X = X;
  g.wfrag = reinterpret_cast<const u32x4*>(wfrag);
  g.bias = nullptr;
  g.eps = nullptr;
  g.clean = clean;
  g.std_out = noise ? noise_std : nullptr;
  g.H = H;
  g.nonfinite = nonfinite;
  g.seed = seed;
  g.T = ds.T;
  g.D = ds.D;
  g.E = ds.E;
  g.NB = NB;
  g.KS = KS;
  g.use_noise = noise ? 1 : 0;
  g.vec_out = vec_outputs(ds.E, clean, noise ? noise_std : nullptr, H);
  g.goff = goff;
  g.row_token = row_token;
  g.G = G;
  g.wgroup = gstride;
  const int bm = router_bm(ds.T, NB);
  // at most (R + G*(bm-1)) / bm row tiles over all groups
  const int64_t mtiles = (static_cast<int64_t>(ds.T) + static_cast<int64_t>(G) * (bm - 1)) / bm;
  const int64_t tiles = mtiles * ceil_div(NB, 8);
  if (tiles > 0x7fff0000LL) return MOE_ERR_UNSUPPORTED;
  const int grid = static_cast<int>(ceil_div64(std::max<int64_t>(tiles, 1), kXcds) * kXcds);
  router_gemm_launch<true>(ds, bm, grid, g, stream);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  select_rows(noise ? H : clean, ds.T, ds.E, ds.k, false, ids, gates, row_stats, stream);
  return launch_status();
}

}  // namespace moe
