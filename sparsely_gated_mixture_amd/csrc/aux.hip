// Auxiliary balancing terms.
//
// "Outrageously Large Neural Networks" summary, section 3.4, "Load-Balancing:
// The Importance and Load Losses": Importance(X) = sum over the batch of the
// gate vectors; Load(X)_i = sum over the batch of P(x,i) = Phi((clean_i -
// kth_excluding(H,k,i)) / Softplus((x Wnoise)_i)); each loss is w * CV(v)^2.
// "Switch Transformer" explainer, "Implementation" step 8: alpha * E * sum_e
// f_e P_e with f the hard (pre-capacity) fractions and P the mean router
// probabilities. The population variance makes the lesson page's chapter-5
// example come out at 0.68.
//
// kth_excluding is read off the row: for an expert among the row's k kept ones
// the k-th largest of the others is the row's (k+1)-th largest score,
// otherwise its k-th; both are the router's row_stats.
//
// Deterministic reductions only (fixed order, no float atomics):
//   aux_rows     (E a multiple of 4, E <= 1024) block b: 64 tokens, one wave
//                per row at a time holding the whole row of clean (and std) as
//                float4 per lane: the row's softmax statistics come from two
//                wave reductions over registers, so clean is read once; each
//                lane keeps running sums for its experts over the wave's rows,
//                and the block's waves (8 for E <= 256, else 4) are added in
//                fixed order at the end.
//   aux_partial  (any other E) block b: 64 tokens; per-row softmax statistics
//                of clean (wave reductions), then thread-per-expert column
//                sums of the gates, P(x,i) and softmax(clean) over the rows.
//   aux_reduce   32 experts x 8 partial lanes per block, in 16 slices of the row
//                blocks (grid.y), strided fixed-order sums, then a fixed tree; fp64.
//   aux_final    one block: the 16 slices added in order per expert, then CV^2
//                (two-pass, fp64), the Switch term and the diagnostics, with
//                wave butterflies and one barrier per group of block sums.
#include "common.h"

namespace moe {
namespace {

constexpr int kRows = 64;  // most token rows per block (fewer when T is small)
constexpr int kThreads = 256;
constexpr int kSlices = 16;  // row-block slices of the column sums (each its own blocks)

struct AuxArgs {
  const int32_t* ids;
  const float* gates;
  const float* clean;
  const float* std_in;
  const float* row_stats;
  const int32_t* counts;
  float* importance;
  float* load;
  float* out;
  float* partial;  // [3][nblk][E]
  double* sums;    // [kSlices][3][E]
  int T, E, k, C, nblk, use_noise;
  int rows;  // token rows per block, <= kRows
  int vec;  // E % 4 == 0 and clean / std 16-byte aligned: float4 row reads
};

// erfc by the Chebyshev fit of Numerical Recipes in C (2nd ed., section 6.2, "erfcc"):
// erfc(x) = t exp(-x^2 + P(t)) with t = 1 / (1 + |x| / 2), fractional error below 1.2e-7 in
// exact arithmetic; evaluated in fp32 with the hardware exp and reciprocal, Phi = erfc / 2
// stays within about 2.2e-7 of the exact value. Branch-free, unlike the library's erfcf,
// which takes a different path per range of |x| and so splits a wave's lanes.
__device__ __forceinline__ float erfc_cheb(float x) {
  const float z = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.f));
  float p = 0.17087277f;
  p = fmaf(t, p, -0.82215223f);
  p = fmaf(t, p, 1.48851587f);
  p = fmaf(t, p, -1.13520398f);
  p = fmaf(t, p, 0.27886807f);
  p = fmaf(t, p, -0.18628806f);
  p = fmaf(t, p, 0.09678418f);
  p = fmaf(t, p, 0.37409196f);
  p = fmaf(t, p, 1.00002368f);
  const float ans = t * __expf(fmaf(-z, z, fmaf(t, p, -1.26551223f)));
  return x >= 0.f ? ans : 2.f - ans;
}
__device__ __forceinline__ float phi(float z) { return 0.5f * erfc_cheb(-z * 0.70710678118654752f); }

__global__ __launch_bounds__(kThreads) void aux_partial(AuxArgs a) {
  constexpr int kU = 8;  // rows in flight per thread in the column pass
  __shared__ float sM[kRows], sS[kRows];
  __shared__ float sR0[kRows], sR1[kRows];
  __shared__ int sId[kRows * MOE_MAX_K];
  __shared__ float sG[kRows * MOE_MAX_K];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * a.rows;
  const int nr = min(a.rows, a.T - t0);
  const int E = a.E, k = a.k;

  for (int i = tid; i < nr * k; i += kThreads) {
    sId[i] = a.ids[static_cast<int64_t>(t0) * k + i];
    sG[i] = a.gates[static_cast<int64_t>(t0) * k + i];
  }
  if (a.use_noise)
    for (int r = tid; r < nr; r += kThreads) {
      sR0[r] = a.row_stats[2 * static_cast<int64_t>(t0 + r)];
      sR1[r] = a.row_stats[2 * static_cast<int64_t>(t0 + r) + 1];
    }
  // per-row softmax statistics of clean: one wave per row
  auto row_stats = [&](int r, float& m, float& s) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float om = __shfl_xor(m, off), os = __shfl_xor(s, off);
      const float mn = fmaxf(m, om);
      s = (m == -INFINITY ? 0.f : s * expf(m - mn)) + (om == -INFINITY ? 0.f : os * expf(om - mn));
      m = mn;
    }
    if (lane == 0) {
      sM[r] = m;
      sS[r] = s;
    }
  };
  for (int r = wave; r < nr; r += kThreads / 64) {
    const float* row = a.clean + static_cast<int64_t>(t0 + r) * E;
    float m = -INFINITY, s = 0.f;
    for (int e = lane; e < E; e += 64) {
      const float x = row[e];
      const float mn = fmaxf(m, x);
      s = s * expf(m - mn) + expf(x - mn);
      m = mn;
    }
    row_stats(r, m, s);
  }
  __syncthreads();

  // column pass: thread per expert, kU rows of loads in flight
  const int64_t plane = static_cast<int64_t>(a.nblk) * E;
  for (int e = tid; e < E; e += kThreads) {
    float imp = 0.f, load = 0.f, pb = 0.f;
    for (int r0 = 0; r0 < nr; r0 += kU) {
      float c[kU], sd[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int r = min(r0 + u, nr - 1);
        const int64_t ix = static_cast<int64_t>(t0 + r) * E + e;
        c[u] = a.clean[ix];
        sd[u] = a.use_noise ? a.std_in[ix] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int r = r0 + u;
        if (r >= nr) break;
        bool inside = false;
        for (int j = 0; j < k; ++j)
          if (sId[r * k + j] == e) {
            inside = true;
            imp += sG[r * k + j];
          }
        pb += expf(c[u] - sM[r]) / sS[r];
        if (a.use_noise) {
          const float thr = inside ? sR1[r] : sR0[r];
          const float diff = c[u] - thr;
          float pr;
          if (sd[u] > 0.f) pr = phi(diff / sd[u]);
          else pr = diff > 0.f ? 1.f : (diff == 0.f ? 0.5f : 0.f);
          load += pr;
        }
      }
    }
    const int64_t o = static_cast<int64_t>(blockIdx.x) * E + e;
    a.partial[o] = imp;
    a.partial[plane + o] = load;
    a.partial[2 * plane + o] = pb;
  }
}

// Wave reductions without the LDS permute path: inside each row of 16 lanes, data-parallel
// moves exchange partners (lane ^ 1, lane ^ 2 by quad permutes, then the half-row and row
// mirrors, which pair whole quads and whole half-rows), so every lane of a row holds the
// same bits; the four rows are then read out and combined in a fixed order. The result is
// the same in every lane.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  v = fmaxf(v, dpp<kRowMirror>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// NV float4 chunks per lane per row: lane l holds experts 256*v + 4*l + i. kT threads a
// block, U rows of loads in flight per wave.
template <int NV, int kT, int U>
__global__ __launch_bounds__(kT) void aux_rows(AuxArgs a) {
  constexpr int kWaves = kT / 64;
  __shared__ float sR0[kRows], sR1[kRows];
  __shared__ int sId[kRows * MOE_MAX_K];
  __shared__ float sG[kRows * MOE_MAX_K];
  __shared__ float4 sRed[kWaves - 1][3][NV * 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * a.rows;
  const int nr = min(a.rows, a.T - t0);
  const int E = a.E, k = a.k;
  const bool noise = a.use_noise != 0;

  for (int i = tid; i < nr * k; i += kT) {
    sId[i] = a.ids[static_cast<int64_t>(t0) * k + i];
    sG[i] = a.gates[static_cast<int64_t>(t0) * k + i];
  }
  if (noise)
    for (int r = tid; r < nr; r += kT) {
      sR0[r] = a.row_stats[2 * static_cast<int64_t>(t0 + r)];
      sR1[r] = a.row_stats[2 * static_cast<int64_t>(t0 + r) + 1];
    }
  __syncthreads();

  float imp[NV][4], lsum[NV][4], pb[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) imp[v][i] = lsum[v][i] = pb[v][i] = 0.f;

  for (int rb = wave; rb < nr; rb += kWaves * U) {
    float4 c[U][NV], sd[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(rb + kWaves * u, nr - 1);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int e = 256 * v + 4 * lane;
        const int64_t ix = static_cast<int64_t>(t0 + r) * E + e;
        c[u][v] = e < E ? *reinterpret_cast<const float4*>(a.clean + ix)
                        : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        sd[u][v] = (noise && e < E) ? *reinterpret_cast<const float4*>(a.std_in + ix)
                                    : make_float4(1.f, 1.f, 1.f, 1.f);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + kWaves * u;
      if (r >= nr) break;  // uniform across the wave
      float m = -INFINITY;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        m = fmaxf(m, fmaxf(fmaxf(c[u][v].x, c[u][v].y), fmaxf(c[u][v].z, c[u][v].w)));
      m = wave_max(m);
      float ex[NV][4], s = 0.f;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        ex[v][0] = __expf(c[u][v].x - m);
        ex[v][1] = __expf(c[u][v].y - m);
        ex[v][2] = __expf(c[u][v].z - m);
        ex[v][3] = __expf(c[u][v].w - m);
        s += (ex[v][0] + ex[v][1]) + (ex[v][2] + ex[v][3]);
      }
      const float inv = 1.f / wave_sum(s);
      bool in[NV][4];
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) in[v][i] = false;
      for (int j = 0; j < k; ++j) {
        const int d = sId[r * k + j] - 4 * lane;
        const float g = sG[r * k + j];
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool hit = d == 256 * v + i;
            in[v][i] |= hit;
            imp[v][i] += hit ? g : 0.f;
          }
      }
      const float r0 = noise ? sR0[r] : 0.f, r1 = noise ? sR1[r] : 0.f;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const float cv[4] = {c[u][v].x, c[u][v].y, c[u][v].z, c[u][v].w};
        const float sv[4] = {sd[u][v].x, sd[u][v].y, sd[u][v].z, sd[u][v].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[v][i] += ex[v][i] * inv;
          if (noise) {
            const float diff = cv[i] - (in[v][i] ? r1 : r0);
            float pr;
            if (sv[i] > 0.f) pr = phi(__fdividef(diff, sv[i]));
            else pr = diff > 0.f ? 1.f : (diff == 0.f ? 0.5f : 0.f);
            lsum[v][i] += pr;
          }
        }
      }
    }
  }

  // fixed-order sum over the waves: wave 0 + wave 1 + wave 2 + ... in index order
  if (wave > 0)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      sRed[wave - 1][0][v * 64 + lane] = make_float4(imp[v][0], imp[v][1], imp[v][2], imp[v][3]);
      sRed[wave - 1][1][v * 64 + lane] = make_float4(lsum[v][0], lsum[v][1], lsum[v][2], lsum[v][3]);
      sRed[wave - 1][2][v * 64 + lane] = make_float4(pb[v][0], pb[v][1], pb[v][2], pb[v][3]);
    }
  __syncthreads();
  if (wave == 0) {
    const int64_t plane = static_cast<int64_t>(a.nblk) * E;
    float* out[3] = {a.partial, a.partial + plane, a.partial + 2 * plane};
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e = 256 * v + 4 * lane;
      if (e >= E) continue;
      float4 q[3] = {make_float4(imp[v][0], imp[v][1], imp[v][2], imp[v][3]),
                     make_float4(lsum[v][0], lsum[v][1], lsum[v][2], lsum[v][3]),
                     make_float4(pb[v][0], pb[v][1], pb[v][2], pb[v][3])};
#pragma unroll
      for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const float4 o = sRed[w][t][v * 64 + lane];
          q[t].x += o.x;
          q[t].y += o.y;
          q[t].z += o.z;
          q[t].w += o.w;
        }
#pragma unroll
      for (int t = 0; t < 3; ++t)
        *reinterpret_cast<float4*>(out[t] + static_cast<int64_t>(blockIdx.x) * E + e) = q[t];
    }
  }
}

// Fixed-order fp64 reductions over the block's kThreads threads: a butterfly in each wave,
// then the waves added in order (w0 + w1) + (w2 + w3). Every thread gets the result.
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}
template <int N>
__device__ void block_sums(double (&v)[N], double (*sh)[kThreads / 64]) {
  static_assert(kThreads == 256, "four waves");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const double w = wave_sum_d(v[q]);
    if (lane == 0) sh[q][wave] = w;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = (sh[q][0] + sh[q][1]) + (sh[q][2] + sh[q][3]);
  __syncthreads();
}
template <int N>
__device__ void block_maxes(double (&v)[N], double (*sh)[kThreads / 64]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const double w = wave_max_d(v[q]);
    if (lane == 0) sh[q][wave] = w;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = fmax(fmax(sh[q][0], sh[q][1]), fmax(sh[q][2], sh[q][3]));
  __syncthreads();
}

// Block (expert group x, slice y): 32 experts x 8 partial lanes over the slice's share of the
// row blocks (fixed order), then a fixed tree; the slice's sums go to sums[y] (fp64).
__global__ __launch_bounds__(kThreads) void aux_reduce(AuxArgs a) {
  __shared__ double s[3][8][32];
  const int el = threadIdx.x & 31, bl = threadIdx.x >> 5;
  const int e = blockIdx.x * 32 + el;
  const int E = a.E;
  const int64_t plane = static_cast<int64_t>(a.nblk) * E;
  const int per = (a.nblk + kSlices - 1) / kSlices;
  const int b0 = blockIdx.y * per, b1 = min(a.nblk, b0 + per);
  double acc[3] = {0.0, 0.0, 0.0};
  if (e < E) {
    int b = b0 + bl;
    for (; b + 24 < b1; b += 32) {  // four blocks of loads in flight, summed in order
      float v[3][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 3; ++q) v[q][u] = a.partial[q * plane + static_cast<int64_t>(b + 8 * u) * E + e];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 3; ++q) acc[q] += v[q][u];
    }
    for (; b < b1; b += 8)
#pragma unroll
      for (int q = 0; q < 3; ++q) acc[q] += a.partial[q * plane + static_cast<int64_t>(b) * E + e];
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) s[q][bl][el] = acc[q];
  __syncthreads();
  if (bl == 0 && e < E) {
    double* out = a.sums + static_cast<int64_t>(blockIdx.y) * 3 * E;
#pragma unroll
    for (int q = 0; q < 3; ++q)
      out[q * E + e] = ((s[q][0][el] + s[q][1][el]) + (s[q][2][el] + s[q][3][el])) +
                       ((s[q][4][el] + s[q][5][el]) + (s[q][6][el] + s[q][7][el]));
  }
}

// One block: per expert the slices in order (slice 0 first), then the scalars.
__global__ __launch_bounds__(kThreads) void aux_final(AuxArgs a) {
  __shared__ double sh[5][kThreads / 64];
  const int E = a.E;
  // the slices in order, per expert; thread t takes experts t, t + kThreads, ... and leaves
  // their totals in slice 0's place (no other thread reads those columns)
  double si = 0, sl = 0, sfp = 0, sc = 0, mxl = -INFINITY, mxc = -INFINITY, drop = 0;
  for (int x = threadIdx.x; x < E; x += kThreads) {
    // every slice's value requested before the first addition (one block: the loads'
    // latency, not their bytes, is what this pass waits on)
    double buf[kSlices][3];
#pragma unroll
    for (int y = 0; y < kSlices; ++y)
#pragma unroll
      for (int q = 0; q < 3; ++q) buf[y][q] = a.sums[(static_cast<int64_t>(y) * 3 + q) * E + x];
    __builtin_amdgcn_sched_barrier(0);  // keeps the scheduler from interleaving them with the sums
    double v[3] = {0.0, 0.0, 0.0};
#pragma unroll
    for (int y = 0; y < kSlices; ++y)
#pragma unroll
      for (int q = 0; q < 3; ++q) v[q] += buf[y][q];
#pragma unroll
    for (int q = 0; q < 2; ++q) a.sums[q * E + x] = v[q];
    if (a.importance) a.importance[x] = static_cast<float>(v[0]);
    if (a.load) a.load[x] = static_cast<float>(v[1]);
    si += v[0];
    sl += v[1];
    const double c = a.counts[x];
    sfp += (c / a.T) * (v[2] / a.T);
    sc += c;
    mxl = fmax(mxl, v[1]);
    mxc = fmax(mxc, c);
    drop += fmax(c - a.C, 0.0);
  }
  double sums5[5] = {si, sl, sfp, sc, drop};
  block_sums(sums5, sh);
  double maxes[2] = {mxl, mxc};
  block_maxes(maxes, sh);
  si = sums5[0];
  sl = sums5[1];
  sfp = sums5[2];
  sc = sums5[3];
  drop = sums5[4];
  const double mi = si / E, ml = sl / E;
  // second pass (the deviations from the means) over the thread's own totals
  double dev[2] = {0.0, 0.0};
  for (int x = threadIdx.x; x < E; x += kThreads) {
    const double v0 = a.sums[x], v1 = a.sums[E + x];
    dev[0] += (v0 - mi) * (v0 - mi);
    dev[1] += (v1 - ml) * (v1 - ml);
  }
  block_sums(dev, sh);
  if (threadIdx.x == 0) {
    const double vi = dev[0] / E, vl = dev[1] / E;
    const double mc = sc / E;
    a.out[0] = static_cast<float>(mi != 0 ? vi / (mi * mi) : 0.0);
    a.out[1] = static_cast<float>(ml != 0 ? vl / (ml * ml) : 0.0);
    a.out[2] = static_cast<float>(E * sfp);
    a.out[3] = static_cast<float>(ml > 0 ? maxes[0] / ml : 0.0);
    a.out[4] = static_cast<float>(mc > 0 ? maxes[1] / mc : 0.0);
    a.out[5] = static_cast<float>(drop);
    a.out[6] = static_cast<float>(si);
    a.out[7] = 0.f;
  }
}

}  // namespace

// Rows per block: kRows, halved (down to 4) while that leaves fewer than 1024 blocks, so
// small batches still spread over the chip.
static int aux_rows_per_block(const Dims& d) {
  int r = kRows;
  while (r > 4 && ceil_div(d.T, r) < 1024) r >>= 1;
  return r;
}
static int aux_blocks(const Dims& d) { return ceil_div(d.T, aux_rows_per_block(d)); }

size_t aux_workspace(const Dims& d) {
  return align256(3 * static_cast<size_t>(aux_blocks(d)) * d.E * sizeof(float)) +
         align256(static_cast<size_t>(kSlices) * 3 * d.E * sizeof(double));
}

moe_status aux_launch(const Dims& d, const int32_t* ids, const float* gates, const float* clean,
                      const float* noise_std, const float* row_stats, const int32_t* counts,
                      float* importance, float* load, float* out, void* ws, hipStream_t stream) {
  AuxArgs a;
  a.ids = ids;
  a.gates = gates;
  a.clean = clean;
  a.use_noise = (d.gating == MOE_GATE_NOISY_TOPK && d.noise) ? 1 : 0;
  a.std_in = a.use_noise ? noise_std : nullptr;
  a.row_stats = a.use_noise ? row_stats : nullptr;
  a.counts = counts;
  a.importance = importance;
  a.load = load;
  a.out = out;
  a.nblk = aux_blocks(d);
  a.rows = aux_rows_per_block(d);
  a.partial = static_cast<float*>(ws);
  a.sums = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                     align256(3 * static_cast<size_t>(a.nblk) * d.E * sizeof(float)));
  a.T = d.T;
  a.E = d.E;
  a.k = d.k;
  a.C = d.C;
  a.vec = (d.E % 4 == 0 && (reinterpret_cast<uintptr_t>(clean) | reinterpret_cast<uintptr_t>(a.std_in)) % 16 == 0)
              ? 1 : 0;
  if (a.vec && d.E <= 256) aux_rows<1, 512, 2><<<a.nblk, 512, 0, stream>>>(a);
  else if (a.vec && d.E <= 512) aux_rows<2, 256, 2><<<a.nblk, 256, 0, stream>>>(a);
  else if (a.vec && d.E <= 1024) aux_rows<4, 256, 1><<<a.nblk, 256, 0, stream>>>(a);
  else aux_partial<<<a.nblk, kThreads, 0, stream>>>(a);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  aux_reduce<<<dim3(ceil_div(d.E, 32), kSlices), kThreads, 0, stream>>>(a);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  aux_final<<<1, kThreads, 0, stream>>>(a);
  return launch_status();
}

}  // namespace moe
