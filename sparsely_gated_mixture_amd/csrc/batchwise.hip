// Batchwise (strictly balanced) mask.
//
// "Outrageously Large Neural Networks" summary, section 3.4, "Strictly Balanced
// Gating": instead of each token keeping its k best experts, each expert keeps
// the m = floor(k T / E) tokens of the batch with the highest dense gate scores
// G_sigma(x) = Softmax(x . Wg); the "Mixture-of-Experts: Sparse Computation"
// lesson, chapter 4, multiplies that mask into the dense softmax and
// renormalises per token (chapter 2's mask form). Every expert gets exactly m
// rows; a token may be kept by any number of experts, or by none (then only
// the residual remains). The batchwise loss compares a threshold mask
// 1[s > T_e] with this mask.
//
// Launches (route):
//   router_pack + router_gemm   clean = X . Wg (+ bias), fp32-exact (router.hip)
//   bw_softmax    32 tokens per block: row max / sum by wave reductions, then
//                 32x64 tiles through LDS so the scores leave expert-major
//                 (probs_t [E, T]) with coalesced stores; clears the mask rows
//   bw_select     one block per expert: radix select (4 passes of 8 bits on the
//                 fp32 bit pattern) of the m-th largest score, then one pass in
//                 token order keeping every score above it and the lowest-index
//                 ties: sel[e*m ..] ascending; sets mask bits (OR, order-free)
//   bw_tok_count, bw_tok_scan, bw_tok_offsets   experts per token and their
//                 exclusive scan (CSR offsets)
//   bw_pairs      (expert, slot) -> the token's CSR entry (rank of the expert
//                 among the token's mask bits): tok_row, slot_pair
//   bw_gates      per token, renormalised dense scores over its experts
// dispatch: bw_gather copies X rows to the expert-major rows (16-byte vectors).
// combine:  bw_combine, a wave per token, fp32 sum over its experts ascending.
// aux:      bw_aux_expert (importance and the batchwise loss per expert, fp64)
//           and bw_aux_final (CV^2, loss, experts-per-token statistics).
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTileTok = 32;   // tokens per softmax block
constexpr int kSelThreads = 512;
constexpr int kHistCopies = 16;  // radix histogram copies (spreads LDS atomics)

__device__ __forceinline__ float bw_wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float bw_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(kThreads) void bw_softmax(const float* __restrict__ clean, int T, int E,
                                                      int W, float* __restrict__ probs_t,
                                                      uint32_t* __restrict__ mask) {
  __shared__ float sMax[kTileTok], sSum[kTileTok];
  __shared__ float tile[kTileTok][65];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * kTileTok;
  const int nt = min(kTileTok, T - t0);
  for (int r = wave; r < nt; r += kThreads / 64) {
    const float* row = clean + static_cast<int64_t>(t0 + r) * E;
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, row[e]);
    m = bw_wave_max(m);
    float s = 0.f;
    for (int e = lane; e < E; e += 64) s += expf(row[e] - m);
    s = bw_wave_sum(s);
    if (lane == 0) {
      sMax[r] = m;
      sSum[r] = s;
    }
  }
  for (int i = tid; i < nt * W; i += kThreads) mask[static_cast<int64_t>(t0) * W + i] = 0u;
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += 64) {
    // load [tokens][64 experts], coalesced along the experts
    for (int i = tid; i < kTileTok * 64; i += kThreads) {
      const int r = i >> 6, c = i & 63;
      float v = 0.f;
      if (r < nt && e0 + c < E) {
        const float x = clean[static_cast<int64_t>(t0 + r) * E + e0 + c];
        v = expf(x - sMax[r]) / sSum[r];
      }
      tile[r][c] = v;
    }
    __syncthreads();
    // store [experts][tokens], coalesced along the tokens
    for (int i = tid; i < 64 * kTileTok; i += kThreads) {
      const int c = i / kTileTok, r = i % kTileTok;
      if (r < nt && e0 + c < E) probs_t[static_cast<int64_t>(e0 + c) * T + t0 + r] = tile[r][c];
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kSelThreads) void bw_select(const float* __restrict__ probs_t, int T,
                                                        int E, int m, int W,
                                                        int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ offsets,
                                                        uint32_t* __restrict__ mask) {
  __shared__ int hist[kHistCopies][256];
  __shared__ int wt[kSelThreads / 64];
  __shared__ uint32_t sPrefix;
  __shared__ int sRemain;
  const int tid = threadIdx.x;
  const int e = blockIdx.x;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(probs_t + static_cast<int64_t>(e) * T);
  int* myhist = hist[tid % kHistCopies];
  if (tid == 0) {
    sPrefix = 0u;
    sRemain = m;
  }
  uint32_t pmask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kHistCopies * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t prefix = sPrefix;
    for (int t = tid; t < T; t += kSelThreads) {
      const uint32_t k = key[t];
      if ((k & pmask) == prefix) atomicAdd(&myhist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    for (int b = tid; b < 256; b += kSelThreads) {
      int c = 0;
#pragma unroll
      for (int q = 0; q < kHistCopies; ++q) c += hist[q][b];
      hist[0][b] = c;
    }
    __syncthreads();
    // bins from the top: thread i holds bin 255 - i; the bin holding the rem-th largest is
    // where the running count (from the top) first reaches rem
    {
      const int rem = sRemain;
      const int bin = 255 - tid;
      const int h = tid < 256 ? hist[0][bin] : 0;
      int excl;
      block_exclusive_scan<kSelThreads>(h, &excl, wt);
      if (tid < 256 && excl < rem && excl + h >= rem) {
        sRemain = rem - excl;
        sPrefix = prefix | (static_cast<uint32_t>(bin) << shift);
      }
    }
    __syncthreads();
    pmask |= 255u << shift;
  }
  const uint32_t kth = sPrefix;
  const int need_eq = sRemain;  // ties at the m-th score to keep, lowest tokens first
  // keep in token order: above kth, or equal with rank < need_eq
  int base_above = 0, base_eq = 0;
  for (int c0 = 0; c0 < T; c0 += kSelThreads * 4) {
    int a[4], q[4];
    int la = 0, lq = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = c0 + tid * 4 + u;
      const uint32_t k = t < T ? key[t] : 0u;
      a[u] = (t < T && k > kth) ? 1 : 0;
      q[u] = (t < T && k == kth) ? 1 : 0;
      la += a[u];
      lq += q[u];
    }
    int excl;  // packed pair: low 16 bits above, high 16 bits equal (a chunk has 2048 tokens)
    const int tot = block_exclusive_scan<kSelThreads>(la | (lq << 16), &excl, wt);
    int ra = base_above + (excl & 0xffff), rq = base_eq + (excl >> 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = c0 + tid * 4 + u;
      const bool take = a[u] || (q[u] && rq < need_eq);
      if (take) {
        const int pos = ra + min(rq, need_eq);
        sel[static_cast<int64_t>(e) * m + pos] = t;
        atomicOr(&mask[static_cast<int64_t>(t) * W + (e >> 5)], 1u << (e & 31));
      }
      ra += a[u];
      rq += q[u];
    }
    base_above += tot & 0xffff;
    base_eq += tot >> 16;
  }
  if (tid == 0) {
    offsets[e] = e * m;
    if (e == E - 1) offsets[E] = E * m;
  }
}

__device__ __forceinline__ int mask_count(const uint32_t* row, int W) {
  int c = 0;
  for (int w = 0; w < W; ++w) c += __popc(row[w]);
  return c;
}

__global__ __launch_bounds__(kThreads) void bw_tok_count(const uint32_t* __restrict__ mask, int T,
                                                        int W, int32_t* __restrict__ tok_count,
                                                        int32_t* __restrict__ block_sum) {
  __shared__ int wt[kThreads / 64];
  const int t = blockIdx.x * kThreads + threadIdx.x;
  const int c = t < T ? mask_count(mask + static_cast<int64_t>(t) * W, W) : 0;
  if (t < T) tok_count[t] = c;
  int excl;
  const int tot = block_exclusive_scan<kThreads>(c, &excl, wt);
  if (threadIdx.x == 0) block_sum[blockIdx.x] = tot;
}

// One block: exclusive scan of the block sums, in chunks of kThreads.
__global__ __launch_bounds__(kThreads) void bw_tok_scan(int32_t* __restrict__ block_sum, int nblk) {
  __shared__ int wt[kThreads / 64];
  int base = 0;
  for (int c0 = 0; c0 < nblk; c0 += kThreads) {
    const int i = c0 + threadIdx.x;
    const int v = i < nblk ? block_sum[i] : 0;
    int excl;
    const int tot = block_exclusive_scan<kThreads>(v, &excl, wt);
    if (i < nblk) block_sum[i] = base + excl;
    base += tot;
  }
}

__global__ __launch_bounds__(kThreads) void bw_tok_offsets(const int32_t* __restrict__ tok_count,
                                                          const int32_t* __restrict__ block_base,
                                                          int T, int32_t* __restrict__ tok_off) {
  __shared__ int wt[kThreads / 64];
  const int t = blockIdx.x * kThreads + threadIdx.x;
  const int c = t < T ? tok_count[t] : 0;
  int excl;
  block_exclusive_scan<kThreads>(c, &excl, wt);
  const int o = block_base[blockIdx.x] + excl;
  if (t < T) tok_off[t] = o;
  if (t == T - 1) tok_off[T] = o + c;
}

__global__ void bw_pairs(const int32_t* __restrict__ sel, const uint32_t* __restrict__ mask,
                         const int32_t* __restrict__ tok_off, int E, int m, int W,
                         int32_t* __restrict__ tok_row, int32_t* __restrict__ slot_pair) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= static_cast<int64_t>(E) * m) return;
  const int e = static_cast<int>(r / m);
  const int t = sel[r];
  const uint32_t* row = mask + static_cast<int64_t>(t) * W;
  int rank = 0;
  for (int w = 0; w < (e >> 5); ++w) rank += __popc(row[w]);
  rank += __popc(row[e >> 5] & ((1u << (e & 31)) - 1u));
  const int j = tok_off[t] + rank;
  tok_row[j] = static_cast<int32_t>(r);
  slot_pair[r] = j;
}

__global__ void bw_gates(const float* __restrict__ probs_t, const int32_t* __restrict__ tok_off,
                         const int32_t* __restrict__ tok_row, int T, int m,
                         float* __restrict__ tok_gate) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int j0 = tok_off[t], j1 = tok_off[t + 1];
  float s = 0.f;
  for (int j = j0; j < j1; ++j) s += probs_t[static_cast<int64_t>(tok_row[j] / m) * T + t];
  for (int j = j0; j < j1; ++j)
    tok_gate[j] = s > 0.f ? probs_t[static_cast<int64_t>(tok_row[j] / m) * T + t] / s : 0.f;
}

template <typename T>
__global__ void bw_gather(const T* __restrict__ X, const int32_t* __restrict__ sel, int64_t rows,
                          int D, T* __restrict__ Xd) {
  constexpr int V = Elem<T>::kVec;
  const int nv = D / V;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * nv) return;
  const int64_t r = i / nv;
  const int c = static_cast<int>(i - r * nv);
  reinterpret_cast<uint4*>(Xd + r * D)[c] =
      reinterpret_cast<const uint4*>(X + static_cast<int64_t>(sel[r]) * D)[c];
}

template <typename T>
__global__ void bw_gather_scalar(const T* __restrict__ X, const int32_t* __restrict__ sel,
                                 int64_t rows, int D, T* __restrict__ Xd) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * D) return;
  const int64_t r = i / D;
  const int c = static_cast<int>(i - r * D);
  Xd[r * D + c] = X[static_cast<int64_t>(sel[r]) * D + c];
}

// A wave per token: Y = R + sum over the token's experts (ascending) of gate * Z[row];
// 16-byte vectors when D allows.
template <typename T>
__global__ __launch_bounds__(kThreads) void bw_combine(const T* __restrict__ Z,
                                                      const int32_t* __restrict__ tok_off,
                                                      const int32_t* __restrict__ tok_row,
                                                      const float* __restrict__ tok_gate,
                                                      const T* __restrict__ R, int Tn, int D,
                                                      T* __restrict__ Y, int* nonfinite) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int j0 = tok_off[t], j1 = tok_off[t + 1];
  bool bad = false;
  if (D % V == 0) {
    const int nv = D / V;
    for (int c = lane; c < nv; c += 64) {
      float y[V];
      if (R) {
        const uint4 rv = reinterpret_cast<const uint4*>(R + static_cast<int64_t>(t) * D)[c];
        const T* rp = reinterpret_cast<const T*>(&rv);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = Elem<T>::to_f32(rp[i]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = 0.f;
      }
      for (int j = j0; j < j1; ++j) {
        const float g = tok_gate[j];
        const uint4 zv = reinterpret_cast<const uint4*>(Z + static_cast<int64_t>(tok_row[j]) * D)[c];
        const T* zp = reinterpret_cast<const T*>(&zv);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = fmaf(g, Elem<T>::to_f32(zp[i]), y[i]);
      }
      T out[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        bad |= !isfinite(y[i]);
        out[i] = Elem<T>::from_f32(y[i]);
      }
      reinterpret_cast<uint4*>(Y + static_cast<int64_t>(t) * D)[c] = *reinterpret_cast<const uint4*>(out);
    }
  } else {
    for (int c = lane; c < D; c += 64) {
      float y = R ? Elem<T>::to_f32(R[static_cast<int64_t>(t) * D + c]) : 0.f;
      for (int j = j0; j < j1; ++j)
        y = fmaf(tok_gate[j], Elem<T>::to_f32(Z[static_cast<int64_t>(tok_row[j]) * D + c]), y);
      bad |= !isfinite(y);
      Y[static_cast<int64_t>(t) * D + c] = Elem<T>::from_f32(y);
    }
  }
  if (nonfinite) note_nonfinite(nonfinite, bad);
}

struct BwAuxArgs {
  const float* probs_t;
  const uint32_t* mask;
  const int32_t* tok_count;
  const float* tok_gate;
  const int32_t* slot_pair;
  const float* thresholds;
  double* per_expert;  // [5][E]: importance, loss; token count sum, max, zero count per slice
  float* importance;
  float* out;
  int T, E, m, W;
};

__device__ double bw_block_sum(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int w = kThreads / 2; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}
__device__ double bw_block_max(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int w = kThreads / 2; w >= 1; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] = fmax(sh[threadIdx.x], sh[threadIdx.x + w]);
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

// One block per expert: importance (its m gates in slot order) and its batchwise loss term.
__global__ __launch_bounds__(kThreads) void bw_aux_expert(BwAuxArgs a) {
  __shared__ double sh[kThreads];
  const int e = blockIdx.x;
  double imp = 0.0;
  for (int s = threadIdx.x; s < a.m; s += kThreads)
    imp += a.tok_gate[a.slot_pair[static_cast<int64_t>(e) * a.m + s]];
  imp = bw_block_sum(imp, sh);
  double loss = 0.0;
  if (a.thresholds) {
    const float thr = a.thresholds[e];
    const float* p = a.probs_t + static_cast<int64_t>(e) * a.T;
    for (int t = threadIdx.x; t < a.T; t += kThreads) {
      const float s = p[t];
      const int kept = (a.mask[static_cast<int64_t>(t) * a.W + (e >> 5)] >> (e & 31)) & 1u;
      const int above = s > thr ? 1 : 0;
      loss += static_cast<double>(above - kept) * (static_cast<double>(s) - thr);
    }
    loss = bw_block_sum(loss, sh);
  }
  // experts-per-token statistics of token slice e (the E blocks split the tokens)
  const int64_t t0 = static_cast<int64_t>(a.T) * e / a.E, t1 = static_cast<int64_t>(a.T) * (e + 1) / a.E;
  double ct = 0, mx = 0, none = 0;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += kThreads) {
    const int c = a.tok_count[t];
    ct += c;
    mx = fmax(mx, static_cast<double>(c));
    none += c == 0 ? 1.0 : 0.0;
  }
  ct = bw_block_sum(ct, sh);
  mx = bw_block_max(mx, sh);
  none = bw_block_sum(none, sh);
  if (threadIdx.x == 0) {
    a.per_expert[e] = imp;
    a.per_expert[a.E + e] = loss;
    a.per_expert[2 * a.E + e] = ct;
    a.per_expert[3 * a.E + e] = mx;
    a.per_expert[4 * a.E + e] = none;
    if (a.importance) a.importance[e] = static_cast<float>(imp);
  }
}

__global__ __launch_bounds__(kThreads) void bw_aux_final(BwAuxArgs a) {
  __shared__ double sh[kThreads];
  const double* imp = a.per_expert;
  const double* loss = a.per_expert + a.E;
  double si = 0, sl = 0;
  for (int e = threadIdx.x; e < a.E; e += kThreads) {
    si += imp[e];
    sl += loss[e];
  }
  si = bw_block_sum(si, sh);
  sl = bw_block_sum(sl, sh);
  const double mi = si / a.E;
  double vi = 0;
  for (int e = threadIdx.x; e < a.E; e += kThreads) vi += (imp[e] - mi) * (imp[e] - mi);
  vi = bw_block_sum(vi, sh) / a.E;
  double ct = 0, mx = 0, none = 0;
  for (int e = threadIdx.x; e < a.E; e += kThreads) {
    ct += a.per_expert[2 * a.E + e];
    mx = fmax(mx, a.per_expert[3 * a.E + e]);
    none += a.per_expert[4 * a.E + e];
  }
  ct = bw_block_sum(ct, sh);
  mx = bw_block_max(mx, sh);
  none = bw_block_sum(none, sh);
  if (threadIdx.x == 0) {
    a.out[0] = static_cast<float>(mi != 0 ? vi / (mi * mi) : 0.0);
    a.out[1] = static_cast<float>(sl);
    a.out[2] = static_cast<float>(ct / a.T);
    a.out[3] = static_cast<float>(mx);
    a.out[4] = static_cast<float>(none);
    a.out[5] = static_cast<float>(si);
    a.out[6] = static_cast<float>(a.m);
    a.out[7] = 0.f;
  }
}

}  // namespace

// ------------------------------------------------------------------ host side
int batchwise_m(const Dims& d) {
  return static_cast<int>(static_cast<int64_t>(d.k) * d.T / d.E);
}
static int mask_words(const Dims& d) { return ceil_div(d.E, 32); }

size_t batchwise_route_workspace(const Dims& d) {
  return align256(router_clean_workspace(d)) +
         align256(static_cast<size_t>(ceil_div(d.T, kThreads)) * sizeof(int32_t));
}
size_t batchwise_aux_workspace(const Dims& d) {
  return align256(5 * static_cast<size_t>(d.E) * sizeof(double));
}

moe_status batchwise_route_launch(const Dims& d, const void* X, const float* Wg, const float* bias,
                                  float* clean, const moe_batchwise_state* st, void* ws,
                                  int* nonfinite, hipStream_t stream) {
  moe_status s = router_clean_launch(d, X, Wg, bias, clean, ws, nonfinite, stream);
  if (s != MOE_OK) return s;
  int32_t* block_sum = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                  align256(router_clean_workspace(d)));
  const int m = batchwise_m(d), W = mask_words(d);
  bw_softmax<<<ceil_div(d.T, kTileTok), kThreads, 0, stream>>>(clean, d.T, d.E, W, st->probs_t,
                                                                 st->mask);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  bw_select<<<d.E, kSelThreads, 0, stream>>>(st->probs_t, d.T, d.E, m, W, st->sel, st->offsets,
                                             st->mask);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  const int nblk = ceil_div(d.T, kThreads);
  bw_tok_count<<<nblk, kThreads, 0, stream>>>(st->mask, d.T, W, st->tok_count, block_sum);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  bw_tok_scan<<<1, kThreads, 0, stream>>>(block_sum, nblk);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  bw_tok_offsets<<<nblk, kThreads, 0, stream>>>(st->tok_count, block_sum, d.T, st->tok_off);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  const int64_t pairs = static_cast<int64_t>(d.E) * m;
  bw_pairs<<<static_cast<int>(ceil_div64(pairs, 256)), 256, 0, stream>>>(
      st->sel, st->mask, st->tok_off, d.E, m, W, st->tok_row, st->slot_pair);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  bw_gates<<<ceil_div(d.T, 256), 256, 0, stream>>>(st->probs_t, st->tok_off, st->tok_row, d.T, m,
                                                   st->tok_gate);
  return launch_status();
}

moe_status batchwise_dispatch_launch(const Dims& d, const void* X, const moe_batchwise_state* st,
                                     void* Xd, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(d.E) * batchwise_m(d);
  if (d.dtype == MOE_BF16) {
    const auto* x = static_cast<const uint16_t*>(X);
    auto* xd = static_cast<uint16_t*>(Xd);
    if (d.D % 8 == 0)
      bw_gather<uint16_t><<<static_cast<int>(ceil_div64(rows * (d.D / 8), 256)), 256, 0, stream>>>(
          x, st->sel, rows, d.D, xd);
    else
      bw_gather_scalar<uint16_t><<<static_cast<int>(ceil_div64(rows * d.D, 256)), 256, 0, stream>>>(
          x, st->sel, rows, d.D, xd);
  } else {
    const auto* x = static_cast<const float*>(X);
    auto* xd = static_cast<float*>(Xd);
    if (d.D % 4 == 0)
      bw_gather<float><<<static_cast<int>(ceil_div64(rows * (d.D / 4), 256)), 256, 0, stream>>>(
          x, st->sel, rows, d.D, xd);
    else
      bw_gather_scalar<float><<<static_cast<int>(ceil_div64(rows * d.D, 256)), 256, 0, stream>>>(
          x, st->sel, rows, d.D, xd);
  }
  return launch_status();
}

moe_status batchwise_combine_launch(const Dims& d, const void* Z, const moe_batchwise_state* st,
                                    const void* residual, void* Y, int* nonfinite,
                                    hipStream_t stream) {
  const int grid = ceil_div(d.T, kThreads / 64);
  if (d.dtype == MOE_BF16)
    bw_combine<uint16_t><<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(Z), st->tok_off, st->tok_row, st->tok_gate,
        static_cast<const uint16_t*>(residual), d.T, d.D, static_cast<uint16_t*>(Y), nonfinite);
  else
    bw_combine<float><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(Z), st->tok_off, st->tok_row, st->tok_gate,
        static_cast<const float*>(residual), d.T, d.D, static_cast<float*>(Y), nonfinite);
  return launch_status();
}

moe_status batchwise_aux_launch(const Dims& d, const moe_batchwise_state* st,
                                const float* thresholds, float* importance, float* out, void* ws,
                                hipStream_t stream) {
  BwAuxArgs a;
  a.probs_t = st->probs_t;
  a.mask = st->mask;
  a.tok_count = st->tok_count;
  a.tok_gate = st->tok_gate;
  a.slot_pair = st->slot_pair;
  a.thresholds = thresholds;
  a.per_expert = static_cast<double*>(ws);
  a.importance = importance;
  a.out = out;
  a.T = d.T;
  a.E = d.E;
  a.m = batchwise_m(d);
  a.W = mask_words(d);
  bw_aux_expert<<<d.E, kThreads, 0, stream>>>(a);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  bw_aux_final<<<1, kThreads, 0, stream>>>(a);
  return launch_status();
}

}  // namespace moe
