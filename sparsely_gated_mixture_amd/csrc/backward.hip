// Backward pass of the MoE layer with a per-token gate (noisy top-k or Switch top-1).
//
// The pages' purpose is training: "Outrageously Large Neural Networks" summary,
// section 3.4 (k > 1 so the gate receives gradient through the softmax over the
// kept experts; the importance and load losses train the gate towards balance);
// the "Mixture-of-Experts: Sparse Computation" lesson, chapter 3, traces the
// backward pass: an incoming gradient splits over the kept experts in
// proportion to their gates, and masked experts are absent from it. The
// selection and the capacity mask are piecewise constant and held fixed, as is
// the noise sample (H = clean + eps * Softplus(raw)); the load estimator's
// threshold is another expert's score and passes its gradient to it. The
// "Switch Transformer" explainer, steps 2 and 8: the Switch gate is the selected
// expert's full-softmax probability, and the balancing term reaches every
// probability through its batch mean (the dispatch fractions are counts, fixed).
//
// Objective: <Y, dY> + w_imp CV^2(Importance) + w_load CV^2(Load) (noisy top-k) or
// <Y, dY> + w_imp CV^2(Importance) + w_switch E sum_e f_e Pbar_e (Switch).
//
// Kernels:
//   cb_backward      a wave per token: dZ[row] = g * dY[t] for each accepted
//                    assignment and dg = <dY[t], Z[row]> (fp32)
//   cv2_grad         d CV^2 / d v for the importance and load vectors
//   gate_backward    4 token rows per wave, one at a time: softmax backward over
//                    the kept scores (plus the importance term), the load term of
//                    every expert through Phi (with the threshold's share going to
//                    the k-th / (k+1)-th expert; their noise redrawn by Philox),
//                    then d raw = d std * sigmoid(raw); writes [dclean | draw]
//                    [T, 2E] and per-block sums of dclean (the bias gradient)
//   switch_dprob,    the Switch gate: the balancing term's share of every
//   switch_gate_backward  probability, then per row dclean = p (dp - <p, dp>)
//   column_sums      the per-block sums, in two passes, in a fixed order
//   wgrad_gemm_tr    per group (and row split), C = A^T B over the group's rows (fp32
//                    output), bf16 with widths that are multiples of 8: operands
//                    row-major in LDS, transposed by the LDS transpose read into MFMA
//                    fragments; 128 x 256 tiles; fixed row order
//   wgrad_gemm       the same for fp32 and for widths that are not multiples of 8:
//                    4x4 / 8x8 register transposes put both operands k-contiguous in
//                    LDS; 128 x 128 tiles. Either way the router's weight gradient (one
//                    group of T rows) is split over rows and the splits summed in order
//                    (split_dw)
//   dx_final         a wave per token: dX = dY + sum of the accepted rows of dXd
//                    + the router's share, fp32 accumulation, one rounding
// The dense GEMMs of the backward (dZ W2^T with the ReLU mask, dH W1^T and the
// router's [dclean | draw] [Wg | Wnoise]^T) run on the forward's grouped GEMM
// kernel with transposed packed weights.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "noise.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Lanes of one wave exchanging values through LDS: the wave executes in lockstep and its LDS
// accesses complete in issue order, so it is enough to keep the compiler from moving memory
// operations across this point.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ------------------------------------------------------------------ combine backward
// 16-byte vectors along D when D is a multiple of the vector width, else one element a lane.
template <typename T>
__global__ __launch_bounds__(kThreads) void cb_backward(
    const T* __restrict__ dY, const T* __restrict__ Z, const int32_t* __restrict__ ids,
    const float* __restrict__ gates, const int32_t* __restrict__ pos,
    const uint8_t* __restrict__ accepted, const int32_t* __restrict__ offsets, int Tn, int D, int k,
    T* __restrict__ dZ, float* __restrict__ dgates) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const bool vec = (D % V) == 0;
  const T* dy = dY + static_cast<int64_t>(t) * D;
  for (int j = 0; j < k; ++j) {
    const int64_t gi = static_cast<int64_t>(t) * k + j;
    if (!accepted[gi]) {
      if (lane == 0) dgates[gi] = 0.f;
      continue;
    }
    const int64_t row = static_cast<int64_t>(offsets[ids[gi]]) + pos[gi];
    const float g = gates[gi];
    const T* z = Z + row * D;
    T* dz = dZ + row * D;
    float dot = 0.f;
    if (vec) {
      for (int c = lane; c < D / V; c += 64) {
        const uint4 yv = reinterpret_cast<const uint4*>(dy)[c];
        const uint4 zv = reinterpret_cast<const uint4*>(z)[c];
        const T* yp = reinterpret_cast<const T*>(&yv);
        const T* zp = reinterpret_cast<const T*>(&zv);
        T out[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const float y = Elem<T>::to_f32(yp[i]);
          dot = fmaf(y, Elem<T>::to_f32(zp[i]), dot);
          out[i] = Elem<T>::from_f32(g * y);
        }
        reinterpret_cast<uint4*>(dz)[c] = *reinterpret_cast<const uint4*>(out);
      }
    } else {
      for (int c = lane; c < D; c += 64) {
        const float y = Elem<T>::to_f32(dy[c]);
        dot = fmaf(y, Elem<T>::to_f32(z[c]), dot);
        dz[c] = Elem<T>::from_f32(g * y);
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) dgates[gi] = dot;
  }
}

// ------------------------------------------------------------------ d CV^2 / d v
// CV^2 = var / mean^2 (population variance): d/dv_e = 2 / (E mean^2) * ((v_e - mean) - var / mean)
__global__ __launch_bounds__(kThreads) void cv2_grad(const float* __restrict__ v, int E, float w,
                                                    float* __restrict__ dv) {
  __shared__ double sh[kThreads];
  double s = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) s += v[e];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int n = kThreads / 2; n >= 1; n >>= 1) {
    if (threadIdx.x < n) sh[threadIdx.x] += sh[threadIdx.x + n];
    __syncthreads();
  }
  const double mean = sh[0] / E;
  __syncthreads();
  double q = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) q += (v[e] - mean) * (v[e] - mean);
  sh[threadIdx.x] = q;
  __syncthreads();
  for (int n = kThreads / 2; n >= 1; n >>= 1) {
    if (threadIdx.x < n) sh[threadIdx.x] += sh[threadIdx.x + n];
    __syncthreads();
  }
  const double var = sh[0] / E;
  for (int e = threadIdx.x; e < E; e += kThreads)
    dv[e] = (w == 0.f || mean == 0.0) ? 0.f
                                      : static_cast<float>(w * 2.0 / (E * mean * mean) *
                                                           ((v[e] - mean) - var / mean));
}

// ------------------------------------------------------------------ gate backward
struct GateArgs {
  const int32_t* ids;
  const float* gates;
  const float* clean;
  const float* std_in;
  const float* row_stats;
  const float* dgates;
  const float* dimp;   // [E] importance term or NULL
  const float* dload;  // [E] load term or NULL (needs noise)
  const float* eps;    // [T, E] the noise the forward was given, or NULL (redrawn by Philox)
  const float* scores; // [T, E] the forward's noisy scores H, or NULL (formed again)
  void* dcat;          // [T, ldc] act dtype: dclean | draw (draw only with noise)
  int ldc;             // 2E with noise, else E
  float* dbias_part;   // [nblk][E] or NULL
  uint64_t seed;
  int T, E, k, noise, dtype;
};

__device__ __forceinline__ float phi_pdf(float z) { return 0.3989422804014327f * expf(-0.5f * z * z); }

constexpr int kGateRowsPerWave = 4;

// The forward's noise sample for (t, e): the given eps, else the same Philox draw.
__device__ __forceinline__ float noise_at(const GateArgs& a, int t, int64_t base, int e) {
  if (a.eps) return a.eps[base + e];
  float g4[4];
  noise4(a.seed, 0, t, e >> 2, g4);
  return g4[e & 3];
}

// W waves per block (blockDim.x / 64: 4, or 2 when E is large) take rows
// (blockIdx.x * kGateRowsPerWave + i) * W + wave, i < kGateRowsPerWave. A wave keeps its row's
// dclean and dstd in LDS, plus its running sum of dclean (the bias gradient). Every wave runs
// every phase of every row (rows past T only skip their memory accesses), so the phases can be
// separated by block barriers.
__global__ __launch_bounds__(kThreads) void gate_backward(GateArgs a) {
  extern __shared__ float sh[];  // [W][3][E]: dclean, dstd, sum of dclean
  const int W = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  float* dcl = sh + wave * 3 * E;
  float* dsd = dcl + E;
  float* acc = dsd + E;
  const bool load_term = a.noise && a.dload;
  for (int e = lane; e < E; e += 64) acc[e] = 0.f;
  // The noise the gradient needs is drawn for the wave's rows together, so that one Philox and
  // Box-Muller evaluation serves many lanes: lane it * k + j draws row it's j-th kept expert's
  // noise here; the (k+1)-th expert's noise term of each row is applied after the loop (lane
  // it keeps that row's pending term).
  float nzk = 0.f;
  if (a.noise && lane < kGateRowsPerWave * k) {
    const int it = lane / k, j = lane - it * k;
    const int t = (blockIdx.x * kGateRowsPerWave + it) * W + wave;
    if (t < a.T) nzk = noise_at(a, t, static_cast<int64_t>(t) * E, a.ids[static_cast<int64_t>(t) * k + j]);
  }
  int pend_bi = -1, pend_t = 0;
  float pend_s = 0.f, pend_d = 0.f;
  for (int it = 0; it < kGateRowsPerWave; ++it) {
    const int t = (blockIdx.x * kGateRowsPerWave + it) * W + wave;
    const bool live = t < a.T;
    const int64_t base = static_cast<int64_t>(live ? t : 0) * E;
    const int32_t* rid = a.ids + static_cast<int64_t>(live ? t : 0) * k;
    for (int e = lane; e < E; e += 64) {
      dcl[e] = 0.f;
      dsd[e] = 0.f;
    }
    wave_sync();
    // softmax backward over the kept scores (plus the importance term)
    const float nz = __shfl(nzk, it * k + (lane < k ? lane : 0));  // lanes < k: their kept expert's
    {
      float gj = 0.f, dgj = 0.f;
      int ej = 0;
      if (live && lane < k) {
        const int64_t gi = static_cast<int64_t>(t) * k + lane;
        ej = a.ids[gi];
        gj = a.gates[gi];
        dgj = a.dgates[gi] + (a.dimp ? a.dimp[ej] : 0.f);
      }
      const float s = wave_sum(gj * dgj);
      if (live && lane < k) {
        const float dh = gj * (dgj - s);
        dcl[ej] += dh;  // a row's experts are distinct: no two lanes share ej
        if (a.noise) dsd[ej] += dh * nz;
      }
    }
    wave_sync();
    // load term: P(t,e) = Phi((clean - thr) / std) for every expert; the threshold is v_{k+1}
    // for the kept experts and v_k for the others. A lane takes 4 consecutive experts (one
    // Philox draw) at a time.
    float s_in = 0.f, s_out = 0.f;
    int bi = 0x7fffffff;
    if (load_term) {
      float best = -INFINITY;
      if (live) {
        const float vk = a.row_stats[2 * static_cast<int64_t>(t)];
        const float vk1 = a.row_stats[2 * static_cast<int64_t>(t) + 1];
        for (int q = lane; 4 * q < E; q += 64) {
          float g4[4] = {0.f, 0.f, 0.f, 0.f};
          if (a.scores) {
            // H comes from the forward: no noise is needed for the non-kept experts
          } else if (a.eps) {
#pragma unroll
            for (int i = 0; i < 4; ++i) g4[i] = 4 * q + i < E ? a.eps[base + 4 * q + i] : 0.f;
          } else {
            noise4(a.seed, 0, t, q, g4);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * q + i;
            if (e >= E) break;
            bool inside = false;
            for (int j = 0; j < k; ++j) inside |= rid[j] == e;
            const float cl = a.clean[base + e], sd = a.std_in[base + e];
            if (!inside) {  // candidate for v_{k+1}: H exactly as the router formed it
              const float h = a.scores ? a.scores[base + e] : fmaf(sd, g4[i], cl);
              if (h > best || (h == best && e < bi)) {
                best = h;
                bi = e;
              }
            }
            const float thr = inside ? vk1 : vk;
            if (!(sd > 0.f) || thr == -INFINITY) continue;
            const float z = (cl - thr) / sd;
            const float dz = a.dload[e] * phi_pdf(z);
            dcl[e] += dz / sd;
            dsd[e] -= dz * z / sd;
            if (inside) s_in += dz / sd;
            else s_out += dz / sd;
          }
        }
      }
      s_in = wave_sum(s_in);
      s_out = wave_sum(s_out);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        if (ob > best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
    }
    const float nz_k = __shfl(nzk, it * k + k - 1);  // v_k's expert is the k-th kept one
    // v_{k+1}: the best other expert; its d std term (noise x s_in) is deferred
    const bool defer = load_term && live && k < E && bi < E;
    wave_sync();
    if (load_term && live && lane == 0) {
      const int ik = rid[k - 1];  // v_k: the last kept expert
      dcl[ik] -= s_out;
      dsd[ik] -= s_out * nz_k;
      if (defer) dcl[bi] -= s_in;
    }
    wave_sync();
    if (defer && lane == it) {
      pend_bi = bi;
      pend_t = t;
      pend_s = s_in;
      pend_d = dsd[bi];
    }
    // write [dclean | draw]; d raw = d std * sigmoid(raw) = d std * (1 - exp(-std))
    if (live) {
      const int64_t o = static_cast<int64_t>(t) * a.ldc;
      for (int e = lane; e < E; e += 64) {
        if (a.dtype == MOE_BF16) {
          uint16_t* d = static_cast<uint16_t*>(a.dcat);
          d[o + e] = f32_to_bf16(dcl[e]);
          if (a.noise && !(defer && e == bi))
            d[o + E + e] = f32_to_bf16(dsd[e] * (1.f - expf(-a.std_in[base + e])));
        } else {
          float* d = static_cast<float*>(a.dcat);
          d[o + e] = dcl[e];
          if (a.noise && !(defer && e == bi)) d[o + E + e] = dsd[e] * (1.f - expf(-a.std_in[base + e]));
        }
        acc[e] += dcl[e];
      }
    }
    // the next row clears this lane's own entries before its first barrier
  }
  // the deferred d raw of each row's (k+1)-th expert: its d std less s_in x its noise
  if (pend_bi >= 0) {
    const int64_t bt = static_cast<int64_t>(pend_t) * E;
    const float v = pend_d - pend_s * noise_at(a, pend_t, bt, pend_bi);
    const float r = v * (1.f - expf(-a.std_in[bt + pend_bi]));
    const int64_t o = static_cast<int64_t>(pend_t) * a.ldc + E + pend_bi;
    if (a.dtype == MOE_BF16) static_cast<uint16_t*>(a.dcat)[o] = f32_to_bf16(r);
    else static_cast<float*>(a.dcat)[o] = r;
  }
  // bias gradient partial: each wave's rows in order, then the waves in order
  if (a.dbias_part) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      float s2 = 0.f;
      for (int w = 0; w < W; ++w) s2 += sh[w * 3 * E + 2 * E + e];
      a.dbias_part[static_cast<int64_t>(blockIdx.x) * E + e] = s2;
    }
  }
}

// ------------------------------------------------------------------ Switch gate backward
// The gate is the selected expert's probability under the full softmax of the clean logits
// (not renormalised); the balancing term w * E * sum f * Pbar reaches every probability as
// dprob[e] = w * E * f_e / T with f = count / T held fixed. Per row: dp = dprob + dG at the
// selected expert, dclean = p * (dp - <p, dp>).
struct SwitchGateArgs {
  const int32_t* ids;    // [T] (k = 1)
  const float* clean;    // [T, E]
  const float* dgates;   // [T]
  const float* dimp;     // [E] importance term or NULL
  const float* dprob;    // [E] balancing term or NULL
  void* dcat;            // [T, E] act dtype: dclean
  float* dbias_part;     // [nblk][E] or NULL
  int T, E, dtype;
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__global__ void switch_dprob(const int32_t* __restrict__ counts, int T, int E, float w,
                             float* __restrict__ dprob) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E)
    dprob[e] = static_cast<float>(static_cast<double>(w) * E * counts[e] /
                                  (static_cast<double>(T) * T));
}

// Rows as gate_backward (W waves, kGateRowsPerWave rows each); a wave keeps the running sum of
// its rows' dclean in LDS for the bias gradient.
__global__ __launch_bounds__(kThreads) void switch_gate_backward(SwitchGateArgs a) {
  extern __shared__ float sh[];  // [W][E]
  const int W = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int E = a.E;
  float* acc = sh + wave * E;
  for (int e = lane; e < E; e += 64) acc[e] = 0.f;
  for (int it = 0; it < kGateRowsPerWave; ++it) {
    const int t = (blockIdx.x * kGateRowsPerWave + it) * W + wave;
    if (t >= a.T) continue;  // wave-uniform; no barrier inside the loop
    const float* cl = a.clean + static_cast<int64_t>(t) * E;
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, cl[e]);
    m = wave_max(m);
    float z = 0.f;
    for (int e = lane; e < E; e += 64) z += expf(cl[e] - m);
    z = wave_sum(z);
    const int es = a.ids[t];
    const float dG = a.dgates[t] + (a.dimp ? a.dimp[es] : 0.f);
    float pd = 0.f;
    if (a.dprob)
      for (int e = lane; e < E; e += 64) pd += expf(cl[e] - m) / z * a.dprob[e];
    const float dot = wave_sum(pd) + expf(cl[es] - m) / z * dG;
    const int64_t o = static_cast<int64_t>(t) * E;
    for (int e = lane; e < E; e += 64) {
      const float pe = expf(cl[e] - m) / z;
      const float dp = (a.dprob ? a.dprob[e] : 0.f) + (e == es ? dG : 0.f);
      const float dc = pe * (dp - dot);
      if (a.dtype == MOE_BF16) static_cast<uint16_t*>(a.dcat)[o + e] = f32_to_bf16(dc);
      else static_cast<float*>(a.dcat)[o + e] = dc;
      acc[e] += dc;
    }
  }
  if (a.dbias_part) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      float s2 = 0.f;
      for (int w = 0; w < W; ++w) s2 += sh[w * E + e];
      a.dbias_part[static_cast<int64_t>(blockIdx.x) * E + e] = s2;
    }
  }
}

// Column sums of a [R, E] fp32 matrix over row slices: out[slice][e] = sum of rows
// slice*per .. min(R, (slice+1)*per) - 1, with per = ceil(R / gridDim.y); four interleaved row
// sets of the slice, each in row order, then the four in order (deterministic).
__global__ __launch_bounds__(kThreads) void column_sums(const float* __restrict__ part, int R,
                                                       int E, float* __restrict__ out) {
  __shared__ double sh[4][64];
  const int el = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + el;
  const int per = (R + gridDim.y - 1) / gridDim.y;
  const int b0 = blockIdx.y * per, b1 = min(R, b0 + per);
  double s = 0;
  if (e < E)
    for (int b = b0 + r; b < b1; b += 4) s += part[static_cast<int64_t>(b) * E + e];
  sh[r][el] = s;
  __syncthreads();
  if (r == 0 && e < E)
    out[static_cast<int64_t>(blockIdx.y) * E + e] =
        static_cast<float>(sh[0][el] + sh[1][el] + sh[2][el] + sh[3][el]);
}

// [Wg | Wnoise]^T packed for the router's input gradient: B[k][n] = Wg[n][k] (k < E) or
// Wnoise[n][k - E], cast to the activation dtype; one thread per (column block, k-step, lane),
// written where the grouped GEMM's fragment strides put it (one expert).
template <typename T>
__global__ void router_pack_t(const float* __restrict__ Wg, const float* __restrict__ Wn, int D,
                              int E, int NB, int KS, PackStrides ps, uint4* __restrict__ out) {
  constexpr int V = Elem<T>::kVec;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(NB) * KS * kWave) return;
  const int lane = static_cast<int>(idx % kWave);
  const int ks = static_cast<int>((idx / kWave) % KS);
  const int nb = static_cast<int>(idx / (static_cast<int64_t>(kWave) * KS));
  const int n = nb * 32 + (lane & 31);
  const int k0 = ks * 2 * V + (lane >> 5) * V;
  T v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int kk = k0 + i;
    float x = 0.f;
    if (n < D && kk < 2 * E) x = kk < E ? Wg[static_cast<int64_t>(n) * E + kk]
                                        : (Wn ? Wn[static_cast<int64_t>(n) * E + kk - E] : 0.f);
    v[i] = Elem<T>::from_f32(x);
  }
  out[(nb * ps.block + (ks / 4) * ps.stage + ks % 4) * kWave + lane] = *reinterpret_cast<const uint4*>(v);
}

__global__ void set_offsets(int32_t* off, int T) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = T;
  }
}

// ------------------------------------------------------------------ weight-gradient GEMM
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ f32x16 wmma(u32x4 a, u32x4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 wmma<uint16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 wmma<float>(u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s]), __uint_as_float(b[s]), c, 0, 0, 0);
  return c;
}

// VB x VB block transpose of 16-byte rows (VB = 16 / sizeof(T)): in[r] holds row r,
// out[c] holds column c.
template <typename T> __device__ __forceinline__ void transpose_block(const u32x4 (&in)[16 / sizeof(T)],
                                                                       u32x4 (&out)[16 / sizeof(T)]);
template <> __device__ __forceinline__ void transpose_block<float>(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = u32x4{in[0][c], in[1][c], in[2][c], in[3][c]};
}
template <> __device__ __forceinline__ void transpose_block<uint16_t>(const u32x4 (&in)[8], u32x4 (&out)[8]) {
  // step 1: within each pair of rows (2a, 2a+1), pair up the 16-bit halves of each dword:
  // p[2a][j] = (row 2a col 2j, row 2a+1 col 2j), p[2a+1][j] = (row 2a col 2j+1, row 2a+1 col 2j+1)
  unsigned p[8][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned x = in[2 * a][j], y = in[2 * a + 1][j];
      p[2 * a][j] = (x & 0xffffu) | (y << 16);
      p[2 * a + 1][j] = (x >> 16) | (y & 0xffff0000u);
    }
  // step 2: column c (rows 0..7) is the dwords of row pairs 0..3 for that column
#pragma unroll
  for (int c = 0; c < 8; ++c)
    out[c] = u32x4{p[0 + (c & 1)][c >> 1], p[2 + (c & 1)][c >> 1], p[4 + (c & 1)][c >> 1],
                   p[6 + (c & 1)][c >> 1]};
}

struct WgradArgs {
  const void* A;   // [rows, M]
  const void* B;   // [rows, N]
  const int32_t* offsets;  // [G + 1]
  float* C;        // [G][S][M][N]: split s of group g's rows
  int G, M, N, S;
};

constexpr int kWT = 128;            // tile M and N
constexpr int kWRows = 64;          // rows (the reduction) per stage
constexpr int kXcds = 8;

// One block per (group, row split, m tile, n tile): C_gs[m, n] = sum over the split's rows r
// of A[r, m] B[r, n]; 4 waves in a 2 x 2 layout, each 64 x 64. The next stage's global loads
// are issued before the current stage's MFMAs. Blocks are remapped so that each XCD (blocks
// are dealt round-robin over the 8 XCDs) takes a contiguous run of (group, split, tile): a
// group's operands then stay in one XCD's L2. Within a group the tiles run along the
// smaller output dimension first, so that the blocks in flight together cover all of the
// smaller operand and a contiguous part of the larger one (each then comes from memory about
// once, instead of the larger one once per sweep along the other dimension).
template <typename T, bool kAligned, bool kRowSplit>
__global__ __launch_bounds__(kThreads) void wgrad_gemm(WgradArgs a) {
  constexpr int VB = 16 / static_cast<int>(sizeof(T));   // elements per 16 bytes
  constexpr int kLine = kWRows * static_cast<int>(sizeof(T));  // LDS bytes per column line
  constexpr int kQ = kLine / 16;                                   // 16-byte quads per line
  // quad q of line l sits at quad (q + l + l / VB) % kQ, so that neighbouring lanes of one
  // stash write (lines VB apart) and of one fragment read (consecutive lines) hit distinct
  // quads (LDS banks)
  auto qaddr = [](int line, int q) { return line * kLine + ((q + line + line / VB) % kQ) * 16; };
  // per stage: A tile [kWRows][kWT] and B tile [kWRows][kWT] -> transposed into
  // lines [kWT][kWRows] (k contiguous)
  __shared__ __align__(16) unsigned char sA[kWT * kLine];
  __shared__ __align__(16) unsigned char sB[kWT * kLine];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int mt = (a.M + kWT - 1) / kWT, nt = (a.N + kWT - 1) / kWT;
  const int tiles = mt * nt;
  const int S = kRowSplit ? a.S : 1;  // the row-split instance serves the router's gradient
  const int total = a.G * S * tiles;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (logical >= total) return;
  const int gs = logical / tiles;  // group * S + split
  const int g = gs / S, sp = gs - g * S;
  const int rem = logical - gs * tiles;
  const int m0 = (a.N > a.M ? rem % mt : rem / nt) * kWT, n0 = (a.N > a.M ? rem / mt : rem % nt) * kWT;
  const int gb = a.offsets[g], ge = a.offsets[g + 1];
  const int chunk = ((ge - gb + S - 1) / S + kWRows - 1) / kWRows * kWRows;
  const int r_begin = min(ge, gb + sp * chunk), r_end = min(ge, r_begin + chunk);
  const T* A = static_cast<const T*>(a.A);
  const T* B = static_cast<const T*>(a.B);
  // loader: blocks of VB rows x VB columns; (kWRows / VB) x (kWT / VB) per operand
  constexpr int kBR = kWRows / VB, kBC = kWT / VB, kBlocks = kBR * kBC;  // per operand
  constexpr int kPer = 2 * kBlocks / kThreads;                            // per thread
  static_assert(kPer * kThreads == 2 * kBlocks, "loader blocks must split evenly");
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  u32x4 in[kPer][VB];
  // kAligned (M and N multiples of VB): every lane issues its loads unconditionally from a
  // clamped in-bounds address, and the rows / columns past the edge are zeroed in stash, so
  // the loads of a stage are all in flight together.
  unsigned vmask[kPer];  // bit i: row i of the lane's block is inside the split and the tile
  auto load = [&](int rs) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int bidx = tid + p * kThreads;
      const bool isA = bidx < kBlocks;
      const int b2 = isA ? bidx : bidx - kBlocks;
      const int rb = b2 / kBC, cb = b2 - rb * kBC;
      const T* src = isA ? A : B;
      const int ld = isA ? a.M : a.N;
      const int c0 = (isA ? m0 : n0) + cb * VB;
      if constexpr (kAligned) {
        const int cc = min(c0, ld - VB);
        unsigned m = 0;
#pragma unroll
        for (int i = 0; i < VB; ++i) {
          const int r = rs + rb * VB + i;
          m |= (r < r_end && c0 < ld) ? (1u << i) : 0u;
          in[p][i] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(min(r, r_end - 1)) * ld + cc);
        }
        vmask[p] = m;
      } else {
#pragma unroll
        for (int i = 0; i < VB; ++i) {
          const int r = rs + rb * VB + i;
          T tmp[VB];
#pragma unroll
          for (int q = 0; q < VB; ++q)
            tmp[q] = (r < r_end && c0 + q < ld) ? src[static_cast<int64_t>(r) * ld + c0 + q] : T(0);
          in[p][i] = *reinterpret_cast<const u32x4*>(tmp);
        }
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int bidx = tid + p * kThreads;
      const bool isA = bidx < kBlocks;
      const int b2 = isA ? bidx : bidx - kBlocks;
      const int rb = b2 / kBC, cb = b2 - rb * kBC;
      if constexpr (kAligned) {
#pragma unroll
        for (int i = 0; i < VB; ++i)
          if (!((vmask[p] >> i) & 1u)) in[p][i] = u32x4{0u, 0u, 0u, 0u};
      }
      u32x4 out[VB];
      transpose_block<T>(in[p], out);
      unsigned char* dst = isA ? sA : sB;
#pragma unroll
      for (int c = 0; c < VB; ++c)
        *reinterpret_cast<u32x4*>(dst + qaddr(cb * VB + c, rb)) = out[c];
    }
  };
  if (r_begin < r_end) load(r_begin);
  for (int rs = r_begin; rs < r_end; rs += kWRows) {
    stash();
    __syncthreads();
    if (rs + kWRows < r_end) load(rs + kWRows);
    // MFMA over the stage: k-steps of 2*VB rows (one 16-byte fragment per lane half)
#pragma unroll
    for (int ks = 0; ks < kWRows / (2 * VB); ++ks) {
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = wm * 64 + i * 32 + (lane & 31);
        fa[i] = *reinterpret_cast<const u32x4*>(sA + qaddr(m, ks * 2 + (lane >> 5)));
        const int n = wn * 64 + i * 32 + (lane & 31);
        fb[i] = *reinterpret_cast<const u32x4*>(sB + qaddr(n, ks * 2 + (lane >> 5)));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = wmma<T>(fa[i], fb[j], acc[i][j]);
    }
    __syncthreads();
  }
  // fp32 output tile
  float* C = a.C + static_cast<int64_t>(gs) * a.M * a.N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + wm * 64 + i * 32 + acc_row(lane, q);
        if (m < a.M && n < a.N) C[static_cast<int64_t>(m) * a.N + n] = acc[i][j][q];
      }
    }
}

// bf16 weight gradient (M and N multiples of 8): both operands are copied row-major into LDS
// as they come from memory, and transposed on the way out by gfx950's LDS transpose read
// (ds_read_b64_tr_b16): in a group of 16 lanes whose lane 4j + q points at row k0 + j,
// columns c0 + 4q .. c0 + 4q + 3, lane i receives column c0 + i of rows k0 .. k0 + 3. Two
// such reads give a lane the 8 k-values of its MFMA operand, with no VALU transposes. A block
// computes a 128 x 256 tile (waves 2 x 2, each 64 x 128); the next 64-row stage's loads are
// in flight during the current stage's MFMAs, and within a stage the transpose reads of the
// next 16-row k-step are interleaved with the current one's MFMAs. Rows past the end of the
// split are zeroed in A only (a zero in either factor removes the product); columns past
// M / N are clamped reads that only feed outputs never stored. Tiles are ordered as in
// wgrad_gemm. LDS rows are padded by 32 bytes so that the four rows of one transpose read
// fall in different banks.
typedef short v4s16 __attribute__((ext_vector_type(4)));
constexpr int kTrRow = kWT * 2 + 32;  // LDS bytes per k row: 128 bf16 + 32 pad (bank rotation)

__device__ __forceinline__ unsigned long long tr_read(const unsigned char* lds_base, int byte_off) {
  typedef __attribute__((address_space(3))) v4s16* lptr;
  typedef __attribute__((address_space(3))) unsigned char* lbyte;
  const v4s16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lptr)((lbyte)(lds_base) + byte_off));
  return __builtin_bit_cast(unsigned long long, v);
}

constexpr int kTN2 = 256;                // tile N of the transpose-read kernel
constexpr int kTrRowB = kTN2 * 2 + 32;   // LDS bytes per k row of B

template <bool kRowSplit>
__global__ __launch_bounds__(kThreads) void wgrad_gemm_tr(WgradArgs a) {
  __shared__ __align__(16) unsigned char sA[kWRows * kTrRow];
  __shared__ __align__(16) unsigned char sB[kWRows * kTrRowB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int mt = (a.M + kWT - 1) / kWT, nt = (a.N + kTN2 - 1) / kTN2;
  const int tiles = mt * nt;
  const int S = kRowSplit ? a.S : 1;
  const int total = a.G * S * tiles;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (logical >= total) return;
  const int gs = logical / tiles;
  const int g = gs / S, sp = gs - g * S;
  const int rem = logical - gs * tiles;
  const int m0 = (a.N > a.M ? rem % mt : rem / nt) * kWT, n0 = (a.N > a.M ? rem / mt : rem % nt) * kTN2;
  const int gb = a.offsets[g], ge = a.offsets[g + 1];
  const int chunk = ((ge - gb + S - 1) / S + kWRows - 1) / kWRows * kWRows;
  const int r_begin = min(ge, gb + sp * chunk), r_end = min(ge, r_begin + chunk);
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  // loader: A 64 rows x 16 segments (4 per thread), B 64 rows x 32 segments (8 per thread)
  constexpr int kSA = kWRows * 16 / kThreads, kSB = kWRows * 32 / kThreads;
  u32x4 ina[kSA], inb[kSB];
  const int csa = tid & 15, csb = tid & 31;
  const int ca = min(m0 + csa * 8, a.M - 8), cb = min(n0 + csb * 8, a.N - 8);
  auto load = [&](int rs) {
#pragma unroll
    for (int p = 0; p < kSA; ++p) {
      const int row = (tid >> 4) + p * 16;
      ina[p] = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(min(rs + row, r_end - 1)) * a.M + ca);
    }
#pragma unroll
    for (int p = 0; p < kSB; ++p) {
      const int row = (tid >> 5) + p * 8;
      inb[p] = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(min(rs + row, r_end - 1)) * a.N + cb);
    }
  };
  auto stash = [&](int rs) {
    const bool tail = rs + kWRows > r_end;
#pragma unroll
    for (int p = 0; p < kSA; ++p) {
      const int row = (tid >> 4) + p * 16;
      u32x4 v = ina[p];
      if (tail && rs + row >= r_end) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sA + row * kTrRow + csa * 16) = v;
    }
#pragma unroll
    for (int p = 0; p < kSB; ++p) {
      const int row = (tid >> 5) + p * 8;
      *reinterpret_cast<u32x4*>(sB + row * kTrRowB + csb * 16) = inb[p];
    }
  };
  const int wm = wave >> 1, wn = wave & 1;  // wave tile 64 (m) x 128 (n)
  const int gq = lane >> 4, jr = (lane >> 2) & 3, qc = lane & 3;
  const int rowq = 8 * (gq >> 1) + jr, colq = 16 * (gq & 1) + 4 * qc;
  // the wave's operand fragments of k-step ks (16 rows of the stage)
  auto frags = [&](int ks, u32x4 (&fa)[2], u32x4 (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int oa = (ks * 16 + rowq) * kTrRow + (wm * 64 + i * 32 + colq) * 2;
      const unsigned long long a0 = tr_read(sA, oa), a1 = tr_read(sA, oa + 4 * kTrRow);
      fa[i] = u32x4{static_cast<unsigned>(a0), static_cast<unsigned>(a0 >> 32),
                    static_cast<unsigned>(a1), static_cast<unsigned>(a1 >> 32)};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ob = (ks * 16 + rowq) * kTrRowB + (wn * 128 + j * 32 + colq) * 2;
      const unsigned long long b0 = tr_read(sB, ob), b1 = tr_read(sB, ob + 4 * kTrRowB);
      fb[j] = u32x4{static_cast<unsigned>(b0), static_cast<unsigned>(b0 >> 32),
                    static_cast<unsigned>(b1), static_cast<unsigned>(b1 >> 32)};
    }
  };
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[i][j][t] = 0.f;
  if (r_begin < r_end) load(r_begin);
  for (int rs = r_begin; rs < r_end; rs += kWRows) {
    stash(rs);
    __syncthreads();
    if (rs + kWRows < r_end) load(rs + kWRows);
    // two fragment sets: the reads of k-step ks + 1 are issued between k-step ks's MFMAs
    u32x4 fa[2][2], fb[2][4];
    frags(0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < kWRows / 16; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < kWRows / 16) frags(ks + 1, fa[c ^ 1], fb[c ^ 1]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = wmma<uint16_t>(fb[c][j], fa[c][i], acc[i][j]);
    }
    // the order the scheduler keeps: the first k-step's 12 transpose reads, then per k-step
    // one MFMA after each pair of the next k-step's reads, and the last k-step's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int ks = 0; ks < kWRows / 16 - 1; ++ks) {
#pragma unroll
      for (int x = 0; x < 6; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __syncthreads();
  }
  // fp32 output tile: the MFMAs take B's fragment as their first operand, so the accumulator
  // holds the tile transposed: lane l has C[m = .. + l % 32][n = .. + 8 (t / 4) + 4 (l / 32)
  // + t % 4], four consecutive n per register quad, stored as one 16-byte vector
  float* C = a.C + static_cast<int64_t>(gs) * a.M * a.N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + i * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 128 + j * 32 + 8 * q + 4 * (lane >> 5);
        if (m < a.M && n < a.N)
          *reinterpret_cast<f32x4*>(C + static_cast<int64_t>(m) * a.N + n) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      }
    }
}

// ------------------------------------------------------------------ 256 x 256 weight gradients
// bf16 operands, M and N multiples of 256, one row split: one persistent block of 8 waves per
// CU walks a list of (group, 256 x 256 output tile)s, each wave accumulating a 128 x 64 part
// (128 fp32 accumulators a lane), two waves a SIMD: a wave's instructions issue in order, and
// while one is held at a load or LDS read the other's MFMAs run (4 waves of 128 x 128 were
// 4-6% slower). Waves 0-3 issue the loads, waves 4-7 only read LDS and compute. A tile's
// operand bytes per stage feed 256 rows and 256 columns, half of what the 128 x 256 kernel
// above moves per FLOP.
//   * A stage is 64 rows of the reduction: the tile's 256 columns of A and of B for those rows,
//     512 bytes a row, brought to LDS by direct global-to-LDS loads (16 bytes a lane, two rows
//     an instruction, whole 128-byte lines) from per-lane 64-bit addresses. Rows past the group
//     are read from a row of zeros, so the tail of a group adds nothing and no row is read twice.
//     In LDS the 16-byte chunks of row r sit at chunk ^ 4 (r % 4): the transpose reads of an
//     MFMA fragment (four rows of 32 or 64 bytes) then fall on distinct banks (no bank-conflict
//     cycles in the counters; chunk ^ 2 (r % 4) had 1.6 per LDS instruction).
//   * The stages of all of a block's tiles form one stream (two stages of A and three of B in
//     LDS, 160 KB): the loads of stage s + 2 are issued between the MFMAs of stage s, one barrier
//     a stage, the first two stages of the next tile are requested before the epilogue. A group
//     has at least two stages (more zero rows for a group of at most 64 rows).
//   * Tiles run group-major, along the smaller output dimension first; each XCD's 32 CUs take a
//     contiguous run of that order together, sharing operands in their L2.
//   * Epilogue: each wave stages 32 x 32 fp32 pieces through a 4 KB LDS tile of its own
//     (128-byte rows, chunks permuted by the row's low three bits), staging the next piece while
//     the previous one's read-back is in flight, and stores whole 128-byte row segments.
constexpr int kWG = 256;                    // tile rows (M) and columns (N)
constexpr int kWGStage = 64 * 512;          // one operand's stage: 64 rows x 256 bf16
constexpr int kWGBOff = 2 * kWGStage;       // B's three slots follow A's two
constexpr int kWGPiece = 4096;              // epilogue staging tile: 32 rows x 128 bytes
constexpr size_t kWGLds = 5 * static_cast<size_t>(kWGStage);  // 160 KB
constexpr int kWGThreads = 512;             // 8 waves

// The source of every row past a group's end.
__device__ __align__(16) const uint4 kZeroRow[32] = {};

typedef __attribute__((address_space(3))) void* wg_lds_t;
__device__ __forceinline__ uint32_t wg_lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((wg_lds_t)(p)));
}
// 16 bytes a lane from the lane's own global address into LDS at lds + 16 * lane (lds
// wave-uniform).
__device__ __forceinline__ void dma16_at(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory");
}
// This wave's vector memory operations (all but the last N) and LDS operations done, then the
// workgroup barrier.
template <int N>
__device__ __forceinline__ void wg_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__global__ __launch_bounds__(kWGThreads, 1) void wgrad_gemm_big(WgradArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = a.M, N = a.N;
  const int MT = M / kWG, NT = N / kWG, per_group = MT * NT;
  const int total = a.G * per_group;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int nblk_xcd = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int first = xcd * per_xcd + local, last = min(total, (xcd + 1) * per_xcd);
  const int n_my = first < last ? (last - first + nblk_xcd - 1) / nblk_xcd : 0;
  if (n_my == 0) return;

  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const int32_t* off = a.offsets;
  struct Tile {
    int g, m0, n0, rb, re, nst;
  };
  auto decode = [&](int m) {  // the block's m-th tile without its group bounds
    const int q = first + m * nblk_xcd;
    Tile T;
    T.g = q / per_group;
    const int rem = q - T.g * per_group;
    const int mt = N > M ? rem % MT : rem / NT, nt = N > M ? rem / MT : rem % NT;
    T.m0 = mt * kWG;
    T.n0 = nt * kWG;
    T.rb = T.re = 0;
    T.nst = 2;
    return T;
  };
  auto tile = [&](int m) {
    Tile T = decode(m);
    T.rb = off[T.g];
    T.re = off[T.g + 1];
    T.nst = max(2, (T.re - T.rb + 63) / 64);
    return T;
  };
  const uint32_t ring = wg_lds_offset(smem);
  // Waves 0-3 load: lane l of loading wave w's load instruction i writes row 16 w + 2 i + l / 32
  // of the stage, LDS chunk l % 32, and fetches the 16 bytes that belong there. The lane's source addresses for
  // the tile being loaded (stage 0; a stage is 64 rows further on) are formed once per tile,
  // so a load costs one 64-bit add and the select of the zero row past the group's end: a
  // wave's instructions issue in order, and a longer address computation before each load
  // holds back its MFMAs.
  const int lw = wave & 3;
  const bool loader = wave < 4;
  const int lrow = 16 * lw + (lane >> 5), lslot = lane & 31;
  // The permuted chunk of row lrow + 2 i depends on i only through its parity, so the lane
  // keeps two addresses an operand (row lrow of the tile at the chunk of even / odd i) and a
  // load adds the uniform 64 kst + 2 i rows.
  const uint16_t* pa[2];
  const uint16_t* pb[2];
  int l_rows = 0;  // rows of the tile being loaded
  auto load_tile = [&](const Tile& T) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int chunk = lslot ^ (4 * ((lrow + 2 * par) & 3));
      pa[par] = A + static_cast<int64_t>(T.rb + lrow) * M + T.m0 + chunk * 8;
      pb[par] = B + static_cast<int64_t>(T.rb + lrow) * N + T.n0 + chunk * 8;
    }
    l_rows = T.re - T.rb;
  };
  auto dma = [&](const uint16_t* p0, int row_elems, int kst, uint32_t slot, int i) {
    const uint16_t* src = p0 + static_cast<int64_t>(kst * 64 + 2 * i) * row_elems;
    const void* from = lrow + 2 * i < l_rows - kst * 64 ? static_cast<const void*>(src)
                                                        : static_cast<const void*>(kZeroRow);
    dma16_at(from, slot + (16 * lw + 2 * i) * 512);
  };
  auto dma_a = [&](uint32_t slot, int kst, int i) { dma(pa[i & 1], M, kst, slot, i); };
  auto dma_b = [&](uint32_t slot, int kst, int i) { dma(pb[i & 1], N, kst, slot, i); };
  auto a_slot = [&](int s) { return ring + static_cast<uint32_t>((s & 1) * kWGStage); };
  auto b_slot = [&](int s) { return ring + static_cast<uint32_t>(kWGBOff + (s % 3) * kWGStage); };

  // wave w computes the 128 x 64 part at rows 128 (w / 4), columns 64 (w % 4): two waves a SIMD
  const int wm = wave >> 2, wn = wave & 3;
  // transpose-read fragments: lane (gq, jr, qc) reads 8 bytes at row 16 ks + 8 (gq / 2) + jr
  // (and 4 rows on), column 32 block + 16 (gq % 2) + 4 qc
  const int gq = lane >> 4, jr = (lane >> 2) & 3, qc = lane & 3;
  const int rowq = 8 * (gq >> 1) + jr, colq = 16 * (gq & 1) + 4 * qc;
  auto fr_off = [&](int ks, int c) {  // byte offset of (row 16 ks + rowq, column c) in a slot
    return (ks * 16 + rowq) * 512 + ((((c >> 3) ^ (4 * jr))) << 4) + 8 * (qc & 1);
  };
  u32x4 fa[2][4], fb[2][2];
  f32x16 acc[4][2];
  auto read = [&](int s, int ks, int b) {
    const unsigned char* pa = smem + (s & 1) * kWGStage;
    const unsigned char* pb = smem + kWGBOff + (s % 3) * kWGStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = fr_off(ks, wm * 128 + i * 32 + colq);
      const unsigned long long x0 = tr_read(pa, o), x1 = tr_read(pa, o + 4 * 512);
      fa[b][i] = u32x4{static_cast<unsigned>(x0), static_cast<unsigned>(x0 >> 32),
                       static_cast<unsigned>(x1), static_cast<unsigned>(x1 >> 32)};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = fr_off(ks, wn * 64 + j * 32 + colq);
      const unsigned long long x0 = tr_read(pb, o), x1 = tr_read(pb, o + 4 * 512);
      fb[b][j] = u32x4{static_cast<unsigned>(x0), static_cast<unsigned>(x0 >> 32),
                       static_cast<unsigned>(x1), static_cast<unsigned>(x1 >> 32)};
    }
  };
  // one k-step's 8 MFMAs in four groups; after group i, dmas(i) issues this k-step's share of
  // the loads
  auto mma_all = [&](int b, auto dmas) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = wmma<uint16_t>(fb[b][j], fa[b][i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      dmas(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  Tile cur = tile(0), nxt = cur;
  if (n_my > 1) nxt = tile(1);
  // Stage s (stage st of the current tile): k-steps 1..3 read one ahead of the MFMAs; the B
  // loads of stage s + 2 (into the B slot stage s - 1 freed) between the MFMAs of k-steps 0..2;
  // before the last k-step, this wave's loads of stage s + 1 are waited for (only B of stage
  // s + 2 may still be in flight) and the barrier passed, after which stage s is no longer read
  // by any wave; the A loads of stage s + 2 (into stage s's A slot) between the last k-step's
  // MFMAs. Stage s + 2 is the current tile's or, for its last two stages, the next tile's.
  auto body = [&](int s, int st, bool more_tiles) {
    const bool in_cur = st + 2 < cur.nst;
    const bool refill = (in_cur || more_tiles) && loader;
    const int k2 = in_cur ? st + 2 : st + 2 - cur.nst;
    // the loads switch to the next tile with its first stage
    if (refill && k2 == 0) load_tile(nxt);
    const uint32_t as2 = a_slot(s + 2), bs2 = b_slot(s + 2);
    auto b_part = [&](int first_i, int count) {
      return [&, first_i, count](int grp) {
        if (refill) {
          for (int i = first_i + (grp * count) / 4; i < first_i + ((grp + 1) * count) / 4; ++i)
            dma_b(bs2, k2, i);
        }
      };
    };
    read(s, 1, 1);
    mma_all(0, b_part(0, 3));
    read(s, 2, 0);
    mma_all(1, b_part(3, 3));
    read(s, 3, 1);
    mma_all(0, b_part(6, 2));
    if (refill) wg_wait_barrier<8>();
    else wg_wait_barrier<0>();
    read(s + 1, 0, 0);
    mma_all(1, [&](int grp) {
      if (refill) {
        dma_a(as2, k2, 2 * grp);
        dma_a(as2, k2, 2 * grp + 1);
      }
    });
  };

  // stages 0 and 1 (tile 0), then wait for stage 0
  load_tile(cur);
  if (loader) {
#pragma unroll
    for (int s0 = 0; s0 < 2; ++s0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dma_a(a_slot(s0), s0, i);
#pragma unroll
      for (int i = 0; i < 8; ++i) dma_b(b_slot(s0), s0, i);
    }
    wg_wait_barrier<16>();
  } else {
    wg_wait_barrier<0>();
  }
  read(0, 0, 0);

  int s = 0;
  for (int m = 0; m < n_my; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const bool more = m + 1 < n_my;
    for (int st = 0; st < cur.nst; ++st, ++s) body(s, st, more);

    // ---- epilogue (the next tile's first two stages are in flight). Register 4q + t of
    // acc[i][j] is C[m = 128 wm + 32 i + l % 32][n = 64 wn + 32 j + 8 q + 4 (l / 32) + t]. Each
    // wave stages the 32 x 32 piece (i, j) in its own 4 KB LDS tile (the eight tiles fill the B
    // slot of the tile's last stage, free until the next tile's first refill; chunk c of row r
    // at c ^ (r % 8)), reads it back as 128-byte rows (instruction p: rows 8p .. 8p+7) and
    // stores them. Step pc stages piece pc, stores piece pc - 1 and reads back piece pc; a
    // wave's LDS operations complete in order, so piece pc is staged only after piece pc - 1
    // has been read back.
    const Tile done = cur;
    // the group bounds of the next-but-one tile are requested before the epilogue's stores
    // and used after them, so the wait for them is no wait for the stores (or for the next
    // tile's first stages, requested before)
    const bool have2 = m + 2 < n_my;
    Tile t2 = nxt;
    int rb2 = 0, re2 = 0;
    if (have2) {
      t2 = decode(m + 2);
      rb2 = off[t2.g];
      re2 = off[t2.g + 1];
    }
    int lq = lane;
    asm volatile("" : "+v"(lq));  // keeps the lane-derived addresses from being hoisted
    unsigned char* stile = smem + kWGBOff + ((s - 1) % 3) * kWGStage + wave * kWGPiece;
    float* C = a.C + static_cast<int64_t>(done.g) * M * N;
    u32x4 rb[2][4];
    auto stage_piece = [&](int pc) {
      const int i = pc >> 1, j = pc & 1;
      unsigned char* t = stile;
      const int row = lq & 31;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = 2 * q + (lq >> 5);
        *reinterpret_cast<f32x4*>(t + row * 128 + ((ch ^ (row & 7)) << 4)) =
            f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      }
    };
    auto read_piece = [&](int pc) {
      const unsigned char* t = stile;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = 8 * p + (lq >> 3), ch = lq & 7;
        rb[pc & 1][p] = *reinterpret_cast<const u32x4*>(t + row * 128 + ((ch ^ (row & 7)) << 4));
      }
    };
    auto store_piece = [&](int pc) {
      const int i = pc >> 1, j = pc & 1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = 8 * p + (lq >> 3), ch = lq & 7;
        const int mrow = done.m0 + wm * 128 + i * 32 + row;
        const int ncol = done.n0 + wn * 64 + j * 32 + 4 * ch;
        *reinterpret_cast<u32x4*>(C + static_cast<int64_t>(mrow) * N + ncol) = rb[pc & 1][p];
      }
    };
#pragma unroll
    for (int pc = 0; pc < 9; ++pc) {
      if (pc < 8) stage_piece(pc);
      if (pc >= 1) store_piece(pc - 1);
      if (pc < 8) read_piece(pc);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave is done with the staging slot before the next tile's first refill reuses it
    __syncthreads();
    cur = nxt;
    if (have2) {
      t2.rb = __builtin_amdgcn_readfirstlane(rb2);
      t2.re = __builtin_amdgcn_readfirstlane(re2);
      t2.nst = max(2, (t2.re - t2.rb + 63) / 64);
      nxt = t2;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------ input gradient
template <typename T>
__global__ __launch_bounds__(kThreads) void dx_final(
    const T* __restrict__ dY, const T* __restrict__ dXd, const T* __restrict__ dXr,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ pos,
    const uint8_t* __restrict__ accepted, const int32_t* __restrict__ offsets, int Tn, int D, int k,
    int residual, T* __restrict__ dX) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= Tn) return;
  int64_t row[MOE_MAX_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    row[j] = -1;
    if (j < k) {
      const int64_t gi = static_cast<int64_t>(t) * k + j;
      if (accepted[gi]) row[j] = static_cast<int64_t>(offsets[ids[gi]]) + pos[gi];
    }
  }
  const int64_t o = static_cast<int64_t>(t) * D;
  if ((D % V) == 0) {
    for (int c = lane; c < D / V; c += 64) {
      float v[V];
      auto add = [&](const T* src) {
        const uint4 u = reinterpret_cast<const uint4*>(src)[c];
        const T* up = reinterpret_cast<const T*>(&u);
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] += Elem<T>::to_f32(up[i]);
      };
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = 0.f;
      if (residual) add(dY + o);
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j)
        if (row[j] >= 0) add(dXd + row[j] * D);
      if (dXr) add(dXr + o);
      T out[V];
#pragma unroll
      for (int i = 0; i < V; ++i) out[i] = Elem<T>::from_f32(v[i]);
      reinterpret_cast<uint4*>(dX + o)[c] = *reinterpret_cast<const uint4*>(out);
    }
  } else {
    for (int c = lane; c < D; c += 64) {
      float v = residual ? Elem<T>::to_f32(dY[o + c]) : 0.f;
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j)
        if (row[j] >= 0) v += Elem<T>::to_f32(dXd[row[j] * D + c]);
      if (dXr) v += Elem<T>::to_f32(dXr[o + c]);
      dX[o + c] = Elem<T>::from_f32(v);
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ host side
moe_status combine_backward_launch(const Dims& d, const void* dY, const void* Z, const int32_t* ids,
                                   const float* gates, const int32_t* pos, const uint8_t* accepted,
                                   const int32_t* offsets, void* dZ, float* dgates,
                                   hipStream_t stream) {
  const int grid = ceil_div(d.T, kThreads / 64);
  if (d.dtype == MOE_BF16)
    cb_backward<uint16_t><<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(Z), ids, gates, pos,
        accepted, offsets, d.T, d.D, d.k, static_cast<uint16_t*>(dZ), dgates);
  else
    cb_backward<float><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(dY), static_cast<const float*>(Z), ids, gates, pos, accepted,
        offsets, d.T, d.D, d.k, static_cast<float*>(dZ), dgates);
  return launch_status();
}

static int wg_device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

moe_status wgrad_launch(const Dims& d, const void* A, const void* B, const int32_t* offsets, int G,
                        int M, int N, float* C, hipStream_t stream, int splits) {
  WgradArgs a{A, B, offsets, C, G, M, N, splits};
  // rows of 16-byte multiples from 16-byte aligned bases: vector loads and stores
  const bool vec = M % 8 == 0 && N % 8 == 0 &&
                   (reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) |
                    reinterpret_cast<uintptr_t>(C)) % 16 == 0;
  const bool tr = d.dtype == MOE_BF16 && vec;  // the transpose-read kernel
  // 256 x 256 tiles, whole ones only, one row split, enough tiles to give every CU one: the
  // persistent kernel (one block per CU)
  if (tr && splits == 1 && M % kWG == 0 && N % kWG == 0 &&
      static_cast<int64_t>(G) * (M / kWG) * (N / kWG) >= wg_device_cus()) {
    static std::once_flag once[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
    bool ok = true;
    std::call_once(once[dev], [&] {
      ok = hipFuncSetAttribute(reinterpret_cast<const void*>(&wgrad_gemm_big),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(kWGLds)) == hipSuccess;
    });
    if (!ok) return MOE_ERR_HIP;
    const int cus = wg_device_cus();
    const int grid = std::max(kXcds, cus / kXcds * kXcds);
    wgrad_gemm_big<<<grid, kWGThreads, kWGLds, stream>>>(a);
    return launch_status();
  }
  const int64_t blocks = static_cast<int64_t>(G) * splits * ceil_div(M, kWT) * ceil_div(N, tr ? kTN2 : kWT);
  if (blocks > 0x7fffffffLL - kXcds) return MOE_ERR_UNSUPPORTED;
  const int grid = static_cast<int>(ceil_div64(blocks, kXcds) * kXcds);
  const bool aligned = vec;
  const bool split = splits > 1;
#define MOE_WGRAD(TY, AL, SP) wgrad_gemm<TY, AL, SP><<<grid, kThreads, 0, stream>>>(a)
  if (d.dtype == MOE_BF16) {
    if (aligned) {
      if (split) wgrad_gemm_tr<true><<<grid, kThreads, 0, stream>>>(a);
      else wgrad_gemm_tr<false><<<grid, kThreads, 0, stream>>>(a);
    }
    else { if (split) MOE_WGRAD(uint16_t, false, true); else MOE_WGRAD(uint16_t, false, false); }
  } else {
    if (aligned) { if (split) MOE_WGRAD(float, true, true); else MOE_WGRAD(float, true, false); }
    else { if (split) MOE_WGRAD(float, false, true); else MOE_WGRAD(float, false, false); }
  }
#undef MOE_WGRAD
  return launch_status();
}

// Columns of [dclean | draw]: 2E for the noisy gate with noise, E otherwise (no draw).
static int router_cols(const Dims& d) {
  return d.gating == MOE_GATE_NOISY_TOPK && d.noise ? 2 * d.E : d.E;
}

static int router_bwd_ks(const Dims& d) {  // k-steps over the router GEMM's inputs
  const int stage = d.dtype == MOE_BF16 ? 64 : 32;
  return ceil_div(router_cols(d), stage) * 4;
}

// Workspace of moe_route_backward: dimp, dload [E]; dbias partials; dcat [T, 2E]; the packed
// [Wg | Wnoise]^T; offsets {0, T}; the router's input-gradient share [T, D]; dWcat [D, 2E].
struct RouteBwdLayout {
  size_t dimp, dload, dbias, dbias2, dcat, wpack, off, dxr, dwcat, total;
};
// Row splits of the router's weight gradient X^T [dclean | draw] (one group of T rows): enough
// blocks to fill the chip, at least 256 rows a split.
static int router_splits(const Dims& d) {
  const int tiles = ceil_div(d.D, kWT) * ceil_div(router_cols(d), kWT);
  return std::max(1, std::min(ceil_div(2048, tiles), ceil_div(d.T, 256)));
}

// Row slices of the first pass over the bias partials (about 32 rows a slice, at most 64).
static int bias_slices(int nblk) { return std::max(1, std::min(64, nblk / 32)); }

static int gate_waves(const Dims& d) { return d.E > 2048 ? 2 : 4; }
static int gate_blocks(const Dims& d) { return ceil_div(d.T, gate_waves(d) * kGateRowsPerWave); }

static RouteBwdLayout route_bwd_layout(const Dims& d) {
  RouteBwdLayout L;
  const size_t el = d.dtype == MOE_BF16 ? 2 : 4;
  const int nblk = gate_blocks(d);
  size_t o = 0;
  L.dimp = o; o += align256(d.E * sizeof(float));
  L.dload = o; o += align256(d.E * sizeof(float));
  L.dbias = o; o += align256(static_cast<size_t>(nblk) * d.E * sizeof(float));
  L.dbias2 = o; o += align256(static_cast<size_t>(bias_slices(nblk)) * d.E * sizeof(float));
  L.dcat = o; o += align256(static_cast<size_t>(d.T) * router_cols(d) * el);
  L.wpack = o; o += align256(static_cast<size_t>(ceil_div(d.D, 32)) * router_bwd_ks(d) * kWave * 16);
  L.off = o; o += 256;
  L.dxr = o; o += align256(static_cast<size_t>(d.T) * d.D * el);
  L.dwcat = o; o += align256(static_cast<size_t>(router_splits(d)) * d.D * router_cols(d) * sizeof(float));
  L.total = o;
  return L;
}
size_t route_backward_workspace(const Dims& d) { return route_bwd_layout(d).total; }

// dWg / dWnoise from the router's split partials [S][D][KC], summed over the splits in order
// (KC = E, or 2E with the noise columns after the clean ones).
__global__ void split_dw(const float* __restrict__ dwcat, int S, int D, int E, int KC,
                         float* __restrict__ dWg, float* __restrict__ dWn) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(D) * E) return;
  const int64_t dd = i / E;
  const int e = static_cast<int>(i - dd * E);
  const int64_t plane = static_cast<int64_t>(D) * KC;
  float g = 0.f, n = 0.f;
  for (int s = 0; s < S; ++s) {
    g += dwcat[s * plane + dd * KC + e];
    if (dWn) n += dwcat[s * plane + dd * KC + E + e];
  }
  dWg[i] = g;
  if (dWn) dWn[i] = n;
}

moe_status route_backward_launch(const Dims& d, uint64_t seed, const void* X, const float* Wg,
                                 const float* Wnoise, const float* eps, const float* scores,
                                 const int32_t* ids,
                                 const float* gates,
                                 const float* clean, const float* noise_std, const float* row_stats,
                                 const float* dgates, const float* importance, const float* load,
                                 const int32_t* counts, float w_imp, float w_load, float w_switch,
                                 const void* dY, const void* dXd,
                                 const int32_t* pos, const uint8_t* accepted, const int32_t* offsets,
                                 void* dX, float* dWg, float* dWnoise, float* dbias, void* ws,
                                 hipStream_t stream) {
  const RouteBwdLayout L = route_bwd_layout(d);
  char* base = static_cast<char*>(ws);
  float* dimp = reinterpret_cast<float*>(base + L.dimp);
  float* dload = reinterpret_cast<float*>(base + L.dload);  // Switch: dprob
  float* dbias_part = reinterpret_cast<float*>(base + L.dbias);
  void* dcat = base + L.dcat;
  uint4* wpack = reinterpret_cast<uint4*>(base + L.wpack);
  int32_t* off = reinterpret_cast<int32_t*>(base + L.off);
  void* dxr = base + L.dxr;
  float* dwcat = reinterpret_cast<float*>(base + L.dwcat);
  const bool sw = d.gating == MOE_GATE_SWITCH_TOP1;
  const bool noise = !sw && d.noise != 0;
  const int KC = router_cols(d);
  if (w_imp != 0.f) {
    cv2_grad<<<1, kThreads, 0, stream>>>(importance, d.E, w_imp, dimp);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  const int nblk = gate_blocks(d), gw = gate_waves(d);
  if (sw) {
    const bool use_bal = w_switch != 0.f;
    if (use_bal) {
      switch_dprob<<<ceil_div(d.E, kThreads), kThreads, 0, stream>>>(counts, d.T, d.E, w_switch,
                                                                     dload);
      if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    }
    SwitchGateArgs sa;
    sa.ids = ids;
    sa.clean = clean;
    sa.dgates = dgates;
    sa.dimp = w_imp != 0.f ? dimp : nullptr;
    sa.dprob = use_bal ? dload : nullptr;
    sa.dcat = dcat;
    sa.dbias_part = dbias ? dbias_part : nullptr;
    sa.T = d.T;
    sa.E = d.E;
    sa.dtype = d.dtype;
    const size_t lds = static_cast<size_t>(gw) * d.E * sizeof(float);
    switch_gate_backward<<<nblk, 64 * gw, lds, stream>>>(sa);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  } else {
    const bool use_load = noise && w_load != 0.f;
    if (use_load) {
      cv2_grad<<<1, kThreads, 0, stream>>>(load, d.E, w_load, dload);
      if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    }
    GateArgs ga;
    ga.ids = ids;
    ga.gates = gates;
    ga.clean = clean;
    ga.std_in = noise ? noise_std : nullptr;
    ga.row_stats = row_stats;
    ga.dgates = dgates;
    ga.dimp = w_imp != 0.f ? dimp : nullptr;
    ga.dload = use_load ? dload : nullptr;
    ga.eps = noise ? eps : nullptr;
    ga.scores = noise ? scores : nullptr;
    ga.dcat = dcat;
    ga.ldc = KC;
    ga.dbias_part = dbias ? dbias_part : nullptr;
    ga.seed = seed;
    ga.T = d.T;
    ga.E = d.E;
    ga.k = d.k;
    ga.noise = noise ? 1 : 0;
    ga.dtype = d.dtype;
    const size_t lds = static_cast<size_t>(gw) * 3 * d.E * sizeof(float);
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&gate_backward),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) != hipSuccess)
      return MOE_ERR_HIP;
    gate_backward<<<nblk, 64 * gw, lds, stream>>>(ga);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  if (dbias) {
    const int sl = bias_slices(nblk);
    float* dbias2 = reinterpret_cast<float*>(base + L.dbias2);
    column_sums<<<dim3(ceil_div(d.E, 64), sl), kThreads, 0, stream>>>(dbias_part, nblk, d.E, dbias2);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
    column_sums<<<dim3(ceil_div(d.E, 64), 1), kThreads, 0, stream>>>(dbias2, sl, d.E, dbias);
    if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  }
  // the router's share of dX: [dclean | draw] [Wg | Wnoise]^T as a one-group GEMM
  Dims dr = d;
  dr.E = 1;
  dr.k = 1;
  dr.D = KC;   // K
  dr.H = d.D;  // N
  dr.C = d.T;
  dr.max_rows = d.T;
  const int NB = ceil_div(d.D, 32), KS = router_bwd_ks(d);
  const int64_t items = static_cast<int64_t>(NB) * KS * kWave;
  const PackStrides ps = pack_strides(dr, 3);
  if (d.dtype == MOE_BF16)
    router_pack_t<uint16_t><<<static_cast<int>(ceil_div64(items, 256)), 256, 0, stream>>>(
        Wg, noise ? Wnoise : nullptr, d.D, d.E, NB, KS, ps, wpack);
  else
    router_pack_t<float><<<static_cast<int>(ceil_div64(items, 256)), 256, 0, stream>>>(
        Wg, noise ? Wnoise : nullptr, d.D, d.E, NB, KS, ps, wpack);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  set_offsets<<<1, 64, 0, stream>>>(off, d.T);
  moe_status s = gemm_launch(dr, 3, dcat, wpack, off, dxr, nullptr, stream);
  if (s != MOE_OK) return s;
  // dWcat = X^T [dclean | draw]
  const int S = router_splits(d);
  s = wgrad_launch(d, X, dcat, off, 1, d.D, KC, dwcat, stream, S);
  if (s != MOE_OK) return s;
  split_dw<<<static_cast<int>(ceil_div64(static_cast<int64_t>(d.D) * d.E, 256)), 256, 0, stream>>>(
      dwcat, S, d.D, d.E, KC, dWg, noise ? dWnoise : nullptr);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  // dX = dY (residual) + the experts' rows + the router's share
  const int grid = ceil_div(d.T, kThreads / 64);
  if (d.dtype == MOE_BF16)
    dx_final<uint16_t><<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(dXd),
        static_cast<const uint16_t*>(dxr), ids, pos, accepted, offsets, d.T, d.D, d.k, dY ? 1 : 0,
        static_cast<uint16_t*>(dX));
  else
    dx_final<float><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(dY), static_cast<const float*>(dXd),
        static_cast<const float*>(dxr), ids, pos, accepted, offsets, d.T, d.D, d.k, dY ? 1 : 0,
        static_cast<float*>(dX));
  return launch_status();
}

moe_status ffn_backward_launch(const Dims& d, const void* Xd, const void* Hd, const void* dZ,
                               const void* W1t, const void* W2t, const int32_t* offsets, void* dHp,
                               void* dXd, float* dW1, float* dW2, hipStream_t stream) {
  // dH (pre-activation) = (dZ W2^T) masked by Hd > 0; dXd = dH W1^T
  moe_status s = gemm_launch(d, 3, dZ, W2t, offsets, dHp, nullptr, stream, Hd);
  if (s != MOE_OK) return s;
  s = gemm_launch(d, 4, dHp, W1t, offsets, dXd, nullptr, stream);
  if (s != MOE_OK) return s;
  if (dW2) {
    s = wgrad_launch(d, Hd, dZ, offsets, d.E, d.H, d.D, dW2, stream);
    if (s != MOE_OK) return s;
  }
  if (dW1) s = wgrad_launch(d, Xd, dHp, offsets, d.E, d.D, d.H, dW1, stream);
  return s;
}

}  // namespace moe
