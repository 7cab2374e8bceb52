// Combine: gate-weighted sum of the kept expert outputs plus the residual.
// "Outrageously Large Neural Networks" summary, section 3.4: the layer output
// is the sum over experts of G(x)_i E_i(x), only nonzero gates contribute.
// "Switch Transformer" explainer, "Implementation" step 7: the selected
// probability multiplies the expert output at the token's own position and the
// input is added back; a dropped assignment contributes nothing, so a token
// with every assignment dropped leaves the layer unchanged.
//
// One wave per token: the token's (row, gate) pairs are uniform across the
// wave; lanes stride over the row in 16-byte vectors, accumulate in fp32 in
// ascending j (a fixed order, no atomics), and round once.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const T* __restrict__ Z, const int32_t* __restrict__ ids, const float* __restrict__ gates,
    const int32_t* __restrict__ pos, const uint8_t* __restrict__ accepted,
    const int32_t* __restrict__ offsets, const T* __restrict__ R, T* __restrict__ Y, int Tn, int D,
    int k, int E, int* nonfinite) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= Tn) return;
  // row of each assignment in Z, -1 when dropped (kept in registers: the
  // loops below are unrolled over MOE_MAX_K so every index is static)
  int64_t row[MOE_MAX_K];
  float gv[MOE_MAX_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    row[j] = -1;
    gv[j] = 0.f;
    if (j < k) {
      const int64_t gi = static_cast<int64_t>(t) * k + j;
      const int e = ids[gi];
      if (accepted[gi] && static_cast<unsigned>(e) < static_cast<unsigned>(E)) {
        row[j] = static_cast<int64_t>(offsets[e]) + pos[gi];
        gv[j] = gates[gi];
      }
    }
  }
  const bool check = nonfinite != nullptr;
  bool bad = false;
  if ((D % V) == 0) {
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
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j) {
        if (row[j] < 0) continue;
        const uint4 zv = reinterpret_cast<const uint4*>(Z + row[j] * D)[c];
        const T* zp = reinterpret_cast<const T*>(&zv);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = fmaf(gv[j], Elem<T>::to_f32(zp[i]), y[i]);
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
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j)
        if (row[j] >= 0) y = fmaf(gv[j], Elem<T>::to_f32(Z[row[j] * D + c]), y);
      bad |= !isfinite(y);
      Y[static_cast<int64_t>(t) * D + c] = Elem<T>::from_f32(y);
    }
  }
  if (check) note_nonfinite(nonfinite, bad);
}

}  // namespace

moe_status combine_launch(const Dims& d, const void* Z, const int32_t* ids, const float* gates,
                          const int32_t* pos, const uint8_t* accepted, const int32_t* offsets,
                          const void* residual, void* Y, int* nonfinite, hipStream_t stream) {
  const int grid = ceil_div(d.T, kThreads / 64);
  if (d.dtype == MOE_BF16)
    combine_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(Z), ids, gates, pos, accepted, offsets,
        static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(Y), d.T, d.D, d.k, d.E, nonfinite);
  else
    combine_kernel<float><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(Z), ids, gates, pos, accepted, offsets,
        static_cast<const float*>(residual), static_cast<float*>(Y), d.T, d.D, d.k, d.E, nonfinite);
  return launch_status();
}

}  // namespace moe
