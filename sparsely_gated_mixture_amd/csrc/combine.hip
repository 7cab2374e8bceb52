// Combine: gate-weighted sum of the kept expert outputs plus the residual.
// "Outrageously Large Neural Networks" summary, section 3.4: the layer output
// is the sum over experts of G(x)_i E_i(x), only nonzero gates contribute.
// "Switch Transformer" explainer, "Implementation" step 7: the selected
// probability multiplies the expert output at the token's own position and the
// input is added back; a dropped assignment contributes nothing, so a token
// with every assignment dropped leaves the layer unchanged.
//
// One wave per token (its index made wave-uniform, so the token's ids, gates and
// slots come through scalar loads): lanes take two 16-byte vectors of the row at a
// time and issue every load of both (residual and the accepted expert rows) before
// the FMAs; fp32 accumulation in ascending j (a fixed order, no atomics), one rounding.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Every row is read once and Y is written once: the loads and stores carry the non-temporal
// hint (streamed, not kept in the caches), which measurably raises the achieved bandwidth.
typedef unsigned int u32v4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ntl(const uint4* p) {
  const u32v4 v = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const T* __restrict__ Z, const int32_t* __restrict__ ids, const float* __restrict__ gates,
    const int32_t* __restrict__ pos, const uint8_t* __restrict__ accepted,
    const int32_t* __restrict__ offsets, const T* __restrict__ R, T* __restrict__ Y, int Tn, int D,
    int k, int E, int* nonfinite) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6));
  if (t >= Tn) return;
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
    // two 16-byte vectors a lane at a time, every load of both issued before the FMAs
    for (int c0 = lane; c0 < nv; c0 += 128) {
      const int c1 = c0 + 64;
      const bool two = c1 < nv;
      uint4 rv[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
      uint4 zv[MOE_MAX_K][2];
      const uint4* rrow = R ? reinterpret_cast<const uint4*>(R + static_cast<int64_t>(t) * D) : nullptr;
      if (R) {
        rv[0] = ntl(rrow + c0);
        if (two) rv[1] = ntl(rrow + c1);
      }
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j) {
        if (row[j] < 0) continue;
        const uint4* zr = reinterpret_cast<const uint4*>(Z + row[j] * D);
        zv[j][0] = ntl(zr + c0);
        if (two) zv[j][1] = ntl(zr + c1);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && !two) break;
        float y[V];
        const T* rp = reinterpret_cast<const T*>(&rv[h]);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = R ? Elem<T>::to_f32(rp[i]) : 0.f;
#pragma unroll
        for (int j = 0; j < MOE_MAX_K; ++j) {
          if (row[j] < 0) continue;
          const T* zp = reinterpret_cast<const T*>(&zv[j][h]);
#pragma unroll
          for (int i = 0; i < V; ++i) y[i] = fmaf(gv[j], Elem<T>::to_f32(zp[i]), y[i]);
        }
        T out[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
          bad |= !isfinite(y[i]);
          out[i] = Elem<T>::from_f32(y[i]);
        }
        uint4* dst = reinterpret_cast<uint4*>(Y + static_cast<int64_t>(t) * D) + (h ? c1 : c0);
        __builtin_nontemporal_store(*reinterpret_cast<const u32v4*>(out), reinterpret_cast<u32v4*>(dst));
      }
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
