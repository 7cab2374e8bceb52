// Internal helpers shared by the HIP sources of the MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ----------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a NaN. gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction when the compiler pairs them).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
  __device__ static uint16_t from_f32(float v) { return f32_to_bf16(v); }
};

// 32x32 MFMA accumulator layout (16 fp32 per lane): register i of lane l
// holds C[row][col] with col = l % 32 and row = 8*(i/4) + 4*(l/32) + i%4.
__device__ __forceinline__ int acc_row(int lane, int i) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// One MFMA "k-step" on 16-byte operand fragments. Lane l supplies row/col
// l % 32 and a contiguous run of k values selected by l / 32; A and B use the
// same run, so the products pair up whatever order the unit sums them in.
//   bf16: 8 values per lane, one 32x32x16 MFMA (k-step 16)
//   fp32: 4 values per lane, four 32x32x2 MFMAs  (k-step 8); MFMA s takes
//         k = 4*(l/32) + s from each lane
__device__ __forceinline__ f32x16 mfma_step_bf16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_step_f32(uint4 a, uint4 b, f32x16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}
template <typename T> __device__ __forceinline__ f32x16 mfma_step(uint4 a, uint4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mfma_step<uint16_t>(uint4 a, uint4 b, f32x16 c) {
  return mfma_step_bf16(a, b, c);
}
template <> __device__ __forceinline__ f32x16 mfma_step<float>(uint4 a, uint4 b, f32x16 c) {
  return mfma_step_f32(a, b, c);
}

// 16-byte load of elements [k0, k0+kVec) of a row of length n, zero past n.
// vec_ok: rows are 16-byte aligned and n % kVec == 0 (then only whole vectors
// are ever partially outside, i.e. entirely outside).
template <typename T>
__device__ __forceinline__ uint4 load_row16(const T* row, int k0, int n, bool vec_ok) {
  constexpr int V = Elem<T>::kVec;
  if (vec_ok) {
    if (k0 < n) return *reinterpret_cast<const uint4*>(row + k0);
    return make_uint4(0, 0, 0, 0);
  }
  T v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = (k0 + i < n) ? row[k0 + i] : T(0);
  return *reinterpret_cast<const uint4*>(v);
}

// ----------------------------------------------------------------- non-finite record
// With check_finite on, kernels get the device's flag word and store 1 into it
// (idempotent plain stores) when a NaN/Inf shows up; otherwise flag is null.
__device__ __forceinline__ void note_nonfinite(int* flag, bool bad) {
  if (bad) *flag = 1;
}

// Exclusive scan of v over a block of N threads (*excl gets this thread's prefix);
// returns the block total. warp_tot holds N / 64 ints of shared memory.
template <int N>
__device__ __forceinline__ int block_exclusive_scan(int v, int* excl, int* warp_tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) warp_tot[w] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < N / 64; ++i) {
    if (i < w) before += warp_tot[i];
    total += warp_tot[i];
  }
  *excl = before + x - v;
  __syncthreads();
  return total;
}

// ----------------------------------------------------------------- host-side checks
struct Dims {
  int T, D, E, H, k;
  int dtype, gating, noise;
  int C;
  int64_t max_rows;
};

moe_status validate(const moe_problem* p, Dims* d);
moe_status launch_status();  // MOE_ERR_HIP if the last launch failed

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace sizes of the individual stages.
size_t route_workspace(const Dims& d);
const float* route_scores(const Dims& d, const void* ws);
size_t dispatch_workspace(const Dims& d);
size_t aux_workspace(const Dims& d);
size_t packed_weight_bytes(const Dims& d, int layer);
// Where the packed expert weights of a layer keep their 1 KB fragments: fragment (e, nb, ks)
// (expert, 32-column block, k-step; 4 k-steps make a k stage) sits at
// e * expert + nb * block + (ks / 4) * stage + ks % 4. Stage order (block 4, stage 4 NB) when
// the layer's groups average at least kStageOrderRows rows, else column-block order (block
// KS, stage 4); expert = NB * KS either way. Every packer and every GEMM takes them from here.
constexpr int64_t kStageOrderRows = 128;
struct PackStrides {
  int64_t expert, block, stage;
};
PackStrides pack_strides(const Dims& d, int layer);

// Stage launchers (arguments already validated).
moe_status route_launch(const Dims& d, const moe_problem* p, const void* X, const float* Wg,
                        const float* Wnoise, const float* bias, const float* eps, int32_t* ids,
                        float* gates, float* clean, float* noise_std, float* row_stats,
                        void* ws, int* nonfinite, hipStream_t stream);
moe_status dispatch_launch(const Dims& d, const void* X, const int32_t* ids, int32_t* pos,
                           uint8_t* accepted, int32_t* counts, int32_t* offsets,
                           int32_t* row_token, void* Xd, void* ws, hipStream_t stream);
moe_status dispatch_noalloc_launch(const Dims& d, const void* X, const int32_t* ids, int32_t* pos,
                                   uint8_t* accepted, int32_t* counts, int32_t* offsets,
                                   int32_t* row_token, void* Xd, hipStream_t stream);
moe_status pack_launch(const Dims& d, int layer, const void* W, void* Wp, hipStream_t stream);
moe_status gemm_launch(const Dims& d, int layer, const void* A, const void* Wp,
                       const int32_t* offsets, void* C, int* nonfinite, hipStream_t stream,
                       const void* mask = nullptr, const int32_t* row_token = nullptr);
moe_status combine_launch(const Dims& d, const void* Z, const int32_t* ids, const float* gates,
                          const int32_t* pos, const uint8_t* accepted, const int32_t* offsets,
                          const void* residual, void* Y, int* nonfinite, hipStream_t stream);
moe_status aux_launch(const Dims& d, const int32_t* ids, const float* gates, const float* clean,
                      const float* noise_std, const float* row_stats, const int32_t* counts,
                      float* importance, float* load, float* out, void* ws, hipStream_t stream);

// Hierarchical MoE (hier.hip, grouped gates in router.hip).
void hier_dims(const Dims& d, const moe_hier* h, Dims* dp, Dims* ds);
size_t route_groups_workspace(const Dims& ds, int G);
moe_status route_groups_launch(const Dims& ds, int G, uint64_t seed, const void* X,
                               const int32_t* goff, const int32_t* row_token, const float* Wsg,
                               const float* Wsn, int32_t* ids, float* gates, float* clean,
                               float* noise_std, float* row_stats, void* ws, int* nonfinite,
                               hipStream_t stream);
size_t hier_route_workspace(const Dims& d, const moe_hier* h);
size_t hier_aux_workspace(const Dims& d, const moe_hier* h);
moe_status hier_route_launch(const Dims& d, const moe_hier* h, const moe_problem* p, const void* X,
                             const float* Wpg, const float* Wpn, const float* Wsg, const float* Wsn,
                             int32_t* ids, float* gates, const moe_hier_state* st, void* ws,
                             int* nonfinite, hipStream_t stream);
moe_status hier_aux_launch(const Dims& d, const moe_hier* h, const moe_hier_state* st,
                           float* importance, float* load, float* out, void* ws, hipStream_t stream);

// Router scores only (router.hip): clean = X . Wg (+ bias), no noise, no selection.
size_t router_clean_workspace(const Dims& d);
moe_status router_clean_launch(const Dims& d, const void* X, const float* Wg, const float* bias,
                               float* clean, void* ws, int* nonfinite, hipStream_t stream);

// Batchwise mask (batchwise.hip).
int batchwise_m(const Dims& d);
size_t batchwise_route_workspace(const Dims& d);
size_t batchwise_aux_workspace(const Dims& d);
moe_status batchwise_route_launch(const Dims& d, const void* X, const float* Wg, const float* bias,
                                  float* clean, const moe_batchwise_state* st, void* ws,
                                  int* nonfinite, hipStream_t stream);
moe_status batchwise_dispatch_launch(const Dims& d, const void* X, const moe_batchwise_state* st,
                                     void* Xd, hipStream_t stream);
moe_status batchwise_combine_launch(const Dims& d, const void* Z, const moe_batchwise_state* st,
                                    const void* residual, void* Y, int* nonfinite,
                                    hipStream_t stream);
moe_status batchwise_aux_launch(const Dims& d, const moe_batchwise_state* st,
                                const float* thresholds, float* importance, float* out, void* ws,
                                hipStream_t stream);

// Backward pass (backward.hip).
size_t route_backward_workspace(const Dims& d);
moe_status combine_backward_launch(const Dims& d, const void* dY, const void* Z, const int32_t* ids,
                                   const float* gates, const int32_t* pos, const uint8_t* accepted,
                                   const int32_t* offsets, void* dZ, float* dgates,
                                   hipStream_t stream);
moe_status wgrad_launch(const Dims& d, const void* A, const void* B, const int32_t* offsets, int G,
                        int M, int N, float* C, hipStream_t stream, int splits = 1);
moe_status ffn_backward_launch(const Dims& d, const void* Xd, const void* Hd, const void* dZ,
                               const void* W1t, const void* W2t, const int32_t* offsets, void* dHp,
                               void* dXd, float* dW1, float* dW2, hipStream_t stream);
moe_status route_backward_launch(const Dims& d, uint64_t seed, const void* X, const float* Wg,
                                 const float* Wnoise, const float* eps, const float* scores,
                                 const int32_t* ids,
                                 const float* gates, const float* clean, const float* noise_std,
                                 const float* row_stats, const float* dgates,
                                 const float* importance, const float* load,
                                 const int32_t* counts, float w_imp, float w_load, float w_switch,
                                 const void* dY, const void* dXd, const int32_t* pos,
                                 const uint8_t* accepted, const int32_t* offsets, void* dX,
                                 float* dWg, float* dWnoise, float* dbias, void* ws,
                                 hipStream_t stream);

}  // namespace moe
