// C ABI entry points: argument validation on the host, then stage launches on
// the caller's stream. Nothing here allocates device memory or synchronises
// (except moe_check_finite, whose job is to synchronise).
#include <math.h>

#include <algorithm>
#include <mutex>

#include "common.h"

namespace moe {

#define MOE_STATUS_TRY(expr)          \
  do {                                \
    const moe_status s_ = (expr);     \
    if (s_ != MOE_OK) return s_;      \
  } while (0)

// Largest expert count: dispatch and the grouped GEMM keep per-expert tables
// in LDS (dispatch: 2E+1+512 ints).
constexpr int kMaxExperts = 4096;

__device__ int g_nonfinite;

moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status validate(const moe_problem* p, Dims* d) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->T < 1 || p->D < 1 || p->E < 1 || p->H < 1) return MOE_ERR_INVALID_ARG;
  if (p->gating != MOE_GATE_NOISY_TOPK && p->gating != MOE_GATE_SWITCH_TOP1 &&
      p->gating != MOE_GATE_BATCHWISE)
    return MOE_ERR_INVALID_ARG;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (p->k < 1 || p->k > p->E) return MOE_ERR_INVALID_ARG;
  if (p->gating == MOE_GATE_SWITCH_TOP1 && p->k != 1) return MOE_ERR_INVALID_ARG;
  if (p->noise != 0 && p->noise != 1) return MOE_ERR_INVALID_ARG;
  if (p->gating == MOE_GATE_BATCHWISE &&
      (p->noise != 0 || static_cast<int64_t>(p->k) * p->T < p->E))
    return MOE_ERR_INVALID_ARG;  // no noise; at least one token per expert
  if (p->check_finite != 0 && p->check_finite != 1) return MOE_ERR_INVALID_ARG;
  if (!isfinite(p->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (p->min_capacity < 1) return MOE_ERR_INVALID_ARG;
  if (p->k > MOE_MAX_K) return MOE_ERR_UNSUPPORTED;
  if (p->E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(p->T) * p->k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  d->T = p->T;
  d->D = p->D;
  d->E = p->E;
  d->H = p->H;
  d->k = p->k;
  d->dtype = p->dtype;
  d->gating = p->gating;
  d->noise = p->noise;
  // capacity: [SWITCH] step 3 (floor, clamp to T, then the minimum), k-scaled
  if (p->capacity_factor > 0.f) {
    const double c = floor(static_cast<double>(p->k) * static_cast<double>(p->T) *
                           static_cast<double>(p->capacity_factor) / static_cast<double>(p->E));
    const double clamped = std::min(static_cast<double>(p->T), c);
    d->C = std::max(p->min_capacity, static_cast<int>(clamped));
  } else {
    d->C = p->T;
  }
  d->max_rows = std::min(static_cast<int64_t>(p->T) * p->k, static_cast<int64_t>(p->E) * d->C);
  return MOE_OK;
}

static int* nonfinite_flag(const moe_problem* p) {
  if (!p->check_finite) return nullptr;
  static std::mutex mu;
  static int* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_nonfinite)) != hipSuccess) return nullptr;
    ptrs[dev] = static_cast<int*>(ptr);
  }
  return ptrs[dev];
}

// Every tensor and workspace pointer given to an entry point must be 16-byte aligned (NULL
// passes): the kernels move rows and packed weights as 16-byte vectors. hipMalloc and the
// PyTorch allocator return 256-byte aligned memory; a view at an odd element offset is
// rejected here instead of being read unaligned.
template <typename... P>
static bool aligned16(P... ptrs) {
  return ((reinterpret_cast<uintptr_t>(ptrs) % 16 == 0) && ...);
}
#define MOE_ALIGNED(...)                                     \
  do {                                                       \
    if (!aligned16(__VA_ARGS__)) return MOE_ERR_INVALID_ARG; \
  } while (0)

static bool hier_state_aligned(const moe_hier_state* st) {
  return aligned16(st->ids_p, st->gates_p, st->clean_p, st->std_p, st->row_stats_p, st->pos_p,
                   st->accepted_p, st->counts_p, st->offsets_p, st->row_token_p, st->clean_s,
                   st->std_s, st->row_stats_s, st->ids_s, st->gates_s);
}

// Hierarchical options on top of a valid flat problem.
static moe_status validate_hier(const moe_problem* p, const moe_hier* h, Dims* d) {
  MOE_STATUS_TRY(validate(p, d));
  if (!h) return MOE_ERR_INVALID_ARG;
  if (p->gating != MOE_GATE_NOISY_TOPK) return MOE_ERR_INVALID_ARG;
  const int a = h->groups, kp = h->k_primary;
  if (a < 1 || a > p->E || p->E % a != 0) return MOE_ERR_INVALID_ARG;
  if (kp < 1 || kp > a || p->k % kp != 0 || p->k / kp > p->E / a) return MOE_ERR_INVALID_ARG;
  if (static_cast<int64_t>(p->T) * kp * (p->E / a) > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

#define MOE_TRY(expr)                 \
  do {                                \
    const moe_status s_ = (expr);     \
    if (s_ != MOE_OK) return s_;      \
  } while (0)

static hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// The per-token top-k entry points (route, dispatch, combine, aux) do not take the
// batchwise mask, which has entry points of its own.
static moe_status validate_topk(const moe_problem* p, Dims* d) {
  MOE_TRY(validate(p, d));
  return d->gating == MOE_GATE_BATCHWISE ? MOE_ERR_INVALID_ARG : MOE_OK;
}

static moe_status flag_for(const moe_problem* p, int** flag) {
  *flag = nonfinite_flag(p);
  if (p->check_finite && !*flag) return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" {

int32_t moe_capacity(const moe_problem* p) {
  Dims d;
  return validate(p, &d) == MOE_OK ? d.C : -1;
}

int64_t moe_max_rows(const moe_problem* p) {
  Dims d;
  return validate(p, &d) == MOE_OK ? d.max_rows : -1;
}

size_t moe_workspace_size(const moe_problem* p, int which) {
  Dims d;
  if (validate_topk(p, &d) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_ROUTE: return route_workspace(d);
    case MOE_WS_DISPATCH: return dispatch_workspace(d);
    case MOE_WS_AUX: return aux_workspace(d);
    default: return 0;
  }
}

size_t moe_packed_weight_bytes(const moe_problem* p, int layer) {
  Dims d;
  if (validate(p, &d) != MOE_OK || layer < 1 || layer > 4) return 0;
  return packed_weight_bytes(d, layer);
}

moe_status moe_route(const moe_problem* p, const void* X, const float* Wg, const float* Wnoise,
                     const float* bias, const float* eps, int32_t* ids, float* gates, float* clean,
                     float* noise_std, float* row_stats, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
  Dims d;
  MOE_TRY(validate_topk(p, &d));
  const bool noise = d.gating == MOE_GATE_NOISY_TOPK && d.noise;
  if (!X || !Wg || !ids || !gates || !clean) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, Wg, Wnoise, bias, eps, ids, gates, clean, noise_std, row_stats, workspace);
  if (noise && (!Wnoise || !noise_std)) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < route_workspace(d)) return MOE_ERR_WORKSPACE;
  int* flag;
  MOE_TRY(flag_for(p, &flag));
  return route_launch(d, p, X, Wg, Wnoise, bias, eps, ids, gates, clean, noise_std, row_stats,
                      workspace, flag, as_stream(hip_stream));
}

moe_status moe_dispatch(const moe_problem* p, const void* X, const int32_t* ids, int32_t* pos,
                        uint8_t* accepted, int32_t* counts, int32_t* offsets, int32_t* row_token,
                        void* Xd, void* workspace, size_t workspace_bytes, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_topk(p, &d));
  if (!X || !ids || !pos || !accepted || !counts || !offsets || !row_token)
    return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, ids, pos, accepted, counts, offsets, row_token, Xd, workspace);
  if (!workspace || workspace_bytes < dispatch_workspace(d)) return MOE_ERR_WORKSPACE;
  return dispatch_launch(d, X, ids, pos, accepted, counts, offsets, row_token, Xd, workspace,
                         as_stream(hip_stream));
}

moe_status moe_dispatch_noalloc(const moe_problem* p, const void* X, const int32_t* ids,
                                int32_t* pos, uint8_t* accepted, int32_t* counts,
                                int32_t* offsets, int32_t* row_token, void* Xd,
                                void* hip_stream) {
  Dims d;
  MOE_TRY(validate_topk(p, &d));
  if (!X || !ids || !pos || !accepted || !counts || !offsets || !row_token)
    return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, ids, pos, accepted, counts, offsets, row_token, Xd);
  if (dispatch_workspace(d) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  return dispatch_noalloc_launch(d, X, ids, pos, accepted, counts, offsets, row_token, Xd,
                                 as_stream(hip_stream));
}

moe_status moe_pack_expert_weights(const moe_problem* p, const void* W1, const void* W2, void* W1p,
                                   void* W2p, void* hip_stream) {
  Dims d;
  MOE_TRY(validate(p, &d));
  if ((W1 && !W1p) || (W2 && !W2p) || (!W1 && !W2)) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(W1, W2, W1p, W2p);
  if (W1) MOE_TRY(pack_launch(d, 1, W1, W1p, as_stream(hip_stream)));
  if (W2) MOE_TRY(pack_launch(d, 2, W2, W2p, as_stream(hip_stream)));
  return MOE_OK;
}

moe_status moe_grouped_gemm(const moe_problem* p, int layer, const void* A, const void* Wp,
                            const int32_t* offsets, void* C, void* hip_stream) {
  Dims d;
  MOE_TRY(validate(p, &d));
  if (layer != 1 && layer != 2) return MOE_ERR_INVALID_ARG;
  if (!A || !Wp || !offsets || !C) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(A, Wp, offsets, C);
  int* flag = nullptr;
  if (layer == 2) MOE_TRY(flag_for(p, &flag));
  return gemm_launch(d, layer, A, Wp, offsets, C, flag, as_stream(hip_stream));
}

moe_status moe_expert_ffn(const moe_problem* p, const void* Xd, const void* W1p, const void* W2p,
                          const int32_t* offsets, void* Hd, void* Z, void* hip_stream) {
  Dims d;
  MOE_TRY(validate(p, &d));
  if (!Xd || !W1p || !W2p || !offsets || !Hd || !Z) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(Xd, W1p, W2p, offsets, Hd, Z);
  int* flag;
  MOE_TRY(flag_for(p, &flag));
  MOE_TRY(gemm_launch(d, 1, Xd, W1p, offsets, Hd, nullptr, as_stream(hip_stream)));
  return gemm_launch(d, 2, Hd, W2p, offsets, Z, flag, as_stream(hip_stream));
}

moe_status moe_grouped_gemm_gather(const moe_problem* p, const void* X, const int32_t* row_token,
                                   const void* W1p, const int32_t* offsets, void* Hd,
                                   void* hip_stream) {
  Dims d;
  MOE_TRY(validate(p, &d));
  if (!X || !row_token || !W1p || !offsets || !Hd) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, row_token, W1p, offsets, Hd);
  return gemm_launch(d, 1, X, W1p, offsets, Hd, nullptr, as_stream(hip_stream), nullptr, row_token);
}

moe_status moe_expert_ffn_gather(const moe_problem* p, const void* X, const int32_t* row_token,
                                 const void* W1p, const void* W2p, const int32_t* offsets,
                                 void* Hd, void* Z, void* hip_stream) {
  Dims d;
  MOE_TRY(validate(p, &d));
  if (!X || !row_token || !W1p || !W2p || !offsets || !Hd || !Z) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, row_token, W1p, W2p, offsets, Hd, Z);
  int* flag;
  MOE_TRY(flag_for(p, &flag));
  MOE_TRY(gemm_launch(d, 1, X, W1p, offsets, Hd, nullptr, as_stream(hip_stream), nullptr, row_token));
  return gemm_launch(d, 2, Hd, W2p, offsets, Z, flag, as_stream(hip_stream));
}

moe_status moe_combine(const moe_problem* p, const void* Z, const int32_t* ids, const float* gates,
                       const int32_t* pos, const uint8_t* accepted, const int32_t* offsets,
                       const void* residual, void* Y, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_topk(p, &d));
  if (!Z || !ids || !gates || !pos || !accepted || !offsets || !Y) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(Z, ids, gates, pos, accepted, offsets, residual, Y);
  int* flag;
  MOE_TRY(flag_for(p, &flag));
  return combine_launch(d, Z, ids, gates, pos, accepted, offsets, residual, Y, flag,
                        as_stream(hip_stream));
}

moe_status moe_aux_loss(const moe_problem* p, const int32_t* ids, const float* gates,
                        const float* clean, const float* noise_std, const float* row_stats,
                        const int32_t* counts, float* importance, float* load, float* out,
                        void* workspace, size_t workspace_bytes, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_topk(p, &d));
  const bool noise = d.gating == MOE_GATE_NOISY_TOPK && d.noise;
  if (!ids || !gates || !clean || !counts || !out) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(ids, gates, clean, noise_std, row_stats, counts, importance, load, out, workspace);
  if (noise && (!noise_std || !row_stats)) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < aux_workspace(d)) return MOE_ERR_WORKSPACE;
  return aux_launch(d, ids, gates, clean, noise_std, row_stats, counts, importance, load, out,
                    workspace, as_stream(hip_stream));
}

size_t moe_hier_workspace_size(const moe_problem* p, const moe_hier* h, int which) {
  Dims d;
  if (validate_hier(p, h, &d) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_ROUTE: return hier_route_workspace(d, h);
    case MOE_WS_AUX: return hier_aux_workspace(d, h);
    default: return 0;
  }
}

moe_status moe_route_hier(const moe_problem* p, const moe_hier* h, const void* X,
                          const float* Wpg, const float* Wpn, const float* Wsg, const float* Wsn,
                          int32_t* ids, float* gates, const moe_hier_state* st, void* workspace,
                          size_t workspace_bytes, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_hier(p, h, &d));
  const bool noise = d.noise != 0;
  if (!X || !Wpg || !Wsg || !ids || !gates || !st) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, Wpg, Wpn, Wsg, Wsn, ids, gates, workspace);
  if (!hier_state_aligned(st)) return MOE_ERR_INVALID_ARG;
  if (noise && (!Wpn || !Wsn || !st->std_p || !st->std_s)) return MOE_ERR_INVALID_ARG;
  if (!st->ids_p || !st->gates_p || !st->clean_p || !st->row_stats_p || !st->pos_p ||
      !st->accepted_p || !st->counts_p || !st->offsets_p || !st->row_token_p || !st->clean_s ||
      !st->row_stats_s || !st->ids_s || !st->gates_s)
    return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < hier_route_workspace(d, h)) return MOE_ERR_WORKSPACE;
  int* flag;
  MOE_TRY(flag_for(p, &flag));
  return hier_route_launch(d, h, p, X, Wpg, Wpn, Wsg, Wsn, ids, gates, st, workspace, flag,
                           as_stream(hip_stream));
}

moe_status moe_aux_loss_hier(const moe_problem* p, const moe_hier* h, const moe_hier_state* st,
                             float* importance,
                             float* load, float* out, void* workspace, size_t workspace_bytes,
                             void* hip_stream) {
  Dims d;
  MOE_TRY(validate_hier(p, h, &d));
  const bool noise = d.noise != 0;
  if (!st || !out) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(importance, load, out, workspace);
  if (!hier_state_aligned(st)) return MOE_ERR_INVALID_ARG;
  if (noise && (!st->std_p || !st->std_s)) return MOE_ERR_INVALID_ARG;
  if (!st->ids_p || !st->gates_p || !st->clean_p || !st->row_stats_p || !st->counts_p ||
      !st->offsets_p || !st->row_token_p || !st->clean_s || !st->row_stats_s || !st->ids_s ||
      !st->gates_s)
    return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < hier_aux_workspace(d, h)) return MOE_ERR_WORKSPACE;
  return hier_aux_launch(d, h, st, importance, load, out, workspace, as_stream(hip_stream));
}

// --------------------------------------------------------------- batchwise mask
static moe_status validate_batchwise(const moe_problem* p, Dims* d) {
  MOE_TRY(validate(p, d));
  return d->gating == MOE_GATE_BATCHWISE ? MOE_OK : MOE_ERR_INVALID_ARG;
}

static bool batchwise_state_ok(const moe_batchwise_state* st) {
  return st && st->probs_t && st->sel && st->offsets && st->mask && st->tok_count && st->tok_off &&
         st->tok_row && st->tok_gate && st->slot_pair &&
         aligned16(st->probs_t, st->sel, st->offsets, st->mask, st->tok_count, st->tok_off,
                   st->tok_row, st->tok_gate, st->slot_pair);
}

int32_t moe_batchwise_m(const moe_problem* p) {
  Dims d;
  return validate_batchwise(p, &d) == MOE_OK ? batchwise_m(d) : -1;
}

size_t moe_batchwise_workspace_size(const moe_problem* p, int which) {
  Dims d;
  if (validate_batchwise(p, &d) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_ROUTE: return batchwise_route_workspace(d);
    case MOE_WS_AUX: return batchwise_aux_workspace(d);
    default: return 0;
  }
}

moe_status moe_route_batchwise(const moe_problem* p, const void* X, const float* Wg,
                               const float* bias, float* clean, const moe_batchwise_state* st,
                               void* workspace, size_t workspace_bytes, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_batchwise(p, &d));
  if (!X || !Wg || !clean || !batchwise_state_ok(st)) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, Wg, bias, clean, workspace);
  if (!workspace || workspace_bytes < batchwise_route_workspace(d)) return MOE_ERR_WORKSPACE;
  int* flag;
  MOE_TRY(flag_for(p, &flag));
  return batchwise_route_launch(d, X, Wg, bias, clean, st, workspace, flag, as_stream(hip_stream));
}

moe_status moe_dispatch_batchwise(const moe_problem* p, const void* X,
                                  const moe_batchwise_state* st, void* Xd, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_batchwise(p, &d));
  if (!X || !Xd || !batchwise_state_ok(st)) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, Xd);
  return batchwise_dispatch_launch(d, X, st, Xd, as_stream(hip_stream));
}

moe_status moe_combine_batchwise(const moe_problem* p, const void* Z, const moe_batchwise_state* st,
                                 const void* residual, void* Y, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_batchwise(p, &d));
  if (!Z || !Y || !batchwise_state_ok(st)) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(Z, residual, Y);
  int* flag;
  MOE_TRY(flag_for(p, &flag));
  return batchwise_combine_launch(d, Z, st, residual, Y, flag, as_stream(hip_stream));
}

moe_status moe_aux_loss_batchwise(const moe_problem* p, const moe_batchwise_state* st,
                                  const float* thresholds, float* importance, float* out,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_batchwise(p, &d));
  if (!out || !batchwise_state_ok(st)) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(thresholds, importance, out, workspace);
  if (!workspace || workspace_bytes < batchwise_aux_workspace(d)) return MOE_ERR_WORKSPACE;
  return batchwise_aux_launch(d, st, thresholds, importance, out, workspace, as_stream(hip_stream));
}

// --------------------------------------------------------------- backward
// The backward covers the per-token gates (noisy top-k and Switch top-1); the gate-specific
// entry points check which one they were given.
static moe_status validate_backward(const moe_problem* p, Dims* d) {
  MOE_TRY(validate(p, d));
  return d->gating == MOE_GATE_BATCHWISE ? MOE_ERR_INVALID_ARG : MOE_OK;
}

moe_status moe_pack_expert_weights_t(const moe_problem* p, const void* W1, const void* W2,
                                     void* W1t, void* W2t, void* hip_stream) {
  Dims d;
  MOE_TRY(validate(p, &d));
  if ((W1 && !W1t) || (W2 && !W2t) || (!W1 && !W2)) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(W1, W2, W1t, W2t);
  if (W2) MOE_TRY(pack_launch(d, 3, W2, W2t, as_stream(hip_stream)));
  if (W1) MOE_TRY(pack_launch(d, 4, W1, W1t, as_stream(hip_stream)));
  return MOE_OK;
}

moe_status moe_combine_backward(const moe_problem* p, const void* dY, const void* Z,
                                const int32_t* ids, const float* gates, const int32_t* pos,
                                const uint8_t* accepted, const int32_t* offsets, void* dZ,
                                float* dgates, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_backward(p, &d));
  if (!dY || !Z || !ids || !gates || !pos || !accepted || !offsets || !dZ || !dgates)
    return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(dY, Z, ids, gates, pos, accepted, offsets, dZ, dgates);
  return combine_backward_launch(d, dY, Z, ids, gates, pos, accepted, offsets, dZ, dgates,
                                 as_stream(hip_stream));
}

moe_status moe_expert_ffn_backward(const moe_problem* p, const void* Xd, const void* Hd,
                                   const void* dZ, const void* W1t, const void* W2t,
                                   const int32_t* offsets, void* dHp, void* dXd, float* dW1,
                                   float* dW2, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_backward(p, &d));
  if (!Xd || !Hd || !dZ || !W1t || !W2t || !offsets || !dHp || !dXd) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(Xd, Hd, dZ, W1t, W2t, offsets, dHp, dXd, dW1, dW2);
  return ffn_backward_launch(d, Xd, Hd, dZ, W1t, W2t, offsets, dHp, dXd, dW1, dW2,
                             as_stream(hip_stream));
}

moe_status moe_expert_ffn_backward_recompute(const moe_problem* p, const void* Xd,
                                             const void* W1p, const void* dZ, const void* W1t,
                                             const void* W2t, const int32_t* offsets,
                                             void* Hd_scratch, void* dHp, void* dXd, float* dW1,
                                             float* dW2, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_backward(p, &d));
  if (!Xd || !W1p || !dZ || !W1t || !W2t || !offsets || !Hd_scratch || !dHp || !dXd)
    return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(Xd, W1p, dZ, W1t, W2t, offsets, Hd_scratch, dHp, dXd, dW1, dW2);
  const hipStream_t s = as_stream(hip_stream);
  MOE_TRY(gemm_launch(d, 1, Xd, W1p, offsets, Hd_scratch, nullptr, s));
  return ffn_backward_launch(d, Xd, Hd_scratch, dZ, W1t, W2t, offsets, dHp, dXd, dW1, dW2, s);
}

moe_status moe_expert_weight_grad(const moe_problem* p, int32_t which, const void* A,
                                  const void* B, const int32_t* offsets, float* C,
                                  void* hip_stream) {
  Dims d;
  MOE_TRY(validate_backward(p, &d));
  if (which != 1 && which != 2) return MOE_ERR_INVALID_ARG;
  if (!A || !B || !offsets || !C) return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(A, B, offsets, C);
  return which == 1 ? wgrad_launch(d, A, B, offsets, d.E, d.D, d.H, C, as_stream(hip_stream))
                    : wgrad_launch(d, A, B, offsets, d.E, d.H, d.D, C, as_stream(hip_stream));
}

size_t moe_backward_workspace_size(const moe_problem* p) {
  Dims d;
  if (validate_backward(p, &d) != MOE_OK) return 0;
  return route_backward_workspace(d);
}

const float* moe_route_scores(const moe_problem* p, const void* route_workspace) {
  Dims d;
  if (validate_topk(p, &d) != MOE_OK) return nullptr;
  return route_scores(d, route_workspace);
}

moe_status moe_route_backward(const moe_problem* p, const void* X, const float* Wg,
                              const float* Wnoise, const float* eps, const float* scores,
                              const int32_t* ids,
                              const float* gates, const float* clean, const float* noise_std,
                              const float* row_stats, const float* dgates, const float* importance,
                              const float* load, float w_imp, float w_load,
                              const void* dY_residual, const void* dXd, const int32_t* pos,
                              const uint8_t* accepted, const int32_t* offsets, void* dX,
                              float* dWg, float* dWnoise, float* dbias, void* workspace,
                              size_t workspace_bytes, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_backward(p, &d));
  if (d.gating != MOE_GATE_NOISY_TOPK) return MOE_ERR_INVALID_ARG;  // Switch: its own entry point
  const bool noise = d.noise != 0;
  if (!isfinite(w_imp) || !isfinite(w_load)) return MOE_ERR_INVALID_ARG;
  if (!X || !Wg || !ids || !gates || !clean || !row_stats || !dgates || !dXd || !pos ||
      !accepted || !offsets || !dX || !dWg)
    return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, Wg, Wnoise, eps, scores, ids, gates, clean, noise_std, row_stats, dgates,
              importance, load, dY_residual, dXd, pos, accepted, offsets, dX, dWg, dWnoise, dbias,
              workspace);
  if (noise && (!Wnoise || !noise_std || !dWnoise)) return MOE_ERR_INVALID_ARG;
  if (w_imp != 0.f && !importance) return MOE_ERR_INVALID_ARG;
  if (w_load != 0.f && noise && !load) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < route_backward_workspace(d)) return MOE_ERR_WORKSPACE;
  return route_backward_launch(d, p->seed, X, Wg, Wnoise, eps, scores, ids, gates, clean,
                               noise_std, row_stats, dgates, importance, load, nullptr, w_imp,
                               w_load, 0.f, dY_residual, dXd, pos, accepted, offsets, dX, dWg,
                               dWnoise, dbias, workspace, as_stream(hip_stream));
}

moe_status moe_route_backward_switch(const moe_problem* p, const void* X, const float* Wg,
                                     const int32_t* ids, const float* clean, const float* dgates,
                                     const float* importance, const int32_t* counts, float w_imp,
                                     float w_switch, const void* dY_residual, const void* dXd,
                                     const int32_t* pos, const uint8_t* accepted,
                                     const int32_t* offsets, void* dX, float* dWg, float* dbias,
                                     void* workspace, size_t workspace_bytes, void* hip_stream) {
  Dims d;
  MOE_TRY(validate_backward(p, &d));
  if (d.gating != MOE_GATE_SWITCH_TOP1) return MOE_ERR_INVALID_ARG;
  if (!isfinite(w_imp) || !isfinite(w_switch)) return MOE_ERR_INVALID_ARG;
  if (!X || !Wg || !ids || !clean || !dgates || !dXd || !pos || !accepted || !offsets || !dX ||
      !dWg)
    return MOE_ERR_INVALID_ARG;
  MOE_ALIGNED(X, Wg, ids, clean, dgates, importance, counts, dY_residual, dXd, pos, accepted,
              offsets, dX, dWg, dbias, workspace);
  if (w_imp != 0.f && !importance) return MOE_ERR_INVALID_ARG;
  if (w_switch != 0.f && !counts) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < route_backward_workspace(d)) return MOE_ERR_WORKSPACE;
  return route_backward_launch(d, p->seed, X, Wg, nullptr, nullptr, nullptr, ids, nullptr, clean,
                               nullptr, nullptr, dgates, importance, nullptr, counts, w_imp, 0.f,
                               w_switch,
                               dY_residual, dXd, pos, accepted, offsets, dX, dWg, nullptr, dbias,
                               workspace, as_stream(hip_stream));
}

moe_status moe_check_finite(void* hip_stream) {
  if (hipStreamSynchronize(as_stream(hip_stream)) != hipSuccess) return MOE_ERR_HIP;
  int v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_nonfinite), sizeof(int), 0, hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_HIP;
  if (v) {
    const int zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_nonfinite), &zero, sizeof(int), 0, hipMemcpyHostToDevice) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_ERR_NONFINITE;
  }
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported problem";
    case MOE_ERR_NONFINITE: return "non-finite value seen";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

}  // extern "C"
