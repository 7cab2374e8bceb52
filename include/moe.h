/*
 * moe.h -- C ABI of the MI355X (gfx950) sparsely-gated Mixture-of-Experts
 * layer: forward pass (flat, hierarchical and batchwise gates) and backward pass
 * (noisy top-k and Switch gates).
 *
 * Pages cited (by title; sections as the pages name them):
 *   [OLNN]   "Outrageously Large Neural Networks: The Sparsely-Gated
 *            Mixture-of-Experts Layer", paper summary page, section 3.4
 *            ("The MoE Output and Gating Network Formulation", "Noisy Top-K
 *            Gating" Steps 1-3, "Load-Balancing: The Importance and Load
 *            Losses").
 *   [SWITCH] "Switch Transformer" explainer page, "Implementation", steps 1-8.
 *   [LESSON] "Mixture-of-Experts: Sparse Computation" lesson page, ch. 1-5.
 *
 * The layer: X[T,D] tokens; router weights Wg, Wnoise [D,E]; E experts, each
 * ReLU(x W1_e) W2_e with W1_e [D,H] and W2_e [H,D]; k experts per token; a
 * capacity factor bounds how many rows each expert accepts.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed, owned
 *     by the caller. The library never allocates device memory; scratch comes
 *     from the caller as `workspace` (size from moe_workspace_size).
 *   - Every tensor and workspace pointer (also those inside moe_hier_state and
 *     moe_batchwise_state) is 16-byte aligned, or NULL where NULL is allowed:
 *     rows move as 16-byte vectors. hipMalloc and the PyTorch allocator give
 *     256-byte alignment; a misaligned pointer is MOE_ERR_INVALID_ARG.
 *   - `hip_stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Every entry point only enqueues work on that stream and returns; it never
 *     synchronises. Counts and offsets stay on the device.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     return a negative moe_status; outputs are then untouched. An error from a
 *     HIP launch returns MOE_ERR_HIP.
 *   - Floating-point activations (X, Xd, Hd, Z, Y) and the expert weights share
 *     one dtype, p->dtype: fp32, or bf16 stored as raw 16-bit patterns. Router
 *     weights, logits, gates and the aux outputs are always fp32.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a size, pointer or option out of range       */
  MOE_ERR_UNSUPPORTED = -2, /* valid, but outside what the kernels implement */
  MOE_ERR_NONFINITE = -3,   /* check_finite saw a NaN/Inf (moe_check_finite) */
  MOE_ERR_HIP = -4,         /* a HIP runtime call failed                    */
  MOE_ERR_WORKSPACE = -5    /* workspace missing or smaller than required   */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_GATE_NOISY_TOPK = 0,  /* [OLNN] 3.4 Noisy Top-K Gating                */
  MOE_GATE_SWITCH_TOP1 = 1, /* [SWITCH] steps 1-2                           */
  MOE_GATE_BATCHWISE = 2    /* [OLNN] 3.4 Strictly Balanced Gating: the
                               moe_*_batchwise entry points only           */
} moe_gating;

/* Largest k the kernels support. */
#define MOE_MAX_K 8

typedef struct {
  int32_t T;                /* tokens (rows of X), >= 1                      */
  int32_t D;                /* model width, >= 1                             */
  int32_t E;                /* experts, >= 1                                 */
  int32_t H;                /* expert hidden width, >= 1                     */
  int32_t k;                /* experts per token, 1 <= k <= min(E, MOE_MAX_K); 1 for Switch */
  int32_t dtype;            /* moe_dtype of X, Xd, Hd, Z, Y, W1, W2           */
  int32_t gating;           /* moe_gating                                    */
  int32_t noise;            /* noisy gate only: 1 adds softplus-scaled noise */
  float capacity_factor;    /* <= 0: no capacity limit ([SWITCH] step 3)     */
  int32_t min_capacity;     /* lower clamp of the capacity, >= 1             */
  uint64_t seed;            /* noise key: eps[t,e] from (seed, t, e)          */
  int32_t check_finite;     /* 1: kernels record NaN/Inf seen in logits, expert
                               outputs and Y; read with moe_check_finite       */
  int32_t reserved;
} moe_problem;

/* Workspace kinds for moe_workspace_size. */
enum { MOE_WS_ROUTE = 0, MOE_WS_DISPATCH = 1, MOE_WS_AUX = 2 };

/* ------------------------------------------------------------------ sizes */

/* Capacity C per expert ([SWITCH] step 3, read for k experts per token):
 * C = max(min_capacity, min(T, floor(k*T*cf/E))), the product in double;
 * cf <= 0 gives C = T (no expert can receive more than T rows).
 * Returns -1 on an invalid problem. */
int32_t moe_capacity(const moe_problem* p);

/* Upper bound on accepted (token, expert) rows: min(T*k, E*C). Sizes row_token,
 * Xd, Hd and Z. Returns -1 on an invalid problem. */
int64_t moe_max_rows(const moe_problem* p);

/* Bytes of workspace needed by moe_route / moe_dispatch / moe_aux_loss
 * (which = MOE_WS_*). 0 on an invalid problem. */
size_t moe_workspace_size(const moe_problem* p, int which);

/* Bytes of one packed expert-weight buffer (layer 1: W1, layer 2: W2). 0 on
 * an invalid problem. */
size_t moe_packed_weight_bytes(const moe_problem* p, int layer);

/* ------------------------------------------------------------------ router */

/* moe_route -- gating network for every token.
 *
 * Noisy top-k ([OLNN] 3.4 "Noisy Top-K Gating", Steps 1-3):
 *   clean = X Wg (+ bias), std = Softplus(X Wnoise), H = clean + eps * std,
 *   keep the k largest H (ties: lower expert index first), gates = softmax
 *   over the k kept values. With p->noise = 0, H = clean.
 * Switch top-1 ([SWITCH] steps 1-2): expert = argmax of softmax(clean)
 *   (first on ties), gate = its softmax probability (not renormalised).
 * Routing is decided on fp32 scores.
 *
 *   X          [T,D]  p->dtype
 *   Wg         [D,E]  fp32
 *   Wnoise     [D,E]  fp32; required iff noisy gate with noise, else ignored
 *   bias       [E]    fp32 added to clean, or NULL
 *   eps        [T,E]  fp32 external noise, or NULL: eps[t,e] is then drawn in
 *                     the kernel from (p->seed, t, e) by Philox4x64-10 and
 *                     Box-Muller (counter (t, e/4, 0, 0), key (seed, 0); the
 *                     four outputs feed experts 4q..4q+3 as cos, sin, cos, sin)
 *   ids        [T,k]  int32 out: kept experts, by score descending, index ascending
 *   gates      [T,k]  fp32 out
 *   clean      [T,E]  fp32 out: X Wg (+ bias)
 *   noise_std  [T,E]  fp32 out: Softplus(X Wnoise); required iff noise is used
 *   row_stats  [T,2]  fp32 out or NULL: k-th and (k+1)-th largest score
 *                     (-inf when k = E); these are the load estimator's
 *                     thresholds ([OLNN] 3.4, load)
 *   workspace  moe_workspace_size(p, MOE_WS_ROUTE) bytes (router weights are
 *              re-laid out there on every call)
 */
moe_status moe_route(const moe_problem* p, const void* X, const float* Wg,
                     const float* Wnoise, const float* bias, const float* eps,
                     int32_t* ids, float* gates, float* clean, float* noise_std,
                     float* row_stats, void* workspace, size_t workspace_bytes,
                     void* hip_stream);

/* The noisy scores H = clean + eps * noise_std [T,E] fp32 that the last moe_route
 * selected on live in its workspace; this returns their device address inside
 * route_workspace (NULL for a gate without noise or an invalid problem). They
 * stay valid until the workspace is used again; moe_route_backward can take them. */
const float* moe_route_scores(const moe_problem* p, const void* route_workspace);

/* --------------------------------------------------------------- dispatch */

/* moe_dispatch -- capacity-bounded, stable dispatch ([SWITCH] steps 3-5).
 *
 * counts[e]   = assignments to e before capacity.
 * pos[t,j]    = number of earlier assignments (token-major: lower t, then
 *               lower j) to the same expert: a stable slot.
 * accepted    = pos < C (C from moe_capacity).
 * offsets     = exclusive scan of min(counts, C); offsets[E] = accepted rows.
 * Expert e owns rows offsets[e] .. offsets[e+1]-1 of Xd, in slot order:
 * row_token[offsets[e] + pos] = t and Xd[offsets[e] + pos] = X[t].
 *
 *   X         [T,D] p->dtype      ids [T,k] int32 (each row: k distinct experts)
 *   pos       [T,k] int32 out     accepted [T,k] uint8 out (1 kept, 0 dropped)
 *   counts    [E] int32 out       offsets [E+1] int32 out
 *   row_token [moe_max_rows] int32 out (rows past offsets[E] untouched)
 *   Xd        [moe_max_rows, D] p->dtype out (rows past offsets[E] untouched),
 *             or NULL: no rows are copied, and the gathered entry points below
 *             read X through row_token instead
 *   workspace moe_workspace_size(p, MOE_WS_DISPATCH) bytes
 * ids outside [0,E) give undefined results (not checked on the device).
 */
moe_status moe_dispatch(const moe_problem* p, const void* X, const int32_t* ids,
                        int32_t* pos, uint8_t* accepted, int32_t* counts,
                        int32_t* offsets, int32_t* row_token, void* Xd,
                        void* workspace, size_t workspace_bytes, void* hip_stream);

/* moe_dispatch_noalloc -- moe_dispatch without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and error rules as
 * moe_dispatch (bit-identical outputs); the scratch it needs (the per-block histogram,
 * E * ceil(T / 64) int32) lives in a fixed device array of MOE_NOALLOC_SCRATCH_BYTES
 * inside the library, which each device holds until the process ends. A problem whose
 * scratch would exceed it returns MOE_ERR_WORKSPACE before anything is enqueued. The call
 * allocates nothing (its first call on a device looks up the array's address once). Every
 * call on one device shares that device's array: calls that may overlap on one device
 * (different streams, or host threads) race and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_dispatch_noalloc(const moe_problem* p, const void* X, const int32_t* ids,
                                int32_t* pos, uint8_t* accepted, int32_t* counts,
                                int32_t* offsets, int32_t* row_token, void* Xd,
                                void* hip_stream);

/* ---------------------------------------------------------------- experts */

/* moe_pack_expert_weights -- re-lay the expert weights for the grouped GEMM.
 * Input is the pages' layout ([SWITCH] step 6): W1 [E,D,H], W2 [E,H,D]
 * (p->dtype). Output buffers hold moe_packed_weight_bytes(p, 1) and (p, 2)
 * bytes. Weights are parameters: pack once, reuse for every forward call.
 * Either input may be NULL to skip that layer.
 * Packed layout of a [E,K,N] weight (V = 8 bf16 or 4 fp32 per 16 bytes;
 * NB = ceil(N/32) column blocks; KS = 4 ceil(K / 8V) k-steps of 2V): 1 KB
 * fragments; the 16 bytes of fragment (e, nb, ks) for lane l (0..63) hold
 * column nb 32 + l%32, rows ks 2V + (l/32) V .. +V-1; zeros past K or N.
 * Fragment (e, nb, ks) is at index e NB KS + nb B + (ks/4) S + ks%4 with
 * (B, S) = (4, 4 NB) (k-stage order) when moe_max_rows(p) >= 128 E, else
 * (KS, 4) (column-block order). The transposed packs of
 * moe_pack_expert_weights_t follow the same rule. */
moe_status moe_pack_expert_weights(const moe_problem* p, const void* W1,
                                   const void* W2, void* W1p, void* W2p,
                                   void* hip_stream);

/* moe_grouped_gemm -- one expert layer as a single grouped GEMM over the
 * expert-major rows (groups given by offsets, read on the device).
 *   layer 1: C[r, 0:H] = ReLU(A[r, 0:D] W1_e)   ([SWITCH] step 6)
 *   layer 2: C[r, 0:D] = A[r, 0:H] W2_e
 * for every row r in offsets[e] .. offsets[e+1]-1. fp32 accumulation; C is
 * rounded to p->dtype (bf16: nearest-even). Rows past offsets[E] untouched.
 *   A   [moe_max_rows, D or H] p->dtype     Wp packed weights of that layer
 *   C   [moe_max_rows, H or D] p->dtype out offsets [E+1] int32 */
moe_status moe_grouped_gemm(const moe_problem* p, int layer, const void* A,
                            const void* Wp, const int32_t* offsets, void* C,
                            void* hip_stream);

/* moe_expert_ffn -- both expert layers: Hd = ReLU(Xd W1_e), Z = Hd W2_e
 * ([SWITCH] step 6; [OLNN] 3.4, experts with one ReLU hidden layer).
 *   Xd [moe_max_rows, D]   Hd [moe_max_rows, H] out   Z [moe_max_rows, D] out */
moe_status moe_expert_ffn(const moe_problem* p, const void* Xd, const void* W1p,
                          const void* W2p, const int32_t* offsets, void* Hd,
                          void* Z, void* hip_stream);

/* moe_grouped_gemm_gather / moe_expert_ffn_gather -- layer 1 (and, for the
 * ffn, layer 2) with the dispatch's gather ([SWITCH] step 5) done by the
 * GEMM's row loads: row r of expert e's group is X[row_token[r]], so the
 * dispatch may be called with Xd = NULL. Results are bit-identical to
 * moe_grouped_gemm(layer 1) / moe_expert_ffn on the Xd that moe_dispatch
 * would have written.
 *   X [T,D] p->dtype   row_token [moe_max_rows] int32 from moe_dispatch
 *   W1p, W2p, offsets, Hd, Z as above */
moe_status moe_grouped_gemm_gather(const moe_problem* p, const void* X,
                                   const int32_t* row_token, const void* W1p,
                                   const int32_t* offsets, void* Hd,
                                   void* hip_stream);
moe_status moe_expert_ffn_gather(const moe_problem* p, const void* X,
                                 const int32_t* row_token, const void* W1p,
                                 const void* W2p, const int32_t* offsets,
                                 void* Hd, void* Z, void* hip_stream);

/* ---------------------------------------------------------------- combine */

/* moe_combine -- gate-weighted sum plus residual ([OLNN] 3.4, the MoE output
 * y = sum_i G(x)_i E_i(x); [SWITCH] step 7):
 *   Y[t] = R[t] + sum over accepted j, ascending, of gates[t,j] * Z[offsets[e]+pos]
 * accumulated in fp32 and rounded once to p->dtype. A token whose assignments
 * were all dropped gets Y[t] = R[t] exactly. residual = NULL gives R = 0.
 *   Z [moe_max_rows, D]  ids, gates, pos, accepted [T,k]  offsets [E+1]
 *   residual [T,D] or NULL   Y [T,D] out (p->dtype) */
moe_status moe_combine(const moe_problem* p, const void* Z, const int32_t* ids,
                       const float* gates, const int32_t* pos,
                       const uint8_t* accepted, const int32_t* offsets,
                       const void* residual, void* Y, void* hip_stream);

/* --------------------------------------------------------------- aux loss */

/* moe_aux_loss -- unweighted balancing terms; the caller applies the loss
 * weights (the pages give 0.1 / 0.01 for w_importance, w_load and alpha = 0.01).
 *   importance[e] = sum of gates routed to e, before capacity   ([OLNN] 3.4)
 *   load[e]       = sum_t Phi((clean - thr) / std), thr = row_stats[t,1] if e is
 *                   among ids[t], else row_stats[t,0] (the k-th largest score
 *                   among the other experts); 0 without noise   ([OLNN] 3.4)
 *   out[0] = CV^2(importance)   out[1] = CV^2(load)   (population variance)
 *   out[2] = E * sum_e f_e * Pbar_e, f = counts / T (before capacity),
 *            Pbar = mean over tokens of softmax(clean)    ([SWITCH] step 8)
 *   out[3] = max(load) / mean(load)   out[4] = max(counts) / mean(counts)
 *   out[5] = dropped assignments = sum_e max(counts_e - C, 0)
 *   out[6] = sum(importance)          out[7] = 0
 *   ids, gates [T,k]; clean [T,E]; noise_std [T,E] (NULL without noise);
 *   row_stats [T,2] (required with noise); counts [E];
 *   importance, load [E] fp32 out (either may be NULL); out [8] fp32 out
 *   workspace moe_workspace_size(p, MOE_WS_AUX) bytes */
moe_status moe_aux_loss(const moe_problem* p, const int32_t* ids,
                        const float* gates, const float* clean,
                        const float* noise_std, const float* row_stats,
                        const int32_t* counts, float* importance, float* load,
                        float* out, void* workspace, size_t workspace_bytes,
                        void* hip_stream);

/* ------------------------------------------------------ hierarchical MoE */

/* Two-level gating ([OLNN] 3.4 "Hierarchical Mixture-of-Experts"; [LESSON]
 * ch. 1 "When n gets too large to gate directly", ch. 5 "Balancing at every
 * level"). The p->E experts form `groups` groups of b = E / groups; a primary
 * noisy top-k gate over the groups keeps k_primary of them per token, and group
 * i's own noisy top-k gate keeps k_s = p->k / k_primary of its b experts for the
 * tokens routed to it (X^(i)). Expert (i, j) is expert i*b + j of p, weighted
 * by Gp(x)_i * G_i(x)_j; a token's p->k assignments list the primary slots in
 * the primary's order, each followed by its group's choices in that gate's
 * order. The final ids / gates then go through moe_dispatch, moe_expert_ffn and
 * moe_combine with p unchanged (capacity applies to the p->E experts).
 * Noise: the primary gate draws as moe_route (key (seed, 0)); group i's gate
 * draws from key (seed, 1 + i), counter (t, j / 4), same Box-Muller pairing.
 * Requires p->gating == MOE_GATE_NOISY_TOPK (noise on or off) and no bias. */
typedef struct {
  int32_t groups;     /* a: 1 <= a <= E, E % a == 0                         */
  int32_t k_primary;  /* 1 <= k_primary <= a, p->k % k_primary == 0,
                         p->k / k_primary <= E / a                           */
} moe_hier;

/* Caller-owned device buffers of both levels (fp32 unless noted). R = T *
 * k_primary secondary rows, grouped: group i holds rows offsets_p[i] ..
 * offsets_p[i+1]-1, its tokens in ascending order. std_p / std_s are NULL
 * when p->noise == 0. Written by moe_route_hier, read by moe_aux_loss_hier. */
typedef struct {
  int32_t* ids_p;       /* [T, k_primary] chosen groups, (score desc, index asc) */
  float*   gates_p;     /* [T, k_primary] softmax over the kept group scores    */
  float*   clean_p;     /* [T, groups]   X . Wpg                                 */
  float*   std_p;       /* [T, groups]   Softplus(X . Wpn)                       */
  float*   row_stats_p; /* [T, 2]        k_primary-th, (k_primary+1)-th score    */
  int32_t* pos_p;       /* [T, k_primary] row of the token inside its group      */
  uint8_t* accepted_p;  /* [T, k_primary] all 1: no capacity between the levels  */
  int32_t* counts_p;    /* [groups]      |X^(i)|                                 */
  int32_t* offsets_p;   /* [groups + 1]  first row of each group                 */
  int32_t* row_token_p; /* [R]           token of each secondary row             */
  float*   clean_s;     /* [R, b]        X[token] . Wsg[group]                   */
  float*   std_s;       /* [R, b]        Softplus(X[token] . Wsn[group])         */
  float*   row_stats_s; /* [R, 2]        k_s-th, (k_s+1)-th secondary score      */
  int32_t* ids_s;       /* [R, k_s]      experts within the group                */
  float*   gates_s;     /* [R, k_s]      softmax over the kept secondary scores  */
} moe_hier_state;

/* Workspace bytes for moe_route_hier (which = MOE_WS_ROUTE) or
 * moe_aux_loss_hier (MOE_WS_AUX); 0 for invalid arguments. */
size_t moe_hier_workspace_size(const moe_problem* p, const moe_hier* h, int which);

/* moe_route_hier -- both gate levels and the final assignments.
 *   X [T,D] (p->dtype); Wpg, Wpn [D, groups]; Wsg, Wsn [groups, D, b] (fp32;
 *   Wpn / Wsn NULL without noise); ids [T, p->k] int32 out; gates [T, p->k] out;
 *   st: every buffer above (std_p / std_s only with noise). */
moe_status moe_route_hier(const moe_problem* p, const moe_hier* h, const void* X,
                          const float* Wpg, const float* Wpn, const float* Wsg,
                          const float* Wsn, int32_t* ids, float* gates,
                          const moe_hier_state* st, void* workspace,
                          size_t workspace_bytes, void* hip_stream);

/* moe_aux_loss_hier -- hierarchical balancing terms, unweighted.
 *   importance[i*b+j] = sum over x of Gp(x)_i * G_i(x)_j          (Importance_H)
 *   load[i*b+j]       = Load_p(X)_i * Load_i(X^(i))_j / |X^(i)|  (Load_H), with
 *                       Load_p the moe_aux_loss load of the primary gate over
 *                       all tokens and Load_i that of group i's gate over
 *                       X^(i); 0 for a group no token reached; 0 without noise
 *   out[0] = CV^2(Importance_H)  out[1] = CV^2(Load_H)
 *   out[2] = CV^2(primary importance)  out[3] = CV^2(primary load)
 *   out[4] = max(Load_H) / mean(Load_H)  out[5] = groups with |X^(i)| = 0
 *   out[6] = sum(Importance_H)  out[7] = 0
 *   st as written by moe_route_hier; importance, load [E] out (either may be
 *   NULL); out [8] out; workspace moe_hier_workspace_size(.., MOE_WS_AUX). */
moe_status moe_aux_loss_hier(const moe_problem* p, const moe_hier* h,
                             const moe_hier_state* st, float* importance,
                             float* load, float* out, void* workspace,
                             size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------- batchwise mask */

/* Strictly balanced gating ([OLNN] 3.4 "Strictly Balanced Gating (Batchwise
 * Mask)"; [LESSON] ch. 4 "A stricter alternative", ch. 2's mask form), for
 * p->gating == MOE_GATE_BATCHWISE (p->noise must be 0; capacity does not apply).
 * Scores s = Softmax(X . Wg (+ bias)) per token (dense, fp32). Each expert e
 * keeps the m = floor(p->k * T / E) tokens with the highest s[., e] (ties to the
 * lower token), so every expert receives exactly m rows; token t gets
 * G(t)_e = s[t,e] / sum of s[t,.] over the experts that kept it, for each of
 * them (any number, possibly none: then Y[t] = residual[t]). Expert-major row
 * e*m + j holds the j-th kept token of expert e (ascending), so the expert FFN
 * runs through moe_expert_ffn with offsets[e] = e*m. */
typedef struct {
  float*    probs_t;    /* [E, T]  scores s, expert-major                        */
  int32_t*  sel;        /* [E*m]   token of expert-major row r                   */
  int32_t*  offsets;    /* [E+1]   e*m                                           */
  uint32_t* mask;       /* [T, ceil(E/32)] bit e%32 of word e/32: t kept by e     */
  int32_t*  tok_count;  /* [T]     experts that kept token t                     */
  int32_t*  tok_off;    /* [T+1]   token t's entries tok_off[t] .. tok_off[t+1]-1 */
  int32_t*  tok_row;    /* [E*m]   per entry: expert-major row (experts ascending) */
  float*    tok_gate;   /* [E*m]   per entry: G(t)_e                             */
  int32_t*  slot_pair;  /* [E*m]   entry index of expert-major row r             */
} moe_batchwise_state;

/* m for the problem, or -1 if invalid (m < 1 is invalid). */
int32_t moe_batchwise_m(const moe_problem* p);

/* Workspace bytes for moe_route_batchwise (MOE_WS_ROUTE) or
 * moe_aux_loss_batchwise (MOE_WS_AUX); 0 if invalid. */
size_t moe_batchwise_workspace_size(const moe_problem* p, int which);

/* moe_route_batchwise -- scores, the mask and the gates.
 *   X [T,D]; Wg [D,E] fp32; bias [E] or NULL; clean [T,E] out (X . Wg + bias);
 *   st: every buffer above, written. */
moe_status moe_route_batchwise(const moe_problem* p, const void* X, const float* Wg,
                               const float* bias, float* clean,
                               const moe_batchwise_state* st, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/* moe_dispatch_batchwise -- Xd[r] = X[sel[r]] for the E*m rows. Xd [E*m, D] out. */
moe_status moe_dispatch_batchwise(const moe_problem* p, const void* X,
                                  const moe_batchwise_state* st, void* Xd,
                                  void* hip_stream);

/* moe_combine_batchwise -- Y[t] = residual[t] + sum over token t's entries
 * (experts ascending) of tok_gate * Z[tok_row], fp32 accumulation, one rounding.
 *   Z [E*m, D] (moe_expert_ffn output); residual [T,D] or NULL; Y [T,D] out. */
moe_status moe_combine_batchwise(const moe_problem* p, const void* Z,
                                 const moe_batchwise_state* st, const void* residual,
                                 void* Y, void* hip_stream);

/* moe_aux_loss_batchwise -- importance[e] = sum of the gates e received;
 *   out[0] = CV^2(importance)
 *   out[1] = L_batchwise = sum_t sum_e (1[s[t,e] > thresholds[e]] - mask[t,e])
 *            * (s[t,e] - thresholds[e])   (0 if thresholds is NULL)
 *   out[2] = mean experts per token (= E*m/T)  out[3] = max experts per token
 *   out[4] = tokens no expert kept  out[5] = sum(importance)  out[6] = m  out[7] = 0
 *   thresholds [E] or NULL; importance [E] out or NULL; out [8] out;
 *   workspace moe_batchwise_workspace_size(p, MOE_WS_AUX). */
moe_status moe_aux_loss_batchwise(const moe_problem* p, const moe_batchwise_state* st,
                                  const float* thresholds, float* importance,
                                  float* out, void* workspace, size_t workspace_bytes,
                                  void* hip_stream);

/* -------------------------------------------------------------- backward */

/* Gradients of the noisy top-k layer ([OLNN] 3.4: the gate trains through the
 * softmax over the kept experts and through the importance and load losses;
 * [LESSON] ch. 3 "trace it forward, then backward"). The selection, the
 * capacity mask and the noise are those of the forward and are held fixed (the
 * selection is piecewise constant); the load estimator's threshold is the k-th
 * or (k+1)-th score of the row and passes its gradient to that expert. The
 * objective is <Y, dY> + w_imp CV^2(importance) + w_load CV^2(load). Order:
 * moe_combine_backward -> moe_expert_ffn_backward -> moe_route_backward, on the
 * forward's buffers. The Switch gate ([SWITCH] steps 2 and 8: the gate is the
 * selected full-softmax probability; the balancing term E * sum f * Pbar trains
 * the router through Pbar, the hard fractions f held fixed) uses the same first
 * two calls, then moe_route_backward_switch. The batchwise mask has no backward
 * here (MOE_ERR_INVALID_ARG). Weight gradients are fp32 and overwrite their
 * outputs. */

/* W1^T and W2^T in MFMA fragment order (layers 4 and 3 of moe_packed_weight_bytes). */
moe_status moe_pack_expert_weights_t(const moe_problem* p, const void* W1, const void* W2,
                                     void* W1t_packed, void* W2t_packed, void* hip_stream);

/* dZ[row] = gate * dY[t] for every accepted assignment (p->dtype); dgates[t,j] =
 * <dY[t], Z[row]> (fp32; 0 for dropped assignments). dY [T,D]; Z, dZ [rows, D]. */
moe_status moe_combine_backward(const moe_problem* p, const void* dY, const void* Z,
                                const int32_t* ids, const float* gates, const int32_t* pos,
                                const uint8_t* accepted, const int32_t* offsets, void* dZ,
                                float* dgates, void* hip_stream);

/* dHp = (dZ W2_e^T) masked where Hd <= 0 (the ReLU derivative) [rows, H];
 * dXd = dHp W1_e^T [rows, D]; dW2_e = Hd_e^T dZ_e [E,H,D] and dW1_e = Xd_e^T dHp_e
 * [E,D,H] (fp32; either may be NULL). Xd, Hd from the forward; Xd must hold the rows,
 * i.e. come from a moe_dispatch called with a non-NULL Xd (a dispatch with Xd = NULL,
 * for the gathered layer 1, leaves it unwritten and the gradients would be wrong). */
moe_status moe_expert_ffn_backward(const moe_problem* p, const void* Xd, const void* Hd,
                                   const void* dZ, const void* W1t_packed,
                                   const void* W2t_packed, const int32_t* offsets, void* dHp,
                                   void* dXd, float* dW1, float* dW2, void* hip_stream);

/* moe_expert_ffn_backward without a stored hidden layer ([LESSON] ch. 4, "recompute
 * instead of store": the experts' hidden activations are not kept from the forward but
 * recomputed in the backward, a second layer-1 pass traded for their memory): first
 * Hd = ReLU(Xd_e W1_e) into the caller's Hd_scratch [rows, H] (p->dtype; overwritten;
 * bitwise equal to the forward's Hd) from W1_packed (moe_pack_expert_weights layout),
 * then exactly moe_expert_ffn_backward on it. */
moe_status moe_expert_ffn_backward_recompute(const moe_problem* p, const void* Xd,
                                             const void* W1_packed, const void* dZ,
                                             const void* W1t_packed, const void* W2t_packed,
                                             const int32_t* offsets, void* Hd_scratch,
                                             void* dHp, void* dXd, float* dW1, float* dW2,
                                             void* hip_stream);

/* One weight gradient of moe_expert_ffn_backward on its own (the same kernel):
 * which = 1: C_e = A_e^T B_e with A = Xd [rows, D], B = dHp [rows, H], C = dW1 [E,D,H];
 * which = 2: A = Hd [rows, H], B = dZ [rows, D], C = dW2 [E,H,D]. fp32 C, overwritten;
 * experts with no rows get zeros. */
moe_status moe_expert_weight_grad(const moe_problem* p, int32_t which, const void* A,
                                  const void* B, const int32_t* offsets, float* C,
                                  void* hip_stream);

/* The gate and router: dclean and d raw from the softmax over the kept scores, the
 * importance term (importance [E] from moe_aux_loss, needed if w_imp != 0) and the
 * load term (load [E], needed if w_load != 0; noise only); then
 *   dX = dY (if dY_residual, the forward used residual = X) + the accepted rows
 *        of dXd + [dclean | d raw] [Wg | Wnoise]^T          [T,D] p->dtype
 *   dWg = X^T dclean, dWnoise = X^T d raw  [D,E] fp32; dbias = sum_t dclean [E]
 *   (dWnoise NULL without noise; dbias may be NULL).
 * eps: the external noise given to moe_route, or NULL if the router drew it.
 * scores: the noisy scores H [T,E] the forward selected on (moe_route_scores), or
 *   NULL: they are then formed again from clean, noise_std and the noise, which
 *   for the load term means redrawing the noise of every expert.
 * workspace moe_backward_workspace_size(p) bytes. */
moe_status moe_route_backward(const moe_problem* p, const void* X, const float* Wg,
                              const float* Wnoise, const float* eps, const float* scores,
                              const int32_t* ids,
                              const float* gates, const float* clean, const float* noise_std,
                              const float* row_stats, const float* dgates,
                              const float* importance, const float* load, float w_imp,
                              float w_load, const void* dY_residual, const void* dXd,
                              const int32_t* pos, const uint8_t* accepted,
                              const int32_t* offsets, void* dX, float* dWg, float* dWnoise,
                              float* dbias, void* workspace, size_t workspace_bytes,
                              void* hip_stream);

/* The Switch gate and router: p = softmax(clean) over all E, g = p[e*];
 *   dp[t,e] = (dgates[t] + w_imp dCV^2(importance)/d importance[e*]) 1[e = e*]
 *             + w_switch E counts[e] / T^2
 *   dclean = p (dp - <p, dp>); then dX, dWg, dbias as moe_route_backward (no noise).
 * ids [T] (k = 1), clean [T,E] = X Wg + bias from moe_route; counts [E] the
 * pre-capacity counts from moe_dispatch (needed if w_switch != 0); importance [E]
 * from moe_aux_loss (needed if w_imp != 0). The objective's balancing term is
 * w_switch * E * sum_e f_e Pbar_e (moe_aux_loss out[2] times w_switch).
 * workspace moe_backward_workspace_size(p) bytes. */
moe_status moe_route_backward_switch(const moe_problem* p, const void* X, const float* Wg,
                                     const int32_t* ids, const float* clean, const float* dgates,
                                     const float* importance, const int32_t* counts, float w_imp,
                                     float w_switch, const void* dY_residual, const void* dXd,
                                     const int32_t* pos, const uint8_t* accepted,
                                     const int32_t* offsets, void* dX, float* dWg, float* dbias,
                                     void* workspace, size_t workspace_bytes, void* hip_stream);
size_t moe_backward_workspace_size(const moe_problem* p);

/* ------------------------------------------------------------------- misc */

/* Synchronises hip_stream, then returns MOE_ERR_NONFINITE if a kernel run with
 * check_finite = 1 on the current device saw a NaN/Inf since the last call
 * (and clears the record), MOE_ERR_HIP on a pending HIP error, else MOE_OK. */
moe_status moe_check_finite(void* hip_stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
