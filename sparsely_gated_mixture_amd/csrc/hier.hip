// Hierarchical (two-level) MoE: gates and balancing terms.
//
// "Outrageously Large Neural Networks" summary, section 3.4, "Hierarchical
// Mixture-of-Experts": a groups of b experts; a primary noisy top-k gate picks
// k_p groups, and group i's own noisy top-k gate picks k_s of its b experts for
// the tokens routed to it (X^(i)); the expert (i, j) output is weighted by
// Gp(x)_i * G_i(x)_j. Importance_H(i,j) sums those products over the batch;
// Load_H(i,j) = Load_p(X)_i * Load_i(X^(i))_j / |X^(i)| (the lesson page,
// chapter 5, "Balancing at every level"). A group no token reaches gets
// Load_H = 0 (0/0 read as 0).
//
// Routing reuses the flat stages:
//   1. the flat router over the a groups (k_p kept, noise key (seed, 0));
//   2. the flat dispatch of the primary choices with no capacity and no copy:
//      group i owns rows offsets_p[i] .. offsets_p[i+1]-1 in token order;
//   3. the router GEMM in grouped mode over those rows: each row block gathers
//      its tokens' X rows, multiplies by its group's packed weights, and draws
//      noise from key (seed, 1 + i); then the flat top-k selection per row;
//   4. hier_compose: expert i*b + j with gate Gp * G_i, primary slot first.
// Balancing: the flat aux over the primary level gives Load_p, Importance_p and
// their CV^2; hier_group_partial sums, per group and 64-row chunk, the product
// gates and the secondary P(x, j) over the group's rows; hier_group_reduce adds
// a group's chunks in order (fp64) and forms Load_H; hier_final takes CV^2.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;  // secondary rows per partial block

__device__ __forceinline__ float phi(float z) { return 0.5f * erfcf(-z * 0.70710678118654752f); }

// One thread per (token, primary slot): final ids and product gates.
__global__ void hier_compose(const int32_t* __restrict__ ids_p, const float* __restrict__ gates_p,
                             const int32_t* __restrict__ pos_p, const int32_t* __restrict__ offsets_p,
                             const int32_t* __restrict__ ids_s, const float* __restrict__ gates_s,
                             int T, int kp, int ks, int b, int32_t* __restrict__ ids,
                             float* __restrict__ gates) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * kp) return;
  const int64_t t = i / kp;
  const int s = static_cast<int>(i - t * kp);
  const int grp = ids_p[i];
  const int64_t r = static_cast<int64_t>(offsets_p[grp]) + pos_p[i];
  const float gp = gates_p[i];
  const int64_t o = t * kp * ks + static_cast<int64_t>(s) * ks;
  for (int j = 0; j < ks; ++j) {
    ids[o + j] = grp * b + ids_s[r * ks + j];
    gates[o + j] = gp * gates_s[r * ks + j];
  }
}

struct HierAuxArgs {
  const int32_t* ids_p;
  const float* gates_p;
  const int32_t* counts_p;
  const int32_t* offsets_p;
  const int32_t* row_token_p;
  const float* clean_s;
  const float* std_s;
  const float* row_stats_s;
  const int32_t* ids_s;
  const float* gates_s;
  const float* load_p;    // [a] from the flat aux of the primary level
  const float* out_p;     // [8] from the flat aux of the primary level
  float* partial;         // [2][nblk][b]: product gates, secondary P
  double* sums;           // [2][E]: Importance_H, Load_H
  float* importance;
  float* load;
  float* out;
  int T, a, b, kp, ks, nblk, use_noise;
};

// Chunk tiles of the groups: block q covers rows of group g, chunk q - cum[g].
__device__ int group_chunk(const int32_t* counts, int a, int q, int* cum, int* wt, int* g_out) {
  const int tid = threadIdx.x;
  const int per = (a + kThreads - 1) / kThreads;
  const int g0 = tid * per, g1 = min(a, g0 + per);
  int s = 0;
  for (int g = g0; g < g1; ++g) s += (counts[g] + kChunk - 1) / kChunk;
  int excl;
  const int total = block_exclusive_scan<kThreads>(s, &excl, wt);
  for (int g = g0; g < g1; ++g) {
    cum[g] = excl;
    excl += (counts[g] + kChunk - 1) / kChunk;
  }
  if (tid == 0) cum[a] = total;
  __syncthreads();
  if (q >= cum[a]) return -1;
  int lo = 0, hi = a;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] > q) hi = mid; else lo = mid + 1;
  }
  *g_out = lo - 1;
  return q - cum[lo - 1];
}

__global__ __launch_bounds__(kThreads) void hier_group_partial(HierAuxArgs a) {
  extern __shared__ int cum[];  // a + 1
  __shared__ int wt[kThreads / 64];
  __shared__ float sGp[kChunk], sR0[kChunk], sR1[kChunk];
  __shared__ int sId[kChunk * MOE_MAX_K];
  __shared__ float sG[kChunk * MOE_MAX_K];
  __shared__ float sRedI[kThreads], sRedL[kThreads];
  int g = 0;
  const int c = group_chunk(a.counts_p, a.a, blockIdx.x, cum, wt, &g);
  if (c < 0) return;  // uniform: past the real chunk count
  const int tid = threadIdx.x;
  const int r0 = a.offsets_p[g] + c * kChunk;
  const int nr = min(kChunk, a.offsets_p[g + 1] - r0);
  const int b = a.b, ks = a.ks, kp = a.kp;
  for (int i = tid; i < nr * ks; i += kThreads) {
    sId[i] = a.ids_s[static_cast<int64_t>(r0) * ks + i];
    sG[i] = a.gates_s[static_cast<int64_t>(r0) * ks + i];
  }
  for (int r = tid; r < nr; r += kThreads) {
    // the primary gate of this row's group for its token
    const int64_t t = a.row_token_p[r0 + r];
    float gp = 0.f;
    for (int s = 0; s < kp; ++s)
      if (a.ids_p[t * kp + s] == g) gp = a.gates_p[t * kp + s];
    sGp[r] = gp;
    if (a.use_noise) {
      sR0[r] = a.row_stats_s[2 * static_cast<int64_t>(r0 + r)];
      sR1[r] = a.row_stats_s[2 * static_cast<int64_t>(r0 + r) + 1];
    }
  }
  __syncthreads();
  // threads = P row slices x be experts (be = min(b, kThreads)); slice s takes rows s, s+P, ..
  const int be = min(b, kThreads);
  const int P = kThreads / be;
  const int slice = tid / be, el = tid - slice * be;
  const int64_t plane = static_cast<int64_t>(a.nblk) * b;
  for (int e0 = 0; e0 < b; e0 += be) {
    const int e = e0 + el;
    float imp = 0.f, load = 0.f;
    if (slice < P && e < b) {
      for (int r = slice; r < nr; r += P) {
        bool inside = false;
        for (int j = 0; j < ks; ++j)
          if (sId[r * ks + j] == e) {
            inside = true;
            imp += sGp[r] * sG[r * ks + j];
          }
        if (a.use_noise) {
          const int64_t ix = static_cast<int64_t>(r0 + r) * b + e;
          const float diff = a.clean_s[ix] - (inside ? sR1[r] : sR0[r]);
          const float sd = a.std_s[ix];
          load += sd > 0.f ? phi(diff / sd) : (diff > 0.f ? 1.f : (diff == 0.f ? 0.5f : 0.f));
        }
      }
    }
    // slices added in fixed order
    sRedI[tid] = imp;
    sRedL[tid] = load;
    __syncthreads();
    if (slice == 0 && e < b) {
      for (int q = 1; q < P; ++q) {
        imp += sRedI[q * be + el];
        load += sRedL[q * be + el];
      }
      const int64_t o = static_cast<int64_t>(blockIdx.x) * b + e;
      a.partial[o] = imp;
      a.partial[plane + o] = load;
    }
    __syncthreads();
  }
}

// One thread per expert (i, j): the group's chunks in order, fp64.
__global__ __launch_bounds__(kThreads) void hier_group_reduce(HierAuxArgs a) {
  extern __shared__ int cum[];  // a + 1
  __shared__ int wt[kThreads / 64];
  int dummy;
  group_chunk(a.counts_p, a.a, 0, cum, wt, &dummy);
  const int E = a.a * a.b;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= E) return;
  const int g = e / a.b, j = e - g * a.b;
  const int64_t plane = static_cast<int64_t>(a.nblk) * a.b;
  double imp = 0.0, ls = 0.0;
  for (int q = cum[g]; q < cum[g + 1]; ++q) {
    imp += a.partial[static_cast<int64_t>(q) * a.b + j];
    ls += a.partial[plane + static_cast<int64_t>(q) * a.b + j];
  }
  const int n = a.counts_p[g];
  const double load = n > 0 ? static_cast<double>(a.load_p[g]) * ls / n : 0.0;
  a.sums[e] = imp;
  a.sums[E + e] = load;
  if (a.importance) a.importance[e] = static_cast<float>(imp);
  if (a.load) a.load[e] = static_cast<float>(load);
}

__device__ double hblock_sum(double v, double* sh) {
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
__device__ double hblock_max(double v, double* sh) {
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

__global__ __launch_bounds__(kThreads) void hier_final(HierAuxArgs a) {
  __shared__ double sh[kThreads];
  const int E = a.a * a.b;
  const double* imp = a.sums;
  const double* load = a.sums + E;
  double si = 0, sl = 0, mx = -INFINITY, empty = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    si += imp[e];
    sl += load[e];
    mx = fmax(mx, load[e]);
  }
  for (int g = threadIdx.x; g < a.a; g += kThreads) empty += a.counts_p[g] == 0 ? 1.0 : 0.0;
  si = hblock_sum(si, sh);
  sl = hblock_sum(sl, sh);
  mx = hblock_max(mx, sh);
  empty = hblock_sum(empty, sh);
  const double mi = si / E, ml = sl / E;
  double vi = 0, vl = 0;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    vi += (imp[e] - mi) * (imp[e] - mi);
    vl += (load[e] - ml) * (load[e] - ml);
  }
  vi = hblock_sum(vi, sh) / E;
  vl = hblock_sum(vl, sh) / E;
  if (threadIdx.x == 0) {
    a.out[0] = static_cast<float>(mi != 0 ? vi / (mi * mi) : 0.0);
    a.out[1] = static_cast<float>(ml != 0 ? vl / (ml * ml) : 0.0);
    a.out[2] = a.out_p[0];
    a.out[3] = a.out_p[1];
    a.out[4] = static_cast<float>(ml > 0 ? mx / ml : 0.0);
    a.out[5] = static_cast<float>(empty);
    a.out[6] = static_cast<float>(si);
    a.out[7] = 0.f;
  }
}

}  // namespace

// ------------------------------------------------------------------ host side
void hier_dims(const Dims& d, const moe_hier* h, Dims* dp, Dims* ds) {
  const int a = h->groups, kp = h->k_primary;
  *dp = d;
  dp->E = a;
  dp->k = kp;
  dp->C = d.T;  // no capacity between the levels
  dp->max_rows = static_cast<int64_t>(d.T) * kp;
  *ds = d;
  ds->T = d.T * kp;
  ds->E = d.E / a;
  ds->k = d.k / kp;
  ds->C = ds->T;
  ds->max_rows = ds->T;
}

size_t hier_route_workspace(const Dims& d, const moe_hier* h) {
  Dims dp, ds;
  hier_dims(d, h, &dp, &ds);
  return std::max({route_workspace(dp), dispatch_workspace(dp), route_groups_workspace(ds, h->groups)});
}

static int hier_aux_blocks(const Dims& ds, int a) {
  return static_cast<int>((ds.T + static_cast<int64_t>(a) * (kChunk - 1)) / kChunk);
}

size_t hier_aux_workspace(const Dims& d, const moe_hier* h) {
  Dims dp, ds;
  hier_dims(d, h, &dp, &ds);
  const int nblk = hier_aux_blocks(ds, h->groups);
  return align256(aux_workspace(dp)) + align256((2 * static_cast<size_t>(h->groups) + 8) * sizeof(float)) +
         align256(2 * static_cast<size_t>(nblk) * ds.E * sizeof(float)) +
         align256(2 * static_cast<size_t>(d.E) * sizeof(double));
}

moe_status hier_route_launch(const Dims& d, const moe_hier* h, const moe_problem* p, const void* X,
                             const float* Wpg, const float* Wpn, const float* Wsg, const float* Wsn,
                             int32_t* ids, float* gates, const moe_hier_state* st, void* ws,
                             int* nonfinite, hipStream_t stream) {
  Dims dp, ds;
  hier_dims(d, h, &dp, &ds);
  const bool noise = d.noise != 0;
  moe_status s = route_launch(dp, p, X, Wpg, noise ? Wpn : nullptr, nullptr, nullptr, st->ids_p,
                              st->gates_p, st->clean_p, noise ? st->std_p : nullptr,
                              st->row_stats_p, ws, nonfinite, stream);
  if (s != MOE_OK) return s;
  s = dispatch_launch(dp, X, st->ids_p, st->pos_p, st->accepted_p, st->counts_p, st->offsets_p,
                      st->row_token_p, nullptr, ws, stream);
  if (s != MOE_OK) return s;
  s = route_groups_launch(ds, h->groups, p->seed, X, st->offsets_p, st->row_token_p, Wsg,
                          noise ? Wsn : nullptr, st->ids_s, st->gates_s, st->clean_s,
                          noise ? st->std_s : nullptr, st->row_stats_s, ws, nonfinite, stream);
  if (s != MOE_OK) return s;
  const int64_t n = static_cast<int64_t>(d.T) * dp.k;
  hier_compose<<<static_cast<int>(ceil_div64(n, 256)), 256, 0, stream>>>(
      st->ids_p, st->gates_p, st->pos_p, st->offsets_p, st->ids_s, st->gates_s, d.T, dp.k, ds.k,
      ds.E, ids, gates);
  return launch_status();
}

moe_status hier_aux_launch(const Dims& d, const moe_hier* h, const moe_hier_state* st,
                           float* importance, float* load, float* out, void* ws, hipStream_t stream) {
  Dims dp, ds;
  hier_dims(d, h, &dp, &ds);
  const bool noise = d.noise != 0;
  char* base = static_cast<char*>(ws);
  void* ws_p = base;
  float* prim = reinterpret_cast<float*>(base + align256(aux_workspace(dp)));  // imp_p, load_p, out_p
  const int a = h->groups;
  const int nblk = hier_aux_blocks(ds, a);
  float* partial = reinterpret_cast<float*>(reinterpret_cast<char*>(prim) +
                                            align256((2 * static_cast<size_t>(a) + 8) * sizeof(float)));
  double* sums = reinterpret_cast<double*>(reinterpret_cast<char*>(partial) +
                                           align256(2 * static_cast<size_t>(nblk) * ds.E * sizeof(float)));
  moe_status s = aux_launch(dp, st->ids_p, st->gates_p, st->clean_p, noise ? st->std_p : nullptr,
                            st->row_stats_p, st->counts_p, prim, prim + a, prim + 2 * a, ws_p, stream);
  if (s != MOE_OK) return s;
  HierAuxArgs ha;
  ha.ids_p = st->ids_p;
  ha.gates_p = st->gates_p;
  ha.counts_p = st->counts_p;
  ha.offsets_p = st->offsets_p;
  ha.row_token_p = st->row_token_p;
  ha.clean_s = st->clean_s;
  ha.std_s = noise ? st->std_s : nullptr;
  ha.row_stats_s = st->row_stats_s;
  ha.ids_s = st->ids_s;
  ha.gates_s = st->gates_s;
  ha.load_p = prim + a;
  ha.out_p = prim + 2 * a;
  ha.partial = partial;
  ha.sums = sums;
  ha.importance = importance;
  ha.load = load;
  ha.out = out;
  ha.T = d.T;
  ha.a = a;
  ha.b = ds.E;
  ha.kp = dp.k;
  ha.ks = ds.k;
  ha.nblk = nblk;
  ha.use_noise = noise ? 1 : 0;
  const size_t lds = (static_cast<size_t>(a) + 1) * sizeof(int);
  hier_group_partial<<<std::max(nblk, 1), kThreads, lds, stream>>>(ha);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  hier_group_reduce<<<ceil_div(d.E, kThreads), kThreads, lds, stream>>>(ha);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  hier_final<<<1, kThreads, 0, stream>>>(ha);
  return launch_status();
}

}  // namespace moe
