// Dispatch: per-expert histogram, stable slots, capacity mask, expert-major
// row gather. "Switch Transformer" explainer, "Implementation" steps 3-5: an
// assignment's slot is the number of earlier assignments (token order) to the
// same expert, it is kept if the slot is below the capacity, and kept tokens
// are packed into expert-major slots. Here the padded [E,C,D] buffer of the
// page becomes a compact [rows, D] buffer with per-expert offsets.
//
// Three launches, all integer work deterministic by construction:
//   1. count: block b (64 tokens) histograms its assignments in LDS and writes
//      its column hist[e][b] (expert-major, so step 2 reads contiguously).
//   2. scan: block e turns hist[e][*] into exclusive per-block bases and writes
//      counts[e].
//   3. place: block b recomputes offsets (exclusive scan over experts of
//      min(count, C)), ranks its assignments in token order with wave ballots,
//      writes pos / accepted / row_token, then copies each token row once
//      into every accepted destination row with 16-byte vectors (the first
//      batch of row loads is issued at the block's start, before the ranking).
#include <mutex>

#include "common.h"

namespace moe {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kTok = 64;       // tokens per block (count / place)
constexpr int kThreads = 256;
constexpr int kScanThreads = 256;

__global__ __launch_bounds__(kThreads) void dispatch_count(const int32_t* __restrict__ ids, int T,
                                                           int k, int E, int nblk,
                                                           int32_t* __restrict__ hist) {
  extern __shared__ int sh[];
  for (int e = threadIdx.x; e < E; e += kThreads) sh[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kTok;
  const int n = min(kTok, T - t0) * k;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int e = ids[static_cast<int64_t>(t0) * k + i];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&sh[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads)
    hist[static_cast<int64_t>(e) * nblk + blockIdx.x] = sh[e];
}

__global__ __launch_bounds__(kScanThreads) void dispatch_scan(int32_t* __restrict__ hist, int nblk,
                                                              int32_t* __restrict__ counts) {
  __shared__ int wt[kScanThreads / 64];
  const int e = blockIdx.x;
  int32_t* col = hist + static_cast<int64_t>(e) * nblk;
  // each thread owns a contiguous run of blocks
  const int per = (nblk + kScanThreads - 1) / kScanThreads;
  const int b0 = threadIdx.x * per, b1 = min(nblk, b0 + per);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += col[b];
  int excl;
  const int total = block_exclusive_scan<kScanThreads>(s, &excl, wt);
  for (int b = b0; b < b1; ++b) {
    const int v = col[b];
    col[b] = excl;
    excl += v;
  }
  if (threadIdx.x == 0) counts[e] = total;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dispatch_place(
    const T* __restrict__ X, const int32_t* __restrict__ ids, const int32_t* __restrict__ hist,
    const int32_t* __restrict__ counts, int Tn, int D, int k, int E, int C, int nblk,
    int32_t* __restrict__ pos, uint8_t* __restrict__ accepted, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, T* __restrict__ Xd) {
  extern __shared__ int sh[];
  int* sOff = sh;              // E + 1
  int* sBase = sh + E + 1;     // E
  int* sRow = sBase + E;       // kTok * MOE_MAX_K destination rows (-1: none)
  __shared__ int wt[kThreads / 64];

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int t0 = b * kTok;
  const int ntok = min(kTok, Tn - t0);

  // The row copy's first batch of token-row loads is issued before anything else, so its
  // latency overlaps the offsets scan and the ranking below (rows are read once: streamed
  // with the non-temporal hint).
  constexpr int V = Elem<T>::kVec;
  constexpr int kU = 4;  // 16-byte vectors in flight per thread (8 is no faster)
  const bool vec_copy = Xd != nullptr && (D % V) == 0;
  const int nv = D / V;  // 16-byte vectors per row (vector path)
  const int items = ntok * nv;
  u32x4 v[kU];
  auto load_batch = [&](int it0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int it = min(it0 + u * kThreads, items - 1);
      const int tl = it / nv, c = it - tl * nv;
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + static_cast<int64_t>(t0 + tl) * D) + c);
    }
  };
  if (vec_copy) load_batch(tid);

  // offsets = exclusive scan over experts of min(counts, C)
  {
    const int per = (E + kThreads - 1) / kThreads;
    const int e0 = tid * per, e1 = min(E, e0 + per);
    int s = 0;
    for (int e = e0; e < e1; ++e) s += min(counts[e], C);
    int excl;
    const int total = block_exclusive_scan<kThreads>(s, &excl, wt);
    for (int e = e0; e < e1; ++e) {
      sOff[e] = excl;
      excl += min(counts[e], C);
    }
    if (tid == 0) sOff[E] = total;
  }
  for (int e = tid; e < E; e += kThreads) sBase[e] = hist[static_cast<int64_t>(e) * nblk + b];
  __syncthreads();
  if (b == 0)
    for (int e = tid; e <= E; e += kThreads) offsets[e] = sOff[e];

  // rank in token-major order: wave 0 walks the block's assignments 64 at a time
  const int n = ntok * k;
  if (tid < 64) {
    const int lane = tid;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int g = 0; g < n; g += 64) {
      const int i = g + lane;
      int e = -1;
      if (i < n) {
        e = ids[static_cast<int64_t>(t0) * k + i];
        if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) e = -1;
      }
      // lanes with the same expert: match on validity and every id bit
      uint64_t peers = __ballot(e >= 0);
      if (e < 0) peers = ~peers;
      for (int bit = 0; bit < nbits; ++bit) {
        const uint64_t m = __ballot(e >= 0 && ((e >> bit) & 1));
        peers &= ((e >= 0) && ((e >> bit) & 1)) ? m : ~m;
      }
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const int rank = __popcll(peers & lt);
      int p = -1, row = -1;
      if (e >= 0) {
        p = sBase[e] + rank;
        if (p < C) row = sOff[e] + p;
      }
      // the last lane of each peer group advances that expert's running base
      const bool last = (peers >> lane) == 1ull;
      if (e >= 0 && last) sBase[e] += __popcll(peers);
      if (i < n) {
        const int64_t gi = static_cast<int64_t>(t0) * k + i;
        pos[gi] = p;
        accepted[gi] = row >= 0 ? 1 : 0;
        sRow[i] = row;
        if (row >= 0) row_token[row] = t0 + i / k;
      }
    }
  }
  __syncthreads();

  // gather: each token row is read once and written to its accepted rows (none without Xd);
  // plain stores (the non-temporal hint on these scattered row writes made the copy slower)
  if (Xd == nullptr) return;
  if (vec_copy) {
    for (int it0 = tid; it0 < items; it0 += kThreads * kU) {
      if (it0 != tid) load_batch(it0);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int it = it0 + u * kThreads;
        if (it >= items) break;
        const int tl = it / nv, c = it - tl * nv;
        for (int j = 0; j < k; ++j) {
          const int row = sRow[tl * k + j];
          if (row >= 0)
            reinterpret_cast<u32x4*>(Xd + static_cast<int64_t>(row) * D)[c] = v[u];
        }
      }
    }
  } else {
    const int nsc = ntok * D;
    for (int it = tid; it < nsc; it += kThreads) {
      const int tl = it / D, c = it - tl * D;
      const T xv = X[static_cast<int64_t>(t0 + tl) * D + c];
      for (int j = 0; j < k; ++j) {
        const int row = sRow[tl * k + j];
        if (row >= 0) Xd[static_cast<int64_t>(row) * D + c] = xv;
      }
    }
  }
}

// Scratch of the allocation-free dispatch: the per-block histogram columns live in this
// fixed array (every word is written by dispatch_count before it is read, so nothing needs
// clearing between calls). Host code never passes the array's name to a kernel: in host code
// that name is a stand-in, not the device address. It uses the address hipGetSymbolAddress
// returns for the current device (each device holds its own copy).
__device__ __align__(256) int32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

}  // namespace

static int dispatch_blocks(const Dims& d) { return ceil_div(d.T, kTok); }

size_t dispatch_workspace(const Dims& d) {
  return align256(static_cast<size_t>(d.E) * dispatch_blocks(d) * sizeof(int32_t));
}

// The device address of `scratch` on the current device, looked up once per device.
static void* noalloc_scratch() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = ptr;
  }
  return ptrs[dev];
}

moe_status dispatch_noalloc_launch(const Dims& d, const void* X, const int32_t* ids, int32_t* pos,
                                   uint8_t* accepted, int32_t* counts, int32_t* offsets,
                                   int32_t* row_token, void* Xd, hipStream_t stream) {
  if (dispatch_workspace(d) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = noalloc_scratch();
  if (!ws) return MOE_ERR_HIP;
  return dispatch_launch(d, X, ids, pos, accepted, counts, offsets, row_token, Xd, ws, stream);
}

moe_status dispatch_launch(const Dims& d, const void* X, const int32_t* ids, int32_t* pos,
                           uint8_t* accepted, int32_t* counts, int32_t* offsets,
                           int32_t* row_token, void* Xd, void* ws, hipStream_t stream) {
  const int nblk = dispatch_blocks(d);
  int32_t* hist = static_cast<int32_t*>(ws);
  dispatch_count<<<nblk, kThreads, d.E * sizeof(int), stream>>>(ids, d.T, d.k, d.E, nblk, hist);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  dispatch_scan<<<d.E, kScanThreads, 0, stream>>>(hist, nblk, counts);
  if (launch_status() != MOE_OK) return MOE_ERR_HIP;
  const size_t lds = (2 * static_cast<size_t>(d.E) + 1 + kTok * MOE_MAX_K) * sizeof(int);
  if (d.dtype == MOE_BF16)
    dispatch_place<uint16_t><<<nblk, kThreads, lds, stream>>>(
        static_cast<const uint16_t*>(X), ids, hist, counts, d.T, d.D, d.k, d.E, d.C, nblk, pos,
        accepted, offsets, row_token, static_cast<uint16_t*>(Xd));
  else
    dispatch_place<float><<<nblk, kThreads, lds, stream>>>(
        static_cast<const float*>(X), ids, hist, counts, d.T, d.D, d.k, d.E, d.C, nblk, pos,
        accepted, offsets, row_token, static_cast<float*>(Xd));
  return launch_status();
}

}  // namespace moe
