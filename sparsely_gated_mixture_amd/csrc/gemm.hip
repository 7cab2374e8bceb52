// Expert FFN as grouped GEMMs on MFMA.
//
// "Switch Transformer" explainer, "Implementation" step 6: every expert e has
// its own W1_e [D,H] and W2_e [H,D]; hidden = ReLU(U_e W1_e), out = hidden W2_e,
// no biases. The "Sparsely-Gated MoE" knowledge-base page (section 3) names the
// production form: one grouped GEMM instead of a loop over experts. Here the
// groups are the expert-major row ranges offsets[e] .. offsets[e+1] written by
// the dispatch; the kernel reads them on the device, so no host sync.
//
// Design (gfx950):
//   * Weights are packed once (moe_pack_expert_weights) into MFMA fragment
//     order: for expert e, 32-column block nb and k-step ks, the 64 lanes'
//     16-byte B operands are contiguous. A wave then streams its B operand
//     straight from memory with one coalesced 1 KB load per fragment; B never
//     touches LDS.
//   * A block computes a BM x 256 tile; its 4 waves split the 256 columns
//     (64 each) and all read the same A rows, which are staged through LDS
//     (128-byte-wide k stages, double buffered, rows padded against bank
//     conflicts).
//   * Tiles are ordered expert-major, then column tile, then row tile, so the
//     row tiles of one expert that share a weight slice run back to back; the
//     block index is remapped so that each XCD (blocks are dealt round-robin
//     over the 8 XCDs) works through a contiguous run of that order and keeps
//     the expert's weights and rows in its own L2.
//   * Every block derives the tile table itself from offsets (one block-wide
//     scan of per-expert row-tile counts); blocks past the real tile count
//     exit at once (the grid is sized by the upper bound on rows).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 256;
constexpr int kAStride = 144;  // 128 data bytes + 16 pad per LDS row
constexpr int kXcds = 8;

struct GemmArgs {
  const void* A;
  const uint4* Wp;
  const int32_t* offsets;
  void* C;
  int* nonfinite;
  int E, K, N;
  int NB;  // 32-column blocks per expert in Wp
  int KS;  // k-steps per column block in Wp (multiple of 4)
};

__device__ __forceinline__ int block_exclusive_scan(int v, int* excl, int* wt) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wt[w] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    if (i < w) before += wt[i];
    total += wt[i];
  }
  *excl = before + x - v;
  __syncthreads();
  return total;
}

template <typename T, int BM, bool kRelu>
__global__ __launch_bounds__(kThreads) void grouped_gemm(GemmArgs g) {
  constexpr int V = Elem<T>::kVec;
  constexpr int kStageElems = 128 / static_cast<int>(sizeof(T));
  constexpr int MB = BM / 32;               // 32-row blocks per tile
  constexpr int kChunks = BM * 8 / kThreads;  // 16-byte A chunks per thread per stage

  extern __shared__ int sCum[];  // E + 1 running row-tile counts
  __shared__ int wt[kThreads / 64];
  __shared__ __align__(16) unsigned char sA[2][BM * kAStride];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = g.E;
  const int32_t* off = g.offsets;

  // ---- tile table
  {
    const int per = (E + kThreads - 1) / kThreads;
    const int e0 = tid * per, e1 = min(E, e0 + per);
    int s = 0;
    for (int e = e0; e < e1; ++e) s += (off[e + 1] - off[e] + BM - 1) / BM;
    int excl;
    const int total = block_exclusive_scan(s, &excl, wt);
    for (int e = e0; e < e1; ++e) {
      sCum[e] = excl;
      excl += (off[e + 1] - off[e] + BM - 1) / BM;
    }
    if (tid == 0) sCum[E] = total;
  }
  __syncthreads();
  const int NT = (g.N + kBN - 1) / kBN;
  const int total_tiles = sCum[E] * NT;
  const int per_xcd = (total_tiles + kXcds - 1) / kXcds;
  const int local = blockIdx.x / kXcds;
  if (local >= per_xcd) return;
  const int logical = (blockIdx.x % kXcds) * per_xcd + local;
  if (logical >= total_tiles) return;
  const int q = logical / NT;
  int lo = 0, hi = E;  // first j with sCum[j] > q
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sCum[mid] > q) hi = mid; else lo = mid + 1;
  }
  const int e = lo - 1;
  const int mt = sCum[e + 1] - sCum[e];
  const int loc = logical - sCum[e] * NT;
  const int n_tile = loc / mt, m_tile = loc - n_tile * mt;
  const int r0 = off[e] + m_tile * BM;
  const int rows = min(BM, off[e + 1] - r0);
  const int n0 = n_tile * kBN;

  const T* A = static_cast<const T*>(g.A);
  const int K = g.K;
  const bool vec_ok = (K % V) == 0;
  const int nst = g.KS / 4;

  // ---- operand streams
  auto load_a = [&](int st, uint4 regs[kChunks]) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 3, seg = c & 7;
      const int rr = r0 + min(r, rows - 1);
      regs[i] = load_row16<T>(A + static_cast<int64_t>(rr) * K, st * kStageElems + seg * V, K, vec_ok);
    }
  };
  auto store_a = [&](int buf, const uint4 regs[kChunks]) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 3, seg = c & 7;
      *reinterpret_cast<uint4*>(&sA[buf][r * kAStride + seg * 16]) = regs[i];
    }
  };
  const int nb0 = n0 / 32 + wave * 2;
  const bool has_b[2] = {nb0 < g.NB, nb0 + 1 < g.NB};
  const uint4* Wb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    Wb[j] = g.Wp + (static_cast<int64_t>(e) * g.NB + (has_b[j] ? nb0 + j : 0)) * g.KS * kWave + lane;
  auto load_b = [&](int st, uint4 b[4][2]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[ks][j] = has_b[j] ? Wb[j][static_cast<int64_t>(st * 4 + ks) * kWave] : make_uint4(0, 0, 0, 0);
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][j][i] = 0.f;

  uint4 areg[kChunks];
  uint4 bcur[4][2], bnxt[4][2];
  load_a(0, areg);
  load_b(0, bcur);
  store_a(0, areg);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nst;
    if (more) {
      load_a(st + 1, areg);
      load_b(st + 1, bnxt);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const uint4 af = *reinterpret_cast<const uint4*>(
            &sA[buf][(m * 32 + (lane & 31)) * kAStride + ks * 32 + (lane >> 5) * 16]);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[m][j] = mfma_step<T>(af, bcur[ks][j], acc[m][j]);
      }
    }
    if (more) {
      store_a(buf ^ 1, areg);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) bcur[ks][j] = bnxt[ks][j];
    }
    __syncthreads();
  }

  // ---- epilogue: (ReLU), round to T, predicated stores
  T* C = static_cast<T*>(g.C);
  const bool check = g.nonfinite != nullptr;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wave * 64 + j * 32 + (lane & 31);
    if (col >= g.N) continue;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = m * 32 + acc_row(lane, i);
        if (row < rows) {
          float v = acc[m][j][i];
          if (kRelu) v = fmaxf(v, 0.f);
          bad |= !isfinite(v);
          C[static_cast<int64_t>(r0 + row) * g.N + col] = Elem<T>::from_f32(v);
        }
      }
  }
  if (check) note_nonfinite(g.nonfinite, bad);
}

// One thread per (expert, column block, k-step, lane): lane's 16-byte B operand.
// Column n = nb*32 + lane%32, k = ks*2V + (lane/32)*V + i; zero padded.
template <typename T>
__global__ void pack_weights(const T* __restrict__ W, int E, int K, int N, int NB, int KS,
                             uint4* __restrict__ out) {
  constexpr int V = Elem<T>::kVec;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(E) * NB * KS * kWave;
  if (idx >= total) return;
  const int lane = static_cast<int>(idx % kWave);
  int64_t rest = idx / kWave;
  const int ks = static_cast<int>(rest % KS);
  rest /= KS;
  const int nb = static_cast<int>(rest % NB);
  const int e = static_cast<int>(rest / NB);
  const int n = nb * 32 + (lane & 31);
  const int k0 = ks * 2 * V + (lane >> 5) * V;
  T v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int k = k0 + i;
    v[i] = (n < N && k < K) ? W[(static_cast<int64_t>(e) * K + k) * N + n] : T(0);
  }
  out[idx] = *reinterpret_cast<const uint4*>(v);
}

constexpr int kBM = 128;

}  // namespace

// ------------------------------------------------------------------ host side
static void layer_dims(const Dims& d, int layer, int* K, int* N) {
  *K = layer == 1 ? d.D : d.H;
  *N = layer == 1 ? d.H : d.D;
}
static int gemm_ks(const Dims& d, int K) {
  const int stage = d.dtype == MOE_BF16 ? 64 : 32;
  return ceil_div(K, stage) * 4;
}

size_t packed_weight_bytes(const Dims& d, int layer) {
  int K, N;
  layer_dims(d, layer, &K, &N);
  return static_cast<size_t>(d.E) * ceil_div(N, 32) * static_cast<size_t>(gemm_ks(d, K)) * kWave * 16;
}

moe_status pack_launch(const Dims& d, int layer, const void* W, void* Wp, hipStream_t stream) {
  int K, N;
  layer_dims(d, layer, &K, &N);
  const int NB = ceil_div(N, 32), KS = gemm_ks(d, K);
  const int64_t total = static_cast<int64_t>(d.E) * NB * KS * kWave;
  const int grid = static_cast<int>(ceil_div64(total, 256));
  if (d.dtype == MOE_BF16)
    pack_weights<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(W), d.E, K, N, NB, KS,
                                                     static_cast<uint4*>(Wp));
  else
    pack_weights<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(W), d.E, K, N, NB, KS,
                                                  static_cast<uint4*>(Wp));
  return launch_status();
}

moe_status gemm_launch(const Dims& d, int layer, const void* A, const void* Wp, const int32_t* offsets,
                       void* C, int* nonfinite, hipStream_t stream) {
  int K, N;
  layer_dims(d, layer, &K, &N);
  GemmArgs g;
  g.A = A;
  g.Wp = static_cast<const uint4*>(Wp);
  g.offsets = offsets;
  g.C = C;
  g.nonfinite = nonfinite;
  g.E = d.E;
  g.K = K;
  g.N = N;
  g.NB = ceil_div(N, 32);
  g.KS = gemm_ks(d, K);
  // upper bound on row tiles: per expert at most ceil(min(C,T)/BM); overall at
  // most (rows + E*(BM-1))/BM
  const int64_t cap = std::min<int64_t>(d.C, d.T);
  const int64_t by_expert = static_cast<int64_t>(d.E) * ceil_div64(cap, kBM);
  const int64_t by_rows = (d.max_rows + static_cast<int64_t>(d.E) * (kBM - 1)) / kBM;
  const int64_t mtiles = std::min(by_expert, by_rows);
  const int64_t tiles = mtiles * ceil_div(N, kBN);
  const int64_t grid = ceil_div64(std::max<int64_t>(tiles, 1), kXcds) * kXcds;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  const size_t lds = (static_cast<size_t>(d.E) + 1) * sizeof(int);
  if (d.dtype == MOE_BF16) {
    if (layer == 1)
      grouped_gemm<uint16_t, kBM, true><<<static_cast<int>(grid), kThreads, lds, stream>>>(g);
    else
      grouped_gemm<uint16_t, kBM, false><<<static_cast<int>(grid), kThreads, lds, stream>>>(g);
  } else {
    if (layer == 1)
      grouped_gemm<float, kBM, true><<<static_cast<int>(grid), kThreads, lds, stream>>>(g);
    else
      grouped_gemm<float, kBM, false><<<static_cast<int>(grid), kThreads, lds, stream>>>(g);
  }
  return launch_status();
}

}  // namespace moe
