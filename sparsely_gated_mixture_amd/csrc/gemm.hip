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
//   * BM is 128 rows, or 64 when 128-row tiles would leave the CUs short of
//     work (small or narrow layers).
//   * The epilogue runs while the block's MFMAs are idle, so it is kept lean:
//     hardware bf16 rounding, ReLU as an integer max on the bit pattern, the
//     non-finite test compiled in only where a flag is given; rows leave as
//     16-byte stores through a wave-private LDS tile.
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
  const void* mask;  // epilogue mode 2: output zeroed where mask[row, col] <= 0 ([rows, N])
  const int32_t* row_token;  // gathered A: row r of the groups is row row_token[r] of A
  int E, K, N;
  int NB;  // 32-column blocks per expert in Wp
  int KS;  // k-steps per column block in Wp (multiple of 4)
};

// ReLU on the bit pattern: a float whose pattern read as a signed integer is negative has its
// sign bit set, so max(bits, 0) maps every negative value and -0 to +0 and keeps the rest (a
// NaN from the accumulation stays NaN, where it can be seen by the non-finite check). One
// integer max instead of the canonicalising float max.
__device__ __forceinline__ float relu(float v) { return __int_as_float(max(__float_as_int(v), 0)); }

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Operands live in native vector registers (the HIP uint4 struct defeats
// register promotion of arrays).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mma<uint16_t>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mma<float>(u32x4 a, u32x4 b, f32x16 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s]), __uint_as_float(b[s]), c, 0, 0, 0);
  return c;
}

// kEpi: 0 plain, 1 ReLU, 2 masked by a second tensor of the output's shape (the ReLU
// derivative in the backward pass: zero where the forward's hidden value is not positive).
// kFullK: K is a multiple of the 128-byte k stage (no tail, no bounds checks on A).
// kVecOut: N * sizeof(T) is a multiple of 16 (row-contiguous 16-byte output stores).
// kCheck: record NaN / Inf outputs in g.nonfinite (only then is the test compiled in).
// kGather: A rows are read through g.row_token (the dispatch's gather done by the A loads).
template <typename T, int BM, int kEpi, bool kFullK, bool kVecOut, bool kCheck, bool kGather>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm(GemmArgs g) {
  constexpr int V = Elem<T>::kVec;
  constexpr int kStageElems = 128 / static_cast<int>(sizeof(T));
  constexpr int MB = BM / 32;                 // 32-row blocks per tile
  constexpr int kChunks = BM * 8 / kThreads;  // 16-byte A chunks per thread per stage
  constexpr int kTStride = 32 + 16 / static_cast<int>(sizeof(T));  // epilogue tile row (elements)

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
    const int total = block_exclusive_scan<kThreads>(s, &excl, wt);
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
  const int nst = g.KS / 4;

  // ---- A stream: thread's chunk i is row arow0 + i*32 (clamped into the group), 16-byte
  // segment aseg of the 128-byte k stage; LDS rows are padded to kAStride bytes.
  const int aseg = tid & 7, arow0 = tid >> 3;
  const T* abase = A + (kGather ? 0 : static_cast<int64_t>(r0) * K);
  const bool vec_ok = (K % V) == 0;
  int atok[kGather ? kChunks : 1];  // gathered: the A row of each chunk
  if constexpr (kGather) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) atok[i] = g.row_token[r0 + min(arow0 + i * (kThreads / 8), rows - 1)];
  }
  u32x4 areg[kChunks];
  auto load_a = [&](int st) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const T* row = abase + static_cast<int64_t>(kGather ? atok[i] : min(arow0 + i * (kThreads / 8), rows - 1)) * K;
      if constexpr (kFullK) {
        areg[i] = *reinterpret_cast<const u32x4*>(row + st * kStageElems + aseg * V);
      } else {
        const uint4 v = load_row16<T>(row, st * kStageElems + aseg * V, K, vec_ok);
        areg[i] = u32x4{v.x, v.y, v.z, v.w};
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      *reinterpret_cast<u32x4*>(&sA[buf][(arow0 + i * (kThreads / 8)) * kAStride + aseg * 16]) = areg[i];
  };

  // ---- B stream: column blocks past N read a valid block (those results are never stored)
  const u32x4* Wb = reinterpret_cast<const u32x4*>(g.Wp);
  const u32x4* W0 = Wb + (static_cast<int64_t>(e) * g.NB + min(n0 / 32 + wave * 2, g.NB - 1)) * g.KS * kWave + lane;
  const u32x4* W1 = Wb + (static_cast<int64_t>(e) * g.NB + min(n0 / 32 + wave * 2 + 1, g.NB - 1)) * g.KS * kWave + lane;

  f32x16 acc[MB][2];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][j][i] = 0.f;

  const int arow = (lane & 31) * kAStride + (lane >> 5) * 16;
  u32x4 bq[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bq[ks][0] = W0[ks * kWave];
    bq[ks][1] = W1[ks * kWave];
  }
  load_a(0);
  store_a(0);
  __syncthreads();

  // ---- main loop: stage st computes from LDS buffer st&1 and B registers, while the next
  // stage's A (registers, then LDS) and B (registers, one k-step at a time) stream in. Every
  // load is unconditional (the last stage re-reads itself) so the wait counts stay exact.
  u32x4 af[2][MB];
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const int stn = min(st + 1, nst - 1);
    load_a(stn);
#pragma unroll
    for (int m = 0; m < MB; ++m)
      af[0][m] = *reinterpret_cast<const u32x4*>(&sA[buf][m * 32 * kAStride + arow]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
          af[(ks + 1) & 1][m] =
              *reinterpret_cast<const u32x4*>(&sA[buf][m * 32 * kAStride + (ks + 1) * 32 + arow]);
      }
      // raised priority while this wave's MFMAs issue: a wave with a k-step's operands
      // ready keeps the matrix unit busy ahead of waves still waiting on loads
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        acc[m][0] = mma<T>(af[ks & 1][m], bq[ks][0], acc[m][0]);
        acc[m][1] = mma<T>(af[ks & 1][m], bq[ks][1], acc[m][1]);
      }
      __builtin_amdgcn_s_setprio(0);
      const int64_t kn = static_cast<int64_t>(stn * 4 + ks) * kWave;
      bq[ks][0] = W0[kn];
      bq[ks][1] = W1[kn];
    }
    store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: (ReLU), round to T, store
  T* C = static_cast<T*>(g.C);
  bool bad = false;
  if constexpr (kVecOut) {
    // each 32x32 tile goes through a wave-private LDS tile so rows leave as 16-byte stores
    T* Ts = reinterpret_cast<T*>(&sA[0][0]) + wave * (32 * kTStride);
    constexpr int kSegs = 32 / V;  // 16-byte segments per tile row
    constexpr int kH = 32 * kSegs / 64;  // 16-byte stores per lane per 32x32 tile
    // mode 2: every mask vector this lane needs is requested before the first store, so the
    // loads overlap each other instead of each waiting in turn
    u32x4 mk[kEpi == 2 ? MB : 1][2][kH];
    if constexpr (kEpi == 2) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int h = 0; h < kH; ++h) {
            const int qd = lane + 64 * h;
            const int grow = m * 32 + qd / kSegs, gcol = n0 + wave * 64 + j * 32 + (qd % kSegs) * V;
            mk[m][j][h] = (grow < rows && gcol < g.N)
                              ? *reinterpret_cast<const u32x4*>(static_cast<const T*>(g.mask) +
                                                                static_cast<int64_t>(r0 + grow) * g.N + gcol)
                              : u32x4{0u, 0u, 0u, 0u};
          }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cbase = n0 + wave * 64 + j * 32;
        if constexpr (sizeof(T) == 2 && !kCheck) {
          // bf16: registers i, i+1 hold rows r, r+1 of the lane's column; one conversion
          // rounds the pair, and the ReLU is a packed 16-bit integer max on the rounded
          // patterns (rounding keeps the sign, so this equals rounding the ReLU)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            s16x2 h = __builtin_bit_cast(
                s16x2, __builtin_convertvector((f32x2){acc[m][j][i], acc[m][j][i + 1]}, bf16x2));
            if (kEpi == 1) h = __builtin_elementwise_max(h, (s16x2){0, 0});
            Ts[acc_row(lane, i) * kTStride + (lane & 31)] = static_cast<uint16_t>(h.x);
            Ts[(acc_row(lane, i) + 1) * kTStride + (lane & 31)] = static_cast<uint16_t>(h.y);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float v = acc[m][j][i];
            if (kEpi == 1) v = relu(v);
            // rows and columns past the tile's edge hold copies of real ones (clamped loads)
            if (kCheck && kEpi != 2) bad |= !isfinite(v);
            Ts[acc_row(lane, i) * kTStride + (lane & 31)] = Elem<T>::from_f32(v);
          }
        }
#pragma unroll
        for (int h = 0; h < kH; ++h) {
          const int qd = lane + 64 * h;
          const int row = qd / kSegs, seg = qd % kSegs;
          u32x4 v = *reinterpret_cast<const u32x4*>(&Ts[row * kTStride + seg * V]);
          const int grow = m * 32 + row, gcol = cbase + seg * V;
          if (grow < rows && gcol < g.N) {
            const int64_t o = static_cast<int64_t>(r0 + grow) * g.N + gcol;
            if constexpr (kEpi == 2) {  // the mask's 16 bytes at the same place: zero where <= 0
              T* ve = reinterpret_cast<T*>(&v);
              const T* me = reinterpret_cast<const T*>(&mk[m][j][h]);
#pragma unroll
              for (int q = 0; q < V; ++q) {
                if (!(Elem<T>::to_f32(me[q]) > 0.f)) ve[q] = T(0);
                if (kCheck) bad |= !isfinite(Elem<T>::to_f32(ve[q]));
              }
            }
            *reinterpret_cast<u32x4*>(&C[o]) = v;
          }
        }
      }
  } else {
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
            if (kEpi == 1) v = relu(v);
            if (kEpi == 2 &&
                !(Elem<T>::to_f32(static_cast<const T*>(g.mask)[static_cast<int64_t>(r0 + row) * g.N + col]) > 0.f))
              v = 0.f;
            if (kCheck) bad |= !isfinite(v);
            C[static_cast<int64_t>(r0 + row) * g.N + col] = Elem<T>::from_f32(v);
          }
        }
    }
  }
  if (kCheck) note_nonfinite(g.nonfinite, bad);
}

// One thread per (expert, column block, k-step, lane): lane's 16-byte B operand.
// Column n = nb*32 + lane%32, k = ks*2V + (lane/32)*V + i; zero padded. kTrans: the
// source is stored [E, N, K] (B = the transpose of a weight, for the backward pass).
template <typename T, bool kTrans>
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
    v[i] = (n < N && k < K) ? W[kTrans ? (static_cast<int64_t>(e) * N + n) * K + k
                                        : (static_cast<int64_t>(e) * K + k) * N + n]
                            : T(0);
  }
  out[idx] = *reinterpret_cast<const uint4*>(v);
}

// The kTrans source ([E, N, K]: a lane's 16-byte operand is contiguous in a row) through LDS:
// a block takes 32 rows (one column block) x 16 k-steps, reads them as whole row segments
// (512 bytes a row, 16 bytes a thread), and writes the 16 fragments in slot order (16 bytes
// a thread, 1 KB a wave). kVec: K % V == 0 and W 16-byte aligned (vector loads).
constexpr int kPackKs = 16;  // k-steps per block
template <typename T, bool kVec>
__global__ __launch_bounds__(256) void pack_weights_t(const T* __restrict__ W, int E, int K, int N,
                                                      int NB, int KS, uint4* __restrict__ out) {
  constexpr int V = Elem<T>::kVec;
  constexpr int kRowBytes = kPackKs * 2 * V * static_cast<int>(sizeof(T));  // 512
  constexpr int kStride = kRowBytes + 16;
  __shared__ __align__(16) unsigned char tile[32 * kStride];
  const int kc = blockIdx.x, nb = blockIdx.y, e = blockIdx.z;
  const int k_base = kc * kPackKs * 2 * V;
#pragma unroll
  for (int p = 0; p < 32 * (kRowBytes / 16) / 256; ++p) {
    const int c = threadIdx.x + 256 * p;
    const int r = c / (kRowBytes / 16), seg = c % (kRowBytes / 16);
    const int n = nb * 32 + r, k0 = k_base + seg * V;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < N) {
      const T* row = W + (static_cast<int64_t>(e) * N + n) * K;
      if (kVec) {
        if (k0 < K) v = *reinterpret_cast<const uint4*>(row + k0);
      } else {
        T t[V];
#pragma unroll
        for (int i = 0; i < V; ++i) t[i] = k0 + i < K ? row[k0 + i] : T(0);
        v = *reinterpret_cast<const uint4*>(t);
      }
    }
    *reinterpret_cast<uint4*>(&tile[r * kStride + seg * 16]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kPackKs * kWave / 256; ++p) {
    const int sl = threadIdx.x + 256 * p;
    const int ksl = sl / kWave, lane = sl % kWave;
    const int ks = kc * kPackKs + ksl;
    if (ks >= KS) break;  // uniform over the thread's remaining slots
    const int r = lane & 31, kb = (ksl * 2 + (lane >> 5)) * V * static_cast<int>(sizeof(T));
    out[((static_cast<int64_t>(e) * NB + nb) * KS + ks) * kWave + lane] =
        *reinterpret_cast<const uint4*>(&tile[r * kStride + kb]);
  }
}

}  // namespace

// ------------------------------------------------------------------ host side
// layer 1: W1 (K = D, N = H); 2: W2 (K = H, N = D); 3: W2 transposed (K = D, N = H);
// 4: W1 transposed (K = H, N = D).
static void layer_dims(const Dims& d, int layer, int* K, int* N) {
  const bool to_h = layer == 1 || layer == 3;
  *K = to_h ? d.D : d.H;
  *N = to_h ? d.H : d.D;
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
  const bool tr = layer >= 3;
  if (tr) {  // the LDS-tiled re-layout of an [E, N, K] source
    const dim3 g3(ceil_div(KS, kPackKs), NB, d.E);
    const int V = d.dtype == MOE_BF16 ? 8 : 4;
    const bool vec = K % V == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0;
    if (d.dtype == MOE_BF16) {
      const auto* w = static_cast<const uint16_t*>(W);
      if (vec) pack_weights_t<uint16_t, true><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, KS, static_cast<uint4*>(Wp));
      else pack_weights_t<uint16_t, false><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, KS, static_cast<uint4*>(Wp));
    } else {
      const auto* w = static_cast<const float*>(W);
      if (vec) pack_weights_t<float, true><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, KS, static_cast<uint4*>(Wp));
      else pack_weights_t<float, false><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, KS, static_cast<uint4*>(Wp));
    }
    return launch_status();
  }
  if (d.dtype == MOE_BF16) {
    const auto* w = static_cast<const uint16_t*>(W);
    if (tr) pack_weights<uint16_t, true><<<grid, 256, 0, stream>>>(w, d.E, K, N, NB, KS, static_cast<uint4*>(Wp));
    else pack_weights<uint16_t, false><<<grid, 256, 0, stream>>>(w, d.E, K, N, NB, KS, static_cast<uint4*>(Wp));
  } else {
    const auto* w = static_cast<const float*>(W);
    if (tr) pack_weights<float, true><<<grid, 256, 0, stream>>>(w, d.E, K, N, NB, KS, static_cast<uint4*>(Wp));
    else pack_weights<float, false><<<grid, 256, 0, stream>>>(w, d.E, K, N, NB, KS, static_cast<uint4*>(Wp));
  }
  return launch_status();
}

template <typename T, int BM, int kEpi, bool kCheck, bool kGather>
static void launch_kc(const GemmArgs& g, int grid, size_t lds, hipStream_t stream) {
  constexpr int V = Elem<T>::kVec;
  const bool full = g.K % (128 / static_cast<int>(sizeof(T))) == 0;
  const bool vout = g.N % V == 0;
  if (full && vout) grouped_gemm<T, BM, kEpi, true, true, kCheck, kGather><<<grid, kThreads, lds, stream>>>(g);
  else if (full) grouped_gemm<T, BM, kEpi, true, false, kCheck, kGather><<<grid, kThreads, lds, stream>>>(g);
  else if (vout) grouped_gemm<T, BM, kEpi, false, true, kCheck, kGather><<<grid, kThreads, lds, stream>>>(g);
  else grouped_gemm<T, BM, kEpi, false, false, kCheck, kGather><<<grid, kThreads, lds, stream>>>(g);
}

// Only the plain epilogue is ever given a non-finite flag (the forward's layer 2), and only
// layer 1 reads gathered rows.
template <typename T, int BM, int kEpi>
static void launch_k(const GemmArgs& g, int grid, size_t lds, hipStream_t stream) {
  if constexpr (kEpi == 0) {
    if (g.nonfinite) {
      launch_kc<T, BM, kEpi, true, false>(g, grid, lds, stream);
      return;
    }
  }
  if constexpr (kEpi == 1) {
    if (g.row_token) {
      launch_kc<T, BM, kEpi, false, true>(g, grid, lds, stream);
      return;
    }
  }
  launch_kc<T, BM, kEpi, false, false>(g, grid, lds, stream);
}

template <typename T, int BM>
static void launch_typed(const GemmArgs& g, int layer, int grid, size_t lds, hipStream_t stream) {
  if (layer == 1) launch_k<T, BM, 1>(g, grid, lds, stream);
  else if (g.mask) launch_k<T, BM, 2>(g, grid, lds, stream);
  else launch_k<T, BM, 0>(g, grid, lds, stream);
}

// Upper bound on the tiles of BM rows: per expert at most ceil(min(C,T)/BM) row tiles;
// overall at most (rows + E*(BM-1))/BM.
static int64_t gemm_tiles(const Dims& d, int N, int bm) {
  const int64_t cap = std::min<int64_t>(d.C, d.T);
  const int64_t by_expert = static_cast<int64_t>(d.E) * ceil_div64(cap, bm);
  const int64_t by_rows = (d.max_rows + static_cast<int64_t>(d.E) * (bm - 1)) / bm;
  return std::min(by_expert, by_rows) * ceil_div(N, kBN);
}

static int device_cus() {
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

moe_status gemm_launch(const Dims& d, int layer, const void* A, const void* Wp, const int32_t* offsets,
                       void* C, int* nonfinite, hipStream_t stream, const void* mask,
                       const int32_t* row_token) {
  int K, N;
  layer_dims(d, layer, &K, &N);
  GemmArgs g;
  g.A = A;
  g.Wp = static_cast<const uint4*>(Wp);
  g.offsets = offsets;
  g.C = C;
  g.nonfinite = nonfinite;
  g.mask = mask;
  g.row_token = layer == 1 ? row_token : nullptr;
  g.E = d.E;
  g.K = K;
  g.N = N;
  g.NB = ceil_div(N, 32);
  g.KS = gemm_ks(d, K);
  // 128-row tiles, or 64-row ones when the 128-row tiles would not give every CU's two block
  // slots two tiles each (a small or narrow layer): twice the blocks then share the work
  const int bm = gemm_tiles(d, N, 128) < 4LL * device_cus() ? 64 : 128;
  const int64_t tiles = gemm_tiles(d, N, bm);
  const int64_t grid = ceil_div64(std::max<int64_t>(tiles, 1), kXcds) * kXcds;
  if (grid > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  const size_t lds = (static_cast<size_t>(d.E) + 1) * sizeof(int);
  const int gr = static_cast<int>(grid);
  if (d.dtype == MOE_BF16) {
    if (bm == 64) launch_typed<uint16_t, 64>(g, layer, gr, lds, stream);
    else launch_typed<uint16_t, 128>(g, layer, gr, lds, stream);
  } else {
    if (bm == 64) launch_typed<float, 64>(g, layer, gr, lds, stream);
    else launch_typed<float, 128>(g, layer, gr, lds, stream);
  }
  return launch_status();
}

}  // namespace moe
