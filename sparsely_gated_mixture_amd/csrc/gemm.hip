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
//     16-byte B operands are contiguous (one 1 KB fragment). Where the groups are
//     large (kStageOrderRows rows an expert on average) the fragments are ordered
//     [e][ks / 4][nb][ks % 4]: one k stage (4 k-steps) of all of an expert's
//     column blocks is one contiguous run, so a tile's stage of B is one region
//     rather than 4 KB pieces a whole column block apart; with small groups,
//     where each block streams an expert's weights once, [e][nb][ks] (one long
//     run per column block) is faster.
//   * Two kernels. Large bf16 groups (at least 192 rows an expert on average, or
//     96 with K >= 2048) run the persistent 256 x 256 kernel of 8 waves further
//     down, which stages both operands in LDS by direct global-to-LDS loads. The
//     rest run the BM x 256 kernel described here, in which a wave streams its B
//     operand straight from memory with one coalesced 1 KB load per fragment (B
//     never touches LDS).
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
#include <mutex>
#include <type_traits>

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
  int64_t ws_expert, ws_block, ws_stage;  // fragment strides (PackStrides)
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
  const u32x4* W0 = Wb + (e * g.ws_expert + min(n0 / 32 + wave * 2, g.NB - 1) * g.ws_block) * kWave + lane;
  const u32x4* W1 = Wb + (e * g.ws_expert + min(n0 / 32 + wave * 2 + 1, g.NB - 1) * g.ws_block) * kWave + lane;
  const int64_t wstage = g.ws_stage * kWave;  // one k stage

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
      const int64_t kn = stn * wstage + ks * kWave;
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

// ------------------------------------------------------------------ 256 x 256 tiles
// The large-group kernel (bf16, K a multiple of 64): one persistent block of 8 waves per CU
// walks a list of 256 x 256 output tiles. Wave w computes the 128 x 64 part at rows
// 128 (w / 4), columns 64 (w % 4) in 128 fp32 accumulators a lane, so two waves share each
// SIMD: a wave's instructions issue in order, and one whose load or LDS read cannot issue yet
// holds back its own MFMAs while the SIMD's other wave runs its MFMAs (four waves of 128 x 128
// each were 5-6% slower). Both operands go through LDS, so each byte brought to the CU feeds
// 256 rows or columns (the 128 x 256 kernel above re-streams B for every 128 rows): a third
// fewer operand bytes per FLOP.
//   * Operands land in LDS by direct loads (global_load_lds_dwordx4: lane l of a wave writes
//     its 16 bytes at M0 + 16 l), with no registers spent on staging. A stage is 64 deep in k.
//     A: each load instruction moves 8 whole 128-byte row segments (lane l: row l / 8), so
//     every request is a full cache line; rows are gathered through row_token for layer 1. In
//     LDS a row's eight 16-byte segments are XOR-permuted by bits 1-3 of the row index (lane
//     l fetches the segment that belongs at its slot), so the MFMA reads, 32 rows at one k
//     offset, hit distinct banks. B: the packed weights' 1 KB fragments (32 columns x 16 k)
//     are copied as they are and read back as whole 1 KB runs.
//   * LDS holds two stages of A and three of B (32 KB each, 160 KB). One barrier a stage,
//     before its last k-step; the loads of A stage st+2 go out between that k-step's MFMAs and
//     those of B stage st+2 between the MFMAs of stage st's first three k-steps (B's third
//     slot lets them start a stage early), a few at a time, so the wave's in-order issue never
//     stalls behind a burst of loads. Waves 0-3 issue every load (wave w: A rows 64 w .. 64 w
//     + 63 and B column blocks 2 w, 2 w + 1 of the tile), waves 4-7 only read LDS and compute
//     (about 1% faster than spreading the loads over all eight). The loads are issued in
//     inline assembly so the compiler, which cannot tell the ring slots apart, does not wait
//     for every load in flight before each LDS read; the kernel waits for its own loads
//     (vmcnt: a wave's vector memory operations complete in issue order) and its own reads
//     (lgkmcnt) before the barrier.
//   * Tiles: every thread counts the row tiles of its share of the experts once; a tile's
//     expert is then found by a walk over the experts' offsets (uniform loads). After a tile's
//     last k-step the next tile's first stages are already requested, so their latency
//     overlaps the epilogue's work, and no block launch separates the tiles. Each XCD's 32 CUs
//     walk a contiguous run of the tile order (expert, column tile, row tile) together,
//     sharing operands in their L2.
//   * The MFMA takes the weight fragment as its first operand, so the accumulator holds the
//     tile transposed: lane l owns output row l % 32 of its 32 x 32 block and, in registers
//     4q .. 4q+3, four adjacent columns 8q + 4 (l / 32) .. +3. The epilogue stages a wave's
//     32 x 64 pieces in a 4 KB LDS tile of its own (the eight tiles fill the B slot not in
//     use) and stores them back as whole 128-byte row runs (full cache lines).
//   * Epilogues: plain (kEpi 0), ReLU (1), or the backward's dH (2: zero where the stored
//     activation at the same place is not > 0); kCheck records NaN / Inf outputs.
constexpr int kBig = 256;                  // tile rows and columns
constexpr int kMaxGemmExperts = 4096;      // the library's largest E
constexpr int kFragBytes = 1024;           // one 64-lane x 16-byte fragment
constexpr int kStageBytes = kBig * 128;    // one operand's stage: 256 rows (columns) x 64 bf16
constexpr int kBOff = 2 * kStageBytes;     // B's three slots follow A's two
constexpr int kSlot2 = kBOff + 2 * kStageBytes;  // B's third slot: also staging and scratch
constexpr int kStageTile = 4096;           // epilogue staging per wave: 32 rows x 128 bytes
constexpr int kScratch = kSlot2 + kStageBytes - 64;  // scan scratch and the tile broadcast
constexpr size_t kBigLds = 5 * static_cast<size_t>(kStageBytes);  // 160 KB

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(p)));
}
// 16 bytes a lane from global memory at base + voff (base wave-uniform, voff a 32-bit byte
// offset) into LDS at lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
               : "memory");
}
// This wave's vector memory operations (all but the last N) and LDS reads done, then the
// workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// 1 if either bf16 of a packed pair has an all-ones exponent (NaN or infinity; rounding keeps
// both, and a value past the bf16 range becomes infinite)
__device__ __forceinline__ bool bf16_pair_nonfinite(s16x2 h) {
  const uint32_t u = __builtin_bit_cast(uint32_t, h);
  return ((u & 0x7f80u) == 0x7f80u) | ((u & 0x7f800000u) == 0x7f800000u);
}
// Eight bf16 values with each one zeroed where the mask's bf16 at the same place is not > 0
// (a NaN mask zeroes it).
__device__ __forceinline__ u32x4 relu_mask_bf16x8(u32x4 v, u32x4 mq) {
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const uint32_t mw = mq[w2];
    uint32_t vw = v[w2];
    if (!(__uint_as_float(mw << 16) > 0.f)) vw &= 0xffff0000u;
    if (!(__uint_as_float(mw & 0xffff0000u) > 0.f)) vw &= 0x0000ffffu;
    v[w2] = vw;
  }
  return v;
}

constexpr int kThreads8 = 512;

template <int kEpi, bool kCheck, bool kGather>
__global__ __launch_bounds__(kThreads8, 1) void grouped_gemm_big(GemmArgs g) {
  static_assert(!kCheck || kEpi == 0, "the check is compiled for the plain epilogue only");
  extern __shared__ __align__(16) unsigned char smem[];
  int* wt = reinterpret_cast<int*>(smem + kScratch);       // 8 ints: block scan
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = g.E;
  const int32_t* off = g.offsets;

  // ---- row tiles per expert: thread tid owns experts e0 .. e1-1 and keeps the number of row
  // tiles before them (excl) and in them (mine)
  const int per = (E + kThreads8 - 1) / kThreads8;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int mine = 0;
  for (int e = e0; e < e1; ++e) mine += (off[e + 1] - off[e] + kBig - 1) / kBig;
  int excl;
  const int row_tiles = block_exclusive_scan<kThreads8>(mine, &excl, wt);
  const int NT = (g.N + kBig - 1) / kBig;
  const int total_tiles = row_tiles * NT;
  const int per_xcd = (total_tiles + kXcds - 1) / kXcds;
  const int nblk_xcd = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int first = xcd * per_xcd + local, last = min(total_tiles, (xcd + 1) * per_xcd);
  const int n_my = first < last ? (last - first + nblk_xcd - 1) / nblk_xcd : 0;
  if (n_my == 0) return;

  const int K = g.K;
  const int nst = K / 64;
  const unsigned char* Ab = static_cast<const unsigned char*>(g.A);
  const unsigned char* Wp = reinterpret_cast<const unsigned char*>(g.Wp);
  // lane l of loading wave w's A load instruction i writes row 64 w + 8 i + l / 8 of the stage,
  // slot l % 8, and fetches the row segment that belongs at that slot
  auto aseg = [&](int i) { return ((lane & 7) ^ ((4 * i + (lane >> 4)) & 7)) * 16; };
  const uint32_t ring = lds_offset(smem);
  const int wm = wave >> 2, wn = wave & 3;

  struct Tile {
    int e, r0, rows, n0;
  };
  int we = 0, wcum = 0;
  auto locate = [&](int m) {
    const int logical = first + m * nblk_xcd;
    const int q = logical / NT;
    int t = (off[we + 1] - off[we] + kBig - 1) / kBig;
    while (wcum + t <= q) {
      wcum += t;
      ++we;
      t = (off[we + 1] - off[we] + kBig - 1) / kBig;
    }
    const int loc = logical - wcum * NT;
    const int n_tile = loc / t, m_tile = loc - n_tile * t;
    Tile T;
    T.e = we;
    T.r0 = off[we] + m_tile * kBig;
    T.rows = min(kBig, off[we + 1] - T.r0);
    T.n0 = n_tile * kBig;
    return T;
  };
  const int lw = wave & 3;  // loader index (waves 0-3 load)
  const bool loader = wave < 4;
  int tok[8];
  auto request_rows = [&](const Tile& T) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = min(64 * lw + 8 * i + (lane >> 3), T.rows - 1);
      tok[i] = kGather ? g.row_token[T.r0 + r] : T.r0 + r;
    }
  };
  auto sources = [&](const Tile& T, uint32_t (&ao)[8], const unsigned char* (&bb)[2]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ao[i] = static_cast<uint32_t>(static_cast<int64_t>(tok[i]) * K * 2 + aseg(i));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nb = min(T.n0 / 32 + 2 * lw + j, g.NB - 1);
      bb[j] = Wp + (T.e * g.ws_expert + nb * g.ws_block) * kFragBytes;
    }
  };
  uint32_t ao_cur[8], ao_nxt[8];
  const unsigned char* bb_cur[2];
  const unsigned char* bb_nxt[2];
  const uint32_t boff = lane * 16;

  auto dma_a = [&](int s, int kst, int i) {
    dma16(Ab, ao_cur[i] + kst * 128, ring + (s & 1) * kStageBytes + (64 * lw + 8 * i) * 128);
  };
  auto dma_b = [&](int s, int kst, int n) {
    const int j = n >> 2, ks = n & 3;
    dma16(bb_cur[j], boff + static_cast<uint32_t>(kst * static_cast<int>(g.ws_stage) + ks) * kFragBytes,
          ring + kBOff + (s % 3) * kStageBytes + ((2 * lw + j) * 4 + ks) * kFragBytes);
  };

  f32x16 acc[4][2];
  int a_lane = (lane & 31) * 128;
  int a_xor = (lane >> 1) & 7, a_half = lane >> 5;
  u32x4 fa[2][4], fb[2][2];
  auto read = [&](int s, int ks, int b) {
    const unsigned char* pa = smem + (s & 1) * kStageBytes;
    const unsigned char* pb = smem + kBOff + (s % 3) * kStageBytes;
    const int slot = ((2 * ks + a_half) ^ a_xor) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[b][i] = *reinterpret_cast<const u32x4*>(pa + (wm * 4 + i) * 32 * 128 + a_lane + slot);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[b][j] = *reinterpret_cast<const u32x4*>(pb + ((wn * 2 + j) * 4 + ks) * kFragBytes + lane * 16);
  };
  // one k-step's 8 MFMAs in four groups; after group i, dmas(i) issues this k-step's share of
  // the loads
  auto mma_all = [&](int b, auto dmas) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mma<uint16_t>(fb[b][j], fa[b][i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      dmas(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Stage s: a loading wave issues 8 B loads over
  // k-steps 0..2 (3, 3, 2) and 8 A loads in the last k-step (two a group). Before the last
  // k-step its loads of stage s + 1 are waited for (only the B loads of stage s + 2 may still be
  // in flight) and every wave passes the barrier.
  const int S = n_my * nst;
  auto body = [&](int s, int st) {
    const bool refill = s + 2 < S;
    const int kst2 = st + 2 >= nst ? st + 2 - nst : st + 2;
    if (st == nst - 2 && refill) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ao_cur[i] = ao_nxt[i];
      bb_cur[0] = bb_nxt[0];
      bb_cur[1] = bb_nxt[1];
    }
    const bool rl = refill && loader;
    read(s, 1, 1);
    mma_all(0, [&](int grp) {
      if (rl && grp < 3) dma_b(s + 2, kst2, grp);
    });
    read(s, 2, 0);
    mma_all(1, [&](int grp) {
      if (rl && grp < 3) dma_b(s + 2, kst2, 3 + grp);
    });
    read(s, 3, 1);
    mma_all(0, [&](int grp) {
      if (rl && grp < 2) dma_b(s + 2, kst2, 6 + grp);
    });
    if (rl) wait_barrier<8>();
    else wait_barrier<0>();
    read(s + 1, 0, 0);
    mma_all(1, [&](int grp) {
      if (rl) {
        dma_a(s + 2, kst2, 2 * grp);
        dma_a(s + 2, kst2, 2 * grp + 1);
      }
    });
  };

  uint16_t* C = static_cast<uint16_t*>(g.C);
  __syncthreads();  // the scan scratch is read by every thread before any load reuses LDS
  Tile cur = locate(0), nxt_t = cur;
  request_rows(cur);
  sources(cur, ao_cur, bb_cur);
  bb_nxt[0] = bb_cur[0];
  bb_nxt[1] = bb_cur[1];
#pragma unroll
  for (int i = 0; i < 8; ++i) ao_nxt[i] = ao_cur[i];
  if (n_my > 1) {
    nxt_t = locate(1);
    request_rows(nxt_t);
    sources(nxt_t, ao_nxt, bb_nxt);
  }
  if (loader) {
#pragma unroll
    for (int s0 = 0; s0 < 2; ++s0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dma_a(s0, s0, i);
#pragma unroll
      for (int n = 0; n < 8; ++n) dma_b(s0, s0, n);
    }
    wait_barrier<16>();
  } else {
    wait_barrier<0>();
  }
  read(0, 0, 0);

  bool bad = false;
  int s = 0;
  for (int m = 0; m < n_my; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int st = 0; st < nst; ++st, ++s) body(s, st);

    // ---- epilogue: the wave's four 32 x 64 pieces (row block i, both column blocks) through
    // its 4 KB LDS tile (in the B slot of the tile's last stage), rows stored as 128-byte runs
    const Tile done = cur;
    cur = nxt_t;
    const bool more2 = m + 2 < n_my;
    if (more2) {
      nxt_t = locate(m + 2);
      request_rows(nxt_t);
    }
    int lq = lane;
    asm volatile("" : "+v"(lq));
    unsigned char* stile = smem + kBOff + ((s - 1) % 3) * kStageBytes + wave * kStageTile;
    u32x4 rb[4];
    auto stage_piece = [&](int i) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x16& a = acc[i][jj];
          s16x2 h0 = __builtin_bit_cast(s16x2, __builtin_convertvector((f32x2){a[4 * qd], a[4 * qd + 1]}, bf16x2));
          s16x2 h1 = __builtin_bit_cast(s16x2, __builtin_convertvector((f32x2){a[4 * qd + 2], a[4 * qd + 3]}, bf16x2));
          if (kCheck) bad |= bf16_pair_nonfinite(h0) | bf16_pair_nonfinite(h1);
          if (kEpi == 1) {
            h0 = __builtin_elementwise_max(h0, (s16x2){0, 0});
            h1 = __builtin_elementwise_max(h1, (s16x2){0, 0});
          }
          uint2 v;
          v.x = __builtin_bit_cast(uint32_t, h0);
          v.y = __builtin_bit_cast(uint32_t, h1);
          const int row = lq & 31;
          const int cb = jj * 64 + qd * 16 + (lq >> 5) * 8;
          const int sw = ((cb >> 4) ^ (row & 7)) * 16 + (cb & 15);
          *reinterpret_cast<uint2*>(stile + row * 128 + sw) = v;
        }
    };
    auto read_piece = [&]() {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = 8 * p + (lq >> 3), ch = lq & 7;
        rb[p] = *reinterpret_cast<const u32x4*>(stile + row * 128 + ((ch ^ (row & 7)) * 16));
      }
    };
    // mode 2 (the backward's dH): the mask's 16 bytes at each stored vector, requested before
    // the piece is staged so that their latency is covered
    u32x4 mk[kEpi == 2 ? 4 : 1];
    auto load_mask = [&](int i) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = 8 * p + (lq >> 3), ch = lq & 7;
        const int grow = min(wm * 128 + i * 32 + row, done.rows - 1);
        const int col = done.n0 + wn * 64 + ch * 8;
        mk[p] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(g.mask) +
                                                static_cast<int64_t>(done.r0 + grow) * g.N + col);
      }
    };
    auto store_piece = [&](int i) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = 8 * p + (lq >> 3), ch = lq & 7;
        const int grow = min(wm * 128 + i * 32 + row, done.rows - 1);
        const int col = done.n0 + wn * 64 + ch * 8;
        u32x4 v = rb[p];
        if constexpr (kEpi == 2) v = relu_mask_bf16x8(v, mk[p]);
        *reinterpret_cast<u32x4*>(C + static_cast<int64_t>(done.r0 + grow) * g.N + col) = v;
      }
    };
    // a wave's LDS operations complete in order: piece i + 1 is staged only after piece i has
    // been read back
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kEpi == 2) load_mask(i);
      stage_piece(i);
      read_piece();
      store_piece(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if (more2) sources(nxt_t, ao_nxt, bb_nxt);
  }
  if (kCheck) note_nonfinite(g.nonfinite, bad);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The [E, K, N] source (W1, W2 as the pages lay them out) through LDS: a block takes one k
// stage (4 k-steps, 8V rows of k) of kPackNb column blocks, reads those rows as whole
// kPackNb * 32-column segments, and writes the stage's kPackNb * 4 fragments, one contiguous
// run in stage order (16 bytes a thread, 1 KB a wave). Lane l of fragment (nb, ks) holds
// column nb*32 + l%32, k = ks*2V + (l/32)*V + i; zeros past K or N. kVec: N % V == 0 and W
// 16-byte aligned (vector loads).
constexpr int kPackNb = 8;  // column blocks per block
template <typename T, bool kVec>
__global__ __launch_bounds__(256) void pack_weights(const T* __restrict__ W, int E, int K, int N, int NB,
                                                    PackStrides ps, uint4* __restrict__ out) {
  constexpr int V = Elem<T>::kVec;
  constexpr int kRows = 8 * V;                                          // k rows of a stage
  constexpr int kRowBytes = kPackNb * 32 * static_cast<int>(sizeof(T));  // 512 or 1024
  constexpr int kStride = kRowBytes + 16;
  constexpr int kSegs = kRowBytes / 16;
  __shared__ __align__(16) unsigned char tile[kRows * kStride];
  const int cb = blockIdx.x, q = blockIdx.y, e = blockIdx.z;
  const int n_base = cb * kPackNb * 32, k_base = q * kRows;
  static_assert(kRows * kSegs % 256 == 0, "whole passes");
#pragma unroll
  for (int p = 0; p < kRows * kSegs / 256; ++p) {
    const int c = threadIdx.x + 256 * p;
    const int r = c / kSegs, seg = c % kSegs;
    const int k = k_base + r, n0 = n_base + seg * V;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k < K) {
      const T* row = W + (static_cast<int64_t>(e) * K + k) * N;
      if (kVec) {
        if (n0 < N) v = *reinterpret_cast<const uint4*>(row + n0);
      } else {
        T t[V];
#pragma unroll
        for (int i = 0; i < V; ++i) t[i] = n0 + i < N ? row[n0 + i] : T(0);
        v = *reinterpret_cast<const uint4*>(t);
      }
    }
    *reinterpret_cast<uint4*>(&tile[r * kStride + seg * 16]) = v;
  }
  __syncthreads();
  const int nbs = min(kPackNb, NB - cb * kPackNb);
  const int ksl = threadIdx.x >> 6, lane = threadIdx.x & 63;  // k-step in the stage, lane
  const int col = lane & 31, kr0 = ksl * 2 * V + (lane >> 5) * V;
  for (int nb = 0; nb < nbs; ++nb) {
    T t[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
      t[i] = *reinterpret_cast<const T*>(&tile[(kr0 + i) * kStride + (nb * 32 + col) * static_cast<int>(sizeof(T))]);
    out[(e * ps.expert + (cb * kPackNb + nb) * ps.block + q * ps.stage + ksl) * kWave + lane] =
        *reinterpret_cast<const uint4*>(t);
  }
}

// The kTrans source ([E, N, K]: a lane's 16-byte operand is contiguous in a row) through LDS:
// a block takes 32 rows (one column block) x 16 k-steps, reads them as whole row segments
// (512 bytes a row, 16 bytes a thread), and writes the 16 fragments in slot order (16 bytes
// a thread, 1 KB a wave). kVec: K % V == 0 and W 16-byte aligned (vector loads).
constexpr int kPackKs = 16;  // k-steps per block
template <typename T, bool kVec>
__global__ __launch_bounds__(256) void pack_weights_t(const T* __restrict__ W, int E, int K, int N,
                                                      int NB, int KS, PackStrides ps,
                                                      uint4* __restrict__ out) {
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
    out[(e * ps.expert + nb * ps.block + (ks / 4) * ps.stage + ks % 4) * kWave + lane] =
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

PackStrides pack_strides(const Dims& d, int layer) {
  int K, N;
  layer_dims(d, layer, &K, &N);
  const int64_t NB = ceil_div(N, 32), KS = gemm_ks(d, K);
  const bool stage_order = d.max_rows >= kStageOrderRows * d.E;
  PackStrides ps;
  ps.expert = NB * KS;
  ps.block = stage_order ? 4 : KS;
  ps.stage = stage_order ? 4 * NB : 4;
  return ps;
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
  const PackStrides ps = pack_strides(d, layer);
  const bool tr = layer >= 3;
  if (tr) {  // the LDS-tiled re-layout of an [E, N, K] source
    const dim3 g3(ceil_div(KS, kPackKs), NB, d.E);
    const int V = d.dtype == MOE_BF16 ? 8 : 4;
    const bool vec = K % V == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0;
    if (d.dtype == MOE_BF16) {
      const auto* w = static_cast<const uint16_t*>(W);
      if (vec) pack_weights_t<uint16_t, true><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, KS, ps, static_cast<uint4*>(Wp));
      else pack_weights_t<uint16_t, false><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, KS, ps, static_cast<uint4*>(Wp));
    } else {
      const auto* w = static_cast<const float*>(W);
      if (vec) pack_weights_t<float, true><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, KS, ps, static_cast<uint4*>(Wp));
      else pack_weights_t<float, false><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, KS, ps, static_cast<uint4*>(Wp));
    }
    return launch_status();
  }
  // the [E, K, N] source: a block per (kPackNb column blocks, k stage, expert)
  const dim3 g3(ceil_div(NB, kPackNb), KS / 4, d.E);
  const int V = d.dtype == MOE_BF16 ? 8 : 4;
  const bool vec = N % V == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0;
  if (d.dtype == MOE_BF16) {
    const auto* w = static_cast<const uint16_t*>(W);
    if (vec) pack_weights<uint16_t, true><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, ps, static_cast<uint4*>(Wp));
    else pack_weights<uint16_t, false><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, ps, static_cast<uint4*>(Wp));
  } else {
    const auto* w = static_cast<const float*>(W);
    if (vec) pack_weights<float, true><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, ps, static_cast<uint4*>(Wp));
    else pack_weights<float, false><<<g3, 256, 0, stream>>>(w, d.E, K, N, NB, ps, static_cast<uint4*>(Wp));
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

// The 256 x 256 kernel needs more LDS than the default per-block limit: raise it once per
// device for each instance.
template <int kEpi, bool kCheck, bool kGather>
static moe_status launch_big(const GemmArgs& g, int grid, hipStream_t stream) {
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  bool ok = true;
  std::call_once(once[dev], [&] {
    ok = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_big<kEpi, kCheck, kGather>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(kBigLds)) == hipSuccess;
  });
  if (!ok) return MOE_ERR_HIP;
  grouped_gemm_big<kEpi, kCheck, kGather><<<grid, kThreads8, kBigLds, stream>>>(g);
  return launch_status();
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
  const PackStrides ps = pack_strides(d, layer);
  g.ws_expert = ps.expert;
  g.ws_block = ps.block;
  g.ws_stage = ps.stage;
  // Large groups (bf16, at least 192 rows per expert on average, enough 256 x 256 tiles to give
  // every CU one): the 256 x 256 LDS-staged kernel. With a long k-loop (K >= 2048) it also pays
  // at half that, its row tiles then half empty (switch_bf16's and batchwise_bf16's layer 2,
  // 128 rows an expert: 7% and 5% faster; their layer 1, K = 768 / 512, 1% and 12% slower)
  // (its A row offsets and its B offsets within an expert are 32-bit byte offsets)
  const int64_t a_rows = row_token ? d.T : d.max_rows;
  const int64_t min_rows = K >= 2048 ? 96 : 192;
  if (d.dtype == MOE_BF16 && K % 64 == 0 && K >= 256 && N % kBig == 0 && !(mask && nonfinite) &&
      a_rows * K * 2 < (1LL << 32) &&
      static_cast<int64_t>(g.KS) * g.NB * kFragBytes < (1LL << 32) &&
      d.E <= kMaxGemmExperts && d.max_rows >= min_rows * d.E &&
      gemm_tiles(d, N, kBig) >= device_cus()) {
    // persistent: one block per CU
    const int grid = std::max(kXcds, device_cus() / kXcds * kXcds);
    // (only the plain epilogue is ever given a non-finite flag: the forward's layer 2)
    if (mask) return launch_big<2, false, false>(g, grid, stream);
    if (g.row_token) return launch_big<1, false, true>(g, grid, stream);
    if (layer == 1) return launch_big<1, false, false>(g, grid, stream);
    if (nonfinite) return launch_big<0, true, false>(g, grid, stream);
    return launch_big<0, false, false>(g, grid, stream);
  }
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
