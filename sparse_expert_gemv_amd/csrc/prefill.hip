// Prefill-sized (T > 64) path of the Flint MoE layer on gfx950: the same layer
// as the decode path, computed as matrix-core (MFMA) GEMMs because at these
// batch sizes each expert sees ~T*6/256 tokens and the work is a dense
// contraction per expert.
//
// Five launches on the caller's stream (six for the pre-norm block, whose
// RMSNorm of r into the workspace buffer `normed` comes first, one wave per
// token):
//   1. router  : logits[32 tokens x 256] = X Wr^T per block (bf16 MFMA, fp32
//                accumulate, + bias; four waves, four more keeping their
//                barriers), then in the epilogue the top-k of each token by
//                sigmoid score (each of the eight waves ranks four tokens at a
//                time from the logits parked in LDS), the routing weights,
//                and the block's per-expert slot counts.
//   2. bucket  : every block sums the router blocks' counts, scans them into
//                expert offsets and places its own (token, rank) slots in
//                stable order (ascending slot within an expert); block 0
//                writes the routing table (U ascending) and the grouped-GEMM
//                tile list (256-slot M-tiles of one expert, no padding
//                stored); the inverse permutation is kept for the combine.
//   3. gate/up : grouped GEMM per (256-slot tile, 128 h columns): gathered x
//                rows times the gate and up rows of w13 (bf16 MFMA), SiLU-and-
//                mul in registers, h parked in LDS and stored as fp16 in
//                sorted slot order (the shared expert's tiles cover the tokens
//                in order).
//   4. down    : grouped GEMM per (routed 256-slot tile, 256 output columns):
//                h (fp16) times w2 (bf16 converted to fp16 in registers) into
//                the unweighted fp16 y of each slot, the whole tile parked in
//                LDS and stored as 16-byte vectors.
//   5. shared down + combine : the shared expert's down GEMM per (256
//                tokens, 256 columns) whose epilogue adds sum_j w_j * y_j in
//                rank order (+ r for the block) and rounds once to bf16, the
//                next 8-column unit's y rows in flight while one is summed.
// All GEMMs share one block-level scheme (BlockGemm): A and B tiles move
// from global memory straight into LDS (LDS-direct loads, no register
// staging) through one ring per operand, with rows' 16-byte chunks
// XOR-swizzled so that the fragment reads of consecutive rows hit distinct
// banks.  The ring depths and K chunk per GEMM: gate/up 128-byte chunks (64
// K-elements) with two stages for the gathered x rows (L2-resident) and
// three for the weights (from HBM), 160 KiB; the routed and dense down GEMMs
// 64-byte chunks with two stages of h and four of w2; the router and the
// shared-expert down + combine three and three of 64 (router: 128) bytes.
// The grouped GEMMs run 256 x 256 block tiles on eight waves of 64 x 128
// (32x32x16 MFMAs); the router 32 x 256 on four waves of 32 x 64 (of the
// block's eight).
// Numerics: fp32 accumulation everywhere.  h and y cross the launches as
// fp16 (11-bit significand) carrying a power-of-two bias: h is stored as
// fp16(h * 2^-8), so the down GEMMs produce y * 2^-8, which the routed down
// stores as fp16 and the combine multiplies back by 2^8 (exactly) after the
// weighted sum.  The bias moves fp16's overflow threshold from 65504 to
// 65504 * 2^8 = 1.68e7 for |h| and |y|; values below 2^-6 are stored with
// the fp16 subnormal spacing, an absolute error of at most 2^-17.  w2 is
// widened from bf16 to fp16 exactly for 2^-14 <= |w| <= 65504; smaller
// weights keep an absolute error below 2^-25.
//
// What is computed follows "vLLM Day-0 Support for Recursive's Flint"
// (section "Flint Model Architecture", bullet "MoE Structure"; section
// "Optimization Strategies", bullets "Small-batch MoE Kernels" and
// "Low-Latency Decode Path"), the SiLU form of "Flint on Arc Pro B70"
// (section "norm.py: Triton kernels that assumed CUDA"), and the prefill
// batch size of "RecursiveSI/flint — vLLM serving recipe" (section
// "Benchmarking": prefill 8K).

#include "flint_device.h"
#include "flint_kernels.h"

namespace flint {
namespace {

constexpr int H = kHidden;
constexpr int I = kInter;
constexpr int kThreads = 256;
constexpr int kMT = kPrefillTile;   // tokens per router / scatter block
constexpr int kGM = kGroupTile;     // slots per grouped-GEMM M-tile
// Power-of-two bias of the fp16 h (and so of the down GEMMs' results): see
// the numerics note above.  Multiplying by either is exact.
constexpr float kH16Bias = 1.0f / 256.0f;
constexpr float kH16Unbias = 256.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// 8 bf16 -> 8 fp16 (round to nearest even; exact in fp16's normal range).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4& v) {
  u32x4 r;
  r.x = pack_f16x2(bf16_lo(v.x), bf16_hi(v.x));
  r.y = pack_f16x2(bf16_lo(v.y), bf16_hi(v.y));
  r.z = pack_f16x2(bf16_lo(v.z), bf16_hi(v.z));
  r.w = pack_f16x2(bf16_lo(v.w), bf16_hi(v.w));
  return r;
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Accumulator element r of lane l in a 32x32 MFMA tile: row (r / 4) * 8 +
// (l / 32) * 4 + r % 4, column l % 32.  A and B operands: lane l supplies row
// (column) l % 32 with K elements [(l / 32) * 8, +8) of each 16-wide K step.
__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// Waits until at most n vector-memory operations of this wave are
// outstanding (the LDS-direct loads below count as vector-memory operations
// until their data has landed in LDS).
template <int n>
__device__ __forceinline__ void wait_vmem() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14));
}
// Workgroup barrier that is also a compiler barrier for memory operations.
// Unlike __syncthreads it does not wait for this wave's outstanding loads,
// so loads of later pipeline stages stay in flight across it; the caller
// waits for exactly the stage it needs first (wait_vmem).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Block GEMM C[BM x BN] = A[BM x K] B[BN x K]^T with both operands K-
// contiguous in global memory, fed through an S-stage LDS ring of KC-wide K
// chunks (KC * 2 bytes per row and stage).  With KC = 32 the three-stage
// ring of a 256 x 256 tile takes 96 KiB; KC = 64 moves whole 128-byte lines
// but doubles the ring.
// Global -> LDS moves are LDS-direct loads (global_load_lds, 16 bytes per
// lane): one instruction of a wave fills 1 KiB of LDS, i.e. RPI consecutive
// rows, lane i writing 16-byte chunk i % CPR of row i / CPR.  Within a row
// the 16-byte K chunks are XOR-swizzled by swz(row), which spreads the MFMA
// fragment reads of consecutive rows over all LDS banks; each lane therefore
// fetches the K chunk that belongs at its physical slot.  Thread (wave w,
// lane i) fetches A rows (w * NA + j) * RPI + i / CPR and B rows
// (w * NB + j) * RPI + i / CPR; the caller hands over one global pointer per
// such row, already advanced by chunk_elems(row) elements (fetch_row_a/b and
// chunk_elems give the mapping).  Waves form a WM x WN grid; each owns a
// (BM / WM) x (BN / WN) tile of 32x32x16 MFMAs.  kF16: A is fp16 and B (bf16
// in memory) is converted to fp16 in registers before the MFMA; otherwise
// both are bf16.
template <int BM, int BN, int WM, int WN, bool kF16, int SA, int SB, int KC>
struct BlockGemm {
  static constexpr int kWM = WM, kWN = WN;
  static constexpr int NW = WM * WN;                  // waves per block
  static constexpr int kBlockThreads = 64 * NW;       // the launch's block size
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int RT = TM / 32, CT = TN / 32;
  static constexpr int kRow = KC * 2;                 // LDS bytes per row
  static constexpr int CPR = kRow / 16;               // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                // rows per LDS-direct instruction
  static constexpr int NA = BM / (NW * RPI), NB = BN / (NW * RPI);   // instructions per thread per stage
  static constexpr int NL = NA + NB;
  static constexpr int kStageA = BM * kRow, kStageB = BN * kRow;
  static constexpr int kLds = SA * kStageA + SB * kStageB;   // A ring, then B ring
  // Outstanding loads allowed at the top of a step in steady state: those
  // issued after the last one the step needs (see run).
  static constexpr int kWaitN = SA == SB ? (SA - 2) * NL : NB + (SA - 2) * NL;
  static_assert(KC == 32 || KC == 64, "K chunk");
  static_assert(TM % 32 == 0 && TN % 32 == 0 && BM % (NW * RPI) == 0 && BN % (NW * RPI) == 0, "tile shape");
  static_assert(SA >= 2 && SB >= SA && kWaitN < 64, "pipeline depth");

  f32x16 acc[RT][CT];

  // 64-byte rows: four consecutive rows cover the 64 banks of a 256-byte
  // window, so the chunk index changes every fourth row.  Measured with the
  // LDS bank-conflict counter on the fragment-read pattern (lane l: row
  // l % 32, chunk 2 ks + l / 32): no conflict cycles, against one conflict
  // cycle per active cycle for ((row >> 1) ^ (row >> 3)) & 3.
  __device__ static __forceinline__ int swz(int row) {
    return CPR == 4 ? (row >> 2) & 3 : (row ^ (row >> 1)) & 7;
  }
  __device__ static __forceinline__ int fetch_row_a(int j) {
    return ((threadIdx.x >> 6) * NA + j) * RPI + ((threadIdx.x & 63) / CPR);
  }
  __device__ static __forceinline__ int fetch_row_b(int j) {
    return ((threadIdx.x >> 6) * NB + j) * RPI + ((threadIdx.x & 63) / CPR);
  }
  __device__ static __forceinline__ int chunk_elems(int row) {
    return (((int)threadIdx.x & (CPR - 1)) ^ swz(row)) * 8;
  }

  // rt_n: 32-row sub-tiles of this wave that hold data (the rest are skipped).
  // Returns after a barrier, with the LDS free for reuse.
  __device__ __forceinline__ void run(uint8_t* lds, const uint16_t* const (&ag)[NA],
                                      const uint16_t* const (&bg)[NB], int K, int rt_n_in) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rt_n = __builtin_amdgcn_readfirstlane(rt_n_in);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int nk = K / KC;
    uint8_t* ldsB = lds + SA * kStageA;
    auto issue_a = [&](int kc) {
      uint8_t* st = lds + (kc % SA) * kStageA;
#pragma unroll
      for (int j = 0; j < NA; ++j)
        __builtin_amdgcn_global_load_lds(ag[j] + kc * KC, (lds_ptr_t)(st + (wave * NA + j) * 1024), 16, 0, 0);
    };
    auto issue_b = [&](int kc) {
      uint8_t* st = ldsB + (kc % SB) * kStageB;
#pragma unroll
      for (int j = 0; j < NB; ++j)
        __builtin_amdgcn_global_load_lds(bg[j] + kc * KC, (lds_ptr_t)(st + (wave * NB + j) * 1024), 16, 0, 0);
    };
    // Step kc issues A chunk kc + SA - 1, then B chunk kc + SB - 1; the
    // prologue issues what the steps before 0 would have.  A step needs A
    // and B chunk kc: with SA == SB the later of the two is B chunk kc, with
    // SB > SA it is A chunk kc (B's ring runs further ahead), and kWaitN
    // loads were issued after it.  Near the end fewer were: wait for all.
#pragma unroll
    for (int j = -(SB - 1); j < 0; ++j) {
      if (j + SA - 1 >= 0 && j + SA - 1 < nk) issue_a(j + SA - 1);
      if (j + SB - 1 < nk) issue_b(j + SB - 1);
    }
    // Fragment reads: rows wm*TM + rt*32 + lane%32 (A) and wn*TN + ct*32 +
    // lane%32 (B) all have swz == swz(lane % 32).
    int koff[KC / 16];
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) koff[ks] = (((ks * 2 + (lane >> 5)) ^ swz(lane & 31)) * 16);
    const int a_rd = (wm * TM + (lane & 31)) * kRow;
    const int b_rd = (wn * TN + (lane & 31)) * kRow;
    constexpr int KS = KC / 16;
    auto mfmas = [&](const u32x4 (&af)[RT], u32x4 (&bfr)[CT]) __attribute__((always_inline)) {
      if constexpr (kF16) {
#pragma unroll
        for (int j = 0; j < CT; ++j) bfr[j] = bf16x8_to_f16x8(bfr[j]);
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        if (i >= rt_n) continue;
#pragma unroll
        for (int j = 0; j < CT; ++j) {
          if constexpr (kF16) acc[i][j] = mfma_f16(af[i], bfr[j], acc[i][j]);
          else acc[i][j] = mfma_bf16(af[i], bfr[j], acc[i][j]);
        }
      }
    };
    for (int kc = 0; kc < nk; ++kc) {
      if (kc + SB - 2 < nk) wait_vmem<kWaitN>();
      else wait_vmem<0>();
      stage_barrier();   // chunk kc is in LDS for every wave; the slots of chunk kc - 1 are free
      const uint8_t* sa = lds + (kc % SA) * kStageA;
      const uint8_t* sb = ldsB + (kc % SB) * kStageB;
      if constexpr (SA == SB) {
        // All fragments of the chunk first, then the next chunks' loads
        // (issued while the fragment reads are in flight), then the MFMAs.
        u32x4 af[KS][RT], bfr[KS][CT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int i = 0; i < RT; ++i)
            af[ks][i] = *reinterpret_cast<const u32x4*>(sa + a_rd + i * 32 * kRow + koff[ks]);
#pragma unroll
          for (int j = 0; j < CT; ++j)
            bfr[ks][j] = *reinterpret_cast<const u32x4*>(sb + b_rd + j * 32 * kRow + koff[ks]);
        }
        if (kc + SA - 1 < nk) issue_a(kc + SA - 1);
        if (kc + SB - 1 < nk) issue_b(kc + SB - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mfmas(af[ks], bfr[ks]);
      } else {
        // Deeper B ring (128-byte K chunks): the next chunks' loads first,
        // then each 16-wide K step's fragments and MFMAs.
        if (kc + SA - 1 < nk) issue_a(kc + SA - 1);
        if (kc + SB - 1 < nk) issue_b(kc + SB - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 af[RT], bfr[CT];
#pragma unroll
          for (int i = 0; i < RT; ++i)
            af[i] = *reinterpret_cast<const u32x4*>(sa + a_rd + i * 32 * kRow + koff[ks]);
#pragma unroll
          for (int j = 0; j < CT; ++j)
            bfr[j] = *reinterpret_cast<const u32x4*>(sb + b_rd + j * 32 * kRow + koff[ks]);
          mfmas(af, bfr);
        }
      }
    }
    __syncthreads();
  }

  // For a block's waves past the NW that run the GEMM: the same barriers
  // as run(), nothing else.
  __device__ __forceinline__ void shadow(int K) {
    const int nk = K / KC;
    for (int kc = 0; kc < nk; ++kc) stage_barrier();
    __syncthreads();
  }
};

// Block -> work item, XCD-aware: the hardware deals blocks to the 8 XCDs
// round-robin; item w is given to XCD w / ceil(n/8) so that consecutive items
// (the M-tiles and column blocks of one expert, which read the same weight
// and activation rows) share an XCD's L2.  n is the live item count: the
// grouped GEMMs' grids are sized for the longest possible tile list and
// their kernels read the real length on the device, so that the live items,
// not the grid, are spread over the XCDs.  The grid holds at least
// 8 ceil(n/8) blocks; every item below n gets exactly one, and the caller
// returns for the rest (item >= n).
__device__ __forceinline__ int xcd_item(int n) {
  const int per = (n + 7) / 8;
  const int b = blockIdx.x;
  if (b >= 8 * per) return n;
  return (b % 8) * per + b / 8;
}

constexpr int round8(int n) { return (n + 7) / 8 * 8; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// ---------------------------------------------------------------- 1. router

__device__ __forceinline__ uint32_t ord_f32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// 32 tokens per block (256 blocks at T = 8192, one per CU) with 128-byte K
// chunks: the router matrix is small and shared by every block, so the
// GEMM is bound by each block's latency per K step, not by bytes.
using RouterGemm = BlockGemm<kMT, kMaxExperts, 1, 4, false, 3, 3, 64>;
// RMSNorm rows: n = bf16(r / rms(r) * gamma), one wave per token; lane l
// owns the 16-byte vectors l, l + 64, l + 128, l + 192 of the row.
constexpr int kNormVecPerLane = H / 8 / 64;   // 4

__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const uint16_t* __restrict__ r,
                                                          const uint16_t* __restrict__ gamma,
                                                          float eps, uint16_t* __restrict__ n,
                                                          int T) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (int)(threadIdx.x / 64);
  if (t >= T) return;
  const u32x4* row = reinterpret_cast<const u32x4*>(r + (size_t)t * H);
  const u32x4* gam = reinterpret_cast<const u32x4*>(gamma);
  u32x4 rv[kNormVecPerLane], gv[kNormVecPerLane];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormVecPerLane; ++i) {
    rv[i] = row[lane + 64 * i];
    gv[i] = gam[lane + 64 * i];
  }
#pragma unroll
  for (int i = 0; i < kNormVecPerLane; ++i) ss += sumsq_bf16x8(rv[i]);
  ss = wave_sum_lane63(ss);
  const float inv = rms_inv<H>(__builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                   __builtin_bit_cast(int, ss), 63)), eps);
  u32x4* dst = reinterpret_cast<u32x4*>(n + (size_t)t * H);
#pragma unroll
  for (int i = 0; i < kNormVecPerLane; ++i) dst[lane + 64 * i] = rms_scale_bf16x8(rv[i], gv[i], inv);
}

constexpr int kZRow = kMaxExperts + 1;   // logits row stride in LDS (floats)

// Top-k of G tile rows i0, i0 + di, ... (tokens t0 + i) from the logits
// parked in LDS, one wave, the G selections interleaved round by round.
// Ranks on the logit (the sigmoid is strictly increasing), ties to the lower
// expert index: lane l holds the order-preserving keys of experts 4l ..
// 4l + 3 sorted by (key descending, expert ascending); round j takes the
// wave maximum of the lanes' heads and the lowest lane holding it pops its
// head (lower lanes hold lower experts).  Lane j keeps the j-th pick; the
// routing weights are s_j / sum s (if renormalised) x routed_scale, and each
// pick is counted in hist.  Rows past T are ranked on zero keys and dropped.
template <int G>
__device__ void rank_rows(const LayerArgs& a, const float* zs, int t0, int i0, int di, int* hist) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k, T = a.T;
  uint32_t key[G][4];
  int ex[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int i = i0 + g * di;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      const uint32_t kz = ord_f32(zs[i * kZRow + e]);
      key[g][q] = (e < E && t0 + i < T) ? kz : 0u;
      ex[g][q] = e;
    }
    auto cx = [&](int u, int v) __attribute__((always_inline)) {
      const bool sw = key[g][v] > key[g][u] || (key[g][v] == key[g][u] && ex[g][v] < ex[g][u]);
      const uint32_t ku = key[g][u], kv = key[g][v];
      const int eu = ex[g][u], ev = ex[g][v];
      key[g][u] = sw ? kv : ku;
      key[g][v] = sw ? ku : kv;
      ex[g][u] = sw ? ev : eu;
      ex[g][v] = sw ? eu : ev;
    };
    cx(0, 1);
    cx(2, 3);
    cx(0, 2);
    cx(1, 3);
    cx(1, 2);
  }
  // Rounds unrolled to the largest k (uniform exit at k): the pops and the
  // picks are selects, not branches.
  int my_e[G];
  uint32_t my_key[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    my_e[g] = 0;
    my_key[g] = 0;
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    uint32_t m[G];
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = key[g][0];
    wave_max_u32_lane63_multi<G>(m);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint32_t M = (uint32_t)__builtin_amdgcn_readlane((int)m[g], 63);
      const int win = (int)__builtin_ctzll(__ballot(key[g][0] == M));
      const int best = __builtin_amdgcn_readlane(ex[g][0], win);
      const bool pop = lane == win;
      key[g][0] = pop ? key[g][1] : key[g][0];
      key[g][1] = pop ? key[g][2] : key[g][1];
      key[g][2] = pop ? key[g][3] : key[g][2];
      key[g][3] = pop ? 0u : key[g][3];
      ex[g][0] = pop ? ex[g][1] : ex[g][0];
      ex[g][1] = pop ? ex[g][2] : ex[g][1];
      ex[g][2] = pop ? ex[g][3] : ex[g][2];
      my_e[g] = lane == j ? best : my_e[g];
      my_key[g] = lane == j ? M : my_key[g];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = t0 + i0 + g * di;
    const float sc = lane < k ? sigmoid(unord_f32(my_key[g])) : 0.f;
    const float sum = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum_lane63(sc)), 63));
    if (t < T && lane < k) {
      const float w = (a.renormalize ? sc / sum : sc) * a.routed_scale;
      a.ws.ids[t * k + lane] = my_e[g];
      a.ws.wts[t * k + lane] = w;
      if (a.ids_out) a.ids_out[t * k + lane] = my_e[g];
      if (a.wts_out) a.wts_out[t * k + lane] = w;
      atomicAdd(&hist[my_e[g]], 1);
    }
  }
}

// Eight waves: the first four run the GEMM (the others only keep its
// barriers), then all eight rank the tile's rows, two waves per SIMD
// instead of one (the ranking is a chain of dependent wave reductions).
constexpr int kRouterThreads = 2 * RouterGemm::kBlockThreads;

__global__ __launch_bounds__(kRouterThreads) void prefill_router_kernel(LayerArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[cmax(RouterGemm::kLds, kMT * kZRow * 4)];
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E;
  const int t0 = blockIdx.x * kMT;
  for (int i = tid; i < kMaxExperts; i += kRouterThreads) hist[i] = 0;
  const bool gemm = wave < RouterGemm::NW;

  // logits[t0 .. t0+64) x [0, 256): token rows clamped to T-1, experts to E-1.
  const uint16_t* ag[RouterGemm::NA];
  const uint16_t* bg[RouterGemm::NB];
#pragma unroll
  for (int i = 0; i < RouterGemm::NA; ++i) {
    const int r = RouterGemm::fetch_row_a(i);
    ag[i] = a.x + (size_t)min(t0 + r, T - 1) * H + RouterGemm::chunk_elems(r);
  }
#pragma unroll
  for (int i = 0; i < RouterGemm::NB; ++i) {
    const int r = RouterGemm::fetch_row_b(i);
    bg[i] = a.router_w + (size_t)min(r, E - 1) * H + RouterGemm::chunk_elems(r);
  }
  RouterGemm g;
  float* zs = reinterpret_cast<float*>(lds);
  if (gemm) {
    g.run(lds, ag, bg, H, RouterGemm::RT);   // LDS is free afterwards
#pragma unroll
    for (int rt = 0; rt < RouterGemm::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < RouterGemm::CT; ++ct) {
        const int e = wave * RouterGemm::TN + ct * 32 + (lane & 31);
        const float b = (a.router_b && e < E) ? a.router_b[e] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) zs[(rt * 32 + acc_row(r, lane)) * kZRow + e] = g.acc[rt][ct][r] + b;
      }
  } else {
    g.shadow(H);
  }
  __syncthreads();
  if (tid < E)
    for (int i = 0; i < kMT && t0 + i < T; ++i) a.ws.logits[(size_t)(t0 + i) * E + tid] = zs[i * kZRow + tid];

  // Top-k: wave w ranks tile rows w, w + 8, w + 16, w + 24 (rank_rows).
  constexpr int kRW = kRouterThreads / 64;
  static_assert(kMT == 4 * kRW, "four rows per wave");
  rank_rows<4>(a, zs, t0, wave, kRW, hist);
  __syncthreads();
  for (int e = tid; e < E; e += kRouterThreads) a.ws.pre.counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// ---------------------------------------------------------------- 2. bucketing

// Stable counting sort of the T*k slots by expert, one launch of nb blocks
// (one per router block).  Block b sums the router's per-block expert counts
// itself, four threads per expert each over a quarter of the blocks,
// kBucketBatch counts per round trip: before[e] over the blocks ahead of b
// and total[e] over all.  The totals' exclusive scan over experts gives the
// group offsets; the block places each of its slots at offset + before +
// its rank among the block's slots of the same expert (read from per-expert
// occupancy bitmaps), so slots ascend within every group.  Block 0 also
// writes the routing table's header (U and the group offsets) and the
// M-tile list.
constexpr int kBucketThreads = 1024;
constexpr int kBucketParts = kBucketThreads / kMaxExperts;   // 4
constexpr int kBucketBatch = 16;

// Exclusive prefix sum of v over threads [0, 256) (one value per expert).
// Every thread of the block calls it; threads >= 256 pass 0 and get 0.
__device__ __forceinline__ int expert_excl_scan(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63 && wave < 4) s_wave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave && w < 4; ++w) base += s_wave[w];
  __syncthreads();
  return threadIdx.x < kMaxExperts ? base + incl - v : 0;
}

__global__ __launch_bounds__(kBucketThreads) void prefill_bucket_kernel(LayerArgs a, int nb) {
  constexpr int kWords = kMT * kMaxTopK / 32;        // bitmap words per expert
  __shared__ uint32_t occ[kMaxExperts * kWords];
  __shared__ int s_part[2][kBucketParts][kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_wave[4];
  __shared__ int s_tot[2];
  const int tid = threadIdx.x;
  const int e = tid % kMaxExperts, part = tid / kMaxExperts;
  const bool lead = part == 0;
  const int T = a.T, E = a.E, k = a.k;
  const int b = blockIdx.x;
  const int s0 = b * kMT * k;
  const int ns = min(kMT, T - b * kMT) * k;
  const PrefillWs& p = a.ws.pre;
  for (int q = tid; q < kMaxExperts * kWords; q += kBucketThreads) occ[q] = 0;

  const int per = (nb + kBucketParts - 1) / kBucketParts;
  const int b0 = min(nb, part * per), b1 = min(nb, b0 + per);
  int before = 0, total = 0;
  if (e < E)
    for (int c0 = b0; c0 < b1; c0 += kBucketBatch) {
      int c[kBucketBatch];
#pragma unroll
      for (int q = 0; q < kBucketBatch; ++q) c[q] = c0 + q < b1 ? p.counts[(size_t)(c0 + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < kBucketBatch; ++q) {
        total += c[q];
        before += c0 + q < b ? c[q] : 0;
      }
    }
  s_part[0][part][e] = before;
  s_part[1][part][e] = total;
  __syncthreads();   // the partials and the cleared bitmaps
  for (int q = tid; q < ns; q += kBucketThreads) {
    const int ex = a.ws.ids[s0 + q];
    atomicOr(&occ[ex * kWords + (q >> 5)], 1u << (q & 31));
  }
  int cnt = 0, bef = 0;
  if (lead && e < E)
    for (int q = 0; q < kBucketParts; ++q) {
      cnt += s_part[1][q][e];
      bef += s_part[0][q][e];
    }
  const int off = expert_excl_scan(cnt, s_wave);   // its barriers also publish the bitmaps
  if (lead) s_base[e] = off + bef;
  __syncthreads();

  int32_t* route = a.ws.route;
  int32_t* slots = route + 2 + 2 * E;
  for (int q = tid; q < ns; q += kBucketThreads) {
    const int ex = a.ws.ids[s0 + q];
    const uint32_t* m = occ + ex * kWords;
    int rank = __popc(m[q >> 5] & ((1u << (q & 31)) - 1u));
    for (int w = 0; w < (q >> 5); ++w) rank += __popc(m[w]);
    const int pos = s_base[ex] + rank;
    slots[pos] = s0 + q;
    p.pos[s0 + q] = pos;
  }

  if (b == 0) {   // block-uniform: the scans below synchronise the block
    const int active = cnt > 0;
    const int aidx = expert_excl_scan(active, s_wave);
    const int ntile = (cnt + kGM - 1) / kGM;
    const int tile0 = expert_excl_scan(ntile, s_wave);
    if (tid == kMaxExperts - 1) {
      s_tot[0] = aidx + active;
      s_tot[1] = tile0 + ntile;
    }
    if (active) {
      route[1 + aidx] = e;
      route[1 + E + aidx] = off;
      for (int q = 0; q < ntile; ++q) {
        int32_t* tl = p.tiles + 1 + 3 * (tile0 + q);
        tl[0] = e;
        tl[1] = off + q * kGM;
        tl[2] = min(kGM, cnt - q * kGM);
      }
    }
    __syncthreads();
    if (tid == 0) {
      route[0] = s_tot[0];
      route[1 + E + s_tot[0]] = T * k;
      p.tiles[0] = s_tot[1];
    }
  }
}

// ---------------------------------------------------------------- 4. gate/up

// Block tile: 256 slots x 256 rows of w13 = the gate and up rows of 128 h
// columns, eight waves.  Wave (wm, wn) owns slots [64 wm, +64) and h columns
// [64 wn, +64) of the block's 128: its B tiles ct = 0, 1 are gate rows and
// ct = 2, 3 the up rows of the same columns, so SiLU-and-mul pairs
// acc[.][ct] with acc[.][ct + 2] in registers.  The 256-slot M-tile stages a
// third fewer operand bytes per MFMA than a 128-slot one at the same waves
// per SIMD (one 96 KiB block per CU).
using GateUpGemm = BlockGemm<kGM, 256, 4, 2, false, 2, 3, 64>;
constexpr int kGuColBlocks = I / 128;   // 4

__global__ __launch_bounds__(GateUpGemm::kBlockThreads, 1) void prefill_gateup_kernel(LayerArgs a,
                                                                                    int n_shared_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[GateUpGemm::kLds];
  const PrefillWs& p = a.ws.pre;
  const int n_items = (n_shared_tiles + p.tiles[0]) * kGuColBlocks;
  const int item = xcd_item(n_items);
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / 2, wn = wave % 2;
  const int T = a.T, k = a.k, E = a.E;
  const int q = item / kGuColBlocks, nb = item % kGuColBlocks;   // column blocks of a tile adjacent
  const int32_t* slots = a.ws.route + 2 + 2 * E;

  const uint8_t* w13;
  int start, count, hrow0;
  const bool shared = q < n_shared_tiles;
  if (shared) {
    start = q * kGM;
    count = min(kGM, T - start);
    hrow0 = T * k + start;
    w13 = a.shared.w13;
  } else {
    const int rq = q - n_shared_tiles;
    const int32_t* tl = p.tiles + 1 + 3 * rq;
    w13 = a.routed.w13 + (size_t)tl[0] * 2 * I * H * 2;
    start = tl[1];
    count = tl[2];
    hrow0 = start;
  }
  const uint16_t* W = reinterpret_cast<const uint16_t*>(w13);
  const uint16_t* ag[GateUpGemm::NA];
  const uint16_t* bg[GateUpGemm::NB];
#pragma unroll
  for (int i = 0; i < GateUpGemm::NA; ++i) {
    const int fr = GateUpGemm::fetch_row_a(i);
    const int r = min(fr, count - 1);
    const int tok = shared ? start + r : slots[start + r] / k;
    ag[i] = a.x + (size_t)tok * H + GateUpGemm::chunk_elems(fr);
  }
#pragma unroll
  for (int i = 0; i < GateUpGemm::NB; ++i) {
    const int n = GateUpGemm::fetch_row_b(i);          // B row of the block tile
    const int bw = n >> 7, ct = (n >> 5) & 3;          // owning wave column, MFMA tile
    const int col = nb * 128 + bw * 64 + (ct & 1) * 32 + (n & 31);
    bg[i] = W + (size_t)((ct >> 1) * I + col) * H + GateUpGemm::chunk_elems(n);
  }
  const int rt_n = max(0, min(GateUpGemm::RT, (count - wm * GateUpGemm::TM + 31) / 32));
  GateUpGemm g;
  g.run(lds, ag, bg, H, rt_n);

  // The tile's h (256 slots x 128 columns, fp16) parked in LDS, then stored
  // as 16-byte vectors.
  constexpr int kHRow = 128 + 8;   // halves per LDS row
  static_assert(kGM * kHRow * 2 <= GateUpGemm::kLds, "the h tile fits the ring's LDS");
  _Float16* hs = reinterpret_cast<_Float16*>(lds);
#pragma unroll
  for (int rt = 0; rt < GateUpGemm::RT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * GateUpGemm::TM + rt * 32 + acc_row(r, lane);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float gv = g.acc[rt][ct][r], uv = g.acc[rt][ct + 2][r];
        hs[row * kHRow + wn * 64 + ct * 32 + (lane & 31)] = (_Float16)(silu(gv) * uv * kH16Bias);
      }
    }
  __syncthreads();
  _Float16* h16 = p.h16;
#pragma unroll
  for (int i = 0; i < kGM * 16 / GateUpGemm::kBlockThreads; ++i) {
    const int u = tid + i * GateUpGemm::kBlockThreads;
    const int row = u >> 4, c8 = (u & 15) * 8;
    if (row < count)
      *reinterpret_cast<u32x4*>(h16 + (size_t)(hrow0 + row) * I + nb * 128 + c8) =
          *reinterpret_cast<const u32x4*>(hs + row * kHRow + c8);
  }
}

// ---------------------------------------------------------------- 5. down (routed)

// Block tile: 256 slots x 256 output columns, eight waves; wave (wm, wn)
// owns slots [64 wm, +64) x columns [128 wn, +128).
using DownGemm = BlockGemm<kGM, 256, 4, 2, true, 3, 3, 32>;
constexpr int kDnColBlocks = H / 256;   // 8
// The routed down GEMM and the dense MLP's down GEMM stream their w2 rows
// through a four-deep ring (h, from L2, through a two-deep one): routed down
// 237.8 -> 228 us, dense down (I_d 14336) 756 -> 664 us at T = 8192, against
// three and three.  The combine's shared-expert GEMM keeps three and three
// (65 -> 71 us with four).
using DownGemmB4 = BlockGemm<kGM, 256, 4, 2, true, 2, 4, 32>;
// Epilogue: the fp16 y tile (256 slots x 256 columns) is parked row-major in
// LDS by all eight waves at once and stored as 16-byte vectors (the block's
// LDS is sized for it: 132 KiB; two halves through the ring's 96 KiB, one
// half's waves parking while the others waited, measured 7 us slower).
constexpr int kYRow = 256 + 8;          // halves per LDS row of the parked tile
static_assert(kGM * kMaxTopK % DownGemm::kBlockThreads == 0, "slot positions per thread");

__global__ __launch_bounds__(DownGemmB4::kBlockThreads, 1) void prefill_down_kernel(LayerArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[cmax(DownGemmB4::kLds, kGM * kYRow * 2)];
  const PrefillWs& p = a.ws.pre;
  const int n_items = p.tiles[0] * kDnColBlocks;
  const int item = xcd_item(n_items);
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / 2, wn = wave % 2;
  const int q = item / kDnColBlocks, nb = item % kDnColBlocks;
  const int32_t* tl = p.tiles + 1 + 3 * q;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.routed.w2) + (size_t)tl[0] * H * I;
  const int start = tl[1], count = tl[2];
  const uint16_t* h16 = reinterpret_cast<const uint16_t*>(p.h16);
  const uint16_t* ag[DownGemmB4::NA];
  const uint16_t* bg[DownGemmB4::NB];
#pragma unroll
  for (int i = 0; i < DownGemmB4::NA; ++i) {
    const int fr = DownGemmB4::fetch_row_a(i);
    ag[i] = h16 + (size_t)(start + min(fr, count - 1)) * I + DownGemmB4::chunk_elems(fr);
  }
#pragma unroll
  for (int i = 0; i < DownGemmB4::NB; ++i) {
    const int n = DownGemmB4::fetch_row_b(i);
    bg[i] = W + (size_t)(nb * 256 + n) * I + DownGemmB4::chunk_elems(n);
  }
  const int rt_n = max(0, min(DownGemmB4::RT, (count - wm * DownGemmB4::TM + 31) / 32));
  DownGemmB4 g;
  g.run(lds, ag, bg, I, rt_n);   // LDS is free afterwards
  // The whole y tile (fp16) parked in LDS by every wave at once, then
  // stored as 16-byte vectors.
  _Float16* ys = reinterpret_cast<_Float16*>(lds);
#pragma unroll
  for (int rt = 0; rt < DownGemmB4::RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < DownGemmB4::CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ys[(wm * DownGemmB4::TM + rt * 32 + acc_row(r, lane)) * kYRow + wn * DownGemmB4::TN + ct * 32 +
           (lane & 31)] = (_Float16)g.acc[rt][ct][r];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kGM * 32 / DownGemmB4::kBlockThreads; ++i) {
    const int u = tid + i * DownGemmB4::kBlockThreads;
    const int row = u >> 5, c8 = (u & 31) * 8;
    if (row < count)
      *reinterpret_cast<u32x4*>(p.y16 + (size_t)(start + row) * H + nb * 256 + c8) =
          *reinterpret_cast<const u32x4*>(ys + row * kYRow + c8);
  }
}

// ---------------------------------------------------------------- 6. shared down + combine

// Block tile: 256 tokens x 256 output columns of the shared expert's down
// GEMM.  Epilogue in four parts of 64 tokens: the owning waves park their
// accumulators in LDS, then every thread finishes 8 consecutive columns of a
// token at a time: out = shared + sum_j w_j y_j in rank order, one bf16
// rounding, 16-byte loads of y and stores of out.  KT is the number of y
// loads per unit (6 for k <= 6, else 8), fixed so that the next unit's loads
// can be in flight under exact wait counts.
constexpr int kCbRow = 256 + 4;   // floats per LDS row of the parked tile
constexpr int kCbLds = cmax(DownGemm::kLds, DownGemm::TM * kCbRow * 4);

template <int KT>
__global__ __launch_bounds__(DownGemm::kBlockThreads, 1) void prefill_shared_combine_kernel(LayerArgs a,
                                                                                         int n_items) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kCbLds];
  __shared__ int s_pos[kGM * kMaxTopK];     // y row and weight of each (token, rank) of the tile
  __shared__ float s_w[kGM * kMaxTopK];
  const int item = xcd_item(n_items);
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / 2, wn = wave % 2;
  const int T = a.T, k = a.k;
  const int q = item / kDnColBlocks, nb = item % kDnColBlocks;
  const PrefillWs& p = a.ws.pre;
  const int t0 = q * kGM, count = min(kGM, T - t0);
  // The tile's slot positions and weights are requested before the GEMM and
  // parked in LDS after it, so that the combine's y loads depend on no
  // global round trip of their own.
  constexpr int kPw = kGM * kMaxTopK / DownGemm::kBlockThreads;
  int pos_r[kPw];
  float w_r[kPw];
#pragma unroll
  for (int i = 0; i < kPw; ++i) {
    const int e = tid + i * DownGemm::kBlockThreads;
    if (e < count * k) {
      pos_r[i] = p.pos[t0 * k + e];
      w_r[i] = a.ws.wts[t0 * k + e];
    }
  }
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.shared.w2);
  const uint16_t* h16 = reinterpret_cast<const uint16_t*>(p.h16);
  const uint16_t* ag[DownGemm::NA];
  const uint16_t* bg[DownGemm::NB];
#pragma unroll
  for (int i = 0; i < DownGemm::NA; ++i) {
    const int fr = DownGemm::fetch_row_a(i);
    ag[i] = h16 + (size_t)(T * k + t0 + min(fr, count - 1)) * I + DownGemm::chunk_elems(fr);
  }
#pragma unroll
  for (int i = 0; i < DownGemm::NB; ++i) {
    const int n = DownGemm::fetch_row_b(i);
    bg[i] = W + (size_t)(nb * 256 + n) * I + DownGemm::chunk_elems(n);
  }
  const int rt_n = max(0, min(DownGemm::RT, (count - wm * DownGemm::TM + 31) / 32));
  DownGemm g;
  g.run(lds, ag, bg, I, rt_n);   // LDS is free afterwards
#pragma unroll
  for (int i = 0; i < kPw; ++i) {
    const int e = tid + i * DownGemm::kBlockThreads;
    if (e < count * k) {
      s_pos[e] = pos_r[i];
      s_w[e] = w_r[i];
    }
  }

  float* park = reinterpret_cast<float*>(lds);
  // Thread tid's combine units: 64 tokens x 32 groups of 8 columns per part,
  // kUnits per thread; unit it + 1's y rows are requested before unit it is
  // summed (every unit issues KT loads, ranks past k re-read rank k - 1 and
  // rows past count row count - 1, so the wait counts stay exact).
  constexpr int kUnits = DownGemm::TM * 32 / DownGemm::kBlockThreads;
  constexpr int kIters = DownGemm::kWM * kUnits;
  u32x4 yv[2][KT];
  float wj[2][KT];
  u32x4 rr[2];
  auto load_unit = [&](int it, int buf) __attribute__((always_inline)) {
    const int part = it / kUnits, s = it % kUnits;
    const int u = tid + s * DownGemm::kBlockThreads;
    const int row = u >> 5, c8 = (u & 31) * 8;
    const int lrow = min(part * DownGemm::TM + row, count - 1);
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int jj = min(j, k - 1);
      wj[buf][j] = s_w[lrow * k + jj];
      yv[buf][j] = *reinterpret_cast<const u32x4*>(p.y16 + (size_t)s_pos[lrow * k + jj] * H + nb * 256 + c8);
    }
    if (a.resid) rr[buf] = *reinterpret_cast<const u32x4*>(a.resid + (size_t)(t0 + lrow) * H + nb * 256 + c8);
  };
  __syncthreads();   // s_pos and s_w
  load_unit(0, 0);
#pragma unroll
  for (int part = 0; part < DownGemm::kWM; ++part) {
    if (wm == part) {
#pragma unroll
      for (int rt = 0; rt < DownGemm::RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < DownGemm::CT; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            park[(rt * 32 + acc_row(r, lane)) * kCbRow + wn * DownGemm::TN + ct * 32 + (lane & 31)] =
                g.acc[rt][ct][r];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kUnits; ++s) {
      const int it = part * kUnits + s;
      if (it + 1 < kIters) load_unit(it + 1, (it + 1) & 1);
      const int buf = it & 1;
      const int u = tid + s * DownGemm::kBlockThreads;
      const int row = u >> 5, c8 = (u & 31) * 8;
      const int lrow = part * DownGemm::TM + row;
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(park + row * kCbRow + c8);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(park + row * kCbRow + c8 + 4);
      float o[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        if (j < k) {
          const float w = wj[buf][j];
          const u32x4 y = yv[buf][j];
          o[0] = fmaf(w, f16_lo(y.x), o[0]);
          o[1] = fmaf(w, f16_hi(y.x), o[1]);
          o[2] = fmaf(w, f16_lo(y.y), o[2]);
          o[3] = fmaf(w, f16_hi(y.y), o[3]);
          o[4] = fmaf(w, f16_lo(y.z), o[4]);
          o[5] = fmaf(w, f16_hi(y.z), o[5]);
          o[6] = fmaf(w, f16_lo(y.w), o[6]);
          o[7] = fmaf(w, f16_hi(y.w), o[7]);
        }
      }
      if (lrow < count) {
        const int t = t0 + lrow;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] *= kH16Unbias;   // shared + weighted routed y, unbiased
        if (a.resid) {
          const u32x4 r = rr[buf];
          o[0] += bf16_lo(r.x);
          o[1] += bf16_hi(r.x);
          o[2] += bf16_lo(r.y);
          o[3] += bf16_hi(r.y);
          o[4] += bf16_lo(r.z);
          o[5] += bf16_hi(r.z);
          o[6] += bf16_lo(r.w);
          o[7] += bf16_hi(r.w);
        }
        u32x4 ob;
        ob.x = pack_bf16x2_rne(o[0], o[1]);
        ob.y = pack_bf16x2_rne(o[2], o[3]);
        ob.z = pack_bf16x2_rne(o[4], o[5]);
        ob.w = pack_bf16x2_rne(o[6], o[7]);
        *reinterpret_cast<u32x4*>(a.out + (size_t)t * H + nb * 256 + c8) = ob;
      }
    }
    __syncthreads();
  }
}
// Both instances explicitly: with only the launch sites, the compiler left
// the second one's host handle undefined.
template __global__ void prefill_shared_combine_kernel<6>(LayerArgs, int);
template __global__ void prefill_shared_combine_kernel<8>(LayerArgs, int);

// ---------------------------------------------------------------- dense MLP

// Gate/up GEMM of the dense MLP (layers 0 and 1): tile (128 tokens, 128 h
// columns) with the gate and up rows of w13 [2 I_d][H] as B, SiLU-and-mul
// epilogue, h fp16 [T][I_d].  Items run token-tile-major so that the column
// blocks of one token tile share its x rows on one XCD.
__global__ __launch_bounds__(GateUpGemm::kBlockThreads, 1) void dense_gateup_gemm_kernel(DenseArgs a,
                                                                                      int n_items) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[GateUpGemm::kLds];
  const int item = xcd_item(n_items);
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / 2, wn = wave % 2;
  const int n_cb = a.inter / 128;
  const int q = item / n_cb, nb = item % n_cb;
  const int start = q * kGM, count = min(kGM, a.T - start);
  const uint16_t* ag[GateUpGemm::NA];
  const uint16_t* bg[GateUpGemm::NB];
#pragma unroll
  for (int i = 0; i < GateUpGemm::NA; ++i) {
    const int fr = GateUpGemm::fetch_row_a(i);
    ag[i] = a.x + (size_t)(start + min(fr, count - 1)) * H + GateUpGemm::chunk_elems(fr);
  }
#pragma unroll
  for (int i = 0; i < GateUpGemm::NB; ++i) {
    const int n = GateUpGemm::fetch_row_b(i);
    const int bw = n >> 7, ct = (n >> 5) & 3;
    const int col = nb * 128 + bw * 64 + (ct & 1) * 32 + (n & 31);
    bg[i] = a.w13 + (size_t)((ct >> 1) * a.inter + col) * H + GateUpGemm::chunk_elems(n);
  }
  const int rt_n = max(0, min(GateUpGemm::RT, (count - wm * GateUpGemm::TM + 31) / 32));
  GateUpGemm g;
  g.run(lds, ag, bg, H, rt_n);
#pragma unroll
  for (int rt = 0; rt < GateUpGemm::RT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * GateUpGemm::TM + rt * 32 + acc_row(r, lane);
      if (row < count) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int col = nb * 128 + wn * 64 + ct * 32 + (lane & 31);
          const float gv = g.acc[rt][ct][r], uv = g.acc[rt][ct + 2][r];
          a.h16[(size_t)(start + row) * a.inter + col] = (_Float16)(silu(gv) * uv * kH16Bias);
        }
      }
    }
}

// Down GEMM of the dense MLP: tile (128 tokens, 256 output columns), h fp16
// times w2 (widened to fp16 into LDS), K = I_d; epilogue adds r for the
// pre-norm block and rounds once to bf16.
__global__ __launch_bounds__(DownGemmB4::kBlockThreads, 1) void dense_down_gemm_kernel(DenseArgs a, int n_items) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[DownGemmB4::kLds];
  const int item = xcd_item(n_items);
  if (item >= n_items) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / 2, wn = wave % 2;
  const int q = item / kDnColBlocks, nb = item % kDnColBlocks;
  const int start = q * kGM, count = min(kGM, a.T - start);
  const uint16_t* h16 = reinterpret_cast<const uint16_t*>(a.h16);
  const uint16_t* ag[DownGemmB4::NA];
  const uint16_t* bg[DownGemmB4::NB];
#pragma unroll
  for (int i = 0; i < DownGemmB4::NA; ++i) {
    const int fr = DownGemmB4::fetch_row_a(i);
    ag[i] = h16 + (size_t)(start + min(fr, count - 1)) * a.inter + DownGemmB4::chunk_elems(fr);
  }
#pragma unroll
  for (int i = 0; i < DownGemmB4::NB; ++i) {
    const int n = DownGemmB4::fetch_row_b(i);
    bg[i] = a.w2 + (size_t)(nb * 256 + n) * a.inter + DownGemmB4::chunk_elems(n);
  }
  const int rt_n = max(0, min(DownGemmB4::RT, (count - wm * DownGemmB4::TM + 31) / 32));
  DownGemmB4 g;
  g.run(lds, ag, bg, a.inter, rt_n);
#pragma unroll
  for (int rt = 0; rt < DownGemmB4::RT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * DownGemmB4::TM + rt * 32 + acc_row(r, lane);
      if (row < count) {
#pragma unroll
        for (int ct = 0; ct < DownGemmB4::CT; ++ct) {
          const int col = nb * 256 + wn * DownGemmB4::TN + ct * 32 + (lane & 31);
          const size_t idx = (size_t)(start + row) * H + col;
          float o = g.acc[rt][ct][r] * kH16Unbias;
          if (a.resid) o += bf16_lo(a.resid[idx]);
          a.out[idx] = f32_to_bf16_rne(o);
        }
      }
    }
}

}  // namespace

hipError_t launch_dense_prefill(const DenseArgs& a, hipStream_t stream, Launcher& launch) {
  const int n_tiles = (a.T + kGM - 1) / kGM;
  const int n_gu = n_tiles * (a.inter / 128);
  launch(dense_gateup_gemm_kernel, dim3(round8(n_gu)), dim3(GateUpGemm::kBlockThreads), stream, a, n_gu);
  const int n_dn = n_tiles * kDnColBlocks;
  launch(dense_down_gemm_kernel, dim3(round8(n_dn)), dim3(DownGemmB4::kBlockThreads), stream, a, n_dn);
  return hipGetLastError();
}

void launch_rmsnorm(const uint16_t* r, const uint16_t* gamma, float eps, uint16_t* n, int T,
                    hipStream_t stream, Launcher& launch) {
  launch(rmsnorm_kernel, dim3((T + kThreads / 64 - 1) / (kThreads / 64)), dim3(kThreads), stream, r,
         gamma, eps, n, T);
}

int prefill_tiles_max(int T, int E, int k) {
  return (T * k + kGM - 1) / kGM + E;  // bounds the sum over experts of ceil(count / kGM)
}

hipError_t launch_prefill(const LayerArgs& a, hipStream_t stream, Launcher& launch) {
  const int nb = (a.T + kMT - 1) / kMT;
  const int n_routed_max = prefill_tiles_max(a.T, a.E, a.k);
  const int n_shared = (a.T + kGM - 1) / kGM;
  if (a.norm_w) launch_rmsnorm(a.resid, a.norm_w, a.eps, a.normed, a.T, stream, launch);
  launch(prefill_router_kernel, dim3(nb), dim3(kRouterThreads), stream, a);
  launch(prefill_bucket_kernel, dim3(nb), dim3(kBucketThreads), stream, a, nb);
  // The grouped GEMMs' grids cover the longest possible tile list; the
  // kernels read the real one.
  const int n_gu = (n_shared + n_routed_max) * kGuColBlocks;
  launch(prefill_gateup_kernel, dim3(round8(n_gu)), dim3(GateUpGemm::kBlockThreads), stream, a, n_shared);
  const int n_dn = n_routed_max * kDnColBlocks;
  launch(prefill_down_kernel, dim3(round8(n_dn)), dim3(DownGemm::kBlockThreads), stream, a);
  const int n_sc = n_shared * kDnColBlocks;
  if (a.k <= 6)
    launch(prefill_shared_combine_kernel<6>, dim3(round8(n_sc)), dim3(DownGemm::kBlockThreads), stream, a, n_sc);
  else
    launch(prefill_shared_combine_kernel<8>, dim3(round8(n_sc)), dim3(DownGemm::kBlockThreads), stream, a, n_sc);
  return hipGetLastError();
}

}  // namespace flint
