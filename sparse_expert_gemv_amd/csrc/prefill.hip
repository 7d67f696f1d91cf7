// Prefill-sized (T > 64) path of the Flint MoE layer on gfx950: the same layer
// as the decode path, computed as matrix-core (MFMA) GEMMs because at these
// batch sizes each expert sees ~T*6/256 tokens and the work is a dense
// contraction per expert.
//
// Six launches on the caller's stream:
//   1. router  : logits[64 tokens x 256] = X Wr^T per block (bf16 MFMA, fp32
//                accumulate, + bias), top-k per token by sigmoid score, the
//                routing weights, and the block's per-expert slot counts.
//   2. scan    : one block turns the counts into expert offsets, the routing
//                table (U ascending) and the grouped-GEMM tile list (64 slots
//                per tile, no padding stored).
//   3. scatter : stable counting sort of the (token, rank) slots by expert,
//                ascending slot order within an expert; the inverse
//                permutation is kept for the combine.
//   4. gate/up : grouped GEMM per (expert tile, 128 h columns): gathered x
//                rows times the gate and up rows of w13 (bf16 MFMA), SiLU-and-
//                mul in registers, h stored as fp16 in sorted slot order (the
//                shared expert's tiles cover tokens in order).
//   5. down    : grouped GEMM per (routed expert tile, 256 output columns):
//                h (fp16) times w2 (bf16 widened to fp16 in registers, exact
//                for |w| >= 2^-14) into fp32 y per slot.
//   6. shared down + combine : the shared expert's down GEMM per (64 tokens,
//                256 columns) whose epilogue adds sum_j w_j * y_j in rank order
//                and rounds once to bf16.
// Numerics: fp32 accumulation everywhere; h is fp16 (11-bit significand) and
// y is fp32, so the only roundings of the decode path's fp32 arithmetic that
// this path adds are those of h to fp16 and of tiny w2 values to fp16
// subnormals.
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
constexpr int kMT = kPrefillTile;   // rows (slots or tokens) per M-tile

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

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// A wave's 64x64 tile: two 32-row tiles (rt) x two 32-column tiles (ct).
// MFMA 32x32x16 lane layout: lane l feeds row/column l % 32 with K elements
// [(l / 32) * 8, +8) of each 16-wide K step; accumulator element r of lane l
// is row (r / 4) * 8 + (l / 32) * 4 + r % 4, column l % 32.
struct Tile64 {
  f32x16 acc[2][2];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }
};

__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// C += A B^T over K: a[rt] and b[ct] point at the lane's A row / B row; both
// K-contiguous.  kF16: operands are fp16 (B widened from bf16 on the fly).
template <int K, bool kF16>
__device__ __forceinline__ void mma_k(Tile64& t, const uint16_t* const (&a)[2],
                                      const uint16_t* const (&b)[2]) {
  const int ko = ((threadIdx.x & 63) >> 5) * 8;
#pragma unroll 4
  for (int k = 0; k < K; k += 16) {
    const u32x4 a0 = ld16(a[0] + k + ko), a1 = ld16(a[1] + k + ko);
    u32x4 b0 = ld16(b[0] + k + ko), b1 = ld16(b[1] + k + ko);
    if constexpr (kF16) {
      b0 = bf16x8_to_f16x8(b0);
      b1 = bf16x8_to_f16x8(b1);
      t.acc[0][0] = mfma_f16(a0, b0, t.acc[0][0]);
      t.acc[0][1] = mfma_f16(a0, b1, t.acc[0][1]);
      t.acc[1][0] = mfma_f16(a1, b0, t.acc[1][0]);
      t.acc[1][1] = mfma_f16(a1, b1, t.acc[1][1]);
    } else {
      t.acc[0][0] = mfma_bf16(a0, b0, t.acc[0][0]);
      t.acc[0][1] = mfma_bf16(a0, b1, t.acc[0][1]);
      t.acc[1][0] = mfma_bf16(a1, b0, t.acc[1][0]);
      t.acc[1][1] = mfma_bf16(a1, b1, t.acc[1][1]);
    }
  }
}

// Block -> work item, XCD-aware: the hardware deals blocks to the 8 XCDs
// round-robin; item w is given to XCD w / ceil(n/8) so that consecutive items
// (the M-tiles of one expert at one column range, which read the same weight
// rows) share an XCD's L2.  The grid is n rounded up to a multiple of 8, so
// every item below n has exactly one block; blocks past n return.
__device__ __forceinline__ int xcd_item(int n) {
  const int per = (n + 7) / 8;
  const int b = blockIdx.x;
  return (b % 8) * per + b / 8;
}

constexpr int round8(int n) { return (n + 7) / 8 * 8; }

// ---------------------------------------------------------------- 1. router

__device__ __forceinline__ uint32_t ord_f32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ __launch_bounds__(kThreads) void prefill_router_kernel(LayerArgs a) {
  __shared__ float zs[kMT][kMaxExperts + 1];
  __shared__ int hist[kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, E = a.E, k = a.k;
  const int t0 = blockIdx.x * kMT;
  for (int i = threadIdx.x; i < kMaxExperts; i += kThreads) hist[i] = 0;

  // logits[t0 .. t0+64) x [64 wave, +64): rows clamped to T-1, experts to E-1.
  const uint16_t* ap[2];
  const uint16_t* bp[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) ap[rt] = a.x + (size_t)min(t0 + rt * 32 + (lane & 31), T - 1) * H;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
    bp[ct] = a.router_w + (size_t)min(wave * 64 + ct * 32 + (lane & 31), E - 1) * H;
  Tile64 tile;
  tile.zero();
  mma_k<H, false>(tile, ap, bp);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int e = wave * 64 + ct * 32 + (lane & 31);
      const float b = (a.router_b && e < E) ? a.router_b[e] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) zs[rt * 32 + acc_row(r, lane)][e] = tile.acc[rt][ct][r] + b;
    }
  __syncthreads();
  for (int q = threadIdx.x; q < kMT * E; q += kThreads) {
    const int i = q / E, e = q - i * E;
    if (t0 + i < T) a.ws.logits[(size_t)(t0 + i) * E + e] = zs[i][e];
  }

  // Top-k per token, one wave per token: ties to the lower expert index.
  for (int i = wave; i < kMT && t0 + i < T; i += 4) {
    const int t = t0 + i;
    uint64_t key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      key[q] = e < E ? (((uint64_t)ord_f32(zs[i][e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0;
    }
    float zsel[kMaxTopK];
    int isel[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      zsel[j] = 0.f;
      isel[j] = 0;
      if (j < k) {
        const uint64_t best =
            wave_max_u64(max_u64(max_u64(key[0], key[1]), max_u64(key[2], key[3])));
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (key[q] == best) key[q] = 0;
        isel[j] = (int)(0xFFFFFFFFu - (uint32_t)best);
        zsel[j] = unord_f32((uint32_t)(best >> 32));
      }
    }
    float s[kMaxTopK], sum = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      s[j] = sigmoid(zsel[j]);
      if (j < k) sum += s[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && lane == j) {
        const float w = (a.renormalize ? s[j] / sum : s[j]) * a.routed_scale;
        a.ws.ids[t * k + j] = isel[j];
        a.ws.wts[t * k + j] = w;
        if (a.ids_out) a.ids_out[t * k + j] = isel[j];
        if (a.wts_out) a.wts_out[t * k + j] = w;
        atomicAdd(&hist[isel[j]], 1);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) a.ws.pre.counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// ---------------------------------------------------------------- 2. scan

// Exclusive prefix sum over 256 values held one per thread (256 threads).
__device__ __forceinline__ int block_excl_scan256(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  __syncthreads();
  return base + incl - v;
}

__global__ __launch_bounds__(kThreads) void prefill_scan_kernel(LayerArgs a, int nb) {
  __shared__ int s_wave[4];
  __shared__ int s_tot[2];
  const int e = threadIdx.x;  // one thread per expert (E <= 256)
  const int E = a.E, T = a.T, k = a.k;
  const PrefillWs& p = a.ws.pre;
  int cnt = 0;
  if (e < E)
    for (int b = 0; b < nb; ++b) cnt += p.counts[(size_t)b * E + e];
  const int off = block_excl_scan256(cnt, s_wave);
  const int active = cnt > 0;
  const int aidx = block_excl_scan256(active, s_wave);
  const int ntile = (cnt + kMT - 1) / kMT;
  const int tile0 = block_excl_scan256(ntile, s_wave);
  if (e == kThreads - 1) {
    s_tot[0] = aidx + active;
    s_tot[1] = tile0 + ntile;
  }
  // Per (block, expert) base = expert offset + counts of earlier blocks.
  if (e < E) {
    int run = off;
    for (int b = 0; b < nb; ++b) {
      const int c = p.counts[(size_t)b * E + e];
      p.base[(size_t)b * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  int32_t* route = a.ws.route;
  if (active) {
    route[1 + aidx] = e;
    route[1 + E + aidx] = off;
    for (int q = 0; q < ntile; ++q) {
      int32_t* tl = p.tiles + 1 + 3 * (tile0 + q);
      tl[0] = e;
      tl[1] = off + q * kMT;
      tl[2] = min(kMT, cnt - q * kMT);
    }
  }
  if (e == 0) {
    route[0] = s_tot[0];
    route[1 + E + s_tot[0]] = T * k;
    p.tiles[0] = s_tot[1];
  }
}

// ---------------------------------------------------------------- 3. scatter

__global__ __launch_bounds__(kThreads) void prefill_scatter_kernel(LayerArgs a) {
  constexpr int kSlotsMax = kMT * kMaxTopK;        // 512
  constexpr int kWords = kSlotsMax / 32;           // 16
  __shared__ uint32_t occ[kMaxExperts * kWords];  // 16 KiB
  const int T = a.T, E = a.E, k = a.k;
  const int s0 = blockIdx.x * kMT * k;
  const int ns = min(kMT, T - blockIdx.x * kMT) * k;
  const PrefillWs& p = a.ws.pre;
  for (int i = threadIdx.x; i < kMaxExperts * kWords; i += kThreads) occ[i] = 0;
  __syncthreads();
  for (int q = threadIdx.x; q < ns; q += kThreads) {
    const int e = a.ws.ids[s0 + q];
    atomicOr(&occ[e * kWords + (q >> 5)], 1u << (q & 31));
  }
  __syncthreads();
  int32_t* slots = a.ws.route + 2 + 2 * E;
  for (int q = threadIdx.x; q < ns; q += kThreads) {
    const int e = a.ws.ids[s0 + q];
    const uint32_t* m = occ + e * kWords;
    int rank = __popc(m[q >> 5] & ((1u << (q & 31)) - 1u));
    for (int w = 0; w < (q >> 5); ++w) rank += __popc(m[w]);
    const int pos = p.base[(size_t)blockIdx.x * E + e] + rank;
    slots[pos] = s0 + q;
    p.pos[s0 + q] = pos;
  }
}

// ---------------------------------------------------------------- 4. gate/up

// Work items: (shared tiles, then routed tiles) x 4 quarters of the 512 h
// columns; each of the 4 waves owns 32 h columns = 32 gate + 32 up rows.
__global__ __launch_bounds__(kThreads) void prefill_gateup_kernel(LayerArgs a, int n_shared_tiles,
                                                                  int n_items) {
  const int item = xcd_item(n_items);
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, k = a.k, E = a.E;
  const int n_tiles = n_items / 4;
  const int quarter = item / n_tiles;          // column range major: tiles of one expert adjacent
  const int ti = item - quarter * n_tiles;
  const PrefillWs& p = a.ws.pre;
  const int32_t* slots = a.ws.route + 2 + 2 * E;

  const uint8_t* w13;
  int start, count, hrow0;
  bool shared = ti < n_shared_tiles;
  if (shared) {
    start = ti * kMT;
    count = min(kMT, T - start);
    hrow0 = T * k + start;
    w13 = a.shared.w13;
  } else {
    const int rt = ti - n_shared_tiles;
    if (rt >= p.tiles[0]) return;
    const int32_t* tl = p.tiles + 1 + 3 * rt;
    w13 = a.routed.w13 + (size_t)tl[0] * 2 * I * H * 2;
    start = tl[1];
    count = tl[2];
    hrow0 = start;
  }
  const uint16_t* W = reinterpret_cast<const uint16_t*>(w13);
  const int col = quarter * 128 + wave * 32 + (lane & 31);   // h column of this lane
  const uint16_t* ap[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = min(rt * 32 + (lane & 31), count - 1);
    const int tok = shared ? start + r : slots[start + r] / k;
    ap[rt] = a.x + (size_t)tok * H;
  }
  const uint16_t* bp[2] = {W + (size_t)col * H, W + (size_t)(I + col) * H};
  Tile64 tile;
  tile.zero();
  mma_k<H, false>(tile, ap, bp);
  _Float16* h16 = a.ws.pre.h16;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rt * 32 + acc_row(r, lane);
      if (row < count) {
        const float g = tile.acc[rt][0][r], u = tile.acc[rt][1][r];
        h16[(size_t)(hrow0 + row) * I + col] = (_Float16)(silu(g) * u);
      }
    }
}

// ---------------------------------------------------------------- 5. down (routed)

// Work items: 8 eighths of the 2048 output columns x routed tiles; each wave
// owns 64 columns (two 32-column tiles).
__global__ __launch_bounds__(kThreads) void prefill_down_kernel(LayerArgs a, int n_items) {
  const int item = xcd_item(n_items);
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_tiles = n_items / 8;
  const int eighth = item / n_tiles;
  const int ti = item - eighth * n_tiles;
  const PrefillWs& p = a.ws.pre;
  if (ti >= p.tiles[0]) return;
  const int32_t* tl = p.tiles + 1 + 3 * ti;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.routed.w2) + (size_t)tl[0] * H * I;
  const int start = tl[1], count = tl[2];
  const uint16_t* h16 = reinterpret_cast<const uint16_t*>(p.h16);
  const uint16_t* ap[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
    ap[rt] = h16 + (size_t)(start + min(rt * 32 + (lane & 31), count - 1)) * I;
  const int c0 = eighth * 256 + wave * 64;
  const uint16_t* bp[2] = {W + (size_t)(c0 + (lane & 31)) * I, W + (size_t)(c0 + 32 + (lane & 31)) * I};
  Tile64 tile;
  tile.zero();
  mma_k<I, true>(tile, ap, bp);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rt * 32 + acc_row(r, lane);
        if (row < count) p.y32[(size_t)(start + row) * H + c0 + ct * 32 + (lane & 31)] = tile.acc[rt][ct][r];
      }
}

// ---------------------------------------------------------------- 6. shared down + combine

__global__ __launch_bounds__(kThreads) void prefill_shared_combine_kernel(LayerArgs a, int n_items) {
  const int item = xcd_item(n_items);
  if (item >= n_items) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, k = a.k;
  const int n_tiles = n_items / 8;
  const int eighth = item / n_tiles;
  const int ti = item - eighth * n_tiles;
  const PrefillWs& p = a.ws.pre;
  const int t0 = ti * kMT, count = min(kMT, T - t0);
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.shared.w2);
  const uint16_t* h16 = reinterpret_cast<const uint16_t*>(p.h16);
  const uint16_t* ap[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
    ap[rt] = h16 + (size_t)(T * k + t0 + min(rt * 32 + (lane & 31), count - 1)) * I;
  const int c0 = eighth * 256 + wave * 64;
  const uint16_t* bp[2] = {W + (size_t)(c0 + (lane & 31)) * I, W + (size_t)(c0 + 32 + (lane & 31)) * I};
  Tile64 tile;
  tile.zero();
  mma_k<I, true>(tile, ap, bp);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rt * 32 + acc_row(r, lane);
      if (row >= count) continue;
      const int t = t0 + row;
      int pos[kMaxTopK];
      float w[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) {
          pos[j] = p.pos[t * k + j];
          w[j] = a.ws.wts[t * k + j];
        }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int c = c0 + ct * 32 + (lane & 31);
        float o = tile.acc[rt][ct][r];
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
          if (j < k) o = fmaf(w[j], p.y32[(size_t)pos[j] * H + c], o);
        a.out[(size_t)t * H + c] = f32_to_bf16_rne(o);
      }
    }
}

}  // namespace

int prefill_tiles_max(int T, int E, int k) {
  return (T * k + kMT - 1) / kMT + E;  // sum over experts of ceil(count / 64)
}

hipError_t launch_prefill(const LayerArgs& a, hipStream_t stream, Launcher& launch) {
  const int nb = (a.T + kMT - 1) / kMT;
  const int n_routed_max = prefill_tiles_max(a.T, a.E, a.k);
  const int n_shared = nb;
  launch(prefill_router_kernel, dim3(nb), dim3(kThreads), stream, a);
  launch(prefill_scan_kernel, dim3(1), dim3(kThreads), stream, a, nb);
  launch(prefill_scatter_kernel, dim3(nb), dim3(kThreads), stream, a);
  const int n_gu = (n_shared + n_routed_max) * 4;
  launch(prefill_gateup_kernel, dim3(round8(n_gu)), dim3(kThreads), stream, a, n_shared, n_gu);
  const int n_dn = n_routed_max * 8;
  launch(prefill_down_kernel, dim3(round8(n_dn)), dim3(kThreads), stream, a, n_dn);
  const int n_sc = n_shared * 8;
  launch(prefill_shared_combine_kernel, dim3(round8(n_sc)), dim3(kThreads), stream, a, n_sc);
  return hipGetLastError();
}

}  // namespace flint
