// Decode-sized (T <= 64) bf16 path of the Flint MoE layer on gfx950.
//
// Three launches on the caller's stream:
//   1. router_topk_shared : router GEMV (bf16 x bf16 -> fp32) for every token;
//      the last router block of a token picks its top-k by sigmoid score and
//      writes the routing weights; the last token to finish buckets all
//      (token, rank) slots by expert.  Extra blocks of the same launch run the
//      shared expert's gate/up GEMV, which needs nothing but x.
//   2. gateup_routed      : fused gate/up GEMV + SiLU-and-mul over the union
//      of selected experts; each expert's 4 MiB of w13 rows is streamed once
//      for all of its tokens.
//   3. down_combine       : down GEMV of every active expert and the shared
//      expert; each block owns 8 output rows, scales by the routing weights
//      and reduces across experts in a fixed order (no atomics), then rounds
//      once to bf16.
// What is computed follows "vLLM Day-0 Support for Recursive's Flint"
// (section "Flint Model Architecture", bullet "MoE Structure"; section
// "Optimization Strategies", bullets "Small-batch MoE Kernels" and
// "Low-Latency Decode Path") and the SiLU form of "Flint on Arc Pro B70"
// (section "norm.py: Triton kernels that assumed CUDA").

#include "flint_device.h"
#include "flint_kernels.h"

namespace flint {
namespace {

constexpr int H = kHidden;
constexpr int I = kInter;
constexpr int kVecH = H / 8;                  // 16-byte vectors per H row (256)
constexpr int kVecPerLaneH = kVecH / kWave;   // 4
constexpr int kRouterRowsPerBlock = 16;       // 4 waves x 4 rows
constexpr int kPairsPerBlock = 8;             // gate/up unit: 8 (gate, up) row pairs
constexpr int kUnitsPerExpert = I / kPairsPerBlock;  // 64
constexpr int kXChunk = 8;                    // tokens staged in LDS at a time
constexpr int kDownRows = 8;                  // output rows per down block
constexpr int kDownThreads = 512;

static_assert(H % (8 * kWave) == 0, "H must be a multiple of 512");
static_assert(I == 8 * kWave, "down GEMV maps one 16-byte vector of a w2 row per lane");

// Slot list of one routed expert: entry j is slot s = t*k + rank.
struct RoutedList {
  const int32_t* slots;
  int k;
  __device__ int token(int j) const { return slots[j] / k; }
  __device__ int hrow(int j) const { return slots[j]; }
};

// All T tokens of the shared expert; h rows follow the T*k routed rows.
struct SharedList {
  int base;
  __device__ int token(int j) const { return j; }
  __device__ int hrow(int j) const { return base + j; }
};

// One block (4 waves) computes h = silu(gate) * up for the row pairs
// [p0, p0 + 8) of one expert, for `count` tokens.  Wave w owns pairs
// p0 + 2w and p0 + 2w + 1: four 4 KiB rows held in registers while the
// tokens' x vectors stream through LDS.
template <class List>
__device__ __forceinline__ void gateup_block(const uint16_t* __restrict__ w13, int p0, int count,
                                             const List& list, const uint16_t* __restrict__ x,
                                             float* __restrict__ h, u32x4* xs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int p = p0 + 2 * wave;
  const u32x4* rows[4] = {
      reinterpret_cast<const u32x4*>(w13 + (size_t)p * H),
      reinterpret_cast<const u32x4*>(w13 + (size_t)(p + 1) * H),
      reinterpret_cast<const u32x4*>(w13 + (size_t)(I + p) * H),
      reinterpret_cast<const u32x4*>(w13 + (size_t)(I + p + 1) * H)};
  u32x4 wv[4][kVecPerLaneH];
#pragma unroll
  for (int i = 0; i < kVecPerLaneH; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[r][i] = rows[r][lane + i * kWave];

  for (int c0 = 0; c0 < count; c0 += kXChunk) {
    const int n = min(kXChunk, count - c0);
    __syncthreads();
    for (int q = threadIdx.x; q < n * kVecH; q += blockDim.x) {
      const int j = q / kVecH;
      const int col = q - j * kVecH;
      xs[q] = reinterpret_cast<const u32x4*>(x + (size_t)list.token(c0 + j) * H)[col];
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kVecPerLaneH; ++i) {
        const u32x4 xv = xs[j * kVecH + lane + i * kWave];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = dot8_bf16(wv[r][i], xv, acc[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = wave_sum_lane63(acc[r]);
      if (lane == kWave - 1) {
        float* hr = h + (size_t)list.hrow(c0 + j) * I + p;
        hr[0] = silu(acc[0]) * acc[2];
        hr[1] = silu(acc[1]) * acc[3];
      }
    }
  }
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ord_f32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Top-k of token t by score, one wave.  Ranks on the logit (the sigmoid is
// strictly increasing), ties to the lower expert index: key = (logit, ~e).
// Logits were written by other blocks of this launch: coherent loads.
__device__ void topk_token(const LayerArgs& a, int t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int E = a.E, k = a.k;
  uint64_t key[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    key[q] = 0;
    if (e < E) {
      const float z = load_coherent(a.ws.logits + (size_t)t * E + e);
      key[q] = ((uint64_t)ord_f32(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
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
  float s[kMaxTopK];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    s[j] = sigmoid(zsel[j]);
    if (j < k) sum += s[j];
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && lane == j) {
      const float w = (a.renormalize ? s[j] / sum : s[j]) * a.routed_scale;
      store_coherent(a.ws.ids + t * k + j, isel[j]);
      store_coherent(a.ws.wts + t * k + j, w);
      if (a.ids_out) a.ids_out[t * k + j] = isel[j];
      if (a.wts_out) a.wts_out[t * k + j] = w;
    }
  }
}

// Bucket every (token, rank) slot by expert, 256 threads.  Slots of one
// expert are placed in ascending slot order: the rank of slot s among its
// expert's slots is the number of set bits below s in that expert's
// occupancy mask.
__device__ void bucket_all(const LayerArgs& a, void* smem) {
  constexpr int kMaskWords = kDecodeMaxT * kMaxTopK / 32;  // 16
  int* cnt = reinterpret_cast<int*>(smem);                   // [256]
  int* off = cnt + kMaxExperts;                              // [256]
  uint32_t* occ = reinterpret_cast<uint32_t*>(off + kMaxExperts);  // [256][16]
  const int E = a.E;
  const int nslots = a.T * a.k;
  const int tid = threadIdx.x;
  for (int i = tid; i < kMaxExperts; i += blockDim.x) cnt[i] = 0;
  for (int i = tid; i < kMaxExperts * kMaskWords; i += blockDim.x) occ[i] = 0;
  __syncthreads();
  for (int s = tid; s < nslots; s += blockDim.x) {
    const int e = load_coherent(a.ws.ids + s);
    atomicAdd(&cnt[e], 1);
    atomicOr(&occ[e * kMaskWords + (s >> 5)], 1u << (s & 31));
  }
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    int c[4], sc = 0, sf = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      c[q] = e < E ? cnt[e] : 0;
      sc += c[q];
      sf += c[q] > 0;
    }
    const int ic = wave_incl_scan(sc);   // inclusive scans over lanes
    const int iff = wave_incl_scan(sf);
    int o = ic - sc, act = iff - sf;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) {
        a.ws.counts[e] = c[q];
        a.ws.offsets[e] = o;
        off[e] = o;
        if (c[q] > 0) a.ws.active[act++] = e;
        o += c[q];
      }
    }
    if (lane == kWave - 1) {
      a.ws.offsets[E] = ic;
      *a.ws.n_active = iff;
    }
  }
  __syncthreads();
  for (int s = tid; s < nslots; s += blockDim.x) {
    const int e = load_coherent(a.ws.ids + s);
    const uint32_t* m = occ + e * kMaskWords;
    int rank = __popc(m[s >> 5] & ((1u << (s & 31)) - 1u));
    for (int w = 0; w < (s >> 5); ++w) rank += __popc(m[w]);
    a.ws.slots[off[e] + rank] = s;
  }
}

__global__ __launch_bounds__(256) void router_topk_shared_kernel(LayerArgs a, int n_router_blocks,
                                                                 int blocks_per_token) {
  __shared__ u32x4 smem[kXChunk * kVecH];  // 32 KiB: x staging or bucketing tables
  __shared__ int s_last;

  if ((int)blockIdx.x >= n_router_blocks) {
    const int unit = blockIdx.x - n_router_blocks;
    gateup_block(reinterpret_cast<const uint16_t*>(a.shared.w13), unit * kPairsPerBlock, a.T,
                 SharedList{a.T * a.k}, a.x, a.ws.h, smem);
    return;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t = blockIdx.x / blocks_per_token;
  const int g = blockIdx.x - t * blocks_per_token;
  const int e0 = g * kRouterRowsPerBlock + wave * 4;

  const u32x4* xr = reinterpret_cast<const u32x4*>(a.x + (size_t)t * H);
  u32x4 xv[kVecPerLaneH];
  u32x4 wv[4][kVecPerLaneH];
#pragma unroll
  for (int i = 0; i < kVecPerLaneH; ++i) xv[i] = xr[lane + i * kWave];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = min(e0 + r, a.E - 1);
    const u32x4* row = reinterpret_cast<const u32x4*>(a.router_w + (size_t)e * H);
#pragma unroll
    for (int i = 0; i < kVecPerLaneH; ++i) wv[r][i] = row[lane + i * kWave];
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kVecPerLaneH; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = dot8_bf16(wv[r][i], xv[i], acc[r]);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    acc[r] = wave_sum_lane63(acc[r]);
    const int e = e0 + r;
    if (lane == kWave - 1 && e < a.E)
      store_coherent(a.ws.logits + (size_t)t * a.E + e,
                     acc[r] + (a.router_b ? a.router_b[e] : 0.f));
  }
  // The last router block of token t sees every logit of t.
  if (!last_block_ticket(&a.ws.header[kTokCounterBase + t], blocks_per_token, &s_last)) return;
  if (wave == 0) topk_token(a, t);
  // The last token to finish sees every token's selection.
  if (!last_block_ticket(&a.ws.header[0], a.T, &s_last)) return;
  bucket_all(a, smem);
}

__global__ __launch_bounds__(256) void gateup_routed_kernel(LayerArgs a) {
  __shared__ u32x4 xs[kXChunk * kVecH];
  const int ai = blockIdx.x / kUnitsPerExpert;
  const int unit = blockIdx.x - ai * kUnitsPerExpert;
  if (ai >= *a.ws.n_active) return;
  const int e = a.ws.active[ai];
  const int off = a.ws.offsets[e];
  const int cnt = a.ws.counts[e];
  const uint16_t* w13 = reinterpret_cast<const uint16_t*>(a.routed.w13) + (size_t)e * 2 * I * H;
  gateup_block(w13, unit * kPairsPerBlock, cnt, RoutedList{a.ws.slots + off, a.k}, a.x, a.ws.h, xs);
}

// The w2 rows [r0, r0 + 8) of one item (an active expert, or the shared
// expert as the last item): one 16-byte vector per row per lane.
struct DownItem {
  const uint16_t* w2;
  const int32_t* list;  // routed: slot ids; shared: nullptr (tokens 0..T-1)
  int cnt;
};

__device__ __forceinline__ DownItem down_item(const LayerArgs& a, int item, int nA) {
  DownItem it;
  if (item < nA) {
    const int e = a.ws.active[item];
    it.w2 = reinterpret_cast<const uint16_t*>(a.routed.w2) + (size_t)e * H * I;
    it.list = a.ws.slots + a.ws.offsets[e];
    it.cnt = a.ws.counts[e];
  } else {
    it.w2 = reinterpret_cast<const uint16_t*>(a.shared.w2);
    it.list = nullptr;
    it.cnt = a.T;
  }
  return it;
}

__device__ __forceinline__ void load_rows(u32x4 (&wv)[kDownRows], const uint16_t* w2, int r0,
                                          int lane) {
#pragma unroll
  for (int r = 0; r < kDownRows; ++r)
    wv[r] = reinterpret_cast<const u32x4*>(w2 + (size_t)(r0 + r) * I)[lane];
}

// Each block owns output rows [r0, r0 + 8).  Waves take the items (active
// experts, then the shared expert) round-robin, keeping the next item's rows
// in flight while the current one is reduced.  Per (slot, row) the 64-lane
// partial dot products are summed in a fixed tree and parked in LDS; the
// block then combines shared + sum_j w_j * routed_j in a fixed order.
__global__ __launch_bounds__(kDownThreads) void down_combine_kernel(LayerArgs a) {
  __shared__ float part[(kMaxTopK + 1) * kDecodeMaxT * kDownRows];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  constexpr int kWaves = kDownThreads / kWave;
  const int r0 = blockIdx.x * kDownRows;
  const int T = a.T, k = a.k;
  const int nA = *a.ws.n_active;

  int item = wave;
  u32x4 cur[kDownRows], nxt[kDownRows];
  DownItem it{}, it_next{};
  if (item <= nA) {
    it_next = down_item(a, item, nA);
    load_rows(nxt, it_next.w2, r0, lane);
  }
  for (; item <= nA; item += kWaves) {
    it = it_next;
#pragma unroll
    for (int r = 0; r < kDownRows; ++r) cur[r] = nxt[r];
    if (item + kWaves <= nA) {
      it_next = down_item(a, item + kWaves, nA);
      load_rows(nxt, it_next.w2, r0, lane);
    }
    for (int j = 0; j < it.cnt; ++j) {
      const int hrow = it.list ? it.list[j] : T * k + j;
      const f32x4* hp = reinterpret_cast<const f32x4*>(a.ws.h + (size_t)hrow * I) + lane * 2;
      const f32x4 h0 = hp[0], h1 = hp[1];
      float acc[kDownRows];
#pragma unroll
      for (int r = 0; r < kDownRows; ++r) {
        float v = bf16_lo(cur[r].x) * h0.x;
        v = fmaf(bf16_hi(cur[r].x), h0.y, v);
        v = fmaf(bf16_lo(cur[r].y), h0.z, v);
        v = fmaf(bf16_hi(cur[r].y), h0.w, v);
        v = fmaf(bf16_lo(cur[r].z), h1.x, v);
        v = fmaf(bf16_hi(cur[r].z), h1.y, v);
        v = fmaf(bf16_lo(cur[r].w), h1.z, v);
        v = fmaf(bf16_hi(cur[r].w), h1.w, v);
        acc[r] = wave_sum_lane63(v);
      }
      if (lane == kWave - 1)
#pragma unroll
        for (int r = 0; r < kDownRows; ++r) part[hrow * kDownRows + r] = acc[r];
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < T * kDownRows; q += kDownThreads) {
    const int t = q / kDownRows;
    const int r = q - t * kDownRows;
    float o = part[(T * k + t) * kDownRows + r];
    for (int j = 0; j < k; ++j) o = fmaf(a.ws.wts[t * k + j], part[(t * k + j) * kDownRows + r], o);
    a.out[(size_t)t * H + r0 + r] = f32_to_bf16_rne(o);
  }
}

}  // namespace

hipError_t launch_decode_bf16(const LayerArgs& a, hipStream_t stream, StageEvents* ev) {
  StageEvents none;
  StageEvents& e = ev ? *ev : none;
  const int bpt = (a.E + kRouterRowsPerBlock - 1) / kRouterRowsPerBlock;
  const int n_router = a.T * bpt;
  e.mark(stream);
  hipLaunchKernelGGL(router_topk_shared_kernel, dim3(n_router + kUnitsPerExpert), dim3(256), 0,
                     stream, a, n_router, bpt);
  const int max_active = min(a.E, a.T * a.k);
  e.mark(stream);
  hipLaunchKernelGGL(gateup_routed_kernel, dim3(max_active * kUnitsPerExpert), dim3(256), 0, stream,
                     a);
  e.mark(stream);
  hipLaunchKernelGGL(down_combine_kernel, dim3(H / kDownRows), dim3(kDownThreads), 0, stream, a);
  e.mark(stream);
  return hipGetLastError();
}

}  // namespace flint
