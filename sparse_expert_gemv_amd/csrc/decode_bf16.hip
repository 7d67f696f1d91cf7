// Decode-sized (T <= 64) bf16 path of the Flint MoE layer on gfx950: the
// whole layer in one launch.
//
// The layer is cut into work items of ~64 KiB of weights each, in an order
// where an item only ever waits for items before it:
//   router    (token t, 16 router rows)   T * ceil(E/16) items
//   shared    (8 gate/up row pairs of the shared expert, all T tokens)  64
//   gate/up   (active expert a, 8 row pairs)   max|U| * 64
//   down      (expert, 64 output rows): the shared expert first, then each
//             active expert                   (1 + max|U|) * 32
// Block b takes items b, b + G, b + 2G, ... (G = resident blocks), so the
// phases overlap: the shared expert streams while tokens are routed, the
// down rows of early experts stream while later experts finish gate/up.
// Hand-offs between blocks use completion counters in the workspace header
// and coherent (write-through) stores/loads, never whole-cache flushes:
//   - the last router item of token t picks its top-k; the last token to
//     finish buckets every (token, rank) slot by expert into the routing
//     table (U ascending, slots grouped by expert in ascending slot order)
//     and raises the routed flag;
//   - each block reads the routing table once into LDS;
//   - gate/up item (a, .) needs the table; 64 finished items of active
//     expert a complete its h;
//   - down item (a, tile) issues its weight loads, then waits for expert a's
//     h and writes y for its rows; the last of the |U| + 1 down items of a
//     tile combines it: out = y_shared + sum_j w_j y_j in a fixed order,
//     rounded once to bf16;
//   - the last block to run out of items resets every counter to zero.
// Every wait is bounded; a timeout sets an error word instead of hanging.
//
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
constexpr int kThreads = 256;
constexpr int kVecH = H / 8;                  // 16-byte vectors per H row (256)
constexpr int kVecPerLaneH = kVecH / kWave;   // 4
constexpr int kRouterRowsPerItem = 16;        // 4 waves x 4 rows
constexpr int kPairsPerItem = 8;              // gate/up item: 8 (gate, up) row pairs
constexpr int kUnitsPerExpert = I / kPairsPerItem;  // 64
constexpr int kTileRows = 64;                 // down item: 64 output rows (16 per wave)
constexpr int kRowsPerWave = kTileRows / 4;
constexpr int kTiles = H / kTileRows;         // 32
constexpr int kXChunk = 8;                    // tokens staged in LDS at a time
constexpr uint32_t kSpinLimit = 1u << 18;  // ~0.3 s of polling

static_assert(H % (8 * kWave) == 0, "H must be a multiple of 512");
static_assert(I == 8 * kWave, "down GEMV maps one 16-byte vector of a w2 row per lane");
static_assert(kTiles <= 32, "tile tickets");
static_assert(kDecodeMaxT * kMaxTopK <= 32767 && kMaxExperts <= 32767, "int16 routing table");

struct Plan {
  int G;            // blocks in the grid
  int rg;           // router items per token
  int n_router;     // T * rg
  int g_shared;     // first shared gate/up item
  int g_routed;     // first routed gate/up item
  int d_shared;     // first down item (shared expert)
  int d_routed;     // first routed down item
  int n_items;
  int max_active;   // min(E, T*k)
};

// ---------------------------------------------------------------- waiting

// Thread 0 polls `*p >= target` with a bounded number of sleeps; the value
// it saw is returned to every thread.  A timeout raises the sticky error word.
__device__ __forceinline__ uint32_t block_wait(const uint32_t* p, uint32_t target, uint32_t* err,
                                               int* s_val) {
  if (threadIdx.x == 0) {
    uint32_t it = 0, v;
    while ((v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < target) {
      if (++it == kSpinLimit) {
        __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    *s_val = (int)v;
  }
  __syncthreads();
  const uint32_t v = (uint32_t)*s_val;
  __syncthreads();
  return v;
}

// |U| once routing is done (each block polls one of the replicated flags).
__device__ __forceinline__ int wait_routed(const uint32_t* hdr, uint32_t* err, int* s_val) {
  const uint32_t* flag = hdr + kHdrRouted + (blockIdx.x % kRoutingReplicas) * kLine;
  return (int)block_wait(flag, 1u, err, s_val) - 1;
}

// Every thread drains its stores, then thread 0 adds 1 to *counter.
__device__ __forceinline__ void block_signal(uint32_t* counter) {
  drain_memory_ops();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- gate/up

// Tokens of one gate/up or down item.  Routed: entry j is slot
// s = slots[j] (token s / k, h row s).  Shared: entry j is token j, h row
// base + j.
struct TokenList {
  const int16_t* slots;  // LDS, or nullptr for the shared expert
  int k;
  int base;
  __device__ __forceinline__ int tok(int j) const { return slots ? slots[j] / k : j; }
  __device__ __forceinline__ int hrow(int j) const { return slots ? slots[j] : base + j; }
};

// One block (4 waves) computes h = silu(gate) * up for the row pairs
// [p0, p0 + 8) of one expert, for `count` tokens.  Wave w owns pairs
// p0 + 2w and p0 + 2w + 1: four 4 KiB rows held in registers while the
// tokens' x vectors stream through LDS.
__device__ __forceinline__ void gateup_item(const uint16_t* __restrict__ w13, int p0, int count,
                                            const TokenList& list, const uint16_t* __restrict__ x,
                                            float* h, u32x4* xs) {
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
    for (int q = threadIdx.x; q < n * kVecH; q += kThreads) {
      const int j = q / kVecH;
      const int col = q - j * kVecH;
      xs[q] = reinterpret_cast<const u32x4*>(x + (size_t)list.tok(c0 + j) * H)[col];
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
        store_coherent(hr, silu(acc[0]) * acc[2]);
        store_coherent(hr + 1, silu(acc[1]) * acc[3]);
      }
    }
  }
}

// ---------------------------------------------------------------- routing

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
__device__ void route_token(const LayerArgs& a, int t) {
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
      const int e = isel[j];
      const float w = (a.renormalize ? s[j] / sum : s[j]) * a.routed_scale;
      store_coherent(a.ws.ids + t * k + j, e);
      store_coherent(a.ws.wts + t * k + j, w);
      if (a.ids_out) a.ids_out[t * k + j] = e;
      if (a.wts_out) a.wts_out[t * k + j] = w;
    }
  }
}

// Bucket every (token, rank) slot by expert into the routing table, one
// block of 256 threads.  U is ascending; the slots of one expert are in
// ascending slot order: the rank of slot s among its expert's slots is the
// number of set bits below s in that expert's occupancy mask.
__device__ void build_route_table(const LayerArgs& a, void* smem) {
  constexpr int kMaskWords = kDecodeMaxT * kMaxTopK / 32;  // 16
  int* cnt = reinterpret_cast<int*>(smem);                   // [256]
  int* aoff = cnt + kMaxExperts;                             // [256] offset of expert e
  uint32_t* occ = reinterpret_cast<uint32_t*>(aoff + kMaxExperts);  // [256][16]
  const int E = a.E;
  const int nslots = a.T * a.k;
  const int tid = threadIdx.x;
  int32_t* route = a.ws.route;
  int32_t* r_active = route + 1;
  int32_t* r_off = route + 1 + E;
  int32_t* r_slots = route + 2 + 2 * E;
  for (int i = tid; i < kMaxExperts; i += kThreads) cnt[i] = 0;
  for (int i = tid; i < kMaxExperts * kMaskWords; i += kThreads) occ[i] = 0;
  __syncthreads();
  for (int s = tid; s < nslots; s += kThreads) {
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
    const int ic = wave_incl_scan(sc);
    const int iff = wave_incl_scan(sf);
    int o = ic - sc, act = iff - sf;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      aoff[e] = o;
      if (c[q] > 0) {
        store_coherent(r_active + act, e);
        store_coherent(r_off + act, o);
        ++act;
      }
      o += c[q];
    }
    if (lane == kWave - 1) {
      store_coherent(route, iff);
      store_coherent(r_off + iff, ic);
    }
  }
  __syncthreads();
  for (int s = tid; s < nslots; s += kThreads) {
    const int e = load_coherent(a.ws.ids + s);
    const uint32_t* m = occ + e * kMaskWords;
    int rank = __popc(m[s >> 5] & ((1u << (s & 31)) - 1u));
    for (int w = 0; w < (s >> 5); ++w) rank += __popc(m[w]);
    store_coherent(r_slots + aoff[e] + rank, s);
  }
}

__device__ void router_item(const LayerArgs& a, const Plan& P, int item, int* s_flag, void* smem) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t = item / P.rg;
  const int g = item - t * P.rg;
  const int e0 = g * kRouterRowsPerItem + wave * 4;

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
  uint32_t* hdr = a.ws.header;
  // The last router item of token t sees every logit of t.
  if (!last_block_ticket(hdr + kHdrTokTicket + t * kLine, P.rg, s_flag)) return;
  if (wave == 0) route_token(a, t);
  // The last token to finish sees every token's selection: it builds the
  // routing table, then publishes |U| + 1.
  if (!last_block_ticket(hdr + kHdrTokensDone, a.T, s_flag)) return;
  build_route_table(a, smem);
  drain_memory_ops();
  __syncthreads();
  if (threadIdx.x < kRoutingReplicas) {
    const uint32_t n = (uint32_t)load_coherent(a.ws.route);
    __hip_atomic_store(hdr + kHdrRouted + threadIdx.x * kLine, n + 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- down

// Down item: rows [r0, r0 + 64) of one expert's w2 (wave w: 16 rows, one
// 16-byte vector per row per lane), for each of the expert's slots:
// y[hrow][row] = w2[row] . h[hrow], summed over the 64 lanes in a fixed tree.
// Slots go in chunks of 16: their h rows are staged in LDS with coalesced
// coherent loads, the results collect in LDS and leave as one batch of
// stores, so no load waits behind this item's own write-through stores.
constexpr int kDownChunk = 16;

__device__ __forceinline__ void load_down_weights(u32x4 (&wv)[kRowsPerWave],
                                                  const uint16_t* __restrict__ w2, int r0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rw = r0 + wave * kRowsPerWave;
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
    wv[r] = reinterpret_cast<const u32x4*>(w2 + (size_t)(rw + r) * I)[lane];
}

__device__ __forceinline__ void down_rows(u32x4 (&wv)[kRowsPerWave], int r0, int count,
                                          const TokenList& list, const float* h, float* y,
                                          float* hs, float* ys) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int c0 = 0; c0 < count; c0 += kDownChunk) {
    const int n = min(kDownChunk, count - c0);
    __syncthreads();
    for (int q = threadIdx.x; q < n * I; q += kThreads) {
      const int j = q / I;
      hs[q] = load_coherent(h + (size_t)list.hrow(c0 + j) * I + (q - j * I));
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      // Keep the weights packed across slots: widening all 16 rows to fp32
      // once would cost 128 registers.
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) asm volatile("" : "+v"(wv[r]));
      const f32x4 h0 = *reinterpret_cast<const f32x4*>(hs + j * I + lane * 8);
      const f32x4 h1 = *reinterpret_cast<const f32x4*>(hs + j * I + lane * 8 + 4);
      float acc[kRowsPerWave];
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        float v = bf16_lo(wv[r].x) * h0.x;
        v = fmaf(bf16_hi(wv[r].x), h0.y, v);
        v = fmaf(bf16_lo(wv[r].y), h0.z, v);
        v = fmaf(bf16_hi(wv[r].y), h0.w, v);
        v = fmaf(bf16_lo(wv[r].z), h1.x, v);
        v = fmaf(bf16_hi(wv[r].z), h1.y, v);
        v = fmaf(bf16_lo(wv[r].w), h1.z, v);
        v = fmaf(bf16_hi(wv[r].w), h1.w, v);
        acc[r] = wave_sum_lane63(v);
      }
      if (lane == kWave - 1)
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) ys[j * kTileRows + wave * kRowsPerWave + r] = acc[r];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < n * kTileRows; q += kThreads) {
      const int j = q / kTileRows;
      store_coherent(y + (size_t)list.hrow(c0 + j) * H + r0 + (q - j * kTileRows), ys[q]);
    }
  }
}

// out rows [r0, r0 + 64) of every token: shared + sum_j w_j * y_j, fixed order.
__device__ void combine_tile(const LayerArgs& a, int r0) {
  const int T = a.T, k = a.k;
  for (int q = threadIdx.x; q < T * kTileRows; q += kThreads) {
    const int t = q / kTileRows;
    const int r = r0 + (q - t * kTileRows);
    float o = load_coherent(a.ws.y + (size_t)(T * k + t) * H + r);
    for (int j = 0; j < k; ++j)
      o = fmaf(load_coherent(a.ws.wts + t * k + j),
               load_coherent(a.ws.y + (size_t)(t * k + j) * H + r), o);
    a.out[(size_t)t * H + r] = f32_to_bf16_rne(o);
  }
}

// ---------------------------------------------------------------- kernel

// The routing table, copied once per block into LDS.
struct RouteLds {
  int n;                              // |U|, or -1 before the block has read it
  int16_t active[kMaxExperts];
  int16_t off[kMaxExperts + 1];
  int16_t slots[kDecodeMaxT * kMaxTopK];
};

__device__ __forceinline__ void ensure_routes(const LayerArgs& a, RouteLds& rt, uint32_t* err,
                                              int* s_val) {
  if (rt.n >= 0) return;  // block-uniform
  const int n = wait_routed(a.ws.header, err, s_val);
  const int E = a.E, ns = a.T * a.k;
  const int32_t* route = a.ws.route;
  for (int q = threadIdx.x; q < n; q += kThreads) rt.active[q] = (int16_t)load_coherent(route + 1 + q);
  for (int q = threadIdx.x; q <= n; q += kThreads) rt.off[q] = (int16_t)load_coherent(route + 1 + E + q);
  for (int q = threadIdx.x; q < ns; q += kThreads) rt.slots[q] = (int16_t)load_coherent(route + 2 + 2 * E + q);
  if (threadIdx.x == 0) rt.n = n;
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void moe_decode_kernel(LayerArgs a, Plan P) {
  __shared__ u32x4 xs[kXChunk * kVecH];   // 32 KiB: x staging (gate/up), h staging (down),
                                          // bucketing tables (routing)
  __shared__ float ys[kDownChunk * kTileRows];
  __shared__ RouteLds rt;
  __shared__ int s_flag, s_val;
  uint32_t* hdr = a.ws.header;
  uint32_t* err = hdr + kHdrError;
  const int T = a.T, k = a.k;
  if (threadIdx.x == 0) rt.n = -1;
  __syncthreads();

  for (int item = blockIdx.x; item < P.n_items; item += P.G) {
    if (item < P.n_router) {
      router_item(a, P, item, &s_flag, xs);
    } else if (item < P.g_routed) {
      // Shared expert gate/up: all T tokens, h rows T*k + t.
      const int unit = item - P.g_shared;
      gateup_item(reinterpret_cast<const uint16_t*>(a.shared.w13), unit * kPairsPerItem, T,
                  TokenList{nullptr, k, T * k}, a.x, a.ws.h, xs);
      block_signal(hdr + kHdrSharedDone);
    } else if (item < P.d_shared) {
      // Routed gate/up: active index ai, unit.
      const int ai = (item - P.g_routed) / kUnitsPerExpert;
      const int unit = (item - P.g_routed) - ai * kUnitsPerExpert;
      ensure_routes(a, rt, err, &s_val);
      if (ai >= rt.n) continue;
      const int e = rt.active[ai];
      const uint16_t* w13 = reinterpret_cast<const uint16_t*>(a.routed.w13) + (size_t)e * 2 * I * H;
      gateup_item(w13, unit * kPairsPerItem, rt.off[ai + 1] - rt.off[ai],
                  TokenList{rt.slots + rt.off[ai], k, 0}, a.x, a.ws.h, xs);
      block_signal(hdr + kHdrExpertDone + ai * kLine);
    } else {
      // Down: (expert, 64-row tile); the shared expert's tiles come first.
      const int di = item - P.d_shared;
      const int ei = di / kTiles;          // 0: shared, 1 + ai: active index ai
      const int tile = di - ei * kTiles;
      ensure_routes(a, rt, err, &s_val);
      const int ai = ei - 1;
      if (ai >= rt.n) continue;
      u32x4 wv[kRowsPerWave];
      TokenList list{nullptr, k, T * k};
      int cnt = T;
      if (ei == 0) {
        load_down_weights(wv, reinterpret_cast<const uint16_t*>(a.shared.w2), tile * kTileRows);
        block_wait(hdr + kHdrSharedDone, (uint32_t)kUnitsPerExpert, err, &s_val);
      } else {
        const int e = rt.active[ai];
        load_down_weights(wv, reinterpret_cast<const uint16_t*>(a.routed.w2) + (size_t)e * H * I,
                          tile * kTileRows);
        list.slots = rt.slots + rt.off[ai];
        cnt = rt.off[ai + 1] - rt.off[ai];
        block_wait(hdr + kHdrExpertDone + ai * kLine, (uint32_t)kUnitsPerExpert, err, &s_val);
      }
      down_rows(wv, tile * kTileRows, cnt, list, a.ws.h, a.ws.y, reinterpret_cast<float*>(xs), ys);
      // The last of the |U| + 1 down items of this tile combines it.
      if (last_block_ticket(hdr + kHdrTileTicket + tile * kLine, (uint32_t)(rt.n + 1), &s_flag))
        combine_tile(a, tile * kTileRows);
    }
  }

  // The last block to finish resets the per-forward counters.
  if (!last_block_ticket(hdr + kHdrExit, (uint32_t)P.G, &s_flag)) return;
  const int n_active = load_coherent(a.ws.route);
  for (int i = threadIdx.x; i < n_active; i += kThreads)
    __hip_atomic_store(hdr + kHdrExpertDone + i * kLine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x < kRoutingReplicas)
    __hip_atomic_store(hdr + kHdrRouted + threadIdx.x * kLine, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0)
    __hip_atomic_store(hdr + kHdrSharedDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int decode_grid_limit() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, moe_decode_kernel, kThreads, 0) !=
      hipSuccess)
    return 0;
  return cus * min(per_cu, 4);
}

hipError_t launch_decode_bf16(const LayerArgs& a, int grid_limit, hipStream_t stream,
                              StageEvents* ev) {
  Plan P;
  P.rg = (a.E + kRouterRowsPerItem - 1) / kRouterRowsPerItem;
  P.n_router = a.T * P.rg;
  P.max_active = min(a.E, a.T * a.k);
  P.g_shared = P.n_router;
  P.g_routed = P.g_shared + kUnitsPerExpert;
  P.d_shared = P.g_routed + P.max_active * kUnitsPerExpert;
  P.d_routed = P.d_shared + kTiles;
  P.n_items = P.d_routed + P.max_active * kTiles;
  P.G = min(P.n_items, grid_limit);
  StageEvents none;
  StageEvents& e = ev ? *ev : none;
  e.mark(stream);
  hipLaunchKernelGGL(moe_decode_kernel, dim3(P.G), dim3(kThreads), 0, stream, a, P);
  e.mark(stream);
  return hipGetLastError();
}

}  // namespace flint
