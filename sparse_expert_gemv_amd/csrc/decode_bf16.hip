// Decode-sized (T <= 64) bf16 path of the Flint MoE layer on gfx950.
//
// Three launches on the caller's stream, each cut into blocks that move
// ~64 KiB of weights:
//   1. route   : router GEMV, 16 rows x one token per block.  The last block
//                of a token picks its top-k by sigmoid score; the last token
//                to finish buckets every (token, rank) slot by expert into
//                the routing table (U ascending, slots grouped by expert in
//                ascending slot order).  Extra blocks of the same launch run
//                the shared expert's gate/up GEMV, which needs only x.
//   2. gate/up : (active expert a, 8 gate/up row pairs) per block: the rows
//                are streamed once for all of a's tokens; SiLU-and-mul in
//                registers; h stays fp32.
//   3. down    : (expert, 64 output rows) per block, the shared expert
//                included: y = w2 rows . h for each of the expert's slots;
//                the last of the |U| + 1 blocks of a row tile combines it:
//                out = y_shared + sum_j w_j y_j in a fixed order, rounded once
//                to bf16.
// Hand-offs inside a launch use completion tickets in the workspace header
// and coherent (write-through) stores/loads, never whole-cache flushes;
// between launches the stream order is enough.
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
constexpr int kXChunk = 4;                    // tokens staged in LDS at a time (16 KiB)

static_assert(H % (8 * kWave) == 0, "H must be a multiple of 512");
static_assert(I == 8 * kWave, "down GEMV maps one 16-byte vector of a w2 row per lane");
static_assert(kTiles <= 32, "tile tickets");
static_assert(kDecodeMaxT * kMaxTopK <= 32767 && kMaxExperts <= 32767, "int16 routing table");

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
        hr[0] = silu(acc[0]) * acc[2];
        hr[1] = silu(acc[1]) * acc[3];
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

__device__ void router_block(const LayerArgs& a, int rg, int item, int* s_flag, void* smem) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t = item / rg;
  const int g = item - t * rg;
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
  if (!last_block_ticket(hdr + kHdrTokTicket + t * kLine, rg, s_flag)) return;
  if (wave == 0) route_token(a, t);
  // The last token to finish sees every token's selection: it builds the
  // routing table (read by the next launches).
  if (!last_block_ticket(hdr + kHdrTokensDone, a.T, s_flag)) return;
  build_route_table(a, smem);
}

// ---------------------------------------------------------------- down

// Down item: rows [r0, r0 + 64) of one expert's w2 (wave w: 16 rows, one
// 16-byte vector per row per lane), for each of the expert's slots:
// y[hrow][row] = w2[row] . h[hrow], summed over the 64 lanes in a fixed tree.
// Slots go in chunks of 16: their h rows are staged in LDS with coalesced
// loads, the results collect in LDS and leave as one batch of coherent
// stores (the tile's combining block reads them in this launch).
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
      hs[q] = h[(size_t)list.hrow(c0 + j) * I + (q - j * I)];
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
      o = fmaf(a.ws.wts[t * k + j], load_coherent(a.ws.y + (size_t)(t * k + j) * H + r), o);
    a.out[(size_t)t * H + r] = f32_to_bf16_rne(o);
  }
}

// ---------------------------------------------------------------- kernel

// ---------------------------------------------------------------- kernels

// LDS of the route kernel: x staging, or the bucketing tables (counts,
// offsets and 16-word occupancy masks of 256 experts).
constexpr int kRouteLdsVec = (2 * kMaxExperts * 4 + kMaxExperts * (kDecodeMaxT * kMaxTopK / 32) * 4) / 16;
static_assert(kRouteLdsVec >= kXChunk * kVecH, "route LDS holds the x staging");

__global__ __launch_bounds__(kThreads) void route_kernel(LayerArgs a, int rg, int n_router) {
  __shared__ u32x4 xs[kRouteLdsVec];
  __shared__ int s_flag;
  if ((int)blockIdx.x < n_router) {
    router_block(a, rg, blockIdx.x, &s_flag, xs);
  } else {
    // Shared expert gate/up: all T tokens, h rows T*k + t.
    const int unit = blockIdx.x - n_router;
    gateup_item(reinterpret_cast<const uint16_t*>(a.shared.w13), unit * kPairsPerItem, a.T,
                TokenList{nullptr, a.k, a.T * a.k}, a.x, a.ws.h, xs);
  }
}

// Slots of active expert ai (its count returned), copied from the routing
// table into LDS; -1 if ai is not an active index.
__device__ __forceinline__ int load_expert_slots(const LayerArgs& a, int ai, int16_t* s_slots,
                                                 int* s_meta) {
  const int32_t* route = a.ws.route;
  const int E = a.E;
  if (threadIdx.x == 0) {
    const int n = route[0];
    s_meta[0] = n;
    if (ai < n) {
      s_meta[1] = route[1 + ai];
      s_meta[2] = route[1 + E + ai];
      s_meta[3] = route[1 + E + ai + 1];
    }
  }
  __syncthreads();
  if (ai >= s_meta[0]) return -1;
  const int off = s_meta[2], cnt = s_meta[3] - s_meta[2];
  for (int q = threadIdx.x; q < cnt; q += kThreads) s_slots[q] = (int16_t)route[2 + 2 * E + off + q];
  __syncthreads();
  return cnt;
}

__global__ __launch_bounds__(kThreads) void gateup_kernel(LayerArgs a) {
  __shared__ u32x4 xs[kXChunk * kVecH];
  __shared__ int16_t s_slots[kDecodeMaxT];
  __shared__ int s_meta[4];
  const int ai = blockIdx.x / kUnitsPerExpert;
  const int unit = blockIdx.x - ai * kUnitsPerExpert;
  const int cnt = load_expert_slots(a, ai, s_slots, s_meta);
  if (cnt < 0) return;
  const int e = s_meta[1];
  const uint16_t* w13 = reinterpret_cast<const uint16_t*>(a.routed.w13) + (size_t)e * 2 * I * H;
  gateup_item(w13, unit * kPairsPerItem, cnt, TokenList{s_slots, a.k, 0}, a.x, a.ws.h, xs);
}

__global__ __launch_bounds__(kThreads) void down_kernel(LayerArgs a) {
  __shared__ float hs[kDownChunk * I];     // 32 KiB: h staging
  __shared__ float ys[kDownChunk * kTileRows];
  __shared__ int16_t s_slots[kDecodeMaxT];
  __shared__ int s_meta[4];
  __shared__ int s_flag;
  const int ei = blockIdx.x / kTiles;      // 0: shared expert, 1 + ai: active index ai
  const int tile = blockIdx.x - ei * kTiles;
  const int T = a.T, k = a.k;
  u32x4 wv[kRowsPerWave];
  TokenList list{nullptr, k, T * k};
  int cnt = T;
  if (ei == 0) {
    load_down_weights(wv, reinterpret_cast<const uint16_t*>(a.shared.w2), tile * kTileRows);
    if (threadIdx.x == 0) s_meta[0] = a.ws.route[0];
    __syncthreads();
  } else {
    cnt = load_expert_slots(a, ei - 1, s_slots, s_meta);
    if (cnt < 0) return;
    load_down_weights(wv, reinterpret_cast<const uint16_t*>(a.routed.w2) + (size_t)s_meta[1] * H * I,
                      tile * kTileRows);
    list.slots = s_slots;
  }
  const int n_active = s_meta[0];
  down_rows(wv, tile * kTileRows, cnt, list, a.ws.h, a.ws.y, hs, ys);
  // The last of the |U| + 1 blocks of this row tile combines it.
  if (last_block_ticket(a.ws.header + kHdrTileTicket + tile * kLine, (uint32_t)(n_active + 1), &s_flag))
    combine_tile(a, tile * kTileRows);
}

}  // namespace

hipError_t launch_decode_bf16(const LayerArgs& a, hipStream_t stream, StageEvents* ev) {
  StageEvents none;
  StageEvents& e = ev ? *ev : none;
  const int rg = (a.E + kRouterRowsPerItem - 1) / kRouterRowsPerItem;
  const int n_router = a.T * rg;
  const int max_active = min(a.E, a.T * a.k);
  e.mark(stream);
  hipLaunchKernelGGL(route_kernel, dim3(n_router + kUnitsPerExpert), dim3(kThreads), 0, stream, a, rg,
                     n_router);
  e.mark(stream);
  hipLaunchKernelGGL(gateup_kernel, dim3(max_active * kUnitsPerExpert), dim3(kThreads), 0, stream, a);
  e.mark(stream);
  hipLaunchKernelGGL(down_kernel, dim3((1 + max_active) * kTiles), dim3(kThreads), 0, stream, a);
  e.mark(stream);
  return hipGetLastError();
}

}  // namespace flint
