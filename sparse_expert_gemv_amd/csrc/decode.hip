// Decode-sized (T <= 64) path of the Flint MoE layer on gfx950, for bf16 and
// NVFP4 (W4A16) expert weights.
//
// Three launches on the caller's stream:
//   1. route   : router GEMV over 64 blocks of four expert rows each (4
//                waves, one row each, plus 4 waves that only rank tokens
//                for the bare layer's ticketed routing at T <= 8; for the
//                pre-norm block every block normalises the rows it stages,
//                block 0 storing them; bare layer with T > 8: 16 waves,
//                each all four rows for its tokens).
//                The last block to finish picks every token's top-k by
//                sigmoid score (a wave per token), computes the routing
//                weights and buckets every (token, rank) slot by expert into
//                the routing table (U ascending, slots grouped by expert in
//                ascending slot order).  For small batches (T <= 4,
//                T * k <= 16) the launch ends with the logits and every
//                routed gate/up block routes the batch itself.
//   2. gate/up : 64 blocks for the shared expert (first, so that they stream
//                from the start: they need no routing), then (active expert
//                a, 8 gate/up row pairs) per block; the rows are streamed
//                once for all of the expert's tokens; SiLU-and-mul in
//                registers; h stays fp32 for bf16 weights and is stored
//                as bf16 for NVFP4 (W4A16: 16-bit activations).
//   3. down    : 8 output rows of every token per block, over the shared
//                expert and the |U| active experts, each expert's w2 rows
//                read once; the partial dot products meet in LDS and combine
//                as out = shared + sum_j w_j * routed_j (+ r for the
//                pre-norm block) in a fixed order, rounded once to bf16.
//                NVFP4 with 2 <= T <= 8: down_small_kernel, the same blocks
//                with each wave's share of the table read into registers,
//                the h rows parked in LDS and all of the wave's experts'
//                codes in flight at once.
// The one hand-off inside a launch (router blocks -> routing block) uses a
// completion ticket in the workspace header and coherent (write-through)
// stores/loads, never whole-cache flushes; between launches the stream
// order is enough.

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
constexpr int kRouteWaves = kThreads / kWave;
constexpr int kRouterRows = kRouteWaves;      // router: one expert row per wave
constexpr int kRouteXChunk = 8;               // tokens staged in LDS at a time (32 KiB), pre-norm block
constexpr int kRouteBareMinT = 8;            // larger bare-layer batches: the 16-wave router
constexpr int kRouteBareThreads = 1024;       // bare-layer router: 16 waves per block
constexpr int kRouteBareWaves = kRouteBareThreads / kWave;
constexpr int kRouteBareXChunk = 32;          // tokens staged in LDS at a time (128 KiB), bare layer
constexpr int kPairsPerItem = 8;              // gate/up item: 8 (gate, up) row pairs
constexpr int kUnitsPerExpert = I / kPairsPerItem;  // 64
constexpr int kXChunk = 4;                    // tokens staged in LDS at a time (16 KiB)

static_assert(H % (8 * kWave) == 0, "H must be a multiple of 512");
static_assert(kVecH == kThreads, "x staging: one 16-byte vector of a token per thread");
static_assert(kDecodeMaxT <= kThreads, "gate/up: one slot per thread");
static_assert(kMaxExperts + 1 <= 512, "down: one work-list item per thread");
static_assert(I == 8 * kWave, "down GEMV maps one 16-byte vector of a w2 row per lane");
static_assert(kDecodeMaxT * kMaxTopK <= 32767 && kMaxExperts <= 32767, "int16 routing table");

// ---------------------------------------------------------------- gate/up

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Barrier for LDS hand-offs only: waits for this wave's LDS operations, not
// for its outstanding global loads (which __syncthreads also waits for), so
// weight loads issued earlier stay in flight across it.  Also a compiler
// barrier for memory operations.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt: no wait
  asm volatile("s_barrier" ::: "memory");
}

// Waits until this wave's vector-memory operations, LDS-direct loads
// included, have completed.  The compiler does not reliably count LDS-direct
// loads as outstanding LDS writes at a later __syncthreads, so every barrier
// that publishes them is preceded by this explicit wait.
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt: no wait
}

// One x row (H bf16 = kVecH 16-byte vectors, one per thread) into LDS with
// an LDS-direct load: no registers, and a thread's loads for several rows
// are all in flight before the barrier that waits for them.  Lane l of a
// wave writes the 16 bytes at the wave's LDS base + 16 l, so LDS position t
// (t < kVecH) receives the vector thread t loads: vector t, or with kPermute
// vector 4 (t % 64) + t / 64, the order in which the NVFP4 gate/up rows read
// x (lane l's i-th vector covers columns [32 l + 8 i, +8)), so that their
// reads of position l + 64 i stay free of bank conflicts.
template <bool kPermute = false>
__device__ __forceinline__ void stage_x_row(u32x4* dst, const uint16_t* row) {
  const int wave_base = threadIdx.x & ~(kWave - 1);
  const int src = kPermute ? 4 * (threadIdx.x & (kWave - 1)) + threadIdx.x / kWave : threadIdx.x;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(row) + src,
                                   (lds_ptr_t)(dst + wave_base), 16, 0, 0);
}

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

// Gate/up rows of one wave: gate p, p+1 and up p, p+1 (p = p0 + 2 * wave);
// lane l holds columns [8l + 512i, 8l + 512i + 8) of each row, i = 0..3.
template <bool kFp4>
struct GateUpRows;

// bf16: 16 bytes per row per i.
template <>
struct GateUpRows<false> {
  u32x4 w[4][kVecPerLaneH];
  float g;  // tensor scale (1 for bf16)
  // Gate rows p, p+1 and up rows inter+p, inter+p+1 of a w13 [2 inter][H].
  __device__ __forceinline__ void load_rows(const uint16_t* w13, int inter, int p0) {
    const int lane = threadIdx.x & (kWave - 1);
    const int p = p0 + 2 * (threadIdx.x / kWave);
    const int row[4] = {p, p + 1, inter + p, inter + p + 1};
#pragma unroll
    for (int i = 0; i < kVecPerLaneH; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        w[r][i] = load_stream(reinterpret_cast<const u32x4*>(w13 + (size_t)row[r] * H) + lane + i * kWave);
    g = 1.0f;
  }
  __device__ __forceinline__ void load(const Bank& bank, int e, int p0) {
    load_rows(reinterpret_cast<const uint16_t*>(bank.w13) + (size_t)e * 2 * I * H, I, p0);
  }
  __device__ __forceinline__ float dot(int r, int i, const u32x4& xv, float acc) const {
    return dot8_bf16(w[r][i], xv, acc);
  }
  __device__ __forceinline__ void pin() {}
};

// NVFP4: lane l holds columns [32 l, 32 l + 32) of each of its 4 rows as one
// 16-byte load of E2M1 codes (words i = 0..3: columns [32 l + 8 i, +8)) and
// the two E4M3 scales of those columns' 16-element blocks as one 2-byte load;
// the x vectors arrive in the matching order (stage_x_row<true>).  The codes
// convert exactly to bf16 and meet x in bf16 dot products; the block scale
// multiplies each 8-element partial sum, the tensor scale the row total.
template <>
struct GateUpRows<true> {
  uint32_t q[4][kVecPerLaneH];   // codes: [row][word]
  uint32_t sc[4];                // two E4M3 bytes (blocks 2l, 2l + 1) per row
  float g;
  __device__ __forceinline__ void load(const Bank& bank, int e, int p0) {
    const uint8_t* w13 = bank.w13 + (size_t)e * 2 * I * (H / 2);
    const uint8_t* s13 = bank.w13_scale + (size_t)e * 2 * I * (H / 16);
    const int lane = threadIdx.x & (kWave - 1);
    const int p = p0 + 2 * (threadIdx.x / kWave);
    const int row[4] = {p, p + 1, I + p, I + p + 1};
    static_assert(H / 2 == 16 * kWave && H / 16 == 2 * kWave, "one 16-byte code vector per lane");
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32x4 v = load_stream(reinterpret_cast<const u32x4*>(w13 + (size_t)row[r] * (H / 2)) + lane);
      q[r][0] = v.x;
      q[r][1] = v.y;
      q[r][2] = v.z;
      q[r][3] = v.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sc[r] = load_stream(reinterpret_cast<const uint16_t*>(s13 + (size_t)row[r] * (H / 16)) + lane);
    g = bank.w13_gscale[e];
  }
  __device__ __forceinline__ float dot(int r, int i, const u32x4& xv, float acc) const {
    // x words go through dot2_bf16's scalar parameters: bit-casting a vector
    // element in place (bit_cast<bf16x2>(xv.y)) is miscompiled to element 0
    // by the ROCm 7.2 clang used here.
    const uint32_t c = q[r][i];
    float p = dot2_bf16(fp4x2_to_bf16x2<0>(c), xv.x, 0.f);
    p = dot2_bf16(fp4x2_to_bf16x2<1>(c), xv.y, p);
    p = dot2_bf16(fp4x2_to_bf16x2<2>(c), xv.z, p);
    p = dot2_bf16(fp4x2_to_bf16x2<3>(c), xv.w, p);
    const float s = i < 2 ? __builtin_amdgcn_cvt_f32_fp8((int)sc[r], 0)
                          : __builtin_amdgcn_cvt_f32_fp8((int)sc[r], 1);
    return fmaf(p, s, acc);
  }
  // Keep the codes packed across tokens: widening every word once, outside
  // the token loop, would need four times the registers.
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < kVecPerLaneH; ++i) asm volatile("" : "+v"(q[r][i]));
      asm volatile("" : "+v"(sc[r]));
    }
  }
};

// One block (4 waves) computes h = silu(gate) * up for the row pairs
// [p0, p0 + 8) of one expert, for `count` tokens, with the wave's rows
// already loaded (in flight while the token list was fetched); the tokens'
// x vectors stream through LDS.
template <bool kFp4, int kChunk = kXChunk>
__device__ __forceinline__ void gateup_compute(GateUpRows<kFp4>& wv, int p0, int count,
                                               const TokenList& list, const uint16_t* __restrict__ x,
                                               float* h, u32x4* xs, int hstride = I) {
  const int lane = threadIdx.x & (kWave - 1);
  const int p = p0 + 2 * (threadIdx.x / kWave);
  // The first chunk's x rows are requested while the weights are still in
  // flight; the barrier at the top of the loop waits for both.
  auto stage = [&](int c0) {
    const int n = min(kChunk, count - c0);
    for (int j = 0; j < n; ++j) stage_x_row<kFp4>(xs + j * kVecH, x + (size_t)list.tok(c0 + j) * H);
  };
  if (count > 0) stage(0);
  for (int c0 = 0; c0 < count; c0 += kChunk) {
    const int n = min(kChunk, count - c0);
    wait_vmem_all();
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      wv.pin();
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kVecPerLaneH; ++i) {
        const u32x4 xv = xs[j * kVecH + lane + i * kWave];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = wv.dot(r, i, xv, acc[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = wave_sum_lane63(acc[r]) * wv.g;
      if (lane == kWave - 1) {
        if constexpr (kFp4) {
          // W4A16: h crosses to the down launch as 16-bit activations (bf16).
          uint16_t* hr = reinterpret_cast<uint16_t*>(h) + (size_t)list.hrow(c0 + j) * hstride + p;
          *reinterpret_cast<uint32_t*>(hr) = pack_bf16x2_rne(silu(acc[0]) * acc[2], silu(acc[1]) * acc[3]);
        } else {
          float* hr = h + (size_t)list.hrow(c0 + j) * hstride + p;
          hr[0] = silu(acc[0]) * acc[2];
          hr[1] = silu(acc[1]) * acc[3];
        }
      }
    }
    if (c0 + kChunk < count) {
      lds_barrier();   // every wave is done with this chunk's x
      stage(c0 + kChunk);
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

// Top-k by score of tokens t0, t0 + dt, ... (n <= G of them), one wave,
// the G selections interleaved round by round.  Ranks on the logit (the
// sigmoid is strictly increasing), ties to the lower expert index.  Lane l
// holds the order-preserving keys of experts 4l .. 4l + 3 (0 = empty: no
// finite logit maps to 0), sorted by (key descending, expert ascending), so
// the lane's head is its best candidate; round j takes the wave maximum M
// of the heads, the lowest lane whose head equals M wins (lower lanes hold
// lower experts, and a lane's equal keys are ordered by expert), and the
// winner pops its head.  Lane j keeps the j-th pick, computes its sigmoid
// score and writes its slot.  The selected experts also go to
// s_ids[t * k + j] (LDS).
// kCoherent: the logits were stored by other blocks of the same launch;
// otherwise by an earlier launch.  to_global: also store ids and weights to
// the workspace and the caller's copies (one block per forward does).
template <int G, bool kCoherent = true>
__device__ void route_tokens(const LayerArgs& a, int t0, int dt, int n, int* s_ids,
                             bool to_global = true) {
  const int lane = threadIdx.x & (kWave - 1);
  const int E = a.E, k = a.k;
  uint32_t key[G][4];
  int ex[G][4];
  float z[G][4];
  // Unconditional (clamped) loads: all of them in flight at once.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int t = min(t0 + min(g, n - 1) * dt, a.T - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* zp = a.ws.logits + (size_t)t * E + min(lane * 4 + q, E - 1);
      z[g][q] = kCoherent ? load_coherent(zp) : *zp;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      key[g][q] = lane * 4 + q < E ? ord_f32(z[g][q]) : 0u;
      ex[g][q] = lane * 4 + q;
    }
    // Five compare-exchanges sort the four (key desc, expert asc).
    auto cx = [&](int i, int j) __attribute__((always_inline)) {
      const bool sw = key[g][j] > key[g][i] || (key[g][j] == key[g][i] && ex[g][j] < ex[g][i]);
      const uint32_t ki = key[g][i], kj = key[g][j];
      const int ei = ex[g][i], ej = ex[g][j];
      key[g][i] = sw ? kj : ki;
      key[g][j] = sw ? ki : kj;
      ex[g][i] = sw ? ej : ei;
      ex[g][j] = sw ? ei : ej;
    };
    cx(0, 1);
    cx(2, 3);
    cx(0, 2);
    cx(1, 3);
    cx(1, 2);
  }
  int my_e[G];
  uint32_t my_key[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    my_e[g] = 0;
    my_key[g] = 0;
  }
#pragma unroll 1
  for (int j = 0; j < k; ++j) {
    uint32_t m[G];
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = key[g][0];
    wave_max_u32_lane63_multi<G>(m);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint32_t M = (uint32_t)__builtin_amdgcn_readlane((int)m[g], 63);
      const int win = (int)__builtin_ctzll(__ballot(key[g][0] == M));
      const int best = __builtin_amdgcn_readlane(ex[g][0], win);
      if (lane == win) {
        key[g][0] = key[g][1];
        key[g][1] = key[g][2];
        key[g][2] = key[g][3];
        key[g][3] = 0u;
        ex[g][0] = ex[g][1];
        ex[g][1] = ex[g][2];
        ex[g][2] = ex[g][3];
      }
      if (lane == j) {
        my_e[g] = best;
        my_key[g] = M;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g >= n) break;
    const int t = t0 + g * dt;
    const float sc = lane < k ? sigmoid(unord_f32(my_key[g])) : 0.f;
    const float sum = __shfl(wave_sum_lane63(sc), kWave - 1);
    if (lane < k) {
      s_ids[t * k + lane] = my_e[g];
      if (to_global) {
        const float w = (a.renormalize ? sc / sum : sc) * a.routed_scale;
        a.ws.ids[t * k + lane] = my_e[g];
        a.ws.wts[t * k + lane] = w;
        if (a.ids_out) a.ids_out[t * k + lane] = my_e[g];
        if (a.wts_out) a.wts_out[t * k + lane] = w;
      }
    }
  }
}

// Bucket every (token, rank) slot by expert into the routing table (one
// block; s_ids holds the selected experts).  U is ascending; the slots of one
// expert are in ascending slot order: the rank of slot s among its expert's
// slots is the number of set bits below s in that expert's occupancy mask.
constexpr int kMaskWords = kDecodeMaxT * kMaxTopK / 32;  // 16
struct RouteLds {
  int ids[kDecodeMaxT * kMaxTopK];
  int cnt[kMaxExperts];
  int aoff[kMaxExperts];     // offset of expert e's slots
  int aidx[kMaxExperts];     // active index of expert e
  uint32_t occ[kMaxExperts * kMaskWords];
};

__device__ void build_route_table(const LayerArgs& a, RouteLds& L) {
  const int E = a.E;
  const int nslots = a.T * a.k;
  const int tid = threadIdx.x, nthr = blockDim.x;
  int32_t* route = a.ws.route;
  int32_t* r_active = route + 1;
  int32_t* r_off = route + 1 + E;
  int32_t* r_slots = route + 2 + 2 * E;
  for (int s = tid; s < nslots; s += nthr) {
    const int e = L.ids[s];
    atomicAdd(&L.cnt[e], 1);
    atomicOr(&L.occ[e * kMaskWords + (s >> 5)], 1u << (s & 31));
  }
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    int c[4], sc = 0, sf = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      c[q] = e < E ? L.cnt[e] : 0;
      sc += c[q];
      sf += c[q] > 0;
    }
    const int ic = wave_incl_scan(sc);
    const int iff = wave_incl_scan(sf);
    int o = ic - sc, act = iff - sf;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      L.aoff[e] = o;
      L.aidx[e] = act;
      if (c[q] > 0) {
        r_active[act] = e;
        r_off[act] = o;
        int32_t* rec = a.ws.items + (size_t)act * item_record_ints(a.T);
        rec[0] = e;
        rec[1] = c[q];
        ++act;
      }
      o += c[q];
    }
    if (lane == kWave - 1) {
      route[0] = iff;
      r_off[iff] = ic;
    }
  }
  __syncthreads();
  for (int s = tid; s < nslots; s += nthr) {
    const int e = L.ids[s];
    const uint32_t* m = L.occ + e * kMaskWords;
    int rank = __popc(m[s >> 5] & ((1u << (s & 31)) - 1u));
    for (int w = 0; w < (s >> 5); ++w) rank += __popc(m[w]);
    r_slots[L.aoff[e] + rank] = s;
    a.ws.items[(size_t)L.aidx[e] * item_record_ints(a.T) + 2 + rank] = s;
  }
}

// The end of a router launch: the last block to finish (it sees every
// logit) routes every token — wave w takes tokens w, w + kWaves, ..., up to
// 4 at a time, interleaved — and builds the routing table.
// `routers` is the number of blocks that computed logits (the grid, unless
// only some of the launch's blocks route); with reset_oproj the routing block
// also clears the low-latency path's projection counter, which every router
// block has read by the time it takes its ticket here.
template <int kWaves>
__device__ __forceinline__ void route_tail(const LayerArgs& a, RouteLds& L, int* s_flag,
                                           uint32_t routers, bool reset_oproj = false) {
  const int wave = threadIdx.x / kWave;
  if (!last_block_ticket(a.ws.header + kHdrRouterDone, routers, s_flag)) return;
  if (reset_oproj && threadIdx.x == 0)
    __hip_atomic_store(a.ws.header + kHdrOprojDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int mine = (a.T - wave + kWaves - 1) / kWaves;
  if (mine == 1) {
    route_tokens<1>(a, wave, kWaves, 1, L.ids);
  } else if (mine == 2) {
    route_tokens<2>(a, wave, kWaves, 2, L.ids);
  } else {
    for (int g0 = 0; g0 < mine; g0 += 4)
      route_tokens<4>(a, wave + g0 * kWaves, kWaves, min(4, mine - g0), L.ids);
  }
  lds_barrier();   // the selections are in LDS; their global stores need not land yet
  build_route_table(a, L);
}

// Lane exchange for the transposed reduction: lane l reads lane l ^ 4 (or
// l ^ 8) within its row of 16, as two bank-masked DPP row shifts.
__device__ __forceinline__ float xor4(float v) {
  const int x = __builtin_bit_cast(int, v);
  int r = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0x5, true);   // row_shl:4 into banks 0, 2
  r = __builtin_amdgcn_update_dpp(r, x, 0x114, 0xF, 0xA, true);       // row_shr:4 into banks 1, 3
  return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ float xor8(float v) {
  const int x = __builtin_bit_cast(int, v);
  int r = __builtin_amdgcn_update_dpp(0, x, 0x108, 0xF, 0x3, true);   // row_shl:8 into banks 0, 1
  r = __builtin_amdgcn_update_dpp(r, x, 0x118, 0xF, 0xC, true);       // row_shr:8 into banks 2, 3
  return __builtin_bit_cast(float, r);
}

// Sums v[0..7] over the 64 lanes: each exchange step halves the values a
// lane keeps (lanes that differ in bit b keep complementary halves), so the
// 8 sums cost 3 + 3 lane exchanges instead of 8 full reductions.  On return
// lane l holds the total of v[bitrev3(l % 8)].
__device__ __forceinline__ float wave_sum8_transposed(float (&v)[8]) {
  const int lane = threadIdx.x & (kWave - 1);
  {
    const bool b = lane & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float send = b ? v[i] : v[i + 4];
      const float keep = b ? v[i + 4] : v[i];
      v[i] = keep + dpp<0xB1>(send);   // lane ^ 1
    }
  }
  {
    const bool b = lane & 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float send = b ? v[i] : v[i + 2];
      const float keep = b ? v[i + 2] : v[i];
      v[i] = keep + dpp<0x4E>(send);   // lane ^ 2
    }
  }
  float t;
  {
    const bool b = lane & 4;
    const float send = b ? v[0] : v[1];
    const float keep = b ? v[1] : v[0];
    t = keep + xor4(send);
  }
  t += xor8(t);
  t += __shfl_xor(t, 16);
  t += __shfl_xor(t, 32);
  return t;
}

__device__ __forceinline__ int bitrev3(int x) { return ((x & 1) << 2) | (x & 2) | ((x & 4) >> 2); }

// A 16-byte vector written by another block of the same launch: four
// coherent 32-bit loads.
__device__ __forceinline__ u32x4 load_coherent_x4(const uint16_t* p) {
  const int32_t* q = reinterpret_cast<const int32_t*>(p);
  return u32x4{(uint32_t)load_coherent(q), (uint32_t)load_coherent(q + 1),
               (uint32_t)load_coherent(q + 2), (uint32_t)load_coherent(q + 3)};
}

// Pre-norm block: rows c0 .. c0+n-1 of n = bf16(r / rms(r) * gamma) into
// LDS, made in registers from r (thread i owns the 16-byte vector i of each
// row, gv the matching 8 gains).  The sums of squares meet in s_ss; with
// store_normed the block also stores the rows to `normed`, the input of the
// gate/up launch.  kCoherent: r was written by other blocks of this launch.
// Contains a __syncthreads: every thread of the block calls it.
template <bool kCoherent = false>
__device__ __forceinline__ void stage_normed_rows(const LayerArgs& a, int c0, int n, u32x4* xs,
                                                  const u32x4& gv, float* s_ss, bool store_normed) {
  static_assert(kRouteXChunk == 8, "one transposed 8-value reduction per chunk");
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  u32x4 rv[kRouteXChunk];
  float ss[kRouteXChunk];
#pragma unroll
  for (int j = 0; j < kRouteXChunk; ++j) {
    rv[j] = u32x4{0u, 0u, 0u, 0u};
    if (j < n) {
      const uint16_t* src = a.resid + (size_t)(c0 + j) * H + 8 * threadIdx.x;
      rv[j] = kCoherent ? load_coherent_x4(src) : *reinterpret_cast<const u32x4*>(src);
    }
  }
#pragma unroll
  for (int j = 0; j < kRouteXChunk; ++j) ss[j] = sumsq_bf16x8(rv[j]);
  // Lane l < 8 of each wave gets the wave's sum for row bitrev3(l).
  const float t = wave_sum8_transposed(ss);
  if (lane < kRouteXChunk) s_ss[wave * kRouteXChunk + bitrev3(lane)] = t;
  __syncthreads();
  // Lane l computes the scale of row l % 8 once; the rows' scales are then
  // read from lanes 0..7.
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kRouteWaves; ++w) tot += s_ss[w * kRouteXChunk + (lane & (kRouteXChunk - 1))];
  const float inv = rms_inv<H>(tot, a.eps);
#pragma unroll
  for (int j = 0; j < kRouteXChunk; ++j) {
    if (j < n) {
      const float inv_j = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv), j));
      const u32x4 v = rms_scale_bf16x8(rv[j], gv, inv_j);
      xs[j * kVecH + threadIdx.x] = v;
      if (store_normed) reinterpret_cast<u32x4*>(a.normed + (size_t)(c0 + j) * H)[threadIdx.x] = v;
    }
  }
}

// Bounded wait (one thread) until *counter reaches target.  Every wave gets
// past it: after kSpinLimit polls it gives up and sets *expired, which the
// caller's tests check, so that a wait that cannot end still lets the grid
// drain.
constexpr int kSpinLimit = 1 << 22;
__device__ __forceinline__ void wait_count(uint32_t* counter, uint32_t target, uint32_t* expired) {
  for (int i = 0; i < kSpinLimit; ++i) {
    if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
    __builtin_amdgcn_s_sleep(2);
  }
  __hip_atomic_store(expired, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Router of the pre-norm block, block rb of `routers`: wave w computes the
// logits of expert 4 rb + w for all T tokens, whose rows stream through LDS
// kRouteXChunk at a time, normalised from r on the way in (kCoherentR: r was
// written by other blocks of the same launch); router block 0 also stores
// n for the gate/up launch.  The last router block to finish routes every
// token and builds the routing table.
// With wait_oproj (the fused low-latency path) the block waits, once its
// router rows are on their way, until every projection block has counted in.
template <bool kCoherentR>
__device__ void route_norm_block(const LayerArgs& a, int rb, int routers, u32x4* xs, RouteLds& L,
                                 float* s_ss, int* s_flag, bool wait_oproj) {
  constexpr int XC = kRouteXChunk;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int e = rb * kRouterRows + wave;
  const int er = min(e, a.E - 1);
  for (int i = threadIdx.x; i < kMaxExperts; i += kThreads) L.cnt[i] = 0;
  for (int i = threadIdx.x; i < kMaxExperts * kMaskWords; i += kThreads) L.occ[i] = 0;
  u32x4 wv[kVecPerLaneH];
  const u32x4* row = reinterpret_cast<const u32x4*>(a.router_w + (size_t)er * H);
#pragma unroll
  for (int i = 0; i < kVecPerLaneH; ++i) wv[i] = load_stream(row + lane + i * kWave);
  const float bias = a.router_b ? a.router_b[er] : 0.f;
  const u32x4 gv = reinterpret_cast<const u32x4*>(a.norm_w)[threadIdx.x];
  if (wait_oproj) {
    if (threadIdx.x == 0) wait_count(a.ws.header + kHdrOprojDone, gridDim.x, a.ws.header + kHdrWaitExpired);
    __syncthreads();
  }
  auto stage = [&](int c0) __attribute__((always_inline)) {
    stage_normed_rows<kCoherentR>(a, c0, min(XC, a.T - c0), xs, gv, s_ss, rb == 0);
  };
  stage(0);   // in flight together with the router rows
  for (int c0 = 0; c0 < a.T; c0 += XC) {
    const int n = min(XC, a.T - c0);
    __syncthreads();   // the chunk's normalised rows are in LDS
    float acc[XC];
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      acc[j] = 0.f;
      if (j < n) {
#pragma unroll
        for (int i = 0; i < kVecPerLaneH; ++i) acc[j] = dot8_bf16(wv[i], xs[j * kVecH + lane + i * kWave], acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      if (j < n) {
        const float z = wave_sum_lane63(acc[j]);
        if (lane == kWave - 1 && e < a.E) store_coherent(a.ws.logits + (size_t)(c0 + j) * a.E + e, z + bias);
      }
    }
    if (c0 + XC < a.T) {
      lds_barrier();   // every wave is done with this chunk's x
      stage(c0 + XC);
    }
  }
  route_tail<kRouteWaves>(a, L, s_flag, routers, wait_oproj);
}

// Threads of a route_kernel block: 4 waves (one router row each); the bare
// layer's ticketed routing adds 4 waves that only rank tokens in the
// routing block (one token per wave at T = 8).  The pre-norm block's row
// staging maps one thread to each 16-byte vector of a row.
__host__ __device__ constexpr int route_threads(bool norm, bool fused) {
  return norm || fused ? kThreads : 2 * kThreads;
}

// Router of the pre-norm block and of small bare-layer batches: wave w of
// block b computes the logits of expert 4b + w for all T tokens; the
// tokens' rows stream through LDS kRouteXChunk at a time (for the pre-norm
// block, normalised from r on the way in).  The last block to finish routes
// every token and builds the routing table; with kFused (small batches,
// fused_routing_applies) the launch ends with the logits and the gate/up
// launch routes instead.
template <bool kNorm, bool kFused>
__global__ __launch_bounds__(route_threads(kNorm, kFused)) void route_kernel(LayerArgs a) {
  constexpr int XC = kRouteXChunk;
  constexpr int kNT = route_threads(kNorm, kFused);
  __shared__ u32x4 xs[XC * kVecH];
  __shared__ RouteLds L;
  __shared__ int s_flag;
  __shared__ float s_ss[kRouteWaves * kRouteXChunk];
  if constexpr (kNorm && !kFused) {
    route_norm_block<false>(a, blockIdx.x, gridDim.x, xs, L, s_ss, &s_flag, false);
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  // Waves kRouterRows and up (bare layer, ticketed routing) only rank tokens.
  const bool gemv = wave < kRouterRows;
  const int e = blockIdx.x * kRouterRows + wave;
  const int er = min(e, a.E - 1);
  if (!kFused) {
    for (int i = threadIdx.x; i < kMaxExperts; i += kNT) L.cnt[i] = 0;
    for (int i = threadIdx.x; i < kMaxExperts * kMaskWords; i += kNT) L.occ[i] = 0;
  }
  u32x4 wv[kVecPerLaneH];
  const u32x4* row = reinterpret_cast<const u32x4*>(a.router_w + (size_t)er * H);
  if (gemv) {
#pragma unroll
    for (int i = 0; i < kVecPerLaneH; ++i) wv[i] = load_stream(row + lane + i * kWave);
  }
  const float bias = a.router_b ? a.router_b[er] : 0.f;
  if constexpr (!kNorm && kFused) {
    // Small batch (T <= kRouteWaves): each wave reads the T x rows straight
    // from memory with its router row; no LDS staging, no block barrier.
    static_assert(kRouteWaves <= kRouteXChunk, "one chunk");
    u32x4 xv[kRouteWaves][kVecPerLaneH];
#pragma unroll
    for (int j = 0; j < kRouteWaves; ++j) {
      if (j < a.T) {
#pragma unroll
        for (int i = 0; i < kVecPerLaneH; ++i)
          xv[j][i] = reinterpret_cast<const u32x4*>(a.x + (size_t)j * H)[lane + i * kWave];
      }
    }
#pragma unroll
    for (int j = 0; j < kRouteWaves; ++j) {
      if (j < a.T) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < kVecPerLaneH; ++i) acc = dot8_bf16(wv[i], xv[j][i], acc);
        const float z = wave_sum_lane63(acc);
        if (lane == kWave - 1 && e < a.E) a.ws.logits[(size_t)j * a.E + e] = z + bias;
      }
    }
    return;
  }
  u32x4 gv{};
  if (kNorm) gv = reinterpret_cast<const u32x4*>(a.norm_w)[threadIdx.x];
  auto stage = [&](int c0) __attribute__((always_inline)) {
    const int n = min(XC, a.T - c0);
    if (kNorm) {
      stage_normed_rows(a, c0, n, xs, gv, s_ss, blockIdx.x == 0);
    } else if (threadIdx.x < kVecH) {
      for (int j = 0; j < n; ++j) stage_x_row(xs + j * kVecH, a.x + (size_t)(c0 + j) * H);
    }
  };
  stage(0);   // in flight together with the router rows
  for (int c0 = 0; c0 < a.T; c0 += XC) {
    const int n = min(XC, a.T - c0);
    wait_vmem_all();
    __syncthreads();
    float acc[XC];
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      acc[j] = 0.f;
      if (gemv && j < n) {
#pragma unroll
        for (int i = 0; i < kVecPerLaneH; ++i) acc[j] = dot8_bf16(wv[i], xs[j * kVecH + lane + i * kWave], acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < XC; ++j) {
      if (gemv && j < n) {
        const float z = wave_sum_lane63(acc[j]);
        if (lane == kWave - 1 && e < a.E) {
          float* zp = a.ws.logits + (size_t)(c0 + j) * a.E + e;
          if (kFused) *zp = z + bias;
          else store_coherent(zp, z + bias);
        }
      }
    }
    if (c0 + XC < a.T) {
      lds_barrier();   // every wave is done with this chunk's x
      stage(c0 + XC);
    }
  }
  if (kFused) return;
  route_tail<kNT / kWave>(a, L, &s_flag, gridDim.x);
}

// Router of larger bare-layer batches (T > kRouteBareMinT): 16 waves per
// block, and every wave holds all four of the block's router rows (experts
// 4b .. 4b + 3) and computes them for its tokens (wave w: tokens w, w + 16
// of each chunk of kRouteBareXChunk staged in LDS), so each x vector is
// read from LDS once per block rather than once per row; the 8 (row, token)
// sums of a wave meet in one transposed 8-value reduction.  The routing
// tail then has 16 waves for the top-k.  Every wave reading all four rows
// (64 KiB per wave from L2) does not pay off for small batches.
__global__ __launch_bounds__(kRouteBareThreads) void route_bare_kernel(LayerArgs a) {
  static_assert(kRouteBareXChunk == 2 * kRouteBareWaves, "two tokens per wave and chunk");
  __shared__ u32x4 xs[kRouteBareXChunk * kVecH];
  __shared__ RouteLds L;
  __shared__ int s_flag;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int e0 = blockIdx.x * kRouterRows;
  for (int i = threadIdx.x; i < kMaxExperts; i += kRouteBareThreads) L.cnt[i] = 0;
  for (int i = threadIdx.x; i < kMaxExperts * kMaskWords; i += kRouteBareThreads) L.occ[i] = 0;
  u32x4 wv[kRouterRows][kVecPerLaneH];
#pragma unroll
  for (int r = 0; r < kRouterRows; ++r) {
    const u32x4* row = reinterpret_cast<const u32x4*>(a.router_w + (size_t)min(e0 + r, a.E - 1) * H);
#pragma unroll
    for (int i = 0; i < kVecPerLaneH; ++i) wv[r][i] = load_stream(row + lane + i * kWave);
  }
  // Lane l < 8 stores the sum for row bitrev3(l) / 2 of token bitrev3(l) % 2.
  const int my_r = bitrev3(lane & 7) >> 1, my_g = bitrev3(lane & 7) & 1;
  const int my_e = e0 + my_r;
  const float bias = a.router_b && lane < 8 ? a.router_b[min(my_e, a.E - 1)] : 0.f;
  // Thread i stages 16-byte vector i % 256 of rows 4p + i / 256 (p = 0, 1, ...).
  auto stage = [&](int c0) __attribute__((always_inline)) {
    const int n = min(kRouteBareXChunk, a.T - c0);
    const int v = threadIdx.x & (kVecH - 1);
    for (int j = threadIdx.x / kVecH; j < n; j += kRouteBareThreads / kVecH)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(a.x + (size_t)(c0 + j) * H) + v,
                                       (lds_ptr_t)(xs + j * kVecH + (v & ~(kWave - 1))), 16, 0, 0);
  };
  stage(0);   // in flight together with the router rows
  for (int c0 = 0; c0 < a.T; c0 += kRouteBareXChunk) {
    const int n = min(kRouteBareXChunk, a.T - c0);
    wait_vmem_all();
    __syncthreads();
    if (wave < n) {
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int j = wave + g * kRouteBareWaves;
        if (j < n) {
#pragma unroll
          for (int i = 0; i < kVecPerLaneH; ++i) {
            const u32x4 xv = xs[j * kVecH + lane + i * kWave];
#pragma unroll
            for (int r = 0; r < kRouterRows; ++r) acc[r * 2 + g] = dot8_bf16(wv[r][i], xv, acc[r * 2 + g]);
          }
        }
      }
      const float z = wave_sum8_transposed(acc);
      const int j = wave + my_g * kRouteBareWaves;
      if (lane < 8 && j < n && my_e < a.E) {
        store_coherent(a.ws.logits + (size_t)(c0 + j) * a.E + my_e, z + bias);
      }
    }
    if (c0 + kRouteBareXChunk < a.T) {
      lds_barrier();   // every wave is done with this chunk's x
      stage(c0 + kRouteBareXChunk);
    }
  }
  route_tail<kRouteBareWaves>(a, L, &s_flag, gridDim.x);
}

// Routing of a small batch inside one block, from the logits of the router
// launch: every routed gate/up block repeats it, which costs less than a
// completion ticket and a one-block routing step between the two launches
// as long as every wave ranks at most one token and the whole grid is
// resident at once (fused_routing_applies).  Wave w ranks token w; wave 0
// then sorts the slots by (expert, slot) — slot s
// lands at the number of slots with a smaller expert plus the earlier
// slots of its own — and marks where each expert's run starts, which gives
// U in ascending order.  Item `ai` (the ai-th expert of U) is returned in
// meta = {|U|, expert, first sorted position, slot count}; its slots are
// sorted_s[pos .. pos + count).  The writer block also stores the ids,
// the weights and the routing table for the down launch.
constexpr int kFusedMaxSlots = 16;   // (1 + 16) x 64 gate/up blocks: resident at 5 per CU
__host__ __device__ constexpr bool fused_routing_applies(int T, int k) {
  return T <= kRouteWaves && T * k <= kFusedMaxSlots;
}

struct FusedRouteLds {
  int ids[kWave];
  int sorted_e[kWave];
  int16_t sorted_s[kWave];
  int meta[4];
};

__device__ void fused_route(const LayerArgs& a, int ai, bool writer, FusedRouteLds& L) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int T = a.T, E = a.E, nslots = a.T * a.k;
  if (wave < T) route_tokens<1, false>(a, wave, kRouteWaves, 1, L.ids, writer);
  __syncthreads();
  if (wave == 0 && lane < nslots) {
    const int e = L.ids[lane];
    int less = 0, before = 0;
    for (int j = 0; j < nslots; ++j) {
      const int ej = L.ids[j];
      less += ej < e;
      before += (ej == e) & (j < lane);
    }
    L.sorted_e[less + before] = e;
    L.sorted_s[less + before] = (int16_t)lane;
  }
  __syncthreads();
  if (wave == 0) {
    const int p = lane;
    const int e = p < nslots ? L.sorted_e[p] : -1;
    const bool first = p < nslots && (p == 0 || e != L.sorted_e[p > 0 ? p - 1 : 0]);
    const uint64_t fm = __ballot(first);
    const int n = __popcll(fm);
    const int uidx = __popcll(fm & ((1ull << p) - 1ull));
    const uint64_t above = p < kWave - 1 ? fm >> (p + 1) : 0ull;
    const int next = above ? p + 1 + (int)__builtin_ctzll(above) : nslots;
    if (first && uidx == ai) {
      L.meta[1] = e;
      L.meta[2] = p;
      L.meta[3] = next - p;
    }
    if (lane == 0) L.meta[0] = n;
    if (writer) {
      int32_t* route = a.ws.route;
      if (first) {
        route[1 + uidx] = e;
        route[1 + E + uidx] = p;
      }
      if (p < nslots) route[2 + 2 * E + p] = L.sorted_s[p];
      if (lane == 0) {
        route[0] = n;
        route[1 + E + n] = nslots;
      }
    }
  }
  __syncthreads();
}

// Blocks [0, kUnitsPerExpert): the shared expert for all T tokens (h rows
// T*k + t); then routed items.  kFused: the routed blocks route the batch
// themselves (fused_route) instead of reading the routing table.
template <bool kFp4, bool kFused>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5)))
void gateup_kernel(LayerArgs a) {
  __shared__ u32x4 xs[kXChunk * kVecH];
  __shared__ int16_t s_slots[kDecodeMaxT];
  __shared__ int s_meta[4];
  __shared__ FusedRouteLds FL;
  if ((int)blockIdx.x < kUnitsPerExpert) {
    const int unit = blockIdx.x;
    GateUpRows<kFp4> wv;
    wv.load(a.shared, 0, unit * kPairsPerItem);
    gateup_compute(wv, unit * kPairsPerItem, a.T, TokenList{nullptr, a.k, a.T * a.k}, a.x, a.ws.h, xs);
    return;
  }
  const int b = blockIdx.x - kUnitsPerExpert;
  const int ai = b / kUnitsPerExpert;
  const int unit = b - ai * kUnitsPerExpert;
  if (kFused && a.T == 1) {
    // One token: every wave ranks it (the same picks in every wave), so no
    // block barrier precedes the weight loads.  The k picks are distinct;
    // the item's expert is the ai-th smallest, its one slot the pick's rank
    // j (slot j of token 0).  Wave 0 of the first routed block stores the
    // ids, the weights and the routing table.
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int k = a.k, E = a.E;
    const bool writer = b == 0 && wave == 0;
    int* ids = FL.ids + wave * kMaxTopK;   // this wave's picks (written and read by this wave)
    route_tokens<1, false>(a, 0, 1, 1, ids, writer);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the picks are in LDS
    const int ej = lane < k ? ids[lane] : 0x7FFFFFFF;
    int rank = 0;
    for (int i = 0; i < k; ++i) rank += ids[i] < ej;
    const uint64_t hit = __ballot(lane < k && rank == ai);
    if (writer) {
      int32_t* route = a.ws.route;
      if (lane < k) {
        route[1 + rank] = ej;
        route[1 + E + rank] = rank;
        route[2 + 2 * E + rank] = lane;
      }
      if (lane == 0) {
        route[0] = k;
        route[1 + E + k] = k;
      }
    }
    const int slot = (int)__builtin_ctzll(hit);   // ai < k: exactly one lane
    const int e = __builtin_amdgcn_readlane(ej, slot);
    GateUpRows<kFp4> wv;
    wv.load(a.routed, e, unit * kPairsPerItem);
    gateup_compute<kFp4, kXChunk>(wv, unit * kPairsPerItem, 1, TokenList{nullptr, a.k, slot}, a.x, a.ws.h, xs);
    return;
  }
  if (kFused) {
    fused_route(a, ai, b == 0, FL);
    if (ai >= FL.meta[0]) return;
    const int e = FL.meta[1], off = FL.meta[2], cnt = FL.meta[3];
    GateUpRows<kFp4> wv;
    wv.load(a.routed, e, unit * kPairsPerItem);
    gateup_compute(wv, unit * kPairsPerItem, cnt, TokenList{FL.sorted_s + off, a.k, 0}, a.x, a.ws.h, xs);
    return;
  }
  // |U| and item ai's record (expert, slot count, slots) in one round trip
  // (ai < min(E, T k), the number of records the table has room for); the
  // weights and the x rows are then requested together.
  const int rec_ints = item_record_ints(a.T);
  static_assert(2 + kDecodeMaxT < kThreads - 1, "record and |U| loads on distinct threads");
  int v = 0;
  if ((int)threadIdx.x < rec_ints) v = a.ws.items[(size_t)ai * rec_ints + threadIdx.x];
  if (threadIdx.x == kThreads - 1) s_meta[0] = a.ws.route[0];
  if (threadIdx.x < 2) s_meta[1 + threadIdx.x] = v;
  else if ((int)threadIdx.x < rec_ints) s_slots[threadIdx.x - 2] = (int16_t)v;
  __syncthreads();
  if (ai >= s_meta[0]) return;
  const int e = s_meta[1], cnt = s_meta[2];
  GateUpRows<kFp4> wv;
  wv.load(a.routed, e, unit * kPairsPerItem);
  gateup_compute(wv, unit * kPairsPerItem, cnt, TokenList{s_slots, a.k, 0}, a.x, a.ws.h, xs);
}


// The low-latency path's next-layer norm at the end of the down launch.
__device__ void next_norm_tail(const LayerArgs& a);
__device__ __forceinline__ void down_combine(const LayerArgs& a, const float* part, const float* s_wts,
                                             int r0);

// Down + combine.  Block b owns output rows [8b, 8b + 8) of every token and
// walks the |U| active experts and then the shared expert; wave w takes
// items w, w + 8, ... and keeps the next item's rows (and its first slot's
// h) in flight while it reduces the current one.  Lane l holds columns
// [8l, 8l + 8) of each row.  Per (h row, output row) the 64-lane partial
// dot products are summed in a fixed tree and parked in LDS; the block then
// combines out = shared + sum_j w_j * routed_j in a fixed order.
constexpr int kDownRowsPerBlock = 8;
constexpr int kDownThreads = 512;
constexpr int kDownWaves = kDownThreads / kWave;
constexpr int kDnSlots = 2;       // slots per work entry (their h rows prefetched together)
constexpr int kMaxDownWork = 640; // >= T*k/2 + (E + 1) + T/2 for T <= 64, k <= 8
// Work entry code: item << 5 | sub-entry (int16: item <= 256, sub-entry < 32).
constexpr int kDnSubBits = 5;
static_assert(kDecodeMaxT / kDnSlots <= (1 << kDnSubBits) &&
              (kMaxExperts << kDnSubBits) + (1 << kDnSubBits) - 1 <= 32767, "work entry code");
static_assert(kDecodeMaxT * kMaxTopK / kDnSlots + kMaxExperts + 1 + kDecodeMaxT / kDnSlots <= kMaxDownWork,
              "work list size");

// A work entry: slots [j0, j0 + nj) of one item (item 0: the shared
// expert, whose slots are the T tokens; item i > 0: active expert i - 1).
struct DownItem {
  int e;            // expert index in its bank
  bool shared;
  int off;          // routed: the item's slots start at slots[off]
  int j0, nj;
  // The item has more slots than one entry takes, so the block's other
  // entries of it read the same rows: load them through the caches (the
  // repeats then hit L2) rather than with the streaming hint.
  bool cached;
};

__device__ __forceinline__ DownItem shared_entry(const LayerArgs& a, int q) {
  DownItem d;
  d.shared = true;
  d.e = 0;
  d.off = 0;
  d.j0 = q * kDnSlots;
  d.nj = min(kDnSlots, a.T - d.j0);
  d.cached = a.T > kDnSlots;
  return d;
}

__device__ __forceinline__ DownItem down_entry(const LayerArgs& a, int entry,
                                               const int16_t* s_active, const int16_t* s_off) {
  const int item = entry >> kDnSubBits, q = entry & ((1 << kDnSubBits) - 1);
  if (item == 0) return shared_entry(a, q);
  DownItem d;
  d.shared = false;
  d.e = s_active[item - 1];
  d.off = s_off[item - 1];
  d.j0 = q * kDnSlots;
  d.nj = min(kDnSlots, s_off[item] - d.off - d.j0);
  d.cached = s_off[item] - d.off > kDnSlots;
  return d;
}

__device__ __forceinline__ int down_hrow(const LayerArgs& a, const DownItem& d, int j,
                                         const int16_t* s_slots) {
  return d.shared ? a.T * a.k + d.j0 + j : s_slots[d.off + d.j0 + j];
}

// The 8 rows of one work entry in a lane, plus the h of its slots.
template <bool kFp4>
struct DownRows;

template <>
struct DownRows<false> {
  u32x4 w[kDownRowsPerBlock];
  f32x4 h0[kDnSlots], h1[kDnSlots];
  template <bool kCached>
  __device__ __forceinline__ void load(const LayerArgs& a, const DownItem& d, int r0) {
    const Bank& bank = d.shared ? a.shared : a.routed;
    const uint16_t* w2 = reinterpret_cast<const uint16_t*>(bank.w2) + (size_t)d.e * H * I;
    const int lane = threadIdx.x & (kWave - 1);
    if (kCached && __builtin_amdgcn_readfirstlane((int)d.cached)) {
#pragma unroll
      for (int r = 0; r < kDownRowsPerBlock; ++r)
        w[r] = reinterpret_cast<const u32x4*>(w2 + (size_t)(r0 + r) * I)[lane];
    } else {
#pragma unroll
      for (int r = 0; r < kDownRowsPerBlock; ++r)
        w[r] = load_stream(reinterpret_cast<const u32x4*>(w2 + (size_t)(r0 + r) * I) + lane);
    }
  }
  // Slot j's h row (fp32): lane l's columns [8l, 8l + 8).
  __device__ __forceinline__ void load_h(const LayerArgs& a, int j, int hrow) {
    const int lane = threadIdx.x & (kWave - 1);
    const f32x4* hp = reinterpret_cast<const f32x4*>(a.ws.h + (size_t)hrow * I) + lane * 2;
    h0[j] = hp[0];
    h1[j] = hp[1];
  }
  __device__ __forceinline__ float scale() const { return 1.0f; }
  // Lane partial of row r: its 8 columns of w2 . h.
  __device__ __forceinline__ float partial(int r, const f32x4& a0, const f32x4& a1) const {
    const u32x4 v = w[r];
    float s = bf16_lo(v.x) * a0.x;
    s = fmaf(bf16_hi(v.x), a0.y, s);
    s = fmaf(bf16_lo(v.y), a0.z, s);
    s = fmaf(bf16_hi(v.y), a0.w, s);
    s = fmaf(bf16_lo(v.z), a1.x, s);
    s = fmaf(bf16_hi(v.z), a1.y, s);
    s = fmaf(bf16_lo(v.w), a1.z, s);
    s = fmaf(bf16_hi(v.w), a1.w, s);
    return s;
  }
};

// NVFP4 (W4A16): one wave instruction covers four rows, 16 lanes per row.
// Lane l holds columns [32 c, 32 c + 32), c = l % 16, of rows 4 i + l / 16
// (i = 0, 1): 16 bytes of E2M1 codes and, in one 16-bit load, the E4M3
// scales of its two 16-column blocks; and the same 32 columns of each
// slot's h, which the gate/up launch of this format stores as bf16 (the
// 16-bit activations of W4A16).  Every E2M1 value is a bf16 value, so the
// products run on dot2_bf16 with fp32 accumulation; the block scales are
// applied to the two 16-column sums and the tensor scale to the row total.
template <>
struct DownRows<true> {
  u32x4 q[2];
  uint32_t sc[2];
  float g;
  u32x4 h[kDnSlots][4];
  template <bool kCached>
  __device__ __forceinline__ void load(const LayerArgs& a, const DownItem& d, int r0) {
    static_assert(I / 2 == 16 * 16 && I / 16 == 16 * 2, "16 lanes x 16 bytes of codes per row");
    const Bank& bank = d.shared ? a.shared : a.routed;
    const uint8_t* w2 = bank.w2 + (size_t)d.e * H * (I / 2);
    const uint8_t* s2 = bank.w2_scale + (size_t)d.e * H * (I / 16);
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 15;
    if (kCached && __builtin_amdgcn_readfirstlane((int)d.cached)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = r0 + 4 * i + (lane >> 4);
        q[i] = reinterpret_cast<const u32x4*>(w2 + (size_t)row * (I / 2))[c];
        sc[i] = reinterpret_cast<const uint16_t*>(s2 + (size_t)row * (I / 16))[c];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = r0 + 4 * i + (lane >> 4);
        q[i] = load_stream(reinterpret_cast<const u32x4*>(w2 + (size_t)row * (I / 2)) + c);
        sc[i] = load_stream(reinterpret_cast<const uint16_t*>(s2 + (size_t)row * (I / 16)) + c);
      }
    }
    g = bank.w2_gscale[d.e];
  }
  // Slot j's h row (bf16): columns [32 c, 32 c + 32).
  __device__ __forceinline__ void load_h(const LayerArgs& a, int j, int hrow) {
    const int c = threadIdx.x & 15;
    const u32x4* hp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.ws.h) +
                                                     (size_t)hrow * I) + c * 4;
#pragma unroll
    for (int v = 0; v < 4; ++v) h[j][v] = hp[v];
  }
};

template <bool kFp4, bool kCached>
__device__ __forceinline__ void prefetch_entry(DownRows<kFp4>& p, const LayerArgs& a, const DownItem& d,
                                               int r0, const int16_t* s_slots) {
  p.template load<kCached>(a, d, r0);
  // Entries past nj re-read slot 0's h (in bounds, unused).
#pragma unroll
  for (int j = 0; j < kDnSlots; ++j) p.load_h(a, j, down_hrow(a, d, j < d.nj ? j : 0, s_slots));
}

template <bool kFp4>
__device__ __forceinline__ void down_entry_rows(const LayerArgs& a, const DownItem& d,
                                                const DownRows<kFp4>& p, const int16_t* s_slots,
                                                float* part) {
  const int lane = threadIdx.x & (kWave - 1);
  if constexpr (kFp4) {
    // Codes to bf16 once per entry (shared by its slots); per slot and row
    // the 16 lanes' partials meet in a fixed butterfly, which leaves the row
    // total in all of them.
    u32x4 wv[2][4];
    float s_lo[2], s_hi[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t cw[4] = {p.q[i].x, p.q[i].y, p.q[i].z, p.q[i].w};
#pragma unroll
      for (int w = 0; w < 4; ++w)
        wv[i][w] = u32x4{fp4x2_to_bf16x2<0>(cw[w]), fp4x2_to_bf16x2<1>(cw[w]), fp4x2_to_bf16x2<2>(cw[w]),
                         fp4x2_to_bf16x2<3>(cw[w])};
      s_lo[i] = __builtin_amdgcn_cvt_f32_fp8((int)p.sc[i], 0);
      s_hi[i] = __builtin_amdgcn_cvt_f32_fp8((int)p.sc[i], 1);
    }
#pragma unroll
    for (int j = 0; j < kDnSlots; ++j) {
      if (j >= d.nj) break;
      float v[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float lo = dot8_bf16(wv[i][1], p.h[j][1], dot8_bf16(wv[i][0], p.h[j][0], 0.f));
        const float hi = dot8_bf16(wv[i][3], p.h[j][3], dot8_bf16(wv[i][2], p.h[j][2], 0.f));
        v[i] = fmaf(hi, s_hi[i], lo * s_lo[i]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v[i] += dpp<0xB1>(v[i]);    // lane ^ 1
        v[i] += dpp<0x4E>(v[i]);    // lane ^ 2
        v[i] += dpp<0x141>(v[i]);   // row_half_mirror: sums of 8
        v[i] += dpp<0x140>(v[i]);   // row_mirror: sums of 16
      }
      if ((lane & 15) == 0) {
        float* dst = part + down_hrow(a, d, j, s_slots) * kDownRowsPerBlock + (lane >> 4);
        dst[0] = v[0] * p.g;
        dst[4] = v[1] * p.g;
      }
    }
  } else {
  #pragma unroll
    for (int j = 0; j < kDnSlots; ++j) {
      if (j >= d.nj) break;
      float v[kDownRowsPerBlock];
  #pragma unroll
      for (int r = 0; r < kDownRowsPerBlock; ++r) v[r] = p.partial(r, p.h0[j], p.h1[j]);
      const float tot = wave_sum8_transposed(v);
      if (lane < kDownRowsPerBlock)
        part[down_hrow(a, d, j, s_slots) * kDownRowsPerBlock + bitrev3(lane)] = tot * p.scale();
    }
  }
}

// Down + combine.  Block b owns output rows [8b, 8b + 8) of every token.
// Its work: the shared expert and every active expert, cut into entries of
// up to kDnSlots slots (an expert hit by many tokens spreads over several
// waves), the shared expert's first: they need no routing table, so their
// rows and h are requested while the table is still on its way.  Wave w
// takes entries w, w + 8, ... and keeps the next two
// entries' w2 rows and h rows in flight while it reduces the current one
// (two-slot entries keep three buffers within the register budget).  Lane l holds
// columns [8l, 8l + 8) of each bf16 row (NVFP4: see DownRows<true>).  Per
// (h row, output row) the lanes' partial dot products are summed in a fixed
// tree and parked in LDS; the block then combines
// out = shared + sum_j w_j * routed_j in a fixed order.
// kCached (batches above 8 tokens, where experts with many slots are
// common): items cut into several entries load their rows through the caches
// (DownItem::cached).  The smaller batches keep the one streaming load path:
// the second path's code alone measured ~1 us slower at T = 1 and T = 8.
template <bool kFp4, bool kCached>
__global__ __launch_bounds__(kDownThreads) void down_kernel(LayerArgs a) {
  __shared__ int16_t s_active[kMaxExperts];
  __shared__ int16_t s_off[kMaxExperts + 1];
  __shared__ int16_t s_slots[kDecodeMaxT * kMaxTopK];
  __shared__ float s_wts[kDecodeMaxT * kMaxTopK];
  __shared__ int16_t s_work[kMaxDownWork];
  __shared__ int s_scan[kDownWaves];
  __shared__ float part[(kMaxTopK + 1) * kDecodeMaxT * kDownRowsPerBlock];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r0 = blockIdx.x * kDownRowsPerBlock;
  const int T = a.T, k = a.k, E = a.E;
  const int32_t* route = a.ws.route;
  if (T == 1 && k < kDownWaves) {
    // One token: k + 1 entries of one slot each and no work list.  Wave 0
    // takes the shared expert (no table needed), wave w <= k the (w - 1)-th
    // expert of U and its slot, read straight from the routing table.
    const int w0 = __builtin_amdgcn_readfirstlane(wave);
    if ((int)threadIdx.x < k) s_wts[threadIdx.x] = a.ws.wts[threadIdx.x];
    if (w0 <= k) {
      DownItem d;
      if (w0 == 0) {
        d = shared_entry(a, 0);
      } else {
        const int ai = w0 - 1;
        d.shared = false;
        d.e = route[1 + ai];
        d.off = ai;
        d.j0 = 0;
        d.nj = 1;
        d.cached = false;
        if (lane == 0) s_slots[ai] = (int16_t)route[2 + 2 * E + ai];   // read back by this wave only
      }
      DownRows<kFp4> p;
      prefetch_entry<kFp4, false>(p, a, d, r0, s_slots);
      down_entry_rows(a, d, p, s_slots, part);
    }
  } else {
    // The routing table in one round trip (whole arrays, no dependence on |U|;
    // one element of each per thread), requested before the shared expert's
    // entries so that waiting for it leaves those in flight.
    const int q = threadIdx.x;
    int v_act = 0, v_off = 0, v_slot = 0;
    float v_wt = 0.f;
    if (q < E) v_act = route[1 + q];
    if (q <= E) v_off = route[1 + E + q];
    if (q < T * k) {
      v_slot = route[2 + 2 * E + q];
      v_wt = a.ws.wts[q];   // for the combine, fetched with the table
    }
    const int n = route[0];

    // Three entries per wave in flight: the one being reduced and the next
    // two (rows and h), rotated through pa, pb, pc.  The shared expert's
    // entries are the first n_sh of the work list.
    const int n_sh = (T + kDnSlots - 1) / kDnSlots;
    DownRows<kFp4> pa, pb, pc;
    DownItem da{}, db{}, dc{};
    int w = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform: scalar branches below
    // Each path stores the table on its own, so that the wait for the table
    // leaves exactly that path's entry loads in flight (at a join, the wait
    // would have to assume none were issued and wait for all); the distinct
    // asm markers keep the copies from being merged.
    auto store_table = [&]() __attribute__((always_inline)) {
      if (q < E) s_active[q] = (int16_t)v_act;
      if (q <= E) s_off[q] = (int16_t)v_off;
      if (q < T * k) {
        s_slots[q] = (int16_t)v_slot;
        s_wts[q] = v_wt;
      }
    };
    if (w + kDownWaves < n_sh) {
      da = shared_entry(a, w);
      prefetch_entry<kFp4, kCached>(pa, a, da, r0, s_slots);
      db = shared_entry(a, w + kDownWaves);
      prefetch_entry<kFp4, kCached>(pb, a, db, r0, s_slots);
      store_table();
      asm volatile("; down: two shared entries in flight" ::: "memory");
    } else if (w < n_sh) {
      da = shared_entry(a, w);
      prefetch_entry<kFp4, kCached>(pa, a, da, r0, s_slots);
      store_table();
      asm volatile("; down: one shared entry in flight" ::: "memory");
    } else {
      store_table();
    }
    lds_barrier();

    // Work list: item 0 (the shared expert, T slots) and items 1..n (active
    // expert i - 1) contribute ceil(cnt / kDnSlots) entries each, laid out by
    // an exclusive scan.
    const int it = threadIdx.x;
    const int cnt = it == 0 ? T : (it <= n ? s_off[it] - s_off[it - 1] : 0);
    const int nsub = (cnt + kDnSlots - 1) / kDnSlots;
    const int incl = wave_incl_scan(nsub);
    if (lane == kWave - 1) s_scan[wave] = incl;
    lds_barrier();
    int base = incl - nsub, total = 0;
    for (int v = 0; v < kDownWaves; ++v) {
      if (v < wave) base += s_scan[v];
      total += s_scan[v];
    }
    for (int j = 0; j < nsub; ++j) s_work[base + j] = (int16_t)((it << kDnSubBits) | j);
    lds_barrier();

    if (w >= n_sh && w < total) {
      da = down_entry(a, s_work[w], s_active, s_off);
      prefetch_entry<kFp4, kCached>(pa, a, da, r0, s_slots);
    }
    if (w + kDownWaves >= n_sh && w + kDownWaves < total) {
      db = down_entry(a, s_work[w + kDownWaves], s_active, s_off);
      prefetch_entry<kFp4, kCached>(pb, a, db, r0, s_slots);
    }
    while (w < total) {
      if (w + 2 * kDownWaves < total) {
        dc = down_entry(a, s_work[w + 2 * kDownWaves], s_active, s_off);
        prefetch_entry<kFp4, kCached>(pc, a, dc, r0, s_slots);
      }
      down_entry_rows(a, da, pa, s_slots, part);
      w += kDownWaves;
      if (w >= total) break;
      if (w + 2 * kDownWaves < total) {
        da = down_entry(a, s_work[w + 2 * kDownWaves], s_active, s_off);
        prefetch_entry<kFp4, kCached>(pa, a, da, r0, s_slots);
      }
      down_entry_rows(a, db, pb, s_slots, part);
      w += kDownWaves;
      if (w >= total) break;
      if (w + 2 * kDownWaves < total) {
        db = down_entry(a, s_work[w + 2 * kDownWaves], s_active, s_off);
        prefetch_entry<kFp4, kCached>(pb, a, db, r0, s_slots);
      }
      down_entry_rows(a, dc, pc, s_slots, part);
      w += kDownWaves;
    }
  }
  __syncthreads();
  down_combine(a, part, s_wts, r0);
}

// The combine of a down block (rows [r0, r0 + 8)), once every (h row, output
// row) partial is in part: out = shared + sum_j w_j * routed_j in rank order,
// the residual added, one bf16 rounding; with a next-layer norm, the row
// pairs and the token's partial sum of squares are stored for its tail.
__device__ __forceinline__ void down_combine(const LayerArgs& a, const float* part, const float* s_wts,
                                             int r0) {
  const int T = a.T, k = a.k;
  const bool next_norm = a.norm_next_w != nullptr;
  static_assert(kDecodeMaxT * kDownRowsPerBlock <= kDownThreads, "one (token, row) per thread");
  if ((int)threadIdx.x < T * kDownRowsPerBlock) {
    const int q = threadIdx.x;
    const int t = q / kDownRowsPerBlock;
    const int r = q - t * kDownRowsPerBlock;
    float o = part[(T * k + t) * kDownRowsPerBlock + r];
    for (int j = 0; j < k; ++j)
      o = fmaf(s_wts[t * k + j], part[(t * k + j) * kDownRowsPerBlock + r], o);
    if (a.resid) o += bf16_lo(a.resid[(size_t)t * H + r0 + r]);
    const uint16_t ob = f32_to_bf16_rne(o);
    if (!next_norm) {
      a.out[(size_t)t * H + r0 + r] = ob;
    } else {
      // The 8 rows of token t are 8 consecutive lanes of one wave: their
      // squares (of the stored bf16 values) summed in a fixed tree, the row
      // pairs stored as write-through 32-bit words for the norm tail.
      const float v = bf16_lo(ob);
      float ss = v * v;
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      const uint32_t odd = (uint32_t)__shfl_xor((int)ob, 1);
      if ((r & 1) == 0)
        store_coherent(reinterpret_cast<int32_t*>(a.out + (size_t)t * H + r0 + r), (int32_t)(ob | (odd << 16)));
      if (r == 0) store_coherent(a.ws.norm_part + (size_t)blockIdx.x * T + t, ss);
    }
  }
  if (next_norm) next_norm_tail(a);
}

// NVFP4 down + combine for small batches (2 <= T <= kDnSmallMaxT): the same
// row-owner blocks (block b: output rows [8b, 8b + 8)) as down_kernel, laid
// out so that all of a wave's loads are in flight together and every wait
// is exact.  Each wave reads its share of the routing table into registers
// (lane s: its s-th active expert), then the h rows it stages for the block
// (bf16, 1 KiB each; T k + T of them) and the shared expert's rows; once the
// table has arrived it requests all kS of its experts' codes (wave w:
// active experts w, w + 8, ...; an entry covers all of the expert's slots),
// parks the h rows in LDS and reduces the shared expert's token w and then
// each expert as its codes land.  Every wave issues the same loads whatever
// the batch (an index past the end repeats a valid one), and only ordinary
// loads precede the waits (with an LDS-direct load in flight the compiler
// waits for every load), so each wait leaves exactly the later loads in
// flight; only reductions are skipped.
constexpr int kDnSmallMaxT = 8;
constexpr int kDnSmallHRows = kDnSmallMaxT * kMaxTopK + kDnSmallMaxT;   // 72 rows of 1 KiB
constexpr int kDnSmallHVec = I / 8;                                     // 16-byte vectors per h row
constexpr int kDnSmallHPerWave = (kDnSmallHRows + kDownWaves - 1) / kDownWaves;
static_assert(kDnSmallHVec == kWave, "one h row per wave instruction");
static_assert(kDnSmallMaxT * kMaxTopK <= kDownWaves * 8 && kDnSmallMaxT * kMaxTopK <= kWave,
              "every active expert has a wave slot; every slot id a lane");

// Experts per wave (kS) for a batch: the eight waves cover T k slots.
__host__ __device__ constexpr int down_small_slots(int T, int k) { return T * k <= 6 * kDownWaves ? 6 : 8; }

__host__ __device__ constexpr bool down_small_applies(int T, bool nvfp4) {
  return nvfp4 && T >= 2 && T <= kDnSmallMaxT;
}

// One expert's tensor scale and its 8 rows of E2M1 codes and E4M3 block
// scales in a lane (lane l: columns [32 c, 32 c + 32), c = l % 16, of rows
// r0 + 4 i + l / 16).
struct DnCodes {
  float g;
  u32x4 q[2];
  uint16_t sc[2];
  __device__ __forceinline__ void load(const Bank& bank, int e, int r0) {
    g = bank.w2_gscale[e];
    const uint8_t* w2 = bank.w2 + (size_t)e * H * (I / 2);
    const uint8_t* s2 = bank.w2_scale + (size_t)e * H * (I / 16);
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = r0 + 4 * i + (lane >> 4);
      q[i] = load_stream(reinterpret_cast<const u32x4*>(w2 + (size_t)row * (I / 2)) + c);
      sc[i] = load_stream(reinterpret_cast<const uint16_t*>(s2 + (size_t)row * (I / 16)) + c);
    }
  }
};

// The vector of bf16 h row `row` that LDS position `lane` of the row holds:
// position 16 v + c takes vector 4 c + v, so that lane c's four reads
// (columns [32 c, 32 c + 32)) are consecutive across the 16 lanes of a row
// group.
__device__ __forceinline__ u32x4 load_h_vec(const float* h, int row) {
  const int lane = threadIdx.x & (kWave - 1);
  const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(h) + (size_t)row * I);
  return src[4 * (lane & 15) + (lane >> 4)];
}

// The partials of one expert entry for h rows hrow(j), j < n: per row, the
// two 16-column block sums scaled by their E4M3 scales, the 16 lanes of a
// row group summed in a fixed butterfly, times the tensor scale.
template <typename HRow>
__device__ __forceinline__ void dn_small_rows(const DnCodes& p, float g, const u32x4* hs, int n, HRow hrow,
                                              float* part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 15;
  u32x4 wv[2][4];
  float s_lo[2], s_hi[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t cw[4] = {p.q[i].x, p.q[i].y, p.q[i].z, p.q[i].w};
#pragma unroll
    for (int w = 0; w < 4; ++w)
      wv[i][w] = u32x4{fp4x2_to_bf16x2<0>(cw[w]), fp4x2_to_bf16x2<1>(cw[w]), fp4x2_to_bf16x2<2>(cw[w]),
                       fp4x2_to_bf16x2<3>(cw[w])};
    s_lo[i] = __builtin_amdgcn_cvt_f32_fp8((int)p.sc[i], 0);
    s_hi[i] = __builtin_amdgcn_cvt_f32_fp8((int)p.sc[i], 1);
  }
  for (int j = 0; j < n; ++j) {
    const int hr = hrow(j);
    const u32x4* hp = hs + hr * kDnSmallHVec + c;
    const u32x4 h0 = hp[0], h1 = hp[16], h2 = hp[32], h3 = hp[48];
    float v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float lo = dot8_bf16(wv[i][1], h1, dot8_bf16(wv[i][0], h0, 0.f));
      const float hi = dot8_bf16(wv[i][3], h3, dot8_bf16(wv[i][2], h2, 0.f));
      v[i] = fmaf(hi, s_hi[i], lo * s_lo[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v[i] += dpp<0xB1>(v[i]);    // lane ^ 1
      v[i] += dpp<0x4E>(v[i]);    // lane ^ 2
      v[i] += dpp<0x141>(v[i]);   // row_half_mirror: sums of 8
      v[i] += dpp<0x140>(v[i]);   // row_mirror: sums of 16
    }
    if (c == 0) {
      float* dst = part + hr * kDownRowsPerBlock + (lane >> 4);
      dst[0] = v[0] * g;
      dst[4] = v[1] * g;
    }
  }
}

template <int kS>
__global__ __launch_bounds__(kDownThreads) void down_small_kernel(LayerArgs a) {
  static_assert(kS < kWave, "a lane for the stand-in expert");
  __shared__ u32x4 hs[kDnSmallHRows * kDnSmallHVec];   // 72 KiB
  __shared__ float s_wts[kDnSmallMaxT * kMaxTopK];
  __shared__ float part[kDnSmallHRows * kDownRowsPerBlock];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int r0 = blockIdx.x * kDownRowsPerBlock;
  const int T = a.T, k = a.k, E = a.E;
  const int nh = T * k + T;
  const int32_t* route = a.ws.route;

  // The scheduling fences keep this issue order: table, h rows, shared
  // rows | experts, so that each wait leaves exactly the later loads in
  // flight.
  // 1. This wave's share of the routing table: lane s < kS the active index
  // i = w + 8 s (expert, slot range), the other lanes the first active
  // expert (the stand-in for indices past the end); lane l slot id l.
  const int li = lane < kS ? wave + lane * kDownWaves : 0;
  const int v_act = route[1 + min(li, E - 1)];
  const int v_off0 = route[1 + E + min(li, E)];
  const int v_off1 = route[1 + E + min(li + 1, E)];
  const int v_slot = route[2 + 2 * E + min(lane, T * k - 1)];
  const int v_n = route[0];
  const float v_wt = a.ws.wts[min((int)threadIdx.x, T * k - 1)];
  const float g_sh = a.shared.w2_gscale[0];
  __builtin_amdgcn_sched_barrier(0);
  // 2. The h rows this wave parks (w, w + 8, ...; past nh the last row
  // again, to its own place).
  u32x4 hv[kDnSmallHPerWave];
#pragma unroll
  for (int i = 0; i < kDnSmallHPerWave; ++i) hv[i] = load_h_vec(a.ws.h, min(wave + i * kDownWaves, nh - 1));
  // 3. The shared expert's rows (every wave: wave t reduces token t).
  DnCodes sh;
  sh.load(a.shared, 0, r0);
  __builtin_amdgcn_sched_barrier(0);
  const int n = __builtin_amdgcn_readfirstlane(v_n);
  const int act0 = __builtin_amdgcn_readlane(v_act, kS);

  // 4. All of this wave's experts, then the h rows into LDS as they land.
  DnCodes pe[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s)
    pe[s].load(a.routed, wave + s * kDownWaves < n ? __builtin_amdgcn_readlane(v_act, s) : act0, r0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kDnSmallHPerWave; ++i)
    hs[min(wave + i * kDownWaves, nh - 1) * kDnSmallHVec + lane] = hv[i];
  s_wts[min((int)threadIdx.x, T * k - 1)] = v_wt;   // past the end: the last weight again
  lds_barrier();
  if (wave < T) dn_small_rows(sh, g_sh, hs, 1, [&](int) { return T * k + wave; }, part);
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    if (wave + s * kDownWaves < n) {
      const int off = __builtin_amdgcn_readlane(v_off0, s);
      const int cnt = __builtin_amdgcn_readlane(v_off1, s) - off;
      dn_small_rows(pe[s], pe[s].g, hs, cnt, [&](int j) { return __builtin_amdgcn_readlane(v_slot, off + j); },
                    part);
    }
  }
  __syncthreads();
  down_combine(a, part, s_wts, r0);
}
// Both instances explicitly: with only the launch sites, the compiler can
// leave the second one's host handle undefined.
template __global__ void down_small_kernel<6>(LayerArgs);
template __global__ void down_small_kernel<8>(LayerArgs);

// ---------------------------------------------------------------- low-latency decode path

// The attention output projection with the residual add, for up to
// kLowLatMaxT tokens: block b owns output rows [8b, 8b + 8), wave w rows
// 8b + 2w and 8b + 2w + 1 (8 KiB of Wo each; lane l holds columns
// [8l + 512i, +8), i = 0..7), and the T tokens' attention rows are staged in
// LDS.  r1[t][row] = bf16(r[t][row] + sum_k Wo[row][k] a[t][k]) with fp32
// accumulation and one rounding; a wave stores its two rows of a token as
// one 32-bit word (kCoherent: write-through, for readers in the same launch).
constexpr int kAttnVec = kAttnWidth / 8;              // 512 16-byte vectors per row
constexpr int kAttnVecPerLane = kAttnVec / kWave;     // 8
constexpr int kOprojRows = H / kOprojBlocks;          // 8 per block
static_assert(kOprojRows == 2 * kRouteWaves, "two projection rows per wave");
static_assert(kAttnVec % kThreads == 0, "attention row staging");

struct OprojLds {
  u32x4 attn[kLowLatMaxT * kAttnVec];   // 64 KiB; then the router's chunk of normalised rows
  RouteLds route;
  float ss[kRouteWaves * kRouteXChunk];
  int flag;
};
static_assert(kRouteXChunk * kVecH <= kLowLatMaxT * kAttnVec, "router chunk fits the attention staging");

template <bool kCoherent>
__device__ __forceinline__ void oproj_rows(const LayerArgs& a, u32x4* xs_attn) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int row0 = blockIdx.x * kOprojRows + 2 * wave;
  const int T = a.T;
  u32x4 w[2][kAttnVecPerLane];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < kAttnVecPerLane; ++i)
      w[r][i] = load_stream(reinterpret_cast<const u32x4*>(a.wo + (size_t)(row0 + r) * kAttnWidth) + lane +
                            i * kWave);
  for (int j = 0; j < T; ++j)
#pragma unroll
    for (int u = 0; u < kAttnVec / kThreads; ++u) {
      const int v = threadIdx.x + u * kThreads;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(a.attn + (size_t)j * kAttnWidth) + v,
                                       (lds_ptr_t)(xs_attn + j * kAttnVec + (v & ~(kWave - 1))), 16, 0, 0);
    }
  // r's two entries of every token (one 32-bit word each), in flight with the rest.
  uint32_t rp[kLowLatMaxT];
#pragma unroll
  for (int j = 0; j < kLowLatMaxT; ++j)
    rp[j] = j < T ? *reinterpret_cast<const uint32_t*>(a.resid0 + (size_t)j * H + row0) : 0u;
  wait_vmem_all();
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kLowLatMaxT; ++j) {
    if (j >= T) break;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int i = 0; i < kAttnVecPerLane; ++i) {
      const u32x4 xv = xs_attn[j * kAttnVec + lane + i * kWave];
      acc0 = dot8_bf16(w[0][i], xv, acc0);
      acc1 = dot8_bf16(w[1][i], xv, acc1);
    }
    acc0 = wave_sum_lane63(acc0);
    acc1 = wave_sum_lane63(acc1);
    if (lane == kWave - 1) {
      const uint32_t r1 = pack_bf16x2_rne(bf16_lo(rp[j]) + acc0, bf16_hi(rp[j]) + acc1);
      int32_t* dst = reinterpret_cast<int32_t*>(a.ws.resid1 + (size_t)j * H + row0);
      if (kCoherent) store_coherent(dst, (int32_t)r1);
      else *dst = (int32_t)r1;
    }
  }
}

// The projection, and with kFused the routing fused into it ("vLLM Day-0
// Support for Recursive's Flint", section "Optimization Strategies", bullet
// "Low-Latency Decode Path"): every block takes a ticket once its r1 rows
// are stored; the last `routers` blocks to arrive become the router blocks
// (the ticket order makes the waits deadlock-free: a waiting block has
// finished its projection and holds one of at most `routers` of the chip's
// block slots while the rest of the grid, already started or free to start,
// completes), wait until every projection block has counted in, and run the
// pre-norm router and the routing tail on r1.
template <bool kFused>
__global__ __launch_bounds__(kThreads) void oproj_kernel(LayerArgs a) {
  __shared__ OprojLds S;
  oproj_rows<kFused>(a, S.attn);
  if constexpr (kFused) {
    drain_memory_ops();
    __syncthreads();
    if (threadIdx.x == 0)
      S.flag = (int)__hip_atomic_fetch_add(a.ws.header + kHdrOprojDone, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int ticket = S.flag;
    const int routers = (a.E + kRouterRows - 1) / kRouterRows;
    const int first = (int)gridDim.x - routers;
    if (ticket < first) return;
    route_norm_block<true>(a, ticket - first, routers, S.attn, S.route, S.ss, &S.flag, true);
  }
}

// The next layer's norm, fused into the down launch: every down block has
// stored its rows of out (r2) write-through and its per-token partial sums of
// their squares; the last block to finish adds the partials in a fixed order,
// and writes bf16(r2 / rms(r2) * gamma_next) for every token.
__device__ void next_norm_tail(const LayerArgs& a) {
  __shared__ float s_inv[kDecodeMaxT];
  __shared__ int s_flag;
  if (!last_block_ticket(a.ws.header + kHdrDownDone, gridDim.x, &s_flag)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int T = a.T;
  for (int t = wave; t < T; t += kDownWaves) {
    float v = 0.f;
    for (int b = lane; b < (int)gridDim.x; b += kWave) v += load_coherent(a.ws.norm_part + (size_t)b * T + t);
    v = wave_sum_lane63(v);
    if (lane == kWave - 1) s_inv[t] = rms_inv<H>(v, a.eps);
  }
  __syncthreads();
  const int vi = threadIdx.x & (kVecH - 1);
  const u32x4 g = reinterpret_cast<const u32x4*>(a.norm_next_w)[vi];
  for (int t = threadIdx.x / kVecH; t < T; t += kDownThreads / kVecH) {
    const u32x4 rv = load_coherent_x4(a.out + (size_t)t * H + 8 * vi);
    reinterpret_cast<u32x4*>(a.normed_next + (size_t)t * H)[vi] = rms_scale_bf16x8(rv, g, s_inv[t]);
  }
}

// ---------------------------------------------------------------- dense MLP

// Gate/up of the dense MLP: block u computes gate rows [8u, 8u + 8) and the
// matching up rows of w13 [2 I_d][H] for all T tokens (the routed gate/up
// scheme with the whole MLP as one group of tokens, x rows staged 8 at a
// time since every block sees all T tokens), h fp32 [T][I_d].
constexpr int kDenseXChunk = 8;   // 32 KiB of x rows in LDS
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5)))
void dense_gateup_kernel(DenseArgs a) {
  __shared__ u32x4 xs[kDenseXChunk * kVecH];
  const int p0 = blockIdx.x * kPairsPerItem;
  GateUpRows<false> wv;
  wv.load_rows(a.w13, a.inter, p0);
  gateup_compute<false, kDenseXChunk>(wv, p0, a.T, TokenList{nullptr, 1, 0}, a.x, a.h, xs, a.inter);
}

// Down of the dense MLP: block b owns output rows [8b, 8b + 8) for every
// token; wave w takes the 512-column K chunks w, w + 8, ... of those rows
// (lane l: columns [8l, 8l + 8) of a chunk), with the next chunk's rows in
// flight while it computes.  Tokens go in groups of 8 whose lane partials
// stay in registers across all of the wave's chunks and are reduced across
// lanes once per token; the 8 waves' sums meet in LDS and are added in wave
// order, then r (pre-norm block) and one bf16 rounding.
constexpr int kDenseG = 8;

// One wave's 8 rows x 8 columns of a w2 chunk, widened to fp32.
struct DenseW2Rows {
  u32x4 w[kDownRowsPerBlock];
  __device__ __forceinline__ void load(const DenseArgs& a, int r0, int c) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int r = 0; r < kDownRowsPerBlock; ++r)
      w[r] = load_stream(reinterpret_cast<const u32x4*>(a.w2 + (size_t)(r0 + r) * a.inter + c * kDenseChunk) + lane);
  }
  __device__ __forceinline__ void widen(float (&f)[kDownRowsPerBlock][8]) const {
#pragma unroll
    for (int r = 0; r < kDownRowsPerBlock; ++r) {
      f[r][0] = bf16_lo(w[r].x); f[r][1] = bf16_hi(w[r].x);
      f[r][2] = bf16_lo(w[r].y); f[r][3] = bf16_hi(w[r].y);
      f[r][4] = bf16_lo(w[r].z); f[r][5] = bf16_hi(w[r].z);
      f[r][6] = bf16_lo(w[r].w); f[r][7] = bf16_hi(w[r].w);
    }
  }
};

__device__ __forceinline__ void dense_accumulate(const DenseArgs& a, const float (&wf)[kDownRowsPerBlock][8],
                                                 int c, int t0, int G,
                                                 float (&acc)[kDenseG][kDownRowsPerBlock]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int t = 0; t < kDenseG; ++t) {
    if (t < G) {
      const f32x4* hp = reinterpret_cast<const f32x4*>(a.h + (size_t)(t0 + t) * a.inter + c * kDenseChunk) + lane * 2;
      const f32x4 h0 = hp[0], h1 = hp[1];
      const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
      for (int r = 0; r < kDownRowsPerBlock; ++r) {
        float s = acc[t][r];
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(wf[r][i], hv[i], s);
        acc[t][r] = s;
      }
    }
  }
}

__global__ __launch_bounds__(kDownThreads) void dense_down_kernel(DenseArgs a) {
  __shared__ float part[kDownWaves * kDenseG * kDownRowsPerBlock];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r0 = blockIdx.x * kDownRowsPerBlock;
  const int C = a.inter / kDenseChunk;
  for (int t0 = 0; t0 < a.T; t0 += kDenseG) {
    const int G = min(kDenseG, a.T - t0);
    float acc[kDenseG][kDownRowsPerBlock];
#pragma unroll
    for (int t = 0; t < kDenseG; ++t)
#pragma unroll
      for (int r = 0; r < kDownRowsPerBlock; ++r) acc[t][r] = 0.f;
    // The next chunk's rows are requested as soon as the current ones are
    // widened, so one chunk is always in flight while the wave computes.
    DenseW2Rows p;
    if (wave < C) p.load(a, r0, wave);
    for (int c = wave; c < C; c += kDownWaves) {
      float wf[kDownRowsPerBlock][8];
      p.widen(wf);
      if (c + kDownWaves < C) p.load(a, r0, c + kDownWaves);
      dense_accumulate(a, wf, c, t0, G, acc);
    }
#pragma unroll
    for (int t = 0; t < kDenseG; ++t) {
      const float tot = wave_sum8_transposed(acc[t]);
      if (lane < kDownRowsPerBlock)
        part[(wave * kDenseG + t) * kDownRowsPerBlock + bitrev3(lane)] = tot;
    }
    __syncthreads();
    if ((int)threadIdx.x < G * kDownRowsPerBlock) {
      const int t = threadIdx.x / kDownRowsPerBlock;
      const int r = threadIdx.x - t * kDownRowsPerBlock;
      float o = 0.f;
      for (int w = 0; w < kDownWaves; ++w) o += part[(w * kDenseG + t) * kDownRowsPerBlock + r];
      const size_t idx = (size_t)(t0 + t) * H + r0 + r;
      if (a.resid) o += bf16_lo(a.resid[idx]);
      a.out[idx] = f32_to_bf16_rne(o);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_dense_decode(const DenseArgs& a, hipStream_t stream, Launcher& launch) {
  launch(dense_gateup_kernel, dim3(a.inter / kPairsPerItem), dim3(kThreads), stream, a);
  launch(dense_down_kernel, dim3(H / kDownRowsPerBlock), dim3(kDownThreads), stream, a);
  return hipGetLastError();
}

// The down launch for a decode-sized batch: the small-batch kernel for
// NVFP4 weights at 2 <= T <= 8, the cached-entry form above T = 8 tokens.
template <bool kFp4>
static void launch_down(const LayerArgs& a, hipStream_t stream, Launcher& launch) {
  if (a.T > kRouteBareMinT)
    launch(down_kernel<kFp4, true>, dim3(H / kDownRowsPerBlock), dim3(kDownThreads), stream, a);
  else if (down_small_applies(a.T, kFp4) && down_small_slots(a.T, a.k) == 6)
    launch(down_small_kernel<6>, dim3(H / kDownRowsPerBlock), dim3(kDownThreads), stream, a);
  else if (down_small_applies(a.T, kFp4))
    launch(down_small_kernel<8>, dim3(H / kDownRowsPerBlock), dim3(kDownThreads), stream, a);
  else
    launch(down_kernel<kFp4, false>, dim3(H / kDownRowsPerBlock), dim3(kDownThreads), stream, a);
}

template <bool kFp4>
static hipError_t launch_decode_impl(const LayerArgs& a, hipStream_t stream, Launcher& launch) {
  const int n_router = (a.E + kRouterRows - 1) / kRouterRows;
  const int n_routed = min(a.E, a.T * a.k) * kUnitsPerExpert;
  const dim3 g_route(n_router), g_gateup(kUnitsPerExpert + n_routed);
  if (fused_routing_applies(a.T, a.k)) {
    if (a.norm_w)
      launch(route_kernel<true, true>, g_route, dim3(kThreads), stream, a);
    else
      launch(route_kernel<false, true>, g_route, dim3(kThreads), stream, a);
    launch(gateup_kernel<kFp4, true>, g_gateup, dim3(kThreads), stream, a);
  } else {
    if (a.norm_w)
      launch(route_kernel<true, false>, g_route, dim3(kThreads), stream, a);
    else if (a.T > kRouteBareMinT)
      launch(route_bare_kernel, g_route, dim3(kRouteBareThreads), stream, a);
    else
      launch(route_kernel<false, false>, g_route, dim3(route_threads(false, false)), stream, a);
    launch(gateup_kernel<kFp4, false>, g_gateup, dim3(kThreads), stream, a);
  }
  launch_down<kFp4>(a, stream, launch);
  return hipGetLastError();
}

hipError_t launch_decode(const LayerArgs& a, hipStream_t stream, Launcher& launch) {
  return a.nvfp4 ? launch_decode_impl<true>(a, stream, launch)
                 : launch_decode_impl<false>(a, stream, launch);
}

template <bool kFp4>
static hipError_t launch_lowlat_impl(const LayerArgs& a, bool fused, hipStream_t stream, Launcher& launch) {
  const int n_router = (a.E + kRouterRows - 1) / kRouterRows;
  const int n_routed = min(a.E, a.T * a.k) * kUnitsPerExpert;
  if (fused) {
    launch(oproj_kernel<true>, dim3(kOprojBlocks), dim3(kThreads), stream, a);
  } else {
    launch(oproj_kernel<false>, dim3(kOprojBlocks), dim3(kThreads), stream, a);
    launch(route_kernel<true, false>, dim3(n_router), dim3(kThreads), stream, a);
  }
  launch(gateup_kernel<kFp4, false>, dim3(kUnitsPerExpert + n_routed), dim3(kThreads), stream, a);
  if (fused) {
    launch_down<kFp4>(a, stream, launch);
  } else {
    LayerArgs b = a;
    b.norm_next_w = nullptr;
    launch_down<kFp4>(b, stream, launch);
    if (a.norm_next_w) launch_rmsnorm(a.out, a.norm_next_w, a.eps, a.normed_next, a.T, stream, launch);
  }
  return hipGetLastError();
}

hipError_t launch_lowlat(const LayerArgs& a, bool fused, hipStream_t stream, Launcher& launch) {
  static_assert(kOprojBlocks * (H / kOprojBlocks) == H, "projection rows");
  static_assert(kOprojBlocks >= (kMaxExperts + kRouterRows - 1) / kRouterRows, "router blocks");
  return a.nvfp4 ? launch_lowlat_impl<true>(a, fused, stream, launch)
                 : launch_lowlat_impl<false>(a, fused, stream, launch);
}

}  // namespace flint
