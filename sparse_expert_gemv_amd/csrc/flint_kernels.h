// Launch interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace flint {

constexpr int kHidden = 2048;      // H
constexpr int kInter = 512;        // I
constexpr int kMaxExperts = 256;   // E upper bound (four router scores per lane)
constexpr int kMaxTopK = 8;
constexpr int kDecodeMaxT = 64;    // largest T taken by the GEMV (decode) kernels
constexpr int kPrefillTile = 32;   // tokens per router / scatter block (prefill-sized T)
constexpr int kGroupTile = 256;    // slots per grouped-GEMM M-tile (prefill-sized T)
// Workspace header: uint32 completion counters, each on its own 256-byte
// line so that tickets on one never queue behind atomics on another.  All
// are zero before a forward starts and zero after it ends.
constexpr int kLine = 64;                       // words per 256-byte line
constexpr int kHdrRouterDone = 0 * kLine;       // decode: router blocks done
constexpr int kHdrOprojDone = 1 * kLine;        // low-latency path: projection blocks done
constexpr int kHdrDownDone = 2 * kLine;         // low-latency path: down blocks done
constexpr int kHdrWaitExpired = 3 * kLine;      // set to 1 if a bounded wait ever gave up
constexpr int kHeaderWords = 84 * kLine;        // 21 KiB

// Low-latency decode path (the attention output projection, the MoE layer
// and the next layer's norm around it), for up to kLowLatMaxT tokens.
constexpr int kLowLatMaxT = 8;
constexpr int kAttnWidth = 4096;                // attention output: 32 heads x 128
constexpr int kOprojBlocks = 256;               // projection blocks (8 output rows each)

// Routing table (int32), written once per forward by the block that
// finishes routing:
//   [0]                      |U|
//   [1, 1 + E)               U, ascending expert ids (first |U| valid)
//   [1 + E, 2 + 2E)          offsets by active index: slots of U[a] are
//                            slots[off[a], off[a + 1]), off[|U|] = T*k
//   [2 + 2E, 2 + 2E + T*k)   slot ids s = t*k + j, grouped by active index,
//                            ascending within a group
__host__ __device__ constexpr int route_table_ints(int E, int T, int k) { return 2 + 2 * E + T * k; }
// Item records (decode-sized T, written with the routing table): record a
// (a < |U|) = {U[a], slot count c, its c slots ascending}, a fixed stride of
// item_record_ints(T) ints (an expert holds at most T slots), so that a
// gate/up block reads its expert and token list in one round trip.
__host__ __device__ constexpr int item_record_ints(int T) { return 2 + T; }

// Regions used only by the prefill-sized path.
struct PrefillWs {
  int32_t* counts;    // [nb][E]: slots per (router block of kPrefillTile tokens, expert)
  int32_t* tiles;     // [0] = routed tiles; then (expert, start, count) per kGroupTile-slot tile
  int32_t* pos;       // [T*k]: sorted position of slot s
  _Float16* h16;      // [T*k + T][I]: h in sorted slot order, then the shared expert's
  _Float16* y16;      // [T*k][H]: unweighted down projection per sorted slot
};

// Workspace regions, as device pointers.
struct Workspace {
  uint32_t* header;   // kHeaderWords counters (see above)
  float* logits;      // [T][E]
  int32_t* ids;       // [T][k]
  float* wts;         // [T][k]
  int32_t* route;     // routing table (see above)
  float* h;           // [T*k + T][I] (decode-sized T)
  int32_t* items;     // [min(E, T*k)][item_record_ints(T)] item records (decode-sized T)
  uint16_t* resid1;   // low-latency path: r1 = bf16(r + Wo a) [T][H]
  float* norm_part;   // low-latency path: per down block, per token sums of squares [blocks][T]
  PrefillWs pre;      // prefill-sized T
  void* extra;
};

// Weights of one bank in the form the kernels read them.
struct Bank {
  const uint8_t* w13;        // per expert: bf16 [2I][H] or E2M1 [2I][H/2]
  const uint8_t* w2;         // per expert: bf16 [H][I]  or E2M1 [H][I/2]
  const uint8_t* w13_scale;  // NVFP4: E4M3 [2I][H/16]
  const uint8_t* w2_scale;   // NVFP4: E4M3 [H][I/16]
  const float* w13_gscale;   // NVFP4: [n]
  const float* w2_gscale;    // NVFP4: [n]
};

struct LayerArgs {
  const uint16_t* x;         // [T][H]: the layer's input (the block's normalised r)
  uint16_t* out;             // [T][H]
  // Pre-norm block only (all nullptr for the bare layer): x is the workspace
  // buffer `normed`, filled by the first kernel from r and gamma; the last
  // kernel adds r to the output before its bf16 rounding.
  const uint16_t* resid;     // r [T][H]
  const uint16_t* norm_w;    // gamma [H]
  uint16_t* normed;          // [T][H], == x
  float eps;
  // Low-latency decode path only (nullptr otherwise): the first kernel
  // computes r1 = bf16(resid0 + wo attn) into ws.resid1, which is then the
  // block's r (resid); with norm_next_w the down kernel also writes the next
  // layer's normalised input bf16(RMSNorm(out) * norm_next_w) to normed_next.
  const uint16_t* attn;      // [T][kAttnWidth]
  const uint16_t* wo;        // [H][kAttnWidth]
  const uint16_t* resid0;    // r [T][H]
  const uint16_t* norm_next_w;   // gamma_next [H] or nullptr
  uint16_t* normed_next;     // [T][H]
  const uint16_t* router_w;  // [E][H]
  const float* router_b;     // [E] or nullptr
  Bank routed, shared;
  int32_t* ids_out;          // caller copy or nullptr
  float* wts_out;            // caller copy or nullptr
  Workspace ws;
  int T, E, k;
  int renormalize;
  float routed_scale;
  int nvfp4;
};

// Launches the path's kernels.  With timing events, kernel i is launched with
// hipExtLaunchKernelGGL so that events[2i] and events[2i+1] take the start and
// end timestamps of that kernel's own execution (see flint_moe_forward_timed).
struct Launcher {
  hipEvent_t* events = nullptr;
  int n = 0;
  int used = 0;   // kernels launched so far
  template <typename F, typename... Args>
  void operator()(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
    if (events && 2 * used + 1 < n)
      hipExtLaunchKernelGGL(kernel, grid, block, 0, s, events[2 * used], events[2 * used + 1], 0,
                            args...);
    else
      hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
    ++used;
  }
};

// Dense SwiGLU MLP (Flint's layers 0 and 1): out = W2 (silu(W13[0:I] x) *
// W13[I:2I] x) (+ r for the pre-norm block), bf16 weights.
constexpr int kDenseChunk = 512;          // K columns of w2 per decode work item
constexpr int kDenseMaxInter = 32768;     // I_d upper bound (multiple of kDenseChunk)
struct DenseArgs {
  const uint16_t* x;       // [T][H] the MLP's input (the block's normalised r)
  uint16_t* out;           // [T][H]
  const uint16_t* resid;   // r [T][H] for the pre-norm block, else nullptr
  const uint16_t* w13;     // [2 I][H], rows [0, I) gate, [I, 2I) up
  const uint16_t* w2;      // [H][I]
  float* h;                // [T][I] fp32 (decode-sized T; bf16, 1 KiB rows, for NVFP4)
  _Float16* h16;           // [T][I] fp16 (prefill-sized T)
  int T, inter;
};

// RMSNorm of T rows of kHidden: n = bf16(r / sqrt(mean(r^2) + eps) * gamma),
// one wave per row.
void launch_rmsnorm(const uint16_t* r, const uint16_t* gamma, float eps, uint16_t* n, int T,
                    hipStream_t stream, Launcher& launch);

// The dense MLP for T <= kDecodeMaxT (GEMV kernels) and for larger T (MFMA).
hipError_t launch_dense_decode(const DenseArgs& a, hipStream_t stream, Launcher& launch);
hipError_t launch_dense_prefill(const DenseArgs& a, hipStream_t stream, Launcher& launch);

// The decode path (T <= kDecodeMaxT) for bf16 or NVFP4 expert weights.
hipError_t launch_decode(const LayerArgs& a, hipStream_t stream, Launcher& launch);

// The low-latency decode path (T <= kLowLatMaxT).  fused: three launches
// (projection + residual + norm + router + routing; gate/up; down + residual
// + next norm); otherwise five (projection + residual; norm + router +
// routing; gate/up; down + residual; next norm).
hipError_t launch_lowlat(const LayerArgs& a, bool fused, hipStream_t stream, Launcher& launch);

// The prefill path (T > kDecodeMaxT), bf16 expert weights.
hipError_t launch_prefill(const LayerArgs& a, hipStream_t stream, Launcher& launch);
int prefill_tiles_max(int T, int E, int k);

}  // namespace flint
