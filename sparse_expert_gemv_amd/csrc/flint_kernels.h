// Launch interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flint {

constexpr int kHidden = 2048;      // H
constexpr int kInter = 512;        // I
constexpr int kMaxExperts = 256;   // E upper bound (four router scores per lane)
constexpr int kMaxTopK = 8;
constexpr int kDecodeMaxT = 64;    // largest T taken by the GEMV (decode) kernels
constexpr int kHeaderWords = 1024;  // workspace header: uint32 counters (4 KiB)

// Header words.  All are zero before a forward starts and zero after it ends.
constexpr int kHdrTokensDone = 0;   // tokens whose selection is complete
constexpr int kHdrRoutingDone = 1;  // 1 once every token is routed
constexpr int kHdrNActive = 2;      // |U|
constexpr int kHdrExit = 3;         // blocks that finished all their items
constexpr int kHdrError = 4;        // sticky: a bounded wait timed out
constexpr int kHdrSharedDone = 5;   // shared-expert gate/up items done
constexpr int kHdrTokTicket = 64;   // [64]  router items done per token
constexpr int kHdrCounts = 128;     // [256] slots routed to each expert
constexpr int kHdrExpertDone = 384; // [256] gate/up items done per active index
constexpr int kHdrTileTicket = 640; // [32]  down items done per 64-row output tile

// Workspace regions, as device pointers.
struct Workspace {
  uint32_t* header;   // kHeaderWords counters (see above)
  float* logits;      // [T][E]
  int32_t* ids;       // [T][k]
  float* wts;         // [T][k]
  int32_t* active;    // [E]: the union U, first n_active entries, in completion order
  int32_t* lists;     // [E][T]: slot ids routed to expert e, first counts[e] entries
  float* h;           // [T*k + T][I]
  float* y;           // [T*k + T][H]: per-slot down projections (unweighted)
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
  const uint16_t* x;         // [T][H]
  uint16_t* out;             // [T][H]
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

// Optional per-kernel timing: records events[used++] on the stream before each
// kernel and once after the last (see flint_moe_forward_timed).
struct StageEvents {
  hipEvent_t* events = nullptr;
  int n = 0;
  int used = 0;
  void mark(hipStream_t s) {
    if (events && used < n) hipEventRecord(events[used++], s);
  }
};

// Blocks a decode launch may use on the current device (resident capacity).
int decode_grid_limit();

hipError_t launch_decode_bf16(const LayerArgs& a, int grid_limit, hipStream_t stream,
                              StageEvents* ev);

}  // namespace flint
