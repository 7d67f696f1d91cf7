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
constexpr int kHeaderWords = 256;  // workspace header: uint32 counters
constexpr int kTokCounterBase = 64;

// Workspace regions, as device pointers.
struct Workspace {
  uint32_t* header;   // [0]: tokens-done counter; [64 + t]: router blocks done for token t
  float* logits;      // [T][E]
  int32_t* ids;       // [T][k]
  float* wts;         // [T][k]
  int32_t* n_active;  // [1]
  int32_t* active;    // [E]
  int32_t* counts;    // [E]
  int32_t* offsets;   // [E + 1]
  int32_t* slots;     // [T*k]
  float* h;           // [T*k + T][I]
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

hipError_t launch_decode_bf16(const LayerArgs& a, hipStream_t stream, StageEvents* ev);

}  // namespace flint
