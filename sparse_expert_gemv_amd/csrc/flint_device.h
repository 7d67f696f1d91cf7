// Device-side helpers shared by the gfx950 kernels of the Flint MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// a.lo*b.lo + a.hi*b.hi + c for two packed bf16 pairs, fp32 accumulate
// (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Eight bf16 products of two 16-byte vectors accumulated into c.
__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& b, float c) {
  c = dot2_bf16(a.x, b.x, c);
  c = dot2_bf16(a.y, b.y, c);
  c = dot2_bf16(a.z, b.z, c);
  c = dot2_bf16(a.w, b.w, c);
  return c;
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// SiLU in the form g / (1 + exp(-g)).
__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

// DPP move of v; lanes whose row is masked off, or whose source is out of
// range, read 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF, true));
}

// Sum over the 64 lanes of a wave; the total is valid in lane 63.
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v += dpp<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);       // row_half_mirror: sums of 8
  v += dpp<0x140>(v);       // row_mirror: sums of 16
  v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Device-scope (all XCDs) completion ticket: returns the previous count.
// Release of this block's earlier global writes, acquire of the others'.
__device__ __forceinline__ uint32_t ticket_acq_rel(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_release_zero(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace flint
