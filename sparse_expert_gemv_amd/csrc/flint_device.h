// Device-side helpers shared by the gfx950 kernels of the Flint MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

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

// Byte kByte of c holds two E2M1 codes (low nibble first); returns them as a
// packed bf16 pair (exact: every E2M1 value is a bf16 value).
template <int kByte>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, kByte));
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even, two values at a time (lo in bits
// 0..15): gfx950's packed conversion v_cvt_pk_bf16_f32 in the default
// rounding mode.  Checked on the device against the integer form
// (u + 0x7FFF + bit 16 of u) >> 16 for every non-NaN fp32 pattern: identical;
// NaN stays NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return (uint16_t)(pack_bf16x2_rne(f, 0.f) & 0xFFFFu);
}

// Sum of the squares of 8 bf16 values (one 16-byte vector), fp32.
__device__ __forceinline__ float sumsq_bf16x8(const u32x4& v) {
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

// RMSNorm's scale 1 / sqrt(mean of squares + eps) for a row of kN elements
// whose squares sum to `sumsq` (the form of "Flint on Arc Pro B70", section
// "norm.py: Triton kernels that assumed CUDA": a division by the square
// root, no approximate reciprocal square root).
template <int kN>
__device__ __forceinline__ float rms_inv(float sumsq, float eps) {
  return 1.0f / __builtin_sqrtf(sumsq * (1.0f / kN) + eps);
}

// bf16(x * inv * gamma) for 8 elements: x and gamma bf16, result RNE.
__device__ __forceinline__ u32x4 rms_scale_bf16x8(const u32x4& x, const u32x4& g, float inv) {
  const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_lo(xw[i]) * inv * bf16_lo(gw[i]);
    const float hi = bf16_hi(xw[i]) * inv * bf16_hi(gw[i]);
    o[i] = pack_bf16x2_rne(lo, hi);
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

// silu(g) = g * sigma(g), with the hardware reciprocal (about 1 ulp) in place
// of an IEEE division: a tenth of the instructions, which the prefill gate/up
// epilogue (64 of them per thread and tile) feels: 320 -> 312 us.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

// DPP move of v; lanes whose row is masked off, or whose source is out of
// range, read 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF, true));
}

// Weight loads: every weight byte is read once per forward, so the loads
// carry the non-temporal hint and do not displace the small data that is
// read many times (x, h, routing tables) from L2 and the Infinity Cache.
template <typename V>
__device__ __forceinline__ V load_stream(const V* p) { return __builtin_nontemporal_load(p); }

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

// Unsigned maximum over the 64 lanes, complete in lane 63 (0 is the
// identity: lanes outside a row mask and out-of-range sources read 0).
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, true);
}
// G independent maxima at once (their DPP chains interleave); lane 63.
template <int G>
__device__ __forceinline__ void wave_max_u32_lane63_multi(uint32_t (&v)[G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max(v[g], dpp_u32<0xB1>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max(v[g], dpp_u32<0x4E>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max(v[g], dpp_u32<0x141>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max(v[g], dpp_u32<0x140>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max(v[g], dpp_u32<0x142, 0xA>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max(v[g], dpp_u32<0x143, 0xC>(v[g]));
}
__device__ __forceinline__ uint32_t wave_max_u32_lane63(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  v = max(v, dpp_u32<0x142, 0xA>(v));
  v = max(v, dpp_u32<0x143, 0xC>(v));
  return v;
}

// Cross-block hand-off without whole-L2 writeback/invalidate: values that
// another block reads in the same launch are stored and loaded as relaxed
// agent-scope atomics (write-through / coherent-level accesses, "sc1"); a
// block drains its own outstanding memory operations (s_waitcnt 0) and
// synchronises before taking a completion ticket, so every value it stored
// is visible device-wide when the ticket is counted.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void drain_memory_ops() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Block-wide completion ticket: all threads drain their stores, then thread 0
// counts the block in; returns true (to every thread) in the block that
// completes the count of `expected` blocks, after resetting the counter.
__device__ __forceinline__ bool last_block_ticket(uint32_t* counter, uint32_t expected,
                                                  int* s_flag) {
  drain_memory_ops();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == expected - 1;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// DPP move of a 64-bit value (two 32-bit halves).
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, kCtrl, kRowMask, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), kCtrl, kRowMask, 0xF, true);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maxima over the 64 lanes of G independent values, returned to every lane;
// each step is applied to all G values before the next, so their DPP chains
// interleave.
template <int G>
__device__ __forceinline__ void wave_max_u64_multi(uint64_t (&v)[G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max_u64(v[g], dpp64<0xB1>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max_u64(v[g], dpp64<0x4E>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max_u64(v[g], dpp64<0x141>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max_u64(v[g], dpp64<0x140>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max_u64(v[g], dpp64<0x142, 0xA>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = max_u64(v[g], dpp64<0x143, 0xC>(v[g]));
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v[g], 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v[g] >> 32), 63);
    v[g] = ((uint64_t)hi << 32) | lo;
  }
}

// Maximum over the 64 lanes, returned to every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp64<0xB1>(v));
  v = max_u64(v, dpp64<0x4E>(v));
  v = max_u64(v, dpp64<0x141>(v));
  v = max_u64(v, dpp64<0x140>(v));
  v = max_u64(v, dpp64<0x142, 0xA>(v));
  v = max_u64(v, dpp64<0x143, 0xC>(v));
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, true);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, true);  // row_bcast:31
  return v;
}

}  // namespace flint
