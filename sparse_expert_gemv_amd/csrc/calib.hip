// Streaming-read probe: the HBM read rate a plain, perfectly coalesced stream
// reaches on this part, measured so that the layer's achieved bandwidth can be
// set beside what is achievable as well as beside the nominal 8 TB/s.  It
// reads every 16-byte vector of a buffer once with non-temporal loads (as the
// layer reads its weights) and folds the words into one XOR per block, so the
// loads cannot be dropped and the result can be checked on the host.

#include "flint_device.h"
#include "flint_moe.h"

namespace flint {
namespace {

// One-shot blocks, as the layer's gate/up launch reads its weights: block b
// owns the contiguous 64 KiB at b * 64 KiB and issues all of its loads
// before it uses any (16 vectors of 16 bytes per thread), then exits; a grid
// of ceil(bytes / 64 KiB) blocks covers the buffer.
constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 16;
constexpr size_t kCalibChunkVec = (size_t)kCalibThreads * kCalibUnroll;   // 64 KiB
static_assert(FLINT_MOE_CALIB_SINK_WORDS % 4 == 0, "sink size");

__global__ __launch_bounds__(kCalibThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                    size_t n, uint32_t* sink) {
  __shared__ uint32_t s_acc[kCalibThreads / kWave];
  const size_t base = (size_t)blockIdx.x * kCalibChunkVec + threadIdx.x;
  u32x4 v[kCalibUnroll];
#pragma unroll
  for (int u = 0; u < kCalibUnroll; ++u) {
    const size_t i = base + (size_t)u * kCalibThreads;
    v[u] = i < n ? load_stream(src + i) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kCalibUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & (kWave - 1)) == 0) s_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0;
#pragma unroll
    for (int w = 0; w < kCalibThreads / kWave; ++w) b ^= s_acc[w];
    atomicXor(sink + blockIdx.x % FLINT_MOE_CALIB_SINK_WORDS, b);
  }
}

}  // namespace
}  // namespace flint

extern "C" __attribute__((visibility("default"))) flint_status flint_moe_calib_stream_read(
    const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0 ||
      (uintptr_t)sink % 4 != 0)
    return FLINT_ERR_INVALID_ARG;
  const size_t n = bytes / 16;
  const size_t blocks = (n + flint::kCalibChunkVec - 1) / flint::kCalibChunkVec;
  if (blocks > 0x7FFFFFFFu) return FLINT_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(flint::stream_read_kernel, dim3((unsigned)blocks), dim3(flint::kCalibThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<const flint::u32x4*>(src), n,
                     sink);
  return hipGetLastError() == hipSuccess ? FLINT_OK : FLINT_ERR_HIP;
}
