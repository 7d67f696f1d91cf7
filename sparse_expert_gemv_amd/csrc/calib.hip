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

constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 8;   // 128 bytes of loads in flight per thread
static_assert(FLINT_MOE_CALIB_SINK_WORDS % 4 == 0, "sink size");

__global__ __launch_bounds__(kCalibThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                    size_t n, uint32_t* sink) {
  __shared__ uint32_t s_acc[kCalibThreads / kWave];
  const size_t stride = (size_t)gridDim.x * kCalibThreads;
  size_t i = (size_t)blockIdx.x * kCalibThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kCalibUnroll - 1) * stride < n; i += kCalibUnroll * stride) {
    u32x4 v[kCalibUnroll];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) v[u] = load_stream(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = load_stream(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & (kWave - 1)) == 0) s_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0;
#pragma unroll
    for (int w = 0; w < kCalibThreads / kWave; ++w) b ^= s_acc[w];
    sink[blockIdx.x] = b;
  }
}

}  // namespace
}  // namespace flint

extern "C" __attribute__((visibility("default"))) flint_status flint_moe_calib_stream_read(
    const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0 ||
      (uintptr_t)sink % 4 != 0)
    return FLINT_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(flint::stream_read_kernel, dim3(FLINT_MOE_CALIB_SINK_WORDS),
                     dim3(flint::kCalibThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const flint::u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? FLINT_OK : FLINT_ERR_HIP;
}
