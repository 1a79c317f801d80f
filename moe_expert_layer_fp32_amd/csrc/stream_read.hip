// Streaming read of a device buffer: the practical HBM read ceiling that the
// weight-streaming products are measured against (gfx950).
//
// Each of STREAM_READ_WGS workgroups reads one contiguous slice of the
// buffer front to back with 16-byte loads, STREAM_READ_AHEAD loads per
// thread in flight, and folds what it read with XOR into one 32-bit word
// (written to sink[workgroup]), so no load can be dropped and the result is
// checkable: the XOR of all sink words equals the XOR of the buffer's 32-bit
// words.
#include <cstdint>

#include "common.h"
#include "moe.h"

namespace moe {

constexpr int STREAM_READ_THREADS = 512;   // with 2048 workgroups: the fastest shape measured (2 GiB, ~6.2-6.3 TB/s)
constexpr int STREAM_READ_AHEAD = 4;

__global__ __launch_bounds__(STREAM_READ_THREADS) void stream_read_kernel(const u32x4* __restrict__ src, size_t words,
                                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[STREAM_READ_THREADS / WAVE];
  const size_t per = (words + gridDim.x - 1) / gridDim.x;
  const size_t w0 = blockIdx.x * per;
  const size_t w1 = w0 + per < words ? w0 + per : words;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = w0 + threadIdx.x;
  constexpr size_t STEP = size_t(STREAM_READ_THREADS) * STREAM_READ_AHEAD;
  for (; i + (STREAM_READ_AHEAD - 1) * STREAM_READ_THREADS < w1; i += STEP) {
    u32x4 v[STREAM_READ_AHEAD];
#pragma unroll
    for (int d = 0; d < STREAM_READ_AHEAD; ++d) v[d] = src[i + size_t(d) * STREAM_READ_THREADS];
#pragma unroll
    for (int d = 0; d < STREAM_READ_AHEAD; ++d) acc ^= v[d];
  }
  for (; i < w1; i += STREAM_READ_THREADS) acc ^= src[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = WAVE / 2; o > 0; o >>= 1) x ^= uint32_t(__shfl_xor(int(x), o, WAVE));
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  if (lane == 0) part[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int w = 0; w < STREAM_READ_THREADS / WAVE; ++w) y ^= part[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace moe

extern "C" moe_status moe_stream_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (bytes == 0) return MOE_OK;
  if (!buf || !sink || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(moe::stream_read_kernel, dim3(MOE_STREAM_READ_WGS), dim3(moe::STREAM_READ_THREADS), 0,
                     static_cast<hipStream_t>(stream), static_cast<const moe::u32x4*>(buf), bytes / 16,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
