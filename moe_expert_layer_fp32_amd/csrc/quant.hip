// Per-row symmetric int8 quantisation for the W8A8 layer (gfx950).
//
// The pages quantise activations before they move and send the codes with
// their scales (page on DeepSeek-V3/R1 on Ascend (Huxiu), section
// 通信通信并发; int8 matmuls as QuantBatchMatmul, page "基于Atlas 900 A3
// SuperPoD的LongCat-Flash模型推理性能优化实践", section 优化措施三). Rule,
// per row: s = amax / 127 and q = clamp(rint(v / s), -127, 127), in fp32
// with correctly rounded division and round-half-to-even; a zero row gets
// s = 0 and q = 0. One workgroup per row: a max reduction, then the codes.
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ inline void load4(const void* in, int in_bf16, size_t off, float v[4]) {
  if (in_bf16) {
    const u32x2 p = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(in) + off);
    v[0] = __uint_as_float(p[0] << 16);
    v[1] = __uint_as_float(p[0] & 0xFFFF0000u);
    v[2] = __uint_as_float(p[1] << 16);
    v[3] = __uint_as_float(p[1] & 0xFFFF0000u);
  } else {
    const f32x4 p = *reinterpret_cast<const f32x4*>(static_cast<const float*>(in) + off);
    v[0] = p[0]; v[1] = p[1]; v[2] = p[2]; v[3] = p[3];
  }
}

// One workgroup of QUANT_THREADS per row: each thread loads its QUANT_V
// 4-column groups of the row in one batch (strided by the workgroup, so
// every load instruction is contiguous across the workgroup) and keeps them
// in registers, the row maximum meets in LDS, and the codes are made from
// the registers. Rows longer than QUANT_THREADS * QUANT_V * 4 take several
// batches (the second pass re-reads them).
constexpr int QUANT_THREADS = 256;
constexpr int QUANT_V = 8;

__global__ __launch_bounds__(QUANT_THREADS) void quant_rows_kernel(const void* in, int in_bf16, int cols,
                                                                   int max_rows, const int* offsets, int first,
                                                                   int n_groups, int8_t* q, float* s) {
  __shared__ float wmax[QUANT_THREADS / WAVE];
  const int r = blockIdx.x;
  const int rows = offsets ? offsets[first + n_groups] - offsets[first] : max_rows;
  if (r >= rows) return;   // whole workgroup
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const size_t base = size_t(r) * cols;
  constexpr int STEP = QUANT_THREADS * 4;   // columns per batch entry
  const int batches = ceil_div(cols, STEP * QUANT_V);
  float v[QUANT_V][4];
  auto load_batch = [&](int b) {
#pragma unroll
    for (int i = 0; i < QUANT_V; ++i) {
      const int c = (b * QUANT_V + i) * STEP + threadIdx.x * 4;
      if (c < cols) load4(in, in_bf16, base + c, v[i]);
      else v[i][0] = v[i][1] = v[i][2] = v[i][3] = 0.f;
    }
  };
  float amax = 0.f;
  for (int b = 0; b < batches; ++b) {
    load_batch(b);
#pragma unroll
    for (int i = 0; i < QUANT_V; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
  }
  amax = wave_max(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < QUANT_THREADS / WAVE; ++w) amax = fmaxf(amax, wmax[w]);
  const float sc = amax / 127.0f;
  for (int b = 0; b < batches; ++b) {
    if (batches > 1) load_batch(b);   // one batch: the registers still hold the row
#pragma unroll
    for (int i = 0; i < QUANT_V; ++i) {
      const int c = (b * QUANT_V + i) * STEP + threadIdx.x * 4;
      if (c >= cols) continue;
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float qf = 0.f;
        if (sc > 0.f) qf = fminf(fmaxf(rintf(v[i][j] / sc), -127.f), 127.f);
        packed |= (uint32_t(int32_t(qf)) & 0xFFu) << (8 * j);
      }
      *reinterpret_cast<uint32_t*>(q + base + c) = packed;
    }
  }
  if (threadIdx.x == 0) s[r] = sc;
}

hipError_t launch_quant_rows(const void* in, int in_bf16, int cols, int max_rows, const int* offsets,
                             int first, int n_groups, int8_t* q, float* s, hipStream_t stream) {
  if (max_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(max_rows), dim3(QUANT_THREADS), 0, stream, in, in_bf16, cols, max_rows,
                     offsets, first, n_groups, q, s);
  return hipGetLastError();
}

}  // namespace moe
