// Weighted combine / unpermute for gfx950.
//
// The step after the experts: every token gathers the outputs of its k
// selections back into token order and sums them with its gate weights
// (the Combine of the Dispatch/Combine pair, page on DeepSeek-V3/R1 on
// Ascend (Huxiu), section MOE 算子优化), plus the always-on shared expert
// (same page, opening section: one shared expert per card). A
// zero-computation expert contributes its input (page "LongCat-Flash与
// GLM-4.6V ...", section 拆解MoE困局), read straight from x: it never enters
// the expert rows. One workgroup per token; each thread owns 4 consecutive
// columns; the sum runs in fp32 in a fixed order (shared, then slot 0..k-1)
// and is rounded once, so the result is deterministic without atomics.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int COMB_THREADS = 256;
constexpr int COMB_MAX_K = 16;

__global__ __launch_bounds__(COMB_THREADS) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  __shared__ int s_kind[COMB_MAX_K];    // 0 absent, 1 ffn row, 2 identity
  __shared__ int s_row[COMB_MAX_K];
  __shared__ float s_w[COMB_MAX_K];
  if (threadIdx.x < a.k) {
    const int j = threadIdx.x;
    const int e = a.topk_idx[size_t(t) * a.k + j];
    int kind = 0, row = -1;
    if (e >= a.ffn_begin && e < a.ffn_begin + a.n_ffn) {
      const int p = a.slot_pos[size_t(t) * a.k + j];
      if (p >= 0) {
        kind = 1;
        row = p - a.offsets[a.ffn_begin];
      }
    } else if (e >= a.zero_begin && e < a.zero_begin + a.n_zero) {
      kind = 2;
    }
    s_kind[j] = kind;
    s_row[j] = row;
    s_w[j] = a.topk_w[size_t(t) * a.k + j];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < a.d; c += COMB_THREADS * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (a.shared_rows) acc = *reinterpret_cast<const f32x4*>(a.shared_rows + size_t(t) * a.d + c);
    for (int j = 0; j < a.k; ++j) {
      const int kind = s_kind[j];
      const float w = s_w[j];
      if (kind == 1) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(a.rows + size_t(s_row[j]) * a.d + c);
        acc += w * u;
      } else if (kind == 2) {
        f32x4 u;
        if (a.x_bf16) {
          const u32x2 p = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.x) + size_t(t) * a.d + c);
          u = f32x4{__uint_as_float(p[0] << 16), __uint_as_float(p[0] & 0xFFFF0000u),
                    __uint_as_float(p[1] << 16), __uint_as_float(p[1] & 0xFFFF0000u)};
        } else {
          u = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + size_t(t) * a.d + c);
        }
        acc += w * u;
      }
    }
    if (a.x_bf16) {
      u32x2 p;
      p[0] = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
      p[1] = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.y) + size_t(t) * a.d + c) = p;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.y) + size_t(t) * a.d + c) = acc;
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(COMB_THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
