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
// columns; the sum runs in fp32 in a fixed order (shared row, the expert
// rows in slot order, then x times the summed identity weights) and is
// rounded once, so the result is deterministic without atomics.
#include "common.h"
#include "kernels.h"
#include <type_traits>

namespace moe {

constexpr int COMB_THREADS = 256;
constexpr int COMB_MAX_K = 16;

// Four consecutive values of an expert-output row, fp32 or bf16 (RB).
template <bool RB>
struct Row4 {
  using raw = typename std::conditional<RB, u32x2, f32x4>::type;
  static __device__ __forceinline__ raw load(const void* base, size_t off) {
    return RB ? *reinterpret_cast<const raw*>(static_cast<const uint16_t*>(base) + off)
              : *reinterpret_cast<const raw*>(static_cast<const float*>(base) + off);
  }
  static __device__ __forceinline__ f32x4 widen(raw v) {
    if constexpr (RB)
      return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
                   __uint_as_float(v[1] & 0xFFFF0000u)};
    else
      return v;
  }
};

// KMAX >= k: the rows of a column chunk are all loaded before any is added,
// so the loads of a chunk are in flight together. Sum order: shared row,
// expert rows in selection order, then the identity part (x times the
// summed identity weights). RB: the expert rows are bf16.
template <int KMAX, bool RB>
__global__ __launch_bounds__(COMB_THREADS) void combine_kernel(CombineArgs a) {
  using R = Row4<RB>;
  const int t = blockIdx.x;
  // The token's expert rows in selection order (compacted), their weights,
  // and the summed weight of its identity selections.
  __shared__ int s_row[COMB_MAX_K];
  __shared__ float s_w[COMB_MAX_K];
  __shared__ int s_n;
  __shared__ float s_wid;
  // Lane j of the first wavefront reads selection j (all k at once), the
  // expert rows are compacted in selection order with a ballot, and the
  // identity weights are added in selection order.
  if (threadIdx.x < WAVE) {
    const int j = threadIdx.x;
    int e = -1, p = -1;
    float w = 0.f;
    if (j < a.k) {
      e = a.topk_idx[size_t(t) * a.k + j];
      w = a.topk_w[size_t(t) * a.k + j];
      p = a.slot_pos[size_t(t) * a.k + j];
    }
    const int base = a.offsets[a.ffn_begin];
    const bool row = j < a.k && e >= a.ffn_begin && e < a.ffn_begin + a.n_ffn && p >= 0;
    const bool ident = j < a.k && e >= a.zero_begin && e < a.zero_begin + a.n_zero;
    const uint64_t rows = __ballot(row);
    if (row) {
      const int q = __popcll(rows & ((1ull << j) - 1));
      s_row[q] = p - base;
      s_w[q] = w;
    }
    const float wz = ident ? w : 0.f;
    float wid = 0.f;
    for (int jj = 0; jj < a.k; ++jj) wid += __shfl(wz, jj, WAVE);
    if (j == 0) {
      s_n = __popcll(rows);
      s_wid = wid;
    }
  }
  __syncthreads();
  const int n = s_n;
  const float wid = s_wid;
  for (int c = threadIdx.x * 4; c < a.d; c += COMB_THREADS * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (a.shared_rows) acc = R::widen(R::load(a.shared_rows, size_t(t) * a.d + c));
    // all row loads of the chunk first (n is the same for the workgroup)
    typename R::raw u[KMAX];
#pragma unroll
    for (int q = 0; q < KMAX; ++q)
      if (q < n) u[q] = R::load(a.rows, size_t(s_row[q]) * a.d + c);
    f32x4 ux = {0.f, 0.f, 0.f, 0.f};
    if (wid != 0.f) {
      if (a.x_bf16) {
        const u32x2 p = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.x) + size_t(t) * a.d + c);
        ux = f32x4{__uint_as_float(p[0] << 16), __uint_as_float(p[0] & 0xFFFF0000u), __uint_as_float(p[1] << 16),
                   __uint_as_float(p[1] & 0xFFFF0000u)};
      } else {
        ux = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + size_t(t) * a.d + c);
      }
    }
#pragma unroll
    for (int q = 0; q < KMAX; ++q)
      if (q < n) acc += s_w[q] * R::widen(u[q]);
    if (wid != 0.f) acc += wid * ux;
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

template <bool RB>
hipError_t launch_combine_k(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(a.T), block(COMB_THREADS);
  if (a.k <= 2) hipLaunchKernelGGL((combine_kernel<2, RB>), grid, block, 0, stream, a);
  else if (a.k <= 4) hipLaunchKernelGGL((combine_kernel<4, RB>), grid, block, 0, stream, a);
  else if (a.k <= 8) hipLaunchKernelGGL((combine_kernel<8, RB>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((combine_kernel<16, RB>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  if (a.rows_bf16) return launch_combine_k<true>(a, stream);
  return launch_combine_k<false>(a, stream);
}

}  // namespace moe
