// One-time weight packing for gfx950 (not part of a layer call).
//
// The kernels stream weights as matrix-core operand fragments: a fragment is
// 16 output columns x KF reduction elements, stored lane by lane exactly as
// a wavefront loads it (lane l: column l % 16, reduction elements
// (l / 16) * KF/4 ...), so one fragment is one contiguous 1 KiB (bf16,
// int8) or 256 B (fp32) read. Blocks of 8 fragment columns (128 output
// columns) are stored one after the other; inside a block, step by step
// along the reduction, the planes of a step (W1 and W3 of the SwiGLU pair,
// or the three bf16 planes of the router) and in each plane the block's
// fragments side by side (frag_offset in common.h).
//
// Router planes: an fp32 weight w splits exactly into three bf16 values,
// hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid (each residual is exact
// in fp32 and the last fits bf16's 8 significant bits), so a bf16 x times
// each plane is an exact fp32 product and the router matmul keeps fp32
// accuracy on bf16 matrix cores.
#include "common.h"
#include "kernels.h"

namespace moe {

template <class Tr>
__global__ void pack_experts_kernel(const typename Tr::elem_t* __restrict__ src0,
                                    const typename Tr::elem_t* __restrict__ src1, int planes, int G,
                                    int K, int N, uint8_t* __restrict__ dst) {
  constexpr int PER = Tr::KF / 4;   // elements per lane
  const int KT = K / Tr::KF, NT = N / TILE_N;
  const size_t total = size_t(G) * NT * KT * planes * FRAG_LANES;
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < total; i += size_t(gridDim.x) * blockDim.x) {
    size_t r = i;
    const int lane = int(r % FRAG_LANES); r /= FRAG_LANES;
    const int p = int(r % planes); r /= planes;
    const int kt = int(r % KT); r /= KT;
    const int nt = int(r % NT); r /= NT;
    const int g = int(r);
    const typename Tr::elem_t* src = (p == 0) ? src0 : src1;
    const int n = nt * TILE_N + (lane & 15);
    const int k0 = kt * Tr::KF + (lane >> 4) * PER;
    typename Tr::elem_t v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = src[(size_t(g) * K + k0 + j) * N + n];
    constexpr int FB = frag_bytes<Tr>();
    const size_t o = size_t(g) * NT * KT * planes * FB + frag_offset(nt, kt, p, NT, KT, planes, FB) + lane * Tr::BPL;
    auto* out = reinterpret_cast<typename Tr::elem_t*>(dst + o);
#pragma unroll
    for (int j = 0; j < PER; ++j) out[j] = v[j];
  }
}

__device__ inline float bf16_trunc_value(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

template <int PLANES>
__global__ void pack_router_kernel(const float* __restrict__ wr, int K, int E, uint8_t* __restrict__ dst) {
  // PLANES == 1: fp32 fragments (KF 4); PLANES == 3: bf16 fragments (KF 32).
  constexpr int KF = PLANES == 1 ? TrF32::KF : TrBF16::KF;
  constexpr int PER = KF / 4;
  const int KT = K / KF, NT = ceil_div(E, TILE_N);
  const size_t total = size_t(NT) * KT * PLANES * FRAG_LANES;
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < total; i += size_t(gridDim.x) * blockDim.x) {
    size_t r = i;
    const int lane = int(r % FRAG_LANES); r /= FRAG_LANES;
    const int p = int(r % PLANES); r /= PLANES;
    const int kt = int(r % KT); r /= KT;
    const int nt = int(r);
    const int n = nt * TILE_N + (lane & 15);
    const int k0 = kt * KF + (lane >> 4) * PER;
    constexpr int BPL = PLANES == 1 ? TrF32::BPL : TrBF16::BPL;
    const size_t o = frag_offset(nt, kt, p, NT, KT, PLANES, FRAG_LANES * BPL) + lane * BPL;
    if (PLANES == 1) {
      *reinterpret_cast<float*>(dst + o) = n < E ? wr[size_t(k0) * E + n] : 0.f;
    } else {
      uint16_t* out = reinterpret_cast<uint16_t*>(dst + o);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const float w = n < E ? wr[size_t(k0 + j) * E + n] : 0.f;
        const uint16_t hi = f32_to_bf16(w);
        const float r1 = w - bf16_trunc_value(hi);
        const uint16_t mid = f32_to_bf16(r1);
        const float r2 = r1 - bf16_trunc_value(mid);
        const uint16_t lo = f32_to_bf16(r2);
        out[j] = p == 0 ? hi : (p == 1 ? mid : lo);
      }
    }
  }
}

hipError_t launch_pack_experts(const void* src0, const void* src1, int planes, GemmElem elem, int G, int K,
                               int N, void* dst, hipStream_t stream) {
  const dim3 grid(2048), block(256);
  switch (elem) {
    case ELEM_BF16:
      hipLaunchKernelGGL(pack_experts_kernel<TrBF16>, grid, block, 0, stream,
                         static_cast<const uint16_t*>(src0), static_cast<const uint16_t*>(src1), planes, G, K,
                         N, static_cast<uint8_t*>(dst));
      break;
    case ELEM_I8:
      hipLaunchKernelGGL(pack_experts_kernel<TrI8>, grid, block, 0, stream, static_cast<const int8_t*>(src0),
                         static_cast<const int8_t*>(src1), planes, G, K, N, static_cast<uint8_t*>(dst));
      break;
    case ELEM_F32:
      hipLaunchKernelGGL(pack_experts_kernel<TrF32>, grid, block, 0, stream, static_cast<const float*>(src0),
                         static_cast<const float*>(src1), planes, G, K, N, static_cast<uint8_t*>(dst));
      break;
  }
  return hipGetLastError();
}

hipError_t launch_pack_router(const float* wr, GemmElem elem, int K, int E, void* dst, hipStream_t stream) {
  const dim3 grid(1024), block(256);
  if (elem == ELEM_F32)
    hipLaunchKernelGGL(pack_router_kernel<1>, grid, block, 0, stream, wr, K, E, static_cast<uint8_t*>(dst));
  else
    hipLaunchKernelGGL(pack_router_kernel<3>, grid, block, 0, stream, wr, K, E, static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

}  // namespace moe
