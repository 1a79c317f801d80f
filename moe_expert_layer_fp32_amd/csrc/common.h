// Device-side types and helpers shared by the gfx950 kernels of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int FRAG_LANES = 64;   // one matrix-core operand = 64 lanes
constexpr int TILE_N = 16;       // output columns per fragment
constexpr int ROW_BLOCK = 16;    // rows (tokens) per matrix-core column block
constexpr int MAX_ROW_BLOCKS = 8;
constexpr int TILE_M = ROW_BLOCK * MAX_ROW_BLOCKS;  // 128 rows per m-tile
constexpr int WG_WAVES = 4;
constexpr int WG_THREADS = WG_WAVES * WAVE;
constexpr int WG_N = WG_WAVES * TILE_N;             // 64 output columns per workgroup

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---------------------------------------------------------------------------
// Matrix-core traits. Each trait describes one 16x16 output MFMA family:
// operand A is a 16 (rows) x KF (reduction) tile, B a KF x 16 tile; lane l
// holds row / column (l % 16) and the KF/4 reduction elements starting at
// (l / 16) * KF/4, i.e. BPL contiguous bytes of a row-major row. The
// accumulator lane l holds D[(l/16)*4 + j][l % 16], j = 0..3.
// ---------------------------------------------------------------------------
struct TrBF16 {
  using op_t = bf16x8;
  using acc_t = f32x4;
  using elem_t = uint16_t;
  static constexpr int KF = 32;
  static constexpr int BPL = 16;
  __device__ static inline acc_t mfma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t load(const uint8_t* p) {
    return __builtin_bit_cast(op_t, *reinterpret_cast<const u32x4*>(p));
  }
  __device__ static inline acc_t zero() { return acc_t{0.f, 0.f, 0.f, 0.f}; }
  __device__ static inline float to_f32(acc_t a, int j) { return a[j]; }
};

struct TrI8 {
  using op_t = i32x4;   // 16 int8 codes
  using acc_t = i32x4;
  using elem_t = int8_t;
  static constexpr int KF = 64;
  static constexpr int BPL = 16;
  __device__ static inline acc_t mfma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t load(const uint8_t* p) {
    return __builtin_bit_cast(op_t, *reinterpret_cast<const u32x4*>(p));
  }
  __device__ static inline acc_t zero() { return acc_t{0, 0, 0, 0}; }
  __device__ static inline float to_f32(acc_t a, int j) { return float(a[j]); }
};

struct TrF32 {
  using op_t = float;
  using acc_t = f32x4;
  using elem_t = float;
  static constexpr int KF = 4;
  static constexpr int BPL = 4;
  __device__ static inline acc_t mfma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t load(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }
  __device__ static inline acc_t zero() { return acc_t{0.f, 0.f, 0.f, 0.f}; }
  __device__ static inline float to_f32(acc_t a, int j) { return a[j]; }
};

// Bytes of one packed fragment of a trait.
template <class Tr>
__host__ __device__ constexpr int frag_bytes() { return FRAG_LANES * Tr::BPL; }

// ---------------------------------------------------------------------------
// wavefront reductions
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, WAVE);
    v = w > v ? w : v;
  }
  return v;
}

}  // namespace moe
