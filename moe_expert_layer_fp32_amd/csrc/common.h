// Device-side types and helpers shared by the gfx950 kernels of libmoe.so.
#pragma once

#include <hip/hip_ext.h>
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

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

// Launch with optional start / stop timing events stamped by the kernel's
// own dispatch (no event is recorded when both are null).
template <typename K, typename... Args>
inline hipError_t launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t start, hipEvent_t stop,
                               Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, start, stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}
// A launcher that launches nothing still records its events (in order).
inline hipError_t record_events(hipEvent_t start, hipEvent_t stop, hipStream_t s) {
  if (start) {
    const hipError_t e = hipEventRecord(start, s);
    if (e != hipSuccess) return e;
  }
  return stop ? hipEventRecord(stop, s) : hipSuccess;
}

// SiLU of the SwiGLU epilogues, v * sigmoid(v), from the hardware base-2
// exponent and reciprocal (each correct to about 1 ulp): for |v| up to ~20
// the result is within a few fp32 ulps of the exact value, and beyond that
// silu is v or 0 to fp32 precision. An IEEE division here costs the
// gate/up launch about 2 us per call (measured on the 64-expert decode
// layer), for accuracy far below the bf16 rounding of h.
__device__ inline float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

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

// Packed weight layout of one matrix (one expert): fragments of 16 columns
// (ntile nt) x KF reduction elements (step kt) of each plane s, grouped in
// column blocks of FRAG_BLOCK fragments; inside a block the order is
// [kt][s][fragment], so the 128 columns a workgroup of the tiled kernel owns
// are one contiguous stretch of memory, read front to back (per-workgroup
// contiguous streams keep the HBM rows open; one stream per fragment column
// does not). The last block of a matrix may be narrower.
constexpr int FRAG_BLOCK = 8;
__host__ __device__ inline int frag_block_width(int nt, int NT) {
  const int b0 = nt / FRAG_BLOCK * FRAG_BLOCK;
  return NT - b0 < FRAG_BLOCK ? NT - b0 : FRAG_BLOCK;
}
__host__ __device__ inline size_t frag_offset(int nt, int kt, int s, int NT, int KT, int S, int FB) {
  const int cb = nt / FRAG_BLOCK, j = nt % FRAG_BLOCK;
  const int w = frag_block_width(nt, NT);
  return (size_t(cb) * FRAG_BLOCK * KT * S + (size_t(kt) * S + s) * w + j) * size_t(FB);
}

// ---------------------------------------------------------------------------
// wavefront reductions
//
// Data-parallel-primitive moves inside each row of 16 lanes: after a quad
// swap of neighbours, a quad swap of pairs, the half-row mirror and the row
// mirror, every lane holds the combination of its whole row (the operation
// must be commutative: partner lanes then compute identical values). The
// four row results are read into scalar registers and combined in lane
// order, so every lane gets the same value and the order never varies.
// ---------------------------------------------------------------------------
constexpr int DPP_QUAD_1032 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline uint32_t lane_u32(uint32_t v, int l) { return uint32_t(__builtin_amdgcn_readlane(int(v), l)); }
__device__ inline float lane_f32(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

template <class Op>
__device__ inline float row_reduce_f32(float v, Op op) {
  v = op(v, dpp_f32<DPP_QUAD_1032>(v));
  v = op(v, dpp_f32<DPP_QUAD_2301>(v));
  v = op(v, dpp_f32<DPP_ROW_HALF_MIRROR>(v));
  v = op(v, dpp_f32<DPP_ROW_MIRROR>(v));
  return v;
}

// All 64 lanes of the wavefront must be active.
__device__ inline float wave_max(float v) {
  v = row_reduce_f32(v, [](float a, float b) { return fmaxf(a, b); });
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ inline float wave_sum(float v) {
  v = row_reduce_f32(v, [](float a, float b) { return a + b; });
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<DPP_QUAD_1032>(v));
  v = max(v, dpp_u32<DPP_QUAD_2301>(v));
  v = max(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
  v = max(v, dpp_u32<DPP_ROW_MIRROR>(v));
  return max(max(lane_u32(v, 0), lane_u32(v, 16)), max(lane_u32(v, 32), lane_u32(v, 48)));
}
__device__ inline uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<DPP_QUAD_1032>(v));
  v = min(v, dpp_u32<DPP_QUAD_2301>(v));
  v = min(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
  v = min(v, dpp_u32<DPP_ROW_MIRROR>(v));
  return min(min(lane_u32(v, 0), lane_u32(v, 16)), min(lane_u32(v, 32), lane_u32(v, 48)));
}

}  // namespace moe
