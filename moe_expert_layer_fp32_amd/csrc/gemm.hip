// Grouped-row matrix-core product for gfx950.
//
// One kernel serves the router matmul (three exact bf16 planes of W_r
// accumulated, or fp32), the expert gate/up projection with its SwiGLU
// epilogue, and the down projection, for the resident routed experts (rows
// grouped by expert through the routing offsets) and for the shared expert
// (all tokens).
//
// Work split: a workgroup owns 64 output columns (4 wavefronts x one
// 16-column tile each) of one m-tile (up to 128 rows) of one group. Every
// wavefront streams its own weight fragments straight from HBM into
// registers - the packed layout makes each fragment load one contiguous
// 1 KiB read - and never shares them, so each weight byte of a tile is read
// exactly once. An expert with few tokens therefore runs as a weight stream
// whose matrix-core work only covers the ceil(n_e/16) row blocks it has (the
// GEMV end of the per-expert GEMV/GEMM choice of SwiftGMM, page
// "华为技术披露集 VOL.12：昇腾×盘古", section SwiftGMM); an expert with many
// tokens gets several m-tiles of 8 full row blocks, each reusing a weight
// fragment 8 times in registers (the GEMM end). Which expert gets how many
// tiles is decided on the device from the routing offsets, so no count ever
// travels to the host. The activation rows (the "left matrix" that SwiftGMM
// loads once and keeps resident) are the small operand: they are re-read
// from L2 by the four wavefronts of a workgroup.
#include "common.h"
#include "kernels.h"

namespace moe {

// Locate m-tile `tile` among the groups. Returns false when the tile is past
// the last one (the grid is sized by an upper bound). Wave-uniform.
__device__ inline bool locate_tile(const GemmArgs& a, int tile, int& g, int& row0, int& nrows,
                                   int& out0) {
  if (a.offsets == nullptr) {
    g = 0;
    row0 = tile * TILE_M;
    nrows = min(TILE_M, a.dense_rows - row0);
    out0 = row0;
    return nrows > 0;
  }
  const int lane = threadIdx.x & (WAVE - 1);
  const int base = a.offsets[a.first];
  // Each lane owns 4 consecutive groups (n_groups <= 256).
  int cnt[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gg = lane * 4 + i;
    int c = 0;
    if (gg < a.n_groups) {
      const int n = a.offsets[a.first + gg + 1] - a.offsets[a.first + gg];
      c = ceil_div(n, TILE_M);
    }
    cnt[i] = c;
    local += c;
  }
  int incl = local;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int v = __shfl_up(incl, d, WAVE);
    if (lane >= d) incl += v;
  }
  const int excl = incl - local;
  const uint64_t hit = __ballot(tile >= excl && tile < incl);
  if (hit == 0) return false;
  const int src = __builtin_ctzll(hit);
  // Resolve the group inside lane `src`.
  int my_g = -1, my_mt = 0;
  if (lane == src) {
    int t = tile - excl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (my_g < 0) {
        if (t < cnt[i]) {
          my_g = lane * 4 + i;
          my_mt = t;
        } else {
          t -= cnt[i];
        }
      }
    }
  }
  g = __shfl(my_g, src, WAVE);
  const int mt = __shfl(my_mt, src, WAVE);
  const int gbeg = a.offsets[a.first + g];
  const int gend = a.offsets[a.first + g + 1];
  row0 = gbeg + mt * TILE_M;
  nrows = min(TILE_M, gend - row0);
  out0 = row0 - base;
  return true;
}

__device__ inline float silu(float v) { return v / (1.0f + expf(-v)); }

template <class Tr, int S, int EPI>
__global__ __launch_bounds__(WG_THREADS) void gemm_rows_kernel(GemmArgs a) {
  constexpr int FB = frag_bytes<Tr>();
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int ntile = blockIdx.x * WG_WAVES + wave;
  if (ntile * TILE_N >= a.N) return;   // wave-uniform; the kernel has no barriers

  int g, row0, nrows, out0;
  if (!locate_tile(a, blockIdx.y, g, row0, nrows, out0)) return;
  const int nblk = ceil_div(nrows, ROW_BLOCK);
  const int KT = a.K / Tr::KF;

  // B row of each of this lane's row blocks (rows past the end re-read the
  // last valid row; their results are never stored).
  const uint8_t* bp[MAX_ROW_BLOCKS];
  float bsc[MAX_ROW_BLOCKS];
#pragma unroll
  for (int mb = 0; mb < MAX_ROW_BLOCKS; ++mb) {
    const int r = min(mb * ROW_BLOCK + (lane & 15), nrows - 1);
    const int brow = a.sorted_slot ? a.sorted_slot[row0 + r] / a.k : out0 + r;
    bp[mb] = a.B + size_t(brow) * a.ldb + (lane >> 4) * Tr::BPL;
    bsc[mb] = a.b_scale ? a.b_scale[brow] : 1.0f;
  }
  const uint8_t* ap = a.A + size_t(g) * a.a_group_stride +
                      size_t(ntile) * KT * S * FB + lane * Tr::BPL;

  typename Tr::acc_t acc[NACC][MAX_ROW_BLOCKS];
#pragma unroll
  for (int s = 0; s < NACC; ++s)
#pragma unroll
    for (int mb = 0; mb < MAX_ROW_BLOCKS; ++mb) acc[s][mb] = Tr::zero();

  constexpr int BSTEP = 4 * Tr::BPL;   // bytes of B row per reduction step
#pragma unroll 4
  for (int kt = 0; kt < KT; ++kt) {
    typename Tr::op_t w[S];
#pragma unroll
    for (int s = 0; s < S; ++s) w[s] = Tr::load(ap + size_t(kt * S + s) * FB);
#pragma unroll
    for (int mb = 0; mb < MAX_ROW_BLOCKS; ++mb) {
      if (mb < nblk) {
        const typename Tr::op_t b = Tr::load(bp[mb] + size_t(kt) * BSTEP);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int sa = (EPI == EPI_SWIGLU) ? s : 0;
          acc[sa][mb] = Tr::mfma(w[s], b, acc[sa][mb]);
        }
      }
    }
  }

  // Epilogue: lane holds columns c0..c0+3 of row (lane % 16) of each block.
  const int c0 = ntile * TILE_N + (lane >> 4) * 4;
  float cs0[4] = {1.f, 1.f, 1.f, 1.f}, cs1[4] = {1.f, 1.f, 1.f, 1.f}, bias[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (a.a_scale0) cs0[j] = a.a_scale0[size_t(g) * a.a_scale_stride + c0 + j];
    if (EPI == EPI_SWIGLU && a.a_scale1) cs1[j] = a.a_scale1[size_t(g) * a.a_scale_stride + c0 + j];
    if (EPI == EPI_SUM && a.bias && c0 + j < a.n_valid) bias[j] = a.bias[c0 + j];
  }
#pragma unroll
  for (int mb = 0; mb < MAX_ROW_BLOCKS; ++mb) {
    if (mb >= nblk) break;
    const int r = mb * ROW_BLOCK + (lane & 15);
    if (r >= nrows) continue;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (EPI == EPI_SWIGLU) {
        const float ga = Tr::to_f32(acc[0][mb], j) * bsc[mb] * cs0[j];
        const float up = Tr::to_f32(acc[1][mb], j) * bsc[mb] * cs1[j];
        v[j] = silu(ga) * up;
      } else {
        v[j] = Tr::to_f32(acc[0][mb], j) * bsc[mb] * cs0[j] + bias[j];
      }
    }
    uint8_t* op = a.out + size_t(out0 + r) * a.ldo;
    if (a.out_bf16) {
      u32x2 p;
      p[0] = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
      p[1] = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
      *reinterpret_cast<u32x2*>(op + size_t(c0) * 2) = p;
    } else {
      *reinterpret_cast<f32x4*>(op + size_t(c0) * 4) = f32x4{v[0], v[1], v[2], v[3]};
    }
  }
}

int gemm_tiles_bound(int max_rows, int n_groups) {
  return ceil_div(max_rows, TILE_M) + n_groups;
}
int gemm_tiles_dense(int rows) { return ceil_div(rows, TILE_M); }

template <class Tr, int S, int EPI>
static hipError_t launch_one(const GemmArgs& a, hipStream_t stream) {
  if (a.tiles_y <= 0) return hipSuccess;
  dim3 grid(ceil_div(a.N, WG_N), a.tiles_y);
  hipLaunchKernelGGL((gemm_rows_kernel<Tr, S, EPI>), grid, dim3(WG_THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, GemmElem elem, int planes, GemmEpi epi,
                       hipStream_t stream) {
  if (epi == EPI_SWIGLU) {
    switch (elem) {
      case ELEM_BF16: return launch_one<TrBF16, 2, EPI_SWIGLU>(a, stream);
      case ELEM_I8: return launch_one<TrI8, 2, EPI_SWIGLU>(a, stream);
      case ELEM_F32: return launch_one<TrF32, 2, EPI_SWIGLU>(a, stream);
    }
  } else {
    switch (elem) {
      case ELEM_BF16:
        return planes == 3 ? launch_one<TrBF16, 3, EPI_SUM>(a, stream)
                           : launch_one<TrBF16, 1, EPI_SUM>(a, stream);
      case ELEM_I8: return launch_one<TrI8, 1, EPI_SUM>(a, stream);
      case ELEM_F32: return launch_one<TrF32, 1, EPI_SUM>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
