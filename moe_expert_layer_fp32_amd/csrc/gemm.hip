// Grouped-row matrix-core product for gfx950.
//
// One kernel serves the router matmul (three exact bf16 planes of W_r
// accumulated, or fp32), the expert gate/up projection with its SwiGLU
// epilogue, and the down projection, for the resident routed experts (rows
// grouped by expert through the routing offsets) and for the shared expert
// (all tokens).
//
// Work split: a workgroup of 4 wavefronts owns one m-tile (up to 32 rows)
// of one group and 16 * 4/WK output columns: the wavefronts form WN = 4/WK
// column tiles of 16 times WK slices of the reduction (WK = 1, 2 or 4, chosen
// on the host so that the device has enough wavefronts streaming; the WK
// partial sums are added through LDS in a fixed order). Every wavefront
// streams its own weight fragments straight from HBM into registers - each
// fragment load is one contiguous 1 KiB read - and
// never shares them, so each weight byte of a tile is read exactly once; the
// loads run a fixed number of steps ahead of the matrix cores, which is what
// keeps enough bytes in flight for HBM. An expert's matrix-core work only
// covers the ceil(n_e/16) row blocks it has, so this is a weight stream in
// the sense of SwiftGMM's GEMV mode (page "华为技术披露集 VOL.12：昇腾×盘古",
// section SwiftGMM). The host picks this kernel from the shape alone: dense
// products of at most 64 rows and products whose reduction is not a whole
// number of 256-byte rows (which the tiled kernel of gemm_lds.hip cannot
// stage); every other product, routed or dense, goes to the tiled kernel,
// where the per-expert choice between its 64-row and 128-row tiles is made
// on the device. Which expert gets how many tiles is decided on the device
// from the routing offsets, so no count ever travels to the host. The
// activation rows (the "left matrix" SwiftGMM loads once and keeps resident)
// are the small operand, re-read from L2.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int STREAM_MB = 2;                       // row blocks per streaming tile
constexpr int MAX_RED_MB = STREAM_MB;
constexpr int STREAM_TILE = STREAM_MB * ROW_BLOCK; // 32 rows

// Locate m-tile `tile` among the groups. Returns false when the tile is past
// the last one (the grid is sized by an upper bound). Wave-uniform.
__device__ inline bool locate_tile(const GemmArgs& a, int tile, int& g, int& row0, int& nrows,
                                   int& out0) {
  if (a.offsets == nullptr) {
    g = 0;
    row0 = tile * a.dense_tile_rows;
    nrows = min(a.dense_tile_rows, a.dense_rows - row0);
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
      if (a.max_group_rows == 0 || n <= a.max_group_rows) c = ceil_div(n, STREAM_TILE);
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
  row0 = gbeg + mt * STREAM_TILE;
  nrows = min(STREAM_TILE, gend - row0);
  out0 = row0 - base;
  return true;
}


// One wavefront's 16 output columns of one m-tile with MB row blocks, over
// the reduction steps [kt0, kt1). Operands are software-pipelined D steps
// ahead in registers: the loads of step kt + D are issued right after step
// kt's matrix-core work, so each wavefront keeps D steps of weight fragments
// (1 KiB each) and activation fragments in flight. With WK > 1 the partial
// sums of the WK wavefronts sharing the columns meet in LDS and the first of
// them, in slice order, finishes the tile.
template <class Tr, int S, int EPI, int MB>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int g, int row0, int nrows, int out0, int ntile,
                                          bool live, int WK, int wk, int wn, int kt0, int kt1, int lane) {
  constexpr int FB = frag_bytes<Tr>();
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int D = S == 3 ? 4 : (MB == 1 ? 8 : 6);
  constexpr int BSTEP = 4 * Tr::BPL;   // bytes of a B row per reduction step
  using op_t = typename Tr::op_t;
  using acc_t = typename Tr::acc_t;
  const int KT = a.K / Tr::KF;
  const int nst = kt1 - kt0;

  acc_t acc[NACC][MB];
#pragma unroll
  for (int s = 0; s < NACC; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[s][mb] = Tr::zero();

  if (live && nst > 0) {
    // B row of each row block (rows past the end re-read the last valid row;
    // their results are never stored).
    const uint8_t* bp[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = min(mb * ROW_BLOCK + (lane & 15), nrows - 1);
      const int brow = a.sorted_slot ? a.sorted_slot[row0 + r] / a.k : out0 + r;
      bp[mb] = a.B + size_t(brow) * a.ldb + (lane >> 4) * Tr::BPL + size_t(kt0) * BSTEP;
    }
    const int NT = a.N / TILE_N;
    const size_t FBW = size_t(frag_block_width(ntile, NT)) * FB;   // stride of one plane step
    const uint8_t* ap = a.A + size_t(g) * a.a_group_stride + frag_offset(ntile, kt0, 0, NT, KT, S, FB) + lane * Tr::BPL;

    op_t wq[D][S];
    op_t bq[D][MB];
    // Every stage load is unconditional (a step past the end re-reads the
    // last step, from cache), so the number of loads in flight is the same on
    // every path and the waits before each stage only drain that stage.
    auto load_stage = [&](int p, int kt) {
#pragma unroll
      for (int s = 0; s < S; ++s) wq[p][s] = Tr::load(ap + size_t(kt * S + s) * FBW);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) bq[p][mb] = Tr::load(bp[mb] + size_t(kt) * BSTEP);
    };
    auto mma_stage = [&](int p) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int sa = (EPI == EPI_SWIGLU) ? s : 0;
          acc[sa][mb] = Tr::mfma(wq[p][s], bq[p][mb], acc[sa][mb]);
        }
    };
#pragma unroll
    for (int p = 0; p < D; ++p) load_stage(p, min(p, nst - 1));
    int kb = 0;
    for (; kb + D <= nst; kb += D) {
#pragma unroll
      for (int p = 0; p < D; ++p) {
        mma_stage(p);
        load_stage(p, min(kb + p + D, nst - 1));
        // keep each refill right after its stage (the scheduler would
        // otherwise bunch them at the end of the loop body)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int rem = nst - kb;
#pragma unroll
    for (int p = 0; p < D; ++p)
      if (p < rem) mma_stage(p);
  }

  if (WK > 1) {
    // One slot per wavefront: the partial sums of the later slices.
    __shared__ acc_t red[WG_WAVES][NACC * MAX_RED_MB][WAVE];
    const int WN = WG_WAVES / WK;
    if (wk > 0) {
#pragma unroll
      for (int s = 0; s < NACC; ++s)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) red[wn + wk * WN][s * MB + mb][lane] = acc[s][mb];
    }
    __syncthreads();
    if (wk > 0) return;
    for (int w = 1; w < WK; ++w)
#pragma unroll
      for (int s = 0; s < NACC; ++s)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[s][mb] += red[wn + w * WN][s * MB + mb][lane];
  }
  if (!live) return;

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
  for (int mb = 0; mb < MB; ++mb) {
    const int r = mb * ROW_BLOCK + (lane & 15);
    if (r >= nrows) continue;
    const int brow = a.sorted_slot ? a.sorted_slot[row0 + r] / a.k : out0 + r;
    const float bsc = a.b_scale ? a.b_scale[brow] : 1.0f;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (EPI == EPI_SWIGLU) {
        const float ga = Tr::to_f32(acc[0][mb], j) * bsc * cs0[j];
        const float up = Tr::to_f32(acc[1][mb], j) * bsc * cs1[j];
        v[j] = silu_f(ga) * up;
      } else {
        v[j] = Tr::to_f32(acc[0][mb], j) * bsc * cs0[j] + bias[j];
      }
    }
    uint8_t* op = a.out + size_t(out0 + r) * a.ldo;
    if (a.out_bf16) {
      u32x2 pk;
      pk[0] = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
      pk[1] = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
      *reinterpret_cast<u32x2*>(op + size_t(c0) * 2) = pk;
    } else {
      *reinterpret_cast<f32x4*>(op + size_t(c0) * 4) = f32x4{v[0], v[1], v[2], v[3]};
    }
  }
}

constexpr int NUM_XCD = 8;

template <class Tr, int S, int EPI>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(3))) void gemm_rows_kernel(
    GemmArgs a) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  // Blocks are dealt round-robin to the 8 XCDs (each with its own L2). Map
  // them so that each XCD runs a contiguous range of logical tiles, m-tile
  // fastest: tiles sharing a weight column block then share one L2.
  const int nbx = gridDim.x * gridDim.y;
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  const int q = nbx / NUM_XCD;
  const int logical = b < q * NUM_XCD ? (b % NUM_XCD) * q + b / NUM_XCD : b;
  const int tile = logical % a.tiles_y;
  const int nblock = logical / a.tiles_y;
  const int WK = a.ksplit;
  const int WN = WG_WAVES / WK;
  const int wn = wave % WN, wk = wave / WN;
  const int ntile = nblock * WN + wn;
  const bool live = ntile * TILE_N < a.N;

  int g, row0, nrows, out0;
  if (!locate_tile(a, tile, g, row0, nrows, out0)) return;   // whole workgroup
  g = __builtin_amdgcn_readfirstlane(g);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  nrows = __builtin_amdgcn_readfirstlane(nrows);
  out0 = __builtin_amdgcn_readfirstlane(out0);
  const int KT = a.K / Tr::KF;
  const int kt0 = wk * KT / WK, kt1 = (wk + 1) * KT / WK;
  if (nrows <= ROW_BLOCK)
    gemm_tile<Tr, S, EPI, 1>(a, g, row0, nrows, out0, ntile, live, WK, wk, wn, kt0, kt1, lane);
  else
    gemm_tile<Tr, S, EPI, 2>(a, g, row0, nrows, out0, ntile, live, WK, wk, wn, kt0, kt1, lane);
}

int gemm_tiles_bound(int max_rows, int n_groups) {
  return ceil_div(max_rows, STREAM_TILE) + n_groups;
}
int gemm_stream_ksplit(long col_tiles, int KT) {
  // Aim for about 12 streaming wavefronts per compute unit (3 per SIMD) and
  // keep at least 16 steps per slice.
  const long want = 256L * 12;
  if (col_tiles * 2 <= want && KT >= 64) return 4;
  if ((col_tiles <= want && KT >= 32) || (col_tiles <= 2 * want && KT >= 128)) return 2;
  return 1;
}

int gemm_tiles_dense(int rows, int n_cols, int* tile_rows) {
  (void)n_cols;
  *tile_rows = STREAM_TILE;
  return ceil_div(rows, STREAM_TILE);
}

template <class Tr, int S, int EPI>
static hipError_t launch_one(const GemmArgs& a, hipStream_t stream, KernelEvents ev) {
  if (a.tiles_y <= 0) return record_events(ev.start, ev.stop, stream);
  const int wn = WG_WAVES / a.ksplit;
  dim3 grid(ceil_div(a.N, wn * TILE_N), a.tiles_y);   // linearised and remapped in the kernel
  return launch_timed((gemm_rows_kernel<Tr, S, EPI>), grid, dim3(WG_THREADS), stream, ev.start, ev.stop, a);
}

hipError_t launch_gemm(const GemmArgs& a, GemmElem elem, int planes, GemmEpi epi,
                       hipStream_t stream, KernelEvents ev) {
  if (epi == EPI_SWIGLU) {
    switch (elem) {
      case ELEM_BF16: return launch_one<TrBF16, 2, EPI_SWIGLU>(a, stream, ev);
      case ELEM_I8: return launch_one<TrI8, 2, EPI_SWIGLU>(a, stream, ev);
      case ELEM_F32: return launch_one<TrF32, 2, EPI_SWIGLU>(a, stream, ev);
    }
  } else {
    switch (elem) {
      case ELEM_BF16:
        return planes == 3 ? launch_one<TrBF16, 3, EPI_SUM>(a, stream, ev)
                           : launch_one<TrBF16, 1, EPI_SUM>(a, stream, ev);
      case ELEM_I8: return launch_one<TrI8, 1, EPI_SUM>(a, stream, ev);
      case ELEM_F32: return launch_one<TrF32, 1, EPI_SUM>(a, stream, ev);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
