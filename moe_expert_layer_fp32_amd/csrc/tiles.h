// Device-side tile bookkeeping of the tiled matrix-core kernel: locating the
// m-tiles of row groups (experts) from the routing offsets.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int TILE_MAX_GROUPS = 256;   // 4 groups per lane of one wavefront

// The routing offsets of the groups [first, first + n_groups] copied into
// LDS once per workgroup (one global round trip); every later tile lookup
// reads only LDS. All threads of the workgroup call it; null offsets
// (a dense product) copy nothing.
__device__ inline void stage_offsets(const GemmArgs& a, int* offs) {
  if (a.offsets == nullptr) return;
  for (int i = threadIdx.x; i <= a.n_groups; i += blockDim.x) offs[i] = a.offsets[a.first + i];
  __syncthreads();
}

// m-tiles (rows per tile tm) of the four groups lane*4 .. lane*4+3 whose row
// count lies in [lo, hi].
__device__ inline int lane_tiles(const GemmArgs& a, const int* offs, int tm, int lo, int hi, int (&cnt)[4]) {
  const int lane = threadIdx.x & (WAVE - 1);
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gg = lane * 4 + i;
    int c = 0;
    if (gg < a.n_groups) {
      const int n = offs[gg + 1] - offs[gg];
      if (n >= lo && n <= hi) c = ceil_div(n, tm);
    }
    cnt[i] = c;
    local += c;
  }
  return local;
}

// Locate m-tile `tile` among those groups. Wave-uniform; false past the
// last tile. offs: the staged offsets.
__device__ inline bool locate_tile_lds(const GemmArgs& a, const int* offs, int tile, int tm, int lo, int hi, int& g,
                                       int& row0, int& nrows, int& out0) {
  if (a.offsets == nullptr) {
    g = 0;
    row0 = tile * tm;
    nrows = min(tm, a.dense_rows - row0);
    out0 = row0;
    return nrows > 0;
  }
  const int lane = threadIdx.x & (WAVE - 1);
  int cnt[4];
  const int local = lane_tiles(a, offs, tm, lo, hi, cnt);
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
  row0 = offs[g] + mt * tm;
  nrows = min(tm, offs[g + 1] - row0);
  out0 = row0 - offs[0];
  return true;
}

// Number of m-tiles among those groups; dense: ceil(rows / tm). Wave-uniform.
__device__ inline int count_tiles_lds(const GemmArgs& a, const int* offs, int tm, int lo, int hi) {
  if (a.offsets == nullptr) return ceil_div(a.dense_rows, tm);
  int cnt[4];
  int local = lane_tiles(a, offs, tm, lo, hi, cnt);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o, WAVE);
  return local;
}

}  // namespace moe
