// Device-side tile bookkeeping shared by the tiled matrix-core kernels:
// locating the m-tiles of row groups (experts) from the routing offsets.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// Locate m-tile `tile` (rows per tile `tm`) among the groups whose row count
// lies in [lo, hi]. Wave-uniform; false past the last tile.
__device__ inline bool locate_tile_lds(const GemmArgs& a, int tile, int tm, int lo, int hi, int& g, int& row0,
                                       int& nrows, int& out0) {
  if (a.offsets == nullptr) {
    g = 0;
    row0 = tile * tm;
    nrows = min(tm, a.dense_rows - row0);
    out0 = row0;
    return nrows > 0;
  }
  const int lane = threadIdx.x & (WAVE - 1);
  const int base = a.offsets[a.first];
  int cnt[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gg = lane * 4 + i;
    int c = 0;
    if (gg < a.n_groups) {
      const int n = a.offsets[a.first + gg + 1] - a.offsets[a.first + gg];
      if (n >= lo && n <= hi) c = ceil_div(n, tm);
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
  row0 = gbeg + mt * tm;
  nrows = min(tm, gend - row0);
  out0 = row0 - base;
  return true;
}

// Number of m-tiles (rows per tile tm) among the groups whose row count lies
// in [lo, hi]; dense: ceil(rows / tm). Wave-uniform.
__device__ inline int count_tiles_lds(const GemmArgs& a, int tm, int lo, int hi) {
  if (a.offsets == nullptr) return ceil_div(a.dense_rows, tm);
  const int lane = threadIdx.x & (WAVE - 1);
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gg = lane * 4 + i;
    if (gg < a.n_groups) {
      const int n = a.offsets[a.first + gg + 1] - a.offsets[a.first + gg];
      if (n >= lo && n <= hi) local += ceil_div(n, tm);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o, WAVE);
  return local;
}

}  // namespace moe
