// Stable counting sort of the T*k routing slots by expert id (gfx950).
//
// This is the reordering the pages call InitialRouting: every (token, slot)
// pair is placed in expert order before tokens move to their experts (page
// on DeepSeek-V3/R1 on Ascend (Huxiu), section MOE 算子优化). The result
// must be bit-exact and deterministic, so no value depends on atomic order:
//  1. each of the 16 wavefronts of one workgroup takes a contiguous segment
//     of slots and histograms it into its own LDS row (integer LDS atomics:
//     the counts do not depend on their order);
//  2. per expert, the 16 segment counts are prefix-summed down the column
//     and the expert totals across the row (an exclusive scan over <= 256
//     experts), giving counts, offsets and each segment's first position;
//  3. each wavefront walks its segment again, 64 slots at a time in slot
//     order: lanes holding the same expert find each other with ballots
//     over the bits of the id, a lane's rank among equal lanes below it is a
//     popcount, and the segment's running position per expert advances by
//     the group size. Slots of one expert therefore keep ascending slot
//     order (stable), which fixes the permutation uniquely.
// Ids outside [0, E) are not counted; their slot_pos is -1.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PERM_WAVES = 16;
constexpr int PERM_THREADS = PERM_WAVES * WAVE;
constexpr int PERM_MAX_E = 256;

__global__ __launch_bounds__(PERM_THREADS) void permute_kernel(const int* __restrict__ idx, int n, int E,
                                                               int* __restrict__ counts,
                                                               int* __restrict__ offsets,
                                                               int* __restrict__ sorted_slot,
                                                               int* __restrict__ slot_pos) {
  __shared__ int hist[PERM_WAVES][PERM_MAX_E];
  __shared__ int expert_base[PERM_MAX_E + 1];
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;

  for (int i = threadIdx.x; i < PERM_WAVES * PERM_MAX_E; i += PERM_THREADS) (&hist[0][0])[i] = 0;
  __syncthreads();

  // Segment of this wave: [seg0, seg1), a multiple of 64 long.
  const int seg_len = ceil_div(ceil_div(n, PERM_WAVES), WAVE) * WAVE;
  const int seg0 = min(n, wave * seg_len);
  const int seg1 = min(n, seg0 + seg_len);

  for (int s = seg0 + lane; s < seg1; s += WAVE) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&hist[wave][e], 1);
  }
  __syncthreads();

  // Column prefix over waves (thread e), then exclusive scan over experts.
  int total = 0;
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    for (int w = 0; w < PERM_WAVES; ++w) {
      const int c = hist[w][e];
      hist[w][e] = total;     // exclusive prefix within the expert
      total += c;
    }
    counts[e] = total;
  }
  // Scan totals over experts with wave 0..3 (E <= 256): simple two-level scan.
  __shared__ int wave_tot[PERM_MAX_E / WAVE];
  if (threadIdx.x < PERM_MAX_E) {
    int incl = total;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
      const int v = __shfl_up(incl, d, WAVE);
      if (lane >= d) incl += v;
    }
    if (lane == WAVE - 1) wave_tot[wave] = incl;
    expert_base[threadIdx.x + 1] = incl;   // provisional (within 64-block)
  }
  __syncthreads();
  if (threadIdx.x < PERM_MAX_E) {
    int add = 0;
    for (int w = 0; w < wave; ++w) add += wave_tot[w];
    expert_base[threadIdx.x + 1] += add;
  }
  if (threadIdx.x == 0) expert_base[0] = 0;
  __syncthreads();
  if (threadIdx.x <= E) offsets[threadIdx.x] = expert_base[threadIdx.x];
  if (threadIdx.x < E) {
    const int e = threadIdx.x;
    for (int w = 0; w < PERM_WAVES; ++w) hist[w][e] += expert_base[e];   // segment start per expert
  }
  __syncthreads();

  // Stable placement, 64 slots at a time in slot order.
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
  for (int c = seg0; c < seg1; c += WAVE) {
    const int s = c + lane;
    const bool in = s < seg1;
    const int e = in ? idx[s] : -1;
    const bool ok = in && e >= 0 && e < E;
    uint64_t same = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bit = __ballot(ok && ((e >> b) & 1));
      same &= ((e >> b) & 1) ? bit : ~bit;
    }
    if (ok) {
      const int rank = __popcll(same & below);
      const int pos = hist[wave][e] + rank;
      sorted_slot[pos] = s;
      slot_pos[s] = pos;
    } else if (in) {
      slot_pos[s] = -1;
    }
    // The first lane of each id group advances that id's running position.
    // (All lanes read hist above before any lane writes it: one wavefront,
    // program order.)
    __builtin_amdgcn_wave_barrier();
    if (ok && (same & below) == 0) hist[wave][e] += __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_permute(const int* topk_idx, int n_slots, int E, int* counts, int* offsets,
                          int* sorted_slot, int* slot_pos, hipStream_t stream) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_THREADS), 0, stream, topk_idx, n_slots, E,
                     counts, offsets, sorted_slot, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
