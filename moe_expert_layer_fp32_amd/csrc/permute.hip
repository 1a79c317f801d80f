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
//
// Many slots (more than 8192; prefill: T*k = 65536) spread the same steps
// over several workgroups, each owning a contiguous chunk of 2048 slots: one pass histograms
// every chunk into the workspace; a second pass gives each chunk its
// starting position per expert (the expert's offset plus the counts of the
// chunks before it, summed in chunk order) and places the chunk's slots as
// above. The result is the same permutation, bit for bit.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PERM_WAVES = 16;
constexpr int PERM_THREADS = PERM_WAVES * WAVE;
constexpr int PERM_MAX_E = 256;
constexpr int PERM_SEG_IDS = PERMUTE_ONE_WG / PERM_THREADS;   // ids per lane of a segment
constexpr int PERM_BATCH = 16;   // chunk histograms read together
static_assert(PERMUTE_CHUNK <= PERMUTE_ONE_WG, "a chunk must fit one workgroup's registers");

// Histogram of the chunk [chunk * blockIdx.x, ...) of each workgroup into
// chunk_hist[blockIdx.x][E] (integer LDS atomics: order-independent).
__global__ __launch_bounds__(PERM_THREADS) void permute_hist_kernel(const int* __restrict__ idx, int n, int E,
                                                                    int chunk, int* __restrict__ chunk_hist) {
  __shared__ int hist[PERM_MAX_E];
  for (int i = threadIdx.x; i < PERM_MAX_E; i += PERM_THREADS) hist[i] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * chunk, c1 = min(n, c0 + chunk);
  for (int s = c0 + threadIdx.x; s < c1; s += PERM_THREADS) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) chunk_hist[size_t(blockIdx.x) * E + e] = hist[e];
}

// Placement of the chunk of workgroup blockIdx.x (the whole range when
// chunk_hist is null: one workgroup). Workgroup 0 writes counts and offsets.
__global__ __launch_bounds__(PERM_THREADS) void permute_kernel(const int* __restrict__ idx, int n, int E,
                                                               int chunk, const int* __restrict__ chunk_hist,
                                                               int* __restrict__ counts,
                                                               int* __restrict__ offsets,
                                                               int* __restrict__ sorted_slot,
                                                               int* __restrict__ slot_pos) {
  __shared__ int hist[PERM_WAVES][PERM_MAX_E];
  __shared__ int expert_base[PERM_MAX_E + 1];
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int c0 = chunk_hist ? blockIdx.x * chunk : 0;
  const int c1 = chunk_hist ? min(n, c0 + chunk) : n;

  for (int i = threadIdx.x; i < PERM_WAVES * PERM_MAX_E; i += PERM_THREADS) (&hist[0][0])[i] = 0;
  __syncthreads();

  // Segment of this wave inside the chunk: [seg0, seg1), a multiple of 64 long.
  const int seg_len = ceil_div(ceil_div(c1 - c0, PERM_WAVES), WAVE) * WAVE;
  const int seg0 = min(c1, c0 + wave * seg_len);
  const int seg1 = min(c1, seg0 + seg_len);

  // The segment's ids stay in registers for the placement below (segments
  // are at most PERM_SEG_IDS * 64 slots: one workgroup takes at most
  // PERMUTE_ONE_WG slots, a chunk PERMUTE_CHUNK).
  int ids[PERM_SEG_IDS];
#pragma unroll
  for (int q = 0; q < PERM_SEG_IDS; ++q) {
    const int s = seg0 + q * WAVE + lane;
    ids[q] = s < seg1 ? idx[s] : -1;
  }
#pragma unroll
  for (int q = 0; q < PERM_SEG_IDS; ++q) {
    const int e = ids[q];
    if (e >= 0 && e < E) atomicAdd(&hist[wave][e], 1);
  }
  __syncthreads();

  // Column prefix over waves (thread e), then exclusive scan over experts of
  // the expert totals (over all chunks); `before` = slots of expert e in the
  // chunks ahead of this one.
  int total = 0, before = 0;
  if (int(threadIdx.x) < E) {
    const int e = threadIdx.x;
    for (int w = 0; w < PERM_WAVES; ++w) {
      const int c = hist[w][e];
      hist[w][e] = total;     // exclusive prefix within the expert (this chunk)
      total += c;
    }
    if (chunk_hist) {
      // PERM_BATCH chunk counts loaded at once, then added in chunk order
      // (one memory round trip per batch instead of one per chunk)
      const int nchunks = ceil_div(n, chunk);
      total = 0;
      for (int b0 = 0; b0 < nchunks; b0 += PERM_BATCH) {
        int c[PERM_BATCH];
#pragma unroll
        for (int q = 0; q < PERM_BATCH; ++q)
          c[q] = b0 + q < nchunks ? chunk_hist[size_t(b0 + q) * E + e] : 0;
#pragma unroll
        for (int q = 0; q < PERM_BATCH; ++q) {
          if (b0 + q < int(blockIdx.x)) before += c[q];
          total += c[q];
        }
      }
    }
    if (blockIdx.x == 0) counts[e] = total;
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
  if (blockIdx.x == 0 && int(threadIdx.x) <= E) offsets[threadIdx.x] = expert_base[threadIdx.x];
  if (int(threadIdx.x) < E) {
    const int e = threadIdx.x;
    for (int w = 0; w < PERM_WAVES; ++w) hist[w][e] += expert_base[e] + before;   // segment start per expert
  }
  __syncthreads();

  // Stable placement, 64 slots at a time in slot order.
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
#pragma unroll
  for (int q = 0; q < PERM_SEG_IDS; ++q) {
    const int c = seg0 + q * WAVE;
    if (c >= seg1) break;   // wavefront-uniform
    const int s = c + lane;
    const bool in = s < seg1;
    const int e = in ? ids[q] : -1;
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

int permute_chunks(int n_slots) { return n_slots > PERMUTE_ONE_WG ? ceil_div(n_slots, PERMUTE_CHUNK) : 1; }

hipError_t launch_permute(const int* topk_idx, int n_slots, int E, int* counts, int* offsets,
                          int* sorted_slot, int* slot_pos, int* chunk_hist, hipStream_t stream) {
  const int nchunks = permute_chunks(n_slots);
  if (nchunks == 1) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_THREADS), 0, stream, topk_idx, n_slots, E, n_slots,
                       static_cast<const int*>(nullptr), counts, offsets, sorted_slot, slot_pos);
    return hipGetLastError();
  }
  if (!chunk_hist) return hipErrorInvalidValue;
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nchunks), dim3(PERM_THREADS), 0, stream, topk_idx, n_slots, E,
                     PERMUTE_CHUNK, chunk_hist);
  hipLaunchKernelGGL(permute_kernel, dim3(nchunks), dim3(PERM_THREADS), 0, stream, topk_idx, n_slots, E,
                     PERMUTE_CHUNK, static_cast<const int*>(chunk_hist), counts, offsets, sorted_slot, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
