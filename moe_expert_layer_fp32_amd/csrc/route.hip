// Gating and top-k selection for gfx950: one token per wavefront.
//
// The router product leaves the logits z = x W_r + b in a [T][E_pad] buffer
// (or split-K partial sums that are added here in split order, then the
// bias). Lane l of the wavefront holds experts 4l .. 4l+3 (E <= 256), so a
// token's logits arrive in one 16-byte load per lane and split. Scores are
// the softmax over the E logits or the logistic sigmoid of each (the pages
// give no gate formula; which one a workload uses is part of its
// descriptor). Every reduction is over the whole wavefront: data-parallel
// moves inside each row of 16 lanes, then the four row results read into
// scalar registers, so each round's winner is one value shared by the
// wavefront. A selection round is an argmax: the largest order-preserving
// bits of the logit, then the lowest expert id holding them (equal logits
// go to the lower id):
//  - plain top-k: k rounds over all experts;
//  - group-limited: group scores (sum of the two largest scores of each
//    contiguous group), topk_group rounds over the groups, then k rounds over
//    the experts of the kept groups;
//  - per-group quota (the grouped experts of Pangu Pro MoE, page
//    "华为技术披露集 VOL.12：昇腾×盘古", opening section): per_group_k rounds
//    inside each group, then k rounds to order the chosen by score.
// Softmax and sigmoid are monotone, so selecting on the logit is selecting
// on the score. Weights are the selected scores, renormalised over the k
// selections when asked, times route_scale.
//
// One token per wavefront (not four tokens on rows of 16 lanes) keeps each
// lane's share of a round to four experts and puts four times as many
// wavefronts to work on the same tokens; the rounds are chains of dependent
// steps, so the shorter chain is what counts.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GATE_SLOTS = 4;                    // experts per lane: lane l holds 4l .. 4l+3
constexpr int GATE_MAX_E = GATE_SLOTS * WAVE;    // 256
constexpr int GATE_MAX_GROUPS = WAVE;            // group g's score sits in lane g

__device__ inline uint32_t order_bits(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);   // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One selection round over keys (a candidate's order bits; 0 for no
// candidate): the largest key, then the lowest id holding it (slot j of
// lane l is id l*N + j, so that is the lowest lane holding it, then its
// lowest slot). The winner's key is set to 0 and its id returned, the same
// in every lane; -1 when no candidate is left (every finite logit has order
// bits above 0). All lanes active.
template <int N>
__device__ inline int wave_take_max(uint32_t (&key)[N], int lane) {
  uint32_t m = key[0];
#pragma unroll
  for (int j = 1; j < N; ++j) m = max(m, key[j]);
  m = wave_max_u32(m);
  if (m == 0) return -1;
  int slot = N;
#pragma unroll
  for (int j = N - 1; j >= 0; --j)
    if (key[j] == m) slot = j;
  const uint64_t holders = __builtin_amdgcn_ballot_w64(slot < N);
  const int wl = __builtin_ctzll(holders);
  const int ws = __builtin_amdgcn_readlane(slot, wl);
#pragma unroll
  for (int j = 0; j < N; ++j)
    if (lane == wl && j == ws) key[j] = 0;
  return wl * N + ws;
}

// Inside aligned blocks of L lanes (L a power of two, at most 16): the
// largest key and the lowest id holding it, in every lane of the block.
__device__ inline void pick_better(uint32_t& k, int& id, uint32_t pk, int pid) {
  if (pk > k || (pk == k && pid < id)) {
    k = pk;
    id = pid;
  }
}
template <int CTRL>
__device__ inline void pick_better_dpp(uint32_t& k, int& id) {
  const uint32_t pk = dpp_u32<CTRL>(k);
  const int pid = int(dpp_u32<CTRL>(uint32_t(id)));
  pick_better(k, id, pk, pid);
}
__device__ inline void block_argmax(uint32_t& k, int& id, int L) {
  if (L >= 2) pick_better_dpp<DPP_QUAD_1032>(k, id);
  if (L >= 4) pick_better_dpp<DPP_QUAD_2301>(k, id);
  if (L >= 8) pick_better_dpp<DPP_ROW_HALF_MIRROR>(k, id);
  if (L >= 16) pick_better_dpp<DPP_ROW_MIRROR>(k, id);
}

// Top two of (a1 >= a2) and (b1 >= b2).
__device__ inline void merge_top2(float& a1, float& a2, float b1, float b2) {
  if (b1 > a1) {
    a2 = fmaxf(a1, b2);
    a1 = b1;
  } else {
    a2 = fmaxf(a2, b1);
  }
}
template <int CTRL>
__device__ inline void merge_top2_dpp(float& t1, float& t2) {
  const float b1 = dpp_f32<CTRL>(t1), b2 = dpp_f32<CTRL>(t2);
  merge_top2(t1, t2, b1, b2);
}
// The two largest of every lane's (t1 >= t2), the same pair in every lane.
__device__ inline void wave_top2(float& t1, float& t2) {
  merge_top2_dpp<DPP_QUAD_1032>(t1, t2);
  merge_top2_dpp<DPP_QUAD_2301>(t1, t2);
  merge_top2_dpp<DPP_ROW_HALF_MIRROR>(t1, t2);
  merge_top2_dpp<DPP_ROW_MIRROR>(t1, t2);
  float a1 = lane_f32(t1, 0), a2 = lane_f32(t2, 0);
#pragma unroll
  for (int row = 1; row < WAVE / 16; ++row) merge_top2(a1, a2, lane_f32(t1, 16 * row), lane_f32(t2, 16 * row));
  t1 = a1;
  t2 = a2;
}

// N split-K partial sums (16 bytes per lane each) loaded together, then
// added to acc in split order.
template <int N>
__device__ inline void fold_splits(const float* p, size_t split_stride, int sp0, f32x4& acc) {
  f32x4 part[N];
#pragma unroll
  for (int q = 0; q < N; ++q) part[q] = *reinterpret_cast<const f32x4*>(p + size_t(sp0 + q) * split_stride);
  __builtin_amdgcn_sched_barrier(0);   // every load issued before the first add
#pragma unroll
  for (int q = 0; q < N; ++q) acc += part[q];
}

// GW wavefronts per workgroup, one token each; every wavefront works alone
// (its own LDS row, no barrier).
template <int GW>
__global__ __launch_bounds__(GW * WAVE) void gate_topk_kernel(GateArgs a) {
  __shared__ __align__(16) float sc_lds[GW][GATE_MAX_E];
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int t = blockIdx.x * GW + wave;
  if (t >= a.T) return;   // whole wavefront
  const int e0 = GATE_SLOTS * lane;
  const int col = min(e0, a.ldz - GATE_SLOTS);   // lanes past the row read its last 16 bytes
  float* sc_row = &sc_lds[wave][0];

  f32x4 z4;
  if (!a.partial) {
    z4 = *reinterpret_cast<const f32x4*>(a.z + size_t(t) * a.ldz + col);
  } else {
    // split order: splits 0, 1, 2, ... added one after another
    z4 = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* P = a.partial + size_t(t) * a.ldz + col;
    const size_t ss = size_t(a.T) * a.ldz;
    int sp = 0;
    for (; sp + 16 <= a.splits; sp += 16) fold_splits<16>(P, ss, sp, z4);
    if (sp + 8 <= a.splits) { fold_splits<8>(P, ss, sp, z4); sp += 8; }
    if (sp + 4 <= a.splits) { fold_splits<4>(P, ss, sp, z4); sp += 4; }
    if (sp + 2 <= a.splits) { fold_splits<2>(P, ss, sp, z4); sp += 2; }
    if (sp < a.splits) fold_splits<1>(P, ss, sp, z4);
    if (a.bias) {
      // all four loads issued before any is used (clamped index, no per-slot branch)
      float bv[GATE_SLOTS];
#pragma unroll
      for (int j = 0; j < GATE_SLOTS; ++j) bv[j] = a.bias[min(e0 + j, a.E - 1)];
#pragma unroll
      for (int j = 0; j < GATE_SLOTS; ++j) z4[j] += bv[j];
    }
  }

  float u[GATE_SLOTS], sc[GATE_SLOTS];
  bool valid[GATE_SLOTS];
  uint32_t ob[GATE_SLOTS];
#pragma unroll
  for (int j = 0; j < GATE_SLOTS; ++j) {
    valid[j] = e0 + j < a.E;
    u[j] = valid[j] ? z4[j] : -INFINITY;
    ob[j] = order_bits(u[j]);
  }

  if (a.gate == MOE_GATE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < GATE_SLOTS; ++j) m = fmaxf(m, u[j]);
    m = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < GATE_SLOTS; ++j) {
      sc[j] = valid[j] ? expf(u[j] - m) : 0.f;
      sum += sc[j];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int j = 0; j < GATE_SLOTS; ++j) sc[j] = sc[j] / sum;
  } else {
#pragma unroll
    for (int j = 0; j < GATE_SLOTS; ++j) sc[j] = valid[j] ? 1.0f / (1.0f + expf(-u[j])) : 0.f;
  }
  *reinterpret_cast<f32x4*>(sc_row + e0) = f32x4{sc[0], sc[1], sc[2], sc[3]};

  // key[j]: the slot's order bits while it is a candidate, else 0
  uint32_t key[GATE_SLOTS];
#pragma unroll
  for (int j = 0; j < GATE_SLOTS; ++j) key[j] = valid[j] ? ob[j] : 0u;

  if (a.topk_group > 0 || a.per_group_k > 0) {
    const int gsize = a.E / a.n_group;
    // Aligned groups: every group is L whole lanes (L a power of two, at
    // most 16), so a lane's four slots share one group and a group's
    // reductions stay inside its own lanes.
    const int L = gsize / GATE_SLOTS;
    const bool aligned = gsize % GATE_SLOTS == 0 && L <= 16 && (L & (L - 1)) == 0;
    int grp[GATE_SLOTS];   // the slot's group; 0 for slots past E (never candidates)
#pragma unroll
    for (int j = 0; j < GATE_SLOTS; ++j) grp[j] = valid[j] ? (e0 + j) / gsize : 0;

    if (a.topk_group > 0) {
      // group g's score: the sum of its two largest scores
      uint32_t gkey[1];
      int gdiv;   // a winning lane's group is lane / gdiv
      if (aligned) {
        float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < GATE_SLOTS; ++j)
          if (valid[j]) merge_top2(t1, t2, sc[j], -INFINITY);
        if (L >= 2) merge_top2_dpp<DPP_QUAD_1032>(t1, t2);
        if (L >= 4) merge_top2_dpp<DPP_QUAD_2301>(t1, t2);
        if (L >= 8) merge_top2_dpp<DPP_ROW_HALF_MIRROR>(t1, t2);
        if (L >= 16) merge_top2_dpp<DPP_ROW_MIRROR>(t1, t2);
        // the first lane of each group stands for it
        gkey[0] = (lane % L == 0 && lane / L < a.n_group) ? order_bits(t1 + t2) : 0u;
        gdiv = L;
      } else {
        float gv = -INFINITY;   // lane g: group g's score
        for (int g = 0; g < a.n_group; ++g) {
          float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
          for (int j = 0; j < GATE_SLOTS; ++j)
            if (valid[j] && grp[j] == g) merge_top2(t1, t2, sc[j], -INFINITY);
          wave_top2(t1, t2);
          if (lane == g) gv = t1 + t2;
        }
        gkey[0] = lane < a.n_group ? order_bits(gv) : 0u;
        gdiv = 1;
      }
      uint64_t kept = 0;
      for (int q = 0; q < a.topk_group; ++q) {
        const int gw = wave_take_max<1>(gkey, lane);
        if (gw < 0) break;
        kept |= 1ull << (gw / gdiv);
      }
#pragma unroll
      for (int j = 0; j < GATE_SLOTS; ++j)
        if (!((kept >> grp[j]) & 1ull)) key[j] = 0u;
    } else {
      // per_group_k largest of each group (ties to the lower id)
      bool chosen[GATE_SLOTS];
#pragma unroll
      for (int j = 0; j < GATE_SLOTS; ++j) chosen[j] = false;
      if (aligned) {
        // the groups' rounds run side by side, one round per quota step
        for (int q = 0; q < a.per_group_k; ++q) {
          uint32_t bk = 0u;
          int bid = e0;
#pragma unroll
          for (int j = GATE_SLOTS - 1; j >= 0; --j)
            if (!chosen[j] && key[j] >= bk) {
              bk = key[j];
              bid = e0 + j;
            }
          block_argmax(bk, bid, L);
#pragma unroll
          for (int j = 0; j < GATE_SLOTS; ++j)
            if (bk != 0u && e0 + j == bid) chosen[j] = true;
        }
      } else {
        for (int g = 0; g < a.n_group; ++g) {
          uint32_t in_g[GATE_SLOTS];
#pragma unroll
          for (int j = 0; j < GATE_SLOTS; ++j) in_g[j] = grp[j] == g ? key[j] : 0u;
          for (int q = 0; q < a.per_group_k; ++q) {
            const int win = wave_take_max<GATE_SLOTS>(in_g, lane);
            if (win < 0) break;
#pragma unroll
            for (int j = 0; j < GATE_SLOTS; ++j)
              if (e0 + j == win) chosen[j] = true;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < GATE_SLOTS; ++j)
        if (!chosen[j]) key[j] = 0u;
    }
  }

  // k rounds over the candidates: descending logit, ties to the lower id;
  // lane j keeps selection j.
  int sel_e = -1;
  for (int j = 0; j < a.k; ++j) {
    const int win = wave_take_max<GATE_SLOTS>(key, lane);
    if (win < 0) break;
    if (lane == j) sel_e = win;
  }
  __threadfence_block();   // the scores are in LDS (written by this wavefront)
  const bool mine = lane < a.k && sel_e >= 0;
  const float s = mine ? sc_row[sel_e] : 0.f;
  const float total = wave_sum(s);
  const float wv = (a.renorm ? s / total : s) * a.route_scale;
  if (lane < a.k) {
    a.topk_idx[size_t(t) * a.k + lane] = sel_e;
    a.topk_w[size_t(t) * a.k + lane] = wv;
  }
}

// Four tokens per workgroup from GATE_WIDE_FROM tokens (fewer, larger
// workgroups); below, one token per workgroup spreads the few tokens over
// more compute units.
constexpr int GATE_WIDE_FROM = 2048;
constexpr int GATE_WIDE = 4;

hipError_t launch_gate(const GateArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  if (a.partial && a.splits < 1) return hipErrorInvalidValue;
  if (a.E < 1 || a.E > GATE_MAX_E || a.ldz < a.E || a.ldz % GATE_SLOTS != 0) return hipErrorInvalidValue;
  if ((a.topk_group > 0 || a.per_group_k > 0) && (a.n_group < 1 || a.E % a.n_group != 0)) return hipErrorInvalidValue;
  if (a.topk_group > 0 && a.n_group > GATE_MAX_GROUPS) return hipErrorInvalidValue;
  if (a.T >= GATE_WIDE_FROM)
    hipLaunchKernelGGL((gate_topk_kernel<GATE_WIDE>), dim3(ceil_div(a.T, GATE_WIDE)), dim3(GATE_WIDE * WAVE), 0, stream, a);
  else
    hipLaunchKernelGGL((gate_topk_kernel<1>), dim3(a.T), dim3(WAVE), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router product for few tokens: one workgroup per 16 tokens x 16 experts.
// Its RW wavefronts split the reduction (ROUTER_U fragments per batch, the
// next batch's loads issued before the current batch's matrix-core ops) and
// add their partial tiles in wavefront order through LDS, so the result is
// fixed by the shape alone. Operand A is the packed router fragment (16
// experts), operand B the 16 token rows; with three bf16 planes the three
// products accumulate into one fp32 tile, which equals x times the fp32
// router up to fp32 accumulation.
// ---------------------------------------------------------------------------
constexpr int ROUTER_WAVES = 8;
constexpr int ROUTER_U = 4;

template <class Tr, int S>
__global__ __launch_bounds__(ROUTER_WAVES * WAVE) void router_small_kernel(RouterArgs a) {
  constexpr int FB = frag_bytes<Tr>();
  constexpr int XB = Tr::KF * int(sizeof(typename Tr::elem_t));   // x bytes per fragment step
  using op_t = typename Tr::op_t;
  __shared__ f32x4 red[ROUTER_WAVES][WAVE];

  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);   // wavefront-uniform
  const int t0 = blockIdx.x * ROW_BLOCK, nt = blockIdx.y;
  const int KT = a.K / Tr::KF;
  const int kt0 = wv * KT / ROUTER_WAVES, kt1 = (wv + 1) * KT / ROUTER_WAVES;
  const int NT = a.e_pad / TILE_N;
  const size_t FBW = size_t(frag_block_width(nt, NT)) * FB;   // stride of one plane step
  const uint8_t* wp = a.w + frag_offset(nt, 0, 0, NT, KT, S, FB) + size_t(lane) * Tr::BPL;
  const int tok = min(t0 + (lane & 15), a.T - 1);
  const uint8_t* xp = a.x + size_t(tok) * a.K * sizeof(typename Tr::elem_t) + (lane >> 4) * Tr::BPL;

  typename Tr::acc_t acc = Tr::zero();
  op_t xa[2][ROUTER_U], wb[2][ROUTER_U][S];
  // Buffers are chosen by compile-time constants only (no dynamic indexing
  // of register arrays).
  auto load = [&](auto buf, int kt) {
#pragma unroll
    for (int u = 0; u < ROUTER_U; ++u) {
      const int k = min(kt + u, kt1 - 1);   // clamped: every address is inside the operands
      xa[buf][u] = Tr::load(xp + size_t(k) * XB);
#pragma unroll
      for (int p = 0; p < S; ++p) wb[buf][u][p] = Tr::load(wp + (size_t(k) * S + p) * FBW);
    }
  };
  auto compute = [&](auto buf, int kt) {
#pragma unroll
    for (int u = 0; u < ROUTER_U; ++u) {
      if (kt + u < kt1) {
#pragma unroll
        for (int p = 0; p < S; ++p) acc = Tr::mfma(wb[buf][u][p], xa[buf][u], acc);
      }
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (kt0 < kt1) {
    load(B0{}, kt0);
    for (int kt = kt0; kt < kt1; kt += 2 * ROUTER_U) {
      if (kt + ROUTER_U < kt1) load(B1{}, kt + ROUTER_U);
      __builtin_amdgcn_sched_barrier(0);
      compute(B0{}, kt);
      if (kt + 2 * ROUTER_U < kt1) load(B0{}, kt + 2 * ROUTER_U);
      __builtin_amdgcn_sched_barrier(0);
      compute(B1{}, kt + ROUTER_U);
    }
  }
  red[wv][lane] = f32x4{Tr::to_f32(acc, 0), Tr::to_f32(acc, 1), Tr::to_f32(acc, 2), Tr::to_f32(acc, 3)};
  __syncthreads();
  // thread (j, l) of the first four wavefronts: expert (l/16)*4 + j, token l%16
  if (threadIdx.x < 4 * WAVE) {
    const int l = threadIdx.x & (WAVE - 1), j = threadIdx.x / WAVE;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < ROUTER_WAVES; ++w) v += red[w][l][j];
    const int e = nt * TILE_N + (l >> 4) * 4 + j;
    const int t = t0 + (l & 15);
    if (a.bias && e < a.E) v += a.bias[e];
    if (t < a.T) a.z[size_t(t) * a.e_pad + e] = v;
  }
}

hipError_t launch_router_small(const RouterArgs& a, bool f32, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  const dim3 grid(ceil_div(a.T, ROW_BLOCK), a.e_pad / TILE_N), block(ROUTER_WAVES * WAVE);
  if (f32)
    hipLaunchKernelGGL((router_small_kernel<TrF32, 1>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((router_small_kernel<TrBF16, 3>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
