// Gating and top-k selection for gfx950: one token per row of 16 lanes,
// four tokens per wavefront.
//
// The router product leaves the logits z = x W_r + b in a [T][E_pad] buffer
// (or split-K partial sums that are added here in split order, then the
// bias). Lane r of a row holds experts r, r+16, r+32, ... (PL of them).
// Scores are the softmax over the E logits or the logistic sigmoid of each
// (the pages give no gate formula; which one a workload uses is part of its
// descriptor). Every reduction stays inside the row, as data-parallel moves
// after which all 16 lanes hold the result, so rounds cost a few
// instructions and never leave the vector unit. A selection round is an
// argmax: the largest order-preserving bits of the logit, then the lowest
// expert id holding them (equal logits go to the lower id):
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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int ROW = 16;            // lanes per token
constexpr int GATE_TOKENS = WAVE / ROW;
constexpr int GROUP_SLOTS = 4;     // group-limited routing: n_group <= 64
constexpr int GATE_SPLIT_BATCH = 4;  // split-K partial sums loaded together

__device__ inline uint32_t order_bits(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);   // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Reductions over the 16 lanes of a row; every lane of the row gets the result.
__device__ inline uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp_u32<DPP_QUAD_1032>(v));
  v = max(v, dpp_u32<DPP_QUAD_2301>(v));
  v = max(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
  return max(v, dpp_u32<DPP_ROW_MIRROR>(v));
}
__device__ inline uint32_t row_min_u32(uint32_t v) {
  v = min(v, dpp_u32<DPP_QUAD_1032>(v));
  v = min(v, dpp_u32<DPP_QUAD_2301>(v));
  v = min(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
  return min(v, dpp_u32<DPP_ROW_MIRROR>(v));
}
__device__ inline float row_max_f32(float v) {
  return row_reduce_f32(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ inline float row_sum_f32(float v) {
  return row_reduce_f32(v, [](float x, float y) { return x + y; });
}

// Lowest id (slot i of lane r is id i*16 + r) among the candidates holding
// the largest order bits; -1 when there is no candidate (every finite logit
// has order bits above 0).
template <int N>
__device__ inline int row_argmax(const uint32_t (&ob)[N], const bool (&cand)[N], int r) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) m = max(m, cand[i] ? ob[i] : 0u);
  m = row_max_u32(m);
  uint32_t best = 0xFFFFFFFFu;
#pragma unroll
  for (int i = N - 1; i >= 0; --i)
    if (cand[i] && ob[i] == m) best = uint32_t(i * ROW + r);
  best = row_min_u32(best);
  return m == 0 ? -1 : int(best);
}

template <int N>
__device__ inline void drop(bool (&cand)[N], int id, int r) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i * ROW + r == id) cand[i] = false;
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

// FW wavefronts per workgroup. With split-K partial sums FW > 1: wavefront w
// adds splits w, w + FW, ... (in that order) for the workgroup's four tokens,
// the FW sums meet in LDS and are added in wavefront order; then only the
// first wavefront runs the gate (the others leave after the fold's barrier,
// so they do not share its SIMD with copies of the same work).
// Gate and selection for one token held by a row of 16 lanes (lane r holds
// experts i*16 + r). u: its logits, bias included. sc_row: the row's LDS
// scratch for its scores (written and read by this wavefront only). Lane
// r < k gets selection r: sel_out (expert id) and w_out (its weight). Every
// lane of the wavefront must be active.
template <int PL>
__device__ __forceinline__ void gate_row(const GateArgs& a, float (&u)[PL], const bool (&valid)[PL], int r,
                                         float* sc_row, int& sel_out, float& w_out) {
  float sc[PL];
  uint32_t ob[PL];
  int grp[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    if (!valid[i]) u[i] = -INFINITY;
    ob[i] = order_bits(u[i]);
  }

  if (a.gate == MOE_GATE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < PL; ++i) m = fmaxf(m, u[i]);
    m = row_max_f32(m);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      sc[i] = valid[i] ? expf(u[i] - m) : 0.f;
      sum += sc[i];
    }
    sum = row_sum_f32(sum);
#pragma unroll
    for (int i = 0; i < PL; ++i) sc[i] = sc[i] / sum;
  } else {
#pragma unroll
    for (int i = 0; i < PL; ++i) sc[i] = valid[i] ? 1.0f / (1.0f + expf(-u[i])) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < PL; ++i) sc_row[i * ROW + r] = sc[i];

  bool cand[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) cand[i] = valid[i];

  if (a.topk_group > 0 || a.per_group_k > 0) {
    const int gsize = a.E / a.n_group;
#pragma unroll
    for (int i = 0; i < PL; ++i) grp[i] = valid[i] ? (i * ROW + r) / gsize : -1;
  }
  if (a.topk_group > 0) {
    // group g's score = sum of its two largest scores; slot g/16 of lane g%16
    float gs[GROUP_SLOTS];
    bool gc[GROUP_SLOTS];
#pragma unroll
    for (int j = 0; j < GROUP_SLOTS; ++j) {
      gs[j] = -INFINITY;
      gc[j] = j * ROW + r < a.n_group;
    }
    auto finish_group = [&](int g, float t1, float t2) {
      merge_top2_dpp<DPP_QUAD_1032>(t1, t2);
      merge_top2_dpp<DPP_QUAD_2301>(t1, t2);
      merge_top2_dpp<DPP_ROW_HALF_MIRROR>(t1, t2);
      merge_top2_dpp<DPP_ROW_MIRROR>(t1, t2);
#pragma unroll
      for (int j = 0; j < GROUP_SLOTS; ++j)
        if (j * ROW + r == g) gs[j] = t1 + t2;
    };
    const int gsize = a.E / a.n_group;
    const int spg = gsize / ROW;   // slots per group when groups are whole slots
    if (gsize >= ROW && gsize % ROW == 0 && a.E % ROW == 0) {
      // Slot i of every lane holds experts i*16 .. i*16+15, all in group
      // i / spg: one pass over the slots, a group closed after its last slot
      // (a wave-uniform branch).
      float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        if (i * ROW < a.E) {
          merge_top2(t1, t2, sc[i], -INFINITY);
          if ((i + 1) % spg == 0) {
            finish_group(i / spg, t1, t2);
            t1 = t2 = -INFINITY;
          }
        }
      }
    } else {
      for (int g = 0; g < a.n_group; ++g) {
        float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
        for (int i = 0; i < PL; ++i)
          if (grp[i] == g) merge_top2(t1, t2, sc[i], -INFINITY);
        finish_group(g, t1, t2);
      }
    }
    uint32_t gob[GROUP_SLOTS];
#pragma unroll
    for (int j = 0; j < GROUP_SLOTS; ++j) gob[j] = order_bits(gs[j]);
    uint64_t kept = 0;
    for (int q = 0; q < a.topk_group; ++q) {
      const int gw = row_argmax(gob, gc, r);
      if (gw < 0) break;
      kept |= 1ull << gw;
      drop(gc, gw, r);
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) cand[i] = valid[i] && ((kept >> grp[i]) & 1ull);
  } else if (a.per_group_k > 0) {
    bool chosen[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) chosen[i] = false;
    for (int g = 0; g < a.n_group; ++g) {
      bool in_g[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) in_g[i] = grp[i] == g;
      for (int q = 0; q < a.per_group_k; ++q) {
        const int win = row_argmax(ob, in_g, r);
        if (win < 0) break;
        drop(in_g, win, r);
#pragma unroll
        for (int i = 0; i < PL; ++i)
          if (i * ROW + r == win) chosen[i] = true;
      }
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) cand[i] = chosen[i];
  }

  // k rounds over the candidates: descending logit, ties to the lower id;
  // lane r of the row keeps selection r.
  int sel_e = -1;
  for (int j = 0; j < a.k; ++j) {
    const int win = row_argmax(ob, cand, r);
    if (win < 0) break;
    drop(cand, win, r);
    if (r == j) sel_e = win;
  }
  __threadfence_block();   // the row's scores are in LDS (written by this wavefront)
  const bool mine = r < a.k && sel_e >= 0;
  const float s = mine ? sc_row[sel_e] : 0.f;
  const float total = row_sum_f32(s);
  sel_out = sel_e;
  w_out = (a.renorm ? s / total : s) * a.route_scale;
}


template <int PL, int FW>
__global__ __launch_bounds__(FW * WAVE) void gate_topk_kernel(GateArgs a) {
  __shared__ float sc_lds[GATE_TOKENS][PL * ROW];
  __shared__ float fold[FW][GATE_TOKENS][PL * ROW];
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int r = lane & (ROW - 1), row = lane / ROW;
  const int t_raw = blockIdx.x * GATE_TOKENS + row;
  const bool live = t_raw < a.T;            // dead rows work on a valid token and write nothing
  const int t = live ? t_raw : a.T - 1;

  float u[PL];
  bool valid[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = i * ROW + r;
    valid[i] = e < a.E;
    u[i] = 0.f;
  }
  if (!a.partial) {
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (valid[i]) u[i] = a.z[size_t(t) * a.ldz + i * ROW + r];
  } else {
    // This wavefront's splits, GATE_SPLIT_BATCH loads at a time (clamped
    // split index: every address is valid; absent splits add +0).
    float mine[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) mine[i] = 0.f;
    for (int sp0 = wave; sp0 < a.splits; sp0 += GATE_SPLIT_BATCH * FW) {
      float part[GATE_SPLIT_BATCH][PL];
#pragma unroll
      for (int q = 0; q < GATE_SPLIT_BATCH; ++q) {
        const float* P = a.partial + (size_t(min(sp0 + q * FW, a.splits - 1)) * a.T + t) * a.ldz + r;
#pragma unroll
        for (int i = 0; i < PL; ++i) part[q][i] = P[min(i * ROW, a.ldz - ROW)];
      }
#pragma unroll
      for (int q = 0; q < GATE_SPLIT_BATCH; ++q)
#pragma unroll
        for (int i = 0; i < PL; ++i) mine[i] += (sp0 + q * FW < a.splits && valid[i]) ? part[q][i] : 0.f;
    }
    if (FW == 1) {
#pragma unroll
      for (int i = 0; i < PL; ++i) u[i] = mine[i];
    } else {
#pragma unroll
      for (int i = 0; i < PL; ++i) fold[wave][row][i * ROW + r] = mine[i];
      __syncthreads();
#pragma unroll
      for (int w = 0; w < FW; ++w)
#pragma unroll
        for (int i = 0; i < PL; ++i) u[i] += fold[w][row][i * ROW + r];
    }
    if (a.bias) {
#pragma unroll
      for (int i = 0; i < PL; ++i)
        if (valid[i]) u[i] += a.bias[i * ROW + r];
    }
  }
  if (FW > 1 && wave != 0) return;   // no barrier follows
  int sel_e;
  float wv;
  gate_row<PL>(a, u, valid, r, &sc_lds[row][0], sel_e, wv);
  if (live && r < a.k) {
    a.topk_idx[size_t(t) * a.k + r] = sel_e;
    a.topk_w[size_t(t) * a.k + r] = wv;
  }
}

constexpr int GATE_FOLD_WAVES = 8;
template <int PL>
static hipError_t launch_gate_pl(const GateArgs& a, hipStream_t stream) {
  const dim3 grid(ceil_div(a.T, GATE_TOKENS));
  // Folding over several wavefronts pays for few tokens with many splits;
  // for many tokens the redundant gate work of the extra wavefronts costs more.
  if (a.partial && a.splits > 2 && a.T <= 2048)
    hipLaunchKernelGGL((gate_topk_kernel<PL, GATE_FOLD_WAVES>), grid, dim3(GATE_FOLD_WAVES * WAVE), 0, stream, a);
  else
    hipLaunchKernelGGL((gate_topk_kernel<PL, 1>), grid, dim3(WAVE), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gate(const GateArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  if (a.partial && a.splits < 1) return hipErrorInvalidValue;
  const int pl = ceil_div(a.E, ROW);
  if (pl <= 1) return launch_gate_pl<1>(a, stream);
  if (pl <= 2) return launch_gate_pl<2>(a, stream);
  if (pl <= 4) return launch_gate_pl<4>(a, stream);
  if (pl <= 6) return launch_gate_pl<6>(a, stream);
  if (pl <= 8) return launch_gate_pl<8>(a, stream);
  if (pl <= 12) return launch_gate_pl<12>(a, stream);
  return launch_gate_pl<16>(a, stream);
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
