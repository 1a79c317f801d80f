// Gating and top-k selection for gfx950: one wavefront per token.
//
// The router matmul (gemm.hip) leaves the logits z = x W_r + b in a
// [T][E_pad] buffer. Here each wavefront takes one token: lane l holds
// experts l, l+64, l+128, l+192. Scores are the softmax over the E logits or
// the logistic sigmoid of each (the pages give no gate formula; which one a
// workload uses is part of its descriptor). Selection runs as rounds of a
// wavefront-wide argmax over a 64-bit key (order-preserving bits of the
// logit, then the complemented expert id, so the larger logit wins and equal
// logits go to the lower id) exchanged with cross-lane shuffles:
//  - plain top-k: k rounds over all experts;
//  - group-limited: group scores (sum of the two largest scores of each
//    contiguous group, reduced with shuffles), topk_group rounds over the
//    groups, then k rounds over the experts of the kept groups;
//  - per-group quota (the grouped experts of Pangu Pro MoE, page
//    "华为技术披露集 VOL.12：昇腾×盘古", opening section): per_group_k rounds
//    inside each group, then k rounds to order the chosen by score.
// Softmax and sigmoid are monotone, so selecting on the logit is selecting
// on the score. Weights are the selected scores, renormalised over the k
// selections when asked, times route_scale.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int GATE_PER_LANE = 4;   // E <= 256

__device__ inline uint32_t order_bits(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);   // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline uint64_t make_key(float v, int id) {
  return (uint64_t(order_bits(v)) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(id));
}
__device__ inline int key_id(uint64_t key) { return int(0xFFFFFFFFu - uint32_t(key)); }

// Top two of (a1 >= a2) and (b1 >= b2).
__device__ inline void merge_top2(float& a1, float& a2, float b1, float b2) {
  if (b1 > a1) {
    a2 = fmaxf(a1, b2);
    a1 = b1;
  } else {
    a2 = fmaxf(a2, b1);
  }
}

__global__ __launch_bounds__(256) void gate_topk_kernel(GateArgs a) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int t = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  if (t >= a.T) return;
  const float* zt = a.z + size_t(t) * a.ldz;

  float u[GATE_PER_LANE], sc[GATE_PER_LANE];
  bool valid[GATE_PER_LANE];
#pragma unroll
  for (int i = 0; i < GATE_PER_LANE; ++i) {
    const int e = lane + i * WAVE;
    valid[i] = e < a.E;
    u[i] = valid[i] ? zt[e] : -INFINITY;
  }
  if (a.gate == MOE_GATE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < GATE_PER_LANE; ++i) m = fmaxf(m, u[i]);
    m = wave_max(m);
    float ex[GATE_PER_LANE], sum = 0.f;
#pragma unroll
    for (int i = 0; i < GATE_PER_LANE; ++i) {
      ex[i] = valid[i] ? expf(u[i] - m) : 0.f;
      sum += ex[i];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int i = 0; i < GATE_PER_LANE; ++i) sc[i] = ex[i] / sum;
  } else {
#pragma unroll
    for (int i = 0; i < GATE_PER_LANE; ++i) sc[i] = valid[i] ? 1.0f / (1.0f + expf(-u[i])) : 0.f;
  }

  // Candidate mask per owned expert.
  bool cand[GATE_PER_LANE];
#pragma unroll
  for (int i = 0; i < GATE_PER_LANE; ++i) cand[i] = valid[i];
  const int gsize = a.E / a.n_group;

  if (a.topk_group > 0) {
    // group score = sum of the two largest scores; lane g keeps group g's score.
    float my_gs = -INFINITY;
    for (int g = 0; g < a.n_group; ++g) {
      float t1 = -INFINITY, t2 = -INFINITY;
#pragma unroll
      for (int i = 0; i < GATE_PER_LANE; ++i) {
        const int e = lane + i * WAVE;
        if (valid[i] && e / gsize == g) merge_top2(t1, t2, sc[i], -INFINITY);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float b1 = __shfl_xor(t1, o, WAVE);
        const float b2 = __shfl_xor(t2, o, WAVE);
        merge_top2(t1, t2, b1, b2);
      }
      if (lane == g) my_gs = t1 + t2;
    }
    uint64_t kept = 0;
    for (int r = 0; r < a.topk_group; ++r) {
      const bool live = lane < a.n_group && !((kept >> lane) & 1ull);
      const uint64_t best = wave_max_u64(live ? make_key(my_gs, lane) : 0ull);
      kept |= 1ull << key_id(best);
    }
#pragma unroll
    for (int i = 0; i < GATE_PER_LANE; ++i) {
      const int e = lane + i * WAVE;
      cand[i] = valid[i] && ((kept >> (e / gsize)) & 1ull);
    }
  } else if (a.per_group_k > 0) {
    bool chosen[GATE_PER_LANE] = {false, false, false, false};
    for (int g = 0; g < a.n_group; ++g) {
      for (int r = 0; r < a.per_group_k; ++r) {
        uint64_t mine = 0;
#pragma unroll
        for (int i = 0; i < GATE_PER_LANE; ++i) {
          const int e = lane + i * WAVE;
          if (valid[i] && !chosen[i] && e / gsize == g) {
            const uint64_t kk = make_key(u[i], e);
            mine = kk > mine ? kk : mine;
          }
        }
        const int win = key_id(wave_max_u64(mine));
#pragma unroll
        for (int i = 0; i < GATE_PER_LANE; ++i)
          if (lane + i * WAVE == win) chosen[i] = true;
      }
    }
#pragma unroll
    for (int i = 0; i < GATE_PER_LANE; ++i) cand[i] = chosen[i];
  }

  // k rounds over the candidates, descending logit, ties to the lower id.
  int sel_e = 0;
  float sel_s = 0.f, total = 0.f;
  for (int j = 0; j < a.k; ++j) {
    uint64_t mine = 0;
#pragma unroll
    for (int i = 0; i < GATE_PER_LANE; ++i) {
      if (cand[i]) {
        const uint64_t kk = make_key(u[i], lane + i * WAVE);
        mine = kk > mine ? kk : mine;
      }
    }
    const int win = key_id(wave_max_u64(mine));
    float s_own = 0.f;
#pragma unroll
    for (int i = 0; i < GATE_PER_LANE; ++i) {
      if (lane + i * WAVE == win) {
        cand[i] = false;
        s_own = sc[i];
      }
    }
    const float s_win = __shfl(s_own, win & (WAVE - 1), WAVE);
    total += s_win;
    if (lane == j) {
      sel_e = win;
      sel_s = s_win;
    }
  }
  if (lane < a.k) {
    float wv = a.renorm ? sel_s / total : sel_s;
    wv *= a.route_scale;
    a.topk_idx[size_t(t) * a.k + lane] = sel_e;
    a.topk_w[size_t(t) * a.k + lane] = wv;
  }
}

hipError_t launch_gate(const GateArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  constexpr int waves = 4;
  hipLaunchKernelGGL(gate_topk_kernel, dim3(ceil_div(a.T, waves)), dim3(waves * WAVE), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
