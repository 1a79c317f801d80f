// Tiled matrix-core GEMM for gfx950: the GEMM end of the per-expert
// GEMV/GEMM switch (SwiftGMM's mode switch by load intensity, page
// "华为技术披露集 VOL.12：昇腾×盘古", section SwiftGMM), used for experts and
// dense problems with many rows (prefill experts, the shared expert, the
// router at large T).
//
// Work split: a workgroup (4 wavefronts) owns BM rows x 4*NF output features
// of one group (expert). The BM gathered activation rows are the shared
// operand: they are staged through LDS in 256-byte-per-row chunks (double
// buffered; the global loads of a chunk run two chunks ahead in registers),
// rows padded by 16 bytes so the rows a 32x32 matrix-core operand reads land
// in distinct banks. The weights are not shared between wavefronts (each
// wavefront owns NF features), so they go straight from global memory into
// a register ring 8 matrix-core steps deep, in the packed fragment layout: a
// 32x32 operand is four 256-byte pieces of two adjacent 16-column fragments.
// Each weight fragment is reused for BM rows. Weights that only this tile
// reads (its group has one m-tile) carry the nontemporal hint.
//
// Split-K: when rows x features give too few workgroups to fill the device
// (decode-sized shared expert), the reduction is cut into `splits` ranges;
// each writes raw fp32 (int32 for int8) partial sums, and gemm_reduce_kernel
// adds them in split order and applies the epilogue, so the result does not
// depend on scheduling. A four-way split of 32-row bf16 tiles can instead
// run inside one workgroup (LdsArgs::wave_split): its four wavefronts own the
// same 32 features and one range each, stage the four ranges' activation
// chunks side by side in LDS, and add their sums in range order through LDS
// before one epilogue - the same sums, with no partial sums in memory and no
// reduce launch.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {


struct M32BF16 {
  using op_t = bf16x8;
  using acc_t = f32x16;
  using part_t = float;
  static constexpr int KF = 32, KM = 16, BPL = 16, ESZ = 2;
  static constexpr bool SCALED = false;   // no per-row / per-column scales
  __device__ static inline acc_t mfma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t load(const uint8_t* p) {
    return __builtin_bit_cast(op_t, *reinterpret_cast<const u32x4*>(p));
  }
  template <bool NT>
  __device__ static inline op_t load_w(const uint8_t* p) {
    if constexpr (NT) return __builtin_bit_cast(op_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
    return load(p);
  }
};
struct M32I8 {
  using op_t = i32x4;
  using acc_t = i32x16;
  using part_t = int;
  static constexpr int KF = 64, KM = 32, BPL = 16, ESZ = 1;
  static constexpr bool SCALED = true;    // int8 codes: activation-row and weight-column scales
  __device__ static inline acc_t mfma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t load(const uint8_t* p) {
    return __builtin_bit_cast(op_t, *reinterpret_cast<const u32x4*>(p));
  }
  template <bool NT>
  __device__ static inline op_t load_w(const uint8_t* p) {
    if constexpr (NT) return __builtin_bit_cast(op_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
    return load(p);
  }
};
struct M32F32 {
  using op_t = float;
  using acc_t = f32x16;
  using part_t = float;
  static constexpr int KF = 4, KM = 2, BPL = 4, ESZ = 4;
  static constexpr bool SCALED = false;
  __device__ static inline acc_t mfma(op_t a, op_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline op_t load(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }
  template <bool NT>
  __device__ static inline op_t load_w(const uint8_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const float*>(p));
    return load(p);
  }
};

constexpr int CH_BYTES = 256;              // bytes of one row per LDS chunk
constexpr int LDS_ROW = CH_BYTES + 16;     // padded row stride (4-bank shift per row)

template <class Tr, int S, int EPI, int NF, int BM, int RA, bool W_NT, int KW>
__device__ __forceinline__ void gemm_lds_tile(const GemmArgs& a, const LdsArgs& L,
                                              uint8_t (&lds)[2][KW * BM * LDS_ROW], int g, int row0, int nrows,
                                              int out0, int nblock, int split) {
  constexpr int FT = NF / 32;                  // 32-feature tiles per wavefront
  constexpr int MBK = BM / 32;                 // 32-row blocks per tile
  constexpr int FB = FRAG_LANES * Tr::BPL;     // packed fragment bytes
  constexpr int CH_ELEMS = CH_BYTES / Tr::ESZ;
  constexpr int CH_KT = CH_ELEMS / Tr::KF;     // packed reduction steps per chunk
  constexpr int CH_KS = CH_ELEMS / Tr::KM;     // matrix-core steps per chunk
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int LOADS = BM * CH_BYTES / (WG_THREADS * 16);   // 16-byte B loads per thread per chunk
  using op_t = typename Tr::op_t;
  using acc_t = typename Tr::acc_t;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  // KW > 1: the wavefronts split the reduction instead of the features (KW
  // equal ranges of chunks, one per wavefront, all on the same WN * NF
  // features); their sums are added at the end in range order, as the
  // split-K reduce pass adds slices, so no partial sums leave the workgroup.
  constexpr int WN = WG_WAVES / KW;
  const int wave_n = wave % WN, wave_k = wave / WN;

  const int KT = a.K / Tr::KF;
  const int KC = a.K / CH_ELEMS;               // chunks in the whole reduction
  const int c_base = split * KC / L.splits;    // this slice's chunks (KW ranges of nch)
  const int nch = ((split + 1) * KC / L.splits - c_base) / KW;
  const int c_begin = c_base + wave_k * nch;   // this wavefront's range

  // ---- A: this wavefront's feature tiles, straight from global ----
  // A wavefront past the last feature tile (N not a multiple of the block)
  // computes a copy of the last tile and stores nothing.
  const int ft_first = (nblock * WN + wave_n) * FT;
  const bool wave_live = ft_first * 32 < a.N;
  const int ft0 = wave_live ? ft_first : a.N / 32 - FT;
  const int r32 = lane & 31, half = lane >> 5;
  // The wavefront's 2*FT fragment columns lie in one block of the packed
  // layout (2*ft0 is a multiple of 2*FT, and 2*FT divides the block).
  const int NT = a.N / 16;
  const size_t FBW = size_t(frag_block_width(2 * ft0, NT)) * FB;   // stride of one plane step
  const uint8_t* abase = a.A + size_t(g) * a.a_group_stride + frag_offset(2 * ft0 + (r32 >> 4), 0, 0, NT, KT, S, FB) +
                         (half * 16 + (r32 & 15)) * Tr::BPL;
  // Ring of RA matrix-core steps of weight operands, refilled RA steps ahead
  // across chunk boundaries. Every load is unconditional (steps past the end
  // re-read the last one), so the waits only drain the step being used.
  static_assert((2 * CH_KS) % RA == 0, "ring must divide two chunks");
  op_t aring[RA][FT][S];
  const int nsteps = nch * CH_KS;
  auto load_a = [&](int slot, int i) {
    const int kt = c_begin * CH_KT + (i >> 1);
    const int h = i & 1;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int s = 0; s < S; ++s)
        aring[slot][f][s] = Tr::template load_w<W_NT>(abase + (size_t(kt) * S + s) * FBW + size_t(2 * f) * FB +
                                                    h * 2 * 16 * Tr::BPL);
  };


  // ---- epilogue operands that depend on columns only, loaded now so their
  // latency hides under the main loop (none for unscaled, bias-free products;
  // a load in the epilogue would also wait for every load still in flight) ----
  const bool final_out = L.splits == 1;   // split-K slices write raw partial sums
  // int8 weight scales of columns c0..c0+3; the widest int8 tile (64
  // features, 128 rows) has no registers to spare and reads them at the end
  constexpr bool EARLY_CS = Tr::SCALED && !(NF == 64 && BM == 128);
  f32x4 ep_cs[NACC][FT][4];
  f32x4 ep_bias[FT][4];                   // sums: logit bias of columns c0..c0+3 (0 past n_valid)
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int c0 = (ft0 + f) * 32 + 8 * jg + 4 * half;
#pragma unroll
      for (int s = 0; s < NACC; ++s) {
        ep_cs[s][f][jg] = f32x4{1.f, 1.f, 1.f, 1.f};
        const float* sp = s == 0 ? a.a_scale0 : a.a_scale1;
        if constexpr (EARLY_CS)
          if (final_out && sp) ep_cs[s][f][jg] = *reinterpret_cast<const f32x4*>(sp + size_t(g) * a.a_scale_stride + c0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ep_bias[f][jg][j] = 0.f;
        if constexpr (EPI == EPI_SUM)
          if (final_out && a.bias && c0 + j < a.n_valid) ep_bias[f][jg][j] = a.bias[c0 + j];
      }
    }

  // ---- B staging: this thread's rows and byte column inside a chunk ----
  // (int8: the threads at byte column 0 also fetch their row's activation
  // scale, which reaches the epilogue's lanes through LDS)
  __shared__ float bs_lds[BM];
  // The rows' slot ids are loaded together (one round trip, not one per
  // load: a test of the table pointer around each load made the compiler
  // wait after each), then the row addresses and (int8) row scales follow.
  const uint8_t* bsrc[LOADS];
  int bdst[LOADS];
  float bsv[LOADS];
  int brow[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int lin = threadIdx.x + i * WG_THREADS;
    brow[i] = out0 + min(lin / (CH_BYTES / 16), nrows - 1);
  }
  if (a.sorted_slot) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) brow[i] = a.sorted_slot[row0 + (brow[i] - out0)];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) brow[i] /= a.k;
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int lin = threadIdx.x + i * WG_THREADS;
    const int r = lin / (CH_BYTES / 16);
    const int col = (lin % (CH_BYTES / 16)) * 16;
    bsrc[i] = a.B + size_t(brow[i]) * a.ldb + size_t(c_base) * CH_BYTES + col;
    bdst[i] = r * LDS_ROW + col;
    bsv[i] = 1.f;
  }
  if constexpr (Tr::SCALED) {
    if (final_out && a.b_scale) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const float v = a.b_scale[brow[i]];
        if (((threadIdx.x + i * WG_THREADS) % (CH_BYTES / 16)) == 0) bsv[i] = v;
      }
    }
  }
  float ep_bs[MBK];   // activation scale of epilogue row m * 32 + r32
#pragma unroll
  for (int m = 0; m < MBK; ++m) ep_bs[m] = 1.f;
  // Two register stages of chunk loads (parity of the chunk index); with
  // KW ranges, chunk c of every range (range q in LDS rows q * BM ...).
  u32x4 bstage[2][KW][LOADS];
  auto load_b = [&](int st, int c) {
#pragma unroll
    for (int q = 0; q < KW; ++q)
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        bstage[st][q][i] = *reinterpret_cast<const u32x4*>(bsrc[i] + size_t(q * nch + c) * CH_BYTES);
  };
  auto store_b = [&](int st, int buf) {
#pragma unroll
    for (int q = 0; q < KW; ++q)
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        *reinterpret_cast<u32x4*>(&lds[buf][q * BM * LDS_ROW + bdst[i]]) = bstage[st][q][i];
  };

  acc_t acc[NACC][FT][MBK];
#pragma unroll
  for (int s = 0; s < NACC; ++s)
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int m = 0; m < MBK; ++m)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[s][f][m][j] = 0;

  // One chunk: matrix-core steps from LDS buffer `buf`, then the next chunk
  // (loaded two chunks ago into register stage `st`) goes to the other
  // buffer and that stage is refilled with the chunk after next.
  auto read_b = [&](op_t (&dst)[MBK], int buf, int ks) {
#pragma unroll
    for (int m = 0; m < MBK; ++m)
      dst[m] = Tr::load(&lds[buf][(wave_k * BM + m * 32 + r32) * LDS_ROW + ks * (Tr::KM * Tr::ESZ) + half * Tr::BPL]);
  };
  // One chunk. Inside a step: read the next step's LDS operands, run this
  // step's matrix-core work, refill this step's weight slot RA steps ahead;
  // scheduling barriers keep that order (left alone, the compiler sinks the
  // refills to the end of the chunk, which empties the weight ring). After
  // the chunk the next chunk (loaded two chunks ago into register stage
  // `st`) goes to the other LDS buffer and the stage is refilled.
  auto chunk = [&](auto st_tag, int c) {
    constexpr int st = decltype(st_tag)::value;
    const int buf = c & 1;
    op_t bfa[MBK], bfb[MBK];
    read_b(bfa, buf, 0);
#pragma unroll
    for (int ks = 0; ks < CH_KS; ++ks) {
      const int slot = ((st ^ 1) * CH_KS + ks) % RA;   // chunk c has parity st ^ 1
      op_t(&cur)[MBK] = (ks & 1) ? bfb : bfa;
      op_t(&nxt)[MBK] = (ks & 1) ? bfa : bfb;
      if (ks + 1 < CH_KS) read_b(nxt, buf, ks + 1);
#pragma unroll
      for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int m = 0; m < MBK; ++m) {
            const int sa = (EPI == EPI_SWIGLU) ? s : 0;
            acc[sa][f][m] = Tr::mfma(aring[slot][f][s], cur[m], acc[sa][f][m]);
          }
      load_a(slot, min(c * CH_KS + ks + RA, nsteps - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    store_b(st, buf ^ 1);          // chunk c + 1 (a copy nobody reads after the last)
    load_b(st, min(c + 3, nch - 1));
    __syncthreads();
  };

  if (nch > 0) {
    load_b(0, 0);
    load_b(1, min(1, nch - 1));
#pragma unroll
    for (int r = 0; r < RA; ++r) load_a(r, min(r, nsteps - 1));
    store_b(0, 0);
    load_b(0, min(2, nch - 1));
    if constexpr (Tr::SCALED) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int lin = threadIdx.x + i * WG_THREADS;
        if (lin % (CH_BYTES / 16) == 0) bs_lds[lin / (CH_BYTES / 16)] = bsv[i];
      }
    }
    __syncthreads();
    // read before the chunk barriers below, so the next tile may rewrite bs_lds
    if constexpr (Tr::SCALED) {
#pragma unroll
      for (int m = 0; m < MBK; ++m) ep_bs[m] = bs_lds[m * 32 + r32];
    }
    // chunk c stores chunk c + 1 from stage (c + 1) & 1
    int c = 0;
    for (; c + 2 <= nch; c += 2) {
      chunk(std::integral_constant<int, 1>{}, c);
      chunk(std::integral_constant<int, 0>{}, c + 1);
    }
    if (c < nch) chunk(std::integral_constant<int, 1>{}, c);
  }
  if constexpr (KW > 1) {
    // The ranges' sums meet in LDS buffer 1 (free: every read of the chunks
    // came before the last chunk's barrier, and the next tile writes buffer
    // 1 only after its first barrier, which range 0's wavefronts reach once
    // done here); they add the others in range order and run the epilogue.
    using part_t = typename Tr::part_t;
    constexpr int PER = NACC * FT * MBK * 16;   // accumulator elements per lane
    static_assert((KW - 1) * PER * WAVE * WN * sizeof(part_t) <= sizeof(lds[1]), "range sums must fit the LDS");
    part_t* red = reinterpret_cast<part_t*>(&lds[1][0]);
    auto at = [&](int q, int s, int f, int m, int j) {
      return red + (((size_t(q - 1) * WN + wave_n) * PER + ((s * FT + f) * MBK + m) * 16 + j) * WAVE + lane);
    };
    if (wave_k > 0) {
#pragma unroll
      for (int s = 0; s < NACC; ++s)
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
          for (int m = 0; m < MBK; ++m)
#pragma unroll
            for (int j = 0; j < 16; ++j) *at(wave_k, s, f, m, j) = acc[s][f][m][j];
    }
    __syncthreads();
    if (wave_k > 0) return;
    for (int q = 1; q < KW; ++q)
#pragma unroll
      for (int s = 0; s < NACC; ++s)
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
          for (int m = 0; m < MBK; ++m)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[s][f][m][j] += *at(q, s, f, m, j);
  }
  if (!wave_live) return;

  // ---- epilogue ----
  // acc[.][f][m] element j: feature ft*32 + 8*(j/4) + 4*half + j%4, row m*32 + r32.
#pragma unroll
  for (int m = 0; m < MBK; ++m) {
    const int r = m * 32 + r32;
    if (r >= nrows) continue;
    const int orow = out0 + r;
    const float bs = ep_bs[m];
#pragma unroll
    for (int f = 0; f < FT; ++f) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int c0 = (ft0 + f) * 32 + 8 * jg + 4 * half;
        if (L.splits > 1) {
          // raw partial sums: [split][row][S * N], plane s at column s * N + c
          typename Tr::part_t* P = reinterpret_cast<typename Tr::part_t*>(L.partial) +
                                   (size_t(split) * L.part_rows + orow) * size_t(NACC) * a.N;
#pragma unroll
          for (int s = 0; s < NACC; ++s) {
            typename Tr::part_t v4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = acc[s][f][m][jg * 4 + j];
            *reinterpret_cast<u32x4*>(P + size_t(s) * a.N + c0) = __builtin_bit_cast(u32x4, v4);
          }
          continue;
        }
        if constexpr (Tr::SCALED && !EARLY_CS) {
#pragma unroll
          for (int s = 0; s < NACC; ++s) {
            const float* sp = s == 0 ? a.a_scale0 : a.a_scale1;
            if (sp) ep_cs[s][f][jg] = *reinterpret_cast<const f32x4*>(sp + size_t(g) * a.a_scale_stride + c0);
          }
        }
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float cs0 = ep_cs[0][f][jg][j];
          if (EPI == EPI_SWIGLU) {
            const float cs1 = ep_cs[NACC - 1][f][jg][j];
            const float ga = float(acc[0][f][m][jg * 4 + j]) * bs * cs0;
            const float up = float(acc[1][f][m][jg * 4 + j]) * bs * cs1;
            v[j] = silu_f(ga) * up;
          } else {
            v[j] = float(acc[0][f][m][jg * 4 + j]) * bs * cs0 + ep_bias[f][jg][j];
          }
        }
        uint8_t* op = a.out + size_t(orow) * a.ldo;
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
  }
}

// Persistent over tiles: the grid is a fixed number of workgroups (a
// multiple of 8); the tiles (column block x m-tile) are counted on the
// device from the offsets, cut into 8 contiguous ranges, one per XCD
// (blocks are dealt to the XCDs round-robin, so block b runs on XCD b % 8),
// and each workgroup walks its XCD's range with a stride of the workgroups
// on that XCD. The order is m-tile fastest (group_m <= 1): tiles sharing a
// weight column block run close together in time on one L2. With
// group_m > 1 it walks panels of group_m m-tiles, m-tile fastest inside a
// panel and column block next: the workgroups running together on an XCD
// then share both the weights of a few column blocks and the activation
// rows of a few m-tiles in its L2 (the order for dense products with many
// m-tiles, whose activation rows are re-read once per column block).
#ifndef MOE_RING_S2_BM64
#define MOE_RING_S2_BM64 4
#endif
// 32-row tiles (one row block) hold half the accumulators of 64-row ones:
// an 8-step ring at two wavefronts per SIMD fits their registers.
template <class Tr, int S, int EPI, int NF, int BM>
constexpr int ring_steps() { return S == 1 || BM == 128 || BM == 32 ? 8 : MOE_RING_S2_BM64; }
template <class Tr, int S, int EPI, int NF, int BM>
constexpr int lds_waves_per_eu() { return BM <= 64 && NF == 32 && ring_steps<Tr, S, EPI, NF, BM>() <= 8 ? 2 : 1; }

template <class Tr, int S, int EPI, int NF, int BM, int KW>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(lds_waves_per_eu<Tr, S, EPI, NF, BM>())))
void gemm_lds_kernel(GemmArgs a, LdsArgs L) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][KW * BM * LDS_ROW];
  __shared__ int offs[TILE_MAX_GROUPS + 1];
  stage_offsets(a, offs);
  const int tiles = count_tiles_lds(a, offs, BM, L.min_rows, L.max_rows);
  const int nblocks = ceil_div(a.N, (WG_WAVES / KW) * NF);
  const int total = tiles * nblocks;
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per_xcd_wg = nwg / 8;
  const int q = ceil_div(total, 8);
  const int lo = xcd * q, hi = min(total, lo + q);
  const int gm = max(L.group_m, 1);
  for (int logical = lo + slot; logical < hi; logical += per_xcd_wg) {
    int tile, nblock;
    if (gm == 1) {
      tile = logical % tiles;
      nblock = logical / tiles;
    } else {
      const int pstart = logical / (gm * nblocks) * gm;   // first m-tile of the panel
      const int pm = min(gm, tiles - pstart);              // the last panel may be short
      const int within = logical - pstart * nblocks;
      nblock = within / pm;
      tile = pstart + within % pm;
    }
    int g, row0, nrows, out0;
    if (!locate_tile_lds(a, offs, tile, BM, L.min_rows, L.max_rows, g, row0, nrows, out0)) break;
    g = __builtin_amdgcn_readfirstlane(g);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    out0 = __builtin_amdgcn_readfirstlane(out0);
    // Weights of a group whose rows fit one m-tile are read by this tile
    // alone (other tiles of the launch are other groups, other column
    // blocks or other reduction slices): they are loaded with the
    // nontemporal hint, which keeps them from displacing the activation rows
    // (re-read by every column block) in the L2. Groups with several m-tiles
    // re-read their weights and load them normally.
    const bool once = a.offsets ? offs[g + 1] - offs[g] <= BM : a.dense_rows <= BM;
    constexpr int RA = ring_steps<Tr, S, EPI, NF, BM>();
    if (once)
      gemm_lds_tile<Tr, S, EPI, NF, BM, RA, true, KW>(a, L, lds, g, row0, nrows, out0, nblock, blockIdx.z);
    else
      gemm_lds_tile<Tr, S, EPI, NF, BM, RA, false, KW>(a, L, lds, g, row0, nrows, out0, nblock, blockIdx.z);
  }
}

constexpr int REDUCE_BATCH = 4;
// Sum of the split partials in split order, then the epilogue of the
// product. One thread per 4 output columns of one row; rows of the selected
// groups only.
template <typename PT, int EPI>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs a, LdsArgs L) {
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  const int cols4 = a.N / 4;
  // The groups' offsets in LDS: the row-to-group search below reads them
  // there instead of making a dependent global round trip per step.
  __shared__ int offs[TILE_MAX_GROUPS + 1];
  stage_offsets(a, offs);
  // Rows to reduce: the compacted rows of the groups (known on the device
  // only), or the dense rows; a grid-stride loop covers them.
  int base = 0, rows = min(a.dense_rows, L.part_rows);
  if (a.offsets) {
    base = offs[0];
    rows = min(offs[a.n_groups] - base, L.part_rows);
  }
  const size_t total = size_t(rows) * cols4;
  for (size_t idx = blockIdx.x * size_t(blockDim.x) + threadIdx.x; idx < total;
       idx += size_t(gridDim.x) * blockDim.x) {
    const int orow = int(idx / cols4);
    const int c0 = int(idx % cols4) * 4;
    // Which group holds this compacted row, and is it one this product covered?
    int g = 0, brow = orow;
    if (a.offsets) {
      const int srow = orow + base;
      int lo = 0, hi = a.n_groups - 1;   // last group whose start <= srow
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (offs[mid] <= srow) lo = mid; else hi = mid - 1;
      }
      g = lo;
      const int n = offs[g + 1] - offs[g];
      if (n < L.min_rows || n > L.max_rows) continue;
      brow = a.sorted_slot ? a.sorted_slot[srow] / a.k : orow;
    }
    float sum[NACC][4];
#pragma unroll
    for (int s = 0; s < NACC; ++s) {
      PT t[4] = {0, 0, 0, 0};
      // REDUCE_BATCH slices loaded together (clamped slice index: every
      // address is valid), then added in slice order
      for (int sp0 = 0; sp0 < L.splits; sp0 += REDUCE_BATCH) {
        PT q4[REDUCE_BATCH][4];
#pragma unroll
        for (int b = 0; b < REDUCE_BATCH; ++b) {
          const int sp = min(sp0 + b, L.splits - 1);
          const PT* P = reinterpret_cast<const PT*>(L.partial) +
                        (size_t(sp) * L.part_rows + orow) * size_t(NACC) * a.N + size_t(s) * a.N + c0;
#pragma unroll
          for (int j = 0; j < 4; ++j) q4[b][j] = P[j];
        }
#pragma unroll
        for (int b = 0; b < REDUCE_BATCH; ++b)
          if (sp0 + b < L.splits)
#pragma unroll
            for (int j = 0; j < 4; ++j) t[j] += q4[b][j];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[s][j] = float(t[j]);
    }
    const float bs = a.b_scale ? a.b_scale[brow] : 1.f;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float cs0 = a.a_scale0 ? a.a_scale0[size_t(g) * a.a_scale_stride + c0 + j] : 1.f;
      if (EPI == EPI_SWIGLU) {
        const float cs1 = a.a_scale1 ? a.a_scale1[size_t(g) * a.a_scale_stride + c0 + j] : 1.f;
        v[j] = silu_f(sum[0][j] * bs * cs0) * (sum[1][j] * bs * cs1);
      } else {
        const float bias = (a.bias && c0 + j < a.n_valid) ? a.bias[c0 + j] : 0.f;
        v[j] = sum[0][j] * bs * cs0 + bias;
      }
    }
    uint8_t* op = a.out + size_t(orow) * a.ldo;
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

hipError_t launch_gemm_reduce(const GemmArgs& a, const LdsArgs& L, GemmElem elem, GemmEpi epi, hipStream_t stream,
                              hipEvent_t stop) {
  const size_t threads = size_t(L.part_rows) * (a.N / 4);
  const dim3 grid(unsigned(std::min<size_t>((threads + 255) / 256, 2048)));   // grid-stride beyond
  if (elem == ELEM_I8)
    return epi == EPI_SWIGLU ? launch_timed((gemm_reduce_kernel<int, EPI_SWIGLU>), grid, dim3(256), stream, nullptr, stop, a, L)
                             : launch_timed((gemm_reduce_kernel<int, EPI_SUM>), grid, dim3(256), stream, nullptr, stop, a, L);
  return epi == EPI_SWIGLU ? launch_timed((gemm_reduce_kernel<float, EPI_SWIGLU>), grid, dim3(256), stream, nullptr, stop, a, L)
                           : launch_timed((gemm_reduce_kernel<float, EPI_SUM>), grid, dim3(256), stream, nullptr, stop, a, L);
}

int lds_chunk_elems(GemmElem elem) { return CH_BYTES / (elem == ELEM_F32 ? 4 : (elem == ELEM_BF16 ? 2 : 1)); }

template <class Tr, int S, int EPI, int NF, int BM, int KW = 1>
static hipError_t launch_lds_one(const GemmArgs& a, const LdsArgs& L, hipStream_t stream, KernelEvents ev) {
  // persistent grid: at most `tiles_y` m-tiles per column block exist
  const long bound = long(ceil_div(a.N, (WG_WAVES / KW) * NF)) * a.tiles_y;
  const int nwg = int(std::max(8L, std::min(bound, long(L.max_wgs)) / 8 * 8));
  const dim3 grid(nwg, 1, L.splits);
  const bool reduce = L.splits > 1 && !L.fold_reduce;
  hipError_t e = launch_timed((gemm_lds_kernel<Tr, S, EPI, NF, BM, KW>), grid, dim3(WG_THREADS), stream, ev.start,
                              reduce ? nullptr : ev.stop, a, L);
  if (e != hipSuccess || !reduce) return e;
  return launch_gemm_reduce(a, L, std::is_same<typename Tr::part_t, int>::value ? ELEM_I8 : ELEM_BF16, GemmEpi(EPI),
                            stream, ev.stop);
}

// 64 features per wavefront for one-plane products only: with two or three
// planes the 64-feature, 128-row tile needs more than the 512 registers of a
// lane (measured: 287 spilled registers with a 4-step ring).
template <class Tr, int S, int EPI>
static hipError_t launch_lds_shape(const GemmArgs& a, const LdsArgs& L, hipStream_t stream, KernelEvents ev) {
  if constexpr (S == 1) {
    if (L.wave_features == 64)
      return L.tile_rows == 64 ? launch_lds_one<Tr, S, EPI, 64, 64>(a, L, stream, ev)
                               : launch_lds_one<Tr, S, EPI, 64, 128>(a, L, stream, ev);
  }
  if (L.wave_split > 1) {
    // the reduction split over the 4 wavefronts: 32-row tiles, bf16, one or
    // two planes, no grid split, whole ranges of 256-byte chunks (the int8
    // two-plane tile would spill: 104 bytes per lane)
    if constexpr (S <= 2 && std::is_same<Tr, M32BF16>::value)
      if (L.wave_split == WG_WAVES && L.tile_rows == 32 && L.splits == 1 && (a.K / (CH_BYTES / Tr::ESZ)) % WG_WAVES == 0)
        return launch_lds_one<Tr, S, EPI, 32, 32, WG_WAVES>(a, L, stream, ev);
    return hipErrorInvalidValue;
  }
  if (L.tile_rows == 32) return launch_lds_one<Tr, S, EPI, 32, 32>(a, L, stream, ev);
  return L.tile_rows == 64 ? launch_lds_one<Tr, S, EPI, 32, 64>(a, L, stream, ev)
                           : launch_lds_one<Tr, S, EPI, 32, 128>(a, L, stream, ev);
}

hipError_t launch_gemm_lds(const GemmArgs& a, const LdsArgs& L, GemmElem elem, int planes, GemmEpi epi,
                           hipStream_t stream, KernelEvents ev) {
  if (a.offsets && (a.n_groups < 1 || a.n_groups > TILE_MAX_GROUPS)) return hipErrorInvalidValue;
  if (a.tiles_y <= 0) return record_events(ev.start, ev.stop, stream);
  if (epi == EPI_SWIGLU) {
    switch (elem) {
      case ELEM_BF16: return launch_lds_shape<M32BF16, 2, EPI_SWIGLU>(a, L, stream, ev);
      case ELEM_I8: return launch_lds_shape<M32I8, 2, EPI_SWIGLU>(a, L, stream, ev);
      case ELEM_F32: return launch_lds_shape<M32F32, 2, EPI_SWIGLU>(a, L, stream, ev);
    }
  } else {
    switch (elem) {
      case ELEM_BF16:
        return planes == 3 ? launch_lds_shape<M32BF16, 3, EPI_SUM>(a, L, stream, ev)
                           : launch_lds_shape<M32BF16, 1, EPI_SUM>(a, L, stream, ev);
      case ELEM_I8: return launch_lds_shape<M32I8, 1, EPI_SUM>(a, L, stream, ev);
      case ELEM_F32: return launch_lds_shape<M32F32, 1, EPI_SUM>(a, L, stream, ev);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
