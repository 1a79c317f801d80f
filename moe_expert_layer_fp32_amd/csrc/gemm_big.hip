// Large-tile bf16 matrix-core GEMM for gfx950: the products of the layer
// that are bound by the matrix cores at prefill sizes (the shared expert over
// thousands of tokens, routed experts with hundreds of rows). It is the GEMM
// end of SwiftGMM's switch between weight streaming and tiled products by
// per-expert load (page "华为技术披露集 VOL.12：昇腾×盘古", section SwiftGMM):
// the "left matrix" (the expert's activation rows) and the weights are both
// staged once per tile step and reused from LDS by every wavefront.
//
// Tile: 256 rows x 256 weight columns, reduction in steps of 64 elements.
// SwiGLU products (two weight planes, W1 gate and W3 up) take one packed
// column block of 128 features with both planes; one-plane products take two
// column blocks (256 features). Four wavefronts in a 2 x 2 arrangement each
// own 128 rows x 128 weight columns: 4 x 4 matrix-core tiles of 32 x 32
// (32x32x16 bf16), 256 fp32 accumulators per lane. For SwiGLU a wavefront's
// 128 weight columns are the same 64 features of both planes, so the
// epilogue pairs gate and up in registers.
//
// Staging: both operands go from global memory straight into LDS with the
// direct-to-LDS 16-byte load (no register round trip), double buffered
// (2 x 64 KiB; one workgroup per compute unit). The weight step of a tile is
// a plain copy of 32 KiB of the packed layout (one or two contiguous runs),
// which the matrix-core operand reads hit without bank conflicts (each
// 16-lane group reads one contiguous 256 bytes). Activation rows are 128
// bytes per step; their 16-byte segments are stored XOR-swizzled by
// (row / 2) mod 8, so the 32 rows a matrix-core operand reads spread over
// all banks. The loads of step c + 1 are issued right after the barrier that
// opens step c and have step c's matrix-core work to land.
//
// Persistent grid over tiles like the other tiled kernel: the tiles (column
// block x m-tile of an expert, or of the dense rows) are counted on the
// device from the routing offsets, cut into 8 contiguous ranges, one per XCD,
// and walked in panels of group_m m-tiles (m-tile fastest inside a panel),
// so the workgroups running together on an XCD share weights and rows in its
// L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

constexpr int BIG_BK = 32;                            // reduction elements per step
constexpr int BIG_W_BYTES = 256 * BIG_BK * 2;         // 16 KiB of weights per step
constexpr int BIG_A_BYTES = BIG_TILE_ROWS * BIG_BK * 2;  // 16 KiB of activation rows per step
constexpr int BIG_STAGE = BIG_W_BYTES + BIG_A_BYTES;  // 32 KiB; four stages in LDS
constexpr int BIG_PIECES = BIG_W_BYTES / 16 / WG_THREADS;   // 16-byte loads per thread per operand (4)
#ifndef MOE_BIG_AHEAD
#define MOE_BIG_AHEAD 3
#endif
constexpr int BIG_AHEAD = MOE_BIG_AHEAD;              // steps in flight beyond the one being read (<= 3)
constexpr int FRAG = 1024;                            // packed fragment bytes (16 columns x 32 bf16)

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates: vector memory counter at most N (0, 8 or 16: the
// loads of the steps still allowed in flight), LDS counter 0, export
// counter untouched. vmcnt is bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8].
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

__device__ __forceinline__ void load_to_lds(const uint8_t* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g),
                                   (lds_void*)(lds_wave_base), 16, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_op(const uint8_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Workgroup barrier for the staging pipeline: this wave's direct-to-LDS
// loads older than the newest `pending` steps' have landed and its LDS reads
// are done, then every wave arrives. No memory fence: the wait is explicit
// (a workgroup-scope release does not wait for loads, and the compiler does
// not follow these LDS writes across loop iterations); the empty asm keeps
// the compiler from moving memory accesses across the barrier.
template <int PENDING_LOADS>
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(PENDING_LOADS));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef uint8_t stage_t[BIG_STAGE];

template <int EPI>
__device__ __forceinline__ void big_tile(const GemmArgs& a, stage_t& l0, stage_t& l1, stage_t& l2, stage_t& l3,
                                         int g, int row0, int nrows, int out0, int nblock) {
  // buffer b by compile-time index: each access names one LDS array, so the
  // compiler can tell a read of one buffer from a load into another
  auto buf = [&](auto bi) -> uint8_t* {
    constexpr int B = decltype(bi)::value & 3;
    if constexpr (B == 0) return l0;
    else if constexpr (B == 1) return l1;
    else if constexpr (B == 2) return l2;
    else return l3;
  };
  constexpr int S = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int LOADS = 2 * BIG_PIECES;           // direct-to-LDS loads per thread and step
  const int t = threadIdx.x, lane = t & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(t / WAVE);   // wave-uniform: LDS bases stay scalar
  const int wm = w & 1, wn = w >> 1;
  const int KT = a.K / 32;                        // packed 32-element steps (= tile steps)
  const int nst = KT;
  const int NT = a.N / 16;                        // fragment columns per plane

  // ---- staging sources of this thread (4 weight and 4 activation pieces
  //      of 16 bytes per step) ----
  // Weights: piece p = i * 256 + t of the step's 16 KiB. SwiGLU: one
  // contiguous run (column block nblock, both planes of one packed step);
  // one plane: two runs of 8 KiB (column blocks 2 nblock and 2 nblock + 1).
  const uint8_t* gbase = a.A + size_t(g) * a.a_group_stride;
  const uint8_t* wsrc0 = gbase + (S == 2 ? frag_offset(nblock * FRAG_BLOCK, 0, 0, NT, KT, 2, FRAG)
                                         : frag_offset(2 * nblock * FRAG_BLOCK, 0, 0, NT, KT, 1, FRAG)) + t * 16;
  const uint8_t* wsrc1 = S == 2 ? wsrc0 + 2 * WG_THREADS * 16
                                : gbase + frag_offset((2 * nblock + 1) * FRAG_BLOCK, 0, 0, NT, KT, 1, FRAG) + t * 16;
  const size_t wstep = size_t(S) * FRAG_BLOCK * FRAG;   // bytes of one packed step of a column block
  // Activations: piece q = i * 256 + t is row i * 64 + t / 4, stored at
  // physical segment t % 4 of the row's 64 bytes, which holds logical
  // segment (t % 4) ^ swizzle; the swizzle (row / 4) % 4 is (t / 16) % 4 for
  // every i. Rows past the tile re-read its last row (their results are not
  // stored).
  const int aseg = (t & 3) ^ ((t >> 4) & 3);
  int brow[BIG_PIECES];
#pragma unroll
  for (int i = 0; i < BIG_PIECES; ++i) brow[i] = min(i * 64 + (t >> 2), nrows - 1);
  if (a.sorted_slot) {
    // all lookups issued before any is used (one round trip)
#pragma unroll
    for (int i = 0; i < BIG_PIECES; ++i) brow[i] = a.sorted_slot[row0 + brow[i]];
#pragma unroll
    for (int i = 0; i < BIG_PIECES; ++i) brow[i] /= a.k;
  } else {
#pragma unroll
    for (int i = 0; i < BIG_PIECES; ++i) brow[i] += out0;
  }
  const uint8_t* asrc[BIG_PIECES];
#pragma unroll
  for (int i = 0; i < BIG_PIECES; ++i) asrc[i] = a.B + size_t(brow[i]) * a.ldb + aseg * 16;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto issue = [&](int c, uint8_t* dst) {
    uint8_t* wdst = dst + w * WAVE * 16;
    uint8_t* adst = dst + BIG_W_BYTES + w * WAVE * 16;
#pragma unroll
    for (int i = 0; i < BIG_PIECES; ++i)
      load_to_lds((S == 2 ? (i < 2 ? wsrc0 : wsrc1) + (i & 1) * WG_THREADS * 16
                          : (i < 2 ? wsrc0 : wsrc1) + (i & 1) * WG_THREADS * 16) + size_t(c) * wstep,
                  wdst + i * WG_THREADS * 16);
#pragma unroll
    for (int i = 0; i < BIG_PIECES; ++i) load_to_lds(asrc[i] + size_t(c) * (BIG_BK * 2), adst + i * WG_THREADS * 16);
  };

  // ---- operand read offsets inside a stage ----
  // Weight operand (src0, 32 features x 16 reduction elements): lane l takes
  // feature l % 32 (fragment l / 16 % 2 of a pair) and elements 8 (l / 32)
  // of the 16 (lanes 16 (2 ks + l / 32) of the 32-element fragment).
  const int wl = ((lane >> 4) & 1) * FRAG + (lane & 15) * 16 + (lane >> 5) * 256;
  // Activation operand (src1, 32 rows x 16 elements): lane l takes row
  // l % 32 and logical segment 2 ks + l / 32, stored at that ^ swizzle.
  const int swz = ((lane & 31) >> 2) & 3;
  int al[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    al[ks] = BIG_W_BYTES + (wm * 128 + (lane & 31)) * (BIG_BK * 2) + 16 * (((2 * ks) | (lane >> 5)) ^ swz);
  auto woff = [&](int ks, int nb) {
    if (S == 2) return (((nb >> 1) * FRAG_BLOCK + wn * 4 + (nb & 1) * 2) * FRAG) + ks * 512 + wl;
    return ((wn * FRAG_BLOCK + nb * 2) * FRAG) + ks * 512 + wl;
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[n][m][j] = 0.f;

  auto read = [&](const uint8_t* sb, int ks, bf16x8 (&wo)[4], bf16x8 (&ao)[4]) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) wo[nb] = lds_op(sb + woff(ks, nb));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) ao[mb] = lds_op(sb + al[ks] + mb * 32 * (BIG_BK * 2));
  };
  auto mma = [&](const bf16x8 (&wo)[4], const bf16x8 (&ao)[4]) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wo[nb], ao[mb], acc[nb][mb], 0, 0, 0);
  };
  // Software pipeline over 32-element steps, skewed by half a step so that
  // no matrix-core work waits for a barrier or an LDS read. Step c lives in
  // buffer c % 4; when a phase starts, the first 16-element slice of step c
  // is already in registers (w0, a0). A phase:
  //   read slice 1 of step c; run slice 0's 16 matrix-core ops;
  //   barrier: step c + 1 has landed (steps c + 2, c + 3 may still be in
  //     flight) and every wave has read all of step c;
  //   issue step c + 4 into buffer c % 4 (with BIG_AHEAD = 3); read
  //   slice 0 of step c + 1;
  //   run slice 1's 16 matrix-core ops (covering that read's latency).
  // The body has no branch: past the last step the issue repeats the last
  // step's loads into a buffer no later step reads, and the last phase's
  // read of "step nst" reads a stale buffer into registers nobody uses (the
  // barrier closing the tile waits for every load). Without a branch every
  // barrier waits for the same count and the compiler keeps track of which
  // buffer each load writes (at a branch it falls back to waiting for every
  // load). Scheduling barriers keep the order (left alone, the compiler
  // sinks each read to just before its use).
  bf16x8 w0[4], a0[4], w1[4], a1[4];
  // Instruction classes of the scheduling groups.
  constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;
  auto phase = [&](auto bi, int c) {
    constexpr int B = decltype(bi)::value;
    // slice 0 of step c; slice 1's operands read one per matrix-core op
    // (at most 8 LDS reads in flight: the counter holds 15)
    read(buf(bi), 1, w1, a1);
    mma(w0, a0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);   // first op only waits for slice 0's reads
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier<(BIG_AHEAD - 1) * LOADS>();
    // slice 1 of step c; the next step's slice-0 operands and the loads of
    // step c + 4 issued one each per matrix-core op
    issue(min(c + BIG_AHEAD + 1, nst - 1), buf(std::integral_constant<int, B + BIG_AHEAD + 1>{}));
    read(buf(std::integral_constant<int, B + 1>{}), 0, w0, a0);
    mma(w1, a1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // nst is a multiple of 4 (K % 128 == 0) and at least 4
  issue(0, buf(I0{}));
  if (BIG_AHEAD > 1) issue(1, buf(I1{}));
  if (BIG_AHEAD > 2) issue(2, buf(I2{}));
  stage_barrier<(BIG_AHEAD - 1) * LOADS>();    // step 0 has landed
  issue(BIG_AHEAD, buf(std::integral_constant<int, BIG_AHEAD>{}));
  read(buf(I0{}), 0, w0, a0);
  __builtin_amdgcn_sched_barrier(0);
  for (int c = 0; c < nst; c += 4) {
    phase(I0{}, c);
    phase(I1{}, c + 1);
    phase(I2{}, c + 2);
    phase(I3{}, c + 3);
  }
  stage_barrier<0>();   // stray loads landed and every read done before the next tile's issue

  // ---- epilogue ----
  // acc[nb][mb] element j: weight column 8 (j / 4) + 4 (l / 32) + j % 4 of
  // n-block nb, row mb * 32 + l % 32 of the wavefront's 128 rows.
  const int half = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int r = wm * 128 + mb * 32 + (lane & 31);
    if (r < nrows) {
      uint8_t* op = a.out + size_t(out0 + r) * a.ldo;
#pragma unroll
      for (int nb = 0; nb < (S == 2 ? 2 : 4); ++nb) {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int c0 = (S == 2) ? nblock * 128 + wn * 64 + nb * 32 + 8 * jg + 4 * half
                                  : (2 * nblock + wn) * 128 + nb * 32 + 8 * jg + 4 * half;
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (S == 2)
              v[j] = silu_f(acc[nb][mb][jg * 4 + j]) * acc[nb + 2][mb][jg * 4 + j];
            else
              v[j] = acc[nb][mb][jg * 4 + j];
          }
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
    // one 32-row block at a time (left alone, the compiler reads every
    // accumulator out at once and spills)
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int EPI>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_big_kernel(GemmArgs a, LdsArgs L) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[BIG_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[BIG_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[BIG_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t lds3[BIG_STAGE];
  __shared__ int offs[TILE_MAX_GROUPS + 1];
  constexpr int FEAT = (EPI == EPI_SWIGLU) ? 128 : 256;   // output features per tile
  stage_offsets(a, offs);
  const int tiles = count_tiles_lds(a, offs, BIG_TILE_ROWS, L.min_rows, L.max_rows);
  const int nblocks = a.N / FEAT;
  const int total = tiles * nblocks;
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per_xcd_wg = nwg / 8;
  const int q = ceil_div(total, 8);
  const int lo = xcd * q, hi = min(total, lo + q);
  const int gm = max(L.group_m, 1);
  for (int logical = lo + slot; logical < hi; logical += per_xcd_wg) {
    const int pstart = logical / (gm * nblocks) * gm;   // first m-tile of the panel
    const int pm = min(gm, tiles - pstart);              // the last panel may be short
    const int within = logical - pstart * nblocks;
    const int nblock = within / pm;
    const int tile = pstart + within % pm;
    int g, row0, nrows, out0;
    if (!locate_tile_lds(a, offs, tile, BIG_TILE_ROWS, L.min_rows, L.max_rows, g, row0, nrows, out0)) break;
    g = __builtin_amdgcn_readfirstlane(g);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    out0 = __builtin_amdgcn_readfirstlane(out0);
    big_tile<EPI>(a, lds0, lds1, lds2, lds3, g, row0, nrows, out0, nblock);
  }
}

bool gemm_big_fits(int N, int K, GemmEpi epi) {
  return K % (4 * BIG_BK) == 0 && N % (epi == EPI_SWIGLU ? 128 : 256) == 0;
}

hipError_t launch_gemm_big(const GemmArgs& a, const LdsArgs& L, GemmEpi epi, hipStream_t stream, KernelEvents ev) {
  if (a.offsets && (a.n_groups < 1 || a.n_groups > TILE_MAX_GROUPS)) return hipErrorInvalidValue;
  if (!gemm_big_fits(a.N, a.K, epi) || L.splits > 1) return hipErrorInvalidValue;
  if (a.tiles_y <= 0) return record_events(ev.start, ev.stop, stream);
  const long bound = long(a.N / (epi == EPI_SWIGLU ? 128 : 256)) * a.tiles_y;
  const int nwg = int(std::max(8L, std::min(bound, long(L.max_wgs)) / 8 * 8));
  if (epi == EPI_SWIGLU)
    return launch_timed((gemm_big_kernel<EPI_SWIGLU>), dim3(nwg), dim3(WG_THREADS), stream, ev.start, ev.stop, a, L);
  return launch_timed((gemm_big_kernel<EPI_SUM>), dim3(nwg), dim3(WG_THREADS), stream, ev.start, ev.stop, a, L);
}

}  // namespace moe
