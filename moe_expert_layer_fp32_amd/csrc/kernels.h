// Host-side launch interface of the gfx950 kernels (one translation unit per
// kernel family; the C ABI in api.cpp drives them).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------------------
// Grouped-row matrix-core product (gemm.hip).
//
// out[row][col] = sum_k B[brow(row)][k] * W_g[k][col] for the rows of each
// group g, with W_g packed as fragments [N/16][K/KF][S][64 lanes][BPL bytes].
// Groups: either one dense group of `dense_rows` rows, or the resident
// experts g = 0..n_groups-1 whose rows are the sorted rows
// [offsets[first+g], offsets[first+g+1]) (written compacted at
// row - offsets[first]). The B row of a sorted row is its token
// sorted_slot[row] / k (gather) or its compacted index.
// ---------------------------------------------------------------------------
enum GemmElem : int { ELEM_F32 = 0, ELEM_BF16 = 1, ELEM_I8 = 2 };
enum GemmEpi : int {
  EPI_SWIGLU = 0,  // S = 2 (W1, W3): out = silu(a) * b
  EPI_SUM = 1,     // S planes accumulated: out = acc (+ bias)
};

struct GemmArgs {
  const uint8_t* A;          // packed weights
  size_t a_group_stride;     // bytes between groups
  int K, N;                  // reduction length, output columns (multiple of 16)
  const uint8_t* B;          // activation rows
  size_t ldb;                // bytes between B rows
  const float* b_scale;      // int8: scale of each B row (indexed like B rows)
  const float* a_scale0;     // int8: per-column scale of plane 0, [G][a_scale_stride]
  const float* a_scale1;     // int8: per-column scale of plane 1 (SwiGLU)
  int a_scale_stride;
  const int* offsets;        // grouped rows when non-null
  int first, n_groups;
  int dense_rows;            // rows of the single dense group (offsets == null)
  const int* sorted_slot;    // gather B rows by token when non-null
  int k;
  uint8_t* out;              // output rows
  size_t ldo;                // bytes between output rows
  int out_bf16;              // 1: bf16 out, 0: fp32 out
  const float* bias;         // EPI_SUM: + bias[col] for col < n_valid
  int n_valid;
  int tiles_y;               // m-tile slots in the grid
  int dense_tile_rows;       // dense group: rows per m-tile (16..128, multiple of 16)
  int max_group_rows;        // grouped rows: only groups with at most this many rows (0: all)
  int ksplit;                // streaming kernel: wavefronts sharing a column tile (1, 2 or 4)
};

// Timing events a launcher attaches to its first / last kernel: the runtime
// stamps them when that kernel starts / ends (hipExtLaunchKernel), so their
// elapsed time is the kernels' own duration, with no marker between kernels.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_gemm(const GemmArgs& a, GemmElem elem, int planes, GemmEpi epi,
                       hipStream_t stream, KernelEvents ev = {});

// Upper bound on the m-tiles of grouped rows (R rows over G groups), and the
// m-tiles of one dense group of `rows` rows.
int gemm_tiles_bound(int max_rows, int n_groups);
// Dense group: rows per m-tile of the streaming kernel (stored in
// *tile_rows) and the number of m-tiles.
int gemm_tiles_dense(int rows, int n_cols, int* tile_rows);
// Reduction split of the streaming kernel for `col_tiles` 16-column tiles
// (summed over groups) and a reduction of KT steps.
int gemm_stream_ksplit(long col_tiles, int KT);

// ---------------------------------------------------------------------------
// Tiled matrix-core GEMM with LDS-staged rows (gemm_lds.hip) for groups or
// dense problems with many rows; same GemmArgs (grouped rows / dense rows,
// packed weights, epilogues). Requires N % (32 * wave_features / 32) == 0 and
// K % lds_chunk_elems(elem) == 0.
// ---------------------------------------------------------------------------
struct LdsArgs {
  int tile_rows;       // rows per m-tile: 64 or 128
  int wave_features;   // output features per wavefront: 32 or 64
  int min_rows, max_rows;   // grouped rows: groups with a row count in [min, max]
  int splits;          // reduction split (1: epilogue in the GEMM kernel)
  void* partial;       // splits > 1: [splits][part_rows][acc planes * N] fp32 / int32
  int part_rows;
  int max_wgs;         // cap of the persistent grid (workgroups per split)
  int fold_reduce;     // splits > 1: launch no reduce pass; the consumer adds
                       // the partial sums in split order (router -> gate)
  int group_m;         // tile order: <= 1 m-tile fastest; else panels of
                       // group_m m-tiles, column block next inside a panel
  int wave_split;      // 0 or 1: the wavefronts of a workgroup own 4 * NF
                       // features; 4: they split the reduction of NF features
                       // into 4 ranges, added in range order inside the
                       // workgroup (32-row tiles, splits == 1, bf16)
};
hipError_t launch_gemm_lds(const GemmArgs& a, const LdsArgs& L, GemmElem elem, int planes, GemmEpi epi,
                           hipStream_t stream, KernelEvents ev = {});
int lds_chunk_elems(GemmElem elem);

// Large-tile bf16 GEMM (gemm_big.hip): 256 rows x 256 weight columns per
// tile, both operands staged in LDS by direct-to-LDS loads, one workgroup per
// compute unit. Same GemmArgs (grouped or dense rows) and LdsArgs (row-count
// class, persistent grid cap, panel order); no reduction split, no scales or
// bias (bf16 SwiGLU gate/up or one-plane products). Fits when K % 64 == 0 and
// N % 128 (SwiGLU) or N % 256 (one plane) == 0. tiles_y: m-tiles of 256 rows.
constexpr int BIG_TILE_ROWS = 256;
bool gemm_big_fits(int N, int K, GemmEpi epi);
hipError_t launch_gemm_big(const GemmArgs& a, const LdsArgs& L, GemmEpi epi, hipStream_t stream,
                           KernelEvents ev = {});
// Reduce pass of a split product: partial sums added in split order, then
// the product's epilogue (stop: optional timing event stamped at its end).
hipError_t launch_gemm_reduce(const GemmArgs& a, const LdsArgs& L, GemmElem elem, GemmEpi epi, hipStream_t stream,
                              hipEvent_t stop);

// ---------------------------------------------------------------------------
// Gating + top-k (route.hip)
// ---------------------------------------------------------------------------
struct GateArgs {
  const float* z;   // [T][ldz] logits, bias included (partial == nullptr)
  int ldz;
  int T, E, k, gate, n_group, topk_group, per_group_k, renorm;
  float route_scale;
  int* topk_idx;
  float* topk_w;
  const float* partial;   // or: [splits][T][ldz] split-K partial sums of x W_r,
  int splits;             //   added in split order, then
  const float* bias;      //   the logit bias [E] (may be null)
};
hipError_t launch_gate(const GateArgs& a, hipStream_t stream);

// Router product for few tokens (route.hip): z[T][e_pad] = x W_r + bias with
// 16 tokens x 16 experts per workgroup and the reduction split over its
// wavefronts; no split-K partials, no reduce pass.
struct RouterArgs {
  const uint8_t* w;   // packed router fragments (1 fp32 plane or 3 bf16 planes)
  const uint8_t* x;   // [T][K] fp32 (1 plane) or bf16 (3 planes)
  int T, K, E, e_pad;
  const float* bias;  // [E] or null
  float* z;           // [T][e_pad]
};
hipError_t launch_router_small(const RouterArgs& a, bool f32, hipStream_t stream);

// ---------------------------------------------------------------------------
// Stable counting sort of slots by expert (permute.hip)
// ---------------------------------------------------------------------------
// Up to PERMUTE_ONE_WG slots the permutation runs on one workgroup with no
// workspace; more use permute_chunks(n) workgroups of PERMUTE_CHUNK slots
// and a chunk_hist workspace of permute_chunks(n) * E ints.
constexpr int PERMUTE_ONE_WG = 8192;
constexpr int PERMUTE_CHUNK = 2048;
int permute_chunks(int n_slots);
hipError_t launch_permute(const int* topk_idx, int n_slots, int E, int* counts, int* offsets,
                          int* sorted_slot, int* slot_pos, int* chunk_hist, hipStream_t stream);

// ---------------------------------------------------------------------------
// Per-row int8 quantisation (quant.hip). rows = fixed count, or (when
// offsets != null) offsets[first + n_groups] - offsets[first] rows.
// in_bf16: 1 for bf16 input rows, 0 for fp32.
// ---------------------------------------------------------------------------
hipError_t launch_quant_rows(const void* in, int in_bf16, int cols, int max_rows,
                             const int* offsets, int first, int n_groups, int8_t* q, float* s,
                             hipStream_t stream);

// ---------------------------------------------------------------------------
// Combine (combine.hip)
// ---------------------------------------------------------------------------
struct CombineArgs {
  const void* x;             // [T][d] fp32 or bf16
  int x_bf16;
  const void* rows;          // compacted routed rows [R][d]
  const void* shared_rows;   // [T][d] or null
  int rows_bf16;             // rows and shared_rows are bf16 (else fp32)
  const int* topk_idx;
  const float* topk_w;
  const int* offsets;        // [E+1]
  const int* slot_pos;       // [T*k]
  int T, d, k, ffn_begin, n_ffn, zero_begin, n_zero;
  void* y;                   // [T][d] fp32 or bf16 (same type as x)
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Weight packing (pack.hip)
// ---------------------------------------------------------------------------
// Expert weights [G][K][N] (element bytes es) from `planes` sources into
// fragments [G][N/16][K/KF][planes][64][BPL].
hipError_t launch_pack_experts(const void* src0, const void* src1, int planes, GemmElem elem,
                               int G, int K, int N, void* dst, hipStream_t stream);
// Router W_r [K][E] fp32 into fragments of ceil(E/16)*16 columns: one fp32
// plane (elem = ELEM_F32) or three exact bf16 planes (elem = ELEM_BF16).
hipError_t launch_pack_router(const float* wr, GemmElem elem, int K, int E, void* dst,
                              hipStream_t stream);

}  // namespace moe
