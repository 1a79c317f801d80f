// C ABI of libmoe.so: argument validation, workspace layout and the order of
// kernel launches for each entry point (declared and documented in moe.h).
// Nothing here allocates, synchronises or copies to the host; every launch
// goes on the caller's stream.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <climits>

#include "kernels.h"
#include "moe.h"

using namespace moe;

#define HIP_TRY(expr)                             \
  do {                                            \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_E = 256;
constexpr int MAX_K = 16;
constexpr int64_t MAX_SLOTS = int64_t(1) << 20;

size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }

int e_pad(const moe_desc* d) { return (d->E + 15) / 16 * 16; }
int x_bytes(const moe_desc* d) { return d->dtype == MOE_DTYPE_F32 ? 4 : 2; }
int w_bytes(const moe_desc* d) { return d->dtype == MOE_DTYPE_F32 ? 4 : (d->dtype == MOE_DTYPE_BF16 ? 2 : 1); }
// Element size of the SwiGLU output h kept between the two projections:
// bf16 for the bf16 layer (the down projection consumes bf16 operands), fp32
// otherwise (fp32 layer; W8A8 requantises it per row).
int h_bytes(const moe_desc* d) { return d->dtype == MOE_DTYPE_BF16 ? 2 : 4; }
bool w8a8(const moe_desc* d) { return d->dtype == MOE_DTYPE_W8A8; }
// Capacity for routed rows on resident experts: T*k, the most the routing
// tables can hold whatever ids they carry.
int r_max(const moe_desc* d) { return d->n_ffn > 0 ? d->T * d->k : 0; }

GemmElem weight_elem(const moe_desc* d) {
  return d->dtype == MOE_DTYPE_F32 ? ELEM_F32 : (d->dtype == MOE_DTYPE_BF16 ? ELEM_BF16 : ELEM_I8);
}
int weight_kf(const moe_desc* d) { return d->dtype == MOE_DTYPE_F32 ? 4 : (d->dtype == MOE_DTYPE_BF16 ? 32 : 64); }
int frag_bytes_of(GemmElem e) { return e == ELEM_F32 ? 64 * 4 : 64 * 16; }
int kf_of(GemmElem e) { return e == ELEM_F32 ? 4 : (e == ELEM_BF16 ? 32 : 64); }
GemmElem router_elem(const moe_desc* d) { return d->dtype == MOE_DTYPE_F32 ? ELEM_F32 : ELEM_BF16; }
// Bytes per element of the expert outputs moe_layer keeps in its workspace:
// bf16 layers keep them in bf16 (the sum over experts still runs in fp32),
// fp32 and W8A8 layers in fp32 (W8A8 rows already carry the int8 error of
// x and h; a further bf16 rounding would add to it).
size_t layer_row_bytes(const moe_desc* d) { return d->dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------
// Which kernel runs each product (decided on the host from shapes only; the
// per-expert part of the choice happens on the device).
//  - Routed experts: the tiled LDS GEMM (see run_routed) whenever the shape
//    tiles, else weight streaming (gemm_rows_kernel).
//  - Dense products (router, shared expert): the tiled GEMM unless M is tiny
//    or the shape does not tile; split-K when the tiles alone would give
//    fewer than TARGET_WGS workgroups.
// ---------------------------------------------------------------------------
constexpr int PREFILL_T = 1024;
constexpr int TARGET_WGS = 256;
constexpr int MAX_DENSE_SPLITS = 32;  // split-K of dense products (partials added in split order)
constexpr int PERSISTENT_WGS = 512;   // grid cap of the tiled kernel (it loops over tiles)
// Tile order of dense products with 128-row tiles: panels of DENSE_GROUP_M
// m-tiles (LdsArgs::group_m). Measured on the prefill shared expert (8192
// rows, one stream): gate/up 474 -> 457 us, down 296 -> 274 us.
constexpr int DENSE_GROUP_M = 8;
// Tile choice defaults (moe_tuning's prefill_tokens, stream_max_rows,
// big_min_rows, dense_big_rows; see moe.h). 256-row tiles: panels of 4
// m-tiles for dense products (4 x 8 tiles of an XCD's 32 compute units run
// together), panels of 2 m-tiles for routed experts (their gathered rows are
// then fetched by fewer XCDs; measured on the prefill workload, two streams:
// 1.595 -> 1.576 ms per call against m-tile fastest, 1.583 with panels of 4).
constexpr int STREAM_MAX_ROWS = 64;
constexpr int BIG_MIN_ROWS = 256;
constexpr int DENSE_BIG_ROWS = 2048;
constexpr int BIG_GROUP_M = 4;
constexpr int BIG_ROUTED_GROUP_M = 2;
constexpr int BIG_WGS = 256;          // one 256-row workgroup per compute unit (128 KiB of LDS)

struct TilePolicy {
  int prefill_tokens = PREFILL_T;
  int stream_max_rows = STREAM_MAX_ROWS;
  int big_min_rows = BIG_MIN_ROWS;
  int dense_big_rows = DENSE_BIG_ROWS;
  // below the prefill threshold: experts with at most this many rows go to
  // the 32-row weight-streaming kernel (0: none; only a caller's theta)
  int decode_stream_rows = 0;
  // below the prefill threshold: the routed experts' tile height (64 or 32)
  int decode_tile_rows = 64;
};
TilePolicy policy_of(const moe_tuning& t) {
  TilePolicy p;
  if (t.prefill_tokens > 0) p.prefill_tokens = t.prefill_tokens;
  if (t.stream_max_rows > 0) p.stream_max_rows = p.decode_stream_rows = t.stream_max_rows;
  if (t.big_min_rows > 0) p.big_min_rows = t.big_min_rows;
  if (t.dense_big_rows > 0) p.dense_big_rows = t.dense_big_rows;
  if (t.decode_tile_rows > 0) p.decode_tile_rows = t.decode_tile_rows;
  return p;
}

struct DensePlan {
  bool lds;
  bool big = false;   // 256-row tiles (gemm_big): no reduction split
  LdsArgs L;
  int tiles_y;
  int tile_rows;
  size_t partial_bytes;
};

// cap > 0: at most that many workgroups (a caller's launch limit); it only
// lowers the split target and the persistent grid, so the plan never needs
// more split-K workspace than the uncapped one. With a policy, bf16 products
// of planes 1 (sum) or 2 (SwiGLU) and at least dense_big_rows rows take the
// 256-row tiles, which need no workspace; without one (workspace sizing) the
// plan is the 64/128-row one, whose split-K partial sums bound every plan's.
DensePlan plan_dense(int M, int N, int K, GemmElem el, int nacc, int cap = 0, const TilePolicy* pol = nullptr,
                     int planes = 0) {
  const int target = cap > 0 ? std::min(cap, TARGET_WGS) : TARGET_WGS;
  DensePlan p{};
  const GemmEpi epi = nacc == 2 ? EPI_SWIGLU : EPI_SUM;
  if (pol && el == ELEM_BF16 && planes == nacc && M >= pol->dense_big_rows && gemm_big_fits(N, K, epi)) {
    p.lds = true;
    p.big = true;
    LdsArgs& L = p.L;
    L.tile_rows = BIG_TILE_ROWS;
    L.splits = 1;
    L.min_rows = 0;
    L.max_rows = INT32_MAX;
    L.part_rows = M;
    L.max_wgs = cap > 0 ? std::min(cap, BIG_WGS) : BIG_WGS;
    L.group_m = BIG_GROUP_M;
    p.tiles_y = ceil_div(M, BIG_TILE_ROWS);
    return p;
  }
  const int ch = lds_chunk_elems(el);
  if (M <= 64 || K % ch != 0 || N % 32 != 0) {
    p.lds = false;
    p.tiles_y = gemm_tiles_dense(M, N, &p.tile_rows);
    return p;
  }
  p.lds = true;
  LdsArgs& L = p.L;
  // 128-row tiles from 1024 rows: below, 64-row tiles (more m-tiles, fewer
  // split-K slices) measured faster (DeepSeek-style decode share, 512 rows:
  // shared gate/up 47 -> 44 us, down 36 -> 30 us, router 19 -> 15 us)
  L.tile_rows = M >= 1024 ? 128 : 64;
  const int mt = ceil_div(M, L.tile_rows);
  L.wave_features = (nacc == 1 && N % 256 == 0 && (N / 256) * mt >= target) ? 64 : 32;
  const int wgs = ceil_div(N, 4 * L.wave_features) * mt;
  const int kc = K / ch;
  int splits = 1;
  if (wgs < target) splits = std::max(1, std::min({ceil_div(target, wgs), kc / 2, MAX_DENSE_SPLITS}));
  L.splits = splits;
  L.min_rows = 0;
  L.max_rows = INT32_MAX;
  L.part_rows = M;
  L.max_wgs = cap > 0 ? std::min(cap, PERSISTENT_WGS) : PERSISTENT_WGS;
  L.group_m = L.tile_rows >= 128 ? DENSE_GROUP_M : 1;
  p.tiles_y = mt;
  p.partial_bytes = splits > 1 ? size_t(splits) * M * nacc * N * 4 : 0;
  return p;
}

bool routed_tiled(const moe_desc* d, int N, int K) {
  return K % lds_chunk_elems(weight_elem(d)) == 0 && N % 32 == 0;
}

// Decode-sized routed products with too few tiles to fill the device (e.g.
// 8 resident experts: 8 x 16 column blocks of 128) split the reduction over
// several workgroups per tile, up to SPLIT_WGS workgroups in all; the partial
// sums are added in split order by the reduce pass. 1 = no split.
constexpr int SPLIT_WGS = 512;
// A split of exactly this many slices on 32-row bf16 tiles runs inside one
// workgroup, one slice per wavefront (LdsArgs::wave_split).
constexpr int WAVE_SPLIT = 4;
int routed_splits(const moe_desc* d, int N, int K) {
  if (d->T >= PREFILL_T || !routed_tiled(d, N, K)) return 1;
  const long wgs = long(d->n_ffn) * ceil_div(N, 128);
  if (wgs >= TARGET_WGS) return 1;
  const int kc = K / lds_chunk_elems(weight_elem(d));
  return std::max(1, std::min({int(ceil_div(SPLIT_WGS, int(wgs))), kc / 2, 8}));
}
// Split-K partial sums of the routed products (the larger of the two).
size_t routed_partial_bytes(const moe_desc* d) {
  if (d->n_ffn == 0) return 0;
  size_t b = 0;
  const int s1 = routed_splits(d, d->inter, d->d), s2 = routed_splits(d, d->d, d->inter);
  if (s1 > 1) b = std::max(b, size_t(s1) * r_max(d) * 2 * d->inter * 4);
  if (s2 > 1) b = std::max(b, size_t(s2) * r_max(d) * 1 * d->d * 4);
  return b;
}

// Split-K partial sums needed by any dense product of this layer.
size_t dense_partial_bytes(const moe_desc* d, bool route, bool shared) {
  size_t b = 0;
  if (route) b = std::max(b, plan_dense(d->T, e_pad(d), d->d, router_elem(d), 1).partial_bytes);
  if (shared && d->shared_inter > 0) {
    b = std::max(b, plan_dense(d->T, d->shared_inter, d->d, weight_elem(d), 2).partial_bytes);
    b = std::max(b, plan_dense(d->T, d->d, d->shared_inter, weight_elem(d), 1).partial_bytes);
  }
  return b;
}

moe_status validate(const moe_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->d <= 0 || d->E < 1 || d->k < 1 || d->k > d->E) return MOE_ERR_INVALID_ARG;
  if (d->gate != MOE_GATE_SOFTMAX && d->gate != MOE_GATE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (d->dtype != MOE_DTYPE_F32 && d->dtype != MOE_DTYPE_BF16 && d->dtype != MOE_DTYPE_W8A8)
    return MOE_ERR_INVALID_ARG;
  if (d->n_group < 1 || d->E % d->n_group != 0) return MOE_ERR_INVALID_ARG;
  if (d->topk_group < 0 || d->per_group_k < 0) return MOE_ERR_INVALID_ARG;
  if (d->topk_group > 0 && d->per_group_k > 0) return MOE_ERR_INVALID_ARG;
  const int gsize = d->E / d->n_group;
  if (d->topk_group > 0) {
    if (d->topk_group > d->n_group || gsize < 2 || d->k > d->topk_group * gsize) return MOE_ERR_INVALID_ARG;
  }
  if (d->per_group_k > 0) {
    if (d->k != d->n_group * d->per_group_k || d->per_group_k > gsize) return MOE_ERR_INVALID_ARG;
  }
  if (d->ffn_begin < 0 || d->n_ffn < 0 || d->ffn_begin + d->n_ffn > d->E) return MOE_ERR_INVALID_ARG;
  if (d->zero_begin < 0 || d->n_zero < 0 || d->zero_begin + d->n_zero > d->E) return MOE_ERR_INVALID_ARG;
  if (d->n_ffn > 0 && d->n_zero > 0 && d->ffn_begin < d->zero_begin + d->n_zero &&
      d->zero_begin < d->ffn_begin + d->n_ffn)
    return MOE_ERR_INVALID_ARG;
  if (d->n_ffn > 0 && d->inter <= 0) return MOE_ERR_INVALID_ARG;
  if (d->shared_inter < 0 || d->inter < 0) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(d->route_scale)) return MOE_ERR_INVALID_ARG;
  // Built shapes.
  if (d->E > MAX_E || d->k > MAX_K) return MOE_ERR_UNSUPPORTED;
  if (int64_t(d->T) * d->k > MAX_SLOTS) return MOE_ERR_UNSUPPORTED;
  if (d->d % 64 != 0 || d->inter % 64 != 0 || d->shared_inter % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (d->topk_group > 0 && d->n_group > 64) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// workspace layouts
// ---------------------------------------------------------------------------
struct Carve {
  uint8_t* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<uint8_t*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += align_up(bytes);
    return p;
  }
};

struct RouteWs { float* z; void* partial; };
RouteWs carve_route(Carve& c, const moe_desc* d) {
  RouteWs r;
  r.z = static_cast<float*>(c.take(size_t(d->T) * e_pad(d) * 4));
  r.partial = c.take(dense_partial_bytes(d, true, false));
  return r;
}

struct FfnWs {
  int8_t* qx; float* sx;      // W8A8 activation codes (shared by routed and shared FFN)
  uint8_t* h; int8_t* qh; float* sh;
  void* partial;              // split-K partial sums of dense products
};
void carve_qx(Carve& c, const moe_desc* d, FfnWs& f) {
  f.qx = nullptr; f.sx = nullptr;
  if (w8a8(d)) {
    f.qx = static_cast<int8_t*>(c.take(size_t(d->T) * d->d));
    f.sx = static_cast<float*>(c.take(size_t(d->T) * 4));
  }
}
void carve_h(Carve& c, const moe_desc* d, int rows, int inter, FfnWs& f) {
  f.h = static_cast<uint8_t*>(c.take(size_t(rows) * inter * h_bytes(d)));
  f.qh = nullptr; f.sh = nullptr;
  if (w8a8(d)) {
    f.qh = static_cast<int8_t*>(c.take(size_t(rows) * inter));
    f.sh = static_cast<float*>(c.take(size_t(rows) * 4));
  }
  f.partial = nullptr;
}

size_t permute_ws_bytes(const moe_desc* d) {
  const int chunks = permute_chunks(d->T * d->k);
  return chunks > 1 ? size_t(chunks) * d->E * 4 : 0;
}

struct LayerWs {
  RouteWs route;
  int32_t *idx, *counts, *offsets, *sorted_slot, *slot_pos;
  int32_t* chunk_hist;
  float* w;
  FfnWs routed, shared;
  void *rows, *shared_rows;   // expert outputs: bf16 in the bf16 layer, else fp32 (layer_row_bytes)
};
LayerWs carve_layer(Carve& c, const moe_desc* d) {
  LayerWs L{};
  const size_t slots = size_t(d->T) * d->k;
  L.route = carve_route(c, d);
  L.idx = static_cast<int32_t*>(c.take(slots * 4));
  L.w = static_cast<float*>(c.take(slots * 4));
  L.counts = static_cast<int32_t*>(c.take(size_t(d->E) * 4));
  L.offsets = static_cast<int32_t*>(c.take(size_t(d->E + 1) * 4));
  L.sorted_slot = static_cast<int32_t*>(c.take(slots * 4));
  L.slot_pos = static_cast<int32_t*>(c.take(slots * 4));
  L.chunk_hist = static_cast<int32_t*>(c.take(permute_ws_bytes(d)));
  carve_qx(c, d, L.routed);
  L.shared.qx = L.routed.qx;
  L.shared.sx = L.routed.sx;
  carve_h(c, d, r_max(d), d->inter, L.routed);
  L.routed.partial = c.take(routed_partial_bytes(d));
  L.rows = c.take(size_t(r_max(d)) * d->d * layer_row_bytes(d));
  if (d->shared_inter > 0) {
    carve_h(c, d, d->T, d->shared_inter, L.shared);
    L.shared.partial = c.take(dense_partial_bytes(d, false, true));
    L.shared_rows = c.take(size_t(d->T) * d->d * layer_row_bytes(d));
  } else {
    L.shared_rows = nullptr;
  }
  return L;
}

// ---------------------------------------------------------------------------
// stages
// ---------------------------------------------------------------------------
// Launch one dense product with its plan (tiled LDS GEMM or streaming).
moe_status run_dense(GemmArgs g, int M, GemmElem el, int planes, GemmEpi epi, void* partial, hipStream_t s,
                     KernelEvents ev, int cap, const TilePolicy& pol) {
  const int nacc = epi == EPI_SWIGLU ? 2 : 1;
  const DensePlan p = plan_dense(M, g.N, g.K, el, nacc, cap, &pol, planes);
  if (p.partial_bytes > plan_dense(M, g.N, g.K, el, nacc).partial_bytes) return MOE_ERR_INVALID_ARG;
  g.offsets = nullptr;
  g.dense_rows = M;
  g.tiles_y = p.tiles_y;
  if (p.big) {
    HIP_TRY(launch_gemm_big(g, p.L, epi, s, ev));
    return MOE_OK;
  }
  if (!p.lds) {
    g.dense_tile_rows = p.tile_rows;
    g.ksplit = gemm_stream_ksplit(g.N / 16, g.K / kf_of(el));
    HIP_TRY(launch_gemm(g, el, planes, epi, s, ev));
    return MOE_OK;
  }
  LdsArgs L = p.L;
  L.partial = partial;
  HIP_TRY(launch_gemm_lds(g, L, el, planes, epi, s, ev));
  return MOE_OK;
}

// Launch one routed product. Shapes that tile go to the tiled kernel: at
// decode sizes one launch with 64-row tiles (an expert with more rows takes
// several); from PREFILL_T tokens up, experts with at most 64 rows use
// 64-row tiles and bigger ones 128-row tiles (each weight fragment reused by
// more rows). Few experts with long rows (fewer than TARGET_WGS tiled
// workgroups, e.g. 8 resident experts of d 7168) split the reduction over
// workgroups (routed_splits); shapes that do not tile stream through
// gemm_rows_kernel, whose wavefronts split the reduction.
// cap > 0: at most that many workgroups in all (split-K slices included).
int capped_wgs(int cap, int splits) { return cap > 0 ? std::min(PERSISTENT_WGS, std::max(1, cap / splits)) : PERSISTENT_WGS; }

// Which experts a routed product covers. From PREFILL_T tokens up the two
// launches (experts with at most 64 rows, experts with more) can be issued
// apart, on different streams; below, only PART_ALL exists.
enum RoutedPart { PART_NONE = 0, PART_SMALL = 1, PART_LARGE = 2, PART_ALL = 3 };

// Whether moe_layer may place the two prefill launches of a routed product on
// different streams: bf16 / fp32 (the W8A8 row quantisation between the
// products covers every expert at once) and both products tiled unsplit.
bool routed_parts_apart(const moe_desc* d, const TilePolicy& pol) {
  return d->T >= pol.prefill_tokens && !w8a8(d) && d->n_ffn > 0 && routed_tiled(d, d->inter, d->d) &&
         routed_tiled(d, d->d, d->inter);
}

moe_status run_routed(GemmArgs g, const moe_desc* d, GemmElem el, int planes, GemmEpi epi, void* partial,
                      hipStream_t s, KernelEvents ev, int cap, int part, const TilePolicy& pol) {
  if (part == PART_NONE) return MOE_OK;
  const bool prefill = d->T >= pol.prefill_tokens;
  // the reduction is split only at the default decode sizes (the workspace
  // holds the partial sums for exactly those)
  const int splits = prefill ? 1 : routed_splits(d, g.N, g.K);
  if (!prefill && pol.decode_stream_rows > 0 && routed_tiled(d, g.N, g.K)) {
    // Decode with a caller's theta: experts with at most theta rows stream
    // their weights through the 32-row kernel (its matrix-core work covers
    // only the row blocks an expert has), the others take the 64-row tiles
    // (reduction split as without theta). Both launches pick their experts
    // on the device from the offsets.
    GemmArgs gs = g;
    gs.max_group_rows = pol.decode_stream_rows;
    gs.tiles_y = gemm_tiles_bound(r_max(d), g.n_groups);
    gs.ksplit = gemm_stream_ksplit(long(g.n_groups) * (g.N / 16), g.K / kf_of(el));
    HIP_TRY(launch_gemm(gs, el, planes, epi, s, KernelEvents{ev.start, nullptr}));
    LdsArgs L{};
    L.wave_features = 32;
    L.splits = splits;
    L.partial = partial;
    L.part_rows = r_max(d);
    L.max_wgs = capped_wgs(cap, splits);
    L.tile_rows = pol.decode_tile_rows;
    L.min_rows = pol.decode_stream_rows + 1;
    L.max_rows = INT32_MAX;
    g.tiles_y = ceil_div(r_max(d), L.tile_rows) + g.n_groups;
    HIP_TRY(launch_gemm_lds(g, L, el, planes, epi, s, KernelEvents{nullptr, ev.stop}));
    return MOE_OK;
  }
  if (splits > 1) {
    LdsArgs L{};
    L.wave_features = 32;
    L.splits = splits;
    L.partial = partial;
    L.part_rows = r_max(d);
    L.max_wgs = capped_wgs(cap, splits);
    L.tile_rows = pol.decode_tile_rows;
    L.min_rows = 1;
    L.max_rows = INT32_MAX;
    g.tiles_y = ceil_div(r_max(d), L.tile_rows) + g.n_groups;
    if (splits == WAVE_SPLIT && L.tile_rows == 32 && el == ELEM_BF16 && planes <= 2 &&
        (g.K / lds_chunk_elems(el)) % WAVE_SPLIT == 0) {
      // The same four reduction ranges, one per wavefront of a workgroup that
      // owns 32 features, added inside it in range order: the sums of the
      // split-K reduce pass, bit for bit, without its launch or the partial
      // sums' round trip through memory.
      L.splits = 1;
      L.wave_split = WAVE_SPLIT;
      L.partial = nullptr;
      L.max_wgs = capped_wgs(cap, 1);
    }
    HIP_TRY(launch_gemm_lds(g, L, el, planes, epi, s, ev));
    return MOE_OK;
  }
  const long tiled_wgs = long(g.n_groups) * ceil_div(g.N, 128);
  if (routed_tiled(d, g.N, g.K) && (tiled_wgs >= TARGET_WGS || prefill)) {
    LdsArgs L{};
    L.wave_features = 32;
    L.splits = 1;
    L.part_rows = r_max(d);
    L.max_wgs = capped_wgs(cap, 1);
    L.tile_rows = prefill ? 64 : pol.decode_tile_rows;
    L.min_rows = 1;
    L.max_rows = INT32_MAX;
    g.tiles_y = ceil_div(r_max(d), L.tile_rows) + g.n_groups;
    if (!prefill) {
      HIP_TRY(launch_gemm_lds(g, L, el, planes, epi, s, ev));
      return MOE_OK;
    }
    // Prefill: experts classed by row count (the per-expert mode switch;
    // which expert is in which class is decided on the device from the
    // offsets). Streaming class: at most theta rows, 64-row tiles; middle
    // class: 128-row tiles; large class: 256-row tiles (bf16 shapes that fit
    // them). PART_SMALL is the streaming class, PART_LARGE the other two.
    const int theta = pol.stream_max_rows;
    const bool big = el == ELEM_BF16 && planes == (epi == EPI_SWIGLU ? 2 : 1) && gemm_big_fits(g.N, g.K, epi) &&
                     pol.big_min_rows <= r_max(d);
    const int big_lo = big ? std::max(theta + 1, pol.big_min_rows) : INT32_MAX;
    const bool has_mid = theta + 1 < big_lo;
    // launches in order: [small], [mid], [big]; the events go on the first
    // and last launch made by this call
    const int n_launch = ((part & PART_SMALL) ? 1 : 0) + ((part & PART_LARGE) ? int(has_mid) + int(big) : 0);
    int k_launch = 0;
    auto events = [&]() {
      KernelEvents e{k_launch == 0 ? ev.start : nullptr, k_launch == n_launch - 1 ? ev.stop : nullptr};
      ++k_launch;
      return e;
    };
    if (part & PART_SMALL) {
      L.max_rows = theta;
      // with at most 64 rows an expert has one 64-row tile
      g.tiles_y = theta <= 64 ? g.n_groups : ceil_div(r_max(d), L.tile_rows) + g.n_groups;
      HIP_TRY(launch_gemm_lds(g, L, el, planes, epi, s, events()));
    }
    if (!(part & PART_LARGE)) return MOE_OK;
    if (has_mid) {
      // 128-row tiles, 64 features per wavefront for one-plane products
      // (twice the matrix-core work per weight fragment)
      L.tile_rows = 128;
      L.min_rows = theta + 1;
      L.max_rows = big_lo - 1;
      L.wave_features = planes == 1 && g.N % 256 == 0 ? 64 : 32;
      g.tiles_y = ceil_div(r_max(d), L.tile_rows) + g.n_groups;
      HIP_TRY(launch_gemm_lds(g, L, el, planes, epi, s, events()));
    }
    if (big) {
      LdsArgs B{};
      B.tile_rows = BIG_TILE_ROWS;
      B.splits = 1;
      B.min_rows = big_lo;
      B.max_rows = INT32_MAX;
      B.part_rows = r_max(d);
      B.max_wgs = cap > 0 ? std::min(cap, BIG_WGS) : BIG_WGS;
      B.group_m = BIG_ROUTED_GROUP_M;
      g.tiles_y = ceil_div(r_max(d), BIG_TILE_ROWS) + g.n_groups;
      HIP_TRY(launch_gemm_big(g, B, epi, s, events()));
    }
    return MOE_OK;
  }
  g.max_group_rows = 0;
  g.tiles_y = gemm_tiles_bound(r_max(d), g.n_groups);
  g.ksplit = gemm_stream_ksplit(long(g.n_groups) * (g.N / 16), g.K / kf_of(el));
  HIP_TRY(launch_gemm(g, el, planes, epi, s, ev));
  return MOE_OK;
}

// Router products small enough that every 16-token block may read the whole
// packed router (at most ROUTER_SMALL_BYTES of router reads in all, at most
// ROUTER_WG_BYTES per workgroup of 16 experts) go to the one-pass router
// kernel; larger ones to the GEMM kernels, whose split-K partial sums the
// gate kernel adds itself (no reduce pass).
constexpr size_t ROUTER_SMALL_BYTES = size_t(32) << 20;
constexpr size_t ROUTER_WG_BYTES = size_t(256) << 10;

bool router_small(const moe_desc* d) {
  const size_t per_k = d->dtype == MOE_DTYPE_F32 ? 4 : 6;   // one fp32 or three bf16 planes
  const size_t router_bytes = size_t(e_pad(d)) * d->d * per_k;
  return size_t(16) * d->d * per_k <= ROUTER_WG_BYTES &&
         size_t(ceil_div(d->T, 16)) * router_bytes <= ROUTER_SMALL_BYTES;
}

moe_status run_route(const moe_desc* d, const moe_weights* w, const void* x, int32_t* idx, float* tw,
                     const RouteWs& ws, hipStream_t s) {
  const bool f32 = d->dtype == MOE_DTYPE_F32;
  GateArgs ga{ws.z, e_pad(d), d->T, d->E, d->k, d->gate, d->n_group, d->topk_group, d->per_group_k,
              d->renorm, d->route_scale, idx, tw, nullptr, 0, nullptr};
  if (router_small(d)) {
    const RouterArgs ra{static_cast<const uint8_t*>(w->router), static_cast<const uint8_t*>(x), d->T, d->d, d->E,
                        e_pad(d), w->logit_bias, ws.z};
    HIP_TRY(launch_router_small(ra, f32, s));
    HIP_TRY(launch_gate(ga, s));
    return MOE_OK;
  }
  GemmArgs g{};
  g.A = static_cast<const uint8_t*>(w->router);
  g.a_group_stride = 0;
  g.K = d->d;
  g.N = e_pad(d);
  g.B = static_cast<const uint8_t*>(x);
  g.ldb = size_t(d->d) * x_bytes(d);
  g.dense_rows = d->T;
  g.out = reinterpret_cast<uint8_t*>(ws.z);
  g.ldo = size_t(e_pad(d)) * 4;
  g.out_bf16 = 0;
  g.bias = w->logit_bias;
  g.n_valid = d->E;
  const GemmElem el = f32 ? ELEM_F32 : ELEM_BF16;
  const DensePlan p = plan_dense(d->T, g.N, g.K, el, 1);
  g.offsets = nullptr;
  g.tiles_y = p.tiles_y;
  if (!p.lds) {
    g.dense_tile_rows = p.tile_rows;
    g.ksplit = gemm_stream_ksplit(g.N / 16, g.K / kf_of(el));
    HIP_TRY(launch_gemm(g, el, f32 ? 1 : 3, EPI_SUM, s));
  } else {
    LdsArgs L = p.L;
    L.partial = ws.partial;
    L.fold_reduce = 1;
    HIP_TRY(launch_gemm_lds(g, L, el, f32 ? 1 : 3, EPI_SUM, s));
    if (L.splits > 1) {
      ga.partial = static_cast<const float*>(ws.partial);
      ga.splits = L.splits;
      ga.bias = w->logit_bias;
    }
  }
  HIP_TRY(launch_gate(ga, s));
  return MOE_OK;
}

moe_status run_quant_x(const moe_desc* d, const void* x, FfnWs& f, hipStream_t s) {
  HIP_TRY(launch_quant_rows(x, 1, d->d, d->T, nullptr, 0, 0, f.qx, f.sx, s));
  return MOE_OK;
}

struct FfnPlan {
  const void* w13; const void* w2;
  const float *s1, *s3, *s2;
  int inter, groups;
  const int32_t* offsets;      // routed only
  int first;
  const int32_t* sorted_slot;  // routed only
  int rows_bound;              // routed: r_max; shared: T
  int cap1 = 0, cap2 = 0;      // workgroup caps of the two products (0: none)
  TilePolicy pol{};            // tile choice (library defaults unless tuned)
};
// The plan with the caller's launch limits for these products applied.
FfnPlan with_caps(FfnPlan p, int cap1, int cap2, const TilePolicy& pol) {
  p.cap1 = cap1;
  p.cap2 = cap2;
  p.pol = pol;
  return p;
}

// part1 / part2: which experts the gate/up and the down product cover
// (routed products from PREFILL_T tokens up; PART_NONE skips the product).
moe_status run_ffn(const moe_desc* d, const FfnPlan& p, const void* x, const FfnWs& f, void* rows, bool rows_bf16,
                   hipStream_t s, hipEvent_t e1b, hipEvent_t e1e, hipEvent_t e2b, hipEvent_t e2e,
                   int part1 = PART_ALL, int part2 = PART_ALL) {
  const GemmElem el = weight_elem(d);
  const int FB = frag_bytes_of(el);
  const int KF = weight_kf(d);
  const bool routed = p.offsets != nullptr;
  if (w8a8(d) && (part1 != PART_ALL || part2 != PART_ALL)) return MOE_ERR_UNSUPPORTED;
  // a dense (shared) product is whole or skipped
  if (!routed && ((part1 != PART_ALL && part1 != PART_NONE) || (part2 != PART_ALL && part2 != PART_NONE)))
    return MOE_ERR_UNSUPPORTED;
  moe_status st;

  GemmArgs g1{};
  g1.A = static_cast<const uint8_t*>(p.w13);
  g1.a_group_stride = size_t(p.inter / 16) * (d->d / KF) * 2 * FB;
  g1.K = d->d;
  g1.N = p.inter;
  g1.B = w8a8(d) ? reinterpret_cast<const uint8_t*>(f.qx) : static_cast<const uint8_t*>(x);
  g1.ldb = size_t(d->d) * (w8a8(d) ? 1 : x_bytes(d));
  g1.b_scale = w8a8(d) ? f.sx : nullptr;
  g1.a_scale0 = w8a8(d) ? p.s1 : nullptr;
  g1.a_scale1 = w8a8(d) ? p.s3 : nullptr;
  g1.a_scale_stride = routed ? p.inter : 0;
  g1.offsets = p.offsets;
  g1.first = p.first;
  g1.n_groups = p.groups;
  g1.dense_rows = d->T;
  g1.sorted_slot = p.sorted_slot;
  g1.k = d->k;
  g1.out = f.h;
  g1.ldo = size_t(p.inter) * h_bytes(d);
  g1.out_bf16 = d->dtype == MOE_DTYPE_BF16;
  const KernelEvents ev1{e1b, e1e}, ev2{e2b, e2e};
  if (part1 != PART_NONE) {
    st = routed ? run_routed(g1, d, el, 2, EPI_SWIGLU, f.partial, s, ev1, p.cap1, part1, p.pol)
                : run_dense(g1, d->T, el, 2, EPI_SWIGLU, f.partial, s, ev1, p.cap1, p.pol);
    if (st != MOE_OK) return st;
  }

  if (w8a8(d)) {
    HIP_TRY(launch_quant_rows(f.h, 0, p.inter, p.rows_bound, p.offsets, p.first, p.groups, f.qh, f.sh, s));
  }

  GemmArgs g2{};
  g2.A = static_cast<const uint8_t*>(p.w2);
  g2.a_group_stride = size_t(d->d / 16) * (p.inter / KF) * FB;
  g2.K = p.inter;
  g2.N = d->d;
  g2.B = w8a8(d) ? reinterpret_cast<const uint8_t*>(f.qh) : f.h;
  g2.ldb = size_t(p.inter) * (w8a8(d) ? 1 : h_bytes(d));
  g2.b_scale = w8a8(d) ? f.sh : nullptr;
  g2.a_scale0 = w8a8(d) ? p.s2 : nullptr;
  g2.a_scale_stride = routed ? d->d : 0;
  g2.offsets = p.offsets;
  g2.first = p.first;
  g2.n_groups = p.groups;
  g2.dense_rows = d->T;
  g2.sorted_slot = nullptr;
  g2.out = static_cast<uint8_t*>(rows);
  g2.ldo = size_t(d->d) * (rows_bf16 ? 2 : 4);
  g2.out_bf16 = rows_bf16;
  if (part2 != PART_NONE) {
    st = routed ? run_routed(g2, d, el, 1, EPI_SUM, f.partial, s, ev2, p.cap2, part2, p.pol)
                : run_dense(g2, d->T, el, 1, EPI_SUM, f.partial, s, ev2, p.cap2, p.pol);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

FfnPlan routed_plan(const moe_desc* d, const moe_weights* w, const int32_t* offsets, const int32_t* ss) {
  return FfnPlan{w->w13, w->w2, w->s1, w->s3, w->s2, d->inter, d->n_ffn, offsets, d->ffn_begin, ss, r_max(d)};
}
FfnPlan shared_plan(const moe_desc* d, const moe_weights* w) {
  return FfnPlan{w->sw13, w->sw2, w->ss1, w->ss3, w->ss2, d->shared_inter, 1, nullptr, 0, nullptr, d->T};
}

bool routed_weights_ok(const moe_desc* d, const moe_weights* w) {
  if (d->n_ffn == 0) return true;
  if (!w->w13 || !w->w2) return false;
  if (w8a8(d) && (!w->s1 || !w->s3 || !w->s2)) return false;
  return true;
}
bool shared_weights_ok(const moe_desc* d, const moe_weights* w) {
  if (d->shared_inter == 0) return true;
  if (!w->sw13 || !w->sw2) return false;
  if (w8a8(d) && (!w->ss1 || !w->ss3 || !w->ss2)) return false;
  return true;
}

CombineArgs combine_args(const moe_desc* d, const void* x, const void* rows, const void* shared_rows, bool rows_bf16,
                         const int32_t* idx, const float* tw, const int32_t* offsets, const int32_t* slot_pos,
                         void* y) {
  CombineArgs c{};
  c.x = x;
  c.x_bf16 = d->dtype != MOE_DTYPE_F32;
  c.rows = rows;
  c.shared_rows = shared_rows;
  c.rows_bf16 = rows_bf16;
  c.topk_idx = idx;
  c.topk_w = tw;
  c.offsets = offsets;
  c.slot_pos = slot_pos;
  c.T = d->T;
  c.d = d->d;
  c.k = d->k;
  c.ffn_begin = d->ffn_begin;
  c.n_ffn = d->n_ffn;
  c.zero_begin = d->zero_begin;
  c.n_zero = d->n_zero;
  c.y = y;
  return c;
}

size_t ws_bytes_of(const moe_desc* d, int op) {
  Carve c(nullptr);
  switch (op) {
    case MOE_OP_ROUTE_TOPK: carve_route(c, d); break;
    case MOE_OP_PERMUTE: c.take(permute_ws_bytes(d)); break;
    case MOE_OP_FFN_ROUTED: {
      FfnWs f{};
      carve_qx(c, d, f);
      carve_h(c, d, r_max(d), d->inter, f);
      c.take(routed_partial_bytes(d));
      break;
    }
    case MOE_OP_FFN_SHARED: {
      FfnWs f{};
      carve_qx(c, d, f);
      carve_h(c, d, d->T, d->shared_inter, f);
      c.take(dense_partial_bytes(d, false, true));
      break;
    }
    case MOE_OP_COMBINE: break;
    case MOE_OP_LAYER: carve_layer(c, d); break;
    default: return 0;
  }
  return c.used;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_desc* desc, int op) {
  if (validate(desc) != MOE_OK) return 0;
  return ws_bytes_of(desc, op);
}

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

size_t moe_packed_bytes(const moe_desc* d, int part) {
  if (validate(d) != MOE_OK) return 0;
  const size_t wb = size_t(w_bytes(d));
  switch (part) {
    case MOE_PACK_ROUTER:
      return d->dtype == MOE_DTYPE_F32 ? size_t(e_pad(d)) * d->d * 4 : size_t(e_pad(d)) * d->d * 3 * 2;
    case MOE_PACK_W13: return size_t(d->n_ffn) * d->d * d->inter * 2 * wb;
    case MOE_PACK_W2: return size_t(d->n_ffn) * d->d * d->inter * wb;
    case MOE_PACK_SW13: return size_t(d->d) * d->shared_inter * 2 * wb;
    case MOE_PACK_SW2: return size_t(d->d) * d->shared_inter * wb;
    default: return 0;
  }
}

moe_status moe_pack_weights(const moe_desc* d, int part, const void* src_a, const void* src_b, void* dst,
                            size_t dst_bytes, void* stream) {
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if (part < MOE_PACK_ROUTER || part > MOE_PACK_SW2) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_packed_bytes(d, part);
  if (need == 0) return MOE_OK;
  if (!src_a || !dst) return MOE_ERR_INVALID_ARG;
  if ((part == MOE_PACK_W13 || part == MOE_PACK_SW13) && !src_b) return MOE_ERR_INVALID_ARG;
  if (dst_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GemmElem el = weight_elem(d);
  hipError_t e = hipSuccess;
  switch (part) {
    case MOE_PACK_ROUTER:
      e = launch_pack_router(static_cast<const float*>(src_a), d->dtype == MOE_DTYPE_F32 ? ELEM_F32 : ELEM_BF16,
                             d->d, d->E, dst, s);
      break;
    case MOE_PACK_W13: e = launch_pack_experts(src_a, src_b, 2, el, d->n_ffn, d->d, d->inter, dst, s); break;
    case MOE_PACK_W2: e = launch_pack_experts(src_a, nullptr, 1, el, d->n_ffn, d->inter, d->d, dst, s); break;
    case MOE_PACK_SW13: e = launch_pack_experts(src_a, src_b, 2, el, 1, d->d, d->shared_inter, dst, s); break;
    case MOE_PACK_SW2: e = launch_pack_experts(src_a, nullptr, 1, el, 1, d->shared_inter, d->d, dst, s); break;
  }
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_route_topk(const moe_desc* d, const moe_weights* w, const void* x, int32_t* topk_idx,
                          float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if (!w || !w->router || !topk_idx || !topk_w || (!x && d->T > 0)) return MOE_ERR_INVALID_ARG;
  const size_t need = ws_bytes_of(d, MOE_OP_ROUTE_TOPK);
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  Carve c(ws);
  const RouteWs r = carve_route(c, d);
  return run_route(d, w, x, topk_idx, topk_w, r, static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_desc* d, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_slot, int32_t* slot_pos, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (d->T > 0 && (!topk_idx || !sorted_slot || !slot_pos)) return MOE_ERR_INVALID_ARG;
  const size_t need = permute_ws_bytes(d);
  if (need > 0 && (ws_bytes < need || !ws)) return MOE_ERR_WORKSPACE;
  return launch_permute(topk_idx, d->T * d->k, d->E, counts, offsets, sorted_slot, slot_pos,
                        static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream)) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status moe_grouped_ffn(const moe_desc* d, const moe_weights* w, int which, const void* x,
                           const int32_t* offsets, const int32_t* sorted_slot, float* rows, void* ws,
                           size_t ws_bytes, void* stream) {
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if (!w || (which != MOE_FFN_ROUTED && which != MOE_FFN_SHARED)) return MOE_ERR_INVALID_ARG;
  const bool routed = which == MOE_FFN_ROUTED;
  if (routed ? d->n_ffn == 0 : d->shared_inter == 0) return MOE_OK;   // nothing to compute
  if (d->T == 0) return MOE_OK;
  if (!x || !rows) return MOE_ERR_INVALID_ARG;
  if (routed && (!offsets || !sorted_slot || !routed_weights_ok(d, w))) return MOE_ERR_INVALID_ARG;
  if (!routed && !shared_weights_ok(d, w)) return MOE_ERR_INVALID_ARG;
  const size_t need = ws_bytes_of(d, routed ? MOE_OP_FFN_ROUTED : MOE_OP_FFN_SHARED);
  if (ws_bytes < need || !ws) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carve c(ws);
  FfnWs f{};
  carve_qx(c, d, f);
  carve_h(c, d, routed ? r_max(d) : d->T, routed ? d->inter : d->shared_inter, f);
  f.partial = c.take(routed ? routed_partial_bytes(d) : dense_partial_bytes(d, false, true));
  if (w8a8(d)) {
    st = run_quant_x(d, x, f, s);
    if (st != MOE_OK) return st;
  }
  const FfnPlan p = routed ? routed_plan(d, w, offsets, sorted_slot) : shared_plan(d, w);
  return run_ffn(d, p, x, f, rows, false, s, nullptr, nullptr, nullptr, nullptr);
}

moe_status moe_combine(const moe_desc* d, const void* x, const float* rows, const float* shared_rows,
                       const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                       const int32_t* slot_pos, void* y, void* stream) {
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  // The kernel reads offsets[ffn_begin] and slot_pos for every selection,
  // whatever n_ffn is, so both tables are required for every call with tokens.
  if (!x || !topk_idx || !topk_w || !y || !offsets || !slot_pos) return MOE_ERR_INVALID_ARG;
  if (d->n_ffn > 0 && !rows) return MOE_ERR_INVALID_ARG;
  if (d->shared_inter > 0 && !shared_rows) return MOE_ERR_INVALID_ARG;
  const CombineArgs c = combine_args(d, x, rows, d->shared_inter > 0 ? shared_rows : nullptr, false, topk_idx, topk_w,
                                     offsets, slot_pos, y);
  return launch_combine(c, static_cast<hipStream_t>(stream)) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_layer(const moe_desc* d, const moe_weights* w, const void* x, void* y, moe_aux* aux, void* ws,
                     size_t ws_bytes, void* stream) {
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if (!w || !w->router || !routed_weights_ok(d, w) || !shared_weights_ok(d, w)) return MOE_ERR_INVALID_ARG;
  if (d->T > 0 && (!x || !y)) return MOE_ERR_INVALID_ARG;
  if (aux) {  // the second stream comes with both of its events, or not at all
    const int given = !!aux->stream2 + !!aux->ev_fork + !!aux->ev_join;
    if (given != 0 && given != 3) return MOE_ERR_INVALID_ARG;
    if (aux->stream2 && aux->stream2 == stream) return MOE_ERR_INVALID_ARG;
    const moe_tuning* t = aux->tuning;
    if (t && (t->shared_ffn1_wgs < 0 || t->shared_ffn2_wgs < 0 || t->routed_ffn1_wgs < 0 || t->routed_ffn2_wgs < 0 ||
              t->prefill_tokens < 0 || t->stream_max_rows < 0 || t->big_min_rows < 0 || t->dense_big_rows < 0 ||
              (t->decode_tile_rows != 0 && t->decode_tile_rows != 32 && t->decode_tile_rows != 64)))
      return MOE_ERR_INVALID_ARG;
  }
  const size_t need = ws_bytes_of(d, MOE_OP_LAYER);
  if (ws_bytes < need || !ws) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carve c(ws);
  LayerWs L = carve_layer(c, d);
  const bool rb = layer_row_bytes(d) == 2;
  moe_aux none{};
  const moe_aux& A = aux ? *aux : none;
  int32_t* idx = A.topk_idx ? A.topk_idx : L.idx;
  float* tw = A.topk_w ? A.topk_w : L.w;
  int32_t* counts = A.counts ? A.counts : L.counts;
  int32_t* offsets = A.offsets ? A.offsets : L.offsets;
  int32_t* sorted_slot = A.sorted_slot ? A.sorted_slot : L.sorted_slot;
  int32_t* slot_pos = A.slot_pos ? A.slot_pos : L.slot_pos;
  const moe_tuning tune = A.tuning ? *A.tuning : moe_tuning{};
  const TilePolicy pol = policy_of(tune);
  auto shared_caps = [&](const FfnPlan& p) { return with_caps(p, tune.shared_ffn1_wgs, tune.shared_ffn2_wgs, pol); };
  auto routed_caps = [&](const FfnPlan& p) { return with_caps(p, tune.routed_ffn1_wgs, tune.routed_ffn2_wgs, pol); };
  if (A.q_x) L.routed.qx = L.shared.qx = A.q_x;
  if (A.s_x) L.routed.sx = L.shared.sx = A.s_x;
  if (d->n_ffn > 0) {
    if (A.h) L.routed.h = static_cast<uint8_t*>(A.h);
    if (A.q_h && w8a8(d)) L.routed.qh = A.q_h;
    if (A.s_h && w8a8(d)) L.routed.sh = A.s_h;
    if (A.rows) L.rows = A.rows;
  }

  const hipEvent_t s1b = static_cast<hipEvent_t>(A.ev_sffn1_begin), s1e = static_cast<hipEvent_t>(A.ev_sffn1_end);
  const hipEvent_t s2b = static_cast<hipEvent_t>(A.ev_sffn2_begin), s2e = static_cast<hipEvent_t>(A.ev_sffn2_end);
  // The shared expert needs only x (and its int8 codes): it is forked onto
  // the caller's second stream, when one is given, before routing starts.
  const bool fork = d->T > 0 && d->shared_inter > 0 && A.stream2 && A.ev_fork && A.ev_join;
  const bool quant = d->T > 0 && w8a8(d);
  const bool apart = fork && routed_parts_apart(d, pol);
  hipStream_t s2 = static_cast<hipStream_t>(A.stream2);
  hipEvent_t ev_join = static_cast<hipEvent_t>(A.ev_join);
  if (fork) {
    HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(A.ev_fork), s));
    HIP_TRY(hipStreamWaitEvent(s2, static_cast<hipEvent_t>(A.ev_fork), 0));
    if (quant) {
      // The int8 codes of x on the second stream, ahead of the shared expert
      // and beside the router (which reads x itself); the routed products
      // wait for this record of ev_join, which is recorded again after the
      // shared expert (a wait takes the record made before it).
      st = run_quant_x(d, x, L.routed, s2);
      if (st != MOE_OK) return st;
      HIP_TRY(hipEventRecord(ev_join, s2));
    }
    // (with the routed products apart, the shared down product is enqueued
    // later, after the small experts' down product)
    st = run_ffn(d, shared_caps(shared_plan(d, w)), x, L.shared, L.shared_rows, rb, s2, s1b, s1e, s2b, s2e,
                 PART_ALL, apart ? PART_NONE : PART_ALL);
    if (st != MOE_OK) return st;
  } else if (quant) {
    st = run_quant_x(d, x, L.routed, s);
    if (st != MOE_OK) return st;
  }
  if (d->T > 0) {
    st = run_route(d, w, x, idx, tw, L.route, s);
    if (st != MOE_OK) return st;
  }
  HIP_TRY(launch_permute(idx, d->T * d->k, d->E, counts, offsets, sorted_slot, slot_pos, L.chunk_hist, s));
  if (d->T == 0) return MOE_OK;
  const hipEvent_t e1b = static_cast<hipEvent_t>(A.ev_ffn1_begin), e1e = static_cast<hipEvent_t>(A.ev_ffn1_end);
  const hipEvent_t e2b = static_cast<hipEvent_t>(A.ev_ffn2_begin), e2e = static_cast<hipEvent_t>(A.ev_ffn2_end);
  const FfnPlan rp = routed_caps(routed_plan(d, w, offsets, sorted_slot));
  if (apart) {
    // Prefill with a second stream: the down product of the experts with at
    // most 64 rows (weight streaming) runs on stream2 between the shared
    // gate/up and the shared down, beside the larger experts' gate/up
    // (matrix-core bound) on `stream`. ev_fork, recorded again after the
    // small experts' gate/up, orders it after their h.
    st = run_ffn(d, rp, x, L.routed, L.rows, rb, s, e1b, nullptr, nullptr, nullptr, PART_SMALL, PART_NONE);
    if (st != MOE_OK) return st;
    HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(A.ev_fork), s));
    st = run_ffn(d, rp, x, L.routed, L.rows, rb, s, nullptr, e1e, e2b, e2e, PART_LARGE, PART_LARGE);
    if (st != MOE_OK) return st;
    HIP_TRY(hipStreamWaitEvent(s2, static_cast<hipEvent_t>(A.ev_fork), 0));
    st = run_ffn(d, rp, x, L.routed, L.rows, rb, s2, nullptr, nullptr, nullptr, nullptr, PART_NONE, PART_SMALL);
    if (st != MOE_OK) return st;
    st = run_ffn(d, shared_caps(shared_plan(d, w)), x, L.shared, L.shared_rows, rb, s2, nullptr, nullptr, s2b, s2e,
                 PART_NONE, PART_ALL);
    if (st != MOE_OK) return st;
  } else if (d->n_ffn > 0) {
    if (fork && quant) HIP_TRY(hipStreamWaitEvent(s, ev_join, 0));   // the codes of x
    st = run_ffn(d, rp, x, L.routed, L.rows, rb, s, e1b, e1e, e2b, e2e);
    if (st != MOE_OK) return st;
  }
  if (fork) {
    HIP_TRY(hipEventRecord(ev_join, s2));   // after the shared expert (and small-expert down) on stream2
    HIP_TRY(hipStreamWaitEvent(s, ev_join, 0));
  } else if (d->shared_inter > 0) {
    st = run_ffn(d, shared_caps(shared_plan(d, w)), x, L.shared, L.shared_rows, rb, s, s1b, s1e, s2b, s2e);
    if (st != MOE_OK) return st;
  }
  const CombineArgs cb = combine_args(d, x, L.rows, L.shared_rows, rb, idx, tw, offsets, slot_pos, y);
  HIP_TRY(launch_combine(cb, s));
  return MOE_OK;
}

}  // extern "C"
