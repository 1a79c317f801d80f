/*
 * moe.h - C ABI of libmoe.so, the MI355X (gfx950) MoE expert layer.
 *
 * One MoE expert layer of a sparse LLM on one device: router matmul and top-k
 * gating, the reordering of tokens by expert, grouped SwiGLU FFN over the
 * resident experts (weight streaming when an expert has few tokens, MFMA
 * tiles when it has many), zero-computation identity experts, the shared
 * expert, and the weighted combine back into token order.
 *
 * Each declaration below cites, by page title and section, the passage that
 * defines the operation it performs. The pages give no formula of the layer;
 * where they are silent the reading taken is stated at the declaration.
 *
 * Conventions for every entry point
 *  - Every tensor pointer is DEVICE memory owned by the caller. The library
 *    never allocates, frees or keeps anything between calls; scratch memory
 *    is the caller's workspace (size from moe_workspace_bytes).
 *  - `stream` is a hipStream_t (NULL = the null stream). All work is enqueued
 *    on it; no entry point synchronises the host or copies device data to
 *    the host, so calls are legal under stream capture.
 *  - Arguments are validated on the host before anything is enqueued; on
 *    error a negative status is returned and nothing was launched.
 *  - Row-major layouts throughout. bf16 is the 16-bit brain float (upper
 *    half of an fp32). Results are deterministic: the same inputs give
 *    bit-identical outputs (no floating-point atomics).
 *  - Preconditions not checked on the device: inputs are finite.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, inconsistent sizes, bad ids */
#define MOE_ERR_UNSUPPORTED (-2) /* shape or option outside what is built */
#define MOE_ERR_WORKSPACE (-3)   /* workspace smaller than moe_workspace_bytes */
#define MOE_ERR_HIP (-4)         /* a HIP call or launch failed */

/* gate */
#define MOE_GATE_SOFTMAX 0 /* scores = softmax over the E logits */
#define MOE_GATE_SIGMOID 1 /* scores = logistic sigmoid of each logit */

/* arithmetic type of the layer */
#define MOE_DTYPE_F32 0  /* x, expert weights, y fp32 */
#define MOE_DTYPE_BF16 1 /* x, expert weights, y bf16; fp32 accumulation */
#define MOE_DTYPE_W8A8 2 /* x, y bf16; int8 weights with fp32 per-output-
                            channel scales; activations quantised to int8 per
                            row inside the layer; int32 accumulation */

/* which FFN moe_grouped_ffn computes */
#define MOE_FFN_ROUTED 0
#define MOE_FFN_SHARED 1

/* weight parts for moe_packed_bytes / moe_pack_weights */
#define MOE_PACK_ROUTER 0 /* src_a = W_r [d][E] fp32                         */
#define MOE_PACK_W13 1    /* src_a = W1, src_b = W3: [n_ffn][d][I]           */
#define MOE_PACK_W2 2     /* src_a = W2: [n_ffn][I][d]                       */
#define MOE_PACK_SW13 3   /* src_a = shared W1, src_b = shared W3: [d][I_s]  */
#define MOE_PACK_SW2 4    /* src_a = shared W2: [I_s][d]                     */

/* ops for moe_workspace_bytes */
#define MOE_OP_ROUTE_TOPK 0
#define MOE_OP_PERMUTE 1
#define MOE_OP_FFN_ROUTED 2
#define MOE_OP_FFN_SHARED 3
#define MOE_OP_COMBINE 4
#define MOE_OP_LAYER 5

/*
 * Layer descriptor (host memory, read during the call only).
 *
 * Sources: sparse activation (each token uses k of E experts) and the
 * zero-computation experts, page "LongCat-Flash与GLM-4.6V，昇腾CANN异构计算深水区
 * 突围详解", section 拆解MoE困局; grouped experts with one quota per group
 * (MoGE), page "华为技术披露集 VOL.12：昇腾×盘古", opening section; one
 * device's share of the routed experts next to one shared expert ("8 routed
 * + 1 shared per card"), page on DeepSeek-V3/R1 on Ascend (Huxiu), opening
 * section. Readings where the pages are silent: the softmax / sigmoid gate
 * is a descriptor field; the group score is the sum of a group's two largest
 * scores; ties go to the lower id.
 *
 * Selection rules (exactly one applies):
 *  - plain: n_group == 1 (or topk_group == 0 and per_group_k == 0): the k
 *    largest scores;
 *  - group-limited: topk_group > 0: experts form n_group contiguous groups of
 *    E/n_group; a group scores the sum of its two largest expert scores; the
 *    topk_group best groups are kept and the k largest scores among their
 *    experts are chosen;
 *  - per-group quota (MoGE): per_group_k > 0: the per_group_k largest of
 *    every group; k must equal n_group * per_group_k.
 * Selections of a token are ordered by descending score; equal scores go to
 * the lower expert (or group) index. A logit bias, when given, is added to
 * the logits before the gate, so it moves both selection and weights.
 * Weights: the selected scores, divided by their sum when renorm != 0, times
 * route_scale.
 *
 * Expert ids [ffn_begin, ffn_begin + n_ffn) are SwiGLU FFN experts resident
 * on this device; [zero_begin, zero_begin + n_zero) are identity experts
 * (output = input); any other id is an expert held elsewhere and contributes
 * nothing here. The two ranges must not overlap.
 *
 * Limits: 1 <= E <= 256; 1 <= k <= min(E, 16); d, inter, shared_inter
 * multiples of 64; T * k <= 2^20; E divisible by n_group; group-limited
 * needs E/n_group >= 2.
 */
typedef struct moe_desc {
    int32_t T;            /* tokens (0 is allowed: every call is a no-op) */
    int32_t d;            /* hidden size */
    int32_t E;            /* experts scored by the router */
    int32_t k;            /* experts selected per token */
    int32_t gate;         /* MOE_GATE_* */
    int32_t n_group;      /* contiguous expert groups (1 = none) */
    int32_t topk_group;   /* group-limited routing: groups kept (0 = off) */
    int32_t per_group_k;  /* MoGE: experts taken from every group (0 = off) */
    int32_t renorm;       /* != 0: divide weights by their sum */
    float route_scale;    /* multiplies every weight */
    int32_t ffn_begin;    /* first resident FFN expert id */
    int32_t n_ffn;        /* resident FFN experts */
    int32_t zero_begin;   /* first identity expert id */
    int32_t n_zero;       /* identity experts */
    int32_t inter;        /* FFN inner size I of the routed experts */
    int32_t shared_inter; /* inner size of the shared expert (0 = none) */
    int32_t dtype;        /* MOE_DTYPE_* */
} moe_desc;

/*
 * Weights (device pointers). Expert and router weights are consumed in the
 * packed layout written by moe_pack_weights (a one-time conversion of the
 * logical x*W layouts; the packed form is private to the library and its
 * size is moe_packed_bytes). Unused members may be NULL.
 */
typedef struct moe_weights {
    const void* router;     /* packed MOE_PACK_ROUTER */
    const float* logit_bias;/* [E] fp32, or NULL */
    const void* w13;        /* packed MOE_PACK_W13 (n_ffn > 0) */
    const void* w2;         /* packed MOE_PACK_W2  (n_ffn > 0) */
    const float* s1;        /* W8A8: [n_ffn][I] scale of W1 columns */
    const float* s3;        /* W8A8: [n_ffn][I] scale of W3 columns */
    const float* s2;        /* W8A8: [n_ffn][d] scale of W2 columns */
    const void* sw13;       /* packed MOE_PACK_SW13 (shared_inter > 0) */
    const void* sw2;        /* packed MOE_PACK_SW2  (shared_inter > 0) */
    const float* ss1;       /* W8A8: [I_s] */
    const float* ss3;       /* W8A8: [I_s] */
    const float* ss2;       /* W8A8: [d]   */
} moe_weights;

/*
 * Launch limits of moe_layer for one layer shape, chosen by the caller from
 * measured runs: the history-based tiling cache of SwiftGMM (page
 * "华为技术披露集 VOL.12：昇腾×盘古", section SwiftGMM：专家计算突击队，闪电速度抵达
 * 推理算力战场) predicts tile parameters from past loads; here the caller
 * times candidate limits and passes the best (tuning.py keeps such a table).
 * Each member caps the workgroups one tiled launch of that product may
 * occupy (all split-K slices together); 0 leaves the library's choice. A cap
 * only narrows a grid and, for the shared expert, its split of the
 * reduction, so no cap needs more workspace; a narrower split adds the
 * partial sums in fewer pieces (results may differ from the uncapped call by
 * fp32 summation order). Capping the shared expert when it runs on stream2
 * leaves compute units to the routing kernels it would otherwise crowd out.
 * Negative members are MOE_ERR_INVALID_ARG. Read during the call only.
 */
typedef struct moe_tuning {
    int32_t shared_ffn1_wgs;  /* shared expert, gate/up projection + SwiGLU */
    int32_t shared_ffn2_wgs;  /* shared expert, down projection */
    int32_t routed_ffn1_wgs;  /* routed experts, gate/up projection + SwiGLU */
    int32_t routed_ffn2_wgs;  /* routed experts, down projection */
    /* Tile choice per expert load: SwiftGMM's switch between streaming an
     * expert's weights (GEMV mode) and tiled products (GEMM mode) by how many
     * tokens the expert received (same page and section). 0 leaves the
     * library's default; each choice changes only which kernel computes a
     * product (fp32 summation order), never the workspace size.
     *  - prefill_tokens: from this many tokens up (default 1024) the routed
     *    experts are classed by their row count as below; with fewer, every
     *    expert takes 64-row tiles in one launch (the reduction split over
     *    workgroups when the experts alone are too few).
     *  - stream_max_rows (theta): from prefill_tokens up, experts with at
     *    most this many rows stream their weights through 64-row tiles
     *    (default 64); larger experts take 128-row tiles, or 256-row tiles
     *    from big_min_rows. Below prefill_tokens, a theta given here sends
     *    experts with at most theta rows to the 32-row weight-streaming
     *    kernel instead (none by default).
     *  - big_min_rows: bf16 experts with at least this many rows take the
     *    256-row tiles (default 256).
     *  - dense_big_rows: bf16 dense products (the shared expert) of at least
     *    this many rows take the 256-row tiles (default 2048).
     *  - decode_tile_rows: below prefill_tokens, the height of the routed
     *    experts' tiles, 64 (default) or 32; any other nonzero value is
     *    MOE_ERR_INVALID_ARG. 32-row tiles halve the padded matrix-core rows
     *    of experts with at most 32 rows; an expert with more takes several
     *    tiles, each reading its weights again, so the choice belongs to a
     *    load bucket whose largest expert fits one tile. */
    int32_t prefill_tokens;
    int32_t stream_max_rows;
    int32_t big_min_rows;
    int32_t dense_big_rows;
    int32_t decode_tile_rows;
} moe_tuning;

/*
 * Optional outputs and hooks of moe_layer; any NULL member is skipped. The
 * table members, when given, are written instead of workspace copies (same
 * contents as moe_route_topk / moe_permute produce). The events are
 * hipEvent_t of the caller, used for timing.
 */
typedef struct moe_aux {
    int32_t* topk_idx;    /* [T][k] */
    float* topk_w;        /* [T][k] */
    int32_t* counts;      /* [E] */
    int32_t* offsets;     /* [E+1] */
    int32_t* sorted_slot; /* [T*k] */
    int32_t* slot_pos;    /* [T*k] */
    int8_t* q_x;          /* W8A8: [T][d] per-token int8 codes of x */
    float* s_x;           /* W8A8: [T] their scales */
    /* Timing events, stamped by the runtime when the routed-expert kernels
     * start and end (hipExtLaunchKernel), so the elapsed time between a
     * begin/end pair is those kernels' own duration, with no marker packet
     * between kernels. Create them with timing enabled. */
    void* ev_ffn1_begin;  /* start / end of the routed-expert gate/up      */
    void* ev_ffn1_end;    /*   projection + SwiGLU (first to last kernel)  */
    void* ev_ffn2_begin;  /* start / end of the routed-expert down         */
    void* ev_ffn2_end;    /*   projection (first to last kernel; with a
                           *   second stream from 1024 tokens up, bf16 and
                           *   fp32: the down product of the experts with
                           *   more than 64 rows, the others' running on
                           *   stream2) */
    /* Shared-expert concurrency: when all three are given (and the layer has
     * a shared expert), the shared FFN runs on stream2, forked from `stream`
     * as soon as its inputs are ready and joined before the combine, so it
     * overlaps routing and the routed experts. This is the multi-stream
     * concurrency of gating, shared expert and feature gathering on the
     * DeepSeek-V3/R1-on-Ascend page (Huxiu), section 模型侧并发优化, item
     * 计算通信并发, and the two-stream overlap on page "LongCat-Flash与
     * GLM-4.6V ...", section 破局之道：多流并行与Single-Batch Overlap.
     * From 1024 tokens up (bf16, fp32) the down product of the experts
     * with at most 64 rows also runs on stream2, after the shared expert;
     * ev_fork is recorded a second time for it, after their gate/up.
     * For W8A8 the int8 codes of x are computed on stream2 too, ahead of
     * the shared expert and beside the router; the routed products on
     * `stream` wait for them through ev_join, which is recorded twice.
     * stream2 must be a non-NULL stream of the same device other than
     * `stream`; the events are hipEvent_t created by the caller. Giving only
     * some of the three, or stream2 equal to `stream`, is
     * MOE_ERR_INVALID_ARG. Results are bit-identical to the single-stream
     * call; work enqueued on `stream` after the call sees the shared expert
     * finished. */
    void* stream2;
    void* ev_fork;
    void* ev_join;
    const moe_tuning* tuning; /* launch limits (see moe_tuning), or NULL */
    /* Optional copies of the routed-expert intermediates: when given, the
     * layer writes them there instead of into its workspace. Rows are the
     * slots of resident FFN experts in expert order (offsets[ffn_begin]
     * onwards), compact, at most T*k of them; only the first
     * R = offsets[ffn_begin + n_ffn] - offsets[ffn_begin] are written.
     * Ignored when the layer has no resident FFN expert. */
    void* h;              /* [T*k][inter] SwiGLU output h = silu(x W1) * (x W3):
                           * float for F32 and W8A8, bf16 for BF16 */
    int8_t* q_h;          /* W8A8: [T*k][inter] int8 codes of h */
    float* s_h;           /* W8A8: [T*k] their per-row scales */
    void* rows;           /* [T*k][d] expert output rows h W2 before the gate
                           * weights: float for F32 and W8A8, bf16 for BF16 */
    /* Timing events of the shared expert's products, stamped like the
     * routed ones above (on the stream the shared expert runs on: stream2
     * when given, else `stream`); ignored without a shared expert. */
    void* ev_sffn1_begin; /* start / end of the shared gate/up + SwiGLU */
    void* ev_sffn1_end;
    void* ev_sffn2_begin; /* start / end of the shared down projection */
    void* ev_sffn2_end;
} moe_aux;

/* Workspace bytes an entry point needs for this descriptor (0 if none). */
size_t moe_workspace_bytes(const moe_desc* desc, int op);

/* Human-readable name of a status code (static storage). */
const char* moe_status_str(moe_status status);

/* Bytes of the packed form of one weight part (MOE_PACK_*). */
size_t moe_packed_bytes(const moe_desc* desc, int part);

/*
 * (A layout conversion of this implementation, not a step of the layer.)
 * Convert one weight part from its logical layout into the packed layout the
 * kernels stream (fragment-major tiles of 16 output columns, each fragment
 * laid out as one matrix-core operand, so a wavefront reads 1 KiB of
 * contiguous memory per load). For MOE_PACK_ROUTER with a bf16 or W8A8
 * layer, W_r is stored as three bf16 planes hi + mid + lo whose sum is
 * exactly W_r (a bf16 activation times each plane is exact in fp32, so the
 * router stays an fp32-accurate product on bf16 matrix cores).
 * src_a / src_b: logical weights in the layer's weight type (fp32, bf16, or
 * int8 for W8A8 experts; the router is always fp32). dst: dst_bytes >=
 * moe_packed_bytes. Enqueued on `stream`.
 */
moe_status moe_pack_weights(const moe_desc* desc, int part, const void* src_a,
                            const void* src_b, void* dst, size_t dst_bytes,
                            void* stream);

/*
 * Router matmul + gating + top-k.
 * Sources: the Router Matmul is one of the weight-streaming operators of
 * page "基于Atlas 900 A3 SuperPoD的LongCat-Flash模型推理性能优化实践", section
 * 优化措施三; selection of k experts per token, page "LongCat-Flash与GLM-4.6V
 * ...", section 拆解MoE困局; per-group quota (MoGE), page "华为技术披露集
 * VOL.12：昇腾×盘古", opening section. Rules: see moe_desc.
 * x: [T][d] (fp32 for MOE_DTYPE_F32, else bf16), device.
 * Out: topk_idx [T][k] int32 expert ids, selections of a token in descending
 * score order; topk_w [T][k] fp32 gate weights. Both device, caller-owned.
 * Logits are fp32-accurate (bf16 x times three exact bf16 planes of W_r).
 * Workspace: moe_workspace_bytes(desc, MOE_OP_ROUTE_TOPK) bytes of device
 * memory. Errors: MOE_ERR_INVALID_ARG (null router, outputs, or x with
 * T > 0), MOE_ERR_WORKSPACE, MOE_ERR_HIP; nothing is launched on error.
 */
moe_status moe_route_topk(const moe_desc* desc, const moe_weights* w,
                          const void* x, int32_t* topk_idx, float* topk_w,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Stable counting sort of the T*k slots (slot s = t*k + j) by expert id:
 * the InitialRouting step that orders every token by expert before tokens
 * move to their experts, page on DeepSeek-V3/R1 on Ascend (Huxiu), section
 * MOE 算子优化. All pointers device, caller-owned.
 * Out: counts [E] (slots per expert), offsets [E+1] (exclusive prefix sum),
 * sorted_slot [T*k] (slots in ascending (expert, s) order), slot_pos [T*k]
 * (inverse: sorted_slot[slot_pos[s]] == s). An id outside [0, E) is dropped:
 * it is not counted and its slot_pos is -1. Bit-exact and deterministic.
 * Workspace: moe_workspace_bytes(desc, MOE_OP_PERMUTE), 0 up to 8192 slots
 * (one workgroup), else a per-chunk histogram of ceil(T*k/2048) * E int32.
 */
moe_status moe_permute(const moe_desc* desc, const int32_t* topk_idx,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                       int32_t* slot_pos, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * Grouped SwiGLU FFN. MOE_FFN_ROUTED: for each resident expert e and each
 * sorted row r in [offsets[e], offsets[e+1]), token t = sorted_slot[r] / k,
 * rows[r - offsets[ffn_begin]] = W2_e^T (silu(x_t W1_e) * (x_t W3_e)).
 * Sources: the grouped matmul over the experts and SwiftGMM's switch between
 * a weight-streaming (GEMV) and a tiled (GEMM) mode by per-expert load, page
 * "华为技术披露集 VOL.12：昇腾×盘古", section SwiftGMM; the SwiGLU form
 * (W1 gate, W3 up, W2 down) is a reading (the pages name no FFN form).
 * The mode is chosen per expert on the device from the offsets (no count
 * reaches the host): below 1024 tokens every expert streams its weights
 * through 64-row matrix-core tiles (an expert with more rows takes several),
 * and when the experts alone give too few workgroups the reduction is split
 * over workgroups; from 1024 tokens up, experts with at most 64 rows stream
 * their weights through 64-row tiles and larger experts run 128-row tiles.
 * Shapes that do not tile (a reduction length that is not a whole number of
 * 256-byte rows, i.e. of 128 bf16, 256 int8 or 64 fp32 elements) use one
 * streaming kernel of 32-row tiles for every expert. MOE_FFN_SHARED: the shared expert
 * (page on DeepSeek-V3/R1 on Ascend (Huxiu), opening section) for every
 * token, rows[t] (offsets, sorted_slot ignored).
 * x: [T][d] (fp32 or bf16 by dtype; W8A8 quantises it per token inside).
 * rows: fp32, capacity T*k rows (routed) or T rows (shared), d columns.
 * All pointers device, caller-owned. Errors: MOE_ERR_INVALID_ARG (null x,
 * rows, weights, or routed tables), MOE_ERR_WORKSPACE, MOE_ERR_HIP.
 */
moe_status moe_grouped_ffn(const moe_desc* desc, const moe_weights* w,
                           int which, const void* x, const int32_t* offsets,
                           const int32_t* sorted_slot, float* rows, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Weighted combine back into token order:
 * y[t] = shared_rows[t] + sum_j topk_w[t][j] * u_tj, where u_tj is
 * rows[slot_pos[t*k+j] - offsets[ffn_begin]] for a resident FFN expert,
 * x[t] for an identity expert and 0 otherwise; fp32 sums in slot order,
 * rounded once to y's type (fp32 for MOE_DTYPE_F32, else bf16).
 * Sources: the Combine of the Dispatch/Combine pair, page on DeepSeek-V3/R1
 * on Ascend (Huxiu), section MOE 算子优化; a zero-computation expert returns
 * its input, page "LongCat-Flash与GLM-4.6V ...", section 拆解MoE困局; the
 * shared expert is added with weight 1 (a reading: the pages show no gate
 * on it).
 * All pointers device, caller-owned. With T > 0, x, topk_idx, topk_w,
 * offsets [E+1], slot_pos [T*k] and y are required for every n_ffn (the
 * kernel reads offsets[ffn_begin] and each selection's slot_pos), rows when
 * n_ffn > 0 and shared_rows when shared_inter > 0 (else it may be NULL);
 * a missing one is MOE_ERR_INVALID_ARG, returned before anything launches.
 */
moe_status moe_combine(const moe_desc* desc, const void* x, const float* rows,
                       const float* shared_rows, const int32_t* topk_idx,
                       const float* topk_w, const int32_t* offsets,
                       const int32_t* slot_pos, void* y, void* stream);

/*
 * The whole layer in one call (the sources of each step are cited at the
 * separate entry points above): (W8A8: quantise x) -> route_topk -> permute
 * -> routed FFN -> shared FFN (on aux->stream2 when given, overlapping the
 * rest) -> combine. x: [T][d]; y: [T][d] (types as in moe_combine). aux may
 * be NULL. The arithmetic is that of the separate entry points, except that
 * the bf16 layer keeps the expert output rows in bf16 between the down
 * projection and the combine (the sum over experts still runs in fp32; fp32
 * and W8A8 layers keep fp32 rows), and that launch limits (aux->tuning) may
 * change how the shared expert splits its reductions (fp32 summation order
 * only). Errors: those of the separate entry points, MOE_ERR_INVALID_ARG for
 * an incomplete stream2/ev_fork/ev_join triple, stream2 equal to stream, or
 * a negative launch limit, and MOE_ERR_WORKSPACE when ws_bytes is below
 * moe_workspace_bytes(desc, MOE_OP_LAYER); these are returned before
 * anything is launched.
 */
moe_status moe_layer(const moe_desc* desc, const moe_weights* w, const void* x,
                     void* y, moe_aux* aux, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * For callers that cannot allocate (code under stream capture that must not
 * call hipMalloc, tight serving loops, hosts that forbid allocation): the
 * whole layer with no workspace argument. The library keeps one device
 * array of MOE_STATIC_WORKSPACE_BYTES per device (held until the process
 * ends) and runs moe_layer with it; the call allocates and frees nothing.
 * The device is the one current on the calling thread; `stream` must belong
 * to it. The first call on a device looks up the array's address there.
 * Arguments, results and errors are those of moe_layer, plus
 * MOE_ERR_WORKSPACE when moe_workspace_bytes(desc, MOE_OP_LAYER) exceeds
 * MOE_STATIC_WORKSPACE_BYTES (returned before any HIP call). The array is
 * not cleared between calls (moe_layer needs no zeroed workspace). Every
 * call on one device shares the one array: calls that overlap on a device
 * (two host threads, or two streams at once) race; the caller orders them.
 */
#define MOE_STATIC_WORKSPACE_BYTES (64u << 20)
moe_status moe_layer_static(const moe_desc* desc, const moe_weights* w, const void* x, void* y,
                            moe_aux* aux, void* stream);

/*
 * Measurement helper, not a step of the layer: the practical HBM read
 * ceiling against which the weight-streaming products are measured (the
 * pages' decode analysis rests on weight movement being the bound: page
 * "华为技术披露集 VOL.12：昇腾×盘古", section SwiftGMM; page
 * "基于Atlas 900 A3 SuperPoD的LongCat-Flash模型推理性能优化实践", section
 * 优化措施三). Reads every byte of the device buffer `buf` (`bytes` a
 * multiple of 16, `buf` 16-byte aligned) once on `stream`, split into
 * MOE_STREAM_READ_WGS contiguous slices, one per workgroup, and writes one
 * 32-bit word per slice to the device array `sink` (MOE_STREAM_READ_WGS
 * words, caller-owned): the XOR of that slice's 32-bit words, so the XOR of
 * all sink words is the XOR of the whole buffer. Nothing else is written;
 * bytes == 0 launches nothing. MOE_ERR_INVALID_ARG (before any launch) for a
 * null pointer, a size not a multiple of 16 or a misaligned pointer.
 */
#define MOE_STREAM_READ_WGS 2048
moe_status moe_stream_read(const void* buf, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
