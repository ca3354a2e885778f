/*
 * ep_mi355x.h -- C ABI of the MI355X (gfx950) MoE expert-parallel dispatch /
 * combine library (libep_mi355x.so).
 *
 * The W expert-parallel ranks are regions of one GPU's memory.  A token t
 * belongs to source rank s = t / Tw (Tw = T / W, each rank owns the same
 * number of tokens, as the global batch of the Huawei CANN
 * "aclnnMoeDistributeDispatchV2" page is Bs * epWorldSize); expert e lives on
 * rank d = e / ne (ne = E / W, the expert-to-rank mapping of
 * _allToAllV_2d_index_push_kernel on the PyTorch compare view
 * "ciflow/h100-symm-mem/166772").
 *
 * Conventions for every entry point:
 *  - Array arguments are DEVICE pointers owned by the caller, row-major and
 *    contiguous.  The library never allocates, never synchronises (except
 *    ep_device_error) and never reads device data on the host.
 *  - bf16 values travel as uint16_t bit patterns, E4M3FN fp8 values as
 *    uint8_t codes.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *    call only enqueues work on it; outputs are ready when the stream
 *    reaches that point.  A call may enqueue several kernels in order (the
 *    plan's look-back path takes two; a row kernel whose grid would exceed
 *    one launch's 2^32 - 1 work-items runs over token slices), all on
 *    `stream`, so a captured graph holds them all.
 *  - Return value: an ep_status.  Argument checks happen on the host before
 *    anything is enqueued; when a check fails nothing was enqueued, and
 *    ep_last_error() describes the first failed check (thread-local).
 *    EP_ERR_HIP reports a failed launch; kernels enqueued by the same call
 *    before it may already have run.
 *    Status classes follow the page above's return codes: null pointer,
 *    invalid value / dtype, unsupported shape.
 *  - Data errors that only the device can see (an expert id outside [0, E)
 *    on a live copy, a 1-D plan that names rows outside a rank's input) do
 *    not abort: the offending copy is dropped and a bit is set in the
 *    device error word, read with ep_device_error().
 *  - Outputs must not overlap inputs (no aliasing), as the all-gather-add
 *    contract of ROCm/aiter PR #6960 requires.
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EP_OK = 0,
    EP_ERR_NULLPTR = 1,     /* a required pointer is NULL                  */
    EP_ERR_INVALID = 2,     /* bad value, alignment, aliasing or dtype     */
    EP_ERR_UNSUPPORTED = 3, /* shape outside the supported limits          */
    EP_ERR_WORKSPACE = 4,   /* workspace too small or not 256-byte aligned */
    EP_ERR_HIP = 5          /* the HIP runtime refused a launch            */
} ep_status;

typedef enum {
    EP_BF16 = 0,       /* expandX rows are bf16, bit copies of x           */
    EP_FP8_E4M3FN = 1, /* expandX rows are OCP E4M3FN codes + fp32 scales  */
    EP_INT8 = 2        /* expandX rows are int8 codes + fp32 scales        */
} ep_dtype;

/* Device error bits (ep_device_error). */
#define EP_DEVERR_BAD_EXPERT 1 /* a live copy named an expert outside [0,E) */
#define EP_DEVERR_SPLITS 2     /* a 1-D plan named rows outside the buffers */
#define EP_DEVERR_PLAN_STALL 4 /* a wait of the plan hit its spin limit (the
                                  workspace was not initialised, or another
                                  stream's kernel held the compute units for
                                  about a second): plan invalid */
#define EP_DEVERR_BAD_ROW 8    /* dispatch/combine met a pos >= cap_rows: that
                                  copy was skipped */

/* Limits: 1 <= K <= 16 and 1 <= E <= 1024 (the dispatch page's top-K and
 * expert-count limits), W >= 1, W divides E and T, T * K < 2^31,
 * H % 8 == 0 for bf16 rows and H % 16 == 0 for fp8 and int8 rows (16-byte
 * vectors), H <= 65536. */
#define EP_MAX_K 16
#define EP_MAX_E 1024
#define EP_MAX_H 65536
#define EP_MAX_SPLITS_W 64

/* Device outputs of ep_plan.  Every pointer except `occ` is required.
 * Sources: the 2-D exchange plan (make2dExchangePlan and
 * test_make_a2a_2d_exchange_plan on the PyTorch compare view
 * "ciflow/h100-symm-mem/166772"), get_occurrence_numbers on the same page,
 * expertTokenNumsOut / epRecvCountsOut on the CANN dispatch page. */
typedef struct {
    int64_t *in_splits;      /* [W][E] live copies from source rank s to expert e     */
    int64_t *src_offsets;    /* [W][E] exclusive scan of in_splits[s][:] over e       */
    int64_t *out_splits;     /* [W][E/W][W] out_splits[d][le][s] = in_splits[s][d*ne+le] */
    int64_t *dst_offsets;    /* [W][E] row of (s, e)'s chunk inside rank e/ne's buffer:
                                sum_{s'<s} in_splits[s'][e]
                                + sum_{le'<le} expert_counts[d*ne+le']                  */
    int64_t *expert_counts;  /* [E] rows each expert receives                          */
    int64_t *expert_offsets; /* [E] exclusive scan of expert_counts (global row start) */
    int64_t *rank_offsets;   /* [W+1] global row where rank d's region starts;
                                rank_offsets[W] = N, the number of live copies         */
    int32_t *pos;            /* [T][K] global expandX row of copy (t,k), -1 if not live */
    int32_t *occ;            /* [T][K] 0-based occurrence inside the (source rank,
                                expert) bucket in flattened (t,k) order, -1 if not
                                live; may be NULL                                      */
} ep_plan_t;

/* Options of ep_plan for consumers that read expandX with a grouped expert
 * GEMM.  A NULL options pointer, or a zero-initialised struct, means: no
 * per-copy mask, no padding, no expert token numbers.
 *   active_copies          [T][K] uint8 or NULL: per-copy mask, the (Bs, K)
 *                          form of xActiveMaskOptional on the CANN dispatch
 *                          page.  A copy is live iff its token is active
 *                          (`active`), its own entry is nonzero and its id is
 *                          in [0, E); a token whose K entries are all zero
 *                          takes no part.
 *   major_align            rows of every expert padded up to a multiple of
 *                          this (<= 0 is read as 1; at most EP_MAX_ALIGN), the
 *                          major_align of the 2-D all-to-all on the PyTorch
 *                          compare view: the padding rows follow the rows of
 *                          the expert's last source rank and are not written.
 *   pad_empty_experts      nonzero: an expert without rows still gets
 *                          major_align rows (the same page's test pads empty
 *                          experts to one unit).
 *   expert_token_nums_type 1: rows each local expert receives; 0: their
 *                          inclusive prefix sum over the rank's local experts
 *                          (expertTokenNumsType on the CANN page).
 *   expert_token_nums      [W][E/W] int64 device output or NULL.
 * With padding, expert_offsets / rank_offsets / dst_offsets / pos place
 * each expert at its aligned start; in_splits, out_splits and expert_counts
 * stay the true counts; rank_offsets[W] is the padded row total, at most
 * ep_expand_rows_bound(). */
typedef struct {
    const uint8_t *active_copies;
    int32_t major_align;
    int32_t pad_empty_experts;
    int32_t expert_token_nums_type;
    int32_t flags;              /* EP_PLAN_* bits, 0 for none */
    int64_t *expert_token_nums;
} ep_plan_opts_t;

/* ep_plan_opts_t.flags.
 * EP_PLAN_LOOKBACK: never take the one-launch plan; the plan then waits
 *   only on tiles that are already running, whatever else the device runs
 *   (the ExchangePlan of the PyTorch compare view never depends on its
 *   blocks being resident together either).  For callers that keep other
 *   kernels that may fill the device running beside the plan.
 * EP_PLAN_TEST_STALL: a test hook for the stall path of the one-launch plan:
 *   the last tile withholds its counts and every wait's budget is a few
 *   hundred polls, so every tile gives up, EP_DEVERR_PLAN_STALL is raised and
 *   the plan is invalid; every kernel still exits normally and the next call
 *   on the same workspace is correct.  No effect when the plan takes the
 *   look-back path. */
#define EP_PLAN_LOOKBACK 1
#define EP_PLAN_TEST_STALL 0x40000000

#define EP_MAX_ALIGN 4096

/* Rows an expandX buffer needs for these dimensions and padding options:
 * T*K plus, per expert, the most padding it can get (E*(align-1), or
 * E*align with pad_empty_experts).  Returns -1 for invalid arguments. */
int64_t ep_expand_rows_bound(int32_t T, int32_t K, int32_t E, int32_t major_align,
                             int32_t pad_empty_experts);

/* Returns 1 if ep_plan / ep_dispatch / ep_combine accept these dimensions
 * and this row dtype, else 0.  Never fails, never touches the GPU (the
 * availability predicate of ROCm/aiter PR #6960's
 * should_custom_ag_lastdim_add). */
int ep_supported(int32_t T, int32_t K, int32_t E, int32_t W, int32_t H, int32_t out_dtype);

/* Bytes of device workspace ep_plan needs for these dimensions (the
 * two-phase GetWorkspaceSize convention of the CANN dispatch page).
 * Returns 0 for dimensions ep_supported rejects. */
size_t ep_workspace_size(int32_t T, int32_t K, int32_t E, int32_t W);

/* Puts a fresh workspace into its initial state (enqueues one fill kernel
 * on `stream`).  Call once after allocating it; ep_plan leaves the
 * workspace in the same state for the next call.  `workspace` must be
 * 256-byte aligned. */
int ep_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/* Exchange plan, stable occurrences and positions.
 *   topk_ids [T][K] int32: top-K expert ids (CANN expertIds is INT32).
 *   active   [T] uint8 or NULL: token t takes part iff active[t] != 0
 *            (xActiveMaskOptional, any 1-D pattern accepted).
 *   plan     device output arrays, see ep_plan_t.
 * A copy (t,k) is live iff its token is active and 0 <= id < E.
 * pos[t][k] = rank_offsets[d] + dst_offsets[s][e] + occ[t][k]: expandX is
 * grouped by destination rank, then local expert, then source rank, then
 * flattened (t,k) order -- the row an index-push puts copy (t,k) to
 * (_allToAllV_2d_index_push_kernel: dst_offsets[expert] + occurrence).
 * `opts` (NULL: none) adds a per-copy mask, expert padding and expert token
 * numbers, see ep_plan_opts_t.
 * The result is deterministic and identical to the serial definition.
 * T == 0 writes the all-zero plan.  The workspace (size from
 * ep_workspace_size, initialised once with ep_workspace_init) must not be
 * used by two calls in flight at the same time.  Its regions are laid out
 * from (T, K, E, W): every call leaves it ready for the next call with the
 * same dimensions; before a call with other dimensions, initialise it
 * again.
 * When its tiles fill at most half of what the device runs at once (and
 * opts does not ask for EP_PLAN_LOOKBACK) the plan is one launch whose
 * tiles exchange counts while running.  Every wait is bounded: if kernels
 * on other streams keep some tiles from being scheduled for about a second,
 * each waiting tile gives up within that one budget and the plan ends with
 * EP_DEVERR_PLAN_STALL rather than hanging.  Larger grids, and
 * EP_PLAN_LOOKBACK, use a look-back that only waits on tiles already
 * running. */
int ep_plan(int32_t T, int32_t K, int32_t E, int32_t W, const int32_t *topk_ids,
            const uint8_t *active, const ep_plan_opts_t *opts, const ep_plan_t *plan,
            void *workspace, size_t ws_bytes, void *stream);

/* ep_plan without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results, options and
 * errors as ep_plan.  The plan's state lives in a static device array of
 * the library (about 3.5 MiB per device, held until the process ends),
 * laid out independently of the dimensions, so calls of any size may follow
 * each other without initialisation.  Limits: the look-back path (taken
 * when the one-launch plan does not fit, or with EP_PLAN_LOOKBACK) holds at
 * most 4096 tiles and 393216 tile-experts (tiles = T*K / 2048, about, never
 * crossing a source rank), else EP_ERR_UNSUPPORTED; the one-launch plan
 * always fits.  Every call on a device shares that device's array: calls
 * that overlap on one device (two streams, two threads) race and must not
 * be issued; calls on different devices are independent.  Allocates
 * nothing; its first call on a device looks up the array's address. */
int ep_plan_noalloc(int32_t T, int32_t K, int32_t E, int32_t W, const int32_t *topk_ids,
                    const uint8_t *active, const ep_plan_opts_t *opts, const ep_plan_t *plan,
                    void *stream);

/* Dispatch scatter: for every copy with pos[t][k] >= 0,
 *   EP_BF16:       expand_x[pos][:] = x[t][:]  (bit copy, H bf16 = 2H bytes)
 *   EP_FP8_E4M3FN: per-token dynamic quantisation (CANN quantMode 2):
 *                  amax = max_h |x[t][h]|, scale = fl32(amax / 448),
 *                  expand_x[pos][h] = E4M3FN_rne_sat(fl32(x[t][h] / scale))
 *                  (all codes 0x00 when scale == 0), expand_scales[pos] = scale
 *                  (dynamicScalesOut: one fp32 scale per expanded row).
 *   EP_INT8:       the same with scale = fl32(amax / 127) and int8 codes:
 *                  the nearest integer of fl32(x[t][h] / scale), ties to even,
 *                  clamped to [-127, 127] (INT8 is the output type of
 *                  quantMode 2 on the CANN page).
 * x [T][H] bf16; expand_x [cap_rows][H] (uint16 bf16, or uint8 codes; H % 16
 * for codes);
 * expand_scales [cap_rows] fp32, required for fp8 and int8, ignored for bf16.
 * weights [T][K] fp32 and expand_weights [cap_rows] fp32, both or neither:
 * expand_weights[pos[t][k]] = weights[t][k], the gate weight carried to each
 * expanded row (expandScalesOut on the CANN dispatch page).
 * cap_rows >= T*K (the worst case: every copy live; with expert padding use
 * ep_expand_rows_bound).  Rows no copy names are not written.  x, expand_x
 * 16-byte aligned; T == 0 enqueues nothing. */
int ep_dispatch(int32_t T, int32_t K, int32_t H, const uint16_t *x, const int32_t *pos,
                int32_t out_dtype, void *expand_x, float *expand_scales, const float *weights,
                float *expand_weights, int64_t cap_rows, void *stream);

/* Weighted combine: for every token t and column h,
 *   out[t][h] = bf16_rne( sum over k = 0..K-1 with pos[t][k] >= 0 of
 *                         w[t][k] * y[pos[t][k]][h] )
 * accumulated in fp32 with one fused multiply-add per k in increasing k,
 * starting from +0 (a token with no live copy gets a +0 row; a copy with
 * pos -1 contributes nothing, as a routed index of -1 with weight 0 in the
 * MoE-finalize pattern of flashinfer PR #4358).  y [cap_rows][H] bf16 (the
 * expert outputs in expandX layout), weights [T][K] fp32 gate scales
 * (expertScalesOptional), out [T][H] bf16.  y, out 16-byte aligned; every
 * pos must be < cap_rows (ep_plan guarantees it). */
int ep_combine(int32_t T, int32_t K, int32_t H, const uint16_t *y, int64_t cap_rows,
               const int32_t *pos, const float *weights, uint16_t *out, void *stream);

/* Dispatch with per-expert smoothing before per-copy dynamic quantisation
 * (scalesOptional, shape (E, H), with quantMode 2 on the CANN dispatch
 * page).  For every live copy (t,k) of expert e = topk_ids[t][k]:
 *   xs[h] = fl32(x[t][h] * smooth_scales[e][h]),
 *   scale = fl32(max_h |xs[h]| / qmax)  (qmax 448 for EP_FP8_E4M3FN, 127 for
 *   EP_INT8), expand_x[pos][h] = code(fl32(xs[h] / scale)) (zero codes when
 *   scale == 0), expand_scales[pos] = scale.
 * Each copy gets its own row and scale.  smooth_scales [E][H] fp32 16-byte
 * aligned; 16 <= H <= 16384, H % 16 == 0; cap_rows >= T*K.  A live copy whose
 * id is outside [0, E) is skipped and raises EP_DEVERR_BAD_EXPERT. */
int ep_dispatch_smooth(int32_t T, int32_t K, int32_t E, int32_t H, const uint16_t *x,
                       const int32_t *topk_ids, const int32_t *pos, const float *smooth_scales,
                       int32_t out_dtype, void *expand_x, float *expand_scales, int64_t cap_rows,
                       void *stream);

/* Combine of quantised expert rows (commQuantMode of the CANN combine: rows
 * travel as codes with one fp32 scale per row):
 *   y[row][h] = fl32(decode(codes[row][h]) * row_scales[row])
 *   out[t][h] = bf16_rne(sum over live k of w[t][k] * y[pos[t][k]][h]),
 * fp32 fused multiply-adds in increasing k from +0, as ep_combine.
 * codes [cap_rows][H] uint8 (E4M3FN or int8 per code_dtype), row_scales
 * [cap_rows] fp32, weights [T][K] fp32, out [T][H] bf16; H % 16 == 0;
 * codes and out 16-byte aligned; every pos must be < cap_rows. */
int ep_combine_quant(int32_t T, int32_t K, int32_t H, const void *codes, int32_t code_dtype,
                     const float *row_scales, int64_t cap_rows, const int32_t *pos,
                     const float *weights, uint16_t *out, void *stream);

/* Combine fused with the layer tail (the MoE-finalize + residual + RMSNorm
 * pattern of flashinfer PR #4358 without its all-reduce; CombineAddRmsNorm
 * on the CANN dispatch page).  For every token t and column h:
 *   c = bf16_rne(sum_k w[t][k] * y[pos[t][k]][h])        (as ep_combine)
 *   residual_out[t][h] = bf16_rne(residual[t][h] + c)    (fp32 add)
 *   norm_out[t][h] = bf16_rne(residual_out[t][h] * gamma[h]
 *                             / sqrt(mean_h(residual_out[t][h]^2) + eps))
 * with the mean's sum of squares accumulated in fp32.  The combined rows
 * are not written (they never reach HBM).  8 <= H <= 16384, H % 8 == 0,
 * eps >= 0; residual, gamma [H], residual_out, norm_out bf16 16-byte
 * aligned; outputs must not overlap inputs or each other.  The result is
 * bit-identical to ep_combine followed by ep_add_rmsnorm. */
int ep_combine_add_rmsnorm(int32_t T, int32_t K, int32_t H, const uint16_t *y, int64_t cap_rows,
                           const int32_t *pos, const float *weights, const uint16_t *residual,
                           const uint16_t *gamma, float eps, uint16_t *residual_out,
                           uint16_t *norm_out, void *stream);

/* The layer tail alone: residual_out = bf16_rne(residual + x) and norm_out
 * as above, for x [T][H] bf16 (the unfused second half of
 * ep_combine_add_rmsnorm).  Same limits. */
int ep_add_rmsnorm(int32_t T, int32_t H, const uint16_t *x, const uint16_t *residual,
                   const uint16_t *gamma, float eps, uint16_t *residual_out, uint16_t *norm_out,
                   void *stream);

/* 1-D uneven all_to_all_single plan (test_make_a2a_exchange_plan on the
 * PyTorch compare view; the uneven-split lowering of aws-neuron/torch-neuronx
 * PR #1035).  in_splits[p][r] = rows rank p sends to rank r.  Outputs,
 * receiver-indexed, all [W][W] except rank_offsets [W+1]:
 *   out_splits[r][p]  = in_splits[p][r]
 *   src_offsets[r][p] = sum_{r'<r} in_splits[p][r']  (row in p's input)
 *   dst_offsets[r][p] = sum_{p'<p} out_splits[r][p'] (row in r's output)
 *   rank_offsets[r]   = rows received by ranks < r; [W] = total rows.
 * 1 <= W <= EP_MAX_SPLITS_W.  One workgroup, enqueued on `stream`. */
int ep_plan_splits(int32_t W, const int64_t *in_splits, int64_t *src_offsets,
                   int64_t *out_splits, int64_t *dst_offsets, int64_t *rank_offsets,
                   void *stream);

/* 1-D uneven all-to-all data move (allToAllGet on the PyTorch compare view):
 * for every receiver r and sender p, rows
 *   in[p][src_offsets[r][p] + i]  ->  out[rank_offsets[r] + dst_offsets[r][p] + i]
 * for i < out_splits[r][p].  in [W][R] rows, out [W*R] rows (the packed
 * receive buffers of all ranks), each row `stride_bytes` long (multiple of
 * 16; in, out 16-byte aligned; W*R*stride_bytes < 2^63, else
 * EP_ERR_UNSUPPORTED).  A chunk that would read past row R of its sender or
 * write past row W*R is skipped and sets EP_DEVERR_SPLITS. */
int ep_dispatch_splits(int32_t W, int64_t R, int64_t stride_bytes, const void *in,
                       const int64_t *src_offsets, const int64_t *out_splits,
                       const int64_t *dst_offsets, const int64_t *rank_offsets, void *out,
                       void *stream);

/* The 1-D all-to-all in one launch: ep_plan_splits and ep_dispatch_splits
 * fused (every workgroup derives its own chunk's offsets from in_splits
 * [W][W], so no plan kernel runs first).  Moves the rows exactly as
 * ep_dispatch_splits does with the plan ep_plan_splits computes, and writes
 * that plan to src_offsets / out_splits / dst_offsets ([W][W]) and
 * rank_offsets ([W+1]), each of which may be NULL (not written).  A chunk
 * whose rows fall outside the buffers is skipped and sets
 * EP_DEVERR_SPLITS.  R == 0 with no plan output requested enqueues
 * nothing; in and out may be NULL when R == 0.  Same row and size limits
 * as ep_dispatch_splits. */
int ep_all_to_all_splits(int32_t W, int64_t R, int64_t stride_bytes, const int64_t *in_splits,
                         const void *in, void *out, int64_t *src_offsets, int64_t *out_splits,
                         int64_t *dst_offsets, int64_t *rank_offsets, void *stream);

/* Thread-local description of the last non-OK status ("" if none).  The
 * status carries the class, as the return codes of the CANN
 * "aclnnMoeDistributeDispatchV2" Returns table do (null pointers,
 * unsupported data types, unsupported shapes or parameter values); this
 * text names the failing check and its values. */
const char *ep_last_error(void);

/* Synchronises `stream`, then returns in *code the device error bits
 * (EP_DEVERR_*) raised on the current device since the previous call, and
 * clears those bits (an atomic AND enqueued on `stream`, then waited for):
 * a bit a kernel on another stream raises meanwhile stays set for the next
 * call.  The kernels of the PyTorch compare view "ciflow/h100-symm-mem/166772"
 * check their device-side preconditions with in-kernel asserts, which abort
 * (CUDA_KERNEL_ASSERT in exchangeSplitAndOffset and allToAllGet); here a
 * data error seen on the device drops the offending copy or chunk, raises a
 * bit, and the caller reads the bits with this call. */
int ep_device_error(void *stream, int32_t *code);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_H */
