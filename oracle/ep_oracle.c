/*
 * ep_oracle.c -- serial CPU oracle for MoE expert-parallel dispatch / combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library; the bf16 and fp8 codecs below are written
 * from the format definitions, not taken from the GPU code.
 *
 * Everything here is a plain, single-threaded transcription of what the
 * method computes, in the order the sources define it.  Sources:
 *   [P1] PyTorch compare view "ciflow/h100-symm-mem/166772" (NVSHMEM
 *        all-to-all exchange plans): get_occurrence_numbers,
 *        test_make_a2a_exchange_plan, test_make_a2a_2d_exchange_plan,
 *        test_all_to_all_v_2d_index_push, make2dExchangePlan,
 *        _allToAllV_2d_index_push_kernel, allToAllGet.
 *   [P3] aws-neuron/torch-neuronx PR #1035 "Fix all_to_all_single lowering
 *        for uneven split sizes", sections "Motivation and Context" and
 *        "Testing".
 *   [P4] Huawei CANN "aclnnMoeDistributeDispatchV2", parameter table
 *        (expertIds, xActiveMaskOptional, expertScalesOptional, quantMode,
 *        dynamicScalesOut) and "Constraints".
 *   [P5] flashinfer PR #4358 (MNNVL CuTe DSL all-reduce fusion), the MoE
 *        finalize pattern: a routed index of -1 carries weight 0.
 * Where the sources are silent the reading taken is stated at the function.
 *
 * Floating point: compiled with -ffp-contract=off and without fast-math, so
 * every float operation is one IEEE-754 binary32 operation rounded to
 * nearest-even (x86-64 SSE), and fmaf() is the correctly rounded fused
 * multiply-add.  The method fixes binary32 for the scales and for the
 * combine accumulation, so the oracle computes those in binary32.
 *
 * Parity pins: every function is pinned by the -m "not gpu" tests (worked
 * examples from [P1] and [P3], brute force, closed forms, library
 * cross-checks).  The two readings that nothing on the pages can pin are
 * marked "parity unpinned" where they occur: quantisation (fp8 or int8,
 * with or without smoothing) divides by the scale, and a row whose amax is
 * 0 gets scale 0 and zero codes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARGS 2

/* Error bit set when a live copy names an expert outside [0, E). */
#define ORC_DEVERR_BAD_EXPERT 1u
/* Error bit set when a 1-D plan names rows outside a rank's input. */
#define ORC_DEVERR_SPLITS 2u

/* ------------------------------------------------------------------ */
/* bf16: the upper 16 bits of an IEEE-754 binary32.                    */
/* ------------------------------------------------------------------ */

float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to bf16, to nearest, ties to the even bf16 pattern.
 * The dropped 16 bits are compared with one half of a bf16 ulp. */
uint16_t oracle_f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u); /* NaN stays a quiet NaN */
    uint32_t keep = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (keep & 1u)))
        keep += 1u; /* a carry into the exponent is the correct result */
    return (uint16_t)keep;
}

/* ------------------------------------------------------------------ */
/* OCP fp8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa     */
/* bits, no infinities, S.1111.111 is NaN, largest finite 448.          */
/* ------------------------------------------------------------------ */

double oracle_e4m3fn_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9); /* subnormal: m/8 * 2^-6 */
    else
        mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/* Encode a binary32 to E4M3FN by the definition: round to the nearest
 * representable magnitude, ties to the code with an even mantissa LSB,
 * and saturate magnitudes beyond 448 to 448.  The search walks the 127
 * non-negative finite codes in increasing order (they are monotonic);
 * the tie test compares against the exact midpoint of the two neighbours,
 * which needs at most five significant bits and so is exact. */
uint8_t oracle_e4m3fn_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (isnan(v))
        return (uint8_t)(sign | 0x7f);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7e);
    int lo = 0; /* largest code with decode(lo) <= a */
    for (int c = 1; c <= 0x7e; ++c) {
        if (oracle_e4m3fn_decode((uint8_t)c) <= a)
            lo = c;
        else
            break;
    }
    double dlo = oracle_e4m3fn_decode((uint8_t)lo);
    if (dlo == a)
        return (uint8_t)(sign | lo);
    int hi = lo + 1; /* lo < 0x7e here because a < 448 */
    double mid = 0.5 * (dlo + oracle_e4m3fn_decode((uint8_t)hi));
    int pick;
    if (a < mid)
        pick = lo;
    else if (a > mid)
        pick = hi;
    else
        pick = (lo & 1) ? hi : lo;
    return (uint8_t)(sign | pick);
}

/* ------------------------------------------------------------------ */
/* 2-D exchange plan and per-copy positions.                           */
/* ------------------------------------------------------------------ */

/*
 * Inputs: ids[T][K] int32 top-K expert ids ([P4] expertIds is INT32);
 * active[T] (NULL: every token active; [P4] xActiveMaskOptional, read as
 * any 1-D mask, not only a true prefix).  Source rank of token t is
 * s = t / Tw with Tw = T / W (each EP rank owns Bs = Tw tokens, [P4]
 * globalBs = Bs * epWorldSize); expert e lives on rank d = e / ne with
 * ne = E / W ([P1] _allToAllV_2d_index_push_kernel: dst_rank =
 * expert / n_local_experts).
 *
 * A copy (t, k) is live when its token is active and 0 <= e < E.  A copy
 * naming an expert outside [0, E) is dropped and flags
 * ORC_DEVERR_BAD_EXPERT in *err.
 *
 * Outputs (all written; any of occ may be NULL):
 *   in_splits[W][E]      live copies from source rank s to expert e
 *                        ([P1] test_all_to_all_v_2d_index_push builds the
 *                        splits with a histogram of the ids; read as an
 *                        exact integer bincount with E bins)
 *   src_offsets[W][E]    exclusive scan of in_splits[s][:] over e
 *   out_splits[W][ne][W] out_splits[d][le][s] = in_splits[s][d*ne+le]
 *                        ([P1] make2dExchangePlan: out_splits is (ne, npes)
 *                        per rank, the transpose of the exchanged splits)
 *   dst_offsets[W][E]    sum_{s'<s} in_splits[s'][e]
 *                        + sum_{le'<le(e)} expert_counts[d(e)*ne+le']
 *                        ([P1] make2dExchangePlan: per-expert scan down the
 *                        ranks plus the per-rank scan over local experts;
 *                        relative to the destination rank's buffer)
 *   expert_counts[E]     sum_s in_splits[s][e]
 *   expert_offsets[E]    exclusive scan of expert_counts
 *   rank_offsets[W+1]    rank_offsets[d] = expert_offsets[d*ne],
 *                        rank_offsets[W] = N, the number of live copies
 *   occ[T][K]            0-based occurrence of the copy inside its
 *                        (source rank, expert) bucket, in flattened (t, k)
 *                        order ([P1] get_occurrence_numbers: the code's
 *                        cumsum - indicator is 0-based; its docstring
 *                        example is 1-based), -1 if not live
 *   pos[T][K]            rank_offsets[d] + dst_offsets[s][e] + occ
 *                        ([P1] _allToAllV_2d_index_push_kernel: destination
 *                        offset = dst_offsets[expert] + occurrence), the
 *                        global row of expandX, -1 if not live
 */
int oracle_plan(int32_t T, int32_t K, int32_t E, int32_t W,
                const int32_t *ids, const uint8_t *active,
                int64_t *in_splits, int64_t *src_offsets, int64_t *out_splits,
                int64_t *dst_offsets, int64_t *expert_counts,
                int64_t *expert_offsets, int64_t *rank_offsets,
                int32_t *pos, int32_t *occ, uint32_t *err)
{
    if (T < 0 || K < 1 || E < 1 || W < 1 || E % W != 0 || T % W != 0)
        return ORC_ERR_ARGS;
    const int64_t Tw = T / W;
    const int32_t ne = E / W;
    uint32_t flags = 0;

    /* Step 1: split counts. */
    for (int64_t i = 0; i < (int64_t)W * E; ++i)
        in_splits[i] = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (active && !active[t])
            continue;
        int64_t s = t / Tw;
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = ids[t * K + k];
            if (e < 0 || e >= E) {
                flags |= ORC_DEVERR_BAD_EXPERT;
                continue;
            }
            in_splits[s * E + e] += 1;
        }
    }

    /* Step 2: per-expert totals, their exclusive scan, rank starts. */
    int64_t n_live = 0;
    for (int32_t e = 0; e < E; ++e) {
        int64_t c = 0;
        for (int32_t s = 0; s < W; ++s)
            c += in_splits[(int64_t)s * E + e];
        expert_counts[e] = c;
        expert_offsets[e] = n_live;
        n_live += c;
    }
    for (int32_t d = 0; d < W; ++d)
        rank_offsets[d] = expert_offsets[(int64_t)d * ne];
    rank_offsets[W] = n_live;

    /* Step 3: source offsets, an exclusive scan over experts per rank. */
    for (int32_t s = 0; s < W; ++s) {
        int64_t run = 0;
        for (int32_t e = 0; e < E; ++e) {
            src_offsets[(int64_t)s * E + e] = run;
            run += in_splits[(int64_t)s * E + e];
        }
    }

    /* Step 4: output splits, the (ne, W) transpose per destination. */
    for (int32_t d = 0; d < W; ++d)
        for (int32_t le = 0; le < ne; ++le)
            for (int32_t s = 0; s < W; ++s)
                out_splits[((int64_t)d * ne + le) * W + s] =
                    in_splits[(int64_t)s * E + (int64_t)d * ne + le];

    /* Step 5: destination offsets inside the destination rank's buffer. */
    for (int32_t s = 0; s < W; ++s) {
        for (int32_t e = 0; e < E; ++e) {
            int32_t d = e / ne, le = e % ne;
            int64_t down = 0;
            for (int32_t s2 = 0; s2 < s; ++s2)
                down += in_splits[(int64_t)s2 * E + e];
            int64_t across = 0;
            for (int32_t l2 = 0; l2 < le; ++l2)
                across += expert_counts[(int64_t)d * ne + l2];
            dst_offsets[(int64_t)s * E + e] = down + across;
        }
    }

    /* Step 6: stable occurrence numbers and global positions.  One counter
     * per (source rank, expert) bucket, walked in flattened (t, k) order:
     * the occurrence of a copy is the number of earlier live copies of the
     * same bucket. */
    int64_t *seen = (int64_t *)calloc((size_t)W * (size_t)E, sizeof(int64_t));
    if (!seen)
        return ORC_ERR_ARGS;
    for (int64_t t = 0; t < T; ++t) {
        int64_t s = t / Tw;
        for (int32_t k = 0; k < K; ++k) {
            int64_t i = t * K + k;
            int32_t e = ids[i];
            pos[i] = -1;
            if (occ)
                occ[i] = -1;
            if ((active && !active[t]) || e < 0 || e >= E)
                continue;
            int64_t o = seen[s * E + e]++;
            if (occ)
                occ[i] = (int32_t)o;
            pos[i] = (int32_t)(rank_offsets[e / ne] + dst_offsets[s * E + e] + o);
        }
    }
    free(seen);
    if (err)
        *err |= flags;
    return ORC_OK;
}

/* Extended plan: the same quantities with the dispatch options a grouped
 * expert GEMM consumes.
 *   active_copies[T][K] (NULL: all): per-copy mask (CANN
 *       xActiveMaskOptional as a (Bs, K) tensor); a copy is live when its
 *       token is active, its own mask entry is set and 0 <= e < E.
 *   major_align >= 1: every expert's rows are padded up to a multiple of
 *       major_align; with pad_empty an expert without rows still gets
 *       major_align rows ([P1] test_make_a2a_2d_exchange_plan, the padding
 *       rule kept as comments: align each expert's sum up, keep empty
 *       experts at one alignment unit, and let the expert's last source
 *       rank chunk absorb the padding).  in_splits, out_splits and
 *       expert_counts stay the true counts; expert_offsets, rank_offsets,
 *       dst_offsets and pos place each expert's rows at its aligned start,
 *       padding rows after the rows of its last source rank.
 *   expert_token_nums[W][ne] (NULL: not written): per destination rank,
 *       the rows each local expert receives (type 1) or their inclusive
 *       prefix sum over local experts (type 0) (CANN expertTokenNumsOut,
 *       expertTokenNumsType; "prefix sum" read as inclusive). */
int oracle_plan_ex(int32_t T, int32_t K, int32_t E, int32_t W, const int32_t *ids,
                   const uint8_t *active, const uint8_t *active_copies, int32_t major_align,
                   int32_t pad_empty, int32_t token_nums_type, int64_t *in_splits,
                   int64_t *src_offsets, int64_t *out_splits, int64_t *dst_offsets,
                   int64_t *expert_counts, int64_t *expert_offsets, int64_t *rank_offsets,
                   int32_t *pos, int32_t *occ, int64_t *expert_token_nums, uint32_t *err)
{
    if (T < 0 || K < 1 || E < 1 || W < 1 || E % W != 0 || T % W != 0 || major_align < 1)
        return ORC_ERR_ARGS;
    const int64_t Tw = T / W;
    const int32_t ne = E / W;
    const int64_t n_copies = (int64_t)T * K;
    uint32_t flags = 0;

    /* Live copies. */
    uint8_t *live = (uint8_t *)calloc((size_t)(n_copies > 0 ? n_copies : 1), 1);
    if (!live)
        return ORC_ERR_ARGS;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t i = t * K + k;
            if (active && !active[t])
                continue;
            if (active_copies && !active_copies[i])
                continue;
            if (ids[i] < 0 || ids[i] >= E) {
                flags |= ORC_DEVERR_BAD_EXPERT;
                continue;
            }
            live[i] = 1;
        }
    }

    /* Counts, true and padded. */
    for (int64_t i = 0; i < (int64_t)W * E; ++i)
        in_splits[i] = 0;
    for (int64_t i = 0; i < n_copies; ++i)
        if (live[i])
            in_splits[(i / K / Tw) * E + ids[i]] += 1;
    int64_t total_rows = 0;
    for (int32_t e = 0; e < E; ++e) {
        int64_t c = 0;
        for (int32_t s = 0; s < W; ++s)
            c += in_splits[(int64_t)s * E + e];
        expert_counts[e] = c;
        int64_t padded = (c + major_align - 1) / major_align * major_align;
        if (pad_empty && padded == 0)
            padded = major_align;
        expert_offsets[e] = total_rows;
        total_rows += padded;
    }
    for (int32_t d = 0; d < W; ++d)
        rank_offsets[d] = expert_offsets[(int64_t)d * ne];
    rank_offsets[W] = total_rows;

    for (int32_t s = 0; s < W; ++s) {
        int64_t run = 0;
        for (int32_t e = 0; e < E; ++e) {
            src_offsets[(int64_t)s * E + e] = run;
            run += in_splits[(int64_t)s * E + e];
        }
    }
    for (int32_t d = 0; d < W; ++d)
        for (int32_t le = 0; le < ne; ++le)
            for (int32_t s = 0; s < W; ++s)
                out_splits[((int64_t)d * ne + le) * W + s] =
                    in_splits[(int64_t)s * E + (int64_t)d * ne + le];
    for (int32_t s = 0; s < W; ++s) {
        for (int32_t e = 0; e < E; ++e) {
            int64_t down = 0;
            for (int32_t s2 = 0; s2 < s; ++s2)
                down += in_splits[(int64_t)s2 * E + e];
            dst_offsets[(int64_t)s * E + e] = expert_offsets[e] - rank_offsets[e / ne] + down;
        }
    }

    int64_t *seen = (int64_t *)calloc((size_t)W * (size_t)E, sizeof(int64_t));
    if (!seen) {
        free(live);
        return ORC_ERR_ARGS;
    }
    for (int64_t i = 0; i < n_copies; ++i) {
        pos[i] = -1;
        if (occ)
            occ[i] = -1;
        if (!live[i])
            continue;
        int64_t s = i / K / Tw;
        int32_t e = ids[i];
        int64_t o = seen[s * E + e]++;
        if (occ)
            occ[i] = (int32_t)o;
        pos[i] = (int32_t)(rank_offsets[e / ne] + dst_offsets[s * E + e] + o);
    }
    free(seen);
    free(live);

    if (expert_token_nums) {
        for (int32_t d = 0; d < W; ++d) {
            int64_t run = 0;
            for (int32_t le = 0; le < ne; ++le) {
                int64_t c = expert_counts[(int64_t)d * ne + le];
                run += c;
                expert_token_nums[(int64_t)d * ne + le] = token_nums_type == 0 ? run : c;
            }
        }
    }
    if (err)
        *err |= flags;
    return ORC_OK;
}

/* Gate weights carried to the expanded rows (CANN expandScalesOut: the
 * weight each expert row is combined with): expand_weights[pos[t][k]] =
 * w[t][k] for every live copy; other entries are not touched. */
int oracle_dispatch_weights(int32_t T, int32_t K, const int32_t *pos, const float *w,
                            float *expand_weights, int64_t cap_rows)
{
    for (int64_t i = 0; i < (int64_t)T * K; ++i) {
        if (pos[i] < 0)
            continue;
        if (pos[i] >= cap_rows)
            return ORC_ERR_ARGS;
        expand_weights[pos[i]] = w[i];
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Dispatch.                                                           */
/* ------------------------------------------------------------------ */

/* bf16 dispatch: expandX[pos[t][k]][:] = x[t][:] bit for bit for every
 * live copy ([P1] _allToAllV_2d_index_push_kernel puts one row of
 * `stride` bytes per (token, k)).  Rows of expandX that no copy names are
 * not touched. */
int oracle_dispatch_bf16(int32_t T, int32_t K, int32_t H, const uint16_t *x,
                         const int32_t *pos, uint16_t *expand_x, int64_t cap_rows)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t p = pos[t * K + k];
            if (p < 0)
                continue;
            if (p >= cap_rows)
                return ORC_ERR_ARGS;
            memcpy(expand_x + p * H, x + t * (int64_t)H, (size_t)H * sizeof(uint16_t));
        }
    }
    return ORC_OK;
}

/* Per-token dynamic fp8 quantisation on dispatch ([P4] quantMode 2,
 * per-token dynamic quantisation, one fp32 dynamic scale per expanded
 * row).  For a token with at least one live copy:
 *   amax  = max_h |x[t][h]|                (exact)
 *   scale = fl32(amax / 448)               (448 = largest E4M3FN value)
 *   q[h]  = E4M3FN(fl32(x[t][h] / scale))  (RNE, saturating)
 * and every live copy gets the same q row and scale[pos] = scale.
 * Readings (parity unpinned; nothing on the pages fixes them): the value
 * is divided by the scale with one IEEE division, not multiplied by a
 * reciprocal; a token whose amax is 0 gets scale 0 and all codes 0x00. */
int oracle_dispatch_fp8(int32_t T, int32_t K, int32_t H, const uint16_t *x,
                        const int32_t *pos, uint8_t *expand_q, float *expand_scales,
                        int64_t cap_rows, uint8_t *row_scratch)
{
    for (int64_t t = 0; t < T; ++t) {
        int live = 0;
        for (int32_t k = 0; k < K; ++k)
            if (pos[t * K + k] >= 0)
                live = 1;
        if (!live)
            continue;
        const uint16_t *xr = x + t * (int64_t)H;
        float amax = 0.0f;
        for (int32_t h = 0; h < H; ++h) {
            float a = fabsf(oracle_bf16_to_f32(xr[h]));
            if (a > amax)
                amax = a;
        }
        float scale = amax / 448.0f;
        for (int32_t h = 0; h < H; ++h) {
            float v = (scale == 0.0f) ? 0.0f : oracle_bf16_to_f32(xr[h]) / scale;
            row_scratch[h] = oracle_e4m3fn_encode(v);
        }
        for (int32_t k = 0; k < K; ++k) {
            int64_t p = pos[t * K + k];
            if (p < 0)
                continue;
            if (p >= cap_rows)
                return ORC_ERR_ARGS;
            memcpy(expand_q + p * H, row_scratch, (size_t)H);
            expand_scales[p] = scale;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Combine.                                                            */
/* ------------------------------------------------------------------ */

/* Weighted combine of the K expert rows of each token:
 *   out[t][h] = bf16_rne( sum_{k=0..K-1, pos>=0} w[t][k] * y[pos[t][k]][h] )
 * accumulated in binary32 with one fused multiply-add per k, in
 * increasing k, starting from +0.  A copy with pos -1 (inactive token or
 * dropped id) contributes nothing ([P5] MoE finalize: a routed index of
 * -1 carries weight 0), so an inactive token's row is +0.  The weights are
 * the gate scales ([P4] expertScalesOptional, FLOAT32, shape (Bs, K)).
 * The pages print no combine formula; this is the reading taken. */
int oracle_combine(int32_t T, int32_t K, int32_t H, const uint16_t *y,
                   int64_t cap_rows, const int32_t *pos, const float *w,
                   uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k)
            if (pos[t * K + k] >= cap_rows)
                return ORC_ERR_ARGS;
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int64_t p = pos[t * K + k];
                if (p < 0)
                    continue;
                acc = fmaf(w[t * K + k], oracle_bf16_to_f32(y[p * H + h]), acc);
            }
            out[t * (int64_t)H + h] = oracle_f32_to_bf16_rne(acc);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Quantisation variants.                                              */
/* ------------------------------------------------------------------ */

#define ORC_Q_FP8 1
#define ORC_Q_INT8 2

/* int8 code of a binary32: the nearest integer, ties to the even one,
 * clamped to [-127, 127] (symmetric per-token quantisation). */
int8_t oracle_int8_encode(float v)
{
    if (isnan(v))
        return 0;
    if (v >= 127.0f)
        return 127;
    if (v <= -127.0f)
        return -127;
    float f = floorf(v);     /* exact: |v| < 127 */
    float frac = v - f;      /* exact */
    float r;
    if (frac > 0.5f)
        r = f + 1.0f;
    else if (frac < 0.5f)
        r = f;
    else
        r = (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
    return (int8_t)r;
}

static double orc_decode(int qtype, uint8_t code)
{
    return qtype == ORC_Q_FP8 ? oracle_e4m3fn_decode(code) : (double)(int8_t)code;
}

/* Dispatch with per-copy dynamic quantisation ([P4] quantMode 2: per-token
 * dynamic quantisation, INT8 on that hardware; scalesOptional: per-expert
 * smoothing parameters of shape (moeExpertNum, H) applied first).  For every
 * live copy (t, k) of expert e:
 *   xs[h]  = smooth ? fl32(x[t][h] * smooth[e][h]) : x[t][h]
 *   amax   = max_h |xs[h]|,  scale = fl32(amax / qmax)  (qmax 448 or 127)
 *   q[h]   = code(fl32(xs[h] / scale))  (E4M3FN RNE saturating, or int8 RNE
 *            clamped to +-127), all codes 0 when scale == 0
 *   expand_q[pos] = q, expand_scales[pos] = scale.
 * Without smoothing every copy of a token carries the same row.
 * Readings (parity unpinned, as for the fp8 dispatch above): one IEEE
 * division by the scale, and zero codes for a row whose amax is 0. */
int oracle_dispatch_quant(int32_t T, int32_t K, int32_t E, int32_t H, const uint16_t *x,
                          const int32_t *ids, const int32_t *pos, const float *smooth,
                          int32_t qtype, uint8_t *expand_q, float *expand_scales,
                          int64_t cap_rows, float *row_scratch)
{
    if (qtype != ORC_Q_FP8 && qtype != ORC_Q_INT8)
        return ORC_ERR_ARGS;
    const float qmax = qtype == ORC_Q_FP8 ? 448.0f : 127.0f;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t p = pos[t * K + k];
            if (p < 0)
                continue;
            if (p >= cap_rows)
                return ORC_ERR_ARGS;
            int32_t e = ids[t * K + k];
            if (smooth && (e < 0 || e >= E))
                return ORC_ERR_ARGS;
            float amax = 0.0f;
            for (int32_t h = 0; h < H; ++h) {
                float v = oracle_bf16_to_f32(x[t * (int64_t)H + h]);
                if (smooth)
                    v = v * smooth[(int64_t)e * H + h];
                row_scratch[h] = v;
                if (fabsf(v) > amax)
                    amax = fabsf(v);
            }
            float scale = amax / qmax;
            for (int32_t h = 0; h < H; ++h) {
                float v = (scale == 0.0f) ? 0.0f : row_scratch[h] / scale;
                expand_q[p * H + h] = qtype == ORC_Q_FP8 ? oracle_e4m3fn_encode(v)
                                                         : (uint8_t)oracle_int8_encode(v);
            }
            expand_scales[p] = scale;
        }
    }
    return ORC_OK;
}

/* Combine reading quantised expert outputs ([P4] commQuantMode of the
 * combine: rows travel quantised, one fp32 scale per row):
 *   y[row][h] = fl32(decode(q[row][h]) * scales[row])
 *   out[t][h] = bf16_rne(sum_k w[t][k] * y[pos[t][k]][h]), fp32 FMA in k order. */
int oracle_combine_quant(int32_t T, int32_t K, int32_t H, const uint8_t *q, int32_t qtype,
                         const float *scales, int64_t cap_rows, const int32_t *pos,
                         const float *w, uint16_t *out)
{
    if (qtype != ORC_Q_FP8 && qtype != ORC_Q_INT8)
        return ORC_ERR_ARGS;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k)
            if (pos[t * K + k] >= cap_rows)
                return ORC_ERR_ARGS;
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int64_t p = pos[t * K + k];
                if (p < 0)
                    continue;
                float v = (float)orc_decode(qtype, q[p * H + h]) * scales[p];
                acc = fmaf(w[t * K + k], v, acc);
            }
            out[t * (int64_t)H + h] = oracle_f32_to_bf16_rne(acc);
        }
    }
    return ORC_OK;
}

/* Round a double to bf16 to nearest, ties to even, in one step (no
 * intermediate binary32 rounding). */
uint16_t oracle_f64_to_bf16_rne(double v)
{
    if (isnan(v))
        return 0x7fc0;
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0x0000;
    /* Candidates: the bf16 values around v.  Truncating the double to
     * binary32 toward zero and then to bf16 keeps the lower neighbour;
     * the upper one is the next bf16 pattern away from zero. */
    double a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    if (a >= 0x1.ffp127) /* at or past halfway between the largest bf16 and 2^128 */
        return (uint16_t)(sign | 0x7f80);
    float f = (float)a; /* nearest float; fix up to truncation below */
    if ((double)f > a)
        f = nextafterf(f, 0.0f);
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t lo = (uint16_t)(u >> 16);
    uint16_t hi = (uint16_t)(lo + 1);
    double dlo = oracle_bf16_to_f32(lo);
    double dhi = oracle_bf16_to_f32(hi);
    uint16_t pick;
    if (a - dlo < dhi - a)
        pick = lo;
    else if (a - dlo > dhi - a)
        pick = hi;
    else
        pick = (lo & 1) ? hi : lo;
    return (uint16_t)(sign | pick);
}

/* Combine fused with the residual add and RMSNorm of the MoE layer's tail
 * ([P5] the MoE-finalize + residual + RMSNorm pattern, without the
 * all-reduce a single GPU does not need; [P4] names CombineAddRmsNorm):
 *   c    = bf16_rne(sum_k w[t][k] * y[pos[t][k]])   (the combine above)
 *   h    = bf16_rne(f32(residual[t]) + f32(c))       (residual_out, prenorm)
 *   n[h] = bf16_rne(h * gamma / sqrt(mean_h(h^2) + eps))   (norm_out)
 * The sum, the add and the bf16 roundings follow the unfused sequence
 * (combine, then add, then norm); the norm statistics and the scaling are
 * taken in double and rounded once. */
int oracle_combine_add_rmsnorm(int32_t T, int32_t K, int32_t H, const uint16_t *y,
                               int64_t cap_rows, const int32_t *pos, const float *w,
                               const uint16_t *residual, const uint16_t *gamma, float eps,
                               uint16_t *residual_out, uint16_t *norm_out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k)
            if (pos[t * K + k] >= cap_rows)
                return ORC_ERR_ARGS;
        double sumsq = 0.0;
        for (int32_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int64_t p = pos[t * K + k];
                if (p < 0)
                    continue;
                acc = fmaf(w[t * K + k], oracle_bf16_to_f32(y[p * H + h]), acc);
            }
            float c = oracle_bf16_to_f32(oracle_f32_to_bf16_rne(acc));
            float r = oracle_bf16_to_f32(residual[t * (int64_t)H + h]) + c;
            uint16_t hb = oracle_f32_to_bf16_rne(r);
            residual_out[t * (int64_t)H + h] = hb;
            double hv = oracle_bf16_to_f32(hb);
            sumsq += hv * hv;
        }
        double inv = 1.0 / sqrt(sumsq / H + (double)eps);
        for (int32_t h = 0; h < H; ++h) {
            double hv = oracle_bf16_to_f32(residual_out[t * (int64_t)H + h]);
            double g = oracle_bf16_to_f32(gamma[h]);
            norm_out[t * (int64_t)H + h] = oracle_f64_to_bf16_rne(hv * inv * g);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* 1-D uneven all_to_all_single.                                        */
/* ------------------------------------------------------------------ */

/* Plan from the send matrix in_splits[p][r] (rows rank p sends to rank r).
 * Receiver-indexed outputs, as rank r's exchange plan holds them ([P1]
 * test_make_a2a_exchange_plan: out_splits is the all-to-all of the input
 * splits, src_offsets the all-to-all of their exclusive scan, dst_offsets
 * the exclusive scan of out_splits):
 *   out_splits[r][p]  = in_splits[p][r]
 *   src_offsets[r][p] = sum_{r'<r} in_splits[p][r']   (row in p's input)
 *   dst_offsets[r][p] = sum_{p'<p} out_splits[r][p']  (row in r's output)
 *   rank_offsets[r]   = sum_{r'<r} sum_p in_splits[p][r'], [W] = total:
 *                       where rank r's receive buffer starts in the packed
 *                       output of all ranks. */
int oracle_a2a_plan(int32_t W, const int64_t *in_splits, int64_t *src_offsets,
                    int64_t *out_splits, int64_t *dst_offsets, int64_t *rank_offsets)
{
    if (W < 1)
        return ORC_ERR_ARGS;
    for (int32_t r = 0; r < W; ++r)
        for (int32_t p = 0; p < W; ++p)
            out_splits[(int64_t)r * W + p] = in_splits[(int64_t)p * W + r];
    for (int32_t r = 0; r < W; ++r) {
        for (int32_t p = 0; p < W; ++p) {
            int64_t so = 0;
            for (int32_t r2 = 0; r2 < r; ++r2)
                so += in_splits[(int64_t)p * W + r2];
            src_offsets[(int64_t)r * W + p] = so;
            int64_t dof = 0;
            for (int32_t p2 = 0; p2 < p; ++p2)
                dof += out_splits[(int64_t)r * W + p2];
            dst_offsets[(int64_t)r * W + p] = dof;
        }
    }
    int64_t run = 0;
    for (int32_t r = 0; r < W; ++r) {
        rank_offsets[r] = run;
        for (int32_t p = 0; p < W; ++p)
            run += out_splits[(int64_t)r * W + p];
    }
    rank_offsets[W] = run;
    return ORC_OK;
}

/* Data move of the 1-D all-to-all ([P1] allToAllGet: receiver r fetches
 * out_splits[r][p] rows from peer p starting at src_offsets[r][p] and
 * stores them at dst_offsets[r][p] of its output).  `in` holds the W
 * ranks' inputs back to back, R rows each; `out` is the packed receive
 * buffer of all ranks, rank r's part starting at rank_offsets[r].  Rows
 * are `row_bytes` long.  A chunk that would read past its sender's R
 * rows, or write past W*R output rows, is skipped and flags
 * ORC_DEVERR_SPLITS. */
int oracle_a2a_copy(int32_t W, int64_t R, int64_t row_bytes, const uint8_t *in,
                    const int64_t *src_offsets, const int64_t *out_splits,
                    const int64_t *dst_offsets, const int64_t *rank_offsets,
                    uint8_t *out, uint32_t *err)
{
    uint32_t flags = 0;
    for (int32_t r = 0; r < W; ++r) {
        for (int32_t p = 0; p < W; ++p) {
            int64_t n = out_splits[(int64_t)r * W + p];
            int64_t src = src_offsets[(int64_t)r * W + p];
            int64_t dst = rank_offsets[r] + dst_offsets[(int64_t)r * W + p];
            if (n < 0 || src < 0 || src + n > R || dst < 0 || dst + n > (int64_t)W * R) {
                flags |= ORC_DEVERR_SPLITS;
                continue;
            }
            for (int64_t i = 0; i < n; ++i)
                memcpy(out + (dst + i) * row_bytes,
                       in + ((int64_t)p * R + src + i) * row_bytes, (size_t)row_bytes);
        }
    }
    if (err)
        *err |= flags;
    return ORC_OK;
}
