/*
 * Drives every entry point of the C ABI down its host-side validation
 * paths (no GPU: every call below fails its checks, or returns early for
 * empty inputs, before anything is enqueued).  Built host-only with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_abi_sanitized.py, which runs it and expects "all checks passed".
 * Pointers are fake, never dereferenced addresses: the checks only compare
 * them.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ep_mi355x.h"

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        printf("FAIL %s: got %d want %d (%s)\n", what, got, want, ep_last_error());
        failures++;
    } else if (want != EP_OK && ep_last_error()[0] == '\0') {
        printf("FAIL %s: no message\n", what);
        failures++;
    }
}

static void check(int cond, const char *what)
{
    if (!cond) {
        printf("FAIL %s\n", what);
        failures++;
    }
}

#define P(off) ((void *)(uintptr_t)(((uintptr_t)1 << 40) + (uintptr_t)(off)))

int main(void)
{
    const uintptr_t G = (uintptr_t)1 << 34; /* spacing of the fake buffers */

    /* predicates and sizes */
    check(ep_supported(64, 2, 8, 2, 128, EP_BF16) == 1, "supported bf16");
    check(ep_supported(64, 2, 8, 2, 136, EP_INT8) == 0, "int8 H % 16");
    check(ep_supported(64, 17, 8, 2, 128, EP_BF16) == 0, "K > 16");
    check(ep_workspace_size(64, 2, 9, 2) == 0, "workspace size of a bad shape");
    check(ep_workspace_size(8192, 8, 256, 16) > 0, "workspace size");
    check(ep_expand_rows_bound(64, 2, 8, 4, 1) == 128 + 32, "rows bound");
    check(ep_expand_rows_bound(64, 2, 8, 5000, 0) == -1, "rows bound, align too large");

    /* workspace */
    expect(ep_workspace_init(NULL, 256, NULL), EP_ERR_NULLPTR, "workspace NULL");
    expect(ep_workspace_init(P(8), 256, NULL), EP_ERR_WORKSPACE, "workspace misaligned");

    /* plan */
    ep_plan_t plan;
    int64_t *a64 = (int64_t *)P(0);
    plan.in_splits = a64;
    plan.src_offsets = (int64_t *)P(1 * G);
    plan.out_splits = (int64_t *)P(2 * G);
    plan.dst_offsets = (int64_t *)P(3 * G);
    plan.expert_counts = (int64_t *)P(4 * G);
    plan.expert_offsets = (int64_t *)P(5 * G);
    plan.rank_offsets = (int64_t *)P(6 * G);
    plan.pos = (int32_t *)P(7 * G);
    plan.occ = (int32_t *)P(8 * G);
    const int32_t *ids = (const int32_t *)P(9 * G);
    void *ws = P(10 * G);
    const size_t wsb = ep_workspace_size(64, 2, 8, 2);
    expect(ep_plan(64, 2, 8, 2, NULL, NULL, NULL, &plan, ws, wsb, NULL), EP_ERR_NULLPTR, "plan ids NULL");
    expect(ep_plan(64, 2, 8, 2, ids, NULL, NULL, NULL, ws, wsb, NULL), EP_ERR_NULLPTR, "plan NULL");
    expect(ep_plan(64, 2, 8, 2, ids, NULL, NULL, &plan, ws, wsb - 4, NULL), EP_ERR_WORKSPACE, "plan small ws");
    expect(ep_plan(63, 2, 8, 2, ids, NULL, NULL, &plan, ws, wsb, NULL), EP_ERR_UNSUPPORTED, "plan T % W");
    expect(ep_plan(64, 0, 8, 2, ids, NULL, NULL, &plan, ws, wsb, NULL), EP_ERR_UNSUPPORTED, "plan K = 0");
    ep_plan_t alias = plan;
    alias.pos = (int32_t *)plan.in_splits;
    expect(ep_plan(64, 2, 8, 2, ids, NULL, NULL, &alias, ws, wsb, NULL), EP_ERR_INVALID, "plan aliasing");
    ep_plan_opts_t opts;
    memset(&opts, 0, sizeof opts);
    opts.major_align = EP_MAX_ALIGN + 1;
    expect(ep_plan(64, 2, 8, 2, ids, NULL, &opts, &plan, ws, wsb, NULL), EP_ERR_UNSUPPORTED, "plan align");
    opts.major_align = 4;
    opts.expert_token_nums_type = 3;
    expect(ep_plan(64, 2, 8, 2, ids, NULL, &opts, &plan, ws, wsb, NULL), EP_ERR_INVALID, "plan token nums type");

    /* dispatch */
    const uint16_t *x = (const uint16_t *)P(11 * G);
    const int32_t *pos = (const int32_t *)P(12 * G);
    void *ex = P(13 * G);
    float *sc = (float *)P(14 * G);
    expect(ep_dispatch(64, 2, 128, x, pos, EP_BF16, ex, NULL, NULL, NULL, 127, NULL), EP_ERR_INVALID, "dispatch cap");
    expect(ep_dispatch(64, 2, 136, x, pos, EP_FP8_E4M3FN, ex, sc, NULL, NULL, 128, NULL), EP_ERR_UNSUPPORTED, "dispatch fp8 H");
    expect(ep_dispatch(64, 2, 128, x, pos, EP_INT8, ex, NULL, NULL, NULL, 128, NULL), EP_ERR_NULLPTR, "dispatch int8 scales");
    expect(ep_dispatch(64, 2, 128, x, pos, 9, ex, NULL, NULL, NULL, 128, NULL), EP_ERR_INVALID, "dispatch dtype");
    expect(ep_dispatch(64, 2, 128, x, pos, EP_BF16, (void *)(x + 128), NULL, NULL, NULL, 128, NULL), EP_ERR_INVALID, "dispatch alias");
    expect(ep_dispatch(0, 2, 128, NULL, NULL, EP_BF16, NULL, NULL, NULL, NULL, 0, NULL), EP_OK, "dispatch empty");

    /* smoothed dispatch and quantised combine */
    const float *smooth = (const float *)P(15 * G);
    expect(ep_dispatch_smooth(64, 2, 8, 128, x, ids, pos, smooth, EP_BF16, ex, sc, 128, NULL), EP_ERR_INVALID, "smooth dtype");
    expect(ep_dispatch_smooth(64, 2, 8, 16400, x, ids, pos, smooth, EP_FP8_E4M3FN, ex, sc, 128, NULL), EP_ERR_UNSUPPORTED, "smooth H");
    expect(ep_dispatch_smooth(64, 2, 8, 128, x, ids, pos, NULL, EP_INT8, ex, sc, 128, NULL), EP_ERR_NULLPTR, "smooth NULL");
    expect(ep_dispatch_smooth(64, 2, 8, 128, x, ids, pos, smooth, EP_INT8, (void *)smooth, sc, 128, NULL), EP_ERR_INVALID, "smooth alias");
    expect(ep_dispatch_smooth(0, 2, 8, 128, NULL, NULL, NULL, NULL, EP_INT8, NULL, NULL, 0, NULL), EP_OK, "smooth empty");
    const float *w = (const float *)P(16 * G);
    uint16_t *out = (uint16_t *)P(17 * G);
    expect(ep_combine_quant(64, 2, 128, ex, EP_BF16, sc, 128, pos, w, out, NULL), EP_ERR_INVALID, "combine_quant dtype");
    expect(ep_combine_quant(64, 2, 128, ex, EP_FP8_E4M3FN, NULL, 128, pos, w, out, NULL), EP_ERR_NULLPTR, "combine_quant NULL");
    expect(ep_combine_quant(64, 2, 128, ex, EP_INT8, sc, 128, pos, w, (uint16_t *)ex, NULL), EP_ERR_INVALID, "combine_quant alias");

    /* combine and tail */
    const uint16_t *y = (const uint16_t *)P(18 * G);
    expect(ep_combine(64, 2, 132, y, 128, pos, w, out, NULL), EP_ERR_UNSUPPORTED, "combine H");
    expect(ep_combine(64, 2, 128, y, -1, pos, w, out, NULL), EP_ERR_INVALID, "combine cap");
    expect(ep_combine(64, 2, 128, y, 128, pos, w, (uint16_t *)y + 512, NULL), EP_ERR_INVALID, "combine alias");
    const uint16_t *res = (const uint16_t *)P(19 * G), *gam = (const uint16_t *)P(20 * G);
    uint16_t *ro = (uint16_t *)P(21 * G), *no = (uint16_t *)P(22 * G);
    expect(ep_combine_add_rmsnorm(64, 2, 16392, y, 128, pos, w, res, gam, 1e-6f, ro, no, NULL), EP_ERR_UNSUPPORTED, "tail H");
    expect(ep_combine_add_rmsnorm(64, 2, 128, y, 128, pos, w, res, gam, -1.0f, ro, no, NULL), EP_ERR_INVALID, "tail eps");
    expect(ep_combine_add_rmsnorm(64, 2, 128, y, 128, pos, w, res, gam, 1e-6f, ro, ro, NULL), EP_ERR_INVALID, "tail outputs alias");
    expect(ep_add_rmsnorm(64, 128, y, res, gam, 1e-6f, NULL, no, NULL), EP_ERR_NULLPTR, "add_rmsnorm NULL");

    /* 1-D all-to-all */
    const int64_t *sp = (const int64_t *)P(23 * G);
    int64_t *so = (int64_t *)P(24 * G), *os = (int64_t *)P(25 * G), *dof = (int64_t *)P(26 * G),
            *ro64 = (int64_t *)P(27 * G);
    expect(ep_plan_splits(65, sp, so, os, dof, ro64, NULL), EP_ERR_UNSUPPORTED, "splits W");
    expect(ep_plan_splits(8, sp, so, so, dof, ro64, NULL), EP_ERR_INVALID, "splits alias");
    expect(ep_dispatch_splits(8, 4096, 4100, P(28 * G), so, os, dof, ro64, P(29 * G), NULL), EP_ERR_UNSUPPORTED, "splits stride");
    expect(ep_dispatch_splits(8, 0, 4096, NULL, so, os, dof, ro64, NULL, NULL), EP_OK, "splits empty");

    /* 1-D all-to-all in one launch */
    const int64_t *isp = (const int64_t *)P(30 * G);
    expect(ep_all_to_all_splits(65, 16, 32, isp, P(28 * G), P(29 * G), so, os, dof, ro64, NULL), EP_ERR_UNSUPPORTED, "fused splits W");
    expect(ep_all_to_all_splits(8, 16, 32, NULL, P(28 * G), P(29 * G), so, os, dof, ro64, NULL), EP_ERR_NULLPTR, "fused splits NULL");
    expect(ep_all_to_all_splits(8, 16, 32, isp, P(28 * G), P(28 * G) , NULL, NULL, NULL, NULL, NULL), EP_ERR_INVALID, "fused splits alias");
    expect(ep_all_to_all_splits(8, 0, 32, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), EP_OK, "fused splits empty");

    /* a long message does not overflow the error buffer */
    expect(ep_dispatch(64, 2, 128, x, pos, EP_BF16, ex, NULL, NULL, NULL, -9223372036854775807LL, NULL),
           EP_ERR_INVALID, "dispatch negative cap");
    printf("last error: %s\n", ep_last_error());

    if (failures) {
        printf("%d checks failed\n", failures);
        return 1;
    }
    printf("all checks passed\n");
    return 0;
}
