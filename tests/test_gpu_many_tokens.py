"""Token counts past what one launch's grid holds.

A launch covers at most 2^32 - 1 work-items per grid dimension, and the row
kernels' grids grow with the token count, so the library launches them over
token slices of at most 2^31 work-items (2^25 tokens of one wave each for the
bf16 dispatch and the combines at H = 8 or 16; 2^23 tokens of one 256-thread
workgroup each for the quantised dispatches and the tail).  Each test here
takes a ragged token count a little past one slice, with narrow rows so the
buffers stay small, and checks tokens on both sides of every slice boundary
against the oracle (the dispatch also over every token, by its definition
expand_x[pos[t][k]] = x[t]).  Positions are reversed, so rows written by one
slice sit in the other slice's range.  The checks over every token go in
chunks of at most 2^22 rows or copies: torch's own gather over ~2^26 rows
at once returned zeros or failed to launch on this ROCm build.
"""
import time

import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
from _gpu_util import bf16_ulp_distance, host

pytestmark = pytest.mark.gpu

WAVE_SLICE = 1 << 25      # tokens per launch with one 64-lane item per token
GROUP_SLICE = 1 << 23     # tokens per launch with one 256-thread workgroup per token


def gen(seed):
    return torch.Generator(device="cuda").manual_seed(seed)


def bf16_rows(n, h, g):
    return torch.randn((n, h), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)


def reversed_pos(T, K):
    """pos[t][k] = T*K - 1 - (t*K + k): a bijection onto [0, T*K)."""
    return (T * K - 1 - torch.arange(T * K, device="cuda", dtype=torch.int32)).view(T, K)


CHUNK = 1 << 22


def check_every_row(ex, x, pos, ew=None, w=None):
    """expand_x[pos[t][k]] == x[t] (and expand_weights[pos[t][k]] == w[t][k])
    for every token, bit for bit, a chunk of tokens at a time."""
    T, K = pos.shape
    H = x.shape[1]
    step = max(1, CHUNK // K)
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        rows = pos[t0:t1].reshape(-1).long()
        got = ex.index_select(0, rows).view(t1 - t0, K, H)
        assert torch.equal(got, x[t0:t1].view(t1 - t0, 1, H).expand(t1 - t0, K, H)), (t0, t1)
        if ew is not None:
            assert torch.equal(ew.index_select(0, rows), w[t0:t1].reshape(-1)), (t0, t1)


def sample_tokens(T, slice_len, n=1500, seed=0):
    rng = np.random.default_rng(seed)
    edges = [0, 1, slice_len - 2, slice_len - 1, slice_len, slice_len + 1, T - 2, T - 1]
    return np.unique(np.concatenate([edges, rng.integers(0, T, n)])).astype(np.int64)


def local_rows(pos_sub):
    """Renumber the sampled tokens' rows 0, 1, ... (the oracle gets only their rows)."""
    return np.arange(pos_sub.size, dtype=np.int32).reshape(pos_sub.shape)


def test_bf16_dispatch_and_combine_past_one_launch():
    T, H, K = WAVE_SLICE + 4099, 8, 2
    print("bf16 dispatch + combine, T", T, flush=True)
    g = gen(1)
    x = bf16_rows(T, H, g)
    pos = reversed_pos(T, K)
    w = torch.rand((T, K), generator=g, device="cuda")
    ex = torch.full((T * K, H), 0x7777, dtype=torch.int16, device="cuda")
    ew = torch.full((T * K,), -1.0, device="cuda")
    ep.ep_dispatch(x, pos, ex, weights=w, expand_weights=ew)
    check_every_row(ex, x, pos, ew, w)                # every row, both slices
    out = torch.full((T, H), 0x1234, dtype=torch.int16, device="cuda")
    ep.ep_combine(ex, pos, w, out)
    torch.cuda.synchronize()
    toks = sample_tokens(T, WAVE_SLICE)
    ti = torch.from_numpy(toks).cuda()
    ps = host(pos[ti])
    y_sub = host(ex[torch.from_numpy(ps.reshape(-1).astype(np.int64)).cuda()], np.uint16)
    x_sub = host(x[ti], np.uint16)
    assert (oracle.dispatch_bf16(x_sub, local_rows(ps), ps.size) == y_sub).all()
    want = oracle.combine(y_sub, local_rows(ps), host(w[ti]))
    assert (host(out[ti], np.uint16) == want).all()
    assert ep.ep_device_error() == 0


def test_fp8_dispatch_past_one_launch():
    T, H, K = GROUP_SLICE + 1027, 16, 2
    print("fp8 dispatch, T", T, flush=True)
    g = gen(2)
    x = bf16_rows(T, H, g)
    pos = reversed_pos(T, K)
    w = torch.rand((T, K), generator=g, device="cuda")
    q = torch.full((T * K, H), 0x33, dtype=torch.uint8, device="cuda")
    sc = torch.full((T * K,), -1.0, device="cuda")
    ew = torch.full((T * K,), -1.0, device="cuda")
    ep.ep_dispatch(x, pos, q, sc, out_dtype=ep.EP_FP8_E4M3FN, weights=w, expand_weights=ew)
    for t0 in range(0, T, CHUNK // K):
        t1 = min(T, t0 + CHUNK // K)
        assert torch.equal(ew.index_select(0, pos[t0:t1].reshape(-1).long()), w[t0:t1].reshape(-1))
    toks = sample_tokens(T, GROUP_SLICE, seed=1)
    ti = torch.from_numpy(toks).cuda()
    ps = host(pos[ti])
    rows = torch.from_numpy(ps.reshape(-1).astype(np.int64)).cuda()
    want_q, want_s = oracle.dispatch_fp8(host(x[ti], np.uint16), local_rows(ps), ps.size)
    assert (host(q[rows]) == want_q).all()
    assert (host(sc[rows]).view(np.uint32) == want_s.view(np.uint32)).all()
    assert ep.ep_device_error() == 0


def test_smoothed_int8_dispatch_past_one_launch():
    T, H, K, E = GROUP_SLICE + 515, 16, 2, 4
    print("smoothed int8 dispatch, T", T, flush=True)
    g = gen(3)
    x = bf16_rows(T, H, g)
    ids = torch.randint(0, E, (T, K), generator=g, device="cuda", dtype=torch.int32)
    pos = reversed_pos(T, K)
    smooth = torch.exp(0.5 * torch.randn((E, H), generator=g, device="cuda"))
    q = torch.full((T * K, H), 0x33, dtype=torch.uint8, device="cuda")
    sc = torch.full((T * K,), -1.0, device="cuda")
    ep.ep_dispatch_smooth(x, ids, pos, smooth, q, sc, out_dtype=ep.EP_INT8)
    toks = sample_tokens(T, GROUP_SLICE, seed=2)
    ti = torch.from_numpy(toks).cuda()
    ps = host(pos[ti])
    rows = torch.from_numpy(ps.reshape(-1).astype(np.int64)).cuda()
    want_q, want_s = oracle.dispatch_quant(host(x[ti], np.uint16), host(ids[ti]), local_rows(ps), E,
                                           oracle.Q_INT8, ps.size, host(smooth))
    assert (host(q[rows]) == want_q).all()
    assert (host(sc[rows]).view(np.uint32) == want_s.view(np.uint32)).all()
    assert ep.ep_device_error() == 0


def test_int8_row_combine_past_one_launch():
    T, H, K = WAVE_SLICE + 2053, 16, 1
    print("int8-row combine, T", T, flush=True)
    g = gen(4)
    codes = torch.randint(-127, 128, (T * K, H), generator=g, device="cuda", dtype=torch.int8)
    scales = torch.rand((T * K,), generator=g, device="cuda") + 0.5
    pos = reversed_pos(T, K)
    w = torch.rand((T, K), generator=g, device="cuda")
    out = torch.full((T, H), 0x1234, dtype=torch.int16, device="cuda")
    ep.ep_combine_quant(codes.view(torch.uint8), scales, pos, w, out, code_dtype=ep.EP_INT8)
    torch.cuda.synchronize()
    toks = sample_tokens(T, WAVE_SLICE, seed=3)
    ti = torch.from_numpy(toks).cuda()
    ps = host(pos[ti])
    rows = torch.from_numpy(ps.reshape(-1).astype(np.int64)).cuda()
    want = oracle.combine_quant(host(codes[rows]).view(np.uint8), oracle.Q_INT8, host(scales[rows]),
                                local_rows(ps), host(w[ti]))
    assert (host(out[ti], np.uint16) == want).all()
    assert ep.ep_device_error() == 0


def test_tail_past_one_launch():
    T, H, K = GROUP_SLICE + 333, 8, 2
    print("combine + residual + RMSNorm, T", T, flush=True)
    g = gen(5)
    y = bf16_rows(T * K, H, g)
    pos = reversed_pos(T, K)
    w = torch.rand((T, K), generator=g, device="cuda")
    res = bf16_rows(T, H, g)
    gamma = (1 + 0.1 * torch.randn((H,), generator=g, device="cuda")).to(torch.bfloat16).view(torch.int16)
    ro = torch.empty((T, H), dtype=torch.int16, device="cuda")
    no = torch.empty_like(ro)
    ep.ep_combine_add_rmsnorm(y, pos, w, res, gamma, 1e-6, ro, no)
    ro1 = torch.empty_like(ro)
    no1 = torch.empty_like(ro)
    x1 = bf16_rows(T, H, g)
    ep.ep_add_rmsnorm(x1, res, gamma, 1e-6, ro1, no1)
    torch.cuda.synchronize()
    toks = sample_tokens(T, GROUP_SLICE, seed=4)
    ti = torch.from_numpy(toks).cuda()
    ps = host(pos[ti])
    rows = torch.from_numpy(ps.reshape(-1).astype(np.int64)).cuda()
    gb = host(gamma, np.uint16)
    want_ro, want_no = oracle.combine_add_rmsnorm(host(y[rows], np.uint16), local_rows(ps), host(w[ti]),
                                                  host(res[ti], np.uint16), gb, 1e-6)
    assert (host(ro[ti], np.uint16) == want_ro).all()
    assert bf16_ulp_distance(host(no[ti], np.uint16), want_no).max() <= 1
    # the tail alone is the fused tail with one row per token and weight 1
    n = toks.size
    want_ro1, want_no1 = oracle.combine_add_rmsnorm(host(x1[ti], np.uint16),
                                                    np.arange(n, dtype=np.int32).reshape(n, 1),
                                                    np.ones((n, 1), np.float32), host(res[ti], np.uint16),
                                                    gb, 1e-6)
    assert (host(ro1[ti], np.uint16) == want_ro1).all()
    assert bf16_ulp_distance(host(no1[ti], np.uint16), want_no1).max() <= 1
    assert ep.ep_device_error() == 0


def test_largest_copy_count_plan_dispatch_combine():
    """T*K just under 2^31 (the largest the interface allows): the plan takes
    its multi-kernel path (about a million tiles), then dispatch (8 launches)
    and combine.  Checked by the definitions, in chunks: every position is
    its expert's offset plus the number of earlier copies routed to that
    expert; the split counts are counts per (source rank, expert) and the
    scans and rank offsets are their sums; every dispatched row is its
    token's row; sampled combined tokens equal the oracle's."""
    K, E, W, H = 8, 8, 8, 8
    T = ((1 << 31) - 1) // K // W * W
    N = T * K
    Tw = T // W
    print("largest copy count: T", T, "copies", N, flush=True)
    t_start = time.time()

    def step(what):
        torch.cuda.synchronize()
        print(f"  {what}: {time.time() - t_start:.1f} s", flush=True)

    g = gen(7)
    ids = torch.randint(0, E, (T, K), generator=g, device="cuda", dtype=torch.int32)
    ws = ep.alloc_workspace(T, K, E, W)
    plan = ep.alloc_plan(T, K, E, W, with_occ=False)
    ep.ep_plan(ids, E, W, plan, ws)
    step("plan")
    assert ep.ep_device_error() == 0
    flat_ids = ids.view(-1)
    flat_pos = plan.pos.view(-1)
    # counts per (source rank, expert)
    splits = np.zeros((W, E), np.int64)
    C = CHUNK
    for s in range(W):
        for c0 in range(s * Tw * K, (s + 1) * Tw * K, C):
            c1 = min((s + 1) * Tw * K, c0 + C)
            splits[s] += host(torch.bincount(flat_ids[c0:c1].long(), minlength=E))
    assert splits.sum() == N
    expert_counts = splits.sum(axis=0)
    expert_offsets = np.concatenate([[0], np.cumsum(expert_counts)[:-1]])
    ne = E // W
    assert (host(plan.in_splits) == splits).all()
    assert (host(plan.expert_counts) == expert_counts).all()
    assert (host(plan.expert_offsets) == expert_offsets).all()
    assert (host(plan.rank_offsets) == np.append(expert_offsets[::ne], N)).all()
    assert (host(plan.src_offsets) == np.cumsum(splits, axis=1) - splits).all()
    assert (host(plan.out_splits).reshape(E, W) == splits.T).all()
    before_rank = np.cumsum(splits, axis=0) - splits            # copies of e from ranks < s
    within_rank = expert_offsets - expert_offsets[(np.arange(E) // ne) * ne]
    assert (host(plan.dst_offsets) == before_rank + within_rank).all()
    step("split counts and scans checked")
    # every position: offset of its expert + earlier copies of that expert
    seen = torch.zeros(E, dtype=torch.int64, device="cuda")
    offs = torch.from_numpy(expert_offsets).cuda()
    experts = torch.arange(E, device="cuda", dtype=torch.int32)
    for i, c0 in enumerate(range(0, N, C)):
        c1 = min(N, c0 + C)
        e = flat_ids[c0:c1]
        onehot = (experts[:, None] == e[None, :]).to(torch.int32)          # [E][copies]
        rank = onehot.cumsum(dim=1, dtype=torch.int32).gather(0, e[None, :].long()).view(-1) - 1
        want = offs[e.long()] + seen[e.long()] + rank
        assert torch.equal(flat_pos[c0:c1].long(), want), c0
        seen += onehot.sum(dim=1)
        del onehot, rank, want
        if i % 128 == 127:
            step(f"positions of {c1} copies checked")
    step("every position checked")
    # dispatch every row, then combine
    x = bf16_rows(T, H, g)
    ex = torch.full((N, H), 0x7777, dtype=torch.int16, device="cuda")
    ep.ep_dispatch(x, plan.pos, ex)
    step("dispatch")
    check_every_row(ex, x, plan.pos)
    step("every dispatched row checked")
    w = torch.rand((T, K), generator=g, device="cuda")
    out = torch.full((T, H), 0x1234, dtype=torch.int16, device="cuda")
    ep.ep_combine(ex, plan.pos, w, out)
    step("combine")
    toks = sample_tokens(T, WAVE_SLICE, seed=5)
    ti = torch.from_numpy(toks).cuda()
    ps = host(plan.pos[ti])
    y_sub = host(ex[torch.from_numpy(ps.reshape(-1).astype(np.int64)).cuda()], np.uint16)
    want = oracle.combine(y_sub, local_rows(ps), host(w[ti]))
    assert (host(out[ti], np.uint16) == want).all()
    assert ep.ep_device_error() == 0
