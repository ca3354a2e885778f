"""Full-size parity in the benchmark's launch configuration.

For the three MoE workloads (T=4096/H=4096/E=64/K=6/W=8 uniform;
T=8192/H=7168/E=256/K=8/W=16 Zipf(1.2) with empty experts;
T=16384/H=7168/E=256/K=8/W=32, 25% of tokens masked, fp8 dispatch) the whole
plan is compared with the oracle bit for bit; dispatch and combine are
checked on a seeded sample of tokens, the oracle evaluating exactly those
tokens (a sub-problem holding their rows), plus the properties that hold at
any size: rows past N keep their sentinel, every live row is written.
"""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import GpuPath, assert_plan_equal, bf16_ulp_distance, dev, host

pytestmark = pytest.mark.gpu

N_SAMPLE = 384


def say(*a):
    print(*a, flush=True)


def sample_tokens(T, seed):
    rng = np.random.default_rng(seed + 777)
    s = rng.choice(T, size=min(N_SAMPLE, T), replace=False)
    return np.sort(np.concatenate([s, [0, T - 1]]))


def sub_problem(pos, tokens):
    """Remaps the sampled tokens' live positions to rows 0..m-1."""
    sub = pos[tokens].copy()
    live = sub >= 0
    rows = sub[live]
    sub[live] = np.arange(rows.size, dtype=np.int32)
    return sub, rows


@pytest.mark.parametrize("idx", [1, 2, 4])
def test_fullsize_workload(idx):
    cfg = workloads.WORKLOADS[idx]
    say("full-size workload", idx, cfg.name)
    ep.ep_device_error()
    inp = workloads.moe_inputs(cfg)
    want = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    N = want.n_rows
    cap = cfg.cap_rows
    g = GpuPath(inp.ids, cfg.E, cfg.W, inp.active)
    g.run_plan()
    assert_plan_equal(g.plan_host(), want)
    say("  plan ok, N =", N)

    x = dev(inp.x)
    toks = sample_tokens(cfg.T, idx)
    sub_pos, rows = sub_problem(want.pos, toks)
    if not cfg.fp8:
        ex = torch.empty((cap, cfg.H), dtype=torch.int16, device="cuda")
        if N < cap:
            ex[N:].fill_(0x7777)
        ep.ep_dispatch(x, g.plan.pos, ex)
        torch.cuda.synchronize()
        # sampled tokens: every live copy's row equals the oracle's dispatch of it
        want_sub = oracle.dispatch_bf16(inp.x[toks], sub_pos, rows.size)
        got_rows = host(ex[dev(rows.astype(np.int64))], np.uint16)
        assert (got_rows == want_sub).all()
        if N < cap:
            assert bool((ex[N:] == 0x7777).all())
        say("  dispatch ok")
        y_dev, y_sub = ex, want_sub          # the combine reads the dispatched rows back
    else:
        q = torch.empty((cap, cfg.H), dtype=torch.uint8, device="cuda")
        sc = torch.full((cap,), -1.0, dtype=torch.float32, device="cuda")
        if N < cap:
            q[N:].fill_(0x33)
        ep.ep_dispatch(x, g.plan.pos, q, sc, out_dtype=ep.EP_FP8_E4M3FN)
        torch.cuda.synchronize()
        want_q, want_s = oracle.dispatch_fp8(inp.x[toks], sub_pos, rows.size)
        ridx = dev(rows.astype(np.int64))
        assert (host(q[ridx]) == want_q).all()
        assert (host(sc[ridx]).view(np.uint32) == want_s.view(np.uint32)).all()
        if N < cap:
            assert bool((q[N:] == 0x33).all()) and bool((sc[N:] == -1.0).all())
        # every live row got a scale (no row was skipped)
        assert bool((sc[:N] >= 0).all())
        say("  fp8 dispatch ok")
        # the bf16 combine reads synthetic expert outputs in expandX layout
        y_host = np.zeros((cap, cfg.H), np.uint16)
        y_host[:N] = workloads.expert_outputs(N, cfg.H, cfg.seed)
        y_dev = dev(y_host)
        y_sub = y_host[rows]
        del y_host

    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    ep.ep_combine(y_dev, g.plan.pos, dev(inp.weights), out)
    torch.cuda.synchronize()
    want_out = oracle.combine(y_sub, sub_pos, inp.weights[toks])
    d = bf16_ulp_distance(host(out[dev(toks.astype(np.int64))], np.uint16), want_out)
    assert d.max() <= 1
    assert (d == 0).all(), f"{int((d > 0).sum())} elements 1 ulp apart"
    if inp.active is not None:
        dead = np.nonzero(inp.active == 0)[0][:64]
        assert (host(out[dev(dead.astype(np.int64))]) == 0).all()
    assert ep.ep_device_error() == 0
    say("  combine ok")
