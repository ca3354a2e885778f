"""Full-size parity in the benchmark's launch configuration, element by element.

For the three MoE workloads (T=4096/H=4096/E=64/K=6/W=8 uniform;
T=8192/H=7168/E=256/K=8/W=16 Zipf(1.2) with empty experts;
T=16384/H=7168/E=256/K=8/W=32, 25% of tokens masked, fp8 dispatch) every
output is compared with the oracle over the whole workload:

- the whole plan, bit for bit;
- every row of the expandX buffer, the rows past N included (they must keep
  their sentinel): bf16 rows bit for bit, or every fp8 code and every fp32
  scale bit for bit;
- every output row of the combine, at 0 bf16 ulp.

The oracle runs over token slices on host threads (tests/_oracle_slices.py).
The T=8192 workload is also combined over independent random expert rows,
so that the K inputs of a token differ (the dispatched rows are K copies of
the token's own row).
"""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
import _oracle_slices as par
from _gpu_util import GpuPath, assert_plan_equal, bf16_ulp_distance, dev, host

pytestmark = pytest.mark.gpu

SENTINEL_BF16 = 0x7777
SENTINEL_Q = 0x33
SENTINEL_SCALE = -1.0


def say(*a):
    print(*a, flush=True)


def assert_rows_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if np.array_equal(got, want):
        return
    bad = np.argwhere(got != want)
    r = bad[0][0]
    raise AssertionError(f"{what}: {len(bad)} elements differ in {len(np.unique(bad[:, 0]))} rows; "
                         f"first at {bad[0].tolist()}: got {got[tuple(bad[0])]}, "
                         f"want {want[tuple(bad[0])]} (row {r})")


def assert_combine_exact(got: np.ndarray, want: np.ndarray, what: str):
    d = bf16_ulp_distance(got, want)
    n = int((d > 0).sum())
    assert n == 0, f"{what}: {n} of {d.size} elements differ (max {int(d.max())} ulp), " \
                   f"first at {np.argwhere(d > 0)[0].tolist()}"


def run_combine(y_dev, pos_dev, w_np):
    T = pos_dev.shape[0]
    H = y_dev.shape[1]
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ep.ep_combine(y_dev, pos_dev, dev(w_np), out)
    torch.cuda.synchronize()
    return host(out, np.uint16)


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
    if not cfg.fp8:
        ex = torch.full((cap, cfg.H), SENTINEL_BF16, dtype=torch.int16, device="cuda")
        ep.ep_dispatch(x, g.plan.pos, ex)
        torch.cuda.synchronize()
        want_ex = par.dispatch_bf16(inp.x, want.pos, cap, SENTINEL_BF16)
        assert_rows_equal(host(ex, np.uint16), want_ex, "expandX (bf16)")
        say(f"  dispatch ok: all {cap} rows ({N} written, {cap - N} sentinels)")
        y_dev, y_host = ex, want_ex      # the combine reads the dispatched rows back
    else:
        q = torch.full((cap, cfg.H), SENTINEL_Q, dtype=torch.uint8, device="cuda")
        sc = torch.full((cap,), SENTINEL_SCALE, dtype=torch.float32, device="cuda")
        ep.ep_dispatch(x, g.plan.pos, q, sc, out_dtype=ep.EP_FP8_E4M3FN)
        torch.cuda.synchronize()
        want_q, want_s = par.dispatch_fp8(inp.x, want.pos, cap, SENTINEL_Q, SENTINEL_SCALE)
        assert_rows_equal(host(sc).view(np.uint32), want_s.view(np.uint32), "fp8 scales")
        assert_rows_equal(host(q), want_q, "fp8 codes")
        say(f"  fp8 dispatch ok: all {cap} rows of codes and scales ({N} written)")
        del q, sc, want_q, want_s
        # the bf16 combine reads synthetic expert outputs in expandX layout
        y_host = np.zeros((cap, cfg.H), np.uint16)
        y_host[:N] = workloads.expert_outputs(N, cfg.H, cfg.seed)
        y_dev = dev(y_host)
    del x

    got = run_combine(y_dev, g.plan.pos, inp.weights)
    want_out = par.combine(y_host, want.pos, inp.weights)
    assert_combine_exact(got, want_out, "combine")
    if inp.active is not None:
        dead = inp.active == 0
        assert (got[dead] == 0).all(), "an inactive token's row is not +0"
    say(f"  combine ok: all {cfg.T} rows at 0 ulp")
    assert ep.ep_device_error() == 0


def test_fullsize_zipf_combine_of_distinct_rows():
    """T=8192, H=7168, E=256, K=8, W=16 (Zipf): the combine over independent
    N(0,1) expert rows, so each token sums K different rows; every output
    row against the oracle at 0 ulp."""
    cfg = workloads.WORKLOADS[2]
    say("full-size combine over distinct rows:", cfg.name)
    ep.ep_device_error()
    inp = workloads.moe_inputs(cfg, with_x=False)
    want = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    N = want.n_rows
    g = GpuPath(inp.ids, cfg.E, cfg.W, inp.active)
    g.run_plan()
    assert_plan_equal(g.plan_host(), want)
    y_host = np.zeros((cfg.cap_rows, cfg.H), np.uint16)
    y_host[:N] = workloads.expert_outputs(N, cfg.H, cfg.seed + 50)
    got = run_combine(dev(y_host), g.plan.pos, inp.weights)
    want_out = par.combine(y_host, want.pos, inp.weights)
    assert_combine_exact(got, want_out, "combine of distinct rows")
    say(f"  combine ok: all {cfg.T} rows at 0 ulp")
    assert ep.ep_device_error() == 0
