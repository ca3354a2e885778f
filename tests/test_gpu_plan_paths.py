"""The plan's two paths and the bounds on its waits.

* EP_PLAN_LOOKBACK forces the look-back path (tiles wait only on tiles that
  took their ticket earlier, so already running): on the T=8192 Zipf and the
  T=16384 masked workloads it equals the oracle and the one-launch plan.
* Two plans that each fill the whole device (512 tiles) run on two streams
  at once on the look-back path, round after round, exact every time.
* The one-launch plan's stall path, forced from the host (EP_PLAN_TEST_STALL:
  the last tile withholds its counts and the waits get a short budget):
  every tile gives up, EP_DEVERR_PLAN_STALL is raised, every kernel exits,
  and the next call on the same workspace is exact.
"""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import GpuPath, assert_plan_equal

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("idx", [2, 4])
def test_lookback_forced_on_the_workloads(idx):
    cfg = workloads.WORKLOADS[idx]
    say("forced look-back plan on", cfg.name)
    inp = workloads.moe_inputs(cfg, with_x=False)
    want = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    g = GpuPath(inp.ids, cfg.E, cfg.W, inp.active)
    for _ in range(3):
        g.run_plan(flags=ep.EP_PLAN_LOOKBACK)
        assert_plan_equal(g.plan_host(), want)
        g.run_plan()
        assert_plan_equal(g.plan_host(), want)
    assert ep.ep_device_error() == 0


def test_two_device_sized_lookback_plans_on_two_streams():
    T, K, E, W = 131072, 8, 64, 8            # 512 tiles each: the whole device
    say("two device-sized look-back plans on two streams")
    rng = np.random.default_rng(21)
    ids_a = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids_b = rng.integers(0, E, size=(T, K)).astype(np.int32)
    want_a, want_b = oracle.plan(ids_a, E, W), oracle.plan(ids_b, E, W)
    a, b = GpuPath(ids_a, E, W), GpuPath(ids_b, E, W)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for it in range(10):
        with torch.cuda.stream(s1):
            a.run_plan(flags=ep.EP_PLAN_LOOKBACK)
        with torch.cuda.stream(s2):
            b.run_plan(flags=ep.EP_PLAN_LOOKBACK)
        torch.cuda.synchronize()
        assert_plan_equal(a.plan_host(), want_a)
        assert_plan_equal(b.plan_host(), want_b)
    assert ep.ep_device_error() == 0


def test_one_launch_plan_stall_gives_up_then_recovers():
    cfg = workloads.WORKLOADS[2]             # 32 tiles: the one-launch plan
    say("one-launch plan, stall forced from the host")
    inp = workloads.moe_inputs(cfg, with_x=False)
    want = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    g = GpuPath(inp.ids, cfg.E, cfg.W, inp.active)
    assert ep.ep_device_error() == 0
    for _ in range(2):
        g.run_plan(flags=ep.EP_PLAN_TEST_STALL)
        assert ep.ep_device_error() == ep.EP_DEVERR_PLAN_STALL
        g.run_plan()
        assert_plan_equal(g.plan_host(), want)
        assert ep.ep_device_error() == 0
