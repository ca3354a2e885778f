"""Plans running beside other kernels on other streams (all at the default
priority).  The one-launch plan needs its tiles resident together and its
waits are bounded; kernels of another stream only delay some tiles' start.
Each plan must still equal the oracle's, and no stall may be flagged."""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import GpuPath, assert_plan_equal, dev

pytestmark = pytest.mark.gpu


def make(T, K, E, W, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    return ids, oracle.plan(ids, E, W)


def test_plans_beside_a_combine_and_beside_each_other():
    T, K, E, W, H = 8192, 8, 256, 16, 4096
    print("concurrent plans", flush=True)
    ids_a, want_a = make(T, K, E, W, 1)
    ids_b, want_b = make(T, K, E, W, 2)
    a = GpuPath(ids_a, E, W)
    b = GpuPath(ids_b, E, W)
    # a large combine for the other stream: T tokens x K rows of H values
    cfg = workloads.MoEConfig("c", T=T, H=H, E=E, K=K, W=W, seed=3)
    inp = workloads.moe_inputs(cfg)
    p = oracle.plan(inp.ids, E, W)
    y = dev(workloads.expert_outputs(cfg.cap_rows, H, 4))
    pos, w = dev(p.pos), dev(inp.weights)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for it in range(20):
        with torch.cuda.stream(s1):
            ep.ep_combine(y, pos, w, out)
            ep.ep_combine(y, pos, w, out)
        with torch.cuda.stream(s2):
            a.run_plan()
        torch.cuda.synchronize()
        assert_plan_equal(a.plan_host(), want_a)
        with torch.cuda.stream(s1):
            a.run_plan()
        with torch.cuda.stream(s2):
            b.run_plan()
        torch.cuda.synchronize()
        assert_plan_equal(a.plan_host(), want_a)
        assert_plan_equal(b.plan_host(), want_b)
    assert ep.ep_device_error() == 0
