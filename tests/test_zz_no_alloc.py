"""ep_plan_noalloc (the plan without a workspace, for callers that cannot
allocate device memory) against ep_plan with a workspace.

Two calls in a row on the library's static per-device array, the second
with fewer tokens (and other dimensions), each compared with ep_plan's plan
and with the oracle; both plan paths (the one-launch plan and the forced
look-back), and a look-back plan beside a one-launch plan of other
dimensions in sequence.  The size limit is refused on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import GpuPath, assert_plan_equal, host

FIELDS = ("in_splits", "src_offsets", "out_splits", "dst_offsets", "expert_counts",
          "expert_offsets", "rank_offsets", "pos", "occ")


def say(*a):
    print(*a, flush=True)


def plans_of(ids, E, W, active, flags):
    """(ep_plan's plan, ep_plan_noalloc's plan) on the same inputs."""
    g = GpuPath(ids, E, W, active)
    g.run_plan(flags=flags)
    T, K = ids.shape
    p = ep.alloc_plan(T, K, E, W)
    for f in FIELDS:
        getattr(p, f).fill_(-9)
    ep.ep_plan_noalloc(g.ids, E, W, p, g.active, flags=flags)
    torch.cuda.synchronize()
    return g.plan_host(), {f: host(getattr(p, f)) for f in FIELDS}


def compare(ids, E, W, active, flags):
    with_ws, no_ws = plans_of(ids, E, W, active, flags)
    for f in FIELDS:
        assert np.array_equal(with_ws[f], no_ws[f]), f
    assert_plan_equal(no_ws, oracle.plan(ids, E, W, active))


@pytest.mark.gpu
@pytest.mark.parametrize("flags", [0, ep.EP_PLAN_LOOKBACK], ids=["one-launch", "look-back"])
def test_two_calls_in_a_row_match_ep_plan(flags):
    say("ep_plan_noalloc, flags", flags)
    assert ep.ep_device_error() == 0
    big = workloads.WORKLOADS[4]                 # T=16384, K=8, E=256, W=32, 25% masked
    inp = workloads.moe_inputs(big, with_x=False)
    compare(inp.ids, big.E, big.W, inp.active, flags)
    rng = np.random.default_rng(5)
    T, K, E, W = 2048, 6, 64, 8                  # the second call: fewer tokens
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    active = (rng.random(T) >= 0.1).astype(np.uint8)
    compare(ids, E, W, active, flags)
    assert ep.ep_device_error() == 0


@pytest.mark.gpu
def test_paths_and_sizes_alternate():
    say("ep_plan_noalloc, alternating paths and sizes")
    rng = np.random.default_rng(6)
    shapes = [(8192, 8, 256, 16, 0), (131072, 8, 64, 8, 0), (64, 2, 8, 2, 0),
              (8448, 16, 1024, 2, 0), (4096, 6, 64, 8, ep.EP_PLAN_LOOKBACK), (8192, 8, 256, 16, 0)]
    for T, K, E, W, flags in shapes:
        ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
        compare(ids, E, W, None, flags)
    assert ep.ep_device_error() == 0


def test_size_beyond_the_static_scratch_is_refused():
    """The look-back state past the static array is refused on the host
    (T*K = 2^24 copies with E = 1024: 8192 tiles)."""
    T, K, E, W = 1 << 21, 8, 1024, 1
    p = ep._PlanT()
    for i, (f, _) in enumerate(ep._PlanT._fields_):
        setattr(p, f, (1 << 40) + (i + 1) * (1 << 34))
    o = ep._PlanOpts()
    o.flags = ep.EP_PLAN_LOOKBACK
    rc = ep.lib.ep_plan_noalloc(T, K, E, W, 1 << 40, None, ctypes.byref(o), ctypes.byref(p), None)
    assert rc == ep.EP_ERR_UNSUPPORTED
    assert b"static scratch" in ep.lib.ep_last_error()

