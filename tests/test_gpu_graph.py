"""Graph capture: plan -> dispatch -> combine recorded once into a HIP graph
(through torch.cuda.CUDAGraph) and replayed with new inputs copied into the
captured buffers between replays, eager work of the program in between.
Every replay is checked against the oracle: the library enqueues only
kernels (no memset, no allocation, no host read-back), and the fused plan
keeps its descriptor epoch in the workspace, so a replay never reads the
previous replay's counts."""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import assert_plan_equal, bf16_ulp_distance, dev, host

pytestmark = pytest.mark.gpu


def inputs(T, H, E, K, W, seed):
    cfg = workloads.MoEConfig("g", T=T, H=H, E=E, K=K, W=W, mask_frac=0.2, seed=seed)
    return workloads.moe_inputs(cfg)


@pytest.mark.parametrize("shape", [(1024, 512, 32, 4, 4), (8448, 16, 1024, 16, 2)],
                         ids=["fused-plan", "look-back-plan"])
def test_graph_replays_match_oracle(shape):
    T, H, E, K, W = shape
    print("graph case", shape, flush=True)
    first = inputs(T, H, E, K, W, 100)
    ids = dev(first.ids)
    x = dev(first.x)
    w = dev(first.weights)
    active = dev(first.active)
    ws = ep.alloc_workspace(T, K, E, W)
    plan = ep.alloc_plan(T, K, E, W)
    cap = T * K
    ex = torch.zeros((cap, H), dtype=torch.int16, device="cuda")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")

    def step():
        ep.ep_plan(ids, E, W, plan, ws, active)
        ep.ep_dispatch(x, plan.pos, ex)
        ep.ep_combine(ex, plan.pos, w, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                      # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    other_ws = ep.alloc_workspace(T, K, E, W)
    other_plan = ep.alloc_plan(T, K, E, W)
    for rep in range(4):
        inp = inputs(T, H, E, K, W, 200 + rep)
        ids.copy_(dev(inp.ids))
        x.copy_(dev(inp.x))
        w.copy_(dev(inp.weights))
        active.copy_(dev(inp.active))
        graph.replay()
        torch.cuda.synchronize()
        want = oracle.plan(inp.ids, E, W, inp.active)
        got = {f: host(getattr(plan, f)) for f in ("in_splits", "src_offsets", "out_splits",
                                                    "dst_offsets", "expert_counts",
                                                    "expert_offsets", "rank_offsets", "pos", "occ")}
        assert_plan_equal(got, want)
        want_ex = oracle.dispatch_bf16(inp.x, want.pos, cap)
        N = want.n_rows
        assert (host(ex[:N], np.uint16) == want_ex[:N]).all()
        want_out = oracle.combine(want_ex, want.pos, inp.weights)
        assert (bf16_ulp_distance(host(out, np.uint16), want_out) == 0).all()
        # the program's own eager work between replays, on another workspace
        ep.ep_plan(dev(inputs(T, H, E, K, W, 300 + rep).ids), E, W, other_plan, other_ws)
        torch.cuda.synchronize()
    assert ep.ep_device_error() == 0
