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


def test_graph_replays_of_the_extensions():
    """Plan with options (per-copy mask, padding, token numbers) -> fp8
    dispatch with gate weights -> smoothed int8 dispatch -> fp8-row combine ->
    fused tail, captured once and replayed with new inputs; every output of
    every replay is checked against the oracle."""
    T, H, E, K, W, align = 512, 1024, 32, 4, 4, 8
    print("graph case: extensions", flush=True)
    rng = np.random.default_rng(7)

    def draw(seed):
        cfg = workloads.MoEConfig("g", T=T, H=H, E=E, K=K, W=W, sigma=2.0, mask_frac=0.2, seed=seed)
        inp = workloads.moe_inputs(cfg)
        copies = (np.random.default_rng(seed + 1).random((T, K)) < 0.8).astype(np.uint8)
        residual = workloads.bf16_bits_from_f32(
            np.random.default_rng(seed + 2).standard_normal((T, H)).astype(np.float32))
        return inp, copies, residual

    inp0, copies0, res0 = draw(400)
    cap = ep.ep_expand_rows_bound(T, K, E, align, True)
    smooth = dev(workloads.smooth_scales(E, H, 3))
    gamma_np = workloads.bf16_bits_from_f32((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    gamma = dev(gamma_np)
    ids, x, w, active = dev(inp0.ids), dev(inp0.x), dev(inp0.weights), dev(inp0.active)
    copies, residual = dev(copies0), dev(res0)
    ws = ep.alloc_workspace(T, K, E, W)
    plan = ep.alloc_plan(T, K, E, W)
    etn = torch.zeros((W, E // W), dtype=torch.int64, device="cuda")
    q8 = torch.zeros((cap, H), dtype=torch.uint8, device="cuda")
    s8 = torch.zeros((cap,), dtype=torch.float32, device="cuda")
    ew = torch.zeros((cap,), dtype=torch.float32, device="cuda")
    qi = torch.zeros((cap, H), dtype=torch.uint8, device="cuda")
    si = torch.zeros((cap,), dtype=torch.float32, device="cuda")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    ro = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    no = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    ybf = torch.zeros((cap, H), dtype=torch.int16, device="cuda")   # bf16 expert rows for the tail

    def step():
        ep.ep_plan(ids, E, W, plan, ws, active, active_copies=copies, major_align=align,
                   pad_empty_experts=True, expert_token_nums=etn, expert_token_nums_type=0)
        ep.ep_dispatch(x, plan.pos, q8, s8, out_dtype=ep.EP_FP8_E4M3FN, weights=w, expand_weights=ew)
        ep.ep_dispatch_smooth(x, ids, plan.pos, smooth, qi, si, out_dtype=ep.EP_INT8)
        ep.ep_combine_quant(q8, s8, plan.pos, w, out, code_dtype=ep.EP_FP8_E4M3FN)
        ep.ep_dispatch(x, plan.pos, ybf)
        ep.ep_combine_add_rmsnorm(ybf, plan.pos, w, residual, gamma, 1e-6, ro, no)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    sm_np = workloads.smooth_scales(E, H, 3)
    for rep in range(3):
        inp, cp, res = draw(500 + rep)
        ids.copy_(dev(inp.ids))
        x.copy_(dev(inp.x))
        w.copy_(dev(inp.weights))
        active.copy_(dev(inp.active))
        copies.copy_(dev(cp))
        residual.copy_(dev(res))
        graph.replay()
        torch.cuda.synchronize()
        want, want_etn = oracle.plan_ex(inp.ids, E, W, inp.active, cp, major_align=align,
                                        pad_empty=True, token_nums_type=0)
        assert (host(plan.pos) == want.pos).all()
        assert (host(etn) == want_etn).all()
        live = want.pos >= 0
        rows = want.pos[live]
        wq, wsc = oracle.dispatch_quant(inp.x, inp.ids, want.pos, E, oracle.Q_FP8, cap)
        assert (host(q8)[rows] == wq[rows]).all()
        assert (host(s8)[rows].view(np.uint32) == wsc[rows].view(np.uint32)).all()
        assert (host(ew)[rows] == inp.weights[live]).all()
        wiq, wis = oracle.dispatch_quant(inp.x, inp.ids, want.pos, E, oracle.Q_INT8, cap, sm_np)
        assert (host(qi)[rows] == wiq[rows]).all()
        assert (host(si)[rows].view(np.uint32) == wis[rows].view(np.uint32)).all()
        want_out = oracle.combine_quant(wq, oracle.Q_FP8, wsc, want.pos, inp.weights)
        assert (bf16_ulp_distance(host(out, np.uint16), want_out) == 0).all()
        ybf_np = oracle.dispatch_bf16(inp.x, want.pos, cap)
        want_ro, want_no = oracle.combine_add_rmsnorm(ybf_np, want.pos, inp.weights, res,
                                                      gamma_np, 1e-6)
        assert (host(ro, np.uint16) == want_ro).all()
        assert bf16_ulp_distance(host(no, np.uint16), want_no).max() <= 1
        # eager work of the program between replays
        ep.ep_plan(dev(draw(600 + rep)[0].ids), E, W, ep.alloc_plan(T, K, E, W), ep.alloc_workspace(T, K, E, W))
        torch.cuda.synchronize()
    assert ep.ep_device_error() == 0
