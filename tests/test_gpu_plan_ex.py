"""GPU parity of the plan options a grouped expert GEMM consumes (per-copy
mask, expert padding, expert token numbers) and of the gate weights carried
to the expanded rows, against the oracle, bit for bit, on both plan paths."""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import assert_plan_equal, dev, host

pytestmark = pytest.mark.gpu

CASES = [
    # T, K, E, W, align, pad_empty, copy_mask, token_nums_type
    (1024, 4, 32, 4, 4, False, False, 1),
    (1024, 4, 32, 4, 16, True, True, 0),
    (3000, 5, 60, 6, 128, True, True, 1),    # ragged tiles, large unit
    (64, 16, 1024, 4, 8, True, False, 0),    # most experts empty
    (8448, 16, 1024, 2, 32, False, True, 1),  # look-back path (66 tiles x 1024 experts)
    (8448, 16, 1024, 2, 1, False, True, 0),   # look-back path, mask only
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}E{c[2]}a{c[4]}{'p' if c[5] else ''}{'m' if c[6] else ''}t{c[7]}" for c in CASES])
def test_plan_options_parity(case):
    T, K, E, W, align, pad_empty, use_mask, typ = case
    print("plan options", case, flush=True)
    rng = np.random.default_rng(T + E + align)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    active = (rng.random(T) < 0.85).astype(np.uint8)
    copies = (rng.random((T, K)) < 0.7).astype(np.uint8) if use_mask else None
    want, want_etn = oracle.plan_ex(ids, E, W, active, copies, major_align=align,
                                    pad_empty=pad_empty, token_nums_type=typ)
    ws = ep.alloc_workspace(T, K, E, W)
    plan = ep.alloc_plan(T, K, E, W)
    etn = torch.full((W, E // W), -5, dtype=torch.int64, device="cuda")
    for _ in range(2):   # twice: the workspace is reused
        ep.ep_plan(dev(ids), E, W, plan, ws, dev(active),
                   active_copies=None if copies is None else dev(copies), major_align=align,
                   pad_empty_experts=pad_empty, expert_token_nums=etn, expert_token_nums_type=typ)
        got = {f: host(getattr(plan, f)) for f in ("in_splits", "src_offsets", "out_splits",
                                                    "dst_offsets", "expert_counts",
                                                    "expert_offsets", "rank_offsets", "pos", "occ")}
        assert_plan_equal(got, want)
        assert (host(etn) == want_etn).all()
    assert int(want.rank_offsets[-1]) <= ep.ep_expand_rows_bound(T, K, E, align, pad_empty)
    assert ep.ep_device_error() == 0


@pytest.mark.parametrize("fp8", [False, True])
def test_dispatch_weights_and_padded_rows(fp8):
    T, H, E, K, W, align = 512, 256, 16, 4, 4, 8
    print("dispatch weights fp8" if fp8 else "dispatch weights bf16", flush=True)
    cfg = workloads.MoEConfig("w", T=T, H=H, E=E, K=K, W=W, sigma=2.0, mask_frac=0.2, seed=77)
    inp = workloads.moe_inputs(cfg)
    want, _ = oracle.plan_ex(inp.ids, E, W, inp.active, major_align=align, pad_empty=True)
    cap = ep.ep_expand_rows_bound(T, K, E, align, True)
    ws = ep.alloc_workspace(T, K, E, W)
    plan = ep.alloc_plan(T, K, E, W)
    ep.ep_plan(dev(inp.ids), E, W, plan, ws, dev(inp.active), major_align=align,
               pad_empty_experts=True)
    assert (host(plan.pos) == want.pos).all()
    ew = torch.full((cap,), -3.0, dtype=torch.float32, device="cuda")
    if fp8:
        q = torch.full((cap, H), 0x11, dtype=torch.uint8, device="cuda")
        sc = torch.full((cap,), -1.0, dtype=torch.float32, device="cuda")
        ep.ep_dispatch(dev(inp.x), plan.pos, q, sc, out_dtype=ep.EP_FP8_E4M3FN,
                       weights=dev(inp.weights), expand_weights=ew)
        want_q, want_s = oracle.dispatch_fp8(inp.x, want.pos, cap, fill_q=0x11, fill_scale=-1.0)
        assert (host(q) == want_q).all()
        assert (host(sc).view(np.uint32) == want_s.view(np.uint32)).all()
    else:
        ex = torch.full((cap, H), 0x2222, dtype=torch.int16, device="cuda")
        ep.ep_dispatch(dev(inp.x), plan.pos, ex, weights=dev(inp.weights), expand_weights=ew)
        assert (host(ex, np.uint16) == oracle.dispatch_bf16(inp.x, want.pos, cap, fill=0x2222)).all()
    want_w = oracle.dispatch_weights(want.pos, inp.weights, cap, fill=-3.0)
    assert (host(ew).view(np.uint32) == want_w.view(np.uint32)).all()
    assert ep.ep_device_error() == 0
