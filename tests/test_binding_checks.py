"""The Python binding refuses tensors smaller than the kernels address, before
any library call (the C ABI sees only pointers and the dimensions, so it
cannot check a buffer's size).  Host-only: the tensors here are CPU tensors,
and every case fails on its size before the device check."""
import pytest
import torch

import combine_ep_plan_02_amd as ep


def i64(*shape):
    return torch.zeros(shape, dtype=torch.int64)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def plan(T, K, E, W, **smaller):
    ne = E // W
    fields = dict(in_splits=i64(W, E), src_offsets=i64(W, E), out_splits=i64(W, ne, W),
                  dst_offsets=i64(W, E), expert_counts=i64(E), expert_offsets=i64(E),
                  rank_offsets=i64(W + 1), pos=i32(T, K), occ=i32(T, K))
    for f, shape in smaller.items():
        fields[f] = torch.zeros(shape, dtype=fields[f].dtype)
    return ep.Plan(**fields)


@pytest.mark.parametrize("field,shape", [("in_splits", (3, 8)), ("out_splits", (4, 2, 3)),
                                         ("rank_offsets", (4,)), ("pos", (63, 2)), ("occ", (1,)),
                                         ("expert_counts", (7,))])
def test_plan_outputs_too_small(field, shape):
    T, K, E, W = 64, 2, 8, 4
    with pytest.raises(ValueError, match=field):
        ep.ep_plan(i32(T, K), E, W, plan(T, K, E, W, **{field: shape}), torch.zeros(1 << 16, dtype=torch.uint8))


def test_plan_options_too_small():
    T, K, E, W = 64, 2, 8, 4
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="active"):
        ep.ep_plan(i32(T, K), E, W, plan(T, K, E, W), ws, torch.zeros(63, dtype=torch.uint8))
    with pytest.raises(ValueError, match="active_copies"):
        ep.ep_plan(i32(T, K), E, W, plan(T, K, E, W), ws, active_copies=torch.zeros(T, dtype=torch.uint8))
    with pytest.raises(ValueError, match="expert_token_nums"):
        ep.ep_plan(i32(T, K), E, W, plan(T, K, E, W), ws, expert_token_nums=i64(E - 1))


def test_dispatch_side_buffers_too_small():
    T, K, H, cap = 16, 2, 32, 40
    x = torch.zeros((T, H), dtype=torch.int16)
    pos = i32(T, K)
    q = torch.zeros((cap, H), dtype=torch.uint8)
    with pytest.raises(ValueError, match="expand_scales"):
        ep.ep_dispatch(x, pos, q, torch.zeros(cap - 1), out_dtype=ep.EP_FP8_E4M3FN)
    ex = torch.zeros((cap, H), dtype=torch.int16)
    with pytest.raises(ValueError, match="weights"):
        ep.ep_dispatch(x, pos, ex, weights=torch.zeros(T * K - 1), expand_weights=torch.zeros(cap))
    with pytest.raises(ValueError, match="expand_weights"):
        ep.ep_dispatch(x, pos, ex, weights=torch.zeros(T, K), expand_weights=torch.zeros(cap - 1))
    with pytest.raises(ValueError, match="expand_scales"):
        ep.ep_dispatch_smooth(x, pos, pos, torch.zeros(4, H), q, torch.zeros(cap - 1))


def test_splits_plan_too_small():
    W, R = 4, 8
    sp = ep.SplitsPlan(i64(W, W), i64(W, W), i64(W, W - 1), i64(W + 1))
    inp = torch.zeros((W, R, 8), dtype=torch.int16)
    out = torch.zeros((W * R, 8), dtype=torch.int16)
    with pytest.raises(ValueError, match="dst_offsets"):
        ep.ep_plan_splits(i64(W, W), sp)
    with pytest.raises(ValueError, match="dst_offsets"):
        ep.ep_dispatch_splits(inp, sp, out)
    with pytest.raises(ValueError, match="dst_offsets"):
        ep.ep_all_to_all_splits(i64(W, W), inp, out, sp)
    with pytest.raises(ValueError, match="in_splits"):
        ep.ep_plan_splits(i64(W, W - 1), ep.alloc_splits_plan(W, device="cpu"))


def test_right_sizes_reach_the_device_check():
    # correctly sized CPU tensors pass the size checks and stop at the device check
    T, K, E, W = 64, 2, 8, 4
    with pytest.raises(ValueError, match="must live on the GPU"):
        ep.ep_plan(i32(T, K), E, W, plan(T, K, E, W), torch.zeros(1 << 16, dtype=torch.uint8))


def test_plan_is_frozen():
    p = plan(64, 2, 8, 4)
    with pytest.raises(Exception):
        p.pos = i32(64, 2)
