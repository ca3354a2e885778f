"""Seeded random shapes through the whole path, each checked against the
oracle: T, K, E, W (W dividing E and T), H, token and per-copy masks,
alignment padding, and bf16 / fp8 / int8 rows.  The shapes reach both plan
paths (tiles of one launch exchanging counts, and the look-back for larger
grids), ragged tiles, E up to 1024, K up to 16 and tiny rows."""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import assert_plan_equal, bf16_ulp_distance, dev, host

pytestmark = pytest.mark.gpu


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    W = int(rng.choice([1, 2, 3, 4, 8, 16]))
    E = W * int(rng.integers(1, max(2, 1024 // W) + 1))
    E = min(E, 1024 - (1024 % W))
    K = int(rng.integers(1, 17))
    Tw = int(rng.integers(1, 600))
    H = int(16 * rng.integers(1, 65))                # up to 1024
    if seed % 5 == 0:
        Tw = int(rng.integers(2000, 6000))           # more tiles: look-back for large E
        H = int(16 * rng.integers(1, 5))
    T = W * Tw
    mask = float(rng.choice([0.0, 0.0, 0.3, 0.9]))
    copy_mask = bool(rng.random() < 0.3)
    align = int(rng.choice([1, 1, 1, 4, 16]))
    rows = ["bf16", "fp8", "int8"][seed % 3]
    return dict(T=T, K=K, E=E, W=W, H=H, mask=mask, copy_mask=copy_mask, align=align, rows=rows)


CASES = list(range(24))


@pytest.mark.parametrize("seed", CASES)
def test_random_shape(seed):
    c = draw_case(seed)
    print("random shape", seed, c, flush=True)
    T, K, E, W, H = c["T"], c["K"], c["E"], c["W"], c["H"]
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids[rng.random((T, K)) < 0.01] = E + 3               # a few invalid ids: dropped and flagged
    active = (rng.random(T) >= c["mask"]).astype(np.uint8) if c["mask"] > 0 else None
    copies = (rng.random((T, K)) < 0.7).astype(np.uint8) if c["copy_mask"] else None
    x = workloads.bf16_bits_from_f32((2.0 * rng.standard_normal((T, H))).astype(np.float32))
    w = rng.random((T, K)).astype(np.float32)
    # a copy with an invalid id is not live: the reference masks it out
    live_mask = (ids < E).astype(np.uint8) if copies is None else (copies * (ids < E)).astype(np.uint8)
    want, _ = oracle.plan_ex(np.where(ids < E, ids, 0).astype(np.int32), E, W, active, live_mask,
                             major_align=c["align"])
    cap = ep.ep_expand_rows_bound(T, K, E, c["align"], False)
    ws = ep.alloc_workspace(T, K, E, W)
    plan = ep.alloc_plan(T, K, E, W)
    ep.ep_device_error()
    ep.ep_plan(dev(ids), E, W, plan, ws, None if active is None else dev(active),
               active_copies=None if copies is None else dev(copies), major_align=c["align"])
    got = {f: host(getattr(plan, f)) for f in ("in_splits", "src_offsets", "out_splits", "dst_offsets",
                                               "expert_counts", "expert_offsets", "rank_offsets",
                                               "pos", "occ")}
    assert_plan_equal(got, want)
    flagged = ep.ep_device_error()
    tok_on = (active if active is not None else np.ones(T, np.uint8))[:, None] != 0
    copy_on = (copies if copies is not None else np.ones((T, K), np.uint8)) != 0
    if ((ids >= E) & tok_on & copy_on).any():
        assert flagged & ep.EP_DEVERR_BAD_EXPERT
    else:
        assert flagged == 0
    N = int(want.rank_offsets[-1])
    pos_d = plan.pos
    live = want.pos >= 0
    rows = want.pos[live]
    if c["rows"] == "bf16":
        ex = torch.full((cap, H), 0x1357, dtype=torch.int16, device="cuda")
        ep.ep_dispatch(dev(x), pos_d, ex)
        want_ex = oracle.dispatch_bf16(x, want.pos, cap, fill=0x1357)
        assert (host(ex, np.uint16) == want_ex).all()
        out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        ep.ep_combine(ex, pos_d, dev(w), out)
        want_out = oracle.combine(want_ex, want.pos, w)
    else:
        dt, oq = (ep.EP_FP8_E4M3FN, oracle.Q_FP8) if c["rows"] == "fp8" else (ep.EP_INT8, oracle.Q_INT8)
        q = torch.full((cap, H), 0x5A, dtype=torch.uint8, device="cuda")
        sc = torch.full((cap,), -1.0, dtype=torch.float32, device="cuda")
        ep.ep_dispatch(dev(x), pos_d, q, sc, out_dtype=dt)
        want_q, want_s = oracle.dispatch_quant(x, np.where(ids < E, ids, 0), want.pos, E, oq, cap,
                                               fill_q=0x5A, fill_scale=-1.0)
        assert (host(q) == want_q).all()
        assert (host(sc).view(np.uint32) == want_s.view(np.uint32)).all()
        out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        ep.ep_combine_quant(q, sc, pos_d, dev(w), out, code_dtype=dt)
        want_out = oracle.combine_quant(want_q, oq, want_s, want.pos, w)
    assert (bf16_ulp_distance(host(out, np.uint16), want_out) == 0).all()
    assert rows.size == int(live.sum()) and N >= rows.size
    assert ep.ep_device_error() == 0
