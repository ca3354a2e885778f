"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import combine_ep_plan_02_amd as ep
import oracle

DEV = "cuda"


def dev(a: np.ndarray) -> torch.Tensor:
    """Host numpy array -> device tensor holding the same bytes."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to(DEV)


def host(t: torch.Tensor, np_dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if np_dtype is not None:
        a = a.view(np_dtype)
    return a


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two arrays of bf16 bit patterns (ordered
    integer mapping; +0 and -0 are 0 apart)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))


class GpuPath:
    """Plan + dispatch + combine of one input set on the GPU."""

    def __init__(self, ids, E, W, active=None, with_occ=True):
        T, K = ids.shape
        self.T, self.K, self.E, self.W = T, K, E, W
        self.ids = dev(ids.astype(np.int32))
        self.active = None if active is None else dev(active.astype(np.uint8))
        self.ws = ep.alloc_workspace(T, K, E, W)
        self.plan = ep.alloc_plan(T, K, E, W, with_occ=with_occ)

    def run_plan(self, flags=0):
        ep.ep_plan(self.ids, self.E, self.W, self.plan, self.ws, self.active, flags=flags)
        return self.plan

    def plan_host(self):
        p = self.plan
        return {f: host(getattr(p, f)) for f in ("in_splits", "src_offsets", "out_splits",
                                                  "dst_offsets", "expert_counts", "expert_offsets",
                                                  "rank_offsets", "pos")} | (
            {"occ": host(p.occ)} if p.occ is not None else {})


def assert_plan_equal(got: dict, want: oracle.Plan):
    for f in ("in_splits", "src_offsets", "out_splits", "dst_offsets", "expert_counts",
              "expert_offsets", "rank_offsets", "pos", "occ"):
        if f not in got:
            continue
        g, w = got[f], getattr(want, f)
        assert g.shape == w.shape, (f, g.shape, w.shape)
        bad = np.argwhere(g != w)
        assert bad.size == 0, f"{f}: {len(bad)} mismatches, first at {bad[0].tolist()}: " \
                              f"got {g[tuple(bad[0])]}, want {w[tuple(bad[0])]}"
