"""GPU parity of the fused combine tail (combine + residual add + RMSNorm) and
of the tail alone, against the oracle.  residual_out is bit-exact; norm_out is
within 1 bf16 ulp (its sum of squares is an fp32 tree on the GPU and a
double sum in the oracle).  The fused kernel is bit-identical to the unfused
pair ep_combine + ep_add_rmsnorm."""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import GpuPath, bf16_ulp_distance, dev, host

pytestmark = pytest.mark.gpu


def tail_inputs(T, H, E, K, W, seed):
    cfg = workloads.MoEConfig("t", T=T, H=H, E=E, K=K, W=W, mask_frac=0.2, seed=seed)
    inp = workloads.moe_inputs(cfg, with_x=False)
    rng = np.random.default_rng(seed + 5)
    y = workloads.expert_outputs(cfg.cap_rows, H, seed)
    residual = workloads.bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    gamma = workloads.bf16_bits_from_f32((1 + 0.2 * rng.standard_normal(H)).astype(np.float32))
    return cfg, inp, y, residual, gamma


@pytest.mark.parametrize("H,K", [(8, 2), (264, 3), (2048, 8), (7168, 8), (16384, 16), (4096, 1)])
def test_tail_parity(H, K):
    T, E, W, eps = 96, 32, 4, 1e-6
    print("tail H", H, "K", K, flush=True)
    cfg, inp, y, residual, gamma = tail_inputs(T, H, E, K, W, H + K)
    p = oracle.plan(inp.ids, E, W, inp.active)
    want_ro, want_no = oracle.combine_add_rmsnorm(y, p.pos, inp.weights, residual, gamma, eps)
    g = GpuPath(inp.ids, E, W, inp.active)
    g.run_plan()
    ro = torch.empty((T, H), dtype=torch.int16, device="cuda")
    no = torch.empty((T, H), dtype=torch.int16, device="cuda")
    yd, wd, rd, gd = dev(y), dev(inp.weights), dev(residual), dev(gamma)
    ep.ep_combine_add_rmsnorm(yd, g.plan.pos, wd, rd, gd, eps, ro, no)
    assert (host(ro, np.uint16) == want_ro).all()
    d = bf16_ulp_distance(host(no, np.uint16), want_no)
    assert d.max() <= 1, d.max()
    assert (d == 0).mean() > 0.99
    # unfused: combine, then the tail alone -- bit-identical to the fused kernel
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ep.ep_combine(yd, g.plan.pos, wd, out)
    ro2 = torch.empty_like(ro)
    no2 = torch.empty_like(no)
    ep.ep_add_rmsnorm(out, rd, gd, eps, ro2, no2)
    assert torch.equal(ro, ro2) and torch.equal(no, no2)
    assert ep.ep_device_error() == 0


def test_tail_alone_parity():
    T, H, eps = 64, 1032, 1e-5
    rng = np.random.default_rng(4)
    x = workloads.bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32) * 3)
    residual = workloads.bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    gamma = workloads.bf16_bits_from_f32(rng.random(H).astype(np.float32) + 0.5)
    pos = np.arange(T, dtype=np.int32).reshape(T, 1)
    want_ro, want_no = oracle.combine_add_rmsnorm(x, pos, np.ones((T, 1), np.float32), residual, gamma, eps)
    ro = torch.empty((T, H), dtype=torch.int16, device="cuda")
    no = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ep.ep_add_rmsnorm(dev(x), dev(residual), dev(gamma), eps, ro, no)
    assert (host(ro, np.uint16) == want_ro).all()
    assert bf16_ulp_distance(host(no, np.uint16), want_no).max() <= 1


def test_tail_fullsize_sampled():
    cfg = workloads.WORKLOADS[2]
    print("tail full size", cfg.name, flush=True)
    inp = workloads.moe_inputs(cfg)
    want = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    g = GpuPath(inp.ids, cfg.E, cfg.W, inp.active)
    g.run_plan()
    ex = torch.empty((cfg.cap_rows, cfg.H), dtype=torch.int16, device="cuda")
    ep.ep_dispatch(dev(inp.x), g.plan.pos, ex)
    rng = np.random.default_rng(12)
    residual = workloads.bf16_bits_from_f32(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))
    gamma = workloads.bf16_bits_from_f32((1 + 0.1 * rng.standard_normal(cfg.H)).astype(np.float32))
    ro = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    no = torch.empty_like(ro)
    ep.ep_combine_add_rmsnorm(ex, g.plan.pos, dev(inp.weights), dev(residual), dev(gamma), 1e-6, ro, no)
    torch.cuda.synchronize()
    toks = np.sort(rng.choice(cfg.T, 256, replace=False))
    sub = want.pos[toks].copy()
    live = sub >= 0
    sub[live] = np.arange(int(live.sum()), dtype=np.int32)
    y_sub = oracle.dispatch_bf16(inp.x[toks], sub, int(live.sum()))
    want_ro, want_no = oracle.combine_add_rmsnorm(y_sub, sub, inp.weights[toks], residual[toks], gamma, 1e-6)
    ti = dev(toks.astype(np.int64))
    assert (host(ro[ti], np.uint16) == want_ro).all()
    assert bf16_ulp_distance(host(no[ti], np.uint16), want_no).max() <= 1
