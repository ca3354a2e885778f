"""The sliced, multi-threaded oracle runner used by the full-size GPU parity
tests gives exactly what the serial oracle gives on the whole input."""
import numpy as np

import oracle
import workloads
import _oracle_slices as par


def test_slices_match_the_serial_oracle():
    cfg = workloads.MoEConfig("slices_T512_H256_E16_K4_W4_mask", T=512, H=256, E=16, K=4, W=4,
                              sigma=3.0, mask_frac=0.25, seed=11)
    inp = workloads.moe_inputs(cfg)
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    cap = cfg.cap_rows
    assert np.array_equal(par.dispatch_bf16(inp.x, p.pos, cap, 0x7777),
                          oracle.dispatch_bf16(inp.x, p.pos, cap, fill=0x7777))
    q, s = par.dispatch_fp8(inp.x, p.pos, cap, 0x33, -1.0)
    wq, ws = oracle.dispatch_fp8(inp.x, p.pos, cap, fill_q=0x33, fill_scale=-1.0)
    assert np.array_equal(q, wq) and np.array_equal(s.view(np.uint32), ws.view(np.uint32))
    y = workloads.expert_outputs(cap, cfg.H, 5)
    assert np.array_equal(par.combine(y, p.pos, inp.weights), oracle.combine(y, p.pos, inp.weights))


def test_quant_and_tail_slices_match_the_serial_oracle():
    cfg = workloads.MoEConfig("slices_T384_H512_E24_K6_W4_mask", T=384, H=512, E=24, K=6, W=4,
                              sigma=3.0, mask_frac=0.25, seed=12)
    inp = workloads.moe_inputs(cfg)
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    cap = cfg.cap_rows
    smooth = workloads.smooth_scales(cfg.E, cfg.H, cfg.seed)
    for qt in (oracle.Q_FP8, oracle.Q_INT8):
        for sm in (None, smooth):
            q, s = par.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, qt, cap, sm, 0x33, -1.0)
            wq, ws = oracle.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, qt, cap, sm, fill_q=0x33,
                                           fill_scale=-1.0)
            assert np.array_equal(q, wq) and np.array_equal(s.view(np.uint32), ws.view(np.uint32))
        assert np.array_equal(par.combine_quant(wq, qt, ws, p.pos, inp.weights),
                              oracle.combine_quant(wq, qt, ws, p.pos, inp.weights))
    y = workloads.expert_outputs(cap, cfg.H, 6)
    res = workloads.expert_outputs(cfg.T, cfg.H, 7)
    gamma = workloads.expert_outputs(1, cfg.H, 8)[0]
    ro, no = par.combine_add_rmsnorm(y, p.pos, inp.weights, res, gamma, 1e-6)
    wro, wno = oracle.combine_add_rmsnorm(y, p.pos, inp.weights, res, gamma, 1e-6)
    assert np.array_equal(ro, wro) and np.array_equal(no, wno)
