"""Pins for the oracle's quantisation variants: int8 per-token dynamic
quantisation, per-expert smoothing scales before quantisation (the CANN
dispatch page's scalesOptional with quantMode 2), and the combine reading
quantised expert rows (its commQuantMode).

* int8 codes equal torch's round-half-to-even of the quotients, clamped.
* Smoothing by all-ones equals plain per-token quantisation; smoothing by a
  power of two per expert leaves the codes unchanged and scales the scale
  by that power (exact).  General smoothing equals torch's float32 product
  followed by the plain quantisation of that row.
* The quantised combine with unit scales equals the bf16 combine of the
  decoded values (fp8 and int8 values are exact in bf16); power-of-two
  scales scale the result exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def test_int8_encode_matches_torch_round():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 60,
                        np.arange(-130, 130, 0.5, dtype=np.float32),
                        np.array([126.5, -126.5, 127.49, 1e9, -1e9, 0.0, -0.0], np.float32)])
    want = torch.round(torch.from_numpy(v)).clamp(-127, 127).to(torch.int8).numpy()
    got = np.array([oracle.int8_encode(float(a)) for a in v], np.int8)
    assert (got == want).all()


def case(T=40, H=64, E=8, K=3, W=2, seed=2, sigma=2.0):
    cfg = workloads.MoEConfig("q", T=T, H=H, E=E, K=K, W=W, sigma=sigma, mask_frac=0.2, seed=seed)
    inp = workloads.moe_inputs(cfg)
    p = oracle.plan(inp.ids, E, W, inp.active)
    return cfg, inp, p


def test_fp8_without_smoothing_equals_plain_dispatch():
    cfg, inp, p = case()
    q, s = oracle.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, oracle.Q_FP8, cfg.cap_rows)
    q2, s2 = oracle.dispatch_fp8(inp.x, p.pos, cfg.cap_rows)
    assert (q == q2).all() and (s.view(np.uint32) == s2.view(np.uint32)).all()
    ones = np.ones((cfg.E, cfg.H), np.float32)
    q3, s3 = oracle.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, oracle.Q_FP8, cfg.cap_rows, ones)
    assert (q3 == q2).all() and (s3.view(np.uint32) == s2.view(np.uint32)).all()


@pytest.mark.parametrize("qtype", [1, 2])
def test_power_of_two_smoothing_scales_exactly(qtype):
    cfg, inp, p = case(seed=5)
    plain_q, plain_s = oracle.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, qtype, cfg.cap_rows)
    pw = (2.0 ** np.arange(-3, cfg.E - 3)).astype(np.float32)
    smooth = np.repeat(pw[:, None], cfg.H, axis=1)
    q, s = oracle.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, qtype, cfg.cap_rows, smooth)
    live = p.pos >= 0
    rows = p.pos[live]
    experts = inp.ids[live]
    assert (q[rows] == plain_q[rows]).all()
    assert (s[rows] == plain_s[rows] * pw[experts]).all()


@pytest.mark.parametrize("qtype", [1, 2])
def test_general_smoothing_is_product_then_plain_quant(qtype):
    cfg, inp, p = case(seed=7, H=48)
    rng = np.random.default_rng(3)
    smooth = (0.5 + rng.random((cfg.E, cfg.H))).astype(np.float32)
    q, s = oracle.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, qtype, cfg.cap_rows, smooth)
    xf = (inp.x.astype(np.uint32) << 16).view(np.float32)
    qmax = np.float32(448.0 if qtype == 1 else 127.0)
    for t in range(cfg.T):
        for k in range(cfg.K):
            r = p.pos[t, k]
            if r < 0:
                continue
            xs = (torch.from_numpy(xf[t]) * torch.from_numpy(smooth[inp.ids[t, k]])).numpy()
            scale = np.float32(np.abs(xs).max()) / qmax
            assert s[r] == scale
            quo = (torch.from_numpy(xs) / torch.tensor(scale)).numpy() if scale != 0 else np.zeros_like(xs)
            if qtype == 1:
                want = torch.from_numpy(quo).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            else:
                want = torch.round(torch.from_numpy(quo)).clamp(-127, 127).to(torch.int8).numpy().view(np.uint8)
            assert (q[r] == want).all(), (t, k)


@pytest.mark.parametrize("qtype", [1, 2])
def test_quant_combine_unit_and_power_of_two_scales(qtype):
    cfg, inp, p = case(seed=9)
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(cfg.cap_rows, cfg.H)).astype(np.uint8)
    if qtype == 1:
        codes[(codes & 0x7F) == 0x7F] = 0x10                 # no NaN codes
        dec = np.array([oracle.e4m3fn_decode(c) for c in range(256)], np.float32)[codes]
    else:
        codes[codes == 0x80] = 0                             # -128 is not a code
        dec = codes.view(np.int8).astype(np.float32)
    ones = np.ones(cfg.cap_rows, np.float32)
    out = oracle.combine_quant(codes, qtype, ones, p.pos, inp.weights)
    ref = oracle.combine(workloads.bf16_bits_from_f32(dec), p.pos, inp.weights)   # dec exact in bf16
    assert (out == ref).all()
    fours = np.full(cfg.cap_rows, 4.0, np.float32)
    out4 = oracle.combine_quant(codes, qtype, fours, p.pos, inp.weights)
    ref4 = oracle.combine(workloads.bf16_bits_from_f32(dec * 4), p.pos, inp.weights)
    assert (out4 == ref4).all()


@pytest.mark.parametrize("qtype", [1, 2])
def test_quant_combine_uses_each_rows_own_scale(qtype):
    """Per-row power-of-two scales (exact in bf16 with the decoded values):
    the result equals the bf16 combine of decode(code) * scale[row], so a
    scale taken from another row (the token's, or a neighbour's) fails."""
    cfg, inp, p = case(seed=13)
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, size=(cfg.cap_rows, cfg.H)).astype(np.uint8)
    if qtype == 1:
        codes[(codes & 0x7F) == 0x7F] = 0x10
        dec = np.array([oracle.e4m3fn_decode(c) for c in range(256)], np.float32)[codes]
    else:
        codes[codes == 0x80] = 0
        dec = codes.view(np.int8).astype(np.float32)
    scales = (2.0 ** rng.integers(-6, 7, cfg.cap_rows)).astype(np.float32)
    out = oracle.combine_quant(codes, qtype, scales, p.pos, inp.weights)
    ref = oracle.combine(workloads.bf16_bits_from_f32(dec * scales[:, None]), p.pos, inp.weights)
    assert (out == ref).all()
    shifted = np.roll(scales, 1)
    assert (oracle.combine_quant(codes, qtype, shifted, p.pos, inp.weights) != ref).any()
