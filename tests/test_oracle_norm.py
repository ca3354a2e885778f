"""Pins for the oracle's fused combine tail (combine + residual add + RMSNorm)
and its one-step double -> bf16 rounding.

* The double -> bf16 rounding is checked against exact rational arithmetic
  (Python fractions): the result is a nearest bf16 value, ties to the even
  pattern.
* residual_out equals torch's CPU bf16 add of the residual and the combined
  rows (the unfused sequence: combine, then add).
* norm_out equals torch's float64 RMSNorm of residual_out times gamma,
  rounded to the nearest bf16 (checked exactly), and meets closed forms: a
  constant row with eps = 0 normalises to +-gamma; scaling the row by a power
  of two does not change it.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads


def bf16_value(bits):
    return float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0])


def nearest_bf16_exact(v: float) -> int:
    """Nearest bf16 pattern by exact comparison, ties to even (finite range)."""
    if v == 0:
        return 0x8000 if np.signbit(v) else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    f = np.float32(abs(v))
    if Fraction(float(f)) > a:
        f = np.nextafter(f, np.float32(0))
    lo = int(np.array([f], np.float32).view(np.uint32)[0]) >> 16
    hi = lo + 1
    dl, dh = a - Fraction(bf16_value(lo)), Fraction(bf16_value(hi)) - a
    pick = lo if dl < dh else hi if dl > dh else (hi if lo & 1 else lo)
    return sign | pick


def test_f64_to_bf16_is_nearest_even():
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    # exact halfway points and their neighbours
    for b in rng.integers(0x0080, 0x7F00, 500):
        mid = (bf16_value(b) + bf16_value(b + 1)) / 2
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid]
    vals += [1e-40, 2.0 ** -134, 2.0 ** -133 * 1.5, 0.0, -0.0]
    for v in vals:
        assert oracle.f64_to_bf16_rne(v) == nearest_bf16_exact(float(v)), v


def tail_case(T=48, H=96, E=16, K=4, W=4, seed=3):
    cfg = workloads.MoEConfig("n", T=T, H=H, E=E, K=K, W=W, mask_frac=0.2, seed=seed)
    inp = workloads.moe_inputs(cfg)
    p = oracle.plan(inp.ids, E, W, inp.active)
    y = workloads.expert_outputs(cfg.cap_rows, H, seed)
    rng = np.random.default_rng(seed + 1)
    residual = workloads.bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    gamma = workloads.bf16_bits_from_f32((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    return inp, p, y, residual, gamma


def to_t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("eps", [1e-6, 1e-2, 0.0])
def test_tail_matches_torch_unfused(eps):
    inp, p, y, residual, gamma = tail_case()
    ro, no = oracle.combine_add_rmsnorm(y, p.pos, inp.weights, residual, gamma, eps)
    c = oracle.combine(y, p.pos, inp.weights)
    want_ro = (to_t(residual).float() + to_t(c).float()).to(torch.bfloat16)
    assert (ro == want_ro.view(torch.int16).numpy().view(np.uint16)).all()
    h = to_t(ro).double()
    ref = h * torch.rsqrt((h * h).mean(dim=1, keepdim=True) + eps) * to_t(gamma).double()
    want_no = np.array([[nearest_bf16_exact(float(v)) for v in row] for row in ref.numpy()], np.uint16)
    # the same double computation up to the last bits of rsqrt: at most one
    # bf16 step apart, and equal almost everywhere
    diff = np.abs(no.astype(np.int32) - want_no.astype(np.int32))
    assert diff.max() <= 1
    assert (diff == 0).mean() > 0.999
    # a wrong mean (H - 1) is caught
    bad = h * torch.rsqrt((h * h).sum(dim=1, keepdim=True) / (h.shape[1] - 1) + eps)
    bad = (bad * to_t(gamma).double()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bad != no).mean() > 0.05


def test_constant_row_normalises_to_gamma():
    T, H = 4, 64
    residual = np.zeros((T, H), np.uint16)
    for t, val in enumerate([1.5, -3.0, 1024.0, 2.0 ** -20]):
        residual[t] = workloads.bf16_bits_from_f32(np.full(H, val, np.float32))
    gamma = workloads.bf16_bits_from_f32(np.linspace(-2, 2, H, dtype=np.float32))
    y = np.zeros((1, H), np.uint16)
    pos = np.full((T, 1), -1, np.int32)                     # no live copy: c = +0
    ro, no = oracle.combine_add_rmsnorm(y, pos, np.zeros((T, 1), np.float32), residual, gamma, 0.0)
    assert (ro == residual).all()
    for t in range(T):
        s = np.sign(bf16_value(residual[t, 0]))
        want = workloads.bf16_bits_from_f32((s * np.array([bf16_value(g) for g in gamma])).astype(np.float32))
        assert (no[t] == want).all()


def test_scale_invariance():
    inp, p, y, residual, gamma = tail_case(seed=11)
    pos = np.full_like(p.pos, -1)
    _, no1 = oracle.combine_add_rmsnorm(y, pos, inp.weights, residual, gamma, 0.0)
    doubled = workloads.bf16_bits_from_f32(
        np.array([[bf16_value(b) * 2 for b in row] for row in residual], np.float32))
    _, no2 = oracle.combine_add_rmsnorm(y, pos, inp.weights, doubled, gamma, 0.0)
    assert (no1 == no2).all()
