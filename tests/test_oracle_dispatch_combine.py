"""Pins for the oracle's dispatch (bf16 and per-token fp8) and weighted combine.

Each check is fixed independently of oracle/ep_oracle.c:
  * bf16 dispatch: the expandX rows equal x gathered by a stable argsort of the
    live expert ids (the layout test_all_to_all_v_2d_index_push of the PyTorch
    compare view ciflow/h100-symm-mem/166772 compares against), rows past N
    keep their sentinel;
  * fp8: closed-form properties of per-token scaling (the amax element maps to
    +-448, relative error bounds of E4M3FN, the scale is the fp32 quotient
    amax / 448 computed by numpy) and torch's float8_e4m3fn cast on the
    quotients x / scale;
  * combine: with unit weights and y = the dispatched rows the result is
    bf16(K_live * x) exactly; the association probe 2^24, 1, -2^24 (flashinfer
    PR #4358, numerical-contract tests) exposes the summation order; an
    inactive token gives +0 rows; the result lies within the fp32
    accumulation bound of the exact sum.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def small_inputs(T=48, H=64, E=8, K=3, W=4, mask_frac=0.3, sigma=1.0, seed=11):
    cfg = workloads.MoEConfig("t", T=T, H=H, E=E, K=K, W=W, sigma=sigma, mask_frac=mask_frac,
                              seed=seed)
    return cfg, workloads.moe_inputs(cfg)


def test_bf16_dispatch_matches_stable_argsort_gather():
    cfg, inp = small_inputs()
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    ex = oracle.dispatch_bf16(inp.x, p.pos, cfg.cap_rows, fill=0xFFFF)
    live = (p.pos >= 0).reshape(-1)
    keys = np.where(live, inp.ids.reshape(-1), cfg.E)
    order = np.argsort(keys, kind="stable")[: p.n_rows]
    expected = inp.x[order // cfg.K]
    assert (ex[: p.n_rows] == expected).all()
    assert (ex[p.n_rows:] == 0xFFFF).all()


def test_fp8_dispatch_closed_form():
    cfg, inp = small_inputs(H=128, sigma=3.0)
    # one all-zero token and one token of subnormal-range magnitudes
    inp.x[0] = 0
    inp.x[1] = workloads.bf16_bits_from_f32(np.full(cfg.H, 1e-39, np.float32))
    if inp.active is not None:
        inp.active[:2] = 1
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    q, sc = oracle.dispatch_fp8(inp.x, p.pos, cfg.cap_rows, fill_q=0x55, fill_scale=-1.0)
    xf = bf16_to_f64(inp.x)
    dec = np.array([oracle.e4m3fn_decode(c) for c in range(256)])
    for t in range(cfg.T):
        rows = p.pos[t][p.pos[t] >= 0]
        if rows.size == 0:
            continue
        amax = np.float32(np.abs(xf[t]).max())
        scale = np.float32(amax) / np.float32(448.0)
        for r in rows:
            assert sc[r] == scale
            assert (q[r] == q[rows[0]]).all()
        if scale == 0:
            assert (q[rows[0]] == 0).all()
            continue
        quot = (xf[t].astype(np.float32) / scale).astype(np.float32)
        ref = torch.tensor(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (q[rows[0]] == ref).all()
        # the amax element lands on +-448
        h = int(np.argmax(np.abs(xf[t])))
        assert dec[q[rows[0]][h]] == np.sign(xf[t][h]) * 448.0
        # E4M3FN keeps 3 mantissa bits: relative error <= 2^-4 in the normal range
        deq = dec[q[rows[0]]] * float(scale)
        normal = np.abs(quot) >= 2.0 ** -6
        assert (np.abs(deq - xf[t])[normal] <= 2.0 ** -4 * np.abs(xf[t])[normal] * (1 + 1e-6)).all()
        assert (np.abs(deq - xf[t])[~normal] <= 2.0 ** -10 * float(scale) * (1 + 1e-6)).all()
    untouched = np.setdiff1d(np.arange(cfg.cap_rows), p.pos[p.pos >= 0])
    assert (q[untouched] == 0x55).all() and (sc[untouched] == -1.0).all()


def test_combine_unit_weights_is_k_times_x():
    cfg, inp = small_inputs(mask_frac=0.25)
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    ex = oracle.dispatch_bf16(inp.x, p.pos, cfg.cap_rows)
    out = oracle.combine(ex, p.pos, np.ones((cfg.T, cfg.K), np.float32))
    k_live = (p.pos >= 0).sum(axis=1)
    # exact in fp32 (<= 12 significant bits); the sum starts from +0, so a
    # token with no live copy gives +0 even where x is negative
    exact = (bf16_to_f64(inp.x) * k_live[:, None]).astype(np.float32) + np.float32(0.0)
    ref = workloads.bf16_bits_from_f32(exact)
    assert (out == ref).all()
    inactive = k_live == 0
    assert inactive.any() and (out[inactive] == 0).all()


@pytest.mark.parametrize("order,expected", [
    ((2.0 ** 24, 1.0, -(2.0 ** 24)), 0.0),
    ((1.0, 2.0 ** 24, -(2.0 ** 24)), 0.0),
    ((2.0 ** 24, -(2.0 ** 24), 1.0), 1.0),
    ((-(2.0 ** 24), 1.0, 2.0 ** 24), 1.0),
])
def test_combine_association_probe(order, expected):
    K, H = 3, 8
    y = workloads.bf16_bits_from_f32(np.repeat(np.array(order, np.float32)[:, None], H, axis=1))
    pos = np.array([[0, 1, 2]], np.int32)
    out = oracle.combine(y, pos, np.ones((1, K), np.float32))
    assert (bf16_to_f64(out) == expected).all()


def test_combine_within_fp32_bound_of_exact_sum():
    cfg, inp = small_inputs(T=64, H=96, E=16, K=5, W=4, mask_frac=0.2, seed=5)
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    y = workloads.expert_outputs(cfg.cap_rows, cfg.H, seed=5)
    w = inp.weights.copy()
    w[:, 0] *= 3.0   # weights not symmetric in k
    out = oracle.combine(y, p.pos, w)
    yf = bf16_to_f64(y)
    exact = np.zeros((cfg.T, cfg.H))
    absum = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for k in range(cfg.K):
            r = p.pos[t, k]
            if r >= 0:
                exact[t] += float(w[t, k]) * yf[r]
                absum[t] += abs(float(w[t, k])) * np.abs(yf[r])
    bound = cfg.K * 2.0 ** -24 * absum + 2.0 ** -8 * np.abs(exact) + 1e-38

    def within(bits):
        return bool((np.abs(bf16_to_f64(bits) - exact) <= bound).all())

    assert within(out)
    # the check is sharp enough to catch a dropped term or permuted weights
    dropped = p.pos.copy()
    dropped[:, -1] = -1
    assert not within(oracle.combine(y, dropped, w))
    assert not within(oracle.combine(y, p.pos, np.ascontiguousarray(w[:, ::-1])))


def test_combine_skips_negative_positions_and_rejects_out_of_range():
    y = workloads.bf16_bits_from_f32(np.array([[1.0, 2.0]], np.float32))
    pos = np.array([[-1, 0]], np.int32)
    out = oracle.combine(y, pos, np.array([[np.inf, 0.5]], np.float32))
    assert bf16_to_f64(out).tolist() == [[0.5, 1.0]]
    with pytest.raises(ValueError):
        oracle.combine(y, np.array([[1, 0]], np.int32), np.ones((1, 2), np.float32))
