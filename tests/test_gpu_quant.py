"""GPU parity of the quantisation variants against the oracle, bit for bit:
int8 per-token dynamic quantisation, per-expert smoothing before fp8 / int8
quantisation (one row and scale per copy), and the combine of quantised expert
rows (codes + one fp32 scale per row), including every one of the 256 codes
of both code types."""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
from _gpu_util import bf16_ulp_distance, dev, host

pytestmark = pytest.mark.gpu

QT = {"fp8": (ep.EP_FP8_E4M3FN, oracle.Q_FP8), "int8": (ep.EP_INT8, oracle.Q_INT8)}

SHAPES = [
    # T, H, E, K, W, mask
    (300, 128, 16, 4, 4, 0.2),      # one group per thread, ragged token count
    (257, 2064, 32, 6, 1, 0.1),     # 129 groups: a ragged second group per thread
    (64, 7168, 64, 8, 8, 0.25),     # 448 groups (two per thread)
    (33, 16384, 8, 2, 1, 0.0),      # the largest smoothed row
    (1, 16, 4, 1, 1, 0.0),          # a single group
]


def case(T, H, E, K, W, mask, seed):
    cfg = workloads.MoEConfig("q", T=T, H=H, E=E, K=K, W=W, sigma=3.0, mask_frac=mask, seed=seed)
    inp = workloads.moe_inputs(cfg)
    # a few all-zero rows: scale 0 and zero codes
    inp.x[::37] = 0
    p = oracle.plan(inp.ids, E, W, inp.active)
    return cfg, inp, p


def sid(s):
    return f"T{s[0]}H{s[1]}E{s[2]}K{s[3]}"


@pytest.mark.parametrize("shape", SHAPES, ids=[sid(s) for s in SHAPES])
def test_int8_dispatch(shape):
    print("int8 dispatch", shape, flush=True)
    cfg, inp, p = case(*shape, seed=sum(shape[:4]))
    cap = cfg.cap_rows
    q = torch.full((cap, cfg.H), 0x5A, dtype=torch.uint8, device="cuda")
    sc = torch.full((cap,), -2.0, dtype=torch.float32, device="cuda")
    ep.ep_dispatch(dev(inp.x), dev(p.pos), q, sc, out_dtype=ep.EP_INT8)
    want_q, want_s = oracle.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, oracle.Q_INT8, cap,
                                           fill_q=0x5A, fill_scale=-2.0)
    assert (host(sc).view(np.uint32) == want_s.view(np.uint32)).all()
    bad = np.argwhere(host(q) != want_q)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[0].tolist()}"
    assert ep.ep_device_error() == 0


@pytest.mark.parametrize("qt", ["fp8", "int8"])
@pytest.mark.parametrize("shape", SHAPES, ids=[sid(s) for s in SHAPES])
def test_smoothed_dispatch(shape, qt):
    print("smoothed dispatch", qt, shape, flush=True)
    dt, oq = QT[qt]
    cfg, inp, p = case(*shape, seed=3 * sum(shape[:4]))
    smooth = workloads.smooth_scales(cfg.E, cfg.H, 5)
    smooth[1, : cfg.H // 2] = 0.0            # an expert that zeroes half of the row
    if cfg.E > 3:
        smooth[3] = 0.0                      # and one that zeroes it all: scale 0
    cap = cfg.cap_rows
    q = torch.full((cap, cfg.H), 0x33, dtype=torch.uint8, device="cuda")
    sc = torch.full((cap,), -1.0, dtype=torch.float32, device="cuda")
    ep.ep_dispatch_smooth(dev(inp.x), dev(inp.ids), dev(p.pos), dev(smooth), q, sc, out_dtype=dt)
    want_q, want_s = oracle.dispatch_quant(inp.x, inp.ids, p.pos, cfg.E, oq, cap, smooth,
                                           fill_q=0x33, fill_scale=-1.0)
    assert (host(sc).view(np.uint32) == want_s.view(np.uint32)).all()
    bad = np.argwhere(host(q) != want_q)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[0].tolist()}"
    assert ep.ep_device_error() == 0


def test_smoothed_dispatch_flags_bad_expert():
    print("smoothed dispatch, expert id out of range", flush=True)
    cfg, inp, p = case(64, 128, 8, 2, 2, 0.0, seed=9)
    ids = inp.ids.copy()
    ids[5, 1] = 8                              # outside [0, E): the copy is skipped
    smooth = workloads.smooth_scales(cfg.E, cfg.H, 1)
    q = torch.zeros((cfg.cap_rows, cfg.H), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((cfg.cap_rows,), dtype=torch.float32, device="cuda")
    ep.ep_device_error()
    ep.ep_dispatch_smooth(dev(inp.x), dev(ids), dev(p.pos), dev(smooth), q, sc)
    assert ep.ep_device_error() & ep.EP_DEVERR_BAD_EXPERT
    live = p.pos >= 0
    live[5, 1] = False
    want_q, want_s = oracle.dispatch_quant(inp.x, inp.ids, np.where(live, p.pos, -1), cfg.E,
                                           oracle.Q_FP8, cfg.cap_rows, smooth)
    assert (host(q) == want_q).all()
    assert ep.ep_device_error() == 0


@pytest.mark.parametrize("qt", ["fp8", "int8"])
def test_combine_decodes_every_code(qt):
    print("quantised combine, every code", qt, flush=True)
    dt, oq = QT[qt]
    H = 256
    codes = np.arange(256, dtype=np.uint8)[None, :].repeat(2, axis=0)
    codes[1] = codes[1][::-1]
    scales = np.array([1.0, 0.25], np.float32)
    pos = np.array([[0, -1], [1, -1], [0, 1]], np.int32)
    w = np.array([[1.0, 0.0], [1.0, 0.0], [0.5, 2.0]], np.float32)
    out = torch.zeros((3, H), dtype=torch.int16, device="cuda")
    ep.ep_combine_quant(dev(codes), dev(scales), dev(pos), dev(w), out, code_dtype=dt)
    got = host(out, np.uint16)
    want = oracle.combine_quant(codes, oq, scales, pos, w)
    nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    both_nan = nan(got) & nan(want)
    assert (both_nan | (got == want)).all()
    if qt == "int8":
        assert not nan(want).any()
    else:
        assert nan(want).sum() == 2 + 2 + 4      # the two NaN codes per row
    assert ep.ep_device_error() == 0


@pytest.mark.parametrize("qt", ["fp8", "int8"])
@pytest.mark.parametrize("shape", [(300, 128, 16, 4, 4, 0.2), (257, 2064, 32, 6, 1, 0.1),
                                   (96, 7168, 64, 8, 8, 0.25), (40, 1024, 32, 16, 4, 0.0),
                                   (50, 4096, 16, 3, 2, 0.0)],
                         ids=["T300H128K4", "T257H2064K6", "T96H7168K8", "T40H1024K16", "T50H4096K3"])
def test_quantised_combine(shape, qt):
    """Expert rows travel as codes + a row scale (quantised by the GPU
    dispatch from synthetic expert outputs), then combine."""
    print("quantised combine", qt, shape, flush=True)
    dt, oq = QT[qt]
    T, H, E, K, W, mask = shape
    cfg, inp, p = case(*shape, seed=11 * K)
    N = p.n_rows
    y = workloads.expert_outputs(N, H, 21)
    ident = np.arange(N, dtype=np.int32)[:, None]
    yq = torch.zeros((N, H), dtype=torch.uint8, device="cuda")
    ys = torch.zeros((N,), dtype=torch.float32, device="cuda")
    if N:
        ep.ep_dispatch(dev(y), dev(ident), yq, ys, out_dtype=dt)
    want_yq, want_ys = oracle.dispatch_quant(y, np.zeros_like(ident), ident, 1, oq, N)
    assert (host(yq) == want_yq).all() and (host(ys).view(np.uint32) == want_ys.view(np.uint32)).all()
    out = torch.full((T, H), 0x1234, dtype=torch.int16, device="cuda")
    ep.ep_combine_quant(yq, ys, dev(p.pos), dev(inp.weights), out, code_dtype=dt)
    want = oracle.combine_quant(want_yq, oq, want_ys, p.pos, inp.weights)
    d = bf16_ulp_distance(host(out, np.uint16), want)
    assert d.max() == 0, f"max {d.max()} ulp at {np.unravel_index(d.argmax(), d.shape)}"
    assert ep.ep_device_error() == 0


def test_fullsize_smoothed_fp8_sampled():
    """The largest workload (T16384 H7168 E256 K8, 25% masked tokens) through
    the smoothed fp8 dispatch and the quantised combine, compared on a sample
    of tokens with the oracle."""
    cfg = workloads.WORKLOADS[4]
    print("full-size smoothed fp8", cfg.name, flush=True)
    inp = workloads.moe_inputs(cfg)
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    smooth = workloads.smooth_scales(cfg.E, cfg.H, 4)
    cap = cfg.cap_rows
    q = torch.zeros((cap, cfg.H), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((cap,), dtype=torch.float32, device="cuda")
    pos_d = dev(p.pos)
    ep.ep_dispatch_smooth(dev(inp.x), dev(inp.ids), pos_d, dev(smooth), q, sc)
    out = torch.zeros((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    ep.ep_combine_quant(q, sc, pos_d, dev(inp.weights), out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    toks = np.sort(np.concatenate([rng.choice(cfg.T, 48, replace=False), [0, cfg.T - 1]]))
    sub = p.pos[toks].copy()
    live = sub >= 0
    rows = sub[live]
    sub[live] = np.arange(rows.size, dtype=np.int32)
    want_q, want_s = oracle.dispatch_quant(inp.x[toks], inp.ids[toks], sub, cfg.E, oracle.Q_FP8,
                                           rows.size, smooth)
    rows_t = torch.from_numpy(rows.astype(np.int64)).cuda()
    assert (host(q[rows_t]) == want_q).all()
    assert (host(sc[rows_t]).view(np.uint32) == want_s.view(np.uint32)).all()
    want_out = oracle.combine_quant(want_q, oracle.Q_FP8, want_s, sub, inp.weights[toks])
    toks_t = torch.from_numpy(toks.astype(np.int64)).cuda()
    assert (bf16_ulp_distance(host(out[toks_t], np.uint16), want_out) == 0).all()
    assert ep.ep_device_error() == 0


def e4m3_values():
    """The 127 non-negative finite E4M3FN values, by code (format definition)."""
    v = []
    for c in range(127):
        e, m = c >> 3, c & 7
        v.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(v)


@pytest.mark.parametrize("qt", ["fp8", "int8"])
def test_smoothed_codes_at_rounding_boundaries(qt):
    """Quotients placed on and within three fp32 ulps of every rounding
    boundary of the code (E4M3FN midpoints, int8 half-integers), both signs,
    at many row scales (including scales outside [2^-60, 2^60] and
    power-of-two ones).  x is all ones, so the smoothed row equals the
    smoothing row, whose column 0 fixes the row maximum."""
    print("quantisation at rounding boundaries", qt, flush=True)
    dt, oq = QT[qt]
    rng = np.random.default_rng(17 if qt == "fp8" else 18)
    if qt == "fp8":
        v = e4m3_values()
        mids, qmax = (v[:-1] + v[1:]) / 2, np.float32(448.0)
    else:
        mids, qmax = np.arange(127) + 0.5, np.float32(127.0)
    T, H = 96, 2048
    E, K = T, 1
    amax = (rng.uniform(0.5, 2.0, T) * 2.0 ** rng.integers(-40, 40, T)).astype(np.float32)
    amax[:4] = np.float32([2.0 ** -70 * 1.37, 2.0 ** 70 * 1.61, 2.0 ** -64, 1.0])
    amax[4:8] = np.float32(2.0) ** np.float32([-3, 0, 5, 17])
    smooth = np.zeros((E, H), np.float32)
    for t in range(T):
        scale = np.float32(amax[t] / qmax)
        cols = [amax[t]]
        for m in mids:
            base = np.float32(np.float32(m) * scale)
            for k in range(-3, 4):
                b = np.array([base], np.float32).view(np.uint32)[0]
                nb = np.array([b + np.uint32(k) if k >= 0 else b - np.uint32(-k)], np.uint32)
                val = nb.view(np.float32)[0]
                if np.isfinite(val) and abs(val) <= amax[t]:
                    cols += [val, -val]
        cols = np.array(cols[:H], np.float32)
        smooth[t, : cols.size] = cols
        smooth[t, cols.size:] = rng.uniform(-1, 1, H - cols.size).astype(np.float32) * amax[t]
    x = np.full((T, H), 0x3F80, np.uint16)                     # bf16 1.0
    ids = np.arange(T, dtype=np.int32)[:, None]
    p = oracle.plan(ids, E, 1)
    q = torch.zeros((T, H), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((T,), dtype=torch.float32, device="cuda")
    ep.ep_dispatch_smooth(dev(x), dev(ids), dev(p.pos), dev(smooth), q, sc, out_dtype=dt)
    want_q, want_s = oracle.dispatch_quant(x, ids, p.pos, E, oq, T, smooth)
    assert (host(sc).view(np.uint32) == want_s.view(np.uint32)).all()
    bad = np.argwhere(host(q) != want_q)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[0].tolist()}"
    assert ep.ep_device_error() == 0


@pytest.mark.parametrize("qt", ["fp8", "int8"])
def test_widest_rows(qt):
    """H = 65536, the widest row the library takes: 16 groups of 16 values per
    thread, 8 kept in registers and the rest re-read in the quantise pass;
    then the combine of those rows."""
    print("widest quantised rows", qt, flush=True)
    dt, oq = QT[qt]
    T, H, E, K, W = 12, 65536, 8, 3, 2
    cfg, inp, p = case(T, H, E, K, W, 0.2, seed=65)
    cap = cfg.cap_rows
    q = torch.full((cap, H), 0x77, dtype=torch.uint8, device="cuda")
    sc = torch.full((cap,), -5.0, dtype=torch.float32, device="cuda")
    ep.ep_dispatch(dev(inp.x), dev(p.pos), q, sc, out_dtype=dt)
    want_q, want_s = oracle.dispatch_quant(inp.x, inp.ids, p.pos, E, oq, cap, fill_q=0x77, fill_scale=-5.0)
    assert (host(sc).view(np.uint32) == want_s.view(np.uint32)).all()
    assert (host(q) == want_q).all()
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    ep.ep_combine_quant(q, sc, dev(p.pos), dev(inp.weights), out, code_dtype=dt)
    want = oracle.combine_quant(want_q, oq, want_s, p.pos, inp.weights)
    assert (bf16_ulp_distance(host(out, np.uint16), want) == 0).all()
    assert (p.pos >= 0).any()
    assert ep.ep_device_error() == 0
