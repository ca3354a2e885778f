"""Full-size parity of the extension kernels the benchmark times beside the
step, element by element, on the two target workloads (T=8192, H=7168,
E=256, K=8, W=16 with Zipf(1.2) routing; T=16384, H=7168, E=256, K=8, W=32
with 25% of tokens masked), in the benchmark's launch configuration:

- the dispatch to int8 rows and the dispatch with per-expert smoothing
  scales to fp8 and int8 rows (quantMode 2 with scalesOptional on the CANN
  "aclnnMoeDistributeDispatchV2" page): every code and every row scale of
  the expandX buffer, the rows past N included (they keep their sentinel);
- the combine of fp8 and int8 expert rows (commQuantMode on the same
  page's combine): every output row at 0 bf16 ulp;
- the combine fused with the residual add and RMSNorm (the MoE-finalize
  pattern of flashinfer PR #4358 without its all-reduce): every
  residual_out element bit for bit, every norm_out element within 1 bf16
  ulp, more than 99% of them equal.

The oracle runs over token slices on host threads (tests/_oracle_slices.py).
"""
import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
import workloads
import _oracle_slices as par
from _gpu_util import GpuPath, assert_plan_equal, bf16_ulp_distance, dev, host

pytestmark = pytest.mark.gpu

SENTINEL_Q = 0x33
SENTINEL_SCALE = -1.0
EPS = 1e-6


def say(*a):
    print(*a, flush=True)


def assert_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if np.array_equal(got, want):
        return
    bad = np.argwhere(got != want)
    raise AssertionError(f"{what}: {len(bad)} elements differ; first at {bad[0].tolist()}: "
                         f"got {got[tuple(bad[0])]}, want {want[tuple(bad[0])]}")


class Case:
    """One target workload with its plan checked against the oracle."""

    def __init__(self, idx: int):
        self.cfg = cfg = workloads.WORKLOADS[idx]
        self.inp = workloads.moe_inputs(cfg)
        self.want = oracle.plan(self.inp.ids, cfg.E, cfg.W, self.inp.active)
        self.g = GpuPath(self.inp.ids, cfg.E, cfg.W, self.inp.active)
        self.g.run_plan()
        assert_plan_equal(self.g.plan_host(), self.want)
        self.N = self.want.n_rows
        self.cap = cfg.cap_rows

    def quant_rows(self, qtype: int, smooth: np.ndarray | None):
        """GPU codes and scales of every expandX row, and the oracle's."""
        cfg = self.cfg
        q = torch.full((self.cap, cfg.H), SENTINEL_Q, dtype=torch.uint8, device="cuda")
        sc = torch.full((self.cap,), SENTINEL_SCALE, dtype=torch.float32, device="cuda")
        code = ep.EP_FP8_E4M3FN if qtype == oracle.Q_FP8 else ep.EP_INT8
        x = dev(self.inp.x)
        if smooth is None:
            ep.ep_dispatch(x, self.g.plan.pos, q, sc, out_dtype=code)
        else:
            ep.ep_dispatch_smooth(x, self.g.ids, self.g.plan.pos, dev(smooth), q, sc, out_dtype=code)
        torch.cuda.synchronize()
        want_q, want_s = par.dispatch_quant(self.inp.x, self.inp.ids, self.want.pos, cfg.E, qtype, self.cap,
                                            smooth, SENTINEL_Q, SENTINEL_SCALE)
        return host(q), host(sc), want_q, want_s


@pytest.fixture(scope="module", params=[2, 4], ids=["zipf_T8192", "mask25_T16384"])
def case(request):
    torch.cuda.synchronize()
    ep.ep_device_error()
    say("full-size extension case:", workloads.WORKLOADS[request.param].name)
    c = Case(request.param)
    yield c
    del c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("qtype,smoothed", [(oracle.Q_INT8, False), (oracle.Q_FP8, True), (oracle.Q_INT8, True)],
                         ids=["int8", "smoothed_fp8", "smoothed_int8"])
def test_fullsize_quantised_dispatch_and_combine(case, qtype, smoothed):
    cfg = case.cfg
    smooth = workloads.smooth_scales(cfg.E, cfg.H, cfg.seed) if smoothed else None
    say(f"  dispatch qtype {qtype} smoothed {smoothed}")
    got_q, got_s, want_q, want_s = case.quant_rows(qtype, smooth)
    assert_equal(got_s.view(np.uint32), want_s.view(np.uint32), "row scales")
    assert_equal(got_q, want_q, "codes")
    say(f"  dispatch ok: all {case.cap} rows of codes and scales ({case.N} written)")
    # the combine of quantised expert rows, from these codes
    code = ep.EP_FP8_E4M3FN if qtype == oracle.Q_FP8 else ep.EP_INT8
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    ep.ep_combine_quant(dev(want_q), dev(want_s), case.g.plan.pos, dev(case.inp.weights), out, code_dtype=code)
    torch.cuda.synchronize()
    want_out = par.combine_quant(want_q, qtype, want_s, case.want.pos, case.inp.weights)
    d = bf16_ulp_distance(host(out, np.uint16), want_out)
    assert int((d > 0).sum()) == 0, f"combine of quantised rows: {int((d > 0).sum())} elements differ"
    say(f"  combine of quantised rows ok: all {cfg.T} rows at 0 ulp")
    assert ep.ep_device_error() == 0


def test_fullsize_combine_add_rmsnorm(case):
    cfg = case.cfg
    rng = np.random.default_rng(cfg.seed + 3000)
    y = np.zeros((case.cap, cfg.H), np.uint16)
    y[:case.N] = workloads.expert_outputs(case.N, cfg.H, cfg.seed + 60)
    residual = workloads.expert_outputs(cfg.T, cfg.H, cfg.seed + 70)
    gamma = workloads.bf16_bits_from_f32((1.0 + 0.1 * rng.standard_normal(cfg.H)).astype(np.float32))
    ro = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    no = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    ep.ep_combine_add_rmsnorm(dev(y), case.g.plan.pos, dev(case.inp.weights), dev(residual), dev(gamma), EPS,
                              ro, no)
    torch.cuda.synchronize()
    want_ro, want_no = par.combine_add_rmsnorm(y, case.want.pos, case.inp.weights, residual, gamma, EPS)
    assert_equal(host(ro, np.uint16), want_ro, "residual_out")
    d = bf16_ulp_distance(host(no, np.uint16), want_no)
    assert d.max() <= 1, f"norm_out: {int((d > 1).sum())} elements more than 1 ulp apart"
    assert (d == 0).mean() > 0.99, f"norm_out: {int((d > 0).sum())} of {d.size} elements 1 ulp apart"
    say(f"  tail ok: residual_out bit for bit, norm_out {int((d > 0).sum())} of {d.size} elements 1 ulp apart")
    assert ep.ep_device_error() == 0
