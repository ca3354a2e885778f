"""Per-token dynamic quantisation without smoothing, over its whole input
domain: every finite bf16 value x against every finite row amax A >= |x|
(about 1.07 G pairs per code type), through ep_dispatch, bit for bit against
the oracle's codes and scales.

A row's scale is fl32(A / qmax) and each code is the encoding of
fl32(x / scale), so the pairs (x, A) are everything the kernel's division and
encoders can see from a bf16 row (per-token dynamic quantisation, quantMode 2
of the CANN "aclnnMoeDistributeDispatchV2" page).  The rows come from
tests/_quant_domain.py; the oracle runs on host threads over slices of rows.
"""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import combine_ep_plan_02_amd as ep
import oracle
from _gpu_util import dev, host
from _quant_domain import batches, domain_rows

pytestmark = pytest.mark.gpu

H = 4096
MAX_ROWS = 16384
QT = {"fp8": (ep.EP_FP8_E4M3FN, oracle.Q_FP8), "int8": (ep.EP_INT8, oracle.Q_INT8)}


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_codes(x: np.ndarray, qt: str, pool: ThreadPoolExecutor, nthreads: int):
    """The oracle's codes and scales for rows x (one copy per row, row r to
    position r), computed over slices of rows in parallel."""
    R = x.shape[0]
    q = np.empty((R, H), np.uint8)
    s = np.empty(R, np.float32)
    bounds = np.linspace(0, R, nthreads + 1).astype(int)

    def run(lo, hi):
        if hi <= lo:
            return
        n = hi - lo
        pos = np.arange(n, dtype=np.int32).reshape(n, 1)
        if qt == "fp8":
            q[lo:hi], s[lo:hi] = oracle.dispatch_fp8(x[lo:hi], pos, n)
        else:
            ids = np.zeros((n, 1), np.int32)
            q[lo:hi], s[lo:hi] = oracle.dispatch_quant(x[lo:hi], ids, pos, 1, oracle.Q_INT8, n)

    list(pool.map(lambda b: run(*b), zip(bounds[:-1], bounds[1:])))
    return q, s


@pytest.mark.parametrize("qt", ["fp8", "int8"])
def test_every_value_against_every_amax(qt):
    code, _ = QT[qt]
    nthreads = host_threads()
    t0 = time.time()
    pairs = 0
    with ThreadPoolExecutor(nthreads) as pool:
        for lo, hi in batches(H, MAX_ROWS):
            x, row_a = domain_rows(lo, hi, H)
            R = x.shape[0]
            pos = torch.arange(R, dtype=torch.int32, device="cuda").view(R, 1)
            q = torch.empty((R, H), dtype=torch.uint8, device="cuda")
            sc = torch.empty((R,), dtype=torch.float32, device="cuda")
            ep.ep_dispatch(dev(x), pos, q, sc, out_dtype=code)
            got_q, got_s = host(q), host(sc)
            want_q, want_s = oracle_codes(x, qt, pool, nthreads)
            bad_s = np.flatnonzero(got_s.view(np.uint32) != want_s.view(np.uint32))
            assert bad_s.size == 0, (f"{qt}: {bad_s.size} scales differ, first amax {int(row_a[bad_s[0]]):#06x}: "
                                     f"got {got_s[bad_s[0]]!r} want {want_s[bad_s[0]]!r}")
            bad = np.argwhere(got_q != want_q)
            if bad.size:
                r, c = bad[0]
                raise AssertionError(f"{qt}: {len(bad)} codes differ in amax [{lo:#06x}, {hi:#06x}); first: "
                                     f"x {int(x[r, c]):#06x} amax {int(row_a[r]):#06x} "
                                     f"got {int(got_q[r, c]):#04x} want {int(want_q[r, c]):#04x}")
            pairs += int((2 * (np.arange(lo, hi, dtype=np.int64) + 1)).sum())
    print(f"{qt}: {pairs} (x, amax) pairs equal in {time.time() - t0:.1f} s on {nthreads} host threads",
          flush=True)
    assert pairs == 0x7F80 * 0x7F81
