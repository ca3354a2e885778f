"""The oracle over token slices on host threads, for full-size parity.

Each call below runs the serial C oracle on contiguous slices of tokens in
parallel (ctypes releases the interpreter lock during the call).  Slices
write disjoint rows: a live copy's position is unique, and the combine's
output rows are the slice's own tokens.  The arithmetic is the oracle's,
unchanged; only the work is split.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def host_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _slices(T: int, n: int):
    b = np.linspace(0, T, n + 1).astype(int)
    return [(int(lo), int(hi)) for lo, hi in zip(b[:-1], b[1:]) if hi > lo]


def _run(fn, T: int):
    n = host_threads()
    with ThreadPoolExecutor(n) as pool:
        list(pool.map(lambda s: fn(*s), _slices(T, 4 * n)))


def dispatch_bf16(x: np.ndarray, pos: np.ndarray, cap_rows: int, fill: int) -> np.ndarray:
    """expandX [cap_rows][H] uint16; rows no copy names hold `fill`."""
    T, H = x.shape
    out = np.full((cap_rows, H), fill, np.uint16)
    _run(lambda lo, hi: oracle.dispatch_bf16(x[lo:hi], pos[lo:hi], cap_rows, out=out), T)
    return out


def dispatch_fp8(x: np.ndarray, pos: np.ndarray, cap_rows: int, fill_q: int, fill_scale: float):
    """(codes [cap_rows][H] uint8, scales [cap_rows] float32); rows no copy
    names hold the fills."""
    T, H = x.shape
    q = np.full((cap_rows, H), fill_q, np.uint8)
    sc = np.full(cap_rows, fill_scale, np.float32)
    _run(lambda lo, hi: oracle.dispatch_fp8(x[lo:hi], pos[lo:hi], cap_rows, q=q, scales=sc), T)
    return q, sc


def combine(y: np.ndarray, pos: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """out [T][H] uint16 for every token."""
    T = pos.shape[0]
    out = np.empty((T, y.shape[1]), np.uint16)

    def run(lo, hi):
        out[lo:hi] = oracle.combine(y, pos[lo:hi], weights[lo:hi])

    _run(run, T)
    return out


def dispatch_quant(x: np.ndarray, ids: np.ndarray, pos: np.ndarray, E: int, qtype: int, cap_rows: int,
                   smooth: np.ndarray | None, fill_q: int, fill_scale: float):
    """Per-copy quantised rows (fp8 or int8, optionally smoothed): (codes
    [cap_rows][H] uint8, scales [cap_rows] float32); rows no copy names hold
    the fills."""
    T, H = x.shape
    q = np.full((cap_rows, H), fill_q, np.uint8)
    sc = np.full(cap_rows, fill_scale, np.float32)
    _run(lambda lo, hi: oracle.dispatch_quant(x[lo:hi], ids[lo:hi], pos[lo:hi], E, qtype, cap_rows,
                                              smooth, q=q, scales=sc), T)
    return q, sc


def combine_quant(codes: np.ndarray, qtype: int, scales: np.ndarray, pos: np.ndarray,
                  weights: np.ndarray) -> np.ndarray:
    """out [T][H] uint16 from quantised expert rows, for every token."""
    T = pos.shape[0]
    out = np.empty((T, codes.shape[1]), np.uint16)

    def run(lo, hi):
        out[lo:hi] = oracle.combine_quant(codes, qtype, scales, pos[lo:hi], weights[lo:hi])

    _run(run, T)
    return out


def combine_add_rmsnorm(y: np.ndarray, pos: np.ndarray, weights: np.ndarray, residual: np.ndarray,
                        gamma: np.ndarray, eps: float):
    """(residual_out, norm_out) [T][H] uint16 each, for every token."""
    T = pos.shape[0]
    ro = np.empty((T, y.shape[1]), np.uint16)
    no = np.empty((T, y.shape[1]), np.uint16)

    def run(lo, hi):
        ro[lo:hi], no[lo:hi] = oracle.combine_add_rmsnorm(y, pos[lo:hi], weights[lo:hi], residual[lo:hi],
                                                          gamma, eps)

    _run(run, T)
    return ro, no
