"""CPU oracle for MoE expert-parallel dispatch / combine (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``ep_oracle.c`` -- a plain,
serial C transcription of the method, with its own bf16 / E4M3FN codecs --
through ctypes, taking and returning numpy arrays.  It shares no code with
the HIP library and never imports it.

Parity pins live in ``tests/test_oracle_*.py``.  Readings that nothing on the
source pages pins (quantisation divides by the scale; a row whose amax is 0
gets scale 0 and zero codes) are marked "parity unpinned" in ``ep_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A compiled oracle to load instead of liboracle.so (not rebuilt); the
# mutation test points it at builds of ep_oracle.c with one planted mistake.
_LIB_OVERRIDE = os.environ.get("EP_ORACLE_LIB")

DEVERR_BAD_EXPERT = 1
DEVERR_SPLITS = 2


def build(force: bool = True) -> str:
    """Compile ep_oracle.c with gcc into oracle/liboracle.so (serial, -O2,
    no FP contraction, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16_rne.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_e4m3fn_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3fn_decode.restype = ctypes.c_double
    lib.oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3fn_encode.restype = ctypes.c_uint8
    lib.oracle_plan.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_plan.restype = ctypes.c_int
    lib.oracle_dispatch_bf16.argtypes = [i32, i32, i32, P, P, P, i64]
    lib.oracle_dispatch_bf16.restype = ctypes.c_int
    lib.oracle_dispatch_fp8.argtypes = [i32, i32, i32, P, P, P, P, i64, P]
    lib.oracle_dispatch_fp8.restype = ctypes.c_int
    lib.oracle_combine.argtypes = [i32, i32, i32, P, i64, P, P, P]
    lib.oracle_combine.restype = ctypes.c_int
    lib.oracle_plan_ex.argtypes = [i32, i32, i32, i32, P, P, P, i32, i32, i32, P, P, P, P, P, P, P,
                                   P, P, P, P]
    lib.oracle_plan_ex.restype = ctypes.c_int
    lib.oracle_int8_encode.argtypes = [ctypes.c_float]
    lib.oracle_int8_encode.restype = ctypes.c_int8
    lib.oracle_dispatch_quant.argtypes = [i32, i32, i32, i32, P, P, P, P, i32, P, P, i64, P]
    lib.oracle_dispatch_quant.restype = ctypes.c_int
    lib.oracle_combine_quant.argtypes = [i32, i32, i32, P, i32, P, i64, P, P, P]
    lib.oracle_combine_quant.restype = ctypes.c_int
    lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_combine_add_rmsnorm.argtypes = [i32, i32, i32, P, i64, P, P, P, P, ctypes.c_float, P, P]
    lib.oracle_combine_add_rmsnorm.restype = ctypes.c_int
    lib.oracle_dispatch_weights.argtypes = [i32, i32, P, P, P, i64]
    lib.oracle_dispatch_weights.restype = ctypes.c_int
    lib.oracle_a2a_plan.argtypes = [i32, P, P, P, P, P]
    lib.oracle_a2a_plan.restype = ctypes.c_int
    lib.oracle_a2a_copy.argtypes = [i32, i64, i64, P, P, P, P, P, P, P]
    lib.oracle_a2a_copy.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


# ---------------------------------------------------------------- codecs

def bf16_to_f32(bits: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(bits)))


def f32_to_bf16_rne(value: float) -> int:
    return int(_load().oracle_f32_to_bf16_rne(float(np.float32(value))))


def e4m3fn_decode(code: int) -> float:
    return float(_load().oracle_e4m3fn_decode(int(code)))


def e4m3fn_encode(value: float) -> int:
    return int(_load().oracle_e4m3fn_encode(float(np.float32(value))))


# ---------------------------------------------------------------- 2-D plan

@dataclass
class Plan:
    in_splits: np.ndarray      # [W][E] int64
    src_offsets: np.ndarray    # [W][E] int64
    out_splits: np.ndarray     # [W][E/W][W] int64
    dst_offsets: np.ndarray    # [W][E] int64
    expert_counts: np.ndarray  # [E] int64
    expert_offsets: np.ndarray  # [E] int64
    rank_offsets: np.ndarray   # [W+1] int64
    pos: np.ndarray            # [T][K] int32
    occ: np.ndarray            # [T][K] int32
    err: int                   # device-error bits the inputs raise

    @property
    def n_rows(self) -> int:
        return int(self.rank_offsets[-1])


def plan(ids: np.ndarray, E: int, W: int, active: np.ndarray | None = None) -> Plan:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    ne = E // W
    act = None if active is None else np.ascontiguousarray(active, dtype=np.uint8)
    out = Plan(
        in_splits=np.zeros((W, E), np.int64), src_offsets=np.zeros((W, E), np.int64),
        out_splits=np.zeros((W, ne, W), np.int64), dst_offsets=np.zeros((W, E), np.int64),
        expert_counts=np.zeros(E, np.int64), expert_offsets=np.zeros(E, np.int64),
        rank_offsets=np.zeros(W + 1, np.int64), pos=np.zeros((T, K), np.int32),
        occ=np.zeros((T, K), np.int32), err=0)
    err = ctypes.c_uint32(0)
    rc = _load().oracle_plan(T, K, E, W, _ptr(ids), _ptr(act), _ptr(out.in_splits),
                             _ptr(out.src_offsets), _ptr(out.out_splits),
                             _ptr(out.dst_offsets), _ptr(out.expert_counts),
                             _ptr(out.expert_offsets), _ptr(out.rank_offsets),
                             _ptr(out.pos), _ptr(out.occ), ctypes.byref(err))
    _check(rc, "plan")
    out.err = int(err.value)
    return out


def plan_ex(ids: np.ndarray, E: int, W: int, active: np.ndarray | None = None,
            active_copies: np.ndarray | None = None, major_align: int = 1,
            pad_empty: bool = False, token_nums_type: int = 1):
    """Extended plan (per-copy mask, expert padding, expert token numbers).
    Returns (Plan, expert_token_nums [W][E/W] int64)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    ne = E // W
    act = None if active is None else np.ascontiguousarray(active, dtype=np.uint8)
    actc = None if active_copies is None else np.ascontiguousarray(active_copies, dtype=np.uint8)
    out = Plan(
        in_splits=np.zeros((W, E), np.int64), src_offsets=np.zeros((W, E), np.int64),
        out_splits=np.zeros((W, ne, W), np.int64), dst_offsets=np.zeros((W, E), np.int64),
        expert_counts=np.zeros(E, np.int64), expert_offsets=np.zeros(E, np.int64),
        rank_offsets=np.zeros(W + 1, np.int64), pos=np.zeros((T, K), np.int32),
        occ=np.zeros((T, K), np.int32), err=0)
    etn = np.zeros((W, ne), np.int64)
    err = ctypes.c_uint32(0)
    rc = _load().oracle_plan_ex(T, K, E, W, _ptr(ids), _ptr(act), _ptr(actc), int(major_align),
                                int(bool(pad_empty)), int(token_nums_type), _ptr(out.in_splits),
                                _ptr(out.src_offsets), _ptr(out.out_splits), _ptr(out.dst_offsets),
                                _ptr(out.expert_counts), _ptr(out.expert_offsets),
                                _ptr(out.rank_offsets), _ptr(out.pos), _ptr(out.occ), _ptr(etn),
                                ctypes.byref(err))
    _check(rc, "plan_ex")
    out.err = int(err.value)
    return out, etn


def dispatch_weights(pos: np.ndarray, weights: np.ndarray, cap_rows: int,
                     fill: float = 0.0) -> np.ndarray:
    """expand_weights [cap_rows] float32: the gate weight of each expanded row."""
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    T, K = pos.shape
    out = np.full(cap_rows, fill, np.float32)
    _check(_load().oracle_dispatch_weights(T, K, _ptr(pos), _ptr(weights), _ptr(out), cap_rows),
           "dispatch_weights")
    return out


# ---------------------------------------------------------------- dispatch

def dispatch_bf16(x_bits: np.ndarray, pos: np.ndarray, cap_rows: int,
                  fill: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """x_bits: [T][H] uint16 bf16 patterns.  Returns expandX [cap_rows][H]
    uint16; rows no copy names keep `fill` (or the contents of `out`)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    T, H = x_bits.shape
    K = pos.shape[1]
    if out is None:
        out = np.full((cap_rows, H), 0 if fill is None else fill, dtype=np.uint16)
    assert out.shape == (cap_rows, H) and out.dtype == np.uint16 and out.flags["C_CONTIGUOUS"]
    _check(_load().oracle_dispatch_bf16(T, K, H, _ptr(x_bits), _ptr(pos), _ptr(out), cap_rows),
           "dispatch_bf16")
    return out


def dispatch_fp8(x_bits: np.ndarray, pos: np.ndarray, cap_rows: int,
                 fill_q: int = 0, fill_scale: float = 0.0,
                 q: np.ndarray | None = None, scales: np.ndarray | None = None):
    """Returns (q [cap_rows][H] uint8 E4M3FN codes, scales [cap_rows] float32).
    With `q` and `scales` given (C-contiguous, [cap_rows][H] uint8 and
    [cap_rows] float32) the rows are written there and the rest is kept."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    T, H = x_bits.shape
    K = pos.shape[1]
    if q is None:
        q = np.full((cap_rows, H), fill_q, dtype=np.uint8)
    if scales is None:
        scales = np.full(cap_rows, fill_scale, dtype=np.float32)
    assert q.shape == (cap_rows, H) and q.dtype == np.uint8 and q.flags["C_CONTIGUOUS"]
    assert scales.shape == (cap_rows,) and scales.dtype == np.float32 and scales.flags["C_CONTIGUOUS"]
    scratch = np.zeros(H, np.uint8)
    _check(_load().oracle_dispatch_fp8(T, K, H, _ptr(x_bits), _ptr(pos), _ptr(q),
                                       _ptr(scales), cap_rows, _ptr(scratch)), "dispatch_fp8")
    return q, scales


# ---------------------------------------------------------------- combine

def combine(y_bits: np.ndarray, pos: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """y_bits: [cap][H] uint16; pos [T][K] int32; weights [T][K] float32.
    Returns out [T][H] uint16 bf16 patterns."""
    y_bits = np.ascontiguousarray(y_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    T, K = pos.shape
    cap, H = y_bits.shape
    out = np.zeros((T, H), np.uint16)
    _check(_load().oracle_combine(T, K, H, _ptr(y_bits), cap, _ptr(pos), _ptr(weights),
                                  _ptr(out)), "combine")
    return out


Q_FP8 = 1
Q_INT8 = 2


def int8_encode(value: float) -> int:
    return int(_load().oracle_int8_encode(float(np.float32(value))))


def dispatch_quant(x_bits, ids, pos, E: int, qtype: int, cap_rows: int,
                   smooth: np.ndarray | None = None, fill_q: int = 0, fill_scale: float = 0.0,
                   q: np.ndarray | None = None, scales: np.ndarray | None = None):
    """Per-copy dynamic quantisation (optionally with per-expert smoothing
    scales [E][H] fp32).  Returns (codes [cap_rows][H] uint8, scales [cap_rows]).
    With `q` and `scales` given (C-contiguous, [cap_rows][H] uint8 and
    [cap_rows] float32) the rows are written there and the rest is kept."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    sm = None if smooth is None else np.ascontiguousarray(smooth, dtype=np.float32)
    T, H = x_bits.shape
    K = pos.shape[1]
    if q is None:
        q = np.full((cap_rows, H), fill_q, np.uint8)
    if scales is None:
        scales = np.full(cap_rows, fill_scale, np.float32)
    assert q.shape == (cap_rows, H) and q.dtype == np.uint8 and q.flags["C_CONTIGUOUS"]
    assert scales.shape == (cap_rows,) and scales.dtype == np.float32 and scales.flags["C_CONTIGUOUS"]
    sc = scales
    scratch = np.zeros(H, np.float32)
    _check(_load().oracle_dispatch_quant(T, K, E, H, _ptr(x_bits), _ptr(ids), _ptr(pos), _ptr(sm),
                                         qtype, _ptr(q), _ptr(sc), cap_rows, _ptr(scratch)),
           "dispatch_quant")
    return q, sc


def combine_quant(codes, qtype: int, scales, pos, weights) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    T, K = pos.shape
    cap, H = codes.shape
    out = np.zeros((T, H), np.uint16)
    _check(_load().oracle_combine_quant(T, K, H, _ptr(codes), qtype, _ptr(scales), cap, _ptr(pos),
                                        _ptr(weights), _ptr(out)), "combine_quant")
    return out


def f64_to_bf16_rne(value: float) -> int:
    return int(_load().oracle_f64_to_bf16_rne(float(value)))


def combine_add_rmsnorm(y_bits, pos, weights, residual_bits, gamma_bits, eps: float):
    """Combine + residual add + RMSNorm.  Returns (residual_out, norm_out),
    [T][H] uint16 bf16 patterns each."""
    y_bits = np.ascontiguousarray(y_bits, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    residual_bits = np.ascontiguousarray(residual_bits, dtype=np.uint16)
    gamma_bits = np.ascontiguousarray(gamma_bits, dtype=np.uint16)
    T, K = pos.shape
    cap, H = y_bits.shape
    ro = np.zeros((T, H), np.uint16)
    no = np.zeros((T, H), np.uint16)
    _check(_load().oracle_combine_add_rmsnorm(T, K, H, _ptr(y_bits), cap, _ptr(pos), _ptr(weights),
                                              _ptr(residual_bits), _ptr(gamma_bits), float(eps),
                                              _ptr(ro), _ptr(no)), "combine_add_rmsnorm")
    return ro, no


# ---------------------------------------------------------------- 1-D all-to-all

@dataclass
class SplitsPlan:
    src_offsets: np.ndarray   # [W][W] receiver-indexed
    out_splits: np.ndarray    # [W][W]
    dst_offsets: np.ndarray   # [W][W]
    rank_offsets: np.ndarray  # [W+1]


def a2a_plan(in_splits: np.ndarray) -> SplitsPlan:
    in_splits = np.ascontiguousarray(in_splits, dtype=np.int64)
    W = in_splits.shape[0]
    p = SplitsPlan(np.zeros((W, W), np.int64), np.zeros((W, W), np.int64),
                   np.zeros((W, W), np.int64), np.zeros(W + 1, np.int64))
    _check(_load().oracle_a2a_plan(W, _ptr(in_splits), _ptr(p.src_offsets), _ptr(p.out_splits),
                                   _ptr(p.dst_offsets), _ptr(p.rank_offsets)), "a2a_plan")
    return p


def a2a_copy(inp: np.ndarray, sp: SplitsPlan, fill: int = 0):
    """inp: [W][R][...] rows of any dtype.  Returns (out [W*R][...], err bits)."""
    inp = np.ascontiguousarray(inp)
    W, R = inp.shape[:2]
    row_bytes = inp[0, 0].nbytes
    out = np.full((W * R,) + inp.shape[2:], fill, dtype=inp.dtype)
    err = ctypes.c_uint32(0)
    _check(_load().oracle_a2a_copy(W, R, row_bytes, _ptr(inp), _ptr(sp.src_offsets),
                                   _ptr(sp.out_splits), _ptr(sp.dst_offsets),
                                   _ptr(sp.rank_offsets), _ptr(out), ctypes.byref(err)),
           "a2a_copy")
    return out, int(err.value)
