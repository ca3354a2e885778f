"""Python binding of libep_mi355x.so (MoE expert-parallel dispatch / combine on
one MI355X, gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream; tensors are passed as
raw device pointers to the C ABI declared in include/ep_mi355x.h, under the
same names (ep_plan, ep_dispatch, ep_combine, ep_plan_splits,
ep_dispatch_splits, ...).  There is no CPU fallback: the first call into the
library raises ImportError when libep_mi355x.so has not been built (the
package itself stays importable so that its build module can run).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from . import build as _build

_LIB_PATH = _build.LIB

EP_OK = 0
EP_ERR_NULLPTR = 1
EP_ERR_INVALID = 2
EP_ERR_UNSUPPORTED = 3
EP_ERR_WORKSPACE = 4
EP_ERR_HIP = 5

EP_BF16 = 0
EP_FP8_E4M3FN = 1
EP_INT8 = 2

EP_DEVERR_BAD_EXPERT = 1
EP_DEVERR_SPLITS = 2
EP_DEVERR_PLAN_STALL = 4
EP_DEVERR_BAD_ROW = 8

EP_PLAN_LOOKBACK = 1
EP_PLAN_TEST_STALL = 0x40000000

_STATUS_NAMES = {1: "EP_ERR_NULLPTR", 2: "EP_ERR_INVALID", 3: "EP_ERR_UNSUPPORTED",
                 4: "EP_ERR_WORKSPACE", 5: "EP_ERR_HIP"}

EXPORTED = ("ep_supported", "ep_workspace_size", "ep_workspace_init", "ep_expand_rows_bound",
            "ep_plan", "ep_plan_noalloc", "ep_dispatch", "ep_dispatch_smooth", "ep_combine", "ep_combine_quant",
            "ep_combine_add_rmsnorm", "ep_add_rmsnorm",
            "ep_plan_splits", "ep_dispatch_splits", "ep_all_to_all_splits", "ep_last_error",
            "ep_device_error")


class EPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _PlanOpts(ctypes.Structure):
    _fields_ = [("active_copies", ctypes.c_void_p), ("major_align", ctypes.c_int32),
                ("pad_empty_experts", ctypes.c_int32), ("expert_token_nums_type", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("expert_token_nums", ctypes.c_void_p)]


class _PlanT(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "in_splits", "src_offsets", "out_splits", "dst_offsets", "expert_counts",
        "expert_offsets", "rank_offsets", "pos", "occ")]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m combine_ep_plan_02_amd.build` "
            "(the HIP library has no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "ep_supported": ([i32, i32, i32, i32, i32, i32], ctypes.c_int),
        "ep_workspace_size": ([i32, i32, i32, i32], sz),
        "ep_workspace_init": ([P, sz, P], ctypes.c_int),
        "ep_expand_rows_bound": ([i32, i32, i32, i32, i32], i64),
        "ep_plan": ([i32, i32, i32, i32, P, P, ctypes.POINTER(_PlanOpts), ctypes.POINTER(_PlanT), P,
                     sz, P], ctypes.c_int),
        "ep_plan_noalloc": ([i32, i32, i32, i32, P, P, ctypes.POINTER(_PlanOpts), ctypes.POINTER(_PlanT),
                             P], ctypes.c_int),
        "ep_dispatch": ([i32, i32, i32, P, P, i32, P, P, P, P, i64, P], ctypes.c_int),
        "ep_dispatch_smooth": ([i32, i32, i32, i32, P, P, P, P, i32, P, P, i64, P], ctypes.c_int),
        "ep_combine": ([i32, i32, i32, P, i64, P, P, P, P], ctypes.c_int),
        "ep_combine_quant": ([i32, i32, i32, P, i32, P, i64, P, P, P, P], ctypes.c_int),
        "ep_combine_add_rmsnorm": ([i32, i32, i32, P, i64, P, P, P, P, ctypes.c_float, P, P, P],
                                   ctypes.c_int),
        "ep_add_rmsnorm": ([i32, i32, P, P, P, ctypes.c_float, P, P, P], ctypes.c_int),
        "ep_plan_splits": ([i32, P, P, P, P, P, P], ctypes.c_int),
        "ep_dispatch_splits": ([i32, i64, i64, P, P, P, P, P, P, P], ctypes.c_int),
        "ep_all_to_all_splits": ([i32, i64, i64, P, P, P, P, P, P, P, P], ctypes.c_int),
        "ep_last_error": ([], ctypes.c_char_p),
        "ep_device_error": ([P, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


class _LazyLib:
    """Loads libep_mi355x.so on first use; raises ImportError if it is missing."""

    _handle = None

    def __getattr__(self, name):
        if _LazyLib._handle is None:
            _LazyLib._handle = _load()
        return getattr(_LazyLib._handle, name)


lib = _LazyLib()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_DEVICE_COUNT = None


def _several_devices() -> bool:
    """More than one visible GPU (only then can a tensor be on another one)."""
    global _DEVICE_COUNT
    if _DEVICE_COUNT is None:
        _DEVICE_COUNT = torch.cuda.device_count()
    return _DEVICE_COUNT > 1


def _ptr(t: torch.Tensor | None, dtype: torch.dtype | tuple | None = None, name: str = "tensor"):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.numel() and _several_devices() and t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _check(rc: int):
    if rc != EP_OK:
        raise EPError(rc, lib.ep_last_error().decode())


def _need_numel(t: torch.Tensor | None, n: int, name: str, shape: str):
    """The kernels address `n` elements of `t` from its sizes alone, so a
    smaller tensor is refused here."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} must hold {shape} = {n} elements (has {t.numel()})")


_BITS16 = (torch.bfloat16, torch.int16, torch.uint16)
_BITS8 = (torch.float8_e4m3fn, torch.uint8, torch.int8)


# --------------------------------------------------------------------- 2-D path

def ep_supported(T: int, K: int, E: int, W: int, H: int, out_dtype: int = EP_BF16) -> bool:
    return bool(lib.ep_supported(T, K, E, W, H, out_dtype))


def ep_workspace_size(T: int, K: int, E: int, W: int) -> int:
    return int(lib.ep_workspace_size(T, K, E, W))


def ep_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    _check(lib.ep_workspace_init(_ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))


def alloc_workspace(T: int, K: int, E: int, W: int, device="cuda", stream=None) -> torch.Tensor:
    """Allocates (torch) and initialises (library fill kernel) a plan workspace."""
    n = ep_workspace_size(T, K, E, W)
    if n == 0:
        raise EPError(EP_ERR_UNSUPPORTED, f"unsupported dimensions T={T} K={K} E={E} W={W}")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    ep_workspace_init(ws, stream)
    return ws


@dataclass(frozen=True)
class Plan:
    """Device outputs of ep_plan (torch tensors allocated by the caller).
    Frozen, so the checked pointer struct can be kept for later calls."""
    in_splits: torch.Tensor
    src_offsets: torch.Tensor
    out_splits: torch.Tensor
    dst_offsets: torch.Tensor
    expert_counts: torch.Tensor
    expert_offsets: torch.Tensor
    rank_offsets: torch.Tensor
    pos: torch.Tensor
    occ: torch.Tensor | None

    def check(self, T: int, K: int, E: int, W: int) -> None:
        """Refuses outputs smaller than ep_plan writes for these dimensions."""
        for f, n, shape in (("in_splits", W * E, "[W][E]"), ("src_offsets", W * E, "[W][E]"),
                            ("out_splits", W * E, "[W][E/W][W]"), ("dst_offsets", W * E, "[W][E]"),
                            ("expert_counts", E, "[E]"), ("expert_offsets", E, "[E]"),
                            ("rank_offsets", W + 1, "[W+1]"), ("pos", T * K, "[T][K]"),
                            ("occ", T * K, "[T][K]")):
            _need_numel(getattr(self, f), n, f, shape)

    def as_struct(self, T: int, K: int, E: int, W: int) -> _PlanT:
        """The C struct of device pointers, after the size check for these
        dimensions; kept for the next call with the same dimensions and the
        same storage (a tensor moved by an in-place resize is checked again)."""
        key = (T, K, E, W) + tuple(None if getattr(self, f) is None else getattr(self, f).data_ptr()
                                   for f, _ in _PlanT._fields_)
        cached = self.__dict__.get("_struct")
        if cached is not None and cached[0] == key:
            return cached[1]
        if E > 0 and W > 0:
            self.check(T, K, E, W)
        s = _PlanT()
        for f, _ in _PlanT._fields_:
            t = getattr(self, f)
            want = torch.int32 if f in ("pos", "occ") else torch.int64
            p = _ptr(t, want, f)
            setattr(s, f, None if p is None else p.value)
        object.__setattr__(self, "_struct", (key, s))
        return s


def alloc_plan(T: int, K: int, E: int, W: int, device="cuda", with_occ: bool = True) -> Plan:
    i64 = dict(dtype=torch.int64, device=device)
    ne = E // W
    return Plan(
        in_splits=torch.empty((W, E), **i64), src_offsets=torch.empty((W, E), **i64),
        out_splits=torch.empty((W, ne, W), **i64), dst_offsets=torch.empty((W, E), **i64),
        expert_counts=torch.empty(E, **i64), expert_offsets=torch.empty(E, **i64),
        rank_offsets=torch.empty(W + 1, **i64),
        pos=torch.empty((T, K), dtype=torch.int32, device=device),
        occ=torch.empty((T, K), dtype=torch.int32, device=device) if with_occ else None)


def ep_expand_rows_bound(T: int, K: int, E: int, major_align: int = 1,
                         pad_empty_experts: bool = False) -> int:
    return int(lib.ep_expand_rows_bound(T, K, E, major_align, int(bool(pad_empty_experts))))


def _plan_opts(T, K, E, active, active_copies, major_align, pad_empty_experts, expert_token_nums,
               expert_token_nums_type, flags):
    """Checks the per-token inputs' sizes and builds ep_plan_opts_t (None
    when every option has its default)."""
    _need_numel(active, T, "active", "[T]")
    _need_numel(active_copies, T * K, "active_copies", "[T][K]")
    _need_numel(expert_token_nums, E, "expert_token_nums", "[E]")
    if (active_copies is None and major_align == 1 and not pad_empty_experts
            and expert_token_nums is None and flags == 0):
        return None
    o = _PlanOpts()
    p = _ptr(active_copies, (torch.uint8, torch.bool), "active_copies")
    o.active_copies = None if p is None else p.value
    o.major_align = int(major_align)
    o.pad_empty_experts = int(bool(pad_empty_experts))
    o.expert_token_nums_type = int(expert_token_nums_type)
    o.flags = int(flags)
    p = _ptr(expert_token_nums, torch.int64, "expert_token_nums")
    o.expert_token_nums = None if p is None else p.value
    return o


def ep_plan(topk_ids: torch.Tensor, E: int, W: int, plan: Plan, workspace: torch.Tensor,
            active: torch.Tensor | None = None, stream=None, *,
            active_copies: torch.Tensor | None = None, major_align: int = 1,
            pad_empty_experts: bool = False, expert_token_nums: torch.Tensor | None = None,
            expert_token_nums_type: int = 1, flags: int = 0) -> Plan:
    T, K = topk_ids.shape
    o = _plan_opts(T, K, E, active, active_copies, major_align, pad_empty_experts,
                   expert_token_nums, expert_token_nums_type, flags)
    st = plan.as_struct(T, K, E, W)
    _check(lib.ep_plan(T, K, E, W, _ptr(topk_ids, torch.int32, "topk_ids"),
                       _ptr(active, (torch.uint8, torch.bool), "active"),
                       None if o is None else ctypes.byref(o), ctypes.byref(st),
                       _ptr(workspace, name="workspace"),
                       workspace.numel() * workspace.element_size(), _stream(stream)))
    return plan


def ep_plan_noalloc(topk_ids: torch.Tensor, E: int, W: int, plan: Plan,
                    active: torch.Tensor | None = None, stream=None, *,
                    active_copies: torch.Tensor | None = None, major_align: int = 1,
                    pad_empty_experts: bool = False, expert_token_nums: torch.Tensor | None = None,
                    expert_token_nums_type: int = 1, flags: int = 0) -> Plan:
    """ep_plan without a workspace: the library's static per-device array
    holds the plan's state (calls that overlap on one device race)."""
    T, K = topk_ids.shape
    o = _plan_opts(T, K, E, active, active_copies, major_align, pad_empty_experts,
                   expert_token_nums, expert_token_nums_type, flags)
    st = plan.as_struct(T, K, E, W)
    _check(lib.ep_plan_noalloc(T, K, E, W, _ptr(topk_ids, torch.int32, "topk_ids"),
                               _ptr(active, (torch.uint8, torch.bool), "active"),
                               None if o is None else ctypes.byref(o), ctypes.byref(st),
                               _stream(stream)))
    return plan


def ep_dispatch(x: torch.Tensor, pos: torch.Tensor, expand_x: torch.Tensor,
                expand_scales: torch.Tensor | None = None, out_dtype: int = EP_BF16,
                stream=None, *, weights: torch.Tensor | None = None,
                expand_weights: torch.Tensor | None = None) -> None:
    T, H = x.shape
    K = pos.shape[1]
    if pos.shape[0] != T:
        raise ValueError("pos must be [T][K] for x [T][H]")
    row_dt = _BITS16 if out_dtype == EP_BF16 else _BITS8
    if expand_x.dim() != 2 or expand_x.shape[1] != H:
        raise ValueError("expand_x must be [cap_rows][H]")
    cap = expand_x.shape[0]
    if out_dtype != EP_BF16:
        _need_numel(expand_scales, cap, "expand_scales", "[cap_rows]")
    _need_numel(weights, T * K, "weights", "[T][K]")
    _need_numel(expand_weights, cap, "expand_weights", "[cap_rows]")
    _check(lib.ep_dispatch(T, K, H, _ptr(x, _BITS16, "x"), _ptr(pos, torch.int32, "pos"), out_dtype,
                           _ptr(expand_x, row_dt, "expand_x"),
                           _ptr(expand_scales, torch.float32, "expand_scales"),
                           _ptr(weights, torch.float32, "weights"),
                           _ptr(expand_weights, torch.float32, "expand_weights"),
                           expand_x.shape[0], _stream(stream)))


def ep_dispatch_smooth(x: torch.Tensor, topk_ids: torch.Tensor, pos: torch.Tensor,
                       smooth_scales: torch.Tensor, expand_x: torch.Tensor,
                       expand_scales: torch.Tensor, out_dtype: int = EP_FP8_E4M3FN,
                       stream=None) -> None:
    T, H = x.shape
    K = pos.shape[1]
    if tuple(topk_ids.shape) != (T, K) or pos.shape[0] != T:
        raise ValueError("topk_ids and pos must be [T][K] for x [T][H]")
    if smooth_scales.dim() != 2 or smooth_scales.shape[1] != H:
        raise ValueError("smooth_scales must be [E][H]")
    if expand_x.dim() != 2 or expand_x.shape[1] != H:
        raise ValueError("expand_x must be [cap_rows][H]")
    _need_numel(expand_scales, expand_x.shape[0], "expand_scales", "[cap_rows]")
    _check(lib.ep_dispatch_smooth(
        T, K, smooth_scales.shape[0], H, _ptr(x, _BITS16, "x"),
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(pos, torch.int32, "pos"),
        _ptr(smooth_scales, torch.float32, "smooth_scales"), out_dtype,
        _ptr(expand_x, _BITS8, "expand_x"), _ptr(expand_scales, torch.float32, "expand_scales"),
        expand_x.shape[0], _stream(stream)))


def ep_combine_quant(codes: torch.Tensor, row_scales: torch.Tensor, pos: torch.Tensor,
                     weights: torch.Tensor, out: torch.Tensor, code_dtype: int = EP_FP8_E4M3FN,
                     stream=None) -> None:
    T, K = pos.shape
    cap, H = codes.shape
    if tuple(out.shape) != (T, H) or tuple(weights.shape) != (T, K):
        raise ValueError("out must be [T][H] and weights [T][K]")
    if row_scales.numel() < cap:
        raise ValueError("row_scales must hold one scale per row of codes")
    _check(lib.ep_combine_quant(T, K, H, _ptr(codes, _BITS8, "codes"), code_dtype,
                                _ptr(row_scales, torch.float32, "row_scales"), cap,
                                _ptr(pos, torch.int32, "pos"),
                                _ptr(weights, torch.float32, "weights"),
                                _ptr(out, _BITS16, "out"), _stream(stream)))


def ep_combine(y: torch.Tensor, pos: torch.Tensor, weights: torch.Tensor, out: torch.Tensor,
               stream=None) -> None:
    T, K = pos.shape
    cap, H = y.shape
    if tuple(out.shape) != (T, H) or tuple(weights.shape) != (T, K):
        raise ValueError("out must be [T][H] and weights [T][K]")
    _check(lib.ep_combine(T, K, H, _ptr(y, _BITS16, "y"), cap, _ptr(pos, torch.int32, "pos"),
                          _ptr(weights, torch.float32, "weights"), _ptr(out, _BITS16, "out"),
                          _stream(stream)))


def ep_combine_add_rmsnorm(y: torch.Tensor, pos: torch.Tensor, weights: torch.Tensor,
                           residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                           residual_out: torch.Tensor, norm_out: torch.Tensor, stream=None) -> None:
    T, K = pos.shape
    cap, H = y.shape
    for n, t in (("residual", residual), ("residual_out", residual_out), ("norm_out", norm_out)):
        if tuple(t.shape) != (T, H):
            raise ValueError(f"{n} must be [T][H]")
    if tuple(gamma.shape) != (H,) or tuple(weights.shape) != (T, K):
        raise ValueError("gamma must be [H] and weights [T][K]")
    _check(lib.ep_combine_add_rmsnorm(
        T, K, H, _ptr(y, _BITS16, "y"), cap, _ptr(pos, torch.int32, "pos"),
        _ptr(weights, torch.float32, "weights"), _ptr(residual, _BITS16, "residual"),
        _ptr(gamma, _BITS16, "gamma"), float(eps), _ptr(residual_out, _BITS16, "residual_out"),
        _ptr(norm_out, _BITS16, "norm_out"), _stream(stream)))


def ep_add_rmsnorm(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                   residual_out: torch.Tensor, norm_out: torch.Tensor, stream=None) -> None:
    T, H = x.shape
    for n, t in (("residual", residual), ("residual_out", residual_out), ("norm_out", norm_out)):
        if tuple(t.shape) != (T, H):
            raise ValueError(f"{n} must be [T][H]")
    if tuple(gamma.shape) != (H,):
        raise ValueError("gamma must be [H]")
    _check(lib.ep_add_rmsnorm(T, H, _ptr(x, _BITS16, "x"), _ptr(residual, _BITS16, "residual"),
                              _ptr(gamma, _BITS16, "gamma"), float(eps),
                              _ptr(residual_out, _BITS16, "residual_out"),
                              _ptr(norm_out, _BITS16, "norm_out"), _stream(stream)))


# --------------------------------------------------------------------- 1-D path

@dataclass
class SplitsPlan:
    src_offsets: torch.Tensor
    out_splits: torch.Tensor
    dst_offsets: torch.Tensor
    rank_offsets: torch.Tensor


def alloc_splits_plan(W: int, device="cuda") -> SplitsPlan:
    i64 = dict(dtype=torch.int64, device=device)
    return SplitsPlan(torch.empty((W, W), **i64), torch.empty((W, W), **i64),
                      torch.empty((W, W), **i64), torch.empty(W + 1, **i64))


def _check_splits_plan(plan: SplitsPlan, W: int):
    for f, n, shape in (("src_offsets", W * W, "[W][W]"), ("out_splits", W * W, "[W][W]"),
                        ("dst_offsets", W * W, "[W][W]"), ("rank_offsets", W + 1, "[W+1]")):
        _need_numel(getattr(plan, f), n, f, shape)


def ep_plan_splits(in_splits: torch.Tensor, plan: SplitsPlan, stream=None) -> SplitsPlan:
    W = in_splits.shape[0]
    if tuple(in_splits.shape) != (W, W):
        raise ValueError("in_splits must be [W][W]")
    _check_splits_plan(plan, W)
    _check(lib.ep_plan_splits(W, _ptr(in_splits, torch.int64, "in_splits"),
                              _ptr(plan.src_offsets, torch.int64, "src_offsets"),
                              _ptr(plan.out_splits, torch.int64, "out_splits"),
                              _ptr(plan.dst_offsets, torch.int64, "dst_offsets"),
                              _ptr(plan.rank_offsets, torch.int64, "rank_offsets"), _stream(stream)))
    return plan


def ep_dispatch_splits(inp: torch.Tensor, plan: SplitsPlan, out: torch.Tensor, stream=None) -> None:
    """inp [W][R][...] rows, out [W*R][...] rows of the same row size."""
    W, R = inp.shape[:2]
    stride = inp[0, 0].numel() * inp.element_size() if R else 16
    if out.shape[0] != W * R or (R and out[0].numel() * out.element_size() != stride):
        raise ValueError("out must hold W*R rows of the input's row size")
    _check_splits_plan(plan, W)
    _check(lib.ep_dispatch_splits(W, R, stride, _ptr(inp, name="in"),
                                  _ptr(plan.src_offsets, torch.int64, "src_offsets"),
                                  _ptr(plan.out_splits, torch.int64, "out_splits"),
                                  _ptr(plan.dst_offsets, torch.int64, "dst_offsets"),
                                  _ptr(plan.rank_offsets, torch.int64, "rank_offsets"),
                                  _ptr(out, name="out"), _stream(stream)))


def ep_all_to_all_splits(in_splits: torch.Tensor, inp: torch.Tensor, out: torch.Tensor,
                         plan: SplitsPlan | None = None, stream=None) -> None:
    """Plan and data move of the 1-D all-to-all in one launch; fills `plan`
    (optional) with what ep_plan_splits computes."""
    W, R = inp.shape[:2]
    if tuple(in_splits.shape) != (W, W):
        raise ValueError("in_splits must be [W][W]")
    stride = inp[0, 0].numel() * inp.element_size() if R else 16
    if out.shape[0] != W * R or (R and out[0].numel() * out.element_size() != stride):
        raise ValueError("out must hold W*R rows of the input's row size")
    if plan is not None:
        _check_splits_plan(plan, W)
    g = (lambda f: _ptr(getattr(plan, f), torch.int64, f)) if plan is not None else (lambda f: None)
    _check(lib.ep_all_to_all_splits(W, R, stride, _ptr(in_splits, torch.int64, "in_splits"),
                                    _ptr(inp, name="in"), _ptr(out, name="out"), g("src_offsets"),
                                    g("out_splits"), g("dst_offsets"), g("rank_offsets"),
                                    _stream(stream)))


def ep_device_error(stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(lib.ep_device_error(_stream(stream), ctypes.byref(code)))
    return int(code.value)


def library_path() -> str:
    return _LIB_PATH
