"""Benchmark: MoE expert-parallel dispatch + combine on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload N] [--gpus 1]

With no --workload, the line is the T=16384, H=7168, E=256, K=8, W=32 step
(25% of tokens masked, per-token fp8 dispatch, bf16 combine) with the
T=8192, H=7168, E=256, K=8, W=16 Zipf step's whole record nested in it
("also_measured"): the two largest MoE workloads.

One step is the whole hot path over one batch of resident synthetic input:
ep_plan (split counts, scans, exchange plan, stable positions) -> ep_dispatch
(scatter into the expert-grouped expandX buffer; per-token fp8 for the fp8
workload) -> ep_combine (weighted gather of the K expert rows per token).
The uneven all-to-all workload times ep_all_to_all_splits (plan and data move
in one launch), with the two-launch form ep_plan_splits -> ep_dispatch_splits
timed beside it.

Prints one JSON line: whole-job tokens/s, the step's algorithmic HBM GB/s,
a roofline record for the dominant kernel (its algorithmic bytes per launch
over its average launch time, HIP events on the launch stream) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD's published peak
CPU_BUDGET_S = 20.0      # the CPU oracle baseline stops repeating past this
METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU"

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch; FETCH_SIZE scaled by 2.0 and WRITE_SIZE by
# 1.0, the factors a plain 1 GiB copy gives), see profiles/.  They describe
# the kernels built from the sources whose digest is `source_sha256` (code
# only, comments and whitespace aside); any other build reports traffic as
# null until the counters are taken again.
TRAFFIC = {
    "source_sha256": "3e2b8e20a40b8db1ee881ece0c6f4da6b883db66a28b65a6608e02955d22aabf",
    "bytes_per_launch": {   # {workload: {phase: bytes}}
        "1": {"ep_plan": 652247, "ep_dispatch": 235782197, "ep_combine": 236513930, "ep_plan_lookback": 965702, "ep_dispatch_smooth": 144423938, "ep_combine_quant": 138720556, "ep_dispatch_int8": 135638980, "ep_combine_quant_int8": 138584940},
        "2": {"ep_plan": 1961759, "ep_dispatch": 1059626988, "ep_combine": 1061201583, "ep_plan_lookback": 2485401, "ep_dispatch_smooth": 876113336, "ep_combine_quant": 600660225, "ep_dispatch_int8": 590466904, "ep_combine_quant_int8": 600736065, "ep_combine_add_rmsnorm": 1294119130, "ep_add_rmsnorm": 469944925},
        "3": {"ep_all_to_all_splits": 268838617, "ep_plan_splits": 5856, "ep_dispatch_splits": 268576667},
        "4": {"ep_plan": 3595139, "ep_dispatch": 885888414, "ep_combine": 1652703245, "ep_plan_lookback": 4564602, "ep_dispatch_smooth": 2301502849, "ep_combine_quant": 969073055, "ep_dispatch_int8": 885969099, "ep_combine_quant_int8": 968471102, "ep_combine_add_rmsnorm": 2118405266, "ep_add_rmsnorm": 939700448},
    },
}


def source_digest() -> str:
    """sha256 of the library's sources with comments and whitespace removed
    (what the compiler sees), so a comment edit keeps the measured traffic."""
    import hashlib
    import re
    d = os.path.join(ROOT, "combine_ep_plan_02_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip")):
            text = open(os.path.join(d, name), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(name.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: int, phase: str):
    if TRAFFIC["source_sha256"] != source_digest():
        return None
    return TRAFFIC["bytes_per_launch"].get(str(workload), {}).get(phase)


def host_cpu() -> dict:
    """The host the CPU baseline ran on: model name and visible threads."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cpu": model, "host_threads": os.cpu_count()}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=None, choices=[0, 1, 2, 3, 4],
                    help="index of the workload to time alone (default: 4, T=16384 H=7168 E=256 "
                         "K=8 W=32 with 25%% masked tokens and fp8 dispatch, as the headline, with "
                         "2, T=8192 H=7168 E=256 K=8 W=16 Zipf, measured after it and nested in "
                         "the same line; 0: the T=64 latency case)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step into a HIP graph and time its replays (no host "
                         "launch cost per kernel; what a launch-bound small step needs)")
    ap.add_argument("--tail", action="store_true",
                    help="end the step with the fused combine + residual add + RMSNorm tail "
                         "(ep_combine_add_rmsnorm) instead of ep_combine; the unfused pair "
                         "ep_combine + ep_add_rmsnorm is timed beside it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=5)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (a known-size "
                         "reference for the HBM byte counters) and exit")
    return ap.parse_args()


# --------------------------------------------------------------------------- MoE

class MoEBench:
    def __init__(self, cfg, torch, ep, workloads, tail=False):
        self.cfg, self.torch, self.ep = cfg, torch, ep
        self.tail = tail
        log(f"[bench] generating inputs for {cfg.name}")
        inp = workloads.moe_inputs(cfg)
        self.inp = inp
        dev = "cuda"
        t = torch
        self.ids = t.from_numpy(inp.ids).to(dev)
        self.x = t.from_numpy(inp.x.view(np.int16)).to(dev)
        self.w = t.from_numpy(inp.weights).to(dev)
        self.active = None if inp.active is None else t.from_numpy(inp.active).to(dev)
        self.ws = ep.alloc_workspace(cfg.T, cfg.K, cfg.E, cfg.W)
        self.plan = ep.alloc_plan(cfg.T, cfg.K, cfg.E, cfg.W)
        cap = cfg.cap_rows
        if cfg.fp8:
            self.ex = t.empty((cap, cfg.H), dtype=t.uint8, device=dev)
            self.scales = t.empty(cap, dtype=t.float32, device=dev)
            # bf16 expert outputs in expandX layout: what the combine reads back
            g = t.Generator(device=dev)
            g.manual_seed(cfg.seed + 1000)
            self.y = t.empty((cap, cfg.H), dtype=t.bfloat16, device=dev)
            for r0 in range(0, cap, 8192):
                self.y[r0:r0 + 8192].normal_(generator=g)
            self.y = self.y.view(t.int16)
        else:
            self.ex = t.empty((cap, cfg.H), dtype=t.int16, device=dev)
            self.scales = None
            self.y = self.ex          # identity expert: combine reads the dispatched rows
        self.out = t.empty((cfg.T, cfg.H), dtype=t.int16, device=dev)
        self.out_dtype = ep.EP_FP8_E4M3FN if cfg.fp8 else ep.EP_BF16
        if tail:
            g = t.Generator(device=dev)
            g.manual_seed(cfg.seed + 2000)
            self.residual = t.empty((cfg.T, cfg.H), dtype=t.bfloat16, device=dev).normal_(generator=g)
            self.residual = self.residual.view(t.int16)
            self.gamma = (1 + 0.1 * t.randn(cfg.H, generator=g, device=dev)).to(t.bfloat16).view(t.int16)
            self.res_out = t.empty((cfg.T, cfg.H), dtype=t.int16, device=dev)
            self.norm_out = t.empty((cfg.T, cfg.H), dtype=t.int16, device=dev)
        # the quantisation variants timed beside the step: smoothed fp8
        # dispatch (per-expert scales [E][H]) and the combine of fp8 expert rows
        self.smooth = t.from_numpy(workloads.smooth_scales(cfg.E, cfg.H, cfg.seed)).to(dev)
        if cfg.fp8:
            self.qx, self.qs = self.ex, self.scales
        else:
            self.qx = t.empty((cap, cfg.H), dtype=t.uint8, device=dev)
            self.qs = t.empty(cap, dtype=t.float32, device=dev)
        # sizes for the byte accounting
        live_tok = cfg.T if inp.active is None else int(inp.active.sum())
        self.live_tokens = live_tok

    def plan_step(self):
        self.ep.ep_plan(self.ids, self.cfg.E, self.cfg.W, self.plan, self.ws, self.active)

    def plan_lookback_step(self):
        self.ep.ep_plan(self.ids, self.cfg.E, self.cfg.W, self.plan, self.ws, self.active,
                        flags=self.ep.EP_PLAN_LOOKBACK)

    def dispatch_step(self):
        self.ep.ep_dispatch(self.x, self.plan.pos, self.ex, self.scales, out_dtype=self.out_dtype)

    def combine_step(self):
        self.ep.ep_combine(self.y, self.plan.pos, self.w, self.out)

    def tail_step(self):
        self.ep.ep_combine_add_rmsnorm(self.y, self.plan.pos, self.w, self.residual, self.gamma,
                                       1e-6, self.res_out, self.norm_out)

    def add_rmsnorm_step(self):
        self.ep.ep_add_rmsnorm(self.out, self.residual, self.gamma, 1e-6, self.res_out,
                               self.norm_out)

    def dispatch_smooth_step(self):
        self.ep.ep_dispatch_smooth(self.x, self.ids, self.plan.pos, self.smooth, self.qx, self.qs,
                                   out_dtype=self.ep.EP_FP8_E4M3FN)

    def combine_quant_step(self):
        self.ep.ep_combine_quant(self.qx, self.qs, self.plan.pos, self.w, self.out,
                                 code_dtype=self.ep.EP_FP8_E4M3FN)

    def dispatch_int8_step(self):
        self.ep.ep_dispatch(self.x, self.plan.pos, self.qx, self.qs, out_dtype=self.ep.EP_INT8)

    def combine_int8_step(self):
        self.ep.ep_combine_quant(self.qx, self.qs, self.plan.pos, self.w, self.out,
                                 code_dtype=self.ep.EP_INT8)

    def phases(self):
        last = ("ep_combine_add_rmsnorm", self.tail_step) if self.tail else \
            ("ep_combine", self.combine_step)
        return [("ep_plan", self.plan_step), ("ep_dispatch", self.dispatch_step), last]

    def extra_phases(self):
        """Kernels timed beside the step: the plan forced onto its look-back
        path, the quantisation variants (smoothed fp8 dispatch, combine of fp8
        expert rows, int8 dispatch and combine of int8 rows) and, with the
        tail, the unfused tail pair."""
        ph = [("ep_plan_lookback", self.plan_lookback_step),
              ("ep_dispatch_smooth", self.dispatch_smooth_step),
              ("ep_combine_quant", self.combine_quant_step),
              ("ep_dispatch_int8", self.dispatch_int8_step),
              ("ep_combine_quant_int8", self.combine_int8_step)]
        if self.tail:
            ph += [("ep_combine", self.combine_step), ("ep_add_rmsnorm", self.add_rmsnorm_step)]
        return ph

    def n_rows(self):
        return int(self.plan.rank_offsets[-1].item())

    def bytes_per_phase(self, N):
        """Algorithmic HBM bytes: what the method must read and write once."""
        c = self.cfg
        tk = c.T * c.K
        mask_b = 0 if self.inp.active is None else c.T
        plan_b = tk * 4 + mask_b + tk * 4 + tk * 4          # ids in; pos, occ out
        row_in = 2 * c.H
        row_out = c.H if c.fp8 else 2 * c.H
        disp_b = self.live_tokens * row_in + N * row_out + tk * 4 + (N * 4 if c.fp8 else 0)
        comb_b = N * 2 * c.H + c.T * 2 * c.H + tk * 4 * 2    # rows in, out rows, pos + weights
        # fused tail: rows in, residual in, residual_out + norm_out, gamma, pos + weights
        tail_b = N * 2 * c.H + 3 * c.T * 2 * c.H + 2 * c.H + tk * 4 * 2
        addn_b = 4 * c.T * 2 * c.H + 2 * c.H                  # x, residual in; two rows out
        # smoothed fp8 dispatch: x rows, the [E][H] fp32 scales once, codes +
        # row scales out, ids + pos; fp8 combine: codes + row scales in, out rows
        smooth_b = self.live_tokens * row_in + c.E * c.H * 4 + N * (c.H + 4) + tk * 4 * 2
        combq_b = N * (c.H + 4) + c.T * 2 * c.H + tk * 4 * 2
        return {"ep_plan": plan_b, "ep_plan_lookback": plan_b, "ep_dispatch": disp_b, "ep_combine": comb_b,
                "ep_combine_add_rmsnorm": tail_b, "ep_add_rmsnorm": addn_b,
                "ep_dispatch_smooth": smooth_b, "ep_combine_quant": combq_b,
                "ep_dispatch_int8": self.live_tokens * row_in + N * (c.H + 4) + tk * 4,
                "ep_combine_quant_int8": combq_b}

    def tokens(self):
        return self.cfg.T

    def live_tokens_count(self):
        return self.live_tokens if self.inp.active is not None else None

    def config_record(self):
        c = self.cfg
        return {"workload": c.name + ("+add_rmsnorm_tail" if self.tail else ""),
                "T": c.T, "H": c.H, "E": c.E, "K": c.K, "W": c.W,
                "routing": c.routing + (f"(s={c.zipf_s}, {c.n_empty} empty experts)"
                                        if c.routing == "zipf" else ""),
                "sigma": c.sigma, "mask_frac": c.mask_frac,
                "dispatch_rows": "fp8_e4m3fn+fp32 scale" if c.fp8 else "bf16",
                "combine_rows": "bf16", "accumulate": "fp32"}

    def dtype(self):
        return "fp8e4m3+bf16" if self.cfg.fp8 else "bf16"

    def cpu_baseline(self, reps):
        """The serial C oracle on the host: the whole plan, then dispatch and
        combine of a bounded sample of tokens (all of them for bf16 rows; the
        first 512 for fp8 rows, whose definitional encoder is slow), scaled
        to tokens/s; repeated up to `reps` times within CPU_BUDGET_S seconds."""
        import oracle
        c, inp = self.cfg, self.inp
        nt = c.T if not c.fp8 else min(c.T, 512)
        p0 = oracle.plan(inp.ids, c.E, c.W, inp.active)
        sub = p0.pos[:nt].copy()
        live = sub >= 0
        sub[live] = np.arange(int(live.sum()), dtype=np.int32)   # the sample's rows, compacted
        m = int(live.sum())
        yrows = workloads_expert_rows(m, c.H, c.seed) if c.fp8 else None
        xs, ws = np.ascontiguousarray(inp.x[:nt]), np.ascontiguousarray(inp.weights[:nt])
        times = []
        spent = 0.0
        for _ in range(reps):
            if times and spent * (len(times) + 1) / len(times) > CPU_BUDGET_S:
                break
            t0 = time.perf_counter()
            p = oracle.plan(inp.ids, c.E, c.W, inp.active)
            t1 = time.perf_counter()
            if c.fp8:
                q, sc = oracle.dispatch_fp8(xs, sub, m)
                out = oracle.combine(yrows, sub, ws)
                del q, sc, out
            else:
                ex = oracle.dispatch_bf16(xs, sub, m)
                out = oracle.combine(ex, sub, ws)
                del ex, out
            t2 = time.perf_counter()
            times.append((t1 - t0) + (t2 - t1) * c.T / nt)
            spent += t2 - t0
            del p
        sec = float(np.median(times))
        return {"value": c.T / sec, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"plan of all {c.T} tokens + dispatch/combine of {nt} tokens "
                          f"(scaled to {c.T}); serial C oracle, one host thread, median of "
                          f"{len(times)}",
                "seconds_per_step": sec}


def workloads_expert_rows(n, H, seed):
    import workloads
    return workloads.expert_outputs(n, H, seed)


# --------------------------------------------------------------------------- 1-D

class SplitsBench:
    def __init__(self, cfg, torch, ep, workloads):
        self.cfg, self.torch, self.ep = cfg, torch, ep
        log(f"[bench] generating inputs for {cfg.name}")
        send, inp = workloads.splits_inputs(cfg)
        self.send_np, self.inp_np = send, inp
        self.send = torch.from_numpy(send).cuda()
        self.inp = torch.from_numpy(inp.view(np.int16)).cuda()
        self.sp = ep.alloc_splits_plan(cfg.W)
        self.out = torch.empty((cfg.W * cfg.R, cfg.H), dtype=torch.int16, device="cuda")

    def phases(self):
        """One launch: the plan and the data move fused (ep_all_to_all_splits)."""
        return [("ep_all_to_all_splits",
                 lambda: self.ep.ep_all_to_all_splits(self.send, self.inp, self.out, self.sp))]

    def extra_phases(self):
        """The two-launch form timed beside it: plan, then move."""
        return [("ep_plan_splits", lambda: self.ep.ep_plan_splits(self.send, self.sp)),
                ("ep_dispatch_splits", lambda: self.ep.ep_dispatch_splits(self.inp, self.sp, self.out))]

    def n_rows(self):
        return self.cfg.W * self.cfg.R

    def bytes_per_phase(self, N):
        c = self.cfg
        W = c.W
        return {"ep_plan_splits": W * W * 8 * 4 + (W + 1) * 8,
                "ep_dispatch_splits": 2 * N * c.H * 2 + 4 * W * W * 8,
                "ep_all_to_all_splits": 2 * N * c.H * 2 + W * W * 8 * 4 + (W + 1) * 8}

    def tokens(self):
        return self.cfg.W * self.cfg.R   # rows moved

    def live_tokens_count(self):
        return None

    def config_record(self):
        c = self.cfg
        return {"workload": c.name, "W": c.W, "R": c.R, "H": c.H, "splits": "randint[0,1024) rescaled"}

    def dtype(self):
        return "bf16"

    def cpu_baseline(self, reps):
        import oracle
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            sp = oracle.a2a_plan(self.send_np)
            out, _ = oracle.a2a_copy(self.inp_np, sp)
            times.append(time.perf_counter() - t0)
            del out
        sec = float(np.median(times))
        n = self.cfg.W * self.cfg.R
        return {"value": n / sec, "unit": "rows/s", "cores": 1, "kind": "oracle",
                "sample": f"whole workload ({n} rows), serial C oracle, median of {reps}",
                "seconds_per_step": sec}


# --------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the W expert-parallel "
                          "ranks are emulated as buffers in one GPU's HBM; run with --gpus 1"}),
              flush=True)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return
    import combine_ep_plan_02_amd as ep
    import workloads

    if args.workload is not None:
        rec = measure(args.workload, args, torch, ep, workloads)
    else:
        # The two largest MoE workloads: the T=16384 fp8 one as the headline,
        # the T=8192 Zipf one measured after it, in full, and nested in the
        # same line.
        rec = measure(4, args, torch, ep, workloads)
        torch.cuda.empty_cache()
        rec["also_measured"] = [measure(2, args, torch, ep, workloads)]
    print(json.dumps(rec), flush=True)


def measure(workload, args, torch, ep, workloads):
    """Times one workload; returns its JSON record."""
    cfg = workloads.WORKLOADS[workload]
    if workload == 3:
        bench = SplitsBench(cfg, torch, ep, workloads)
    else:
        bench = MoEBench(cfg, torch, ep, workloads, tail=args.tail)
    phases = bench.phases()
    stream = torch.cuda.current_stream()

    def step():
        for _, fn in phases:
            fn()

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert ep.ep_device_error() == 0
    eager_step = step
    if args.graph:
        # The library enqueues kernels only (no allocation, memset or host
        # read-back), so the whole step is captured once and replayed.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step()
        torch.cuda.synchronize()
        step = graph.replay
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        assert ep.ep_device_error() == 0

    # Timed region: exactly `steps` steps, synchronised on both sides.
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Cold steps: before every step the 256 MB Infinity Cache is refilled with
    # clean lines of an unrelated 512 MB buffer (a read-only reduction, not
    # timed, after one synchronisation), so no input or output of the
    # previous step is served from it and no dirty line is left to write back.
    log("[bench] cold steps")
    scratch = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    cold = []
    for _ in range(args.steps):
        scratch.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        cold.append((a, b))
    torch.cuda.synchronize()
    cold_list = [a.elapsed_time(b) for a, b in cold]
    cold_ms = float(np.mean(cold_list))
    del scratch

    # Warm steps, one event pair each, for the spread (the wall-clock figure
    # above is the headline; these add the events' own cost per step).
    warm = []
    for _ in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        warm.append((a, b))
    torch.cuda.synchronize()
    warm_list = [a.elapsed_time(b) for a, b in warm]

    # The same steps with an event after each phase as well (eager mode):
    # every kernel's duration inside whole steps, event to event.  Each such
    # figure includes the kernel's launch gap and the event's own cost (~4 us
    # measured on MI355X: an event between two kernels waits for the first to
    # drain), so it is context, and these events stay out of the timings above.
    step_phase_ms = None
    if not args.graph:
        marks = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
                 for _ in range(args.steps)]
        for e in marks:
            e[0].record(stream)
            for j, (_, fn) in enumerate(phases):
                fn()
                e[j + 1].record(stream)
        torch.cuda.synchronize()
        step_phase_ms = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in marks]))
                         for j, (name, _) in enumerate(phases)}

    def spread(ms):
        return {f"p{q}": float(np.percentile(ms, q)) * 1e3 for q in (10, 50, 90)}

    # Per-launch durations: each phase launched `steps` times back to back
    # between two HIP events recorded on the launch stream; the average is
    # the launch duration (one event pair per batch keeps the events' own
    # cost out of the figure).
    log("[bench] per-phase timing")
    phase_ms = {}
    for name, fn in phases + bench.extra_phases():
        fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        phase_ms[name] = a.elapsed_time(b) / args.steps
    eager_step()  # leave the buffers in the state of one whole step
    torch.cuda.synchronize()

    # Cold launches of each step kernel: the Infinity Cache refilled with
    # clean lines of an unrelated 512 MB buffer before every launch, as for
    # the cold steps, one event pair around each launch.
    log("[bench] cold per-phase timing")
    scratch = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    phase_cold_ms = {}
    for name, fn in phases:
        ev = []
        for _ in range(args.steps):
            scratch.sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        phase_cold_ms[name] = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    del scratch
    eager_step()
    torch.cuda.synchronize()
    assert ep.ep_device_error() == 0

    N = bench.n_rows()
    bpp = bench.bytes_per_phase(N)
    step_names = [n for n, _ in phases]
    step_bytes = sum(bpp[n] for n in step_names)
    # The roofline's kernel duration is its per-phase batch average (HIP
    # events on the launch stream around `steps` back-to-back launches, no
    # event between launches).  rocprofv3 traces of the same command give
    # that launch duration within 0.1%, and the same kernel's duration inside
    # whole steps within 1% of it.
    dominant = max(step_names, key=phase_ms.get)
    ach = bpp[dominant] / (phase_ms[dominant] * 1e-3) / 1e9
    tokens = bench.tokens()
    rec = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s" if workload != 3 else "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": bench.dtype(), "data": "synthetic (seeded numpy generators, see workloads.py)",
        "config": bench.config_record() | ({"launch": "hip_graph_replay"} if args.graph else {}),
        "hbm_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "cold_ms_per_step": cold_ms,
        "warm_step_us": spread(warm_list),
        "cold_step_us": spread(cold_list),
        "cold_hbm_gbps": step_bytes / (cold_ms * 1e-3) / 1e9,
        "hbm_frac_of_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "cold_hbm_frac_of_peak": step_bytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "cache_note": "warm steps (value, ms_per_step, hbm_*) reuse one input batch, whose x rows "
                      "the 256 MB Infinity Cache largely keeps between steps; cold_* figures "
                      "refill that cache with an unrelated buffer before every step or launch",
        "algorithmic_bytes_per_step": step_bytes,
        "rows_N": N,
        "source_sha256": source_digest(),
        "phase_us": {k: v * 1e3 for k, v in phase_ms.items()},
        "step_phase_us": ({k: v * 1e3 for k, v in step_phase_ms.items()}
                          if step_phase_ms is not None else None),
        "phase_gbps": {k: bpp[k] / (phase_ms[k] * 1e-3) / 1e9 for k in phase_ms},
        "phase_algorithmic_bytes": {k: bpp[k] for k in phase_ms},
        "phase_cold_us": {k: v * 1e3 for k, v in phase_cold_ms.items()},
        "phase_fabric_bytes": {k: measured_traffic(workload, k) for k in phase_ms},
        "fabric_bytes_note": "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch (L2 fills and "
                             "write-backs over the fabric, Infinity Cache hits included), "
                             "scaled by a plain copy's counts; null for other library sources",
        "step_phases": step_names,
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(workload, dominant),
                     "algorithmic_bytes_per_launch": bpp[dominant],
                     "duration_us": phase_ms[dominant] * 1e3,
                     "cold_duration_us": phase_cold_ms[dominant] * 1e3,
                     "cold_achieved": bpp[dominant] / (phase_cold_ms[dominant] * 1e-3) / 1e9,
                     "cold_frac": bpp[dominant] / (phase_cold_ms[dominant] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "in_step_event_us": (step_phase_ms[dominant] * 1e3
                                          if step_phase_ms is not None else None)},
    }
    live = bench.live_tokens_count()
    if live is not None:
        rec["live_tokens_per_s"] = live / (ms_per_step * 1e-3)
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        # the serial oracle runs pinned to one of the process's cores
        allowed = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(allowed)})
        try:
            rec["cpu_baseline"] = bench.cpu_baseline(args.cpu_reps) | host_cpu() | {"pinned_core": min(allowed)}
        finally:
            os.sched_setaffinity(0, allowed)
    del bench
    return rec


if __name__ == "__main__":
    main()
