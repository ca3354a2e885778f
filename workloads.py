"""Seeded synthetic inputs for MoE dispatch / combine and the uneven all-to-all.

This module only draws random inputs; it holds none of the method's
arithmetic.  Both the HIP path (tests, bench) and the CPU oracle (tests,
bench's CPU baseline) take their inputs from here, byte for byte.

Recipes (numpy ``default_rng(seed)``; bf16 values are fp32 draws rounded to
bf16 by torch's CPU cast, a library routine):

* hidden states ``x`` [T][H]: N(0, sigma) rounded to bf16.
* routing ``ids`` [T][K] int32, K distinct experts per token:
  - "uniform": the K smallest of E iid U(0,1) keys, in key order;
  - "zipf": expert popularity p ~ (rank+1)^-s over a seeded permutation of the
    experts, the ``n_empty`` least popular experts get p = 0 (so they receive
    no token), and K distinct experts are drawn by Gumbel-top-K on log p.
* gate weights ``w`` [T][K] fp32: softmax over the K entries of N(0,1) logits
  (computed in float64, stored as float32; an input, never recomputed).
* active mask [T] uint8: Bernoulli, a token is inactive with prob ``mask_frac``.
* expert outputs ``y`` (the rows the combine reads when the dispatched rows are
  not fed back directly): N(0,1) rounded to bf16.
* 1-D send matrix [W][W] int64: randint[0,1024) per entry, three entries forced
  to 0 (one diagonal, two off-diagonal), each row rescaled to sum to R
  (floor, then the remainder to the largest fractional parts, lower index
  first on ties); rows are senders.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    E: int
    K: int
    W: int
    sigma: float = 1.0
    routing: str = "uniform"
    zipf_s: float = 1.2
    n_empty: int = 0
    mask_frac: float = 0.0
    fp8: bool = False
    seed: int = 0

    @property
    def cap_rows(self) -> int:
        return self.T * self.K


@dataclass(frozen=True)
class SplitsConfig:
    name: str
    W: int
    R: int
    H: int
    seed: int = 3
    zeros: tuple = field(default=((0, 0), (1, 4), (4, 7)))


# The five workloads of the benchmark suite.
WORKLOADS = {
    0: MoEConfig("tiny_T64_H128_E8_K2_W2", T=64, H=128, E=8, K=2, W=2, seed=0),
    1: MoEConfig("T4096_H4096_E64_K6_W8", T=4096, H=4096, E=64, K=6, W=8, seed=1),
    2: MoEConfig("T8192_H7168_E256_K8_W16_zipf1.2", T=8192, H=7168, E=256, K=8, W=16,
                 routing="zipf", zipf_s=1.2, n_empty=16, seed=2),
    3: SplitsConfig("a2a_uneven_W8_R4096_H2048", W=8, R=4096, H=2048, seed=3),
    4: MoEConfig("T16384_H7168_E256_K8_W32_mask25_fp8", T=16384, H=7168, E=256, K=8, W=32,
                 sigma=3.0, mask_frac=0.25, fp8=True, seed=4),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with torch's CPU cast; return the uint16 patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, sigma: float = 1.0,
                chunk_rows: int = 1 << 13) -> np.ndarray:
    """N(0, sigma) draws rounded to bf16, generated in row chunks."""
    shape = tuple(shape)
    out = np.empty(shape, np.uint16)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        a = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        flat[r0:r1] = bf16_bits_from_f32(a)
    return out


def routing_uniform(rng: np.random.Generator, T: int, E: int, K: int) -> np.ndarray:
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int32)


def routing_zipf(rng: np.random.Generator, T: int, E: int, K: int, s: float,
                 n_empty: int) -> np.ndarray:
    perm = rng.permutation(E)              # perm[r] = expert of popularity rank r
    p = np.zeros(E)
    p[perm] = (np.arange(E) + 1.0) ** (-s)
    if n_empty:
        p[perm[E - n_empty:]] = 0.0
    assert E - n_empty >= K, "not enough non-empty experts for K distinct picks"
    with np.errstate(divide="ignore"):
        logp = np.log(p / p.sum())
    g = rng.gumbel(size=(T, E))
    keys = logp[None, :] + g
    return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)


def gate_weights(rng: np.random.Generator, T: int, K: int) -> np.ndarray:
    logits = rng.standard_normal((T, K), dtype=np.float32).astype(np.float64)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: np.ndarray          # [T][H] uint16 (bf16 bits)
    ids: np.ndarray        # [T][K] int32
    weights: np.ndarray    # [T][K] float32
    active: np.ndarray | None  # [T] uint8 or None


def moe_inputs(cfg: MoEConfig, with_x: bool = True) -> MoEInputs:
    rng = np.random.default_rng(cfg.seed)
    if cfg.routing == "uniform":
        ids = routing_uniform(rng, cfg.T, cfg.E, cfg.K)
    elif cfg.routing == "zipf":
        ids = routing_zipf(rng, cfg.T, cfg.E, cfg.K, cfg.zipf_s, cfg.n_empty)
    else:
        raise ValueError(cfg.routing)
    w = gate_weights(rng, cfg.T, cfg.K)
    active = None
    if cfg.mask_frac > 0:
        active = (rng.random(cfg.T) >= cfg.mask_frac).astype(np.uint8)
    x = normal_bf16(rng, (cfg.T, cfg.H), cfg.sigma) if with_x else None
    return MoEInputs(cfg, x, ids, w, active)


def expert_outputs(n_rows: int, H: int, seed: int) -> np.ndarray:
    """Synthetic expert outputs: [n_rows][H] bf16 bits, N(0,1)."""
    return normal_bf16(np.random.default_rng(seed + 1000), (n_rows, H), 1.0)


def smooth_scales(E: int, H: int, seed: int) -> np.ndarray:
    """Per-expert smoothing scales [E][H] fp32: log-normal around 1 (spread
    e^0.5), the range of per-channel activation smoothing factors."""
    rng = np.random.default_rng(seed + 2000)
    return np.exp(0.5 * rng.standard_normal((E, H))).astype(np.float32)


def send_matrix(cfg: SplitsConfig) -> np.ndarray:
    rng = np.random.default_rng(cfg.seed)
    a = rng.integers(0, 1024, size=(cfg.W, cfg.W)).astype(np.int64)
    for (i, j) in cfg.zeros:
        if i < cfg.W and j < cfg.W:
            a[i, j] = 0
    out = np.zeros_like(a)
    for p in range(cfg.W):
        row = a[p].astype(np.float64)
        tot = row.sum()
        if tot == 0:
            row = np.ones(cfg.W)
            tot = float(cfg.W)
        exact = row * cfg.R / tot
        base = np.floor(exact).astype(np.int64)
        rem = cfg.R - int(base.sum())
        frac = exact - base
        order = np.lexsort((np.arange(cfg.W), -frac))  # largest fraction, lower index first
        base[order[:rem]] += 1
        for (i, j) in cfg.zeros:
            if i == p and j < cfg.W:
                assert base[j] == 0
        out[p] = base
    return out


def splits_inputs(cfg: SplitsConfig):
    """Returns (in_splits [W][W] int64, inp [W][R][H] uint16 bf16 bits)."""
    in_splits = send_matrix(cfg)
    rng = np.random.default_rng(cfg.seed + 1)
    inp = normal_bf16(rng, (cfg.W * cfg.R, cfg.H)).reshape(cfg.W, cfg.R, cfg.H)
    return in_splits, inp
