"""Mutation check of the oracle's pins.

Each mutant is oracle/ep_oracle.c with one plausible mistake planted (a
dropped term, an off-by-one, a transposed index, a wrong rounding or
saturation, a missing mask), compiled on the CPU with the oracle's own
flags.  The pin tests (tests/test_oracle_*.py) are run against every
mutant through EP_ORACLE_LIB, and every mutant must make at least one of
them fail: a pin set that lets a mistake through does not pin the oracle.
Nothing here touches the GPU or the HIP library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ep_oracle.c")

# (name, original text, planted text, which occurrence of the original)
MUTANTS = [
    # bf16 and E4M3FN / int8 codecs
    ("bf16 ties round up", "(dropped == 0x8000u && (keep & 1u))", "(dropped == 0x8000u)", 0),
    ("e4m3 subnormal exponent", "ldexp((double)m, -9)", "ldexp((double)m, -10)", 0),
    ("e4m3 normal bias", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 9)", 0),
    ("e4m3 saturates to NaN", "return (uint8_t)(sign | 0x7e);", "return (uint8_t)(sign | 0x7f);", 0),
    ("e4m3 ties away from zero", "pick = (lo & 1) ? hi : lo;", "pick = hi;", 0),
    ("int8 ties round up", "(fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f", "f + 1.0f", 0),
    ("int8 clamps to -128", "if (v <= -127.0f)\n        return -127;", "if (v <= -128.0f)\n        return -128;", 0),
    # plan
    ("mask ignored in split counts", "        if (active && !active[t])\n            continue;\n        int64_t s = t / Tw;",
     "        int64_t s = t / Tw;", 0),
    ("bad expert not flagged", "                flags |= ORC_DEVERR_BAD_EXPERT;\n                continue;\n            }\n            in_splits",
     "                continue;\n            }\n            in_splits", 0),
    ("expert offsets inclusive", "        expert_offsets[e] = n_live;\n        n_live += c;",
     "        n_live += c;\n        expert_offsets[e] = n_live;", 0),
    ("source offsets inclusive", "            src_offsets[(int64_t)s * E + e] = run;\n            run += in_splits[(int64_t)s * E + e];",
     "            run += in_splits[(int64_t)s * E + e];\n            src_offsets[(int64_t)s * E + e] = run;", 0),
    ("out_splits with rank roles swapped", "in_splits[(int64_t)s * E + (int64_t)d * ne + le];",
     "in_splits[(int64_t)d * E + (int64_t)s * ne + le];", 0),
    ("dst offsets without the local-expert term", "dst_offsets[(int64_t)s * E + e] = down + across;",
     "dst_offsets[(int64_t)s * E + e] = down;", 0),
    ("dst offsets count the own rank", "for (int32_t s2 = 0; s2 < s; ++s2)", "for (int32_t s2 = 0; s2 <= s; ++s2)", 0),
    ("rank offsets indexed by rank", "rank_offsets[d] = expert_offsets[(int64_t)d * ne];",
     "rank_offsets[d] = expert_offsets[d];", 0),
    ("occurrence 1-based", "int64_t o = seen[s * E + e]++;", "int64_t o = ++seen[s * E + e];", 0),
    ("position without the rank start", "pos[i] = (int32_t)(rank_offsets[e / ne] + dst_offsets[s * E + e] + o);",
     "pos[i] = (int32_t)(dst_offsets[s * E + e] + o);", 0),
    # extended plan
    ("padding of an aligned count", "int64_t padded = (c + major_align - 1) / major_align * major_align;",
     "int64_t padded = (c + major_align) / major_align * major_align;", 0),
    ("empty experts not padded", "if (pad_empty && padded == 0)", "if (0 && pad_empty && padded == 0)", 0),
    ("per-copy mask ignored", "            if (active_copies && !active_copies[i])\n                continue;\n", "", 0),
    ("token numbers types swapped", "token_nums_type == 0 ? run : c", "token_nums_type == 1 ? run : c", 0),
    ("extended dst offsets not rank-relative", "= expert_offsets[e] - rank_offsets[e / ne] + down;",
     "= expert_offsets[e] + down;", 0),
    ("extended occurrence 1-based", "int64_t o = seen[s * E + e]++;", "int64_t o = ++seen[s * E + e];", 1),
    # dispatch
    ("gate weights transposed", "expand_weights[pos[i]] = w[i];", "expand_weights[pos[i]] = w[(i % K) * T + i / K];", 0),
    ("bf16 row one value short", "memcpy(expand_x + p * H, x + t * (int64_t)H, (size_t)H * sizeof(uint16_t));",
     "memcpy(expand_x + p * H, x + t * (int64_t)H, (size_t)(H - 1) * sizeof(uint16_t));", 0),
    ("fp8 scale over 464", "float scale = amax / 448.0f;", "float scale = amax / 464.0f;", 0),
    ("fp8 amax of signed values", "float a = fabsf(oracle_bf16_to_f32(xr[h]));", "float a = oracle_bf16_to_f32(xr[h]);", 0),
    ("int8 qmax 128", "qtype == ORC_Q_FP8 ? 448.0f : 127.0f", "qtype == ORC_Q_FP8 ? 448.0f : 128.0f", 0),
    ("smoothing row of expert 0", "v = v * smooth[(int64_t)e * H + h];", "v = v * smooth[h];", 0),
    ("quantised amax of signed values", "if (fabsf(v) > amax)\n                    amax = fabsf(v);",
     "if (v > amax)\n                    amax = v;", 0),
    # combine
    ("combine without fused multiply-add", "acc = fmaf(w[t * K + k], oracle_bf16_to_f32(y[p * H + h]), acc);",
     "acc = acc + w[t * K + k] * oracle_bf16_to_f32(y[p * H + h]);", 0),
    ("combine from -0", "            float acc = 0.0f;\n            for (int32_t k = 0; k < K; ++k) {\n                int64_t p = pos[t * K + k];",
     "            float acc = -0.0f;\n            for (int32_t k = 0; k < K; ++k) {\n                int64_t p = pos[t * K + k];", 0),
    ("quantised combine without the row scale", "float v = (float)orc_decode(qtype, q[p * H + h]) * scales[p];",
     "float v = (float)orc_decode(qtype, q[p * H + h]);", 0),
    # tail
    ("double-to-bf16 ties down", "pick = (lo & 1) ? hi : lo;", "pick = lo;", 1),
    ("rms over H - 1", "sqrt(sumsq / H + (double)eps)", "sqrt(sumsq / (H - 1) + (double)eps)", 0),
    ("rms without eps", "sqrt(sumsq / H + (double)eps)", "sqrt(sumsq / H)", 0),
    ("combine not rounded before the add", "float c = oracle_bf16_to_f32(oracle_f32_to_bf16_rne(acc));", "float c = acc;", 0),
    ("norm without gamma", "oracle_f64_to_bf16_rne(hv * inv * g)", "oracle_f64_to_bf16_rne(hv * inv)", 0),
    # 1-D all-to-all
    ("a2a out_splits not transposed", "out_splits[(int64_t)r * W + p] = in_splits[(int64_t)p * W + r];",
     "out_splits[(int64_t)r * W + p] = in_splits[(int64_t)r * W + p];", 0),
    ("a2a source offsets inclusive", "for (int32_t r2 = 0; r2 < r; ++r2)", "for (int32_t r2 = 0; r2 <= r; ++r2)", 0),
    ("a2a destination offsets inclusive", "for (int32_t p2 = 0; p2 < p; ++p2)", "for (int32_t p2 = 0; p2 <= p; ++p2)", 0),
    ("a2a rank offsets inclusive", "        rank_offsets[r] = run;\n        for (int32_t p = 0; p < W; ++p)\n            run += out_splits[(int64_t)r * W + p];",
     "        for (int32_t p = 0; p < W; ++p)\n            run += out_splits[(int64_t)r * W + p];\n        rank_offsets[r] = run;", 0),
    ("a2a bad chunk not flagged", "                flags |= ORC_DEVERR_SPLITS;\n                continue;", "                continue;", 0),
]

PINS = sorted(f for f in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))
              if not f.endswith(("test_oracle_mutants.py", "test_oracle_slices.py")))


def plant(src: str, old: str, new: str, nth: int) -> str:
    at = -1
    for _ in range(nth + 1):
        at = src.find(old, at + 1)
        assert at >= 0, f"occurrence {nth} of {old!r} not in ep_oracle.c"
    return src[:at] + new + src[at + len(old):]


def build(src: str, path: str) -> None:
    c = path[:-3] + ".c"
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-o", path, c, "-lm"], check=True, capture_output=True)


def pins_pass(lib: str) -> bool:
    env = dict(os.environ, EP_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode == 0


def test_mutants_are_planted_where_intended():
    src = open(SRC).read()
    names = [m[0] for m in MUTANTS]
    assert len(names) == len(set(names))
    for name, old, new, nth in MUTANTS:
        assert plant(src, old, new, nth) != src, name


def test_every_mutant_fails_a_pin(tmp_path):
    src = open(SRC).read()
    libs = []
    for i, (name, old, new, nth) in enumerate(MUTANTS):
        lib = str(tmp_path / f"mutant{i}.so")
        build(plant(src, old, new, nth), lib)
        libs.append(lib)
    control = str(tmp_path / "control.so")
    build(src, control)
    workers = max(1, min(8, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as pool:
        passed = list(pool.map(pins_pass, [control] + libs))
    assert passed[0], "the unmodified oracle failed its pins"
    survivors = [MUTANTS[i][0] for i, ok in enumerate(passed[1:]) if ok]
    assert not survivors, f"mutants no pin rejects: {survivors}"
