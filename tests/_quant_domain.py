"""Every input of per-token dynamic quantisation without smoothing, as rows.

The dispatch quantises bf16 rows, and a row's scale depends only on its
largest magnitude A (a bf16 magnitude pattern), so the whole input domain of
one code is the set of pairs (x, A) with x a bf16 pattern and |x| <= A.  For
finite A (magnitude patterns 0 .. 0x7F7F) that is sum over A of 2 (A + 1),
about 1.07 G pairs.  The rows built here hold them all: every row starts with
A itself (so its largest magnitude is A) followed by H - 1 of A's
numerators, the x of magnitude i // 2 and sign bit i % 2 for i = 0, 1, ...,
2 A + 1, with zeros after the last one.

Only bit patterns are enumerated here; nothing of the quantisation itself.
"""
import numpy as np

A_END = 0x7F80  # magnitude patterns below this are the finite bf16 values


def rows_per_amax(a: np.ndarray, H: int) -> np.ndarray:
    """Rows needed for the 2 (A + 1) numerators of each amax pattern A."""
    return (2 * (a.astype(np.int64) + 1) + (H - 2)) // (H - 1)


def batches(H: int, max_rows: int, a_lo: int = 0, a_hi: int = A_END):
    """Consecutive ranges [lo, hi) of amax patterns, each needing at most
    max_rows rows, that together cover [a_lo, a_hi)."""
    a = np.arange(a_lo, a_hi, dtype=np.int64)
    ends = np.cumsum(rows_per_amax(a, H))
    out = []
    lo, done = a_lo, 0
    while lo < a_hi:
        # the last amax whose rows still fit in this batch
        k = int(np.searchsorted(ends, done + max_rows, side="right"))
        hi = max(a_lo + k, lo + 1)
        out.append((lo, hi))
        done = int(ends[hi - a_lo - 1])
        lo = hi
    return out


def domain_rows(a_lo: int, a_hi: int, H: int):
    """Rows [R][H] uint16 holding every (x, A) pair for A in [a_lo, a_hi),
    and each row's A."""
    a = np.arange(a_lo, a_hi, dtype=np.int32)
    n = 2 * (a + 1)                                   # numerators per amax
    per = H - 1
    reps = rows_per_amax(a, H)
    row_a = np.repeat(a, reps)
    first = np.repeat(np.cumsum(reps) - reps, reps)   # first row of each row's A
    chunk = (np.arange(row_a.size) - first).astype(np.int32)
    i = chunk[:, None] * per + np.arange(per, dtype=np.int32)[None, :]
    vals = np.where(i < np.repeat(n, reps)[:, None], (i >> 1) | ((i & 1) << 15), 0)
    x = np.empty((row_a.size, H), np.uint16)
    x[:, 0] = row_a
    x[:, 1:] = vals
    return x, row_a
