"""The rows that enumerate the quantisation domain (tests/_quant_domain.py)
cover every (x, amax) pair, and each row's largest magnitude is its amax."""
import numpy as np
import pytest

from _quant_domain import A_END, batches, domain_rows, rows_per_amax


@pytest.mark.parametrize("a_lo,a_hi,H", [(0, 300, 16), (0, 40, 4096), (32590, A_END, 4096),
                                         (1000, 1100, 272)])
def test_rows_cover_every_pair(a_lo, a_hi, H):
    x, row_a = domain_rows(a_lo, a_hi, H)
    assert x.shape == (int(rows_per_amax(np.arange(a_lo, a_hi), H).sum()), H)
    mag = (x & 0x7FFF).astype(np.int64)
    assert (mag.max(axis=1) == row_a).all()          # the row's amax is its A
    assert (x[:, 0] == row_a).all()
    for a in range(a_lo, a_hi):
        got = np.unique(x[row_a == a][:, 1:])
        want = np.unique(np.concatenate([np.arange(a + 1), np.arange(a + 1) | 0x8000]))
        assert np.array_equal(got, want), a


def test_batches_tile_the_domain():
    H, cap = 4096, 16384
    b = batches(H, cap)
    assert b[0][0] == 0 and b[-1][1] == A_END
    assert all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
    for lo, hi in b:
        assert rows_per_amax(np.arange(lo, hi), H).sum() <= cap
    total = sum(int(rows_per_amax(np.arange(lo, hi), H).sum()) for lo, hi in b)
    assert total == int(rows_per_amax(np.arange(A_END), H).sum())
    # about 1.07 G pairs in all
    pairs = int((2 * (np.arange(A_END, dtype=np.int64) + 1)).sum())
    assert pairs == A_END * (A_END + 1)
