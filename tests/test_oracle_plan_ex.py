"""Pins for the oracle's extended plan (per-copy mask, expert padding, expert
token numbers) and the gate weights carried to the expanded rows.

* Padding: the procedure test_make_a2a_2d_exchange_plan of the PyTorch compare
  view ciflow/h100-symm-mem/166772 keeps as comments -- align each local
  expert's received rows up to the alignment (at least one unit for an empty
  expert), let the expert's last source-rank chunk absorb the difference,
  exclusive-scan the destination's (local expert, source rank) list -- is
  rebuilt here with numpy from the true splits and compared with the
  oracle's destination offsets and rank sizes.
* Positions with padding: the rank of the copy in a stable sort of the live
  copies by expert, shifted by the padding of the experts before it.
* Per-copy mask (the (Bs, K) form of the CANN dispatch page's active mask):
  brute force over every mask of tiny inputs.
* Expert token numbers: counts and their inclusive prefix per rank.
"""
import itertools

import numpy as np
import pytest

import oracle


def padded_rows(counts, align, pad_empty):
    p = (counts + align - 1) // align * align
    if pad_empty:
        p = np.where(p == 0, align, p)
    return p


def brute_positions(ids, E, live, align, pad_empty):
    flat = ids.reshape(-1)
    lv = live.reshape(-1)
    counts = np.bincount(flat[lv], minlength=E)
    pads = padded_rows(counts, align, pad_empty) - counts
    shift = np.concatenate([[0], np.cumsum(pads)[:-1]])
    order = [c for c in sorted(range(flat.size), key=lambda c: (flat[c], c)) if lv[c]]
    pos = np.full(flat.size, -1, np.int64)
    for r, c in enumerate(order):
        pos[c] = r + shift[flat[c]]
    return pos.reshape(ids.shape)


def test_align_one_matches_plain_plan():
    rng = np.random.default_rng(0)
    ids = rng.integers(0, 24, size=(96, 3)).astype(np.int32)
    active = (rng.random(96) < 0.8).astype(np.uint8)
    a = oracle.plan(ids, 24, 4, active)
    b, _ = oracle.plan_ex(ids, 24, 4, active)
    for f in ("in_splits", "src_offsets", "out_splits", "dst_offsets", "expert_counts",
              "expert_offsets", "rank_offsets", "pos", "occ"):
        assert (getattr(a, f) == getattr(b, f)).all(), f


@pytest.mark.parametrize("align,pad_empty", [(1, False), (4, False), (4, True), (16, True), (3, True)])
def test_padding_follows_the_2d_plan_test_procedure(align, pad_empty):
    rng = np.random.default_rng(align)
    W, ne, T, K = 4, 6, 64, 3
    E = W * ne
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids[ids % 5 == 0] = 7        # leave some experts without rows
    p, _ = oracle.plan_ex(ids, E, W, major_align=align, pad_empty=pad_empty)
    for d in range(W):
        lst = p.out_splits[d].copy()                 # [ne][W]: (local expert, source rank)
        for i in range(ne):
            s = int(lst[i].sum())
            a = (s + align - 1) // align * align
            if pad_empty:
                a = max(a, align)
            lst[i][-1] += a - s                      # the last chunk absorbs the padding
        flat = lst.reshape(-1)
        offs = (np.cumsum(flat) - flat).reshape(ne, W)
        for i in range(ne):
            for s in range(W):
                assert p.dst_offsets[s, d * ne + i] == offs[i, s]
        assert p.rank_offsets[d + 1] - p.rank_offsets[d] == flat.sum()
    # true counts are unchanged by the padding
    assert (p.in_splits.sum(axis=0) == p.expert_counts).all()


@pytest.mark.parametrize("align,pad_empty", [(2, False), (4, True)])
def test_padded_positions_brute_force(align, pad_empty):
    rng = np.random.default_rng(5)
    T, K, E, W = 40, 3, 8, 2
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    active = (rng.random(T) < 0.75).astype(np.uint8)
    copies = (rng.random((T, K)) < 0.8).astype(np.uint8)
    p, _ = oracle.plan_ex(ids, E, W, active, copies, major_align=align, pad_empty=pad_empty)
    live = (active.astype(bool)[:, None]) & copies.astype(bool)
    assert p.pos.tolist() == brute_positions(ids, E, live, align, pad_empty).tolist()
    assert int(p.rank_offsets[-1]) == int(padded_rows(p.expert_counts, align, pad_empty).sum())


def test_per_copy_mask_brute_force():
    T, K, E, W = 2, 2, 4, 2
    for combo in itertools.product(range(E), repeat=T * K):
        ids = np.array(combo, np.int32).reshape(T, K)
        for mbits in range(1 << (T * K)):
            copies = np.array([(mbits >> i) & 1 for i in range(T * K)], np.uint8).reshape(T, K)
            p, _ = oracle.plan_ex(ids, E, W, None, copies)
            live = copies.astype(bool)
            assert p.pos.tolist() == brute_positions(ids, E, live, 1, False).tolist()
            assert (p.pos[~live] == -1).all()
            Tw = T // W
            for t in range(T):
                for k in range(K):
                    if live[t, k]:
                        same = [(t2, k2) for t2 in range(T) for k2 in range(K)
                                if (t2 * K + k2) < (t * K + k) and live[t2, k2]
                                and ids[t2, k2] == ids[t, k] and t2 // Tw == t // Tw]
                        assert p.occ[t, k] == len(same)


def test_token_mask_and_copy_mask_combine():
    ids = np.array([[0, 1], [2, 3], [1, 0]], np.int32)
    active = np.array([1, 0, 1], np.uint8)
    copies = np.array([[1, 0], [1, 1], [0, 1]], np.uint8)
    p, _ = oracle.plan_ex(ids, 4, 1, active, copies)
    assert p.pos.tolist() == [[0, -1], [-1, -1], [-1, 1]]


@pytest.mark.parametrize("typ", [0, 1])
def test_expert_token_nums(typ):
    rng = np.random.default_rng(9)
    W, ne, T, K = 4, 5, 48, 2
    E = W * ne
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    p, etn = oracle.plan_ex(ids, E, W, major_align=4, token_nums_type=typ)
    counts = np.bincount(ids.reshape(-1), minlength=E).reshape(W, ne)
    want = np.cumsum(counts, axis=1) if typ == 0 else counts
    assert etn.tolist() == want.tolist()


def test_dispatch_weights_gather():
    rng = np.random.default_rng(3)
    T, K, E, W = 32, 4, 8, 2
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    active = (rng.random(T) < 0.7).astype(np.uint8)
    w = rng.random((T, K)).astype(np.float32)
    p, _ = oracle.plan_ex(ids, E, W, active, major_align=4, pad_empty=True)
    cap = T * K + E * 4
    ew = oracle.dispatch_weights(p.pos, w, cap, fill=-1.0)
    live = p.pos >= 0
    assert (ew[p.pos[live]] == w[live]).all()
    untouched = np.setdiff1d(np.arange(cap), p.pos[live])
    assert (ew[untouched] == -1.0).all()


@pytest.mark.parametrize("align,pad_empty,seed", [(1, False, 0), (4, True, 1), (3, False, 2)])
def test_dispatch_weights_brute_force_row_order(align, pad_empty, seed):
    """expand_weights from the row order alone, without the oracle's
    positions: expandX groups the live copies by destination rank, then
    local expert (together: by expert id, e = d * E/W + le), then source rank,
    then flattened (t, k) order, which for a sort key is (e, t, k) since the
    source rank grows with t; each expert starts at the sum of the padded
    sizes of the experts before it (PyTorch compare view
    "ciflow/h100-symm-mem/166772", the 2-D exchange plan with major_align;
    expandScalesOut on the CANN dispatch page carries each copy's weight to
    its row)."""
    rng = np.random.default_rng(70 + seed)
    T, K, E, W = 48, 5, 12, 3
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids[ids == 4] = 7                                   # expert 4 left empty
    active = (rng.random(T) < 0.75).astype(np.uint8)
    copies = (rng.random((T, K)) < 0.85).astype(np.uint8)
    w = (rng.random((T, K)) + 0.5).astype(np.float32)
    live = [(int(ids[t, k]), t, k) for t in range(T) for k in range(K) if active[t] and copies[t, k]]
    live.sort()
    counts = [sum(1 for e, _, _ in live if e == x) for x in range(E)]
    sizes = [((c + align - 1) // align) * align if (c or not pad_empty) else align for c in counts]
    start = [sum(sizes[:x]) for x in range(E)]
    cap = T * K + E * align
    want = np.full(cap, -1.0, np.float32)
    seen = [0] * E
    for e, t, k in live:
        want[start[e] + seen[e]] = w[t, k]
        seen[e] += 1
    p, _ = oracle.plan_ex(ids, E, W, active, copies, major_align=align, pad_empty=pad_empty)
    got = oracle.dispatch_weights(p.pos, w, cap, fill=-1.0)
    assert (got.view(np.uint32) == want.view(np.uint32)).all()


@pytest.mark.parametrize("align,pad_empty", [(4, False), (16, True), (3, True)])
def test_padding_keeps_the_true_counts(align, pad_empty):
    """Padding moves rows, not counts: in_splits, src_offsets, out_splits and
    expert_counts of a padded plan equal those of the plain plan; the padded
    expert offsets are the exclusive scan of the padded sizes."""
    rng = np.random.default_rng(40 + align)
    T, K, E, W = 96, 4, 24, 4
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids[ids % 7 == 3] = 5                       # some experts left empty
    active = (rng.random(T) < 0.8).astype(np.uint8)
    plain = oracle.plan(ids, E, W, active)
    padded, _ = oracle.plan_ex(ids, E, W, active, major_align=align, pad_empty=pad_empty)
    for f in ("in_splits", "src_offsets", "out_splits", "expert_counts"):
        assert (getattr(padded, f) == getattr(plain, f)).all(), f
    sizes = padded_rows(plain.expert_counts, align, pad_empty)
    assert padded.expert_offsets.tolist() == (np.cumsum(sizes) - sizes).tolist()
