"""Pins for the oracle's 2-D exchange plan, occurrence numbers and positions.

The oracle (oracle/ep_oracle.c) computes occurrences with one counter per
(source rank, expert) bucket.  These tests check it against things fixed
independently of that code:
  * the worked occurrence example of get_occurrence_numbers (PyTorch compare
    view ciflow/h100-symm-mem/166772, test_nvshmem.py), stored in
    tests/golden/occurrence_example.json;
  * brute force over every routing of tiny inputs: occurrences by direct
    pairwise counting, positions as the rank of the copy in a stable sort of
    the live copies by expert (the layout that test_all_to_all_v_2d_index_push
    compares against: rows sorted by expert, then exchanged per expert);
  * structural invariants of the plan on random inputs.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_plan(ids, E, W, active=None):
    """Independent formulation: pairwise counting and a stable sort."""
    T, K = ids.shape
    Tw = T // W
    flat = ids.reshape(-1)
    n = flat.size
    live = np.array([(active is None or active[c // K]) and 0 <= flat[c] < E for c in range(n)])
    src = np.array([(c // K) // Tw for c in range(n)])
    occ = np.full(n, -1, np.int64)
    for c in range(n):
        if live[c]:
            occ[c] = sum(1 for c2 in range(c) if live[c2] and flat[c2] == flat[c] and src[c2] == src[c])
    order = [c for c in sorted(range(n), key=lambda c: (flat[c], c)) if live[c]]
    pos = np.full(n, -1, np.int64)
    for r, c in enumerate(order):
        pos[c] = r
    counts = np.zeros((W, E), np.int64)
    for c in range(n):
        if live[c]:
            counts[src[c], flat[c]] += 1
    return occ.reshape(T, K), pos.reshape(T, K), counts


def test_occurrence_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "occurrence_example.json")))
    ids = np.array(g["input"], np.int32).reshape(-1, 1)
    p = oracle.plan(ids, E=4, W=1)
    expected = np.array(g["docstring_output"]) - 1
    assert p.occ.reshape(-1).tolist() == expected.tolist()
    # one source rank: the position is the rank in the stable sort by expert
    assert p.pos.reshape(-1).tolist() == [0, 3, 1, 5, 2, 4]


@pytest.mark.parametrize("T,K,E,W", [(4, 1, 4, 2), (2, 2, 4, 2), (4, 1, 2, 1)])
def test_brute_force_all_routings(T, K, E, W):
    cases = 0
    for combo in itertools.product(range(E), repeat=T * K):
        ids = np.array(combo, np.int32).reshape(T, K)
        for mbits in range(1 << T):
            active = np.array([(mbits >> t) & 1 for t in range(T)], np.uint8)
            p = oracle.plan(ids, E, W, active)
            occ, pos, counts = brute_plan(ids, E, W, active)
            assert p.occ.tolist() == occ.tolist()
            assert p.pos.tolist() == pos.tolist()
            assert p.in_splits.tolist() == counts.tolist()
            assert p.err == 0
            cases += 1
    assert cases == E ** (T * K) * (1 << T)


def test_brute_force_with_invalid_ids():
    T, K, E, W = 2, 2, 2, 2
    for combo in itertools.product([-1, 0, 1, 2], repeat=T * K):
        ids = np.array(combo, np.int32).reshape(T, K)
        p = oracle.plan(ids, E, W)
        occ, pos, counts = brute_plan(ids, E, W)
        assert p.occ.tolist() == occ.tolist()
        assert p.pos.tolist() == pos.tolist()
        bad = bool(((ids < 0) | (ids >= E)).any())
        assert p.err == (oracle.DEVERR_BAD_EXPERT if bad else 0)


def check_plan_invariants(p, ids, E, W, active):
    T, K = ids.shape
    ne = E // W
    live = ((ids >= 0) & (ids < E))
    if active is not None:
        live &= active.astype(bool)[:, None]
    N = int(live.sum())
    # splits sum to the number of live copies (T*K when all are live)
    assert int(p.in_splits.sum()) == N == p.n_rows
    assert p.expert_counts.tolist() == p.in_splits.sum(axis=0).tolist()
    # offsets are exclusive scans
    assert (np.cumsum(p.expert_counts) - p.expert_counts).tolist() == p.expert_offsets.tolist()
    assert (np.cumsum(p.in_splits, axis=1) - p.in_splits).tolist() == p.src_offsets.tolist()
    # out_splits is the transpose, laid out (local expert, source rank) per destination
    assert p.out_splits.tolist() == p.in_splits.reshape(W, W, ne).transpose(1, 2, 0).tolist()
    # each destination's region holds exactly what it receives
    recv = p.out_splits.reshape(W, -1).sum(axis=1)
    assert np.diff(p.rank_offsets).tolist() == recv.tolist()
    # positions: a bijection onto [0, N), grouped by expert in flattened order
    lp = p.pos[live]
    assert sorted(lp.tolist()) == list(range(N))
    assert (p.pos[~live] == -1).all() and (p.occ[~live] == -1).all()
    flat_ids = ids.reshape(-1)
    flat_live = live.reshape(-1)
    order = np.argsort(np.where(flat_live, flat_ids, E), kind="stable")[:N]
    inv = np.empty(N, np.int64)
    inv[np.arange(N)] = order
    assert (p.pos.reshape(-1)[inv] == np.arange(N)).all()
    # pos = rank start + dst offset + occurrence
    Tw = T // W
    s = (np.arange(T) // Tw)[:, None].repeat(K, axis=1)
    e = ids.clip(0, E - 1)
    d = e // ne
    rebuilt = p.rank_offsets[d] + p.dst_offsets[s, e] + p.occ
    assert (rebuilt[live] == p.pos[live]).all()


@pytest.mark.parametrize("cfg_idx", [0])
def test_plan_invariants_config0(cfg_idx):
    cfg = workloads.WORKLOADS[cfg_idx]
    inp = workloads.moe_inputs(cfg, with_x=False)
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    check_plan_invariants(p, inp.ids, cfg.E, cfg.W, inp.active)
    occ, pos, counts = brute_plan(inp.ids, cfg.E, cfg.W, inp.active)
    assert p.occ.tolist() == occ.tolist() and p.pos.tolist() == pos.tolist()


@pytest.mark.parametrize("seed", range(6))
def test_plan_invariants_random(seed):
    rng = np.random.default_rng(100 + seed)
    W = int(rng.choice([1, 2, 4, 8]))
    E = W * int(rng.integers(1, 9))
    T = W * int(rng.integers(0, 40))
    K = int(rng.integers(1, 6))
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)  # duplicates allowed
    active = (rng.random(T) < 0.7).astype(np.uint8) if seed % 2 else None
    p = oracle.plan(ids, E, W, active)
    check_plan_invariants(p, ids, E, W, active)
    if T * K <= 400:
        occ, pos, counts = brute_plan(ids, E, W, active)
        assert p.occ.tolist() == occ.tolist() and p.pos.tolist() == pos.tolist()


def test_dst_offsets_match_destination_view():
    """dst_offsets as the destination rank sees it (make2dExchangePlan and
    test_make_a2a_2d_exchange_plan): an exclusive scan of the destination's
    (local expert, source rank) split matrix, read back per source."""
    rng = np.random.default_rng(7)
    W, ne, T, K = 4, 3, 48, 2
    E = W * ne
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    p = oracle.plan(ids, E, W)
    for d in range(W):
        mat = p.out_splits[d]                       # [ne][W]
        flat = mat.reshape(-1)
        excl = (np.cumsum(flat) - flat).reshape(ne, W)
        for le in range(ne):
            for s in range(W):
                assert p.dst_offsets[s, d * ne + le] == excl[le, s]


def test_zipf_config_has_empty_experts():
    cfg = workloads.WORKLOADS[2]
    inp = workloads.moe_inputs(cfg, with_x=False)
    p = oracle.plan(inp.ids, cfg.E, cfg.W, inp.active)
    assert int((p.expert_counts == 0).sum()) >= cfg.n_empty
    assert p.n_rows == cfg.T * cfg.K
    check_plan_invariants(p, inp.ids, cfg.E, cfg.W, inp.active)
