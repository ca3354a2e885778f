"""Pins for the oracle's 1-D uneven all_to_all_single (plan + data move).

* The worked example of aws-neuron/torch-neuronx PR #1035 (section Testing):
  two ranks, send matrix [[1, 3], [2, 2]], row k of rank i holding 10*i + k,
  input [4, 8] -> rank 0 receives [0, 10, 11], rank 1 receives
  [1, 2, 3, 12, 13] (tests/golden/a2a_two_rank_example.json).
* A zero-row chunk (the same PR's updated test covers one).
* A second, independent formulation: the PR's padded-even lowering (pad each
  chunk to the input row count, one even all-to-all, trim by the receiver's
  output splits), written here with numpy and compared with the oracle.
* The plan identities of test_make_a2a_exchange_plan (PyTorch compare view
  ciflow/h100-symm-mem/166772): out_splits is the all-to-all (transpose) of
  the input splits, src_offsets the all-to-all of their exclusive scan,
  dst_offsets the exclusive scan of out_splits.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rows_10i_plus_k(W, R, width):
    inp = np.zeros((W, R, width), np.int32)
    for i in range(W):
        for k in range(R):
            inp[i, k, :] = 10 * i + k
    return inp


def per_rank(out, sp, r):
    return out[sp.rank_offsets[r]: sp.rank_offsets[r + 1]]


def padded_even_all_to_all(inp, send):
    """The padded-even lowering: sender p cuts its rows by its own input
    splits and pads every chunk to R rows; one even all-to-all moves chunk
    (p -> r) to rank r; receiver r trims each chunk by its output splits."""
    W, R = inp.shape[:2]
    padded = np.zeros((W, W, R) + inp.shape[2:], inp.dtype)   # [sender][dest][R]
    for p in range(W):
        start = 0
        for r in range(W):
            n = send[p, r]
            padded[p, r, :n] = inp[p, start:start + n]
            start += n
    received = padded.transpose(1, 0, *range(2, padded.ndim))  # [dest][sender][R]
    outs = []
    for r in range(W):
        outs.append(np.concatenate([received[r, p, : send[p, r]] for p in range(W)], axis=0))
    return outs


def test_worked_example_two_ranks():
    g = json.load(open(os.path.join(GOLDEN, "a2a_two_rank_example.json")))
    W, R, width = g["W"], g["R"], g["row_width"]
    send = np.array(g["send_matrix"], np.int64)
    inp = rows_10i_plus_k(W, R, width)
    sp = oracle.a2a_plan(send)
    out, err = oracle.a2a_copy(inp, sp, fill=-1)
    assert err == 0
    for r in range(W):
        got = per_rank(out, sp, r)
        assert list(got.shape) == g["expected_shapes"][str(r)]
        assert got[:, 0].tolist() == g["expected_rows"][str(r)]
        assert (got == got[:, :1]).all()
    # the padded-even formulation gives the same rows
    for r, rows in enumerate(padded_even_all_to_all(inp, send)):
        assert rows[:, 0].tolist() == g["expected_rows"][str(r)]


def test_zero_row_chunk():
    send = np.array([[0, 4], [2, 2]], np.int64)
    inp = rows_10i_plus_k(2, 4, 8)
    sp = oracle.a2a_plan(send)
    out, err = oracle.a2a_copy(inp, sp, fill=-1)
    assert err == 0
    assert per_rank(out, sp, 0)[:, 0].tolist() == [10, 11]
    assert per_rank(out, sp, 1)[:, 0].tolist() == [0, 1, 2, 3, 12, 13]


def test_plan_identities_and_wrong_offset_mode():
    send = np.array([[1, 3], [2, 2]], np.int64)
    sp = oracle.a2a_plan(send)
    assert sp.out_splits.tolist() == send.T.tolist()
    excl = np.cumsum(send, axis=1) - send
    assert sp.src_offsets.tolist() == excl.T.tolist()
    assert sp.dst_offsets.tolist() == (np.cumsum(sp.out_splits, axis=1) - sp.out_splits).tolist()
    # rank 1's rows from rank 0 start after the rows rank 0 keeps for rank 0
    assert sp.src_offsets[1, 0] == 1


@pytest.mark.parametrize("seed", range(5))
def test_random_matches_padded_even(seed):
    rng = np.random.default_rng(seed)
    W = int(rng.integers(1, 9))
    R = int(rng.integers(1, 20))
    send = np.zeros((W, W), np.int64)
    for p in range(W):
        cuts = np.sort(rng.integers(0, R + 1, W - 1))
        send[p] = np.diff(np.concatenate([[0], cuts, [R]]))
    inp = rng.integers(0, 1 << 16, size=(W, R, 3)).astype(np.uint16)
    sp = oracle.a2a_plan(send)
    out, err = oracle.a2a_copy(inp, sp)
    assert err == 0
    ref = padded_even_all_to_all(inp, send)
    for r in range(W):
        assert (per_rank(out, sp, r) == ref[r]).all()


def test_all_to_all_workload_send_matrix():
    cfg = workloads.WORKLOADS[3]
    send = workloads.send_matrix(cfg)
    assert (send.sum(axis=1) == cfg.R).all()
    assert not (send == send.T).all()
    assert send[0, 0] == 0 and send[1, 4] == 0 and send[4, 7] == 0


def test_out_of_range_plan_is_flagged():
    send = np.array([[1, 3], [2, 2]], np.int64)
    sp = oracle.a2a_plan(send)
    sp.src_offsets[1, 0] = 3   # rank 1 would read rows 3..5 of rank 0 (R = 4)
    inp = rows_10i_plus_k(2, 4, 2)
    out, err = oracle.a2a_copy(inp, sp, fill=-1)
    assert err == oracle.DEVERR_SPLITS
