"""Pins for the oracle's block pooling, block scores and top-k selection.

Each test checks the oracle against something other than itself: IEEE worked
examples (tests/golden), exact integer arithmetic, error bounds against fp64,
and the defining property of the kept set checked by brute force.
"""
import itertools
import json
import os

import numpy as np

import oracle
import pytest

from sparse_rank_attention_amd.workloads import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ pooling
def test_pool_tree_order_worked_example(oracle_lib):
    g = _golden("pool_tree_order.json")
    x = np.zeros((64, 1), dtype=np.float32)
    for i, val in g["nonzero"].items():
        x[int(i), 0] = val
    out = oracle_lib.pool(to_bf16_bits(x)[None], 64)
    assert out[0, 0, 0] == np.float32(g["expected_mean"])
    assert g["expected_mean"] != g["sequential_mean"] != g["exact_mean"]


def test_pool_exact_on_small_integers(oracle_lib):
    rng = np.random.default_rng(1)
    n_valid, d = 64 * 5 + 16, 8  # tail block has 16 valid tokens (1/16 exact)
    x = rng.integers(-50, 51, size=(2, 64 * 6, d)).astype(np.float32)
    x[:, n_valid:] = 1e30  # padding must be ignored
    out = oracle_lib.pool(to_bf16_bits(x), n_valid)
    for c in range(6):
        lo, hi = 64 * c, min(64 * c + 64, n_valid)
        exact = x[:, lo:hi].astype(np.float64).sum(axis=1) / (hi - lo)
        np.testing.assert_array_equal(out[:, c].astype(np.float64), exact)


def test_pool_error_bound_random(oracle_lib):
    rng = np.random.default_rng(2)
    n_valid = 64 * 3 + 56  # tail block of 56: 1/56 is inexact
    x = to_bf16_bits(rng.standard_normal((3, 256, 16)).astype(np.float32) * 10)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = oracle_lib.pool(x, n_valid).astype(np.float64)
    u = 2.0 ** -24
    for c in range(4):
        lo, hi = 64 * c, min(64 * c + 64, n_valid)
        blk = xf[:, lo:hi]
        exact = blk.sum(axis=1) / (hi - lo)
        bound = (6 * u * np.abs(blk).sum(axis=1) / (hi - lo)) * (1 + 2 * u) + 2 * u * np.abs(exact)
        assert np.all(np.abs(out[:, c] - exact) <= bound + 1e-300)


# ------------------------------------------------------------------- scores
def test_scores_fma_chain_worked_examples(oracle_lib):
    for case in _golden("score_fma_chain.json")["cases"]:
        qp = np.array(case["qp"], dtype=np.float32)[None, None]
        kp = np.array(case["kp"], dtype=np.float32)[None, None]
        s = oracle_lib.scores(qp, kp)
        assert s[0, 0, 0] == np.float32(case["expected"]), case["why"]


def test_scores_exact_on_integers_and_bound_on_random(oracle_lib):
    rng = np.random.default_rng(3)
    qi = rng.integers(-20, 21, size=(2, 9, 32)).astype(np.float32)
    ki = rng.integers(-20, 21, size=(2, 9, 32)).astype(np.float32)
    s = oracle_lib.scores(qi, ki)
    np.testing.assert_array_equal(s, np.einsum("bid,bjd->bij", qi.astype(np.int64), ki.astype(np.int64)))
    qr = rng.standard_normal((2, 7, 128)).astype(np.float32)
    kr = rng.standard_normal((2, 7, 128)).astype(np.float32)
    s = oracle_lib.scores(qr, kr).astype(np.float64)
    exact = np.einsum("bid,bjd->bij", qr.astype(np.float64), kr.astype(np.float64))
    bound = 128 * 2.0 ** -24 * np.einsum("bid,bjd->bij", np.abs(qr), np.abs(kr)).astype(np.float64)
    assert np.all(np.abs(s - exact) <= bound)


def test_scores_scale_by_power_of_two_exact(oracle_lib):
    rng = np.random.default_rng(4)
    qp = rng.standard_normal((1, 11, 64)).astype(np.float32)
    kp = rng.standard_normal((1, 11, 64)).astype(np.float32)
    s = oracle_lib.scores(qp, kp)
    np.testing.assert_array_equal(oracle_lib.scores(qp * 2, kp), s * 2)
    np.testing.assert_array_equal(oracle_lib.scores(qp, kp * 0.5), s * 0.5)


# ---------------------------------------------------------------- selection
def _is_kept_set(row, kept):
    """Definition: every kept j beats every dropped j' by (score desc, index asc)."""
    kept = set(int(j) for j in kept)
    for a in kept:
        for b in range(len(row)):
            if b in kept:
                continue
            if not (row[a] > row[b] or (row[a] == row[b] and a < b)):
                return False
    return True


def test_select_worked_ties(oracle_lib):
    for case in _golden("select_ties.json")["cases"]:
        row = np.array(case["row"], dtype=np.float32)[None, None]
        m = oracle_lib.select(row, case["kb"])
        assert m[0, 0].tolist() == case["expected"], case["why"]


@pytest.mark.parametrize("seed", range(6))
def test_select_brute_force_tiny(oracle_lib, seed):
    rng = np.random.default_rng(10 + seed)
    nb, kb = 7, 3
    # few distinct values so ties are common
    s = rng.integers(-2, 3, size=(2, nb, nb)).astype(np.float32)
    m = oracle_lib.select(s, kb)
    for bh in range(2):
        for i in range(nb):
            row = s[bh, i]
            sets = [c for c in itertools.combinations(range(nb), kb) if _is_kept_set(row, c)]
            assert len(sets) == 1  # the definition fixes exactly one set
            assert m[bh, i].tolist() == list(sets[0])


def test_select_property_large_random(oracle_lib):
    rng = np.random.default_rng(5)
    nb, kb = 200, 17
    s = rng.standard_normal((2, nb, nb)).astype(np.float32)
    s[:, :, 50:60] = s[:, :, 40:50]  # duplicated columns -> ties
    m = oracle_lib.select(s, kb)
    for bh in range(2):
        for i in range(0, nb, 7):
            assert np.all(np.diff(m[bh, i]) > 0)
            assert _is_kept_set(s[bh, i], m[bh, i])


def test_all_zero_queries_keep_first_blocks(oracle_lib):
    rng = np.random.default_rng(6)
    q = np.zeros((1, 64 * 8, 64), dtype=np.uint16)
    k = to_bf16_bits(rng.standard_normal((1, 64 * 8, 64)).astype(np.float32))
    m = oracle_lib.block_map(q, k, 64 * 8, 3)
    assert np.all(m[0] == np.arange(3))


def test_block_map_invariant_to_power_of_two_scaling(oracle_lib):
    from sparse_rank_attention_amd.workloads import WORKLOADS, make_qkv
    w = WORKLOADS["tiny"]
    q, k, _ = make_qkv(w)
    q, k = q[0], k[0]
    m = oracle_lib.block_map(q, k, w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
    qf = (q.astype(np.uint32) << 16).view(np.float32)
    m2 = oracle_lib.block_map(to_bf16_bits(qf * 4), k, w.n_tokens, oracle.keep_blocks(w.topk, w.nb))
    np.testing.assert_array_equal(m, m2)
