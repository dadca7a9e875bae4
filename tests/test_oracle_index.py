"""Pins for the oracle's index branch (scores, block max-pool, top-k selection).

Every check here comes from something other than the oracle itself: integer
brute force, a separately written full sort, closed forms and invariants the
pages fix.  The pages print no worked example with numbers; the constants they
do print (k = 16 blocks of 128 tokens, 2,048 tokens per query, lefilia.fr
article) are in tests/golden/pages_constants.json.
"""

import json
import os

import numpy as np
import pytest

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def int_matrix(r, shape, lo=-3, hi=3):
    return r.integers(lo, hi + 1, size=shape).astype(np.float64)


# ---------------------------------------------------------------- scores ----

def test_token_scores_match_integer_brute_force():
    r = rng(1)
    d_idx, n_kv = 16, 50
    k_idx = int_matrix(r, (n_kv, d_idx))
    for p in (0, 1, 17, 49):
        q = int_matrix(r, (d_idx,))
        got = O.token_scores(q, k_idx, p)
        assert got.shape == (p + 1,)
        for s in range(p + 1):
            exact = sum(int(q[c]) * int(k_idx[s, c]) for c in range(d_idx))
            assert got[s] == exact


def test_block_max_pool_matches_loop_brute_force():
    r = rng(2)
    block = 8
    for p in (0, 7, 8, 9, 63, 70):
        sc = r.integers(-50, 50, size=p + 1).astype(np.float64)
        got = O.block_max_pool(sc, p, block)
        best = {}
        for s in range(p + 1):
            j = s // block
            best[j] = sc[s] if j not in best else max(best[j], sc[s])
        assert list(got) == [best[j] for j in range(p // block + 1)]


def test_index_scores_never_look_past_p():
    r = rng(3)
    d_idx, n_kv, block, topk = 8, 96, 8, 4
    k_idx = int_matrix(r, (n_kv, d_idx))
    q = int_matrix(r, (d_idx,))
    for p in (5, 30, 47, 95):
        pooled, sel = O.index_topk_row(q, k_idx, p, block, topk)
        k2 = k_idx.copy()
        k2[p + 1:] = 99.0                       # future tokens made huge
        pooled2, sel2 = O.index_topk_row(q, k2, p, block, topk)
        assert np.array_equal(pooled, pooled2)
        assert np.array_equal(sel, sel2)


# ------------------------------------------------------------- selection ----

def lexsort_selection(pooled, jl, topk):
    """Separately written reference: full sort of earlier blocks by
    (score descending, index ascending), keep topk-1, add jl, sort."""
    if jl + 1 <= topk:
        return list(range(jl + 1)) + [-1] * (topk - jl - 1)
    idx = np.arange(jl)
    order = np.lexsort((idx, -pooled[:jl]))      # last key is primary
    chosen = sorted(list(order[: topk - 1]) + [jl])
    return chosen


@pytest.mark.parametrize("topk", [1, 2, 16, 32])
def test_selection_matches_full_sort_with_heavy_ties(topk):
    r = rng(4 + topk)
    for _ in range(300):
        jl = int(r.integers(0, 200))
        # few distinct values -> many ties, as integer index scores give
        pooled = r.integers(-4, 5, size=jl + 1).astype(np.float64)
        got = O.select_blocks(pooled, jl, topk)
        assert list(got) == lexsort_selection(pooled, jl, topk)


def test_selection_all_ties_takes_lowest_indices():
    # all-zero index query -> every score 0 -> the k-1 lowest earlier blocks win
    topk = 16
    for jl in (16, 17, 100, 1023):
        pooled = np.zeros(jl + 1)
        got = O.select_blocks(pooled, jl, topk)
        assert list(got) == list(range(topk - 1)) + [jl]


def test_selection_increasing_scores_is_a_sliding_window():
    topk = 16
    for jl in (20, 64, 500):
        pooled = np.arange(jl + 1, dtype=np.float64)
        got = O.select_blocks(pooled, jl, topk)
        assert list(got) == list(range(jl - topk + 1, jl + 1))


def test_selection_decreasing_scores_keeps_oldest_blocks():
    topk = 16
    jl = 300
    pooled = -np.arange(jl + 1, dtype=np.float64)
    got = O.select_blocks(pooled, jl, topk)
    assert list(got) == list(range(topk - 1)) + [jl]


def test_selection_is_exponential_free():
    """Selection on raw scores equals selection on exp(score) and on the softmax
    of the scores (monotone maps keep the order)."""
    r = rng(7)
    for _ in range(100):
        jl = int(r.integers(16, 300))
        pooled = r.integers(-30, 30, size=jl + 1).astype(np.float64)
        a = O.select_blocks(pooled, jl, 16)
        e = np.exp(pooled - pooled.max())
        b = O.select_blocks(e, jl, 16)
        c = O.select_blocks(e / e.sum(), jl, 16)
        assert np.array_equal(a, b) and np.array_equal(a, c)


def test_selection_structure_invariants():
    r = rng(8)
    for topk in (1, 4, 16):
        for jl in range(0, 60):
            pooled = r.normal(size=jl + 1)
            sel = O.select_blocks(pooled, jl, topk)
            valid = sel[sel >= 0]
            assert jl in valid                                    # local block forced
            assert len(valid) == min(topk, jl + 1)
            assert np.all(valid <= jl)
            assert np.all(np.diff(valid) > 0)                     # ascending, unique
            assert np.all(sel[len(valid):] == -1)                 # padding at the end


def test_pages_constants_budget():
    cfg = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    block, topk, budget = cfg["block"], cfg["topk"], cfg["kv_budget_tokens"]
    assert block * topk == budget
    # a late query at the last token of its block attends exactly the budget
    r = rng(9)
    n_kv, d_idx = 40 * block, 4
    k_idx = int_matrix(r, (n_kv, d_idx))
    q = int_matrix(r, (d_idx,))
    p = n_kv - 1
    _, sel = O.index_topk_row(q, k_idx, p, block, topk)
    assert len(O.visible_positions(sel, p, block, n_kv)) == budget
    # and never more, anywhere
    for p in range(0, n_kv, 97):
        _, sel = O.index_topk_row(q, k_idx, p, block, topk)
        assert len(O.visible_positions(sel, p, block, n_kv)) <= budget


def test_whole_tensor_driver_matches_rows():
    r = rng(10)
    b, n_q, n_kv, h_kv, d_idx, block, topk, pos0 = 2, 9, 80, 3, 8, 8, 4, 71
    q_idx = int_matrix(r, (b, n_q, h_kv, d_idx))
    k_idx = int_matrix(r, (b, n_kv, d_idx))
    bscore, blk = O.msa_index_topk(q_idx, k_idx, pos0, block, topk)
    for bi in range(b):
        for i in range(n_q):
            p = pos0 + i
            for g in range(h_kv):
                pooled, sel = O.index_topk_row(q_idx[bi, i, g], k_idx[bi], p, block, topk)
                assert np.array_equal(bscore[bi, i, g, : len(pooled)], pooled)
                assert np.all(np.isneginf(bscore[bi, i, g, len(pooled):]))
                assert np.array_equal(blk[bi, i, g], sel)
