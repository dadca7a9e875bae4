"""The algorithmic counts behind every roofline fraction bench.py reports,
checked against closed forms and, on small shapes, against the oracle's own
selections counted one (query, group) at a time (no GPU needed).

Closed forms: index scoring costs h_kv * d_idx * 2 flops per (query, causal
token), so a full causal prefill of N tokens costs h_kv * d_idx * N (N + 1)
flops; dense attention costs h_q * d * 4 per (query head, causal key), i.e.
2 h_q d N (N + 1); the sparse main branch attends min(p + 1, (k - 1) B +
(p mod B) + 1) keys when every earlier block is full.
"""

import importlib.util
import os

import numpy as np

from block_sparse_long_score_amd.inputs import WORKLOADS, Shape
from oracle import msa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


B = load_bench()


def test_index_and_dense_flops_closed_forms_at_128k():
    _, s = WORKLOADS["prefill_128k"]
    n = s.n_q
    assert B.index_flops(s) == float(s.h_kv * s.d_idx * n * (n + 1))
    assert B.dense_flops(s) == float(2 * s.h_q * s.d * n * (n + 1))
    assert abs(B.index_flops(s) - 1.7592e13) / 1.7592e13 < 1e-4
    assert abs(B.dense_flops(s) - 2.8148e14) / 2.8148e14 < 1e-4


def test_sparse_flops_at_128k():
    _, s = WORKLOADS["prefill_128k"]
    # rows of the first k blocks see every causal key; later rows (k-1) full blocks plus their own prefix
    p = np.arange(s.n_q, dtype=np.int64)
    vis = np.where(p // s.block + 1 <= s.topk, p + 1, (s.topk - 1) * s.block + p % s.block + 1)
    assert B.sparse_flops(s) == float(s.h_q * s.d * 4 * vis.sum())
    assert abs(B.sparse_flops(s) - 8.4589e12) / 8.4589e12 < 1e-4


def test_visible_counts_match_the_oracle_selection_row_by_row():
    """bench's |V_t| is the number of keys the oracle's main branch attends
    for every (query, group), on shapes where rows have fewer and more causal
    blocks than k, an unaligned chunk and a partial last block."""
    rng = np.random.default_rng(11)
    for s in (Shape(1, 300, 1000, 700, 4, 2, 64, 64, topk=4), Shape(1, 200, 2000, 1800, 4, 1, 64, 64, topk=16),
              Shape(1, 130, 130, 0, 4, 2, 64, 64, topk=2)):
        q_idx = rng.integers(-3, 4, size=(1, s.n_q, s.h_kv, s.d_idx)).astype(np.float64)
        k_idx = rng.integers(-3, 4, size=(1, s.n_kv, s.d_idx)).astype(np.float64)
        _, blk = O.msa_index_topk(q_idx, k_idx, s.pos0, s.block, s.topk)
        want = B.visible_counts(s)
        for t in range(s.n_q):
            for g in range(s.h_kv):
                sel = blk[0, t, g]
                got = len(O.visible_positions(sel[sel >= 0], s.pos0 + t, s.block, s.n_kv))
                assert got == want[t], (s, t, g)


def test_decode_bytes_at_1m_batch8():
    _, s = WORKLOADS["decode_1m_b8"]
    kidx = s.batch * s.n_kv * s.d_idx * 2                       # 2 GiB of index keys
    kv = s.batch * s.topk * s.block * s.h_kv * s.d * 2 * 2       # 64 MiB of selected K and V
    got = B.decode_bytes(s)
    assert kidx == 2 << 30 and kv == 64 << 20
    assert kidx + kv < got < kidx + kv + (8 << 20)              # plus queries, pooled scores, indices, outputs


def test_topk_bytes_count_the_causal_candidates():
    s = Shape(1, 4096, 4096, 0, 4, 1, 64, 64)
    p = np.arange(s.n_q)
    assert B.topk_bytes(s) == float(s.h_kv * ((p // s.block).sum() * 4 + s.n_q * s.topk * 4))
