"""Pins for the oracle's index-branch training target (forward only).

Sources of truth used here, none of them the oracle's target code itself:
  * torch.nn.functional.scaled_dot_product_attention (CPU, float64) with an
    explicit selection mask and block-indicator values: its output row for a
    head is exactly that head's softmax mass per block;
  * closed forms: a zero query spreads each head uniformly over the visible
    tokens, so a block's mass is its share of them; one dominant key gives
    (e^x + n_b - 1) / (e^x + n - 1) to its block;
  * scipy.special.softmax and scipy.stats.entropy (textbook KL) for the loss;
    KL = 0 when the index logits are log(target) up to a constant; a two-block
    closed form; idx_scale = 0 gives log(n) - H(target);
  * invariants: rows are distributions on the selected blocks, padding is 0,
    KL >= 0, padding slots do not change the KL, a shift of all index scores
    does not change it.
"""

import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import msa_oracle as O
from tests.test_oracle_attention import rand_qkv, sdpa_reference, selection_mask


def rng(seed):
    return np.random.default_rng(seed)


def small_forward(seed, h_q=8, h_kv=2, n_q=6, n_kv=96, d=8, block=8, topk=4, pos0=90):
    r = rng(seed)
    b, d_idx = 1, 8
    q, k, v = rand_qkv(r, b, n_q, n_kv, h_q, h_kv, d)
    q_idx = r.integers(-3, 4, size=(b, n_q, h_kv, d_idx)).astype(np.float64)
    k_idx = r.integers(-3, 4, size=(b, n_kv, d_idx)).astype(np.float64)
    bscore, blk = O.msa_index_topk(q_idx, k_idx, pos0, block, topk)
    return q, k, v, bscore, blk, dict(b=b, n_q=n_q, n_kv=n_kv, h_q=h_q, h_kv=h_kv, d=d, block=block,
                                      topk=topk, pos0=pos0)


@pytest.mark.parametrize("h_q,h_kv,pos0,topk", [(8, 2, 90, 4), (4, 1, 5, 4), (16, 4, 60, 3)])
def test_target_rows_are_distributions_on_the_selection(h_q, h_kv, pos0, topk):
    q, k, _, _, blk, c = small_forward(21, h_q=h_q, h_kv=h_kv, pos0=pos0, topk=topk)
    t = O.msa_block_target(q, k, blk, c["pos0"], c["block"])
    assert t.shape == blk.shape
    assert np.all(t[blk < 0] == 0.0)
    assert np.all(t >= 0.0)
    assert np.max(np.abs(t.sum(axis=-1) - 1.0)) < 1e-12


@pytest.mark.parametrize("h_q,h_kv", [(8, 2), (4, 1), (6, 3)])
def test_target_matches_sdpa_with_block_indicator_values(h_q, h_kv):
    q, k, _, _, blk, c = small_forward(22, h_q=h_q, h_kv=h_kv)
    b, n_q, n_kv, block = c["b"], c["n_q"], c["n_kv"], c["block"]
    nblk = n_kv // block
    ind = np.zeros((b, n_kv, h_kv, nblk))
    for s in range(n_kv):
        ind[:, s, :, s // block] = 1.0
    allowed = selection_mask(blk, b, n_q, h_q, h_kv, n_kv, c["pos0"], block)
    per_head = sdpa_reference(q, k, ind, allowed, 1 / math.sqrt(c["d"]))   # [b][n_q][h_q][nblk]
    group = h_q // h_kv
    t = O.msa_block_target(q, k, blk, c["pos0"], block)
    for i in range(n_q):
        for g in range(h_kv):
            want = per_head[0, i, g * group:(g + 1) * group].mean(axis=0)
            for slot, j in enumerate(blk[0, i, g]):
                if j >= 0:
                    assert abs(t[0, i, g, slot] - want[j]) < 1e-12


def test_zero_query_gives_share_of_visible_tokens():
    q, k, _, _, blk, c = small_forward(23, n_kv=100, pos0=93)
    q[:] = 0.0
    t = O.msa_block_target(q, k, blk, c["pos0"], c["block"])
    B = c["block"]
    for i in range(c["n_q"]):
        p = c["pos0"] + i
        for g in range(c["h_kv"]):
            sel = [j for j in blk[0, i, g] if j >= 0]
            counts = {j: min((j + 1) * B, p + 1) - j * B for j in sel}
            total = sum(counts.values())
            for slot, j in enumerate(blk[0, i, g]):
                if j >= 0:
                    assert abs(t[0, i, g, slot] - counts[j] / total) < 1e-14


def test_dominant_key_closed_form():
    b, n_q, n_kv, h_q, h_kv, d, B = 1, 1, 64, 4, 1, 4, 8
    p = 61
    q = np.zeros((b, n_q, h_q, d))
    q[..., 0] = 1.5
    k = np.zeros((b, n_kv, h_kv, d))
    star = 19
    k[0, star, 0, 0] = 4.0
    blk = np.array([[[[0, 2, 5, 7]]]])                # block 2 holds the star key; 7 is the local block
    scale = 0.5
    t = O.msa_block_target(q, k, blk, p, B, scale)
    x = scale * 1.5 * 4.0
    n = 3 * B + (p - 7 * B + 1)                       # blocks 0, 2, 5 full; local block up to p
    den = math.exp(x) + n - 1
    want = [B / den, (math.exp(x) + B - 1) / den, B / den, (p - 7 * B + 1) / den]
    assert np.max(np.abs(t[0, 0, 0] - want)) < 1e-14


def test_kl_matches_scipy_entropy():
    r = rng(24)
    for _ in range(20):
        n = int(r.integers(1, 17))
        nblk = 40
        sel = np.sort(r.choice(nblk, size=n, replace=False))
        row = np.concatenate([sel, -np.ones(16 - n, dtype=np.int64)])
        t = np.concatenate([r.dirichlet(np.ones(n)), np.zeros(16 - n)])
        pooled = r.normal(size=nblk) * 5
        s = float(r.uniform(0.05, 2.0))
        ref = scipy.stats.entropy(t[:n], scipy.special.softmax(s * pooled[sel]))
        assert abs(O.index_kl_row(t, pooled, row, s) - ref) < 1e-12


def test_kl_zero_when_index_matches_target_and_shift_invariant():
    r = rng(25)
    sel = np.array([1, 4, 6, 9, -1, -1])
    t = np.array([0.1, 0.2, 0.3, 0.4, 0.0, 0.0])
    pooled = np.zeros(12)
    s = 0.7
    pooled[sel[:4]] = np.log(t[:4]) / s + 3.25
    assert abs(O.index_kl_row(t, pooled, sel, s)) < 1e-14
    pooled2 = r.normal(size=12)
    a = O.index_kl_row(t, pooled2, sel, s)
    b = O.index_kl_row(t, pooled2 + 11.5, sel, s)
    assert a > 0.0 and abs(a - b) < 1e-12


def test_kl_two_block_closed_form_and_zero_scale():
    t = np.array([0.3, 0.7])
    pooled = np.array([2.0, -1.0])
    s = 0.4
    qa = 1.0 / (1.0 + math.exp(-(s * 2.0 - s * -1.0)))
    want = 0.3 * math.log(0.3 / qa) + 0.7 * math.log(0.7 / (1 - qa))
    assert abs(O.index_kl_row(t, pooled, np.array([0, 1]), s) - want) < 1e-14
    t4 = np.array([0.1, 0.2, 0.3, 0.4])
    want0 = math.log(4) - scipy.stats.entropy(t4)
    assert abs(O.index_kl_row(t4, np.arange(4.0) * 9, np.arange(4), 0.0) - want0) < 1e-14


def test_kl_ignores_padding_and_zero_terms():
    pooled = np.array([0.5, 3.0, -2.0, 1.0])
    t = np.array([0.0, 0.6, 0.4])
    a = O.index_kl_row(t, pooled, np.array([0, 1, 3]), 1.0)
    ref = scipy.stats.entropy(t, scipy.special.softmax(pooled[[0, 1, 3]]))
    assert abs(a - ref) < 1e-12
    b = O.index_kl_row(np.concatenate([t, [0.0, 0.0]]), pooled, np.array([0, 1, 3, -1, -1]), 1.0)
    assert a == b


def test_kl_of_forward_is_nonnegative_and_whole_tensor_driver_matches_rows():
    q, k, _, bscore, blk, c = small_forward(26, pos0=80, n_q=12)
    t = O.msa_block_target(q, k, blk, c["pos0"], c["block"])
    kl = O.msa_index_kl(t, bscore, blk, 0.3)
    assert kl.shape == blk.shape[:3]
    assert np.all(kl >= -1e-15)
    for i in range(c["n_q"]):
        for g in range(c["h_kv"]):
            assert kl[0, i, g] == O.index_kl_row(t[0, i, g], bscore[0, i, g], blk[0, i, g], 0.3)
