"""Pins for the oracle's main branch and dense comparator.

Sources of truth used here, none of them the oracle itself:
  * torch.nn.functional.scaled_dot_product_attention on CPU float64 with an
    explicit boolean mask (a textbook routine, test-only);
  * closed forms: Q = 0 gives the mean of the visible values (and
    lse = log(count)); constant V gives that constant back;
  * a block probe: Q = 0 and one-hot V per block show exactly which blocks and
    how many tokens of each contributed;
  * invariants: no future token matters; decode at position p equals prefill row
    p; a prefill chunk equals the matching rows of a full prefill; with
    k * B >= n_kv the sparse branch equals the dense comparator.
"""

import math

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O


def rng(seed):
    return np.random.default_rng(seed)


def rand_qkv(r, b, n_q, n_kv, h_q, h_kv, d):
    q = r.normal(size=(b, n_q, h_q, d))
    k = r.normal(size=(b, n_kv, h_kv, d))
    v = r.normal(size=(b, n_kv, h_kv, d))
    return q, k, v


def sdpa_reference(q, k, v, allowed, scale):
    """torch SDPA in float64 on CPU.  allowed [b][n_q][h_q][n_kv] bool."""
    b, n_q, h_q, d = q.shape
    h_kv = k.shape[2]
    group = h_q // h_kv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)                       # b h n d
    kt = torch.from_numpy(np.repeat(k, group, axis=2)).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(np.repeat(v, group, axis=2)).permute(0, 2, 1, 3).contiguous()
    mask = torch.from_numpy(allowed).permute(0, 2, 1, 3)               # b h n_q n_kv
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


def causal_mask(b, n_q, h_q, n_kv, pos0):
    m = np.zeros((b, n_q, h_q, n_kv), dtype=bool)
    for i in range(n_q):
        m[:, i, :, : pos0 + i + 1] = True
    return m


def selection_mask(blk, b, n_q, h_q, h_kv, n_kv, pos0, block):
    group = h_q // h_kv
    m = np.zeros((b, n_q, h_q, n_kv), dtype=bool)
    for bi in range(b):
        for i in range(n_q):
            p = pos0 + i
            for h in range(h_q):
                for j in blk[bi, i, h // group]:
                    if j >= 0:
                        lo = j * block
                        hi = min((j + 1) * block, p + 1, n_kv)
                        m[bi, i, h, lo:hi] = True
    return m


@pytest.mark.parametrize("h_q,h_kv", [(4, 1), (4, 4), (8, 2)])
def test_dense_matches_torch_sdpa(h_q, h_kv):
    r = rng(11)
    b, n_q, n_kv, d, pos0 = 2, 7, 40, 16, 33
    q, k, v = rand_qkv(r, b, n_q, n_kv, h_q, h_kv, d)
    scale = 1 / math.sqrt(d)
    out, lse = O.dense_gqa(q, k, v, pos0, scale)
    ref = sdpa_reference(q, k, v, causal_mask(b, n_q, h_q, n_kv, pos0), scale)
    assert np.max(np.abs(out - ref)) < 1e-12


@pytest.mark.parametrize("h_q,h_kv", [(4, 1), (8, 8), (16, 2)])
def test_sparse_matches_torch_sdpa_on_selection_mask(h_q, h_kv):
    r = rng(12)
    b, n_q, n_kv, d, d_idx, block, topk, pos0 = 1, 6, 96, 8, 8, 8, 3, 90
    q, k, v = rand_qkv(r, b, n_q, n_kv, h_q, h_kv, d)
    q_idx = r.integers(-3, 4, size=(b, n_q, h_kv, d_idx)).astype(np.float64)
    k_idx = r.integers(-3, 4, size=(b, n_kv, d_idx)).astype(np.float64)
    out, lse, blk, _ = O.msa_forward(q_idx, k_idx, q, k, v, pos0, block, topk)
    scale = 1 / math.sqrt(d)
    allowed = selection_mask(blk, b, n_q, h_q, h_kv, n_kv, pos0, block)
    ref = sdpa_reference(q, k, v, allowed, scale)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_sparse_equals_dense_when_budget_covers_context():
    """With k*B >= n_kv every causal token is selected, so the sparse attention equals dense causal GQA."""
    r = rng(13)
    b, n_q, n_kv, h_q, h_kv, d, d_idx, block = 1, 64, 64, 4, 2, 16, 8, 8
    q, k, v = rand_qkv(r, b, n_q, n_kv, h_q, h_kv, d)
    q_idx = r.integers(-3, 4, size=(b, n_q, h_kv, d_idx)).astype(np.float64)
    k_idx = r.integers(-3, 4, size=(b, n_kv, d_idx)).astype(np.float64)
    topk = n_kv // block
    out, lse, _, _ = O.msa_forward(q_idx, k_idx, q, k, v, 0, block, topk)
    dout, dlse = O.dense_gqa(q, k, v, 0)
    assert np.max(np.abs(out - dout)) < 1e-12
    assert np.max(np.abs(lse - dlse)) < 1e-12


def test_zero_query_gives_mean_of_visible_values():
    r = rng(14)
    b, n_q, n_kv, h_q, h_kv, d, block, topk, pos0 = 1, 5, 200, 4, 2, 8, 16, 4, 190
    q = np.zeros((b, n_q, h_q, d))
    k = r.normal(size=(b, n_kv, h_kv, d))
    v = r.normal(size=(b, n_kv, h_kv, d))
    blk = np.full((b, n_q, h_kv, topk), -1)
    for i in range(n_q):
        jl = (pos0 + i) // block
        for g in range(h_kv):
            blk[0, i, g] = sorted(r.choice(jl, size=topk - 1, replace=False).tolist() + [jl])
    out, lse = O.msa_sparse_attention(q, k, v, blk, pos0, block)
    for i in range(n_q):
        p = pos0 + i
        for h in range(h_q):
            g = h // (h_q // h_kv)
            toks = [s for j in blk[0, i, g] for s in range(j * block, min((j + 1) * block, p + 1))]
            assert np.allclose(out[0, i, h], v[0, toks, g].mean(axis=0), atol=1e-13)
            assert abs(lse[0, i, h] - math.log(len(toks))) < 1e-13


def test_constant_values_come_back():
    r = rng(15)
    b, n_q, n_kv, h_q, h_kv, d = 1, 4, 50, 4, 1, 8
    q = r.normal(size=(b, n_q, h_q, d)) * 3
    k = r.normal(size=(b, n_kv, h_kv, d))
    v = np.full((b, n_kv, h_kv, d), 0.375)
    out, _ = O.dense_gqa(q, k, v, 40)
    assert np.allclose(out, 0.375, atol=1e-14)


def test_block_probe_shows_exactly_the_selected_blocks():
    """Q = 0 and V[s] = one-hot(block(s)): output component j is the share of
    visible tokens that came from block j."""
    r = rng(16)
    block, topk, d_idx = 8, 4, 8
    n_kv = 12 * block
    nblk = n_kv // block
    b, h_q, h_kv = 1, 2, 2
    pos0, n_q = 60, 30
    q = np.zeros((b, n_q, h_q, nblk))
    k = r.normal(size=(b, n_kv, h_kv, nblk))
    v = np.zeros((b, n_kv, h_kv, nblk))
    for s in range(n_kv):
        v[0, s, :, s // block] = 1.0
    q_idx = r.integers(-3, 4, size=(b, n_q, h_kv, d_idx)).astype(np.float64)
    k_idx = r.integers(-3, 4, size=(b, n_kv, d_idx)).astype(np.float64)
    out, _, blk, _ = O.msa_forward(q_idx, k_idx, q, k, v, pos0, block, topk)
    for i in range(n_q):
        p = pos0 + i
        for g in range(h_kv):
            sel = [j for j in blk[0, i, g] if j >= 0]
            counts = np.zeros(nblk)
            for j in sel:
                counts[j] = min((j + 1) * block, p + 1) - j * block
            assert np.allclose(out[0, i, g], counts / counts.sum(), atol=1e-14)


def test_no_future_token_changes_anything():
    r = rng(17)
    b, n_q, n_kv, h_q, h_kv, d, d_idx, block, topk = 1, 40, 160, 4, 2, 8, 8, 8, 4
    q, k, v = rand_qkv(r, b, n_q, n_kv, h_q, h_kv, d)
    q_idx = r.integers(-3, 4, size=(b, n_q, h_kv, d_idx)).astype(np.float64)
    k_idx = r.integers(-3, 4, size=(b, n_kv, d_idx)).astype(np.float64)
    pos0 = 100
    out, lse, blk, _ = O.msa_forward(q_idx, k_idx, q, k, v, pos0, block, topk)
    for i in (0, 13, 39):
        p = pos0 + i
        k2, v2, ki2, qi2 = k.copy(), v.copy(), k_idx.copy(), q_idx.copy()
        k2[:, p + 1:] = r.normal(size=k2[:, p + 1:].shape) * 10
        v2[:, p + 1:] = r.normal(size=v2[:, p + 1:].shape) * 10
        ki2[:, p + 1:] = 3.0
        qi2[:, i + 1:] = -3.0
        o2, l2, b2, _ = O.msa_forward(qi2, ki2, q, k2, v2, pos0, block, topk)
        assert np.array_equal(b2[:, i], blk[:, i])
        assert np.array_equal(o2[:, i], out[:, i])
        assert np.array_equal(l2[:, i], lse[:, i])


def test_decode_equals_prefill_row_and_chunk_equals_full():
    r = rng(18)
    b, n_kv, h_q, h_kv, d, d_idx, block, topk = 2, 72, 8, 2, 8, 8, 8, 3
    q, k, v = rand_qkv(r, b, n_kv, n_kv, h_q, h_kv, d)
    q_idx = r.integers(-3, 4, size=(b, n_kv, h_kv, d_idx)).astype(np.float64)
    k_idx = r.integers(-3, 4, size=(b, n_kv, d_idx)).astype(np.float64)
    full = O.msa_forward(q_idx, k_idx, q, k, v, 0, block, topk)
    # decode: the last token as a single query against the whole cache
    dec = O.msa_forward(q_idx[:, -1:], k_idx, q[:, -1:], k, v, n_kv - 1, block, topk)
    for a, bb in zip(full[:3], dec[:3]):
        assert np.array_equal(a[:, -1:], bb)
    # chunk: queries 40..59 over a cache of 60 tokens
    c0, c1 = 40, 60
    ch = O.msa_forward(q_idx[:, c0:c1], k_idx[:, :c1], q[:, c0:c1], k[:, :c1], v[:, :c1], c0, block, topk)
    for a, bb in zip(full[:3], ch[:3]):
        assert np.array_equal(a[:, c0:c1], bb)
