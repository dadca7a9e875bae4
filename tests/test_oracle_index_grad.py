"""Pins for the oracle's index-branch backward (gradient of the KL loss with the
target detached and the selection fixed).

Sources of truth used here, none of them the oracle's gradient code:
  * central finite differences of sum(dkl * KL) computed with the oracle's
    forward functions (token scores, pooling, KL; each pinned elsewhere);
  * torch autograd (CPU, float64) through masked scores, a max over each
    block, a log-softmax over the selected blocks and the KL;
  * closed forms: the gradient vanishes when the target equals the index
    distribution; it is linear in dkl; with two equal maxima in a block only
    the lower position receives a key gradient.
"""

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O


def rng(seed):
    return np.random.default_rng(seed)


def continuous_case(seed, b=1, n_q=5, n_kv=64, h_kv=2, d_idx=6, block=8, topk=3, pos0=59):
    r = rng(seed)
    q_idx = r.normal(size=(b, n_q, h_kv, d_idx))
    k_idx = r.normal(size=(b, n_kv, d_idx))
    _, blk = O.msa_index_topk(q_idx, k_idx, pos0, block, topk)
    target = np.zeros(blk.shape)
    for idx in np.ndindex(*blk.shape[:3]):
        live = blk[idx] >= 0
        w = r.uniform(0.1, 1.0, size=int(live.sum()))
        target[idx][live] = w / w.sum()
    dkl = r.uniform(0.5, 2.0, size=blk.shape[:3])
    return q_idx, k_idx, blk, target, dkl, dict(pos0=pos0, block=block)


def kl_loss(q_idx, k_idx, blk, target, dkl, idx_scale, pos0, block):
    b, n_q, h_kv, _ = q_idx.shape
    pooled = np.full(blk.shape[:3] + (k_idx.shape[1] // block + 1,), -np.inf)
    for bi in range(b):
        for i in range(n_q):
            for g in range(h_kv):
                sc = O.token_scores(q_idx[bi, i, g], k_idx[bi], pos0 + i)
                pl = O.block_max_pool(sc, pos0 + i, block)
                pooled[bi, i, g, : len(pl)] = pl
    return float(np.sum(dkl * O.msa_index_kl(target, pooled, blk, idx_scale)))


@pytest.mark.parametrize("idx_scale", [0.7, 0.15])
def test_grad_matches_central_differences(idx_scale):
    q_idx, k_idx, blk, target, dkl, c = continuous_case(41)
    dq, dk = O.index_kl_grad(q_idx, k_idx, blk, target, idx_scale, dkl, c["pos0"], c["block"])
    r = rng(42)
    eps = 1e-6
    for name, x, gr in (("q", q_idx, dq), ("k", k_idx, dk)):
        for _ in range(16):
            idx = tuple(int(r.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            if name == "q":
                fp = kl_loss(xp, k_idx, blk, target, dkl, idx_scale, c["pos0"], c["block"])
                fm = kl_loss(xm, k_idx, blk, target, dkl, idx_scale, c["pos0"], c["block"])
            else:
                fp = kl_loss(q_idx, xp, blk, target, dkl, idx_scale, c["pos0"], c["block"])
                fm = kl_loss(q_idx, xm, blk, target, dkl, idx_scale, c["pos0"], c["block"])
            fd = (fp - fm) / (2 * eps)
            assert abs(fd - gr[idx]) < 1e-7, f"d{name}{idx}: fd {fd} vs {gr[idx]}"


def test_grad_matches_torch_autograd():
    q_idx, k_idx, blk, target, dkl, c = continuous_case(43, b=2, n_q=7, h_kv=3, pos0=57)
    idx_scale, pos0, B = 0.4, c["pos0"], c["block"]
    dq, dk = O.index_kl_grad(q_idx, k_idx, blk, target, idx_scale, dkl, pos0, B)
    qt = torch.from_numpy(q_idx).requires_grad_(True)
    kt = torch.from_numpy(k_idx).requires_grad_(True)
    b, n_q, h_kv, _ = q_idx.shape
    n_kv = k_idx.shape[1]
    loss = torch.zeros((), dtype=torch.float64)
    for bi in range(b):
        sc = torch.einsum("tgd,sd->tgs", qt[bi], kt[bi])
        for i in range(n_q):
            p = pos0 + i
            for g in range(h_kv):
                live = [s for s in range(blk.shape[-1]) if blk[bi, i, g, s] >= 0]
                pooled = torch.stack([sc[i, g, int(blk[bi, i, g, s]) * B: min((int(blk[bi, i, g, s]) + 1) * B, p + 1,
                                                                               n_kv)].max() for s in live])
                logq = torch.log_softmax(idx_scale * pooled, dim=0)
                t = torch.from_numpy(target[bi, i, g, live])
                loss = loss + float(dkl[bi, i, g]) * torch.sum(t * (torch.log(t) - logq))
    loss.backward()
    assert np.max(np.abs(qt.grad.numpy() - dq)) < 1e-12
    assert np.max(np.abs(kt.grad.numpy() - dk)) < 1e-12


def test_grad_vanishes_when_target_matches_and_is_linear_in_dkl():
    q_idx, k_idx, blk, target, dkl, c = continuous_case(44)
    idx_scale = 0.5
    match = np.zeros(blk.shape)
    for bi, i, g in np.ndindex(*blk.shape[:3]):
        sc = O.token_scores(q_idx[bi, i, g], k_idx[bi], c["pos0"] + i)
        pl = O.block_max_pool(sc, c["pos0"] + i, c["block"])
        live = blk[bi, i, g] >= 0
        a = idx_scale * pl[blk[bi, i, g][live]]
        e = np.exp(a - a.max())
        match[bi, i, g][live] = e / e.sum()
    dq, dk = O.index_kl_grad(q_idx, k_idx, blk, match, idx_scale, dkl, c["pos0"], c["block"])
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14
    d1 = O.index_kl_grad(q_idx, k_idx, blk, target, idx_scale, dkl, c["pos0"], c["block"])
    d2 = O.index_kl_grad(q_idx, k_idx, blk, target, idx_scale, 2 * dkl, c["pos0"], c["block"])
    assert np.max(np.abs(d2[0] - 2 * d1[0])) < 1e-12 and np.max(np.abs(d2[1] - 2 * d1[1])) < 1e-12


def test_tied_maxima_send_the_key_gradient_to_the_lower_position():
    B, n_kv, d = 4, 12, 2
    k_idx = np.zeros((1, n_kv, d))
    k_idx[0, 5] = [1.0, 0.0]                           # block 1 (tokens 4..7): positions 5 and 6 tie
    k_idx[0, 6] = [1.0, 0.0]
    k_idx[0, 9] = [0.5, 0.0]                           # block 2, the query's local block
    q_idx = np.zeros((1, 1, 1, d))
    q_idx[0, 0, 0] = [2.0, 0.0]
    blk = np.array([[[[1, 2]]]])
    target = np.array([[[[0.8, 0.2]]]])
    dq, dk = O.index_kl_grad(q_idx, k_idx, blk, target, 1.0, np.ones((1, 1, 1)), 10, B)
    a = np.array([2.0, 1.0])
    qd = np.exp(a) / np.exp(a).sum()
    assert abs(dk[0, 5, 0] - (qd[0] - 0.8) * 2.0) < 1e-14
    assert dk[0, 6, 0] == 0.0
    assert abs(dk[0, 9, 0] - (qd[1] - 0.2) * 2.0) < 1e-14
    assert abs(dq[0, 0, 0, 0] - ((qd[0] - 0.8) * 1.0 + (qd[1] - 0.2) * 0.5)) < 1e-14
