"""Pins for the oracle's main-branch backward (gradients of the selected-block
softmax attention).

Sources of truth used here, none of them the oracle's gradient code:
  * torch autograd (CPU, float64) through scaled_dot_product_attention with the
    explicit selection mask;
  * central finite differences of sum(out * dout), with the oracle's forward
    (itself pinned against SDPA) as the function;
  * invariants: softmax rows sum to 1, so the values' gradients of a group sum
    to the sum of its heads' output gradients; dS rows sum to 0, so the keys'
    gradients of a group sum to 0; constant values give zero query and key
    gradients; blocks nobody selected get zero gradients.
"""

import math

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from tests.test_oracle_attention import rand_qkv, selection_mask


def rng(seed):
    return np.random.default_rng(seed)


def case(seed, h_q=8, h_kv=2, n_q=6, n_kv=96, d=8, block=8, topk=3, pos0=90, b=1):
    r = rng(seed)
    q, k, v = rand_qkv(r, b, n_q, n_kv, h_q, h_kv, d)
    q_idx = r.integers(-3, 4, size=(b, n_q, h_kv, 8)).astype(np.float64)
    k_idx = r.integers(-3, 4, size=(b, n_kv, 8)).astype(np.float64)
    _, blk = O.msa_index_topk(q_idx, k_idx, pos0, block, topk)
    dout = r.normal(size=q.shape)
    return q, k, v, blk, dout, dict(b=b, n_q=n_q, n_kv=n_kv, h_q=h_q, h_kv=h_kv, d=d, block=block, pos0=pos0)


def autograd_reference(q, k, v, dout, allowed, scale):
    group = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3).clone().requires_grad_(True)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).clone().requires_grad_(True)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).clone().requires_grad_(True)
    kr = kt.repeat_interleave(group, dim=1)
    vr = vt.repeat_interleave(group, dim=1)
    mask = torch.from_numpy(allowed).permute(0, 2, 1, 3)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kr, vr, attn_mask=mask, scale=scale)
    out.backward(torch.from_numpy(dout).permute(0, 2, 1, 3))
    return (qt.grad.permute(0, 2, 1, 3).numpy(), kt.grad.permute(0, 2, 1, 3).numpy(),
            vt.grad.permute(0, 2, 1, 3).numpy())


@pytest.mark.parametrize("h_q,h_kv,b", [(8, 2, 1), (4, 1, 2), (6, 6, 1), (16, 4, 1)])
def test_grads_match_torch_autograd(h_q, h_kv, b):
    q, k, v, blk, dout, c = case(31, h_q=h_q, h_kv=h_kv, b=b)
    scale = 1 / math.sqrt(c["d"])
    dq, dk, dv = O.msa_sparse_attention_grad(q, k, v, blk, dout, c["pos0"], c["block"], scale)
    allowed = selection_mask(blk, c["b"], c["n_q"], h_q, h_kv, c["n_kv"], c["pos0"], c["block"])
    rq, rk, rv = autograd_reference(q, k, v, dout, allowed, scale)
    assert np.max(np.abs(dq - rq)) < 1e-12
    assert np.max(np.abs(dk - rk)) < 1e-12
    assert np.max(np.abs(dv - rv)) < 1e-12


def test_grads_match_central_differences():
    q, k, v, blk, dout, c = case(32, n_q=4, n_kv=48, pos0=44, topk=2, d=4)
    dq, dk, dv = O.msa_sparse_attention_grad(q, k, v, blk, dout, c["pos0"], c["block"])

    def loss(qq, kk, vv):
        out, _ = O.msa_sparse_attention(qq, kk, vv, blk, c["pos0"], c["block"])
        return float(np.sum(out * dout))

    r = rng(33)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(r.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = [xp if a is x else a for a in args]
            am = [xm if a is x else a for a in args]
            fd = (loss(*ap) - loss(*am)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7, f"d{name}{idx}: fd {fd} vs {g[idx]}"


def test_value_and_key_gradient_sums():
    q, k, v, blk, dout, c = case(34, h_q=8, h_kv=2, n_q=10, pos0=86)
    dq, dk, dv = O.msa_sparse_attention_grad(q, k, v, blk, dout, c["pos0"], c["block"])
    group = c["h_q"] // c["h_kv"]
    for g in range(c["h_kv"]):
        want = dout[0, :, g * group:(g + 1) * group].sum(axis=(0, 1))
        assert np.max(np.abs(dv[0, :, g].sum(axis=0) - want)) < 1e-12
        assert np.max(np.abs(dk[0, :, g].sum(axis=0))) < 1e-12


def test_constant_values_give_zero_query_and_key_gradients():
    q, k, v, blk, dout, c = case(35)
    v[:] = 0.75
    dq, dk, dv = O.msa_sparse_attention_grad(q, k, v, blk, dout, c["pos0"], c["block"])
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    assert np.max(np.abs(dv)) > 0.1


def test_unselected_blocks_and_future_keys_get_no_gradient():
    q, k, v, blk, dout, c = case(36, n_q=5, pos0=60, n_kv=96, topk=3)
    dq, dk, dv = O.msa_sparse_attention_grad(q, k, v, blk, dout, c["pos0"], c["block"])
    seen = np.zeros((c["n_kv"], c["h_kv"]), dtype=bool)
    for i in range(c["n_q"]):
        for g in range(c["h_kv"]):
            seen[O.visible_positions(blk[0, i, g], c["pos0"] + i, c["block"], c["n_kv"]), g] = True
    assert np.all(dk[0][~seen] == 0.0) and np.all(dv[0][~seen] == 0.0)
    assert not np.any(seen[c["pos0"] + c["n_q"]:])
