"""The autograd wrappers give exactly what the direct library calls give:
the same forward values and, for a weighted-sum loss, the same gradients bit
for bit (the wrappers only allocate and pass buffers).  Numerical parity of
the calls themselves is covered by the backward and target tests."""

import pytest
import torch

from block_sparse_long_score_amd import autograd as A
from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SHAPES = {
    # unaligned chunk, ragged n_q, partial last block, G = 4
    "chunk_ragged_g4": (11, Shape(1, 300, 1000, 700, 8, 2, 128, 128, topk=4)),
    # two sequences, G = 8, d = 64
    "batch2_g8_d64": (12, Shape(2, 257, 2600, 2343, 16, 2, 64, 64, topk=8)),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_sparse_attention_autograd_matches_direct_calls(name):
    cid, s = SHAPES[name]
    inp = make_inputs(s, cid, device="cuda")
    blk, _ = U.run_index(s, inp["q_idx"], inp["k_idx"])
    q, k, v = (inp[x].clone().requires_grad_(True) for x in ("q", "k", "v"))
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    w = torch.randn((s.batch, s.n_q, s.h_q, s.d), device="cuda", generator=g).to(torch.bfloat16)
    out = A.sparse_attention(s, q, k, v, blk)
    (out.float() * w.float()).sum().backward()

    o2 = torch.empty_like(out)
    lse = torch.empty((s.batch, s.n_q, s.h_q), dtype=torch.float32, device="cuda")
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    M.msa_sparse_prefill(s, inp["q"], inp["k"], inp["v"], blk, o2, lse, ws)
    dq, dk, dv = torch.empty_like(inp["q"]), torch.empty_like(inp["k"]), torch.empty_like(inp["v"])
    M.msa_sparse_prefill_backward(s, inp["q"], inp["k"], inp["v"], blk, o2, lse, w, dq, dk, dv, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o2)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)


@pytest.mark.parametrize("name", list(SHAPES))
def test_index_kl_autograd_matches_direct_calls(name):
    cid, s = SHAPES[name]
    inp = make_inputs(s, cid, device="cuda")
    blk, bscore = U.run_index(s, inp["q_idx"], inp["k_idx"])
    bscore = bscore.clone()
    q_idx = inp["q_idx"].clone().requires_grad_(True)
    k_idx = inp["k_idx"].clone().requires_grad_(True)
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    c = torch.rand((s.batch, s.n_q, s.h_kv), device="cuda", generator=g)
    idx_scale = 0.1
    kl = A.index_kl(s, q_idx, k_idx, inp["q"], inp["k"], inp["v"], blk, idx_scale=idx_scale)
    (kl * c).sum().backward()

    target = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.float32, device="cuda")
    kl2 = torch.empty_like(kl)
    out = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device="cuda")
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    M.msa_sparse_prefill_target(s, inp["q"], inp["k"], inp["v"], blk, bscore, target, kl2, out, None, ws,
                                idx_scale=idx_scale)
    dqi = torch.empty((s.batch, s.n_q, s.h_kv, s.d_idx), dtype=torch.float32, device="cuda")
    dki = torch.empty((s.batch, s.n_kv, s.d_idx), dtype=torch.float32, device="cuda")
    M.msa_index_backward(s, inp["q_idx"], inp["k_idx"], blk, bscore, target, c, dqi, dki, ws, idx_scale=idx_scale)
    torch.cuda.synchronize()
    assert torch.equal(kl.detach(), kl2)
    assert torch.equal(q_idx.grad, dqi.to(torch.bfloat16)) and torch.equal(k_idx.grad, dki.to(torch.bfloat16))
