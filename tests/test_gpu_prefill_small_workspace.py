"""msa_sparse_prefill with less than its full workspace runs in query chunks.

Every query's output depends only on its own selected blocks (each partial
result is one query's attention over one block; the merge combines a row's
partials in slot order), so the chunked call must return the one-pass call's
out and lse bit for bit.  Workspaces: one query of one sequence (the
smallest accepted) and 37 queries.
"""

from __future__ import annotations

import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    # chunk at an unaligned offset, ragged n_q, partial last block, G = 4
    "chunk_ragged_g4": (51, Shape(1, 300, 1000, 700, 8, 2, 128, 128, topk=4)),
    # two sequences, MQA group of 16, d = 64
    "batch2_g16_d64": (52, Shape(2, 257, 600, 343, 16, 1, 64, 64, topk=3)),
    # 256-token blocks (the selection is expanded per chunk), G = 8
    "block256_g8": (53, Shape(1, 600, 9000, 8400, 64, 8, 128, 128, block=256, topk=16)),
}


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_small_workspace_gives_the_same_outputs(name):
    cfg, s = CASES[name]
    print(f"[small-ws] {name} {s}", flush=True)
    inp = make_inputs(s, cfg, device="cuda")
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], blk, M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s))

    def run(ws_bytes):
        out = torch.full((s.batch, s.n_q, s.h_q, s.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((s.batch, s.n_q, s.h_q), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        M.msa_sparse_prefill(s, inp["q"], inp["k"], inp["v"], blk, out, lse, ws)
        torch.cuda.synchronize()
        return out, lse

    full = M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, s)
    o0, l0 = run(full)
    assert not bool(torch.isnan(o0).any())
    for n in (1, 37):
        small = M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, s.replace(batch=1, n_q=n))
        assert small < full
        o1, l1 = run(small)
        assert torch.equal(bits(o0), bits(o1)) and torch.equal(bits(l0), bits(l1)), f"{name}: chunks of {n} differ"


@pytest.mark.parametrize("name", ["chunk_ragged_g4", "batch2_g16_d64"])
def test_target_small_workspace_gives_the_same_outputs(name):
    """msa_sparse_prefill_target with a smaller workspace: the same query chunks,
    each followed by its rows' target and KL."""
    cfg, s = CASES[name]
    print(f"[small-ws target] {name} {s}", flush=True)
    inp = make_inputs(s, cfg, device="cuda")
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], blk, M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s))
    bscore = torch.empty((s.batch, s.n_q, s.h_kv, s.nblk), dtype=torch.float32, device="cuda")
    M.msa_index_scores(s, inp["q_idx"], inp["k_idx"], bscore)

    def run(ws_bytes):
        out = torch.full((s.batch, s.n_q, s.h_q, s.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((s.batch, s.n_q, s.h_q), float("nan"), dtype=torch.float32, device="cuda")
        target = torch.full((s.batch, s.n_q, s.h_kv, s.topk), float("nan"), dtype=torch.float32, device="cuda")
        kl = torch.full((s.batch, s.n_q, s.h_kv), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        M.msa_sparse_prefill_target(s, inp["q"], inp["k"], inp["v"], blk, bscore, target, kl, out, lse, ws,
                                    idx_scale=0.1)
        torch.cuda.synchronize()
        return out, lse, target, kl

    full = M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, s)
    ref = run(full)
    assert not bool(torch.isnan(ref[0]).any()) and not bool(torch.isnan(ref[3]).any())
    for n in (1, 37):
        got = run(M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, s.replace(batch=1, n_q=n)))
        for a, b, what in zip(ref, got, ("out", "lse", "target", "kl")):
            assert torch.equal(bits(a), bits(b)), f"{name}: {what} differs with chunks of {n}"
