"""Decode-shaped index top-k (at most 16 query rows per sequence, rows of up
to 8,191 candidates selected by one workgroup of 8 or 16 waves per row):
selections bit-exact against the oracle and against msa_block_topk on the same
pooled scores, for rows of 1,000 to 8,191 candidates, rows of one call on both
sides of a block boundary, k = 1 to 64, sequences of different lengths, and
partial last blocks."""

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = {
    # 3 sequences of 2,344 blocks, partial last block
    "rows_2343_d64": (51, Shape(3, 1, 300000, 299999, 8, 2, 64, 64, topk=16)),
    # 16 rows per sequence from 4 tokens x 4 groups straddling a block boundary
    "four_tokens_boundary": (52, Shape(2, 4, 5000, 4990, 16, 4, 128, 128, topk=16)),
    # k = 64 over 1,562 candidates, 16 rows
    "topk64_rows_1562": (53, Shape(1, 2, 200000, 199998, 8, 8, 64, 64, topk=64)),
    # k = 1: the local block alone
    "topk1": (54, Shape(2, 1, 150000, 149999, 8, 4, 128, 128, topk=1)),
    # a full 1M-token sequence (8,191 candidates)
    "rows_8191": (55, Shape(1, 1, 1048576, 1048575, 16, 2, 128, 64, topk=16)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_index_topk_matches_oracle(name):
    cid, s = CASES[name]
    print(f"case {name}: {s}", flush=True)
    inp = make_inputs(s, cid, device="cuda", which=("q_idx", "k_idx"))
    blk, bscore = U.run_index(s, inp["q_idx"], inp["k_idx"])
    # the stand-alone top-k on the same pooled scores
    blk2 = torch.empty_like(blk)
    M.msa_block_topk(s, bscore.clone(), blk2)
    torch.cuda.synchronize()
    assert torch.equal(blk, blk2), "msa_index_topk differs from msa_block_topk on the same pooled scores"
    rows = [(b, t) for b in range(s.batch) for t in range(s.n_q)]
    kseq = {}

    def kseq_of(b):
        if b not in kseq:
            kseq.clear()
            kseq[b] = U.to64(inp["k_idx"][b])
        return kseq[b]

    U.check_index_rows(s, lambda b, t: U.to64(inp["q_idx"][b, t]), kseq_of, blk, bscore, rows)


def test_varlen_decode_index_topk_long_rows():
    """Sequences of 1 to 250,000 tokens in one call."""
    s = Shape(5, 1, 250000, 249999, 8, 2, 128, 128, topk=16)
    lens = [1, 131072, 131073, 250000, 2000]
    inp = make_inputs(s, 56, device="cuda", which=("q_idx", "k_idx"))
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ws = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
    blk = torch.full((s.batch, 1, s.h_kv, s.topk), -7, dtype=torch.int32, device="cuda")
    M.msa_index_topk_varlen(s, seq_len, inp["q_idx"], inp["k_idx"], blk, ws)
    torch.cuda.synchronize()
    n = s.batch * s.h_kv * s.nblk
    bscore = ws[: n * 4].view(torch.float32).view(s.batch, 1, s.h_kv, s.nblk)
    for b, L in enumerate(lens):
        sb = s.replace(batch=1, n_kv=L, pos0=L - 1)
        kseq = U.to64(inp["k_idx"][b, :L])
        U.check_index_rows(sb, U.to64(inp["q_idx"][b:b + 1]), lambda _b: kseq, blk[b:b + 1], bscore[b:b + 1],
                           [(0, 0)])
