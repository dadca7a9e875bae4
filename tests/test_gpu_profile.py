"""The per-kernel timing hook on the GPU: every launch of a call is recorded
under its kernel name with a positive device time, and recording stops at
msa_profile_end."""

import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu


def test_profile_records_each_launch():
    s = Shape(1, 300, 2000, 1700, 8, 2, 128, 128, topk=8)
    inp = make_inputs(s, 31, device="cuda")
    bscore = torch.empty((s.batch, s.n_q, s.h_kv, s.nblk), dtype=torch.float32, device="cuda")
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device="cuda")
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    M.msa_profile_begin()
    for _ in range(2):
        M.msa_index_scores(s, inp["q_idx"], inp["k_idx"], bscore)
        M.msa_block_topk(s, bscore, blk)
        M.msa_sparse_prefill(s, inp["q"], inp["k"], inp["v"], blk, out, None, ws)
    k = M.msa_profile_end()
    for name in ("index_scores_tiled", "block_topk_rows", "csr_count_chunks", "csr_fill_any", "sparse_kv_outer",
                 "merge_partials"):
        assert name in k, (name, k)
        assert k[name][0] == 2 and k[name][1] > 0.0, (name, k[name])
    M.msa_index_scores(s, inp["q_idx"], inp["k_idx"], bscore)   # not recorded any more
    torch.cuda.synchronize()
    M.msa_profile_begin()
    assert M.msa_profile_end() == {}
