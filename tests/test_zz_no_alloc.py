"""msa_index_topk_noalloc: the allocation-free index top-k on the library's own
scratch, called through the C ABI.  Its selections must equal msa_index_topk's
bit for bit (and the oracle's), on two calls in a row where the second is
smaller than the first, so that stale scratch contents from the first call
cannot leak into the second."""

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SENTINEL = -7


def both(s, seed):
    inp = make_inputs(s, seed, device="cuda")
    ws = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
    ref = torch.full((s.batch, s.n_q, s.h_kv, s.topk), SENTINEL, dtype=torch.int32, device="cuda")
    got = torch.full_like(ref, SENTINEL)
    M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], ref, ws)
    M.msa_index_topk_noalloc(s, inp["q_idx"], inp["k_idx"], got)
    torch.cuda.synchronize()
    return inp, ref, got


def test_noalloc_equals_index_topk_on_two_calls_the_second_smaller():
    shapes = [
        # larger first: a prefill chunk of 3 sequences with a partial last block
        Shape(3, 700, 40000, 39300, 32, 4, 128, 128, topk=16),
        # then a decode batch, much smaller, with 256-token blocks
        Shape(5, 1, 9000, 8999, 16, 4, 128, 64, block=256, topk=8),
    ]
    for i, s in enumerate(shapes):
        print(f"call {i}: {s}", flush=True)
        inp, ref, got = both(s, 61 + i)
        assert not (ref == SENTINEL).any() and not (got == SENTINEL).any()
        assert torch.equal(got, ref), f"call {i}: selections differ from msa_index_topk"
        # and the oracle on a few rows (indices are bit-exact on integer index inputs)
        if s.block == 128:
            rows = [(0, 0), (1, s.n_q // 2), (s.batch - 1, s.n_q - 1)]
            bscore = torch.empty((s.batch, s.n_q, s.h_kv, s.nblk), dtype=torch.float32, device="cuda")
            M.msa_index_scores(s, inp["q_idx"], inp["k_idx"], bscore)
            torch.cuda.synchronize()
            kseq = {b: U.to64(inp["k_idx"][b]) for b in range(s.batch)}
            U.check_index_rows(s, U.to64(inp["q_idx"]), lambda b: kseq[b], got, bscore, rows)


def test_noalloc_rejects_a_call_beyond_the_scratch():
    # 2 * 2048 * 8 * 1024 pooled scores = 128 MiB > 64 MiB (k = 32: off the fused path)
    s = Shape(2, 2048, 131072, 129024, 64, 8, 128, 128, topk=32)
    q_idx = torch.zeros((s.batch, s.n_q, s.h_kv, s.d_idx), dtype=torch.bfloat16, device="cuda")
    k_idx = torch.zeros((s.batch, s.n_kv, s.d_idx), dtype=torch.bfloat16, device="cuda")
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    with pytest.raises(M.MsaError) as e:
        M.msa_index_topk_noalloc(s, q_idx, k_idx, blk)
    assert e.value.name == "MSA_ERR_TOO_LARGE"
