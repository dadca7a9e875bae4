"""Chunked whole-sequence prefill: index branch + sparse attention run chunk by
chunk must reproduce the one-shot calls bit for bit (every row depends only
on itself), for ragged last chunks, several sequences and offset queries, and
match the oracle on sampled rows."""

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = {
    # two sequences, queries at an offset, ragged last chunk (300, 300, 300, 100)
    "batch2_offset_ragged": (51, Shape(2, 1000, 3000, 2000, 16, 4, 128, 128, topk=8), 300),
    # the 4,096-token MQA prefill in chunks of 1,024
    "mqa_4k": (52, Shape(1, 4096, 4096, 0, 4, 1, 64, 64, topk=16), 1024),
    # one chunk larger than the call
    "single_chunk": (53, Shape(1, 700, 2500, 1800, 8, 2, 128, 64, topk=4), 5000),
    # chunk of one query
    "chunk_of_one": (54, Shape(1, 40, 1500, 1460, 8, 8, 64, 128, topk=16), 1),
    # 256-token blocks, ragged last chunk
    "block256": (55, Shape(2, 1000, 6000, 5000, 16, 4, 128, 128, block=256, topk=8), 384),
}


@pytest.mark.parametrize("name", list(CASES))
def test_chunked_equals_one_shot(name):
    cid, s, chunk = CASES[name]
    print(f"case {name}: {s} chunk {chunk}", flush=True)
    inp = make_inputs(s, cid, device="cuda")
    blk_c = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    out_c = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device="cuda")
    lse_c = torch.empty((s.batch, s.n_q, s.h_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, M.msa_prefill_chunked_workspace_size(s, chunk)), dtype=torch.uint8, device="cuda")
    M.msa_prefill_chunked(s, chunk, inp["q_idx"], inp["k_idx"], inp["q"], inp["k"], inp["v"], blk_c, out_c, lse_c, ws)
    blk, bscore = U.run_index(s, inp["q_idx"], inp["k_idx"])
    out, lse = U.run_sparse(s, inp["q"], inp["k"], inp["v"], blk)
    torch.cuda.synchronize()
    assert torch.equal(blk_c, blk)
    assert torch.equal(out_c, out) and torch.equal(lse_c, lse)
    # and the oracle on a few rows, the first and last of each chunk
    rows = sorted({(b, t) for b in range(s.batch) for t0 in range(0, s.n_q, chunk)
                   for t in (t0, min(t0 + chunk, s.n_q) - 1)})[:24]
    kcache = {}

    def kseq(b):
        if b not in kcache:
            kcache[b] = U.to64(inp["k_idx"][b])
        return kcache[b]

    sels = U.check_index_rows(s, lambda b, t: U.to64(inp["q_idx"][b, t]), kseq, blk_c, bscore, rows)
    chk = U.OutCheck(f"chunked {name}")
    U.check_sparse_rows(s, inp["q"], inp["k"], inp["v"], sels, out_c, lse_c, chk)
    chk.verify()


def test_chunked_workspace_is_one_chunk():
    s = Shape(1, 1048576, 1048576, 0, 64, 8, 128, 128, topk=16)
    n = M.msa_prefill_chunked_workspace_size(s, 8192)
    assert 0 < n < 5 * 2**30, n                        # one chunk's pooled scores and partials (~4.1 GiB)
