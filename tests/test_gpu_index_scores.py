"""msa_index_scores on its own: the pooled block scores bit-exact against the
oracle's block max-pool (yhxrc.cn article, section "第一步：索引分支"), and the
output contract that entries past a query's own block are left untouched.

The buffer is filled with a NaN bit pattern the kernel never produces (every
score is finite) before the call.  Every entry j <= (pos0 + t) / 128 must be
overwritten and every later entry must keep the pattern; both are checked over
the whole buffer.  Values are compared on sampled tokens, including every
token of the last, partial row tile.  The shapes hit the scorer's write-out
paths: a last tile whose first wave holds fewer than 128 rows, a group count
that does not divide a wave's 128 rows (tokens straddle waves), row tiles cut
into several workgroup pieces (groups of pooled blocks that start mid-range),
unaligned chunk offsets, and d_idx of 64 and 128.
"""

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs
from oracle import msa_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC0DEAD
ROWS_PER_TILE = 1024                          # (token, group) rows per scorer workgroup tile

SHAPES = {
    # 3 groups: 2,100 rows, the last tile holds 52 rows (one partial wave); chunk at 2,300 (2300 % 128 = 124)
    "g3_partial_tile_unaligned": (41, Shape(1, 700, 3000, 2300, 6, 3, 64, 128)),
    # MQA, two sequences, d_idx = 64, tiles cut into several pieces
    "mqa_b2_didx64": (42, Shape(2, 1000, 1000, 0, 8, 1, 64, 64)),
    # 16 groups, 71 tiles: pairs cut into pieces whose pooled groups start mid-range
    "g16_many_tiles": (43, Shape(1, 4500, 4500, 0, 16, 16, 64, 128)),
}


def sample_tokens(s: Shape, rng) -> list:
    last_tile_row0 = ((s.n_q * s.h_kv - 1) // ROWS_PER_TILE) * ROWS_PER_TILE
    tail = list(range(last_tile_row0 // s.h_kv, s.n_q))
    picks = rng.choice(s.n_q, size=min(40, s.n_q), replace=False).tolist()
    return sorted(set([0, s.n_q - 1] + tail[-200:] + picks))


@pytest.mark.parametrize("name", list(SHAPES))
def test_index_scores_bit_exact_and_causal_entries_untouched(name):
    cid, s = SHAPES[name]
    print(f"case {name}: {s}", flush=True)
    inp = make_inputs(s, cid, device="cuda")
    bscore = torch.empty((s.batch, s.n_q, s.h_kv, s.nblk), dtype=torch.float32, device="cuda")
    bscore.view(torch.int32).fill_(SENTINEL)
    M.msa_index_scores(s, inp["q_idx"], inp["k_idx"], bscore)
    torch.cuda.synchronize()

    bits = bscore.view(torch.int32)
    jl = (s.pos0 + torch.arange(s.n_q, device="cuda")) // s.block
    past = torch.arange(s.nblk, device="cuda")[None, :] > jl[:, None]          # [n_q][nblk]
    past = past[None, :, None, :].expand_as(bits)
    assert torch.all(bits[past] == SENTINEL), "an entry past the query's own block was written"
    assert not torch.any(bits[~past] == SENTINEL), "an entry up to the query's own block was not written"

    rng = np.random.default_rng(1000 * cid + 99)
    q64 = U.to64(inp["q_idx"])
    for b in range(s.batch):
        kseq = U.to64(inp["k_idx"][b])
        got = bscore[b].cpu().numpy()
        for t in sample_tokens(s, rng):
            p = s.pos0 + t
            for g in range(s.h_kv):
                pooled, _ = O.index_topk_row(q64[b, t, g], kseq, p, s.block, s.topk)
                assert np.array_equal(got[t, g, : p // s.block + 1], pooled.astype(np.float32)), (name, b, t, g)
