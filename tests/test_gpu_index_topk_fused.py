"""msa_index_topk_fused: the index branch with the top-k fused into the tiled
scorer (k <= 16), so no pooled scores reach memory.  Each workgroup keeps every
row's best k-1 blocks in LDS as the key blocks stream by, and a merge picks
each row's blocks from the survivors of the 1 to 16 workgroups that swept its
row tile.

Every call is checked two ways: sampled rows bit for bit against the oracle
(oracle.index_topk_row: pooled scores by brute force, repeated first-occurrence
argmax), and every row against msa_block_topk on pooled scores from a separate
msa_index_scores call.  Shapes cover 1 to 16 workgroups per tile (the count the
host picks, capped at 16; with one, the workgroup writes the selection itself),
several sequences, partial tiles and partial last blocks, d_idx 64 and 128,
k = 1, 2, 4, 5, 8 and 16, rows made entirely of ties, and the 131,072-token
workload at full size.  msa_index_topk takes the same path for these shapes,
so every prefill parity test with k <= 16 exercises it as well."""

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import WORKLOADS, Shape, make_inputs, sample_rows
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = {
    "three_pieces_k1": (71, Shape(1, 20000, 20000, 0, 8, 8, 64, 64, topk=1)),
    "two_pieces": (72, Shape(1, 32768, 32768, 0, 16, 8, 64, 128, topk=16)),
    "four_pieces_batch4": (73, Shape(4, 4096, 9000, 4904, 16, 8, 128, 128, topk=16)),
    "eight_pieces_d64": (74, Shape(1, 16384, 40000, 23616, 16, 4, 128, 64, topk=16)),
    "eight_pieces_k8_batch2": (75, Shape(2, 8192, 20000, 11808, 32, 4, 128, 128, topk=8)),
    "ten_pieces_k2": (76, Shape(1, 12000, 12000, 0, 8, 4, 64, 64, topk=2)),
    "sixteen_pieces_batch3": (77, Shape(3, 4096, 70000, 65904, 16, 8, 128, 128, topk=16)),
    "eleven_pieces_small_k4": (79, Shape(1, 300, 1000, 700, 8, 8, 64, 64, topk=4)),
    "one_tile_capped_at_16": (80, Shape(1, 100, 131072, 130972, 16, 8, 128, 128, topk=16)),
    "one_piece_direct_batch64": (81, Shape(64, 4096, 4096, 0, 64, 8, 128, 128, topk=16)),
    "one_piece_direct_k5_d64": (82, Shape(48, 2500, 7000, 4500, 8, 8, 64, 64, topk=5)),
}


def pieces_of(s: Shape) -> int:
    """Workgroups per row tile, read back from the workspace size (128 bytes
    per row and piece; none with one piece, which writes blk_idx itself)."""
    rows = s.batch * s.n_q * s.h_kv
    return max(1, M.msa_workspace_size(M.MSA_OP_INDEX_TOPK_FUSED, s) // (rows * 128))


def run_fused(s: Shape, q_idx, k_idx):
    """The fused selection in a guarded buffer; every row must equal
    msa_block_topk's on separately computed pooled scores, which are
    returned for the oracle comparison."""
    ws = M.alloc_workspace(M.MSA_OP_INDEX_TOPK_FUSED, s)
    g = U.Guarded((s.batch, s.n_q, s.h_kv, s.topk), torch.int32)
    M.msa_index_topk_fused(s, q_idx, k_idx, g.view, ws)
    torch.cuda.synchronize()
    g.check("blk_idx")
    bscore = torch.empty((s.batch, s.n_q, s.h_kv, s.nblk), dtype=torch.float32, device="cuda")
    M.msa_index_scores(s, q_idx, k_idx, bscore)
    ref = torch.empty_like(g.view)
    M.msa_block_topk(s, bscore, ref)
    torch.cuda.synchronize()
    diff = (ref != g.view).nonzero()
    assert diff.numel() == 0, f"fused selection differs from msa_block_topk at {diff[:4].tolist()}"
    return g.view, bscore


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_index_topk(name):
    cid, s = CASES[name]
    p = pieces_of(s)
    print(f"case {name}: {s}, pieces {p}", flush=True)
    assert 1 <= p <= 16
    inp = make_inputs(s, cid, device="cuda", which=("q_idx", "k_idx"))
    blk, bscore = run_fused(s, inp["q_idx"], inp["k_idx"])
    rows = [(b, t) for b in range(s.batch) for t in sample_rows(s.n_q, 6, 1000 * cid + 7, [0, s.n_q - 1])]
    kseq = {}

    def kseq_of(b):
        if b not in kseq:
            kseq.clear()
            kseq[b] = U.to64(inp["k_idx"][b])
        return kseq[b]

    U.check_index_rows(s, lambda b, t: U.to64(inp["q_idx"][b, t]), kseq_of, blk, bscore, rows)


def test_fused_index_topk_all_ties():
    """A zero index query ties every block at pooled score 0: each row keeps
    blocks 0 .. k-2 and its local block."""
    s = Shape(1, 32768, 32768, 0, 16, 8, 64, 128, topk=16)
    inp = make_inputs(s, 78, device="cuda", which=("k_idx",))
    q_idx = torch.zeros((s.batch, s.n_q, s.h_kv, s.d_idx), dtype=torch.bfloat16, device="cuda")
    blk, _ = run_fused(s, q_idx, inp["k_idx"])
    got = blk.cpu().numpy()
    for t in range(0, s.n_q, 517):
        jl = t // s.block
        want = np.arange(jl + 1) if jl + 1 <= s.topk else np.concatenate([np.arange(s.topk - 1), [jl]])
        want = np.concatenate([want, -np.ones(s.topk - len(want), dtype=np.int64)])
        for g in range(s.h_kv):
            assert (got[0, t, g] == want).all(), (t, g, got[0, t, g].tolist())


def test_fused_index_topk_128k():
    """The 131,072-token workload (8 groups, d_idx 128, k 16) at full size:
    one workgroup per row tile writes the selection itself (no workspace,
    against 4 GiB of pooled scores unfused); every row equals msa_block_topk,
    sampled rows the oracle."""
    cid, s = WORKLOADS["prefill_128k"]
    print(f"case prefill_128k fused: {s}, pieces {pieces_of(s)}", flush=True)
    inp = make_inputs(s, cid, device="cuda", which=("q_idx", "k_idx"))
    blk, bscore = run_fused(s, inp["q_idx"], inp["k_idx"])
    k64 = U.to64(inp["k_idx"][0])
    rows = [(0, t) for t in sample_rows(s.n_q, 8, 9107, [0, 127, 128, s.n_q - 1])]
    U.check_index_rows(s, lambda b, t: U.to64(inp["q_idx"][b, t]), lambda b: k64, blk, bscore, rows)
