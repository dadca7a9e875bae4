"""The library's calls inside a HIP graph: a decode step and a prefill step are
captured once (torch.cuda.CUDAGraph on the library's stream argument) and
replayed several times with new inputs written into the captured buffers, with
eager work and synchronisations between the replays; every replay must equal
the eager calls on the same inputs bit for bit.  The library allocates, frees,
sets memory and synchronises nothing, so its launches are all a graph holds.
"""

import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu


def capture(calls):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in calls:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_graph_replays_equal_eager(kind):
    if kind == "decode":
        s = Shape(4, 1, 20000, 19999, 64, 8, 128, 128, topk=16)
    else:
        s = Shape(1, 512, 6000, 5488, 16, 2, 128, 128, topk=8)
    print(f"case {kind}: {s}", flush=True)
    inp = make_inputs(s, 61, device="cuda")
    op = M.MSA_OP_SPARSE_DECODE if kind == "decode" else M.MSA_OP_SPARSE_PREFILL
    ws_i = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
    ws_s = M.alloc_workspace(op, s)
    sparse = M.msa_sparse_decode if kind == "decode" else M.msa_sparse_prefill

    def buffers():
        return (torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda"),
                torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device="cuda"),
                torch.empty((s.batch, s.n_q, s.h_q), dtype=torch.float32, device="cuda"))

    blk, out, lse = buffers()
    calls = [lambda: M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], blk, ws_i),
             lambda: sparse(s, inp["q"], inp["k"], inp["v"], blk, out, lse, ws_s)]
    g = capture(calls)
    gen = torch.Generator(device="cuda")
    for r in range(3):
        gen.manual_seed(900 + r)
        inp["q_idx"].copy_(torch.randint(-3, 4, inp["q_idx"].shape, generator=gen, device="cuda").to(torch.bfloat16))
        inp["q"].copy_(torch.randn(inp["q"].shape, generator=gen, device="cuda").to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        blk_e, out_e, lse_e = buffers()
        ws_i2 = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
        ws_s2 = M.alloc_workspace(op, s)
        M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], blk_e, ws_i2)
        sparse(s, inp["q"], inp["k"], inp["v"], blk_e, out_e, lse_e, ws_s2)
        torch.cuda.synchronize()
        assert torch.equal(blk, blk_e), f"replay {r}: selection"
        assert torch.equal(out, out_e) and torch.equal(lse, lse_e), f"replay {r}: output"
