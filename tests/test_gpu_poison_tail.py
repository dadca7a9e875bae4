"""Keys past the end of the cache are never read.

K, V (and the index keys) are placed at the start of larger buffers whose rest
is NaN.  The sequences' last K/V block is partial, so a kernel that loaded a
whole block and used the rows past n_kv would turn a 0 * NaN into NaN; the
padding keeps such a read inside allocated memory.  Each attention call must
give, bit for bit, what it gives on the same values in plain tensors (the
oracle comparison of the same calls is in the parity tests).
"""

from __future__ import annotations

import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs


pytestmark = pytest.mark.gpu

PAD = 1 << 20        # elements of NaN after each tensor (more than a block of K/V rows)


def poisoned(t: torch.Tensor) -> torch.Tensor:
    buf = torch.full((t.numel() + PAD,), float("nan"), dtype=t.dtype, device=t.device)
    buf[: t.numel()].copy_(t.reshape(-1))
    return buf[: t.numel()].view(t.shape)


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


CASES = {
    # prefill, two sequences, 600 = 4 * 128 + 88 keys (one partial block each)
    "prefill_b2_g8": (41, Shape(2, 200, 600, 400, 64, 8, 128, 128, topk=4)),
    # prefill, one sequence inside a single partial block, d = 64
    "prefill_one_block_d64": (42, Shape(1, 90, 90, 0, 8, 2, 64, 64, topk=16)),
    # decode, three sequences of 5,000 = 39 * 128 + 8 keys
    "decode_b3_g8": (43, Shape(3, 1, 5000, 4999, 64, 8, 128, 128, topk=16)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_keys_past_the_cache_end_are_not_read(name):
    cfg, s = CASES[name]
    print(f"[poison] {name} {s}", flush=True)
    inp = make_inputs(s, cfg, device="cuda")
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], blk, M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s))
    blk_p = torch.empty_like(blk)
    M.msa_index_topk(s, inp["q_idx"], poisoned(inp["k_idx"]), blk_p, M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s))
    torch.cuda.synchronize()
    assert torch.equal(blk, blk_p), "index top-k read index keys past the cache end"

    k_p, v_p = poisoned(inp["k"]), poisoned(inp["v"])
    decode = s.n_q == 1
    for label, call in (("sparse", M.msa_sparse_decode if decode else M.msa_sparse_prefill), ("dense", M.msa_dense_gqa)):
        outs = []
        for k, v in ((inp["k"], inp["v"]), (k_p, v_p)):
            out = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((s.batch, s.n_q, s.h_q), dtype=torch.float32, device="cuda")
            if label == "sparse":
                ws = M.alloc_workspace(M.MSA_OP_SPARSE_DECODE if decode else M.MSA_OP_SPARSE_PREFILL, s)
                call(s, inp["q"], k, v, blk, out, lse, ws)
            else:
                ws = M.alloc_workspace(M.MSA_OP_DENSE_GQA, s)
                call(s, inp["q"], k, v, out, lse, ws)
            torch.cuda.synchronize()
            outs.append((out, lse))
        (o0, l0), (o1, l1) = outs
        assert not bool(torch.isnan(o1).any()), f"{label}: NaN from keys past the cache end"
        assert torch.equal(bits(o0), bits(o1)) and torch.equal(bits(l0), bits(l1)), f"{label}: output depends on memory past the cache end"
