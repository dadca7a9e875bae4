"""Variable-length decode: one call over sequences of different lengths in a
common cache capacity.  Each sequence must give exactly what the oracle gives
for that sequence alone (indices and pooled scores bit-exact, outputs within
the stated tolerances), and full-length sequences exactly what the
fixed-length entry points give."""

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape, make_inputs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def run_varlen(s, seq_len, inp):
    lens = torch.tensor(seq_len, dtype=torch.int32, device="cuda")
    ws_i = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
    blk = torch.empty((s.batch, 1, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    M.msa_index_topk_varlen(s, lens, inp["q_idx"], inp["k_idx"], blk, ws_i)
    n = s.batch * s.h_kv * s.nblk
    bscore = ws_i[: n * 4].view(torch.float32).view(s.batch, 1, s.h_kv, s.nblk).clone()
    out = torch.empty((s.batch, 1, s.h_q, s.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((s.batch, 1, s.h_q), dtype=torch.float32, device="cuda")
    ws_s = M.alloc_workspace(M.MSA_OP_SPARSE_DECODE, s)
    M.msa_sparse_decode_varlen(s, lens, inp["q"], inp["k"], inp["v"], blk, out, lse, ws_s)
    torch.cuda.synchronize()
    return blk, bscore, out, lse


def check_against_oracle(s, seq_len, inp, blk, bscore, out, lse, what):
    chk = U.OutCheck(what)
    for b, n in enumerate(seq_len):
        n = min(max(n, 1), s.n_kv)                    # the documented clamp
        sb = s.replace(batch=1, n_kv=n, pos0=n - 1)
        kseq = U.to64(inp["k_idx"][b, :n])
        sels = U.check_index_rows(sb, U.to64(inp["q_idx"][b:b + 1]), lambda _b: kseq, blk[b:b + 1],
                                  bscore[b:b + 1], [(0, 0)])
        U.check_sparse_rows(sb, inp["q"][b:b + 1], inp["k"][b:b + 1, :n], inp["v"][b:b + 1, :n], sels,
                            out[b:b + 1], lse[b:b + 1], chk)
    chk.verify()


@pytest.mark.parametrize("case", ["mixed_g4", "mixed_mqa_d64", "block256"])
def test_varlen_decode_matches_oracle_per_sequence(case):
    if case == "mixed_g4":
        s = Shape(7, 1, 3000, 2999, 16, 4, 128, 128, topk=8)
        seq_len = [1, 127, 128, 129, 1023, 2000, 3000]
    elif case == "block256":
        s = Shape(7, 1, 9000, 8999, 16, 4, 128, 128, block=256, topk=8)
        seq_len = [1, 255, 256, 257, 3000, 8000, 9000]
    else:
        s = Shape(5, 1, 2500, 2499, 4, 1, 64, 64, topk=16)
        seq_len = [2500, 5, 300, 2047, 1300]
    print(f"case {case}: {s} lengths {seq_len}", flush=True)
    inp = make_inputs(s, 41, device="cuda")
    blk, bscore, out, lse = run_varlen(s, seq_len, inp)
    check_against_oracle(s, seq_len, inp, blk, bscore, out, lse, f"varlen {case}")


def test_varlen_clamps_lengths_into_the_cache():
    """Lengths below 1 or above the capacity act as 1 and as the capacity."""
    s = Shape(3, 1, 1000, 999, 8, 2, 128, 128, topk=4)
    inp = make_inputs(s, 42, device="cuda")
    got = run_varlen(s, [0, 1000 + 77, -5], inp)
    want = run_varlen(s, [1, 1000, 1], inp)
    for a, w in zip(got, want):
        if a.dtype == torch.float32 and a.dim() == 4:     # pooled scores: entries past jl are unspecified
            continue
        assert torch.equal(a, w)
    check_against_oracle(s, [0, 1077, -5], inp, *got, "varlen clamp")


def test_varlen_full_length_equals_fixed_length_decode():
    s = Shape(4, 1, 4000, 3999, 32, 4, 128, 128, topk=16)
    inp = make_inputs(s, 43, device="cuda")
    blk_v, _, out_v, lse_v = run_varlen(s, [s.n_kv] * s.batch, inp)
    blk, _ = U.run_index(s, inp["q_idx"], inp["k_idx"])
    out, lse = U.run_sparse(s, inp["q"], inp["k"], inp["v"], blk)
    torch.cuda.synchronize()
    assert torch.equal(blk_v, blk)
    assert torch.equal(out_v, out) and torch.equal(lse_v, lse)
