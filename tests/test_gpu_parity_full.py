"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, checked on seeded samples of rows the oracle computes one by
one (first and last rows and block-boundary rows always included).

  prefill_32k       every stage on 32,768 tokens; 40 sampled rows (+ dense)
  prefill_128k      131,072 tokens; 24 sampled rows (+ dense on 2 rows)
  decode_256k_b64   64 sequences of 262,144 tokens; 16 sequences
  prefill_chunk_1m  8,192 queries at 1,040,384.. of a 1,048,576 cache; 20 rows
  decode_1m_b8      8 sequences of 1,048,576 tokens; all 8
  topk_full_rows    the top-k alone on 1,048,576 rows of 1,023 candidates; 64 rows
"""

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs, sample_rows
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def run_case(name, n_rows, n_dense_rows, seqs=None):
    cid, s = WORKLOADS[name]
    print(f"case {name}: {s}", flush=True)
    inp = make_inputs(s, cid, device="cuda")
    blk, bscore = U.run_index(s, inp["q_idx"], inp["k_idx"])
    out, lse = U.run_sparse(s, inp["q"], inp["k"], inp["v"], blk)
    torch.cuda.synchronize()
    print(f"  gpu done", flush=True)
    if s.n_q == 1:
        seq_list = list(range(s.batch)) if seqs is None else sample_rows(s.batch, seqs, 1000 * cid + 98)
        rows = [(b, 0) for b in seq_list]
    else:
        boundary = [t for t in range(s.n_q) if (s.pos0 + t) % s.block in (0, s.block - 1)]
        must = boundary[:: max(1, len(boundary) // 6)][:6]
        rows = [(0, t) for t in sample_rows(s.n_q, n_rows, 1000 * cid + 99, must)]
    kcache = {}

    def kseq(b):
        if b not in kcache:
            kcache.clear()
            kcache[b] = U.to64(inp["k_idx"][b])
        return kcache[b]

    sels = U.check_index_rows(s, lambda b, t: U.to64(inp["q_idx"][b, t]), kseq, blk, bscore, rows)
    print(f"  {len(rows)} rows: block scores and selections bit-exact", flush=True)
    chk = U.OutCheck(f"{name} sparse")
    U.check_sparse_rows(s, inp["q"], inp["k"], inp["v"], sels, out, lse, chk)
    chk.verify()
    if n_dense_rows:
        dout, dlse = U.run_dense(s, inp["q"], inp["k"], inp["v"])
        torch.cuda.synchronize()
        dchk = U.OutCheck(f"{name} dense")
        U.check_dense_rows(s, inp["q"], inp["k"], inp["v"], rows[:n_dense_rows], dout, dlse, dchk)
        dchk.verify()


def test_prefill_32k():
    run_case("prefill_32k", 40, 4)


def test_prefill_128k():
    run_case("prefill_128k", 24, 2)


def test_decode_256k_b64():
    run_case("decode_256k_b64", 0, 4, seqs=16)


def test_prefill_chunk_1m():
    run_case("prefill_chunk_1m", 20, 1)


def test_decode_1m_b8():
    run_case("decode_1m_b8", 0, 2)


def test_topk_full_rows():
    """The benchmark's top-k-alone leg at its full size (1,048,576 rows of
    1,023 candidates, the same seeded pooled scores and launch): selections
    bit-exact against the oracle's select_blocks on 64 sampled rows."""
    import importlib.util
    import os

    from block_sparse_long_score_amd import msa as M
    from block_sparse_long_score_amd.inputs import Shape
    from oracle import msa_oracle as O

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_for_topk", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    s = Shape(**bench.TOPK_FULL_SHAPE)
    print(f"case topk_full_rows: {s}", flush=True)
    sc = bench.topk_full_scores(torch, s)
    blk = torch.full((s.batch, s.n_q, s.h_kv, s.topk), -7, dtype=torch.int32, device="cuda")
    M.msa_block_topk(s, sc, blk)
    torch.cuda.synchronize()
    assert not (blk == -7).any(), "a row was not written"
    rows = s.batch * s.n_q * s.h_kv
    flat_sc, flat_blk = sc.view(rows, s.nblk), blk.view(rows, s.topk)
    for r in sample_rows(rows, 64, 3098):
        t = (r // s.h_kv) % s.n_q
        jl = (s.pos0 + t) // s.block
        want = O.select_blocks(flat_sc[r].double().cpu().numpy(), jl, s.topk)
        got = flat_blk[r].cpu().numpy()
        assert np.array_equal(got, want.astype(np.int32)), (r, got.tolist(), want.tolist())
