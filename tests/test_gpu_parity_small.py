"""GPU parity against the fp64 oracle on shapes the oracle finishes in seconds.

Every row of every case is compared: pooled block scores and selected blocks
bit-exact, sparse and dense attention outputs within the stated tolerances.
The cases span several tiles with ragged tails, partial last KV blocks,
unaligned chunk offsets, MQA / G=2 / G=4 / G=8 / G=16 / MHA, d and d_idx of 64
and 128, topk 1 / 3 / 16 / 32, the jl + 1 <= k case, and decode.
"""

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd.inputs import WORKLOADS, Shape, make_inputs
from oracle import msa_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = {
    # the 4096-token MQA workload itself, every row
    "tiny_prefill_4k": (1, WORKLOADS["tiny_prefill_4k"][1]),
    # chunk at an unaligned offset, ragged n_q, partial last block (1000 % 128 = 104), G=4
    "chunk_ragged_g4": (11, Shape(1, 300, 1000, 700, 8, 2, 128, 128, topk=4)),
    # two sequences, G=16, d=d_idx=64, topk=3
    "batch2_g16_d64": (12, Shape(2, 257, 600, 343, 16, 1, 64, 64, topk=3)),
    # MHA (h_q == h_kv), mixed dims, topk=2, tiles of the index kernel cross tokens
    "mha_d128_didx64": (13, Shape(1, 520, 520, 0, 8, 8, 128, 64, topk=2)),
    # G=2, topk=32 >= all causal blocks: every row takes the padded path
    "g2_topk32_all_blocks": (14, Shape(1, 130, 2100, 1970, 16, 8, 64, 128, topk=32)),
    # topk=1: only the local block
    "topk1_local_only": (15, Shape(1, 200, 3000, 2800, 8, 4, 128, 128, topk=1)),
    # two query tokens x 8 groups = 16 rows: the skinny index kernel with n_q > 1
    "two_token_chunk": (16, Shape(1, 2, 3000, 2998, 64, 8, 128, 128, topk=16)),
    # decode: three sequences, partial last block, G=8
    "decode_b3_g8": (17, Shape(3, 1, 5000, 4999, 64, 8, 128, 128, topk=16)),
    # decode MHA with 16 K/V heads, d=64
    "decode_mha16_d64": (18, Shape(2, 1, 1500, 1499, 16, 16, 64, 64, topk=4)),
    # decode with fewer causal blocks than k
    "decode_short": (19, Shape(2, 1, 300, 299, 4, 2, 64, 128, topk=16)),
    # k = 64 (8,192 selected tokens): 63 of up to 93 earlier blocks, G = 8
    "topk64_g8": (20, Shape(1, 300, 12000, 11700, 16, 2, 64, 64, topk=64)),
    # k = 48, rows from below k blocks to twice k, MHA
    "topk48_mha": (21, Shape(1, 257, 12600, 12343, 4, 4, 128, 128, topk=48)),
    # decode with k = 64 over 1,000 blocks
    "decode_topk64": (22, Shape(2, 1, 128000, 127999, 16, 2, 128, 128, topk=64)),
    # 256-token blocks: partial last block (1000 = 3 * 256 + 232), ragged chunk, k = 3
    "block256_chunk_ragged": (23, Shape(1, 300, 1000, 700, 8, 2, 128, 128, block=256, topk=3)),
    # 256-token blocks, G = 8, 15 of up to 35 earlier blocks
    "block256_g8": (24, Shape(1, 600, 9000, 8400, 64, 8, 128, 128, block=256, topk=16)),
    # 256-token blocks, k = 32 (64 blocks of 128 in the main branch), two sequences, d = 64
    "block256_k32_d64": (25, Shape(2, 257, 20000, 19743, 16, 2, 64, 64, block=256, topk=32)),
    # 256-token blocks, decode
    "block256_decode": (26, Shape(3, 1, 50000, 49999, 64, 8, 128, 128, block=256, topk=16)),
    # the whole sequence inside one partial block: every row selects block 0 only
    "single_partial_block": (27, Shape(1, 50, 50, 0, 8, 2, 128, 128, topk=16)),
    # decode of the very first token: one key, one block
    "first_token_decode": (28, Shape(1, 1, 1, 0, 4, 1, 64, 64, topk=16)),
    # two full blocks, k = 2: the second block's rows take both blocks
    "two_full_blocks_k2": (29, Shape(1, 256, 256, 0, 8, 2, 64, 64, topk=2)),
    # 256-token blocks, the sequence inside one partial block
    "block256_single_partial": (30, Shape(1, 100, 100, 0, 8, 2, 64, 64, block=256, topk=4)),
}


def all_rows(s):
    return [(b, t) for b in range(s.batch) for t in range(s.n_q)]


@pytest.mark.parametrize("name", list(CASES))
def test_parity_full_oracle(name):
    cid, s = CASES[name]
    print(f"case {name}: {s}", flush=True)
    inp = make_inputs(s, cid, device="cuda")
    blk, bscore = U.run_index(s, inp["q_idx"], inp["k_idx"])
    torch.cuda.synchronize()
    q_idx64 = U.to64(inp["q_idx"])
    kcache = {}

    def kseq(b):
        if b not in kcache:
            kcache[b] = U.to64(inp["k_idx"][b])
        return kcache[b]

    sels = U.check_index_rows(s, q_idx64, kseq, blk, bscore, all_rows(s))

    out, lse = U.run_sparse(s, inp["q"], inp["k"], inp["v"], blk)
    torch.cuda.synchronize()
    chk = U.OutCheck(f"{name} sparse")
    U.check_sparse_rows(s, inp["q"], inp["k"], inp["v"], sels, out, lse, chk)
    chk.verify()

    dout, dlse = U.run_dense(s, inp["q"], inp["k"], inp["v"])
    torch.cuda.synchronize()
    dchk = U.OutCheck(f"{name} dense")
    rows = all_rows(s)
    if len(rows) > 600:                      # the dense oracle loops per head; sample long cases
        rows = rows[:: max(1, len(rows) // 600)] + [rows[-1]]
    U.check_dense_rows(s, inp["q"], inp["k"], inp["v"], rows, dout, dlse, dchk)
    dchk.verify()


def test_decode_matches_single_token_prefill_path():
    """The decode entry point and the CSR prefill path agree on n_q = 1."""
    s = Shape(2, 1, 4000, 3999, 32, 4, 128, 128, topk=16)
    inp = make_inputs(s, 21, device="cuda")
    blk, _ = U.run_index(s, inp["q_idx"], inp["k_idx"])
    o1, l1 = U.run_sparse(s, inp["q"], inp["k"], inp["v"], blk)
    o2, l2 = U.run_sparse_prefill_path(s, inp["q"], inp["k"], inp["v"], blk)
    torch.cuda.synchronize()
    chk = U.OutCheck("decode vs prefill path")
    chk.add(U.to64(o1), U.to64(o2), l1.cpu().numpy(), l2.cpu().numpy())
    chk.verify()


def test_all_ties_select_lowest_blocks():
    """All-zero index queries: every pooled score ties, so each row keeps blocks
    0..k-2 and its local block (closed form of the lower-index tie rule)."""
    s = Shape(1, 600, 5000, 4400, 16, 2, 64, 128, topk=16)
    inp = make_inputs(s, 22, device="cuda")
    q_idx = torch.zeros_like(inp["q_idx"])
    blk, bscore = U.run_index(s, q_idx, inp["k_idx"])
    got = blk.cpu().numpy()
    for t in range(s.n_q):
        jl = (s.pos0 + t) // s.block
        want = list(range(s.topk - 1)) + [jl]
        assert (got[0, t] == np.array(want)).all(), (t, got[0, t])
    assert float(bscore[0, :, :, :34].abs().max()) == 0.0


def test_caller_selection_with_padding_and_skips():
    """msa_sparse_prefill on a hand-made selection: fewer blocks than k, -1
    padding anywhere, entries beyond the local block skipped."""
    s = Shape(1, 64, 2048, 1984, 8, 2, 128, 128, topk=6)
    inp = make_inputs(s, 23, device="cuda")
    rng = np.random.default_rng(5)
    blk = np.full((1, s.n_q, s.h_kv, s.topk), -1, dtype=np.int32)
    for t in range(s.n_q):
        jl = (s.pos0 + t) // s.block
        for g in range(s.h_kv):
            n = int(rng.integers(1, s.topk))
            chosen = sorted(rng.choice(jl, size=n - 1, replace=False).tolist() + [jl])
            slots = rng.permutation(s.topk)[:n]
            for sl, j in zip(sorted(slots), chosen):
                blk[0, t, g, sl] = j
    blk_t = torch.from_numpy(blk).cuda()
    out, lse = U.run_sparse(s, inp["q"], inp["k"], inp["v"], blk_t)
    torch.cuda.synchronize()
    sels = {(0, t, g): blk[0, t, g] for t in range(s.n_q) for g in range(s.h_kv)}
    chk = U.OutCheck("caller selection")
    U.check_sparse_rows(s, inp["q"], inp["k"], inp["v"], sels, out, lse, chk)
    chk.verify()


def test_repeat_runs_are_bit_identical():
    s = Shape(1, 2048, 6144, 4096, 32, 4, 128, 128, topk=16)
    inp = make_inputs(s, 24, device="cuda")
    b1, _ = U.run_index(s, inp["q_idx"], inp["k_idx"])
    b2, _ = U.run_index(s, inp["q_idx"], inp["k_idx"])
    o1, l1 = U.run_sparse(s, inp["q"], inp["k"], inp["v"], b1)
    o2, l2 = U.run_sparse(s, inp["q"], inp["k"], inp["v"], b2)
    d1, _ = U.run_dense(s, inp["q"], inp["k"], inp["v"])
    d2, _ = U.run_dense(s, inp["q"], inp["k"], inp["v"])
    torch.cuda.synchronize()
    assert torch.equal(b1, b2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(d1, d2)


def test_block_topk_entry_matches_oracle_selection():
    """msa_block_topk alone on float scores with heavy ties (not from the index
    kernel): every row against the oracle's selection rule."""
    s = Shape(2, 300, 70000, 69700, 8, 4, 128, 128, topk=16)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    bscore = torch.randint(-6, 7, (s.batch, s.n_q, s.h_kv, s.nblk), generator=g, device="cuda").float() * 0.5
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    from block_sparse_long_score_amd import msa as M
    M.msa_block_topk(s, bscore, blk)
    sc = bscore.cpu().numpy().astype(np.float64)
    got = blk.cpu().numpy()
    for b in range(s.batch):
        for t in range(s.n_q):
            jl = (s.pos0 + t) // s.block
            for gg in range(s.h_kv):
                want = O.select_blocks(sc[b, t, gg, : jl + 1], jl, s.topk)
                assert (got[b, t, gg] == want).all(), (b, t, gg)


@pytest.mark.parametrize("s", [Shape(1, 200, 20000, 19800, 8, 2, 128, 128, topk=16),
                               Shape(1, 64, 1048576, 1048512, 8, 2, 128, 128, topk=16)])
def test_block_topk_signed_zeros_and_denormals(s):
    """Pooled scores drawn from -0, +0, subnormals of both signs, the smallest
    normal and large magnitudes: -0 ties with +0 (ties go to the lower block)
    and subnormals keep their order, for the per-wave rows and the
    per-workgroup long rows."""
    special = np.array([-0.0, 0.0, 1e-40, -1e-40, 1.4e-45, -1.4e-45, 1.1754944e-38, -1.1754944e-38, 1.0, -1.0,
                        3e38, -3e38], dtype=np.float32)
    rng = np.random.default_rng(5)
    sc32 = special[rng.integers(0, len(special), size=(s.batch, s.n_q, s.h_kv, s.nblk))]
    bscore = torch.from_numpy(sc32).cuda()
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    from block_sparse_long_score_amd import msa as M
    M.msa_block_topk(s, bscore, blk)
    got = blk.cpu().numpy()
    sc = sc32.astype(np.float64)
    for t in range(s.n_q):
        jl = (s.pos0 + t) // s.block
        for gg in range(s.h_kv):
            want = O.select_blocks(sc[0, t, gg, : jl + 1], jl, s.topk)
            assert (got[0, t, gg] == want).all(), (t, gg)


@pytest.mark.parametrize("jl_span,topk", [((1048000, 1048575), 16), ((300000, 300127), 32), ((1040000, 1040200), 1),
                                          ((900000, 900100), 64)])
def test_block_topk_long_rows_workgroup_path(jl_span, topk):
    """Rows longer than 2,048 candidates take the workgroup-per-row kernel
    (quarters selected separately, then merged); heavy ties on every row."""
    lo, hi = jl_span
    n_kv = 1048576
    s = Shape(1, hi - lo, n_kv, lo, 8, 4, 128, 128, topk=topk)
    g = torch.Generator(device="cuda")
    g.manual_seed(78 + topk)
    bscore = torch.randint(-3, 4, (s.batch, s.n_q, s.h_kv, s.nblk), generator=g, device="cuda").float()
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    from block_sparse_long_score_amd import msa as M
    M.msa_block_topk(s, bscore, blk)
    got = blk.cpu().numpy()
    sc = bscore.cpu().numpy().astype(np.float64)
    for t in range(0, s.n_q, max(1, s.n_q // 40)):
        jl = (s.pos0 + t) // s.block
        for gg in range(s.h_kv):
            want = O.select_blocks(sc[0, t, gg, : jl + 1], jl, s.topk)
            assert (got[0, t, gg] == want).all(), (t, gg, got[0, t, gg], want)


def test_block_topk_rows_width_buckets():
    """The per-wave rows kernel holds only as many scores per lane as the
    wave's longest row needs (64, 128, 256, 512 or 1,024 candidates): rows on
    both sides of every width boundary, including waves whose rows straddle
    one (8 rows per wave = 2 tokens x 4 groups here), against the oracle's
    selection on heavy-tie integer scores."""
    s = Shape(1, 131072, 131072, 0, 8, 4, 128, 128, topk=16)
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    bscore = torch.randint(-5, 6, (s.batch, s.n_q, s.h_kv, s.nblk), generator=g, device="cuda").float()
    blk = torch.full((s.batch, s.n_q, s.h_kv, s.topk), -7, dtype=torch.int32, device="cuda")
    from block_sparse_long_score_amd import msa as M
    M.msa_block_topk(s, bscore, blk)
    torch.cuda.synchronize()
    assert not bool((blk == -7).any())
    toks = set()
    for jl in (15, 16, 17, 63, 64, 65, 66, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1000, 1023):
        for t in (128 * jl - 2, 128 * jl - 1, 128 * jl, 128 * jl + 1):
            if 0 <= t < s.n_q:
                toks.add(t)
    toks.update(range(5, s.n_q, 4099))
    sc = bscore[0].cpu().numpy().astype(np.float64)
    got = blk[0].cpu().numpy()
    for t in sorted(toks):
        jl = t // s.block
        for gg in range(s.h_kv):
            want = O.select_blocks(sc[t, gg, : jl + 1], jl, s.topk)
            assert (got[t, gg] == want).all(), (t, gg, got[t, gg].tolist(), want.tolist())
