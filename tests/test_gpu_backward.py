"""GPU parity of the main-branch backward (msa_sparse_prefill_backward) against
the fp64 oracle.

Tolerances, from the arithmetic (u = 2^-8, the unit roundoff of bf16): products
are exact bf16 x bf16 in fp32; P and dS enter the dv, dk and dq contractions
rounded to bf16 (relative u per term), dq leaves the key-outer kernel as one
bf16 partial per selected block, and every gradient is rounded to bf16 once.
The bound per tensor is
    ||err||_2 / ||ref||_2 <= 1e-2   and   max |err| <= 2e-2 * max |ref|,
and per row (one (token, head) of dq, one key of dk / dv) with a norm of at
least a tenth of the largest row
    ||err|| <= 1e-2 * ||ref|| + allow,
where allow is 0 for dk and dv.  For dq it covers the one error that is not
relative to the row: D = rowsum(dout * out) is taken from the forward's bf16
output, as flash-attention backwards do, not from the exact output.  Element d
of that output carries three roundings, each of mean zero and independent of
the others and across d: P_s before P.V (at most u P_s |v_s,d|), its block's
partial c_b = sum_{s in b} P_s v_s (at most u |c_b,d|) and the result o (at
most u |o_d|).  A rounding error of at most u|x| has a variance of at most
(u x)^2 / 3, so the error of D has a standard deviation of at most
    sigma = u * sqrt(sum_d dout_d^2 (sum_s P_s^2 v_s,d^2 + sum_b c_b,d^2 + o_d^2) / 3);
and because every dS_s = P_s (dP_s - D), an error e in D moves the dq row by
exactly -scale * e * sum_s P_s k_s.  The allowance is six such deviations:
    allow = 6 * scale * sigma * ||sum_s P_s k_s||.
It matters in rows that see a handful of keys, where dS cancels almost
completely: there the D term reaches several percent of the row (an fp64
emulation of the kernel's roundings gives 3.5e-2 for the second token of the
4,096-token workload, and 4e-3 with the exact D); elsewhere it is far below
1e-2.  Keeping dq's partials in fp32 would not change it (the same emulation:
3.5e-2).
"""

import math

import numpy as np
import pytest
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import WORKLOADS, Shape, make_inputs
from oracle import msa_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_REL = 2e-2
ROW_REL = 1e-2
BF16_U = 2.0 ** -8
D_SIGMAS = 6.0


def dq_allow(qh, keys, vals, douth, scale, blocks):
    """Per-head allowance for the D term (module docstring) of one (token,
    group): qh, douth [G][d]; keys, vals [n][d] the visible rows; blocks [n]
    the block of each row."""
    kbar, lse = O.softmax_attention(qh, keys, keys, scale)
    p = np.exp(scale * (qh @ keys.T) - lse[:, None])        # the softmax weights, [G][n]
    var = (p * p) @ (vals * vals) + (p @ vals) ** 2
    for j in np.unique(blocks):
        m = blocks == j
        var += (p[:, m] @ vals[m]) ** 2
    sigma = BF16_U * np.sqrt(np.sum(douth * douth * var, axis=1) / 3.0)
    return D_SIGMAS * scale * sigma * np.linalg.norm(kbar, axis=1)


def dq_allow_all(s: Shape, q, k, v, dout, blk):
    """dq_allow for every (b, t, h) row, from fp64 arrays and a selection."""
    scale = O.default_scale(s.d)
    G = s.group
    allow = np.zeros((s.batch, s.n_q, s.h_q))
    for b in range(s.batch):
        for t in range(s.n_q):
            for g in range(s.h_kv):
                pos = O.visible_positions(blk[b, t, g], s.pos0 + t, s.block, s.n_kv)
                hs = slice(g * G, (g + 1) * G)
                allow[b, t, hs] = dq_allow(q[b, t, hs], k[b, pos, g], v[b, pos, g], dout[b, t, hs], scale,
                                           pos // s.block)
    return allow


def make_dout(s: Shape, seed: int):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((s.batch, s.n_q, s.h_q, s.d), generator=g).to(torch.bfloat16).cuda()


def run_backward(s: Shape, inp, blk, dout):
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    out = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((s.batch, s.n_q, s.h_q), dtype=torch.float32, device="cuda")
    M.msa_sparse_prefill(s, inp["q"], inp["k"], inp["v"], blk, out, lse, ws)
    dq = torch.full((s.batch, s.n_q, s.h_q, s.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dk = torch.full((s.batch, s.n_kv, s.h_kv, s.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dv = torch.full_like(dk, float("nan"))
    M.msa_sparse_prefill_backward(s, inp["q"], inp["k"], inp["v"], blk, out, lse, dout, dq, dk, dv, ws)
    return dq, dk, dv


def check_grad(got: np.ndarray, ref: np.ndarray, what: str, allow=None):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = got - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    mx = np.max(np.abs(err)) / max(np.max(np.abs(ref)), 1e-30)
    rows_ref = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    rows_err = np.linalg.norm(err.reshape(-1, ref.shape[-1]), axis=1)
    rows_allow = np.zeros_like(rows_ref) if allow is None else np.asarray(allow, dtype=np.float64).ravel()
    big = rows_ref >= 0.1 * rows_ref.max() if rows_ref.size else rows_ref > 0
    row_rel = float(np.max(rows_err[big] / rows_ref[big])) if np.any(big) else 0.0
    bound = ROW_REL * rows_ref + rows_allow
    row_use = float(np.max(rows_err[big] / bound[big])) if np.any(big) else 0.0
    print(f"  {what}: rel L2 {rel:.2e}, max {mx:.2e}, worst row {row_rel:.2e}, "
          f"worst row / its bound {row_use:.2f}", flush=True)
    assert rel <= REL_L2 and mx <= MAX_REL and row_use <= 1.0, what
    if np.max(np.abs(ref)) == 0.0:
        assert np.max(np.abs(got)) == 0.0, what


CASES = {
    # the 4096-token MQA workload, G = 4, d = 64
    "tiny_prefill_4k": (1, WORKLOADS["tiny_prefill_4k"][1]),
    # unaligned chunk, ragged n_q, partial last block (1000 % 128 = 104), G = 4
    "chunk_ragged_g4": (11, Shape(1, 300, 1000, 700, 8, 2, 128, 128, topk=4)),
    # two sequences, G = 16, d = 64, topk 3
    "batch2_g16_d64": (12, Shape(2, 257, 600, 343, 16, 1, 64, 64, topk=3)),
    # MHA, topk 2
    "mha_d128": (13, Shape(1, 520, 520, 0, 8, 8, 128, 64, topk=2)),
    # G = 2, topk 32 >= every causal block
    "g2_topk32_all_blocks": (14, Shape(1, 130, 2100, 1970, 16, 8, 64, 128, topk=32)),
    # k = 64, 63 of up to 93 earlier blocks, G = 8
    "topk64": (20, Shape(1, 300, 12000, 11700, 16, 2, 64, 64, topk=64)),
    # G = 8 at the real head shape
    "g8_chunk": (31, Shape(1, 700, 6000, 5300, 64, 8, 128, 128, topk=16)),
    # the whole sequence inside one partial block
    "single_partial_block": (27, Shape(1, 50, 50, 0, 8, 2, 128, 128, topk=16)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity_every_row(name):
    cid, s = CASES[name]
    print(f"case {name}: {s}", flush=True)
    inp = make_inputs(s, cid, device="cuda")
    blk, _ = U.run_index(s, inp["q_idx"], inp["k_idx"])
    dout = make_dout(s, 100 + cid)
    dq, dk, dv = run_backward(s, inp, blk, dout)
    dq2, dk2, dv2 = run_backward(s, inp, blk, dout)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), "not deterministic"
    blk_np = blk.cpu().numpy()
    _, blk_ref = O.msa_index_topk(U.to64(inp["q_idx"]), U.to64(inp["k_idx"]), s.pos0, s.block, s.topk)
    assert np.array_equal(blk_np, blk_ref.astype(np.int32))
    q64, k64, v64, do64 = U.to64(inp["q"]), U.to64(inp["k"]), U.to64(inp["v"]), U.to64(dout)
    rq, rk, rv = O.msa_sparse_attention_grad(q64, k64, v64, blk_ref, do64, s.pos0, s.block)
    check_grad(U.to64(dq), rq, f"{name} dq", dq_allow_all(s, q64, k64, v64, do64, blk_ref))
    check_grad(U.to64(dk), rk, f"{name} dk")
    check_grad(U.to64(dv), rv, f"{name} dv")


def test_backward_caller_selection_with_padding():
    """Hand-made selections: fewer blocks than k, -1 padding in any slot; keys
    nobody selected must come back exactly 0."""
    s = Shape(1, 64, 2048, 1984, 8, 2, 128, 128, topk=6)
    inp = make_inputs(s, 23, device="cuda")
    rng = np.random.default_rng(9)
    blk = np.full((1, s.n_q, s.h_kv, s.topk), -1, dtype=np.int32)
    for t in range(s.n_q):
        jl = (s.pos0 + t) // s.block
        for g in range(s.h_kv):
            n = int(rng.integers(1, 4))
            chosen = sorted(rng.choice(np.arange(2, jl), size=n - 1, replace=False).tolist() + [jl])
            slots = sorted(rng.permutation(s.topk)[:n])
            for sl, j in zip(slots, chosen):
                blk[0, t, g, sl] = j
    dout = make_dout(s, 77)
    dq, dk, dv = run_backward(s, inp, torch.from_numpy(blk).cuda(), dout)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = U.to64(inp["q"]), U.to64(inp["k"]), U.to64(inp["v"]), U.to64(dout)
    rq, rk, rv = O.msa_sparse_attention_grad(q64, k64, v64, blk, do64, s.pos0, s.block)
    check_grad(U.to64(dq), rq, "caller dq", dq_allow_all(s, q64, k64, v64, do64, blk))
    check_grad(U.to64(dk), rk, "caller dk")
    check_grad(U.to64(dv), rv, "caller dv")
    assert float(dk[0, : 2 * s.block].abs().max()) == 0.0 and float(dv[0, : 2 * s.block].abs().max()) == 0.0


def test_backward_without_queries_zeroes_key_gradients():
    s = Shape(1, 0, 1000, 0, 8, 2, 64, 64, topk=4)
    k = torch.randn((1, 1000, 2, 64)).to(torch.bfloat16).cuda()
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(k, float("nan"))
    e = torch.empty((1, 0, 8, 64), dtype=torch.bfloat16, device="cuda")
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    M.msa_sparse_prefill_backward(s, e, k, k, torch.empty((1, 0, 2, 4), dtype=torch.int32, device="cuda"), e,
                                  torch.empty((1, 0, 8), dtype=torch.float32, device="cuda"), e, e, dk, dv, ws)
    torch.cuda.synchronize()
    assert float(dk.abs().max()) == 0.0 and float(dv.abs().max()) == 0.0


def test_backward_full_size_prefill_128k_sampled():
    """The 131,072-token workload in the benchmark's launch configuration: dq on
    sampled (token, group) rows, dk and dv on every key of two whole blocks of
    one group (one selected by ~1,300 queries, one near the end)."""
    from block_sparse_long_score_amd.inputs import sample_rows
    cid, s = WORKLOADS["prefill_128k"]
    inp = make_inputs(s, cid, device="cuda")
    blk, bscore = U.run_index(s, inp["q_idx"], inp["k_idx"])
    dout = make_dout(s, 4242)
    dq, dk, dv = run_backward(s, inp, blk, dout)
    torch.cuda.synchronize()
    print("  gpu done", flush=True)
    scale = O.default_scale(s.d)
    G = s.group
    rows = [(0, t) for t in sample_rows(s.n_q, 6, 1000 * cid + 55, [0, s.n_q - 1])]
    kseq = U.to64(inp["k_idx"][0])
    sels = U.check_index_rows(s, lambda b, t: U.to64(inp["q_idx"][b, t]), lambda b: kseq, blk, bscore, rows)
    g_dk = 5
    keys64 = {g: U.to64(inp["k"][0, :, g]) for g in range(s.h_kv)}
    vals64 = {g: U.to64(inp["v"][0, :, g]) for g in range(s.h_kv)}
    ref_dq, got_dq, allow_dq = [], [], []
    for (b, t, g), sel in sels.items():
        pos = O.visible_positions(sel, s.pos0 + t, s.block, s.n_kv)
        qh, doh = U.to64(inp["q"][b, t, g * G:(g + 1) * G]), U.to64(dout[b, t, g * G:(g + 1) * G])
        gq, _, _ = O.softmax_attention_grad(qh, keys64[g][pos], vals64[g][pos], doh, scale)
        ref_dq.append(gq)
        got_dq.append(U.to64(dq[b, t, g * G:(g + 1) * G]))
        allow_dq.append(dq_allow(qh, keys64[g][pos], vals64[g][pos], doh, scale, pos // s.block))
    check_grad(np.stack(got_dq), np.stack(ref_dq), "128k dq rows", np.stack(allow_dq))
    blk_g = blk[0, :, g_dk].cpu().numpy()
    for j in (512, s.nblk - 3):
        ts = np.nonzero((blk_g == j).any(axis=1))[0]
        print(f"  block {j}: {len(ts)} queries", flush=True)
        rk = np.zeros((s.block, s.d))
        rv = np.zeros((s.block, s.d))
        for t in ts:
            pos = O.visible_positions(blk_g[t], s.pos0 + t, s.block, s.n_kv)
            _, gk, gv = O.softmax_attention_grad(U.to64(inp["q"][0, t, g_dk * G:(g_dk + 1) * G]), keys64[g_dk][pos],
                                                 vals64[g_dk][pos], U.to64(dout[0, t, g_dk * G:(g_dk + 1) * G]),
                                                 scale)
            inb = (pos >= j * s.block) & (pos < (j + 1) * s.block)
            rk[pos[inb] - j * s.block] += gk[inb]
            rv[pos[inb] - j * s.block] += gv[inb]
        check_grad(U.to64(dk[0, j * s.block:(j + 1) * s.block, g_dk]), rk, f"128k dk block {j}")
        check_grad(U.to64(dv[0, j * s.block:(j + 1) * s.block, g_dk]), rv, f"128k dv block {j}")


def test_backward_query_rows_past_4_gib():
    """Five sequences of 65,536 queries (h_q = 64, d = 128): the last
    sequence's q, dout and dq rows start past byte 2^32 (token row T with
    T * h_q * d * 2 > 2^32), so the backward's 32 x 32 -> 64-bit address
    products carry into the upper word.  topk = 2 keeps the workspace near
    11 GB.  dq on sampled rows of the last sequence, dk and dv on every key of
    two whole blocks of one of its groups, and the forward's output on the
    same rows."""
    from block_sparse_long_score_amd.inputs import sample_rows
    s = Shape(5, 65536, 65536, 0, 64, 8, 128, 128, topk=2)
    assert (s.batch - 1) * s.n_q * s.h_q * s.d * 2 >= 1 << 32
    print(f"case rows_past_4_gib: {s}", flush=True)
    inp = make_inputs(s, 41, device="cuda")
    blk, bscore = U.run_index(s, inp["q_idx"], inp["k_idx"])
    gen = torch.Generator(device="cuda").manual_seed(4141)
    dout = torch.randn((s.batch, s.n_q, s.h_q, s.d), device="cuda", generator=gen).to(torch.bfloat16)
    dq, dk, dv = run_backward(s, inp, blk, dout)
    torch.cuda.synchronize()
    print("  gpu done", flush=True)
    b = s.batch - 1
    scale = O.default_scale(s.d)
    G = s.group
    rows = [(b, t) for t in sample_rows(s.n_q, 6, 4142, [0, s.n_q - 1, 4095, 4096])]
    kseq = U.to64(inp["k_idx"][b])
    sels = U.check_index_rows(s, lambda bb, t: U.to64(inp["q_idx"][bb, t]), lambda bb: kseq, blk, bscore, rows)
    out, lse = U.run_sparse(s, inp["q"], inp["k"], inp["v"], blk)
    chk = U.OutCheck("rows past 4 GiB: forward out")
    U.check_sparse_rows(s, inp["q"], inp["k"], inp["v"], sels, out, lse, chk)
    chk.verify()
    del out, lse
    keys64, vals64 = {}, {}

    def kv(g):
        if g not in keys64:
            keys64[g], vals64[g] = U.to64(inp["k"][b, :, g]), U.to64(inp["v"][b, :, g])
        return keys64[g], vals64[g]

    ref_dq, got_dq, allow_dq = [], [], []
    for (bb, t, g), sel in sels.items():
        pos = O.visible_positions(sel, s.pos0 + t, s.block, s.n_kv)
        kk, vv = kv(g)
        qh, doh = U.to64(inp["q"][bb, t, g * G:(g + 1) * G]), U.to64(dout[bb, t, g * G:(g + 1) * G])
        gq, _, _ = O.softmax_attention_grad(qh, kk[pos], vv[pos], doh, scale)
        ref_dq.append(gq)
        got_dq.append(U.to64(dq[bb, t, g * G:(g + 1) * G]))
        allow_dq.append(dq_allow(qh, kk[pos], vv[pos], doh, scale, pos // s.block))
    check_grad(np.stack(got_dq), np.stack(ref_dq), "rows past 4 GiB: dq rows", np.stack(allow_dq))
    g_dk = 3
    kk, vv = kv(g_dk)
    blk_g = blk[b, :, g_dk].cpu().numpy()
    for j in (7, s.nblk - 1):
        ts = np.nonzero((blk_g == j).any(axis=1))[0]
        print(f"  block {j}: {len(ts)} queries", flush=True)
        rk = np.zeros((s.block, s.d))
        rv = np.zeros((s.block, s.d))
        for t in ts:
            pos = O.visible_positions(blk_g[t], s.pos0 + t, s.block, s.n_kv)
            _, gk, gv = O.softmax_attention_grad(U.to64(inp["q"][b, t, g_dk * G:(g_dk + 1) * G]), kk[pos], vv[pos],
                                                 U.to64(dout[b, t, g_dk * G:(g_dk + 1) * G]), scale)
            inb = (pos >= j * s.block) & (pos < (j + 1) * s.block)
            rk[pos[inb] - j * s.block] += gk[inb]
            rv[pos[inb] - j * s.block] += gv[inb]
        check_grad(U.to64(dk[b, j * s.block:(j + 1) * s.block, g_dk]), rk, f"rows past 4 GiB: dk block {j}")
        check_grad(U.to64(dv[b, j * s.block:(j + 1) * s.block, g_dk]), rv, f"rows past 4 GiB: dv block {j}")
