"""Helpers shared by the GPU tests: run the library through the binding and
compare against the fp64 oracle with the tolerances the method is held to.

Tolerances (bf16 outputs, fp32 accumulation inside the kernels):
  * block scores (integer-valued index inputs) and block indices: bit-exact;
  * attention outputs: max |err| <= 2e-2 and mean |err| <= 2e-3 over all
    compared elements, plus per-(token, head) ||err||_2 / ||ref||_2 <= 1e-2
    and |lse - lse_ref| <= 1e-3 (stricter guards: with N(0,1) values a late
    row has |o| ~ 0.04, so the absolute bound alone would miss a dropped block).
"""

from __future__ import annotations

import numpy as np
import torch

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import Shape
from oracle import msa_oracle as O

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
ROW_REL = 1e-2
LSE_ABS = 1e-3


def to64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


# Outputs are views into larger buffers whose every element starts as a
# sentinel: NaN for the float outputs, -7 (never a block index or padding) for
# the selections.  After a call, the guard bands on both sides must still hold
# the sentinel bit for bit, and no sentinel may survive inside the output.
GUARD = 4096
_SENTINEL = {torch.bfloat16: float("nan"), torch.float32: float("nan"), torch.int32: -7}
_BITS = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.int32: torch.int32}


class Guarded:
    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape))
        self.dtype = dtype
        self.buf = torch.full((self.n + 2 * GUARD,), _SENTINEL[dtype], dtype=dtype, device="cuda")
        self.sentinel_bits = self.buf[:1].view(_BITS[dtype]).clone()
        self.view = self.buf[GUARD:GUARD + self.n].view(shape)

    def check(self, what: str):
        bits = self.buf.view(_BITS[self.dtype])
        for band, name in ((bits[:GUARD], "before"), (bits[GUARD + self.n:], "after")):
            assert bool((band == self.sentinel_bits).all()), f"{what}: a write landed in the guard band {name} it"
        inside = bits[GUARD:GUARD + self.n]
        assert not bool((inside == self.sentinel_bits).any()), f"{what}: an element was never written"


def run_index(s: Shape, q_idx, k_idx):
    """msa_index_topk's selection, and the pooled scores the selection rests on.
    With 128-token blocks the pooled scores come from a separate
    msa_index_scores call and the selection must equal msa_block_topk's on them
    in every row (so each test checks all rows' selections, not only the rows
    it compares with the oracle); with 256-token blocks they are read from
    msa_index_topk's workspace, where it documents them."""
    ws = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
    g = Guarded((s.batch, s.n_q, s.h_kv, s.topk), torch.int32)
    M.msa_index_topk(s, q_idx, k_idx, g.view, ws)
    torch.cuda.synchronize()
    g.check("blk_idx")
    if s.block == 128:
        bscore = torch.empty((s.batch, s.n_q, s.h_kv, s.nblk), dtype=torch.float32, device="cuda")
        M.msa_index_scores(s, q_idx, k_idx, bscore)
        ref = torch.empty_like(g.view)
        M.msa_block_topk(s, bscore, ref)
        torch.cuda.synchronize()
        diff = (ref != g.view).nonzero()
        assert diff.numel() == 0, f"msa_index_topk differs from msa_block_topk on its pooled scores at {diff[:4].tolist()}"
        return g.view, bscore
    n = s.batch * s.n_q * s.h_kv * s.nblk
    bscore = ws[: n * 4].view(torch.float32).view(s.batch, s.n_q, s.h_kv, s.nblk)
    return g.view, bscore


def _run_out_lse(s: Shape, fn):
    go = Guarded((s.batch, s.n_q, s.h_q, s.d), torch.bfloat16)
    gl = Guarded((s.batch, s.n_q, s.h_q), torch.float32)
    fn(go.view, gl.view)
    torch.cuda.synchronize()
    go.check("out")
    gl.check("lse")
    return go.view, gl.view


def run_sparse(s: Shape, q, k, v, blk):
    if s.n_q == 1:
        ws = M.alloc_workspace(M.MSA_OP_SPARSE_DECODE, s)
        return _run_out_lse(s, lambda out, lse: M.msa_sparse_decode(s, q, k, v, blk, out, lse, ws))
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    return _run_out_lse(s, lambda out, lse: M.msa_sparse_prefill(s, q, k, v, blk, out, lse, ws))


def run_sparse_prefill_path(s: Shape, q, k, v, blk):
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    return _run_out_lse(s, lambda out, lse: M.msa_sparse_prefill(s, q, k, v, blk, out, lse, ws))


def run_dense(s: Shape, q, k, v):
    ws = M.alloc_workspace(M.MSA_OP_DENSE_GQA, s)
    return _run_out_lse(s, lambda out, lse: M.msa_dense_gqa(s, q, k, v, out, lse, ws))


class OutCheck:
    """Accumulates output comparisons, asserts the bounds at the end."""

    def __init__(self, what: str):
        self.what = what
        self.max_abs = 0.0
        self.sum_abs = 0.0
        self.count = 0
        self.worst_rel = 0.0
        self.worst_lse = 0.0

    def add(self, got: np.ndarray, ref: np.ndarray, lse_got=None, lse_ref=None):
        got = np.asarray(got, dtype=np.float64).reshape(-1, ref.shape[-1])
        ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
        err = np.abs(got - ref)
        self.max_abs = max(self.max_abs, float(err.max()))
        self.sum_abs += float(err.sum())
        self.count += err.size
        rel = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
        self.worst_rel = max(self.worst_rel, float(rel.max()))
        if lse_got is not None:
            d = np.abs(np.asarray(lse_got, dtype=np.float64).ravel() - np.asarray(lse_ref).ravel())
            self.worst_lse = max(self.worst_lse, float(d.max()))

    def verify(self):
        mean = self.sum_abs / max(self.count, 1)
        msg = (f"{self.what}: max_abs={self.max_abs:.3e} mean_abs={mean:.3e} "
               f"worst_row_rel={self.worst_rel:.3e} worst_lse={self.worst_lse:.3e} over {self.count} values")
        print(msg)
        assert self.count > 0, msg
        assert self.max_abs <= MAX_ABS, msg
        assert mean <= MEAN_ABS, msg
        assert self.worst_rel <= ROW_REL, msg
        assert self.worst_lse <= LSE_ABS, msg
        return msg


def check_index_rows(s: Shape, q_idx64, kseq64_of, blk_gpu, bscore_gpu, rows):
    """Bit-exact check of pooled scores (j <= jl) and selections on (b, t) rows.
    q_idx64 is an fp64 array [b][t][g][d_idx] or a callable (b, t) -> [g][d_idx];
    kseq64_of(b) returns the fp64 index keys of sequence b."""
    qrow = q_idx64 if callable(q_idx64) else (lambda b, t: q_idx64[b, t])
    sels = {}
    for b, t in rows:
        p = s.pos0 + t
        jl = p // s.block
        kseq = kseq64_of(b)
        bs = bscore_gpu[b, t, :, : jl + 1].cpu().numpy()
        bk = blk_gpu[b, t].cpu().numpy()
        for g in range(s.h_kv):
            pooled, sel = O.index_topk_row(qrow(b, t)[g], kseq, p, s.block, s.topk)
            assert np.array_equal(bs[g], pooled.astype(np.float32)), f"bscore mismatch b={b} t={t} g={g}"
            assert np.array_equal(bk[g], sel.astype(np.int32)), \
                f"selection mismatch b={b} t={t} g={g}: gpu={bk[g].tolist()} oracle={sel.tolist()}"
            sels[(b, t, g)] = sel
    return sels


def gather_rows(x: torch.Tensor, b: int, pos: np.ndarray, g: int) -> np.ndarray:
    idx = torch.as_tensor(pos, dtype=torch.long, device=x.device)
    return to64(x[b].index_select(0, idx)[:, g])


def check_sparse_rows(s: Shape, q, k, v, sels, out, lse, chk: OutCheck, scale=None):
    scale = O.default_scale(s.d) if scale is None else scale
    G = s.group
    for (b, t, g), sel in sels.items():
        p = s.pos0 + t
        pos = O.visible_positions(sel, p, s.block, s.n_kv)
        kk, vv = gather_rows(k, b, pos, g), gather_rows(v, b, pos, g)
        qh = to64(q[b, t, g * G:(g + 1) * G])
        o_ref, l_ref = O.softmax_attention(qh, kk, vv, scale)
        chk.add(to64(out[b, t, g * G:(g + 1) * G]), o_ref, lse[b, t, g * G:(g + 1) * G].cpu().numpy(), l_ref)


def check_dense_rows(s: Shape, q, k, v, rows, out, lse, chk: OutCheck, scale=None):
    scale = O.default_scale(s.d) if scale is None else scale
    G = s.group
    for b, t in rows:
        p = s.pos0 + t
        for g in range(s.h_kv):
            kk = to64(k[b, : p + 1, g])
            vv = to64(v[b, : p + 1, g])
            for hh in range(G):
                h = g * G + hh
                o_ref, l_ref = O.softmax_attention(to64(q[b, t, h])[None, :], kk, vv, scale)
                chk.add(to64(out[b, t, h])[None, :], o_ref, lse[b, t, h:h + 1].cpu().numpy(), l_ref)
