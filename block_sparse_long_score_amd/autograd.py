"""torch.autograd wrappers around the library's training calls.

Two functions, each a pair of library calls (this module only allocates the
buffers and passes them through; every step runs in the HIP kernels):

  * sparse_attention(s, q, k, v, blk_idx): the main branch over a fixed block
    selection.  Forward: msa_sparse_prefill (output and log-sum-exp kept for
    the backward).  Backward: msa_sparse_prefill_backward -> dq, dk, dv.  The
    selection is discrete and gets no gradient (Notion notes
    "Minimax-sparse-Attention", "Detached Gradients").

  * index_kl(s, q_idx, k_idx, q, k, v, blk_idx, idx_scale): the index branch's
    alignment loss per (sequence, query, group) row: KL(target || softmax over
    the selected blocks' pooled index scores), with the target taken from the
    main branch's attention mass per selected block (same notes, "KL Loss
    Alignment").  Forward: msa_index_scores, then msa_sparse_prefill_target.
    Backward: msa_index_backward -> dq_idx, dk_idx; the main-branch inputs get
    no gradient from this loss (the target is detached).

Gradients come back in the inputs' dtype: bf16 for q, k, v; the index-branch
gradients are computed in fp32 and handed back as bf16 like q_idx and k_idx.
"""

from __future__ import annotations

import torch

from . import msa as M
from .inputs import Shape


class _SparseAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, s: Shape, q, k, v, blk_idx, scale: float):
        out = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((s.batch, s.n_q, s.h_q), dtype=torch.float32, device=q.device)
        ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s, device=q.device)
        M.msa_sparse_prefill(s, q, k, v, blk_idx, out, lse, ws, scale=scale)
        ctx.s, ctx.scale = s, scale
        ctx.save_for_backward(q, k, v, blk_idx, out, lse)
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, blk_idx, out, lse = ctx.saved_tensors
        s = ctx.s
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s, device=q.device)
        M.msa_sparse_prefill_backward(s, q, k, v, blk_idx, out, lse, dout.to(torch.bfloat16).contiguous(), dq, dk, dv,
                                      ws, scale=ctx.scale)
        return None, dq, dk, dv, None, None


def sparse_attention(s: Shape, q, k, v, blk_idx, scale: float = 0.0):
    """Main-branch attention over the selected blocks; differentiable in q, k, v.

    Returns the bf16 output [batch, n_q, h_q, d] (the log-sum-exp is computed
    for the backward and not returned)."""
    out, _ = _SparseAttention.apply(s, q, k, v, blk_idx, scale)
    return out


class _IndexKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, s: Shape, q_idx, k_idx, q, k, v, blk_idx, idx_scale: float, scale: float):
        dev = q_idx.device
        bscore = torch.empty((s.batch, s.n_q, s.h_kv, s.nblk), dtype=torch.float32, device=dev)
        M.msa_index_scores(s, q_idx, k_idx, bscore)
        target = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.float32, device=dev)
        kl = torch.empty((s.batch, s.n_q, s.h_kv), dtype=torch.float32, device=dev)
        out = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device=dev)
        ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s, device=dev)
        M.msa_sparse_prefill_target(s, q, k, v, blk_idx, bscore, target, kl, out, None, ws, idx_scale=idx_scale,
                                    scale=scale)
        ctx.s, ctx.idx_scale = s, idx_scale
        ctx.save_for_backward(q_idx, k_idx, blk_idx, bscore, target)
        return kl

    @staticmethod
    def backward(ctx, dkl):
        q_idx, k_idx, blk_idx, bscore, target = ctx.saved_tensors
        s = ctx.s
        dq_idx = torch.empty((s.batch, s.n_q, s.h_kv, s.d_idx), dtype=torch.float32, device=q_idx.device)
        dk_idx = torch.empty((s.batch, s.n_kv, s.d_idx), dtype=torch.float32, device=q_idx.device)
        ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s, device=q_idx.device)
        M.msa_index_backward(s, q_idx, k_idx, blk_idx, bscore, target, dkl.to(torch.float32).contiguous(), dq_idx,
                             dk_idx, ws, idx_scale=ctx.idx_scale)
        return None, dq_idx.to(q_idx.dtype), dk_idx.to(k_idx.dtype), None, None, None, None, None, None


def index_kl(s: Shape, q_idx, k_idx, q, k, v, blk_idx, idx_scale: float = 1.0, scale: float = 0.0):
    """Per-row KL of the index branch's block distribution from the main
    branch's (detached) block attention mass, [batch, n_q, h_kv] fp32;
    differentiable in q_idx and k_idx."""
    return _IndexKL.apply(s, q_idx, k_idx, q, k, v, blk_idx, idx_scale, scale)
