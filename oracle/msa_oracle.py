"""Plain fp64 CPU oracle for the forward path of MiniMax Sparse Attention (MSA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, calls or links this module; only the tests, the smoke
check and the CPU-baseline leg of the benchmark do.  It shares no code, table or
helper with the GPU path.

What the pages say the method computes, and where (pages are cited by site and
section; they carry no equation numbers):

* GQA base: query heads are split into consecutive groups, each group sharing one
  K/V head (Notion notes "Minimax-sparse-Attention", section "what is MHA, MQA,
  GQA?"; yhxrc.cn article, section "第二步：稀疏分支", where heads Q1-Q3 use I1 and
  Q4-Q6 use I2).  Head h belongs to group h // (Hq / Hkv).
* Index branch (yhxrc.cn article, section "第一步：索引分支"): one index query per
  GQA group and token, one index key per token shared by all heads; the token
  score is the plain dot product q_idx . k_idx over every causal token; the token
  scores are max-pooled per KV block; a top-k keeps the best blocks.
* The selection is per query and per GQA group, independently (hamidun.com news,
  "Como o MSA funciona"; lumi-systems news summary).
* The top-k is exponential-free (lumi-systems news summary): selection works on
  the raw pooled scores, no softmax.
* k = 16 blocks of 128 tokens per query, a fixed 2,048-token budget, and the
  query's own (local) block is always part of the selection (lefilia.fr article).
* Main branch: exact softmax attention on the real, uncompressed K/V of only the
  selected blocks (hamidun.com "Como o MSA funciona"; yhxrc.cn "第二步：稀疏分支";
  lefilia.fr article).

Readings where the pages are silent (each also listed in the design notes):
  r1  index score has no scale, activation or per-head weight;
  r2  k counts the local block: local + (k-1) best earlier blocks;
  r3  ties in the pooled score go to the lower block index;
  r4  when the query has at most k causal blocks, all of them are selected and
      the row is padded with -1;
  r5  selected block indices are written in ascending order;
  r6  causality is per token, s <= p, in both branches;
  r7  softmax scale 1/sqrt(d) unless the caller gives one;
  r8  a decode query sits at p = n_kv - 1 (its own K/V are already cached);
  r9  block j covers tokens [j*B, min((j+1)*B, n_kv)).

Index-branch training target (forward only; Notion notes
"Minimax-sparse-Attention", the "KL Loss Alignment" and "Detached Gradients"
points: the main branch's attention distribution is the target the index branch
is trained to imitate through a KL divergence, with no gradient flowing between
the branches).  Readings:
  r14 the main branch's distribution for one (query, group) lives on its
      selected blocks: each head's softmax weights summed per block, then
      averaged over the group's heads (the index branch has one query per
      group, so one distribution per group);
  r15 the index branch's distribution is a softmax of idx_scale times the
      pooled block scores over the same selected blocks (the pages name no
      temperature, so idx_scale is the caller's);
  r16 the loss is KL(target || index) in nats, with 0 log 0 = 0;
  r17 "detached": the target is returned as a plain value, and every
      gradient below treats it as a constant;
  r18 the index-branch gradient of the KL loss treats the target as a
      constant and the selection as fixed; the block max-pool passes the
      gradient of a pooled score to its argmax token, the lowest position
      among equal maxima.

Main-branch backward: the gradients of the selected-block softmax attention
with respect to q, k and v for a fixed selection (the selection itself is
discrete and carries none), written out from the derivative of softmax
attention.

Array conventions (all numpy, float64 inside):
  q_idx [batch][n_q][Hkv][d_idx]     k_idx [batch][n_kv][d_idx]
  q     [batch][n_q][Hq][d]          k, v  [batch][n_kv][Hkv][d]
  query i of a call sits at absolute position p = pos0 + i.

Every function is pinned by tests/test_oracle_*.py against brute force, closed
forms, invariants and a textbook attention routine.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ----------------------------------------------------------------------------
# Index branch, one (query, group) row at a time
# ----------------------------------------------------------------------------

def token_scores(q_idx_row: np.ndarray, k_idx_seq: np.ndarray, p: int) -> np.ndarray:
    """Index score of one query against every causal token s <= p.

    yhxrc.cn article, "第一步：索引分支": the score is the dot product of the
    group's index query with the index key shared by all heads (reading r1: no
    scale).  Returns float64 [p + 1].
    """
    q = np.asarray(q_idx_row, dtype=np.float64)
    keys = np.asarray(k_idx_seq[: p + 1], dtype=np.float64)
    return keys @ q


def block_max_pool(scores: np.ndarray, p: int, block: int) -> np.ndarray:
    """Max-pool token scores per KV block over the causal tokens.

    yhxrc.cn article, "第一步：索引分支" (block max-pooling turns token scores into
    block scores).  Block j covers tokens [j*block, (j+1)*block) clipped to
    s <= p (reading r6).  Returns float64 [p // block + 1]; the last entry is the
    query's own block, pooled over its causal part only.
    """
    jl = p // block
    pooled = np.empty(jl + 1, dtype=np.float64)
    for j in range(jl + 1):
        lo = j * block
        hi = min((j + 1) * block, p + 1)
        pooled[j] = np.max(scores[lo:hi])
    return pooled


def select_blocks(pooled: np.ndarray, jl: int, topk: int) -> np.ndarray:
    """Exponential-free top-k over the pooled block scores, local block forced.

    lumi-systems summary (exponential-free top-k), lefilia.fr article (k blocks,
    local block always included), yhxrc.cn "第一步" (TopK decides which blocks are
    kept).  Readings r2-r5: the local block jl plus the (topk - 1) best earlier
    blocks j < jl, best meaning larger pooled score, ties to the lower index;
    ascending order; -1 padding when fewer than topk blocks exist.

    The top-(topk-1) is taken by repeated first-occurrence argmax, the plainest
    exact statement of "largest score, lower index on ties".
    """
    out = np.full(topk, -1, dtype=np.int64)
    if jl + 1 <= topk:
        out[: jl + 1] = np.arange(jl + 1)
        return out
    cand = np.array(pooled[:jl], dtype=np.float64)
    chosen = []
    for _ in range(topk - 1):
        j = int(np.argmax(cand))          # first maximal index: ties -> lower j
        chosen.append(j)
        cand[j] = NEG_INF                 # pooled scores are finite, so a chosen
                                          # block never wins a later round
    chosen.append(jl)
    out[:] = np.sort(np.array(chosen, dtype=np.int64))
    return out


def index_topk_row(q_idx_row: np.ndarray, k_idx_seq: np.ndarray, p: int,
                   block: int, topk: int):
    """Whole index branch for one (query, group): scores -> pool -> select.

    Returns (pooled [jl + 1] float64, selection [topk] int64).
    """
    sc = token_scores(q_idx_row, k_idx_seq, p)
    pooled = block_max_pool(sc, p, block)
    sel = select_blocks(pooled, p // block, topk)
    return pooled, sel


# ----------------------------------------------------------------------------
# Main branch, one (query, group) row at a time
# ----------------------------------------------------------------------------

def visible_positions(sel: np.ndarray, p: int, block: int, n_kv: int) -> np.ndarray:
    """Token positions the main branch attends to for one (query, group).

    Every token of every selected block, clipped to s <= p (reading r6) and to
    the cache length (reading r9).  Sorted ascending.
    """
    pos = []
    for j in sel:
        if j < 0:
            continue
        lo = int(j) * block
        hi = min((int(j) + 1) * block, p + 1, n_kv)
        pos.extend(range(lo, hi))
    return np.array(sorted(pos), dtype=np.int64)


def softmax_attention(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray,
                      scale: float):
    """Exact softmax attention of several query heads over the given K/V rows.

    hamidun.com "Como o MSA funciona" and yhxrc.cn "第二步：稀疏分支": the attention
    formula runs unchanged, on real K/V.  q_heads [G][d], keys/values [n][d].
    Returns (out [G][d], lse [G]) in float64, where lse is the natural log of the
    softmax normaliser of the scaled logits.
    """
    q = np.asarray(q_heads, dtype=np.float64)
    kk = np.asarray(keys, dtype=np.float64)
    vv = np.asarray(values, dtype=np.float64)
    z = scale * (q @ kk.T)                     # [G][n]
    m = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - m)
    s = np.sum(e, axis=1, keepdims=True)
    out = (e @ vv) / s
    lse = (m + np.log(s))[:, 0]
    return out, lse


def default_scale(d: int) -> float:
    """Reading r7: the usual 1/sqrt(d) softmax scale."""
    return 1.0 / math.sqrt(d)


# ----------------------------------------------------------------------------
# Whole-tensor drivers (loops over rows; for small and medium shapes)
# ----------------------------------------------------------------------------

def msa_index_topk(q_idx: np.ndarray, k_idx: np.ndarray, pos0: int, block: int,
                   topk: int):
    """Index branch for every (batch, query, group).

    Returns (bscore [b][n_q][Hkv][nblk] float64 with -inf where j > p // block,
             blk_idx [b][n_q][Hkv][topk] int64).
    """
    b, n_q, h_kv, _ = q_idx.shape
    n_kv = k_idx.shape[1]
    nblk = -(-n_kv // block)
    bscore = np.full((b, n_q, h_kv, nblk), NEG_INF, dtype=np.float64)
    blk = np.full((b, n_q, h_kv, topk), -1, dtype=np.int64)
    for bi in range(b):
        kseq = np.asarray(k_idx[bi], dtype=np.float64)
        for i in range(n_q):
            p = pos0 + i
            for g in range(h_kv):
                pooled, sel = index_topk_row(q_idx[bi, i, g], kseq, p, block, topk)
                bscore[bi, i, g, : pooled.shape[0]] = pooled
                blk[bi, i, g] = sel
    return bscore, blk


def msa_sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         blk_idx: np.ndarray, pos0: int, block: int,
                         scale: float | None = None):
    """Main branch: every head of group g attends to the group's selected blocks.

    yhxrc.cn "第二步：稀疏分支" (all heads of a group share one selection) and
    lefilia.fr (exact softmax only on the selected blocks).
    Returns (out [b][n_q][Hq][d], lse [b][n_q][Hq]) in float64.
    """
    b, n_q, h_q, d = q.shape
    n_kv, h_kv = k.shape[1], k.shape[2]
    group = h_q // h_kv
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((b, n_q, h_q, d), dtype=np.float64)
    lse = np.zeros((b, n_q, h_q), dtype=np.float64)
    for bi in range(b):
        for i in range(n_q):
            p = pos0 + i
            for g in range(h_kv):
                pos = visible_positions(blk_idx[bi, i, g], p, block, n_kv)
                hs = slice(g * group, (g + 1) * group)
                o, l = softmax_attention(q[bi, i, hs], k[bi, pos, g], v[bi, pos, g], scale)
                out[bi, i, hs] = o
                lse[bi, i, hs] = l
    return out, lse


def dense_gqa(q: np.ndarray, k: np.ndarray, v: np.ndarray, pos0: int,
              scale: float | None = None):
    """Dense causal GQA, the comparator: every head attends to all s <= p.

    Notion notes, "what is MHA, MQA, GQA?" (grouped K/V heads) and hamidun.com
    "Como o MSA funciona" (the all-to-all baseline MSA is measured against).
    Written separately from msa_sparse_attention on purpose.
    """
    b, n_q, h_q, d = q.shape
    h_kv = k.shape[2]
    group = h_q // h_kv
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((b, n_q, h_q, d), dtype=np.float64)
    lse = np.zeros((b, n_q, h_q), dtype=np.float64)
    for bi in range(b):
        for i in range(n_q):
            p = pos0 + i
            for h in range(h_q):
                g = h // group
                o, l = softmax_attention(q[bi, i, h][None, :], k[bi, : p + 1, g],
                                         v[bi, : p + 1, g], scale)
                out[bi, i, h] = o[0]
                lse[bi, i, h] = l[0]
    return out, lse


def msa_forward(q_idx, k_idx, q, k, v, pos0: int, block: int, topk: int,
                scale: float | None = None):
    """Index branch then main branch, in the pages' order.

    Returns (out, lse, blk_idx, bscore).
    """
    bscore, blk = msa_index_topk(q_idx, k_idx, pos0, block, topk)
    out, lse = msa_sparse_attention(q, k, v, blk, pos0, block, scale)
    return out, lse, blk, bscore


# ----------------------------------------------------------------------------
# Index-branch training target (forward only)
# ----------------------------------------------------------------------------

def block_mass_row(q_heads: np.ndarray, keys_seq: np.ndarray, sel: np.ndarray, p: int,
                   block: int, scale: float) -> np.ndarray:
    """Main-branch attention mass per selected block for one (query, group).

    Notion notes "Minimax-sparse-Attention", "KL Loss Alignment" (the main
    branch's attention distribution is the target), readings r14 and r6.
    q_heads [G][d] are the group's query heads, keys_seq [n_kv][d] the group's
    keys.  For each head the softmax weights over the visible tokens are summed
    per selected block; the result is the mean over heads, one value per slot
    of `sel` (0 for -1 padding).
    """
    n_kv = keys_seq.shape[0]
    pos = visible_positions(sel, p, block, n_kv)
    q = np.asarray(q_heads, dtype=np.float64)
    z = scale * (q @ np.asarray(keys_seq[pos], dtype=np.float64).T)     # [G][n]
    w = np.exp(z - np.max(z, axis=1, keepdims=True))
    w /= np.sum(w, axis=1, keepdims=True)
    owner = pos // block
    mass = np.zeros(len(sel), dtype=np.float64)
    for slot, j in enumerate(sel):
        if j >= 0:
            mass[slot] = np.mean(np.sum(w[:, owner == j], axis=1))
    return mass


def msa_block_target(q: np.ndarray, k: np.ndarray, blk_idx: np.ndarray, pos0: int,
                     block: int, scale: float | None = None) -> np.ndarray:
    """The target distribution for every (batch, query, group).

    Returns float64 [b][n_q][Hkv][topk]; each row sums to 1 over its selected
    blocks and is 0 at padding (readings r14, r17).
    """
    b, n_q, h_q, d = q.shape
    h_kv = k.shape[2]
    group = h_q // h_kv
    if scale is None:
        scale = default_scale(d)
    topk = blk_idx.shape[-1]
    target = np.zeros((b, n_q, h_kv, topk), dtype=np.float64)
    for bi in range(b):
        for i in range(n_q):
            for g in range(h_kv):
                target[bi, i, g] = block_mass_row(q[bi, i, g * group:(g + 1) * group], k[bi, :, g],
                                                  blk_idx[bi, i, g], pos0 + i, block, scale)
    return target


def index_kl_row(target_row: np.ndarray, pooled_row: np.ndarray, sel: np.ndarray,
                 idx_scale: float) -> float:
    """KL(target || index distribution) for one (query, group), in nats.

    Readings r15 and r16: the index distribution is the softmax of
    idx_scale * pooled[j] over the selected blocks j; slots with -1 padding
    take no part; a zero target term contributes nothing.
    """
    live = [slot for slot, j in enumerate(sel) if j >= 0]
    a = np.array([idx_scale * float(pooled_row[sel[slot]]) for slot in live], dtype=np.float64)
    log_q = a - (np.max(a) + np.log(np.sum(np.exp(a - np.max(a)))))
    kl = 0.0
    for n, slot in enumerate(live):
        t = float(target_row[slot])
        if t > 0.0:
            kl += t * (math.log(t) - log_q[n])
    return kl


def msa_index_kl(target: np.ndarray, bscore: np.ndarray, blk_idx: np.ndarray,
                 idx_scale: float) -> np.ndarray:
    """KL(target || index distribution) for every (batch, query, group).

    target [b][n_q][Hkv][topk], bscore [b][n_q][Hkv][nblk] pooled index scores,
    blk_idx [b][n_q][Hkv][topk].  Returns float64 [b][n_q][Hkv].
    """
    b, n_q, h_kv, _ = target.shape
    kl = np.zeros((b, n_q, h_kv), dtype=np.float64)
    for bi in range(b):
        for i in range(n_q):
            for g in range(h_kv):
                kl[bi, i, g] = index_kl_row(target[bi, i, g], bscore[bi, i, g], blk_idx[bi, i, g], idx_scale)
    return kl


# ----------------------------------------------------------------------------
# Main-branch backward (gradients of the selected-block softmax attention)
# ----------------------------------------------------------------------------

def softmax_attention_grad(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray,
                           dout: np.ndarray, scale: float):
    """Gradients of softmax attention of several heads over the given K/V rows.

    The derivative of out = softmax(scale * q k^T) v, written out: with P the
    softmax weights, dv = P^T dout, dP = dout v^T, dS = P * (dP - rowsum(dP * P)),
    dq = scale dS k, dk = scale dS^T q.  q_heads, dout [G][d]; keys, values [n][d].
    Returns (dq [G][d], dk [n][d], dv [n][d]) in float64.
    """
    q = np.asarray(q_heads, dtype=np.float64)
    kk = np.asarray(keys, dtype=np.float64)
    vv = np.asarray(values, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    z = scale * (q @ kk.T)
    w = np.exp(z - np.max(z, axis=1, keepdims=True))
    w /= np.sum(w, axis=1, keepdims=True)
    dv = w.T @ do
    dp = do @ vv.T
    ds = w * (dp - np.sum(dp * w, axis=1, keepdims=True))
    dq = scale * (ds @ kk)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def msa_sparse_attention_grad(q: np.ndarray, k: np.ndarray, v: np.ndarray, blk_idx: np.ndarray,
                              dout: np.ndarray, pos0: int, block: int, scale: float | None = None):
    """Gradients of the main branch for a fixed selection (the selection is
    discrete and carries no gradient; the Notion notes' "Detached Gradients").

    q, dout [b][n_q][Hq][d]; k, v [b][n_kv][Hkv][d]; blk_idx [b][n_q][Hkv][topk].
    Every head of group g attends to the group's selected blocks (yhxrc.cn,
    "第二步：稀疏分支"); keys and values collect the gradients of every query that
    saw them.  Returns (dq, dk, dv) in float64, shaped like q, k, v.
    """
    b, n_q, h_q, d = q.shape
    n_kv, h_kv = k.shape[1], k.shape[2]
    group = h_q // h_kv
    if scale is None:
        scale = default_scale(d)
    dq = np.zeros((b, n_q, h_q, d), dtype=np.float64)
    dk = np.zeros((b, n_kv, h_kv, d), dtype=np.float64)
    dv = np.zeros((b, n_kv, h_kv, d), dtype=np.float64)
    for bi in range(b):
        for i in range(n_q):
            p = pos0 + i
            for g in range(h_kv):
                pos = visible_positions(blk_idx[bi, i, g], p, block, n_kv)
                hs = slice(g * group, (g + 1) * group)
                gq, gk, gv = softmax_attention_grad(q[bi, i, hs], k[bi, pos, g], v[bi, pos, g],
                                                    dout[bi, i, hs], scale)
                dq[bi, i, hs] = gq
                dk[bi, pos, g] += gk
                dv[bi, pos, g] += gv
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Index-branch backward (gradient of the KL loss; target detached)
# ----------------------------------------------------------------------------

def block_argmax(scores: np.ndarray, j: int, p: int, block: int) -> int:
    """Position of the largest causal token score in block j (reading r18:
    the max-pool passes its gradient to one token, the lowest position among
    equal maxima)."""
    lo, hi = j * block, min((j + 1) * block, p + 1)
    return lo + int(np.argmax(scores[lo:hi]))


def index_kl_grad(q_idx: np.ndarray, k_idx: np.ndarray, blk_idx: np.ndarray, target: np.ndarray,
                  idx_scale: float, dkl: np.ndarray, pos0: int, block: int):
    """Gradient of sum_rows dkl[row] * KL(target || index distribution) with
    respect to q_idx and k_idx, for a fixed selection and a detached target
    (Notion notes "Minimax-sparse-Attention": "KL Loss Alignment" trains the
    index branch to imitate the main branch, "Detached Gradients" keeps the
    target out of the gradient).

    For a row with live slots s: a_s = idx_scale * pooled[j_s], index_s =
    softmax(a)_s, dKL/da_s = index_s - target_s; the pooled score is a max over
    the block's causal tokens, so its gradient goes to the argmax token s*:
    dq_idx += idx_scale (index_s - target_s) k_idx[s*], dk_idx[s*] += the same
    coefficient times q_idx (times dkl[row]).  Returns float64 (dq_idx, dk_idx)
    shaped like q_idx and k_idx.
    """
    b, n_q, h_kv, _ = q_idx.shape
    dq = np.zeros(q_idx.shape, dtype=np.float64)
    dk = np.zeros(k_idx.shape, dtype=np.float64)
    for bi in range(b):
        kseq = np.asarray(k_idx[bi], dtype=np.float64)
        for i in range(n_q):
            p = pos0 + i
            for g in range(h_kv):
                qrow = np.asarray(q_idx[bi, i, g], dtype=np.float64)
                sc = token_scores(qrow, kseq, p)
                sel = blk_idx[bi, i, g]
                live = [s for s, j in enumerate(sel) if j >= 0]
                if not live:
                    continue
                pooled = block_max_pool(sc, p, block)
                a = np.array([idx_scale * pooled[sel[s]] for s in live])
                e = np.exp(a - a.max())
                qd = e / e.sum()
                for n, s in enumerate(live):
                    coef = dkl[bi, i, g] * idx_scale * (qd[n] - target[bi, i, g, s])
                    star = block_argmax(sc, int(sel[s]), p, block)
                    dq[bi, i, g] += coef * kseq[star]
                    dk[bi, star] += coef * qrow
    return dq, dk
