"""Planted mistakes in the oracle must be caught by its pins.

Each test swaps one oracle function for a plausible wrong version (a flipped
tie-break, a dropped term, an off-by-one mask, a wrong head->group map, a
missing scale) on the CPU and checks that at least one of the pins in
test_oracle_index.py / test_oracle_attention.py fails.
"""

import math

import numpy as np
import pytest

from oracle import msa_oracle as O
from tests import test_oracle_attention as TA
from tests import test_oracle_index as TI


def fails(fn, *a):
    try:
        fn(*a)
    except AssertionError:
        return True
    return False


def mut_select_high_tie(pooled, jl, topk):
    out = np.full(topk, -1, dtype=np.int64)
    if jl + 1 <= topk:
        out[: jl + 1] = np.arange(jl + 1)
        return out
    cand = np.array(pooled[:jl])
    order = np.lexsort((-np.arange(jl), -cand))     # ties -> HIGHER index
    out[:] = np.sort(list(order[: topk - 1]) + [jl])
    return out


def mut_select_no_local(pooled, jl, topk):
    out = np.full(topk, -1, dtype=np.int64)
    n = min(topk, jl + 1)
    order = np.lexsort((np.arange(jl + 1), -np.asarray(pooled[: jl + 1])))
    out[:n] = np.sort(order[:n])
    return out


def mut_pool_excludes_p(scores, p, block):
    jl = p // block
    pooled = np.empty(jl + 1)
    for j in range(jl + 1):
        lo, hi = j * block, min((j + 1) * block, p + 1)
        seg = scores[lo:hi - 1] if hi - 1 > lo else scores[lo:hi]
        pooled[j] = np.max(seg)
    return pooled


def mut_scores_drop_term(q, k_idx, p):
    return np.asarray(k_idx[: p + 1, :-1], dtype=np.float64) @ np.asarray(q[:-1], dtype=np.float64)


def mut_visible_leaks_future(sel, p, block, n_kv):
    pos = []
    for j in sel:
        if j >= 0:
            pos.extend(range(j * block, min((j + 1) * block, p + 2, n_kv)))
    return np.array(sorted(pos), dtype=np.int64)


def mut_dense_wrong_group(q, k, v, pos0, scale=None):
    b, n_q, h_q, d = q.shape
    h_kv = k.shape[2]
    scale = 1 / math.sqrt(d) if scale is None else scale
    out = np.zeros((b, n_q, h_q, d))
    lse = np.zeros((b, n_q, h_q))
    for bi in range(b):
        for i in range(n_q):
            p = pos0 + i
            for h in range(h_q):
                g = h % h_kv                                # interleaved, wrong
                o, l = O.softmax_attention(q[bi, i, h][None], k[bi, : p + 1, g], v[bi, : p + 1, g], scale)
                out[bi, i, h], lse[bi, i, h] = o[0], l[0]
    return out, lse


def mut_attention_no_scale(q_heads, keys, values, scale):
    return ORIG_SOFTMAX(q_heads, keys, values, 1.0)


ORIG_SOFTMAX = O.softmax_attention


def test_flipped_tie_break_is_caught(monkeypatch):
    monkeypatch.setattr(O, "select_blocks", mut_select_high_tie)
    assert fails(TI.test_selection_all_ties_takes_lowest_indices)
    assert fails(TI.test_selection_matches_full_sort_with_heavy_ties, 16)


def test_missing_local_block_is_caught(monkeypatch):
    monkeypatch.setattr(O, "select_blocks", mut_select_no_local)
    assert fails(TI.test_selection_structure_invariants)


def test_pool_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(O, "block_max_pool", mut_pool_excludes_p)
    assert fails(TI.test_block_max_pool_matches_loop_brute_force)


def test_dropped_score_term_is_caught(monkeypatch):
    monkeypatch.setattr(O, "token_scores", mut_scores_drop_term)
    assert fails(TI.test_token_scores_match_integer_brute_force)


def test_future_leak_is_caught(monkeypatch):
    monkeypatch.setattr(O, "visible_positions", mut_visible_leaks_future)
    assert fails(TA.test_no_future_token_changes_anything) or \
        fails(TA.test_sparse_matches_torch_sdpa_on_selection_mask, 4, 1)
    assert fails(TA.test_block_probe_shows_exactly_the_selected_blocks)


def test_wrong_head_group_map_is_caught(monkeypatch):
    monkeypatch.setattr(O, "dense_gqa", mut_dense_wrong_group)
    assert fails(TA.test_dense_matches_torch_sdpa, 8, 2)


def test_missing_scale_is_caught(monkeypatch):
    monkeypatch.setattr(O, "softmax_attention", mut_attention_no_scale)
    assert fails(TA.test_dense_matches_torch_sdpa, 4, 1)


# ---- index-branch training target ------------------------------------------

from tests import test_oracle_target as TT   # noqa: E402

ORIG_MASS_ROW = O.block_mass_row
ORIG_KL_ROW = O.index_kl_row


def mut_mass_summed_over_heads(q_heads, keys_seq, sel, p, block, scale):
    return ORIG_MASS_ROW(q_heads, keys_seq, sel, p, block, scale) * len(q_heads)


def mut_mass_ignores_causality(q_heads, keys_seq, sel, p, block, scale):
    last = max(int(j) for j in sel)
    return ORIG_MASS_ROW(q_heads, keys_seq, sel, max(p, (last + 1) * block - 1), block, scale)


def mut_mass_first_head_only(q_heads, keys_seq, sel, p, block, scale):
    return ORIG_MASS_ROW(q_heads[:1], keys_seq, sel, p, block, scale)


def mut_kl_reversed(target_row, pooled_row, sel, idx_scale):
    live = [s for s, j in enumerate(sel) if j >= 0]
    a = np.array([idx_scale * pooled_row[sel[s]] for s in live])
    qd = np.exp(a - a.max())
    qd /= qd.sum()
    t = np.array([target_row[s] for s in live])
    return float(np.sum(qd * (np.log(qd) - np.log(np.maximum(t, 1e-300)))))


def mut_kl_softmax_over_all_blocks(target_row, pooled_row, sel, idx_scale):
    live = [s for s, j in enumerate(sel) if j >= 0]
    jl = max(int(sel[s]) for s in live)
    a = idx_scale * np.asarray(pooled_row[: jl + 1], dtype=np.float64)
    log_q = a - (a.max() + np.log(np.sum(np.exp(a - a.max()))))
    return float(sum(target_row[s] * (math.log(target_row[s]) - log_q[sel[s]]) for s in live if target_row[s] > 0))


def test_target_summed_over_heads_is_caught(monkeypatch):
    monkeypatch.setattr(O, "block_mass_row", mut_mass_summed_over_heads)
    assert fails(TT.test_target_rows_are_distributions_on_the_selection, 8, 2, 90, 4)


def test_target_without_causal_mask_is_caught(monkeypatch):
    monkeypatch.setattr(O, "block_mass_row", mut_mass_ignores_causality)
    assert fails(TT.test_zero_query_gives_share_of_visible_tokens)
    assert fails(TT.test_target_matches_sdpa_with_block_indicator_values, 8, 2)


def test_target_from_one_head_is_caught(monkeypatch):
    monkeypatch.setattr(O, "block_mass_row", mut_mass_first_head_only)
    assert fails(TT.test_target_matches_sdpa_with_block_indicator_values, 8, 2)


def test_reversed_kl_is_caught(monkeypatch):
    monkeypatch.setattr(O, "index_kl_row", mut_kl_reversed)
    assert fails(TT.test_kl_matches_scipy_entropy)


def test_index_softmax_over_all_blocks_is_caught(monkeypatch):
    monkeypatch.setattr(O, "index_kl_row", mut_kl_softmax_over_all_blocks)
    assert fails(TT.test_kl_zero_when_index_matches_target_and_shift_invariant)


# ---- main-branch backward ---------------------------------------------------

from tests import test_oracle_backward as TB   # noqa: E402


def _grad_parts(q_heads, keys, values, dout, scale):
    q, kk, vv, do = (np.asarray(a, dtype=np.float64) for a in (q_heads, keys, values, dout))
    z = scale * (q @ kk.T)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return q, kk, vv, do, w, do @ vv.T


def mut_grad_no_rowsum(q_heads, keys, values, dout, scale):
    q, kk, vv, do, w, dp = _grad_parts(q_heads, keys, values, dout, scale)
    ds = w * dp                                             # the rowsum term dropped
    return scale * ds @ kk, scale * ds.T @ q, w.T @ do


def mut_grad_dk_unscaled(q_heads, keys, values, dout, scale):
    q, kk, vv, do, w, dp = _grad_parts(q_heads, keys, values, dout, scale)
    ds = w * (dp - np.sum(dp * w, axis=1, keepdims=True))
    return scale * ds @ kk, ds.T @ q, w.T @ do


def mut_grad_rowsum_of_dp(q_heads, keys, values, dout, scale):
    q, kk, vv, do, w, dp = _grad_parts(q_heads, keys, values, dout, scale)
    ds = w * (dp - np.mean(dp, axis=1, keepdims=True))       # unweighted row mean
    return scale * ds @ kk, scale * ds.T @ q, w.T @ do


def test_backward_without_rowsum_is_caught(monkeypatch):
    monkeypatch.setattr(O, "softmax_attention_grad", mut_grad_no_rowsum)
    assert fails(TB.test_value_and_key_gradient_sums)
    assert fails(TB.test_grads_match_torch_autograd, 8, 2, 1)


def test_backward_unscaled_key_gradient_is_caught(monkeypatch):
    monkeypatch.setattr(O, "softmax_attention_grad", mut_grad_dk_unscaled)
    assert fails(TB.test_grads_match_central_differences)


def test_backward_unweighted_rowsum_is_caught(monkeypatch):
    monkeypatch.setattr(O, "softmax_attention_grad", mut_grad_rowsum_of_dp)
    assert fails(TB.test_grads_match_torch_autograd, 4, 1, 2)


# ---- index-branch backward --------------------------------------------------

from tests import test_oracle_index_grad as TG   # noqa: E402


def mut_argmax_last(scores, j, p, block):
    lo, hi = j * block, min((j + 1) * block, p + 1)
    seg = scores[lo:hi]
    return lo + int(len(seg) - 1 - np.argmax(seg[::-1]))


ORIG_KL_GRAD = O.index_kl_grad


def mut_kl_grad_sign(q_idx, k_idx, blk, target, idx_scale, dkl, pos0, block):
    dq, dk = ORIG_KL_GRAD(q_idx, k_idx, blk, target, idx_scale, dkl, pos0, block)
    return -dq, -dk


def mut_kl_grad_no_scale(q_idx, k_idx, blk, target, idx_scale, dkl, pos0, block):
    dq, dk = ORIG_KL_GRAD(q_idx, k_idx, blk, target, idx_scale, dkl, pos0, block)
    return dq / idx_scale, dk / idx_scale


def test_index_grad_tie_to_last_is_caught(monkeypatch):
    monkeypatch.setattr(O, "block_argmax", mut_argmax_last)
    assert fails(TG.test_tied_maxima_send_the_key_gradient_to_the_lower_position)


def test_index_grad_sign_is_caught(monkeypatch):
    monkeypatch.setattr(O, "index_kl_grad", mut_kl_grad_sign)
    assert fails(TG.test_grad_matches_central_differences, 0.7)


def test_index_grad_missing_scale_is_caught(monkeypatch):
    monkeypatch.setattr(O, "index_kl_grad", mut_kl_grad_no_scale)
    assert fails(TG.test_grad_matches_torch_autograd)
