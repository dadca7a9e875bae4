"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments with the documented
status before touching the GPU (every check here returns before any HIP call).
"""

import ctypes
import os
import re

import pytest

from block_sparse_long_score_amd import msa as M
from block_sparse_long_score_amd.inputs import WORKLOADS, Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:msa_status|size_t|const char\*)\s+(msa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = M.lib()
    names = declared_functions()
    assert set(names) == set(M.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = M.lib()
    for code, name in M.STATUS.items():
        assert lib.msa_status_str(code).decode().startswith(name)


def dims(**kw):
    base = dict(batch=1, n_q=256, n_kv=4096, pos0=3840, h_q=8, h_kv=2, d=128, d_idx=128, block=128, topk=16)
    base.update(kw)
    return M.MsaDims(*[base[f] for f, _ in M.MsaDims._fields_])


FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: every call below fails validation
ODD = ctypes.c_void_p(0x10008)


def index_call(d, q=FAKE, k=FAKE, blk=FAKE, ws=FAKE, wsb=1 << 40):
    return M.lib().msa_index_topk(ctypes.byref(d) if d is not None else None, q, k, blk, ws, wsb, None)


def prefill_call(d, q=FAKE, k=FAKE, v=FAKE, blk=FAKE, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40):
    return M.lib().msa_sparse_prefill(ctypes.byref(d) if d is not None else None, q, k, v, blk,
                                      ctypes.c_float(0.0), out, lse, ws, wsb, None)


def decode_call(d, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, blk=FAKE, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return M.lib().msa_sparse_decode(ctypes.byref(d), a["q"], a["k"], a["v"], a["blk"], ctypes.c_float(0.0),
                                     a["out"], a["lse"], a["ws"], a["wsb"], None)


def dense_call(d, ws=FAKE, wsb=0):
    return M.lib().msa_dense_gqa(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.c_float(0.0), FAKE, None, ws, wsb, None)


def test_null_dims_and_pointers():
    assert index_call(None) == NULL
    assert prefill_call(None) == NULL
    assert index_call(dims(), q=None) == NULL
    assert index_call(dims(), blk=None) == NULL
    assert prefill_call(dims(), v=None) == NULL
    assert prefill_call(dims(), out=None) == NULL
    assert M.lib().msa_block_topk(ctypes.byref(dims()), None, FAKE, None) == NULL


@pytest.mark.parametrize("kw", [
    dict(h_q=6, h_kv=4),            # h_q % h_kv
    dict(pos0=4000),                # pos0 + n_q > n_kv
    dict(n_q=-1),
    dict(batch=-2),
    dict(n_kv=0),
    dict(topk=0),
])
def test_shape_errors(kw):
    assert index_call(dims(**kw)) == SHAPE
    assert prefill_call(dims(**kw)) == SHAPE


def test_decode_needs_single_query():
    assert decode_call(dims(n_q=2, pos0=4094)) == SHAPE


@pytest.mark.parametrize("kw,op", [
    (dict(block=64), "both"),
    (dict(topk=65), "both"),
    (dict(d=96), "attn"),
    (dict(d_idx=32), "index"),
    (dict(h_q=64, h_kv=2), "both"),          # group of 32
    (dict(h_q=24, h_kv=8), "both"),          # group of 3
    (dict(n_kv=(1 << 20) + 128, pos0=(1 << 20) - 128), "both"),
])
def test_unsupported(kw, op):
    if op in ("both", "index"):
        assert index_call(dims(**kw)) == UNSUP
    if op in ("both", "attn"):
        assert prefill_call(dims(**kw)) == UNSUP


def test_alignment_and_workspace():
    assert index_call(dims(), q=ODD) == ALIGN
    assert prefill_call(dims(), lse=ODD) == ALIGN
    assert index_call(dims(), ws=None) == WS
    need = M.lib().msa_workspace_size(M.MSA_OP_INDEX_TOPK, ctypes.byref(dims()))
    assert need >= 256 * 2 * 32 * 4
    assert index_call(dims(), wsb=need - 1) == WS
    # msa_sparse_prefill takes a smaller workspace in query chunks, down to
    # one query of one sequence
    one = M.lib().msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(dims(batch=1, n_q=1)))
    need_p = M.lib().msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(dims()))
    assert 0 < one < need_p
    assert prefill_call(dims(), wsb=one - 1) == WS
    assert prefill_call(dims(), ws=None) == WS
    d1 = dims(n_q=1, pos0=4095)
    assert dense_call(d1, ws=None) == WS
    assert dense_call(d1, wsb=M.lib().msa_workspace_size(M.MSA_OP_DENSE_GQA, ctypes.byref(d1)) - 1) == WS


def test_empty_calls_are_noops():
    assert index_call(dims(n_q=0), q=None, k=None, blk=None, ws=None) == OK
    assert prefill_call(dims(batch=0), q=None, k=None, v=None, blk=None, out=None, ws=None) == OK


def fused_path(s) -> bool:
    """msa_index_topk runs the top-k fused into the scorer for prefill-shaped
    calls with 128-token blocks and k <= 16."""
    return s.block == 128 and s.topk <= 16 and s.n_q * s.h_kv > 16


def test_workspace_sizes_cover_their_buffers():
    for name, (_, s) in WORKLOADS.items():
        n_idx = M.msa_workspace_size(M.MSA_OP_INDEX_TOPK, s)
        if fused_path(s):
            assert n_idx == M.msa_workspace_size(M.MSA_OP_INDEX_TOPK_FUSED, s), name
        else:
            assert n_idx >= s.batch * s.n_q * s.h_kv * s.nblk * 4, name
        if s.n_q == 1:
            assert M.msa_workspace_size(M.MSA_OP_SPARSE_DECODE, s) >= s.batch * s.h_kv * s.topk * s.group * (s.d * 2 + 8)
            assert M.msa_workspace_size(M.MSA_OP_DENSE_GQA, s) > 0
        else:
            n_pre = M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, s)
            assert n_pre >= s.batch * s.n_q * s.h_kv * s.topk * s.group * (s.d * 2 + 8), name
            assert M.msa_workspace_size(M.MSA_OP_DENSE_GQA, s) == 0
    assert M.msa_workspace_size(M.MSA_OP_INDEX_TOPK, Shape(1, 10, 5, 0, 8, 2, 128, 128)) == 0   # rejected dims


def varlen_index_call(d, lens=FAKE, **kw):
    a = dict(q=FAKE, k=FAKE, blk=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return M.lib().msa_index_topk_varlen(ctypes.byref(d), lens, a["q"], a["k"], a["blk"], a["ws"], a["wsb"], None)


def varlen_decode_call(d, lens=FAKE, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, blk=FAKE, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return M.lib().msa_sparse_decode_varlen(ctypes.byref(d), lens, a["q"], a["k"], a["v"], a["blk"],
                                            ctypes.c_float(0.0), a["out"], a["lse"], a["ws"], a["wsb"], None)


def test_varlen_argument_checks():
    d1 = dims(n_q=1, pos0=4095)
    assert varlen_index_call(d1, lens=None) == NULL
    assert varlen_decode_call(d1, lens=None) == NULL
    assert varlen_index_call(d1, blk=None) == NULL
    assert varlen_decode_call(d1, out=None) == NULL
    assert varlen_index_call(dims(n_q=2, pos0=4094)) == SHAPE           # one query per sequence
    assert varlen_decode_call(dims(n_q=2, pos0=4094)) == SHAPE
    assert varlen_index_call(dims(n_q=1, pos0=4095, h_q=64, h_kv=32)) == UNSUP   # > 16 index rows
    assert varlen_index_call(d1, q=ODD) == ALIGN
    assert varlen_decode_call(d1, lse=ODD) == ALIGN
    need = M.lib().msa_workspace_size(M.MSA_OP_INDEX_TOPK, ctypes.byref(d1))
    assert varlen_index_call(d1, wsb=need - 1) == WS
    need_d = M.lib().msa_workspace_size(M.MSA_OP_SPARSE_DECODE, ctypes.byref(d1))
    assert varlen_decode_call(d1, wsb=need_d - 1) == WS
    assert varlen_index_call(dims(n_q=1, pos0=4095, batch=0), lens=None, q=None) == OK   # empty: no-op


def test_chunked_prefill_argument_checks():
    lib = M.lib()
    d = dims()
    call = lambda dd, chunk=64, ws=FAKE, wsb=1 << 40, **kw: lib.msa_prefill_chunked(
        ctypes.byref(dd), chunk, kw.get("qi", FAKE), FAKE, kw.get("q", FAKE), FAKE, FAKE, ctypes.c_float(0.0),
        kw.get("blk", FAKE), FAKE, kw.get("lse", None), ws, wsb, None)
    assert call(d, chunk=0) == SHAPE
    assert call(d, qi=None) == NULL
    assert call(d, blk=None) == NULL
    assert call(d, lse=ODD) == ALIGN
    need = lib.msa_prefill_chunked_workspace_size(ctypes.byref(d), 64)
    assert need > 0 and call(d, wsb=need - 1) == WS
    assert lib.msa_prefill_chunked_workspace_size(ctypes.byref(d), 0) == 0
    # the workspace grows with the chunk, not with the call
    big = dims(n_q=4096, pos0=0)
    assert lib.msa_prefill_chunked_workspace_size(ctypes.byref(big), 64) == need
    assert call(dims(n_q=0), qi=None, q=None, blk=None, ws=None) == OK


def test_chunked_workspace_covers_every_chunk():
    """On the fused index path a chunk's index workspace follows its length
    and position: a full chunk swept by one workgroup per row tile needs none,
    a short tail chunk needs survivor lists.  The chunked workspace must hold
    the largest chunk's index workspace and one full chunk's sparse workspace."""
    lib = M.lib()
    for n_q, chunk, pos0, n_kv in ((65536 + 1000, 65536, 0, 70000), (8192 * 3 + 100, 8192, 5000, 40000),
                                   (3000, 1024, 0, 3000)):
        base = Shape(1, n_q, n_kv, pos0, 64, 8, 128, 128)
        total = M.lib().msa_prefill_chunked_workspace_size(ctypes.byref(M.dims_of(base)), chunk)
        idx_max = 0
        for t0 in range(0, n_q, chunk):
            c = base.replace(n_q=min(chunk, n_q - t0), pos0=pos0 + t0)
            idx_max = max(idx_max, M.msa_workspace_size(M.MSA_OP_INDEX_TOPK, c))
        pre = M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, base.replace(n_q=chunk))
        assert total >= idx_max + pre, (n_q, chunk, total, idx_max, pre)
        first = M.msa_workspace_size(M.MSA_OP_INDEX_TOPK, base.replace(n_q=chunk))
        if n_q == 65536 + 1000:
            assert first == 0 < idx_max, (first, idx_max)     # the tail chunk needs more than the first


def test_target_argument_checks():
    lib = M.lib()
    d = dims()

    def call(dd, idx_scale=1.0, ws=FAKE, wsb=1 << 40, **kw):
        return lib.msa_sparse_prefill_target(
            ctypes.byref(dd), FAKE, FAKE, FAKE, kw.get("blk", FAKE), kw.get("bscore", FAKE),
            ctypes.c_float(idx_scale), ctypes.c_float(0.0), FAKE, kw.get("lse", None), kw.get("target", FAKE),
            kw.get("kl", FAKE), ws, wsb, None)

    assert call(d, bscore=None) == NULL
    assert call(d, target=None) == NULL
    assert call(d, kl=None) == NULL
    assert call(d, kl=ODD) == ALIGN
    assert call(d, bscore=ODD) == ALIGN
    assert call(d, idx_scale=float("nan")) == SHAPE
    assert call(d, idx_scale=float("inf")) == SHAPE
    assert call(dims(h_q=6, h_kv=2)) == UNSUP
    # as msa_sparse_prefill: down to one query's workspace, the call runs in query chunks
    one = lib.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(dims(batch=1, n_q=1)))
    assert call(d, wsb=one - 1) == WS
    assert call(d, ws=None) == WS
    assert call(dims(n_q=0), bscore=None, target=None, kl=None, ws=None) == OK


def test_backward_argument_checks():
    lib = M.lib()
    d = dims()

    def call(dd, ws=FAKE, wsb=1 << 40, **kw):
        p = {n: kw.get(n, FAKE) for n in ("q", "k", "v", "blk", "out", "lse", "dout", "dq", "dk", "dv")}
        return lib.msa_sparse_prefill_backward(ctypes.byref(dd), p["q"], p["k"], p["v"], p["blk"], p["out"],
                                               p["lse"], p["dout"], ctypes.c_float(0.0), p["dq"], p["dk"],
                                               p["dv"], ws, wsb, None)

    for n in ("q", "k", "v", "blk", "out", "lse", "dout", "dq", "dk", "dv"):
        assert call(d, **{n: None}) == NULL, n
        assert call(d, **{n: ODD}) == ALIGN, n
    assert call(dims(h_q=6, h_kv=2)) == UNSUP
    assert call(dims(d=96)) == UNSUP
    # h_q * topk * d must stay below 2^31 (32-bit byte strides of dq partial rows)
    assert call(dims(batch=1, n_q=1, n_kv=128, pos0=0, h_q=262144, h_kv=16384, d=128, d_idx=128, topk=64)) == UNSUP
    assert call(dims(batch=1, n_q=1, n_kv=128, pos0=0, h_q=131072, h_kv=8192, d=128, d_idx=128, topk=64),
                wsb=0) == WS
    need = lib.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(d))
    assert call(d, wsb=need - 1) == WS
    assert call(d, ws=None) == WS
    # no queries: only the key gradients (zeros) are written, query-side pointers may be NULL
    d0 = dims(n_q=0)
    assert call(d0, q=None, blk=None, out=None, lse=None, dout=None, dq=None, wsb=0) == WS
    assert call(d0, dk=None) == NULL
    assert call(dims(batch=0), q=None, k=None, v=None, dk=None, dv=None, ws=None) == OK


def test_index_backward_argument_checks():
    lib = M.lib()
    d = dims()
    names = ("qi", "ki", "blk", "bscore", "target", "dkl", "dqi", "dki")

    def call(dd, idx_scale=1.0, ws=FAKE, wsb=1 << 40, **kw):
        p = {n: kw.get(n, FAKE) for n in names}
        return lib.msa_index_backward(ctypes.byref(dd), p["qi"], p["ki"], p["blk"], p["bscore"], p["target"],
                                      p["dkl"], ctypes.c_float(idx_scale), p["dqi"], p["dki"], ws, wsb, None)

    for n in names:
        assert call(d, **{n: None}) == NULL, n
        assert call(d, **{n: ODD}) == ALIGN, n
    assert call(d, idx_scale=float("nan")) == SHAPE
    assert call(dims(d_idx=96)) == UNSUP
    assert call(dims(h_q=256, h_kv=256)) == UNSUP
    need = lib.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(d))
    assert call(d, wsb=need - 1) == WS
    assert call(dims(batch=0), qi=None, ki=None, dki=None, ws=None) == OK


def test_block256_rules():
    """256-token blocks: the forward calls take them (k <= 32), the target and
    backward calls and msa_index_scores do not."""
    lib = M.lib()
    d = dims(block=256, topk=16)
    d33 = dims(block=256, topk=33)
    assert lib.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(d)) > 0
    assert lib.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(d33)) == 0
    assert prefill_call(d33) == UNSUP
    # index workspace holds the 256-token pooled scores and the 128-token ones
    # (compared with a 128-token call off the fused path: k = 17)
    d128 = dims(block=128, topk=17)
    w256 = lib.msa_workspace_size(M.MSA_OP_INDEX_TOPK, ctypes.byref(d))
    w128 = lib.msa_workspace_size(M.MSA_OP_INDEX_TOPK, ctypes.byref(d128))
    assert w256 >= w128 + w128 // 2
    assert lib.msa_index_scores(ctypes.byref(d), FAKE, FAKE, FAKE, None) == UNSUP
    assert lib.msa_sparse_prefill_target(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0),
                                         ctypes.c_float(0.0), FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None) == UNSUP
    assert lib.msa_sparse_prefill_backward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           ctypes.c_float(0.0), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == UNSUP
    assert lib.msa_index_backward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE,
                                  FAKE, FAKE, 1 << 40, None) == UNSUP


def test_entry_count_bound_counts_128_token_selections():
    """The CSR entries of a call (one per selected 128-token block of a
    (sequence, query, group) row) must fit int32; 256-token blocks select
    twice as many 128-token blocks as k."""
    lib = M.lib()
    big = dict(batch=2, n_q=1 << 20, n_kv=1 << 20, pos0=0, h_q=16, h_kv=16, d=64, d_idx=64)
    ok256 = dims(block=256, topk=31, **big)                 # 2 * 2^20 * 16 * 62 < 2^31
    over256 = dims(block=256, topk=32, **big)               # 2 * 2^20 * 16 * 64 = 2^31
    assert lib.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(ok256)) > 0
    assert lib.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(over256)) == 0
    assert prefill_call(over256) == UNSUP
    over128 = dims(block=128, topk=64, **big)               # the same count on 128-token blocks
    assert lib.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, ctypes.byref(over128)) == 0


def test_noalloc_index_topk_host_checks():
    """The allocation-free index top-k validates like msa_index_topk and
    rejects a call larger than its 64 MiB scratch before any HIP call."""
    call = lambda d, q=FAKE, k=FAKE, blk=FAKE: M.lib().msa_index_topk_noalloc(
        ctypes.byref(d) if d is not None else None, q, k, blk, None)
    assert call(None) == NULL
    assert call(dims(), q=None) == NULL
    assert call(dims(), blk=ODD) == ALIGN
    assert call(dims(h_q=6, h_kv=4)) == SHAPE
    assert call(dims(d_idx=96)) == UNSUP
    assert call(dims(batch=0)) == OK
    # 2 * 2048 * 8 * 1024 fp32 pooled scores = 128 MiB (k = 32: not the fused path)
    assert call(dims(batch=2, n_q=2048, n_kv=131072, pos0=129024, h_q=64, h_kv=8, topk=32)) == 7
    assert M.STATUS[7] == "MSA_ERR_TOO_LARGE"


def test_fused_index_topk_host_checks():
    """The fused index top-k validates like msa_index_topk, serves only
    prefill-shaped calls with 128-token blocks and k <= 16, and sizes its
    survivor lists at 1 to 16 lists of 128 bytes per (token, group) row."""
    lib = M.lib()
    call = lambda d, q=FAKE, k=FAKE, blk=FAKE, ws=FAKE, wsb=1 << 40: lib.msa_index_topk_fused(
        ctypes.byref(d) if d is not None else None, q, k, blk, ws, wsb, None)
    size = lambda d: lib.msa_workspace_size(M.MSA_OP_INDEX_TOPK_FUSED, ctypes.byref(d))
    assert call(None) == NULL
    assert call(dims(), k=None) == NULL
    assert call(dims(), blk=ODD) == ALIGN
    assert call(dims(), ws=ODD) == ALIGN
    assert call(dims(), ws=None) == WS
    assert call(dims(), wsb=size(dims()) - 1) == WS
    assert call(dims(pos0=4000)) == SHAPE
    assert call(dims(d_idx=96)) == UNSUP
    for kw in (dict(topk=17), dict(block=256, topk=8), dict(n_q=2, pos0=4094, h_q=8, h_kv=8),
               dict(n_q=1, pos0=4095)):
        assert call(dims(**kw)) == UNSUP, kw
        assert size(dims(**kw)) == 0, kw
    assert call(dims(n_q=0), q=None, k=None, blk=None, ws=None) == OK
    assert size(dims(n_q=3, pos0=4093, h_kv=8, h_q=8)) > 0                  # 24 rows: prefill-shaped
    for name in ("prefill_32k", "prefill_chunk_1m", "tiny_prefill_4k"):
        s = WORKLOADS[name][1]
        rows = s.batch * s.n_q * s.h_kv
        n = M.msa_workspace_size(M.MSA_OP_INDEX_TOPK_FUSED, s)
        assert 2 * rows * 128 <= n <= 16 * rows * 128 + 512, (name, n)
    # one workgroup per row tile (512 tile pairs at 131,072 tokens x 8 groups,
    # 4,096 for the whole 1M-token sequence): the selection is written directly
    for name in ("prefill_128k", "prefill_1m_full"):
        assert M.msa_workspace_size(M.MSA_OP_INDEX_TOPK_FUSED, WORKLOADS[name][1]) == 0, name
    d0 = dims(batch=64, n_q=4096, n_kv=4096, pos0=0, h_q=64, h_kv=8)
    assert size(d0) == 0 and lib.msa_workspace_size(M.MSA_OP_INDEX_TOPK, ctypes.byref(d0)) == 0
