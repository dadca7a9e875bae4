#!/usr/bin/env python3
"""Benchmark of the MSA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the hot path over one batch of synthetic input:
index scoring, block max-pool and exponential-free top-k (msa_index_topk, which
for this shape runs the top-k fused into the scoring kernel) and block-sparse
prefill attention (msa_sparse_prefill) on the 131,072-token prefill workload
(64 query heads on 8 K/V heads, d = d_idx = 128, 128-token blocks, k = 16).  Inputs are resident in HBM before the timed region.
`value` is prefill tokens per second.  The same JSON line also carries:
  * per-stage times measured with HIP events on the stream the library runs on,
  * `roofline` for the dominant kernel (algorithmic flops or bytes per launch
    over its measured average duration),
  * the decode leg (1M-token caches, batch 8: index top-k + sparse decode),
  * the library's own dense causal GQA on the same inputs (speedup),
  * the top-k kernel against torch.topk on the same candidates, and the top-k
    alone on 1,048,576 full rows of 1,023 candidates against torch.topk and
    torch.sort on the same rows,
  * the index branch as two separate calls on the prefill inputs (the scoring
    kernel writes the pooled scores, msa_block_topk reads them), each timed,
  * the other configurations: 32K prefill and the 8,192-query prefill chunk at
    1M (each with the dense comparison), decode of 64 sequences at 256K,
  * `cpu_baseline`: the fp64 oracle timed on a bounded sample of the workload,
    with the host's CPU count and model.
All progress goes to stderr; stdout gets exactly one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "MSA prefill tok/s & decode tok/s at 128K–1M ctx; % MFMA / HBM roofline"
PEAK_BF16_FLOPS = 2.5e15        # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--decode-workload", default="decode_1m_b8")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the decode step replayed as a HIP graph")
    ap.add_argument("--no-varlen", action="store_true", help="skip the variable-length decode leg")
    ap.add_argument("--no-prefill-1m", action="store_true",
                    help="skip the whole 1M-token chunked prefill leg")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-topk-compare", action="store_true")
    ap.add_argument("--no-small-workspace", action="store_true",
                    help="skip the sparse prefill with an eighth of its workspace (query chunks)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations' legs (32K prefill, the 1M prefill chunk, 256K x 64 decode)")
    ap.add_argument("--no-topk-full", action="store_true",
                    help="skip the top-k alone on full 1,024-candidate rows against torch.topk and torch.sort")
    ap.add_argument("--no-target", action="store_true", help="skip the index-branch target (KL) leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the main-branch and index-branch backward legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the measured bf16 GEMM and device-copy reference rates")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


# ------------------------------------------------------------------ counts --

def causal_positions(s):
    import numpy as np
    return s.pos0 + np.arange(s.n_q, dtype=np.int64)


def index_flops(s) -> float:
    """S1: h_kv * d_idx * 2 flops per (query, causal token), all sequences."""
    p = causal_positions(s)
    return float(s.batch * s.h_kv * s.d_idx * 2 * (p + 1).sum())


def visible_counts(s):
    """|V_t|: causal tokens of the local block plus (k-1) full earlier blocks,
    or every causal token when the query has at most k blocks."""
    import numpy as np
    p = causal_positions(s)
    jl = p // s.block
    local = p - jl * s.block + 1
    full = np.minimum(jl, s.topk - 1) * s.block
    return local + full


def sparse_flops(s) -> float:
    """S4: QK^T and PV, 4 * d flops per (query head, visible key)."""
    return float(s.batch * s.h_q * s.d * 4 * visible_counts(s).sum())


def dense_flops(s) -> float:
    p = causal_positions(s)
    return float(s.batch * s.h_q * s.d * 4 * (p + 1).sum())


def topk_bytes(s) -> float:
    """S3: read every candidate pooled score (j < jl) once, write the indices."""
    p = causal_positions(s)
    cand = (p // s.block).sum()
    return float(s.batch * s.h_kv * (cand * 4 + s.n_q * s.topk * 4))


def target_bytes(s) -> float:
    """Index-branch target: per (query, group) row, each live slot's partial
    (m, l) for the G heads and its pooled index score; the row's selection read
    and target written, and its KL."""
    import numpy as np
    p = causal_positions(s)
    live = np.minimum(p // s.block + 1, s.topk).sum()
    rows = s.n_q
    return float(s.batch * s.h_kv * (live * (s.group * 8 + 4) + rows * (s.topk * 8 + 4)))


def decode_bytes(s) -> float:
    """Decode step: index keys of every cached token, the selected K/V, the
    queries, pooled scores written and read, indices, outputs."""
    vis = float(visible_counts(s).sum())
    nblk = s.nblk
    b = s.batch
    kidx = b * s.n_kv * s.d_idx * 2
    kv = b * vis * s.h_kv * s.d * 2 * 2
    small = b * (s.h_kv * s.d_idx * 2 + s.h_q * s.d * 2 * 2 + s.h_kv * nblk * 4 * 2 + s.h_kv * s.topk * 4 * 2)
    return float(kidx + kv + small)


# ----------------------------------------------------------- HBM traffic --

TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")


def measured_traffic(kernel, workload):
    """HBM bytes per launch (read + written) from the committed counter
    summary, or None when there is none for this kernel and workload or the
    kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    from block_sparse_long_score_amd.profiling import kernel_sources_sha256
    e = rec.get(kernel, {}).get(workload)
    if not e or e.get("sources_sha256") != kernel_sources_sha256(kernel):
        return None
    return float(e["read_bytes"] + e["write_bytes"])


# ------------------------------------------------------------------ timing --

LAST_STEPS = []   # per-step times (ms) of the latest time_calls


def step_stats():
    v = sorted(LAST_STEPS)
    n = len(v)
    med = (v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])) if n else None
    return {"median": med, "min": v[0] if n else None}


def measured_references(torch):
    """What this chip sustains on two plain library operations, as context for
    the published peaks: the best of two large bf16 GEMMs (torch.matmul) and a
    device copy of 4 GiB (bytes read + written per second)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, work, reps):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return work * reps / (e0.elapsed_time(e1) * 1e-3)

    gemm, shape = 0.0, None
    for n in (8192, 16384):
        a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
        b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
        r = rate(lambda: torch.matmul(a, b), 2.0 * n ** 3, 10)
        if r > gemm:
            gemm, shape = r, [n, n, n]
        del a, b
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    copy = rate(lambda: dst.copy_(src), 2.0 * src.numel(), 10)
    del src, dst
    torch.cuda.empty_cache()
    return {"bf16_gemm_tflops": gemm / 1e12, "bf16_gemm_shape": shape, "d2d_copy_gbs": copy / 1e9,
            "d2d_copy_bytes": 2 * (4 << 30), "source": "torch.matmul and Tensor.copy_"}


def time_calls(torch, fns, steps, warmup, M=None):
    """Run the list of zero-argument launches `fns` as one step; returns the
    mean per-step wall time (events around the whole timed region) and the mean
    time of each launch (events between launches) in milliseconds.  With the
    binding module M, the library's own per-kernel timing (HIP event pairs
    around each kernel on its stream) runs over the timed region and the
    per-kernel totals are returned as a third value."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    if M is not None:
        M.msa_profile_begin()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        ev[i][0].record()
        for j, f in enumerate(fns):
            f()
            ev[i][j + 1].record()
    end.record()
    torch.cuda.synchronize()
    kernels = M.msa_profile_end() if M is not None else None
    LAST_STEPS[:] = [ev[i][0].elapsed_time(ev[i][len(fns)]) for i in range(steps)]
    total = start.elapsed_time(end) / steps
    per = [sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps for j in range(len(fns))]
    if M is not None:
        return total, per, kernels
    return total, per


# ------------------------------------------------------------ CPU baseline --

def host_cpu():
    """The host the oracle runs on: logical CPU count and CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "cpu_model": model}


def cpu_baseline(s, inp, seconds, seed=99):
    """The fp64 oracle, as it stands, on a seeded sample of query rows of the
    same workload: all groups' index scoring, pooling and selection, then all
    heads' sparse attention, per sampled row."""
    import numpy as np
    from oracle import msa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(x.get("num_threads", 1)) for x in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    log("cpu baseline: copying inputs to host")
    q_idx = inp["q_idx"][0].float().cpu().numpy().astype(np.float64)
    kseq = inp["k_idx"][0].float().cpu().numpy().astype(np.float64)
    q = inp["q"][0].float().cpu().numpy().astype(np.float64)
    k = inp["k"][0].float().cpu().numpy().astype(np.float64)
    v = inp["v"][0].float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    order = rng.permutation(s.n_q)
    scale = O.default_scale(s.d)
    G = s.group
    done = 0
    t0 = time.perf_counter()
    for t in order:
        p = s.pos0 + int(t)
        for g in range(s.h_kv):
            _, sel = O.index_topk_row(q_idx[t, g], kseq, p, s.block, s.topk)
            pos = O.visible_positions(sel, p, s.block, s.n_kv)
            O.softmax_attention(q[t, g * G:(g + 1) * G], k[pos, g], v[pos, g], scale)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "host": host_cpu(),
            "sample": f"{done} query rows drawn uniformly (seed {seed}) from the {s.n_q}-token prefill, "
                      f"all {s.h_kv} groups and {s.h_q} heads each, {el:.1f} s on the host"}


# ------------------------------------------------------ other configurations --

def prefill_config_leg(torch, M, name, steps, warmup, dense_reps=2):
    """One step of the prefill hot path (msa_index_topk, then
    msa_sparse_prefill) on another configuration's inputs, with the library's
    dense GQA on the same inputs."""
    from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs
    cid, s = WORKLOADS[name]
    log(f"prefill leg {name}: {s}")
    inp = make_inputs(s, cid, device="cuda")
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((s.batch, s.n_q, s.h_q), dtype=torch.float32, device="cuda")
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    ws_i = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
    stages = [
        lambda: M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], blk, ws_i),
        lambda: M.msa_sparse_prefill(s, inp["q"], inp["k"], inp["v"], blk, out, lse, ws),
    ]
    ms, (mi, msp) = time_calls(torch, stages, steps, warmup)
    st = step_stats()
    fi, fsp = index_flops(s), sparse_flops(s)
    tokens = s.batch * s.n_q
    leg = {"workload": name, "n_q": s.n_q, "n_kv": s.n_kv, "pos0": s.pos0, "steps": steps,
           "ms_per_step": ms, "ms_per_step_median": st["median"], "ms_per_step_min": st["min"],
           "tok_s": tokens / (ms * 1e-3), "algorithmic_flops": fi + fsp,
           "end_to_end_mfma_frac": (fi + fsp) / (ms * 1e-3) / PEAK_BF16_FLOPS,
           "stages_ms": {"index_topk": mi, "sparse_prefill": msp},
           "index_topk_mfma_frac": fi / (mi * 1e-3) / PEAK_BF16_FLOPS,
           "sparse_prefill_mfma_frac": fsp / (msp * 1e-3) / PEAK_BF16_FLOPS}
    log(f"{name}: step {ms:.3f} ms (index top-k {mi:.3f}, sparse {msp:.3f}) -> "
        f"{leg['tok_s']:.4g} tok/s, {leg['end_to_end_mfma_frac']:.1%} of MFMA peak")
    if dense_reps:
        ms_d, _ = time_calls(torch, [lambda: M.msa_dense_gqa(s, inp["q"], inp["k"], inp["v"], out, lse)],
                             dense_reps, 1)
        fd = dense_flops(s)
        leg["dense_gqa"] = {"ms": ms_d, "mfma_frac": fd / (ms_d * 1e-3) / PEAK_BF16_FLOPS,
                            "msa_speedup": ms_d / ms}
        log(f"{name}: dense GQA {ms_d:.2f} ms ({leg['dense_gqa']['mfma_frac']:.1%} of MFMA peak) -> "
            f"MSA {ms_d / ms:.2f}x faster")
    del inp, blk, out, lse, ws, ws_i
    torch.cuda.empty_cache()
    return leg


def decode_config_leg(torch, M, name, steps, warmup, dense_reps=3):
    """One decode step (index top-k + sparse decode) on another
    configuration's inputs, with the library's dense decode beside it."""
    from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs
    cid, s = WORKLOADS[name]
    log(f"decode leg {name}: {s}")
    inp = make_inputs(s, cid, device="cuda")
    ws_i = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
    ws_s = M.alloc_workspace(M.MSA_OP_SPARSE_DECODE, s)
    blk = torch.empty((s.batch, 1, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((s.batch, 1, s.h_q, s.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((s.batch, 1, s.h_q), dtype=torch.float32, device="cuda")
    calls = [
        lambda: M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], blk, ws_i),
        lambda: M.msa_sparse_decode(s, inp["q"], inp["k"], inp["v"], blk, out, lse, ws_s),
    ]
    ms, (mi, msd) = time_calls(torch, calls, steps, warmup)
    st = step_stats()
    _, _, kern = time_calls(torch, calls, steps, 1, M)
    by = decode_bytes(s)
    leg = {"workload": name, "batch": s.batch, "n_kv": s.n_kv, "steps": steps,
           "ms_per_step": ms, "ms_per_step_median": st["median"], "ms_per_step_min": st["min"],
           "tok_s": s.batch / (ms * 1e-3), "algorithmic_bytes": by,
           "hbm_gbs": by / (ms * 1e-3) / 1e9, "hbm_frac": by / (ms * 1e-3) / PEAK_HBM_BYTES,
           "index_topk_ms": mi, "sparse_decode_ms": msd,
           "kernels": {n: {"launches": c, "avg_ms": t / c} for n, (c, t) in kern.items()}}
    log(f"{name}: step {ms:.3f} ms -> {leg['tok_s']:.4g} tok/s, {leg['hbm_frac']:.1%} of HBM peak")
    if dense_reps:
        dws = M.alloc_workspace(M.MSA_OP_DENSE_GQA, s)
        ms_d, _ = time_calls(torch, [lambda: M.msa_dense_gqa(s, inp["q"], inp["k"], inp["v"], out, lse, dws)],
                             dense_reps, 1)
        kv = float(s.batch * s.n_kv * s.h_kv * s.d * 2 * 2)
        leg["dense_gqa"] = {"ms": ms_d, "kv_bytes": kv, "hbm_frac": kv / (ms_d * 1e-3) / PEAK_HBM_BYTES,
                            "msa_speedup": ms_d / ms}
        log(f"{name}: dense decode {ms_d:.3f} ms -> MSA {ms_d / ms:.2f}x faster")
        del dws
    del inp, ws_i, ws_s, blk, out, lse
    torch.cuda.empty_cache()
    return leg


# The top-k alone on full rows: 1,048,576 (query, group) rows whose local block
# is 1023, so each row has 1,023 candidate blocks (blocks 0..1022) in a
# 1,024-wide row: 1,024 sequences x 128 queries at positions 130,944..131,071
# x 8 groups.  Pooled scores are integers drawn uniformly from [80, 170] (the
# central range of the 128K workload's pooled scores: 1st-99th percentile
# 81-170), so ties are as frequent as in real rows.
TOPK_FULL_SHAPE = dict(batch=1024, n_q=128, n_kv=131072, pos0=130944, h_q=64, h_kv=8, d=128, d_idx=128)
TOPK_FULL_SEED = 3099


def topk_full_scores(torch, s, device="cuda"):
    """The full-row top-k leg's pooled scores; column 1023 (every row's local
    block, never a candidate) is -inf so a library top-k over the whole row
    makes the same choice as msa_block_topk over its 1,023 candidates."""
    g = torch.Generator(device=device)
    g.manual_seed(TOPK_FULL_SEED)
    sc = torch.randint(80, 171, (s.batch, s.n_q, s.h_kv, s.nblk), generator=g, dtype=torch.float32, device=device)
    sc[..., s.nblk - 1] = -math.inf
    return sc


def topk_full_leg(torch, M, steps):
    from block_sparse_long_score_amd.inputs import Shape
    s = Shape(**TOPK_FULL_SHAPE)
    log(f"top-k alone on full rows: {s}")
    sc = topk_full_scores(torch, s)
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device="cuda")
    ms_msa, _ = time_calls(torch, [lambda: M.msa_block_topk(s, sc, blk)], steps, 1)
    ms_topk, _ = time_calls(torch, [lambda: torch.topk(sc, s.topk - 1, dim=-1)], 3, 1)
    ms_sort, _ = time_calls(torch, [lambda: torch.sort(sc, dim=-1, descending=True, stable=True)], 3, 1)
    by = topk_bytes(s)
    rows = s.batch * s.n_q * s.h_kv
    leg = {"rows": rows, "candidates_per_row": s.nblk - 1, "row_entries": s.nblk, "algorithmic_bytes": by,
           "msa_block_topk_ms": ms_msa, "hbm_gbs": by / (ms_msa * 1e-3) / 1e9,
           "hbm_frac": by / (ms_msa * 1e-3) / PEAK_HBM_BYTES,
           "torch_topk_ms": ms_topk, "torch_sort_stable_ms": ms_sort,
           "speedup_vs_torch_topk": ms_topk / ms_msa, "speedup_vs_torch_sort": ms_sort / ms_msa,
           "note": "same 1,024-wide rows for all three (the local-block column is -inf); torch.topk takes k-1 "
                   "per row, torch.sort (stable, descending) orders whole rows; timing only"}
    log(f"top-k full rows: msa {ms_msa:.3f} ms ({leg['hbm_frac']:.1%} of HBM peak), torch.topk {ms_topk:.3f} ms, "
        f"torch.sort {ms_sort:.3f} ms")
    del sc, blk
    torch.cuda.empty_cache()
    return leg


# -------------------------------------------------------------------- main --

def decode_graph_leg(torch, dec, dec_calls, dsteps, warmup, batch, by):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in dec_calls:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for f in dec_calls:
            f()
    ms_g, _ = time_calls(torch, [graph.replay], dsteps, warmup)
    dec["graph_ms_per_step"] = ms_g
    dec["graph_tok_s"] = batch / (ms_g * 1e-3)
    dec["graph_hbm_frac"] = by / (ms_g * 1e-3) / PEAK_HBM_BYTES
    log(f"decode step as a HIP graph {ms_g:.3f} ms -> {dec['graph_tok_s']:.4g} tok/s, "
        f"{dec['graph_hbm_frac'] * 100:.1f}% of HBM peak")
    del graph


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by K/V-head group or by sequence with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_long_score_amd import msa as M
    from block_sparse_long_score_amd.inputs import WORKLOADS, make_inputs

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return

    M.lib()                                            # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = "cuda"
    cid, s = WORKLOADS[args.workload]
    log(f"workload {args.workload}: {s}")
    inp = make_inputs(s, cid, device=dev)
    bscore = torch.empty((s.batch, s.n_q, s.h_kv, s.nblk), dtype=torch.float32, device=dev)
    blk = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.int32, device=dev)
    out = torch.empty((s.batch, s.n_q, s.h_q, s.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((s.batch, s.n_q, s.h_q), dtype=torch.float32, device=dev)
    ws = M.alloc_workspace(M.MSA_OP_SPARSE_PREFILL, s)
    torch.cuda.synchronize()

    # The hot path as a caller runs it: msa_index_topk (for prefill-shaped calls
    # with 128-token blocks and k <= 16 it runs the top-k fused into the
    # scoring kernel, without pooled scores in memory; otherwise scores,
    # pooling and top-k as separate kernels), then msa_sparse_prefill.
    ws_idx = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, s)
    stages = [
        lambda: M.msa_index_topk(s, inp["q_idx"], inp["k_idx"], blk, ws_idx),
        lambda: M.msa_sparse_prefill(s, inp["q"], inp["k"], inp["v"], blk, out, lse, ws),
    ]
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    ms_step, (ms_it, ms_sparse), kern = time_calls(torch, stages, args.steps, args.warmup, M)
    prefill_steps = step_stats()
    tokens = s.batch * s.n_q
    value = tokens / (ms_step * 1e-3)
    f_idx, f_sp = index_flops(s), sparse_flops(s)
    log(f"step {ms_step:.3f} ms: index top-k {ms_it:.3f}, sparse {ms_sparse:.3f} -> {value:.4g} tok/s")

    per_stage = {
        "index_topk": {"ms": ms_it, "bound": "mfma", "achieved": f_idx / (ms_it * 1e-3) / 1e12,
                       "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s"},
        "sparse_prefill": {"ms": ms_sparse, "bound": "mfma", "achieved": f_sp / (ms_sparse * 1e-3) / 1e12,
                           "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s"},
    }
    for v in per_stage.values():
        v["frac"] = v["achieved"] / v["peak"]
    # Per-kernel device times from the library's event pairs over the timed
    # region; the roofline is reported for the kernel with the largest total.
    kernels = {name: {"launches": n, "avg_ms": tot / n, "ms_per_step": tot / args.steps}
               for name, (n, tot) in kern.items()}
    algorithmic = {   # kernel -> (bound, algorithmic work of one launch, peak, unit scale, unit)
        "index_scores_tiled": ("mfma", f_idx, PEAK_BF16_FLOPS, 1e12, "TFLOP/s"),
        "index_topk_tiled": ("mfma", f_idx, PEAK_BF16_FLOPS, 1e12, "TFLOP/s"),
        "sparse_kv_outer": ("mfma", f_sp, PEAK_BF16_FLOPS, 1e12, "TFLOP/s"),
        "block_topk_rows": ("hbm", topk_bytes(s), PEAK_HBM_BYTES, 1e9, "GB/s"),
        "block_topk_wg": ("hbm", topk_bytes(s), PEAK_HBM_BYTES, 1e9, "GB/s"),
    }
    dom_name = max(kern, key=lambda n: kern[n][1])
    if dom_name not in algorithmic:
        raise RuntimeError(f"no algorithmic work defined for the dominant kernel {dom_name}")
    bound, work, peak, scale, unit = algorithmic[dom_name]
    avg = kernels[dom_name]["avg_ms"]
    achieved = work / (avg * 1e-3)
    traffic = measured_traffic(dom_name, args.workload)
    roofline = {"kernel": dom_name, "bound": bound, "achieved": achieved / scale, "peak": peak / scale,
                "unit": unit, "frac": achieved / peak,
                "traffic": traffic,
                "algorithmic_per_launch": work, "avg_launch_ms": avg}
    if traffic is not None:
        # The same launch priced by the HBM bytes it moves (from the committed counters).
        roofline["traffic_gbs"] = traffic / (avg * 1e-3) / 1e9
        roofline["traffic_frac_of_hbm_peak"] = traffic / (avg * 1e-3) / PEAK_HBM_BYTES
    log(f"dominant kernel {dom_name}: {avg:.3f} ms per launch, {achieved / scale:.1f} {unit} "
        f"({achieved / peak:.1%} of peak)" + (f"; moves {traffic / 1e9:.1f} GB of HBM traffic = "
                                              f"{roofline['traffic_frac_of_hbm_peak']:.1%} of HBM peak"
                                              if traffic is not None else ""))

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": s.batch, "n_q": s.n_q, "n_kv": s.n_kv, "pos0": s.pos0,
                   "h_q": s.h_q, "h_kv": s.h_kv, "d": s.d, "d_idx": s.d_idx, "block": s.block, "topk": s.topk},
        "roofline": roofline,
        "stages": per_stage,
        "kernels": kernels,
        "end_to_end_mfma_frac": (f_idx + f_sp) / (ms_step * 1e-3) / PEAK_BF16_FLOPS,
        "ms_per_step_median": prefill_steps["median"],
        "ms_per_step_min": prefill_steps["min"],
    }

    if s.block == 128:
        # The index branch as two separate calls on the same inputs: the
        # scoring kernel writes the pooled scores (the workspace msa_index_topk
        # needs off the fused path), then the top-k reads them.
        ublk = torch.empty_like(blk)
        ms_u, (ms_idx, ms_topk), ku = time_calls(torch, [
            lambda: M.msa_index_scores(s, inp["q_idx"], inp["k_idx"], bscore),
            lambda: M.msa_block_topk(s, bscore, ublk)], 3, 1, M)
        same = bool(torch.equal(ublk, blk))
        result["index_unfused"] = {
            "ms": ms_u, "index_scores_ms": ms_idx, "block_topk_ms": ms_topk,
            "index_scores_mfma_frac": f_idx / (ms_idx * 1e-3) / PEAK_BF16_FLOPS,
            "block_topk_hbm_frac": topk_bytes(s) / (ms_topk * 1e-3) / PEAK_HBM_BYTES,
            "kernels": {name: {"launches": n, "avg_ms": tot / n} for name, (n, tot) in ku.items()},
            "pooled_score_bytes": int(bscore.numel() * 4),
            "index_topk_workspace_bytes": int(M.msa_workspace_size(M.MSA_OP_INDEX_TOPK, s)),
            "same_selection_as_index_topk": same}
        log(f"index branch as separate calls: scores {ms_idx:.3f} ms + top-k {ms_topk:.3f} ms = {ms_u:.3f} ms "
            f"(msa_index_topk {ms_it:.3f} ms), same selection: {same}")
        del ublk

    if s.n_q > 1 and not args.no_small_workspace:
        # msa_sparse_prefill with an eighth of its one-pass workspace: the call
        # takes the queries in chunks whose workspace fits.
        small = max(M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, s.replace(batch=1, n_q=1)),
                    M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, s) // 8)
        ws_small = torch.empty(small, dtype=torch.uint8, device=dev)
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        ms_small, _ = time_calls(torch, [
            lambda: M.msa_sparse_prefill(s, inp["q"], inp["k"], inp["v"], blk, out2, lse2, ws_small)], 3, 1)
        same = bool(torch.equal(out2.view(torch.int16), out.view(torch.int16)) and
                    torch.equal(lse2.view(torch.int32), lse.view(torch.int32)))
        result["sparse_prefill_small_workspace"] = {
            "workspace_bytes": int(small), "one_pass_workspace_bytes": int(M.msa_workspace_size(M.MSA_OP_SPARSE_PREFILL, s)),
            "ms": ms_small, "one_pass_ms": ms_sparse, "same_outputs": same}
        log(f"sparse prefill with {small / 2**30:.2f} GiB of workspace: {ms_small:.3f} ms "
            f"(one pass {ms_sparse:.3f} ms), same outputs: {same}")
        del ws_small, out2, lse2

    if not args.no_topk_compare and s.block == 128:
        # torch.topk on the same candidates: entries at and past each row's
        # local block are set to -inf in a copy, so the library top-k makes
        # the same choice; torch.topk still reads every row entry (4 GiB at
        # 128K) where msa_block_topk reads only the candidates (2 GiB).
        vals = bscore.clone()
        jl = (s.pos0 + torch.arange(s.n_q, device=dev)) // s.block
        col = torch.arange(s.nblk, device=dev)
        vals.masked_fill_((col[None, :] >= jl[:, None])[None, :, None, :], -math.inf)
        ms_torch, _ = time_calls(torch, [lambda: torch.topk(vals, s.topk - 1, dim=-1)], 3, 1)
        del vals
        result["topk_vs_torch"] = {"msa_block_topk_ms": ms_topk, "torch_topk_ms": ms_torch,
                                   "speedup": ms_torch / ms_topk,
                                   "msa_bytes": topk_bytes(s), "torch_bytes": float(bscore.numel() * 4),
                                   "note": "same candidates (torch's copy has -inf at and past each row's local "
                                           "block); torch.topk reads whole rows, msa only the candidates; the "
                                           "equal-work comparison is the topk_full_rows leg"}
        log(f"top-k: msa {ms_topk:.3f} ms vs torch.topk {ms_torch:.3f} ms")

    if not args.no_target and s.block == 128:
        # Index-branch training target (forward only): msa_sparse_prefill plus
        # block_target_kl on the same inputs (its pooled scores are the ones
        # the separate-calls leg above wrote); block_target_kl's own time from
        # the library's event pairs.
        target = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.float32, device=dev)
        kl = torch.empty((s.batch, s.n_q, s.h_kv), dtype=torch.float32, device=dev)
        idx_scale = 1.0 / math.sqrt(s.d_idx)
        ms_t, _, kt = time_calls(torch, [lambda: M.msa_sparse_prefill_target(
            s, inp["q"], inp["k"], inp["v"], blk, bscore, target, kl, out, lse, ws, idx_scale=idx_scale)], 3, 1, M)
        n, tot = kt["block_target_kl"]
        ms_k = tot / n
        tb = target_bytes(s)
        result["index_target"] = {"ms_call": ms_t, "block_target_kl_ms": ms_k, "algorithmic_bytes": tb,
                                  "hbm_gbs": tb / (ms_k * 1e-3) / 1e9, "hbm_frac": tb / (ms_k * 1e-3) / PEAK_HBM_BYTES,
                                  "extra_over_sparse_prefill_ms": ms_t - ms_sparse}
        log(f"index target: call {ms_t:.3f} ms, block_target_kl {ms_k:.3f} ms "
            f"({tb / (ms_k * 1e-3) / PEAK_HBM_BYTES:.1%} of HBM peak)")
        del target, kl

    if not args.no_backward and s.block == 128:
        # Main-branch backward on the same selection: dq, dk, dv from a seeded
        # output gradient; algorithmic work 10 d flops per (query head, visible
        # key) (S, dP, dV, dK, dQ), i.e. 2.5x the forward's S4 count.
        g = torch.Generator().manual_seed(7)
        dout_b = torch.randn((s.batch, s.n_q, s.h_q, s.d), generator=g).to(torch.bfloat16).to(dev)
        dq_b = torch.empty_like(dout_b)
        dk_b = torch.empty_like(inp["k"])
        dv_b = torch.empty_like(inp["v"])
        M.msa_sparse_prefill(s, inp["q"], inp["k"], inp["v"], blk, out, lse, ws)
        ms_b, _, kb = time_calls(torch, [lambda: M.msa_sparse_prefill_backward(
            s, inp["q"], inp["k"], inp["v"], blk, out, lse, dout_b, dq_b, dk_b, dv_b, ws)], 3, 1, M)
        fb = 2.5 * f_sp
        n, tot = kb["sparse_bwd_kv"]
        ms_kv = tot / n
        result["backward"] = {"ms": ms_b, "tok_s": tokens / (ms_b * 1e-3), "algorithmic_flops": fb,
                              "mfma_frac": fb / (ms_b * 1e-3) / PEAK_BF16_FLOPS,
                              "sparse_bwd_kv_ms": ms_kv,
                              "sparse_bwd_kv_mfma_frac": fb / (ms_kv * 1e-3) / PEAK_BF16_FLOPS,
                              "kernels": {name: {"launches": c, "avg_ms": t / c} for name, (c, t) in kb.items()}}
        log(f"backward {ms_b:.2f} ms (sparse_bwd_kv {ms_kv:.2f} ms, "
            f"{fb / (ms_kv * 1e-3) / PEAK_BF16_FLOPS:.1%} of MFMA peak)")
        del dout_b, dq_b, dk_b, dv_b
        # Index-branch backward (gradient of the KL alignment loss) on the
        # same selection, with the target of msa_sparse_prefill_target.
        target = torch.empty((s.batch, s.n_q, s.h_kv, s.topk), dtype=torch.float32, device=dev)
        kl = torch.empty((s.batch, s.n_q, s.h_kv), dtype=torch.float32, device=dev)
        idx_scale = 1.0 / math.sqrt(s.d_idx)
        M.msa_sparse_prefill_target(s, inp["q"], inp["k"], inp["v"], blk, bscore, target, kl, out, lse, ws,
                                    idx_scale=idx_scale)
        dkl = torch.ones_like(kl)
        dqi = torch.empty((s.batch, s.n_q, s.h_kv, s.d_idx), dtype=torch.float32, device=dev)
        dki = torch.empty((s.batch, s.n_kv, s.d_idx), dtype=torch.float32, device=dev)
        ms_i, _, ki = time_calls(torch, [lambda: M.msa_index_backward(
            s, inp["q_idx"], inp["k_idx"], blk, bscore, target, dkl, dqi, dki, ws, idx_scale=idx_scale)], 3, 1, M)
        result["index_backward"] = {"ms": ms_i, "kernels": {name: {"launches": c, "avg_ms": t / c}
                                                            for name, (c, t) in ki.items()}}
        log(f"index backward {ms_i:.2f} ms")
        del target, kl, dkl, dqi, dki

    if not args.no_dense:
        dout = torch.empty_like(out)
        dlse = torch.empty_like(lse)
        ms_dense, _ = time_calls(torch, [lambda: M.msa_dense_gqa(s, inp["q"], inp["k"], inp["v"], dout, dlse)], 2, 1)
        fd = dense_flops(s)
        result["dense_gqa"] = {"ms": ms_dense, "tok_s": tokens / (ms_dense * 1e-3),
                               "mfma_frac": fd / (ms_dense * 1e-3) / PEAK_BF16_FLOPS,
                               "msa_speedup": ms_dense / ms_step}
        log(f"dense GQA {ms_dense:.2f} ms -> MSA speedup {ms_dense / ms_step:.2f}x")
        del dout, dlse

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(s, inp, args.cpu_seconds)
        log(f"cpu baseline: {cpu}")
    result["cpu_baseline"] = cpu

    del ws, out, lse, bscore, blk, inp
    torch.cuda.empty_cache()

    ref = None
    if not args.no_reference:
        ref = measured_references(torch)
        rl = result["roofline"]
        rl["frac_of_measured"] = (rl["achieved"] / ref["bf16_gemm_tflops"] if rl["unit"] == "TFLOP/s"
                                  else rl["achieved"] / ref["d2d_copy_gbs"])
        result["reference"] = ref
        log(f"measured references: bf16 GEMM {ref['bf16_gemm_tflops']:.0f} TFLOP/s, "
            f"device copy {ref['d2d_copy_gbs']:.0f} GB/s; "
            f"dominant kernel at {rl['frac_of_measured']:.1%} of the measured rate for its bound")

    if not args.no_decode:
        did, ds = WORKLOADS[args.decode_workload]
        log(f"decode workload {args.decode_workload}: {ds}")
        dinp = make_inputs(ds, did, device=dev)
        dws_i = M.alloc_workspace(M.MSA_OP_INDEX_TOPK, ds)
        dws_s = M.alloc_workspace(M.MSA_OP_SPARSE_DECODE, ds)
        dblk = torch.empty((ds.batch, 1, ds.h_kv, ds.topk), dtype=torch.int32, device=dev)
        dout = torch.empty((ds.batch, 1, ds.h_q, ds.d), dtype=torch.bfloat16, device=dev)
        dlse = torch.empty((ds.batch, 1, ds.h_q), dtype=torch.float32, device=dev)
        dsteps = max(args.steps, 20)
        dec_calls = [
            lambda: M.msa_index_topk(ds, dinp["q_idx"], dinp["k_idx"], dblk, dws_i),
            lambda: M.msa_sparse_decode(ds, dinp["q"], dinp["k"], dinp["v"], dblk, dout, dlse, dws_s),
        ]
        ms_dec, (ms_di, ms_ds) = time_calls(torch, dec_calls, dsteps, args.warmup)
        dec_steps = step_stats()
        # Per-kernel times from a second pass: event records would weigh on
        # these sub-millisecond steps, so they stay out of the timed one.
        _, _, dkern = time_calls(torch, dec_calls, dsteps, 1, M)
        by = decode_bytes(ds)
        kidx_bytes = float(ds.batch * ds.n_kv * ds.d_idx * 2)
        dec = {"workload": args.decode_workload, "batch": ds.batch, "n_kv": ds.n_kv, "steps": dsteps,
               "ms_per_step": ms_dec, "tok_s": ds.batch / (ms_dec * 1e-3),
               "index_topk_ms": ms_di, "sparse_decode_ms": ms_ds,
               "algorithmic_bytes": by, "hbm_gbs": by / (ms_dec * 1e-3) / 1e9,
               "hbm_frac": by / (ms_dec * 1e-3) / PEAK_HBM_BYTES,
               "kernels": {name: {"launches": n, "avg_ms": tot / n, "ms_per_step": tot / dsteps}
                           for name, (n, tot) in dkern.items()},
               "ms_per_step_median": dec_steps["median"], "ms_per_step_min": dec_steps["min"]}
        if ref:
            dec["hbm_gbs_over_measured_copy"] = dec["hbm_gbs"] / ref["d2d_copy_gbs"]
        if "index_scores_skinny" in dkern:
            n, tot = dkern["index_scores_skinny"]
            dec["index_scores_skinny_hbm_frac"] = kidx_bytes / (tot / n * 1e-3) / PEAK_HBM_BYTES
        log(f"decode step {ms_dec:.3f} ms ({ms_di:.3f} index top-k + {ms_ds:.3f} sparse) -> "
            f"{dec['tok_s']:.4g} tok/s, {dec['hbm_frac'] * 100:.1f}% of HBM peak")
        # The same step captured once in a HIP graph and replayed: a serving
        # loop's form, without launch gaps between its kernels.
        if not args.no_graph:
            decode_graph_leg(torch, dec, dec_calls, dsteps, args.warmup, ds.batch, by)
        if not args.no_dense:
            ddws = M.alloc_workspace(M.MSA_OP_DENSE_GQA, ds)
            ms_dd, _ = time_calls(torch, [lambda: M.msa_dense_gqa(ds, dinp["q"], dinp["k"], dinp["v"], dout, dlse,
                                                                ddws)], 3, 1)
            dec["dense_gqa_ms"] = ms_dd
            dec["msa_speedup"] = ms_dd / ms_dec
            log(f"dense decode {ms_dd:.3f} ms -> MSA decode speedup {ms_dd / ms_dec:.2f}x")
        result["decode"] = dec

    if not args.no_decode and not args.no_varlen:
        # Variable-length decode on the same caches: each sequence holds its
        # own number of tokens of the 1M capacity.
        lens = [ds.n_kv, 786432, 524288, 262144, 100000, 10000, 1000, 100][: ds.batch]
        lens += [ds.n_kv] * (ds.batch - len(lens))
        lens_t = torch.tensor(lens, dtype=torch.int32, device=dev)
        vl_calls = [
            lambda: M.msa_index_topk_varlen(ds, lens_t, dinp["q_idx"], dinp["k_idx"], dblk, dws_i),
            lambda: M.msa_sparse_decode_varlen(ds, lens_t, dinp["q"], dinp["k"], dinp["v"], dblk, dout, dlse, dws_s),
        ]
        ms_vl, _ = time_calls(torch, vl_calls, dsteps, args.warmup)
        by_vl = sum(decode_bytes(ds.replace(batch=1, n_kv=n, pos0=n - 1)) for n in lens)
        result["decode_varlen"] = {"workload": f"{args.decode_workload} caches, per-sequence lengths", "lengths": lens,
                                   "ms_per_step": ms_vl, "tok_s": ds.batch / (ms_vl * 1e-3),
                                   "algorithmic_bytes": by_vl, "hbm_gbs": by_vl / (ms_vl * 1e-3) / 1e9,
                                   "hbm_frac": by_vl / (ms_vl * 1e-3) / PEAK_HBM_BYTES}
        log(f"varlen decode {ms_vl:.3f} ms over lengths {lens} -> "
            f"{result['decode_varlen']['hbm_frac'] * 100:.1f}% of HBM peak")

    if not args.no_decode:
        del dinp, dws_i, dws_s, dblk, dout, dlse
        torch.cuda.empty_cache()

    if not args.no_configs:
        result["configs"] = {
            "prefill_32k": prefill_config_leg(torch, M, "prefill_32k", args.steps, args.warmup),
            "prefill_chunk_1m": prefill_config_leg(torch, M, "prefill_chunk_1m", args.steps, args.warmup),
            "decode_256k_b64": decode_config_leg(torch, M, "decode_256k_b64", max(args.steps, 20), args.warmup),
        }

    if not args.no_topk_full:
        result["topk_full_rows"] = topk_full_leg(torch, M, max(args.steps, 5))

    if not args.no_prefill_1m:
        # A whole 1M-token prefill, chunk by chunk (index branch + sparse
        # attention per 8,192 queries over the growing causal range).
        fid, fs = WORKLOADS["prefill_1m_full"]
        chunk = 8192
        log(f"1M prefill workload prefill_1m_full: {fs}, chunks of {chunk}")
        finp = make_inputs(fs, fid, device=dev)
        fblk = torch.empty((fs.batch, fs.n_q, fs.h_kv, fs.topk), dtype=torch.int32, device=dev)
        fout = torch.empty((fs.batch, fs.n_q, fs.h_q, fs.d), dtype=torch.bfloat16, device=dev)
        fws = torch.empty(M.msa_prefill_chunked_workspace_size(fs, chunk), dtype=torch.uint8, device=dev)
        ms_1m, _ = time_calls(torch, [lambda: M.msa_prefill_chunked(fs, chunk, finp["q_idx"], finp["k_idx"], finp["q"],
                                                                    finp["k"], finp["v"], fblk, fout, None, fws)],
                              2, 1)
        f1 = index_flops(fs) + sparse_flops(fs)
        result["prefill_1m_chunked"] = {
            "workload": "prefill_1m_full", "chunk": chunk, "ms": ms_1m, "tok_s": fs.n_q / (ms_1m * 1e-3),
            "mfma_frac": f1 / (ms_1m * 1e-3) / PEAK_BF16_FLOPS, "algorithmic_flops": f1,
            "workspace_bytes": int(fws.numel())}
        log(f"1M prefill in chunks of {chunk}: {ms_1m:.1f} ms -> {fs.n_q / (ms_1m * 1e-3):.4g} tok/s, "
            f"{result['prefill_1m_chunked']['mfma_frac'] * 100:.1f}% of MFMA peak")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
