"""Seeded synthetic inputs and the workload shapes.

This module holds no arithmetic of the method: it only names shapes and draws
random tensors.  Both the HIP path (through tests and the benchmark) and the
fp64 oracle are fed from here.

Value recipe (the pages describe no input distribution; the workloads stand in
for real model activations):
  * Q, K, V: standard normal draws in float32, rounded to bfloat16 (RNE).
  * index queries / index keys: integers drawn uniformly from [-3, 3], stored as
    bfloat16 (exact).  With d_idx <= 128 every index score is an integer of
    magnitude <= 9 * 128, so fp32 accumulation is exact on any summation order.
Seeds: 1000 * config_id + tensor_id, tensor ids 1 Q, 2 K, 3 V, 4 q_idx, 5 k_idx.
"""

from __future__ import annotations

import dataclasses

import torch

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "q_idx": 4, "k_idx": 5}


@dataclasses.dataclass(frozen=True)
class Shape:
    """One call's sizes.  Query i sits at absolute position pos0 + i."""

    batch: int
    n_q: int
    n_kv: int
    pos0: int
    h_q: int
    h_kv: int
    d: int
    d_idx: int
    block: int = 128
    topk: int = 16

    @property
    def nblk(self) -> int:
        return -(-self.n_kv // self.block)

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# The workloads.  The ids double as the seed base.
WORKLOADS = {
    # 1 sequence, 4096-token causal prefill, MQA (4 query heads on 1 K/V head)
    "tiny_prefill_4k": (1, Shape(1, 4096, 4096, 0, 4, 1, 64, 64)),
    # 1 sequence, 32768-token causal prefill, 64 query heads on 8 K/V heads
    "prefill_32k": (2, Shape(1, 32768, 32768, 0, 64, 8, 128, 128)),
    # 1 sequence, 131072-token causal prefill
    "prefill_128k": (3, Shape(1, 131072, 131072, 0, 64, 8, 128, 128)),
    # 64 single-token decode queries, each against its own 262144-token cache
    "decode_256k_b64": (4, Shape(64, 1, 262144, 262143, 64, 8, 128, 128)),
    # 8192-query prefill chunk at positions 1,040,384 .. 1,048,575 of a 1M cache
    "prefill_chunk_1m": (5, Shape(1, 8192, 1048576, 1040384, 64, 8, 128, 128)),
    # 8 single-token decode queries against 1,048,576-token caches
    "decode_1m_b8": (6, Shape(8, 1, 1048576, 1048575, 64, 8, 128, 128)),
    # a whole 1,048,576-token causal prefill (run in chunks of 8,192 queries)
    "prefill_1m_full": (7, Shape(1, 1048576, 1048576, 0, 64, 8, 128, 128)),
    # selection variants on the 131,072-token prefill's tensors: 32 blocks of
    # 128 (4,096 tokens), and 8 blocks of 256 (the same 2,048-token budget)
    "prefill_128k_k32": (3, Shape(1, 131072, 131072, 0, 64, 8, 128, 128, topk=32)),
    "prefill_128k_b256": (3, Shape(1, 131072, 131072, 0, 64, 8, 128, 128, block=256, topk=8)),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def gaussian_bf16(shape, seed: int, device="cpu") -> torch.Tensor:
    """Standard normal float32 draws rounded to bfloat16."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    return x.to(torch.bfloat16)


def small_int_bf16(shape, seed: int, device="cpu", lo: int = -3, hi: int = 3) -> torch.Tensor:
    """Integers uniform in [lo, hi], stored exactly as bfloat16."""
    g = _gen(seed, device)
    x = torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32, device=device)
    return x.to(torch.bfloat16)


def make_inputs(shape: Shape, config_id: int, device="cpu", which=("q_idx", "k_idx", "q", "k", "v")):
    """Draw the tensors of one call.

    Layouts (row-major, last dim contiguous):
      q_idx [batch][n_q][h_kv][d_idx]   k_idx [batch][n_kv][d_idx]
      q     [batch][n_q][h_q][d]        k, v  [batch][n_kv][h_kv][d]
    """
    s = shape
    out = {}
    base = 1000 * config_id
    if "q_idx" in which:
        out["q_idx"] = small_int_bf16((s.batch, s.n_q, s.h_kv, s.d_idx), base + TENSOR_IDS["q_idx"], device)
    if "k_idx" in which:
        out["k_idx"] = small_int_bf16((s.batch, s.n_kv, s.d_idx), base + TENSOR_IDS["k_idx"], device)
    if "q" in which:
        out["q"] = gaussian_bf16((s.batch, s.n_q, s.h_q, s.d), base + TENSOR_IDS["q"], device)
    if "k" in which:
        out["k"] = gaussian_bf16((s.batch, s.n_kv, s.h_kv, s.d), base + TENSOR_IDS["k"], device)
    if "v" in which:
        out["v"] = gaussian_bf16((s.batch, s.n_kv, s.h_kv, s.d), base + TENSOR_IDS["v"], device)
    return out


def sample_rows(n: int, count: int, seed: int, must=()) -> list:
    """Seeded sample of row indices in [0, n), always holding the first and last
    row and any indices in `must`."""
    g = torch.Generator()
    g.manual_seed(seed)
    picks = set(int(i) for i in must if 0 <= int(i) < n)
    picks.update({0, n - 1})
    if n > len(picks):
        extra = torch.randperm(n, generator=g)[: max(0, count - len(picks))].tolist()
        picks.update(int(i) for i in extra)
    return sorted(picks)[: max(count, len(picks))]
