// C ABI of the MSA forward path: argument validation on the host, workspace
// sizing, and the kernel launch sequence of each entry point.  Declared and
// documented in include/msa.h.
#include "msa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "launch.h"

namespace {

using msa::Dims;

enum : unsigned {
  kNeedD = 1u,      // attention head dimension is used
  kNeedDIdx = 2u,   // index dimension is used
  kDecode = 4u,     // n_q must be 1
  kCsr = 8u,        // per-(b, g, block) lists must fit int32
  kOnly128 = 16u,   // the op works on 128-token blocks only
};

constexpr int64_t kMaxKv = 1 << 20;

msa_status check_dims(const msa_dims* p, unsigned need) {
  if (!p) return MSA_ERR_NULL;
  const msa_dims& d = *p;
  if (d.batch < 0 || d.n_q < 0 || d.n_kv < 1 || d.pos0 < 0 || d.h_q < 1 || d.h_kv < 1 || d.block < 1 ||
      d.topk < 1 || d.d < 1 || d.d_idx < 1)
    return MSA_ERR_SHAPE;
  if (d.h_q % d.h_kv != 0) return MSA_ERR_SHAPE;
  if ((int64_t)d.pos0 + d.n_q > d.n_kv) return MSA_ERR_SHAPE;
  if ((need & kDecode) && d.n_q != 1) return MSA_ERR_SHAPE;
  if (d.block != 128 && d.block != 256) return MSA_ERR_UNSUPPORTED;
  if ((need & kOnly128) && d.block != 128) return MSA_ERR_UNSUPPORTED;
  if (d.topk > 64 || (d.block == 256 && d.topk > 32)) return MSA_ERR_UNSUPPORTED;
  const int g = d.h_q / d.h_kv;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return MSA_ERR_UNSUPPORTED;
  if ((need & kNeedD) && d.d != 64 && d.d != 128) return MSA_ERR_UNSUPPORTED;
  if ((need & kNeedDIdx) && d.d_idx != 64 && d.d_idx != 128) return MSA_ERR_UNSUPPORTED;
  if (d.n_kv > kMaxKv) return MSA_ERR_UNSUPPORTED;
  if (d.batch > 65535) return MSA_ERR_UNSUPPORTED;
  // CSR entries (one per selected 128-token block of a row: twice k for 256-token blocks) are int32 indices.
  const int64_t k128 = d.block == 256 ? 2 * (int64_t)d.topk : d.topk;
  if ((int64_t)d.batch * d.n_q * d.h_kv * k128 >= (int64_t(1) << 31)) return MSA_ERR_UNSUPPORTED;
  if ((int64_t)d.n_q * d.h_kv > (int64_t(1) << 25)) return MSA_ERR_UNSUPPORTED;
  const int64_t nblk = (d.n_kv + 127) / 128;           // the lists are per 128-token block
  if ((need & kCsr) && (int64_t)d.batch * d.h_kv * nblk >= (int64_t(1) << 31)) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

Dims to_dims(const msa_dims& d) {
  return Dims{d.batch, d.n_q, d.n_kv, d.pos0, d.h_q, d.h_kv, d.d, d.d_idx, d.block, d.topk};
}

bool empty(const msa_dims& d) { return d.batch == 0 || d.n_q == 0; }

size_t nrows(const Dims& d) { return (size_t)d.batch * d.n_q * d.h_kv; }

// 256-token blocks run on the 128-token kernels: index scores per 128-token
// block, pooled in pairs; a selection of 256-token blocks expanded into twice
// as many 128-token blocks for the main branch.
Dims index128(const Dims& d) {
  Dims c = d;
  c.block = 128;
  return c;
}
Dims blocks128(const Dims& d) {
  Dims c = index128(d);
  if (d.block == 256) c.topk = 2 * d.topk;
  return c;
}

// Prefill-shaped calls with 128-token blocks and k <= 16 take the fused
// path (survivor lists, or nothing with one workgroup per row tile); the
// others keep the pooled scores at offset 0, for 256-token blocks followed by
// the 128-token pooled scores they come from.
size_t index_ws_bytes(const Dims& d) {
  if (msa::index_topk_fused_applies(d)) return msa::index_topk_fused_ws_bytes(d);
  const size_t own = msa::align_up(nrows(d) * d.nblk() * sizeof(float), 256);
  if (d.block == 128) return own;
  return own + msa::align_up(nrows(d) * index128(d).nblk() * sizeof(float), 256);
}
// The expanded selection of a 256-token-block call, then the main branch's own.
size_t sel_bytes(const Dims& d) {
  return d.block == 128 ? 0 : msa::align_up(nrows(d) * 2 * d.topk * sizeof(int32_t), 256);
}
size_t prefill_ws_bytes(const Dims& d) { return sel_bytes(d) + msa::prefill_ws_layout(blocks128(d)).total; }
// The largest number of queries of one sequence whose sparse-prefill
// workspace fits in `bytes` (0 if not even one query's does).
int prefill_chunk_fitting(const Dims& d, size_t bytes) {
  Dims c = d;
  c.batch = 1;
  auto fits = [&](int n) { c.n_q = n; return prefill_ws_bytes(c) <= bytes; };
  if (!fits(1)) return 0;
  int lo = 1, hi = std::max(d.n_q, 1);                  // fits(lo) holds
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (fits(mid)) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
// Calls fn(c, row, kv_off) for each query chunk of at most cq queries of each
// sequence of d: c is the chunk's dims (one sequence, its queries at
// pos0 + t0 ..), row its first (sequence, query) row, kv_off the element
// offset of its sequence's K/V.  Stops at the first error.
template <class F>
msa_status for_query_chunks(const Dims& d, int cq, F fn) {
  for (int b = 0; b < d.batch; ++b) {
    for (int t0 = 0; t0 < d.n_q; t0 += cq) {
      Dims c = d;
      c.batch = 1;
      c.n_q = std::min(cq, d.n_q - t0);
      c.pos0 = d.pos0 + t0;
      const msa_status st = fn(c, (int64_t)b * d.n_q + t0, (int64_t)b * d.n_kv * d.h_kv * d.d);
      if (st != MSA_OK) return st;
    }
  }
  return MSA_OK;
}
size_t decode_ws_bytes(const Dims& d) { return sel_bytes(d) + msa::sparse_decode_ws_layout(blocks128(d)).total; }

hipError_t run_index_topk(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, int32_t* blk, void* ws,
                          hipStream_t s) {
  if (msa::index_topk_fused_applies(d)) return msa::launch_index_topk_fused(d, q_idx, k_idx, blk, ws, s);
  float* bscore = static_cast<float*>(ws);
  hipError_t e;
  if (d.block == 128) {
    e = msa::launch_index_scores(d, q_idx, k_idx, bscore, s);
  } else {
    float* p128 = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                           msa::align_up(nrows(d) * d.nblk() * sizeof(float), 256));
    e = msa::launch_index_scores(index128(d), q_idx, k_idx, p128, s);
    if (e == hipSuccess) e = msa::launch_pool_block_pairs(d, p128, bscore, s);
  }
  if (e != hipSuccess) return e;
  return msa::launch_block_topk(d, bscore, blk, s);
}

hipError_t run_sparse(const Dims& d, bool decode, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* blk, float scale, uint16_t* out, float* lse, void* ws, hipStream_t s) {
  const Dims c = blocks128(d);
  const int32_t* b = blk;
  void* rest = ws;
  if (d.block != 128) {
    int32_t* b128 = static_cast<int32_t*>(ws);
    const hipError_t e = msa::launch_expand_block_pairs(d, blk, b128, s);
    if (e != hipSuccess) return e;
    b = b128;
    rest = static_cast<char*>(ws) + sel_bytes(d);
  }
  return decode ? msa::launch_sparse_decode(c, q, k, v, b, scale, out, lse, rest, s)
                : msa::launch_sparse_prefill(c, q, k, v, b, scale, out, lse, rest, s);
}

unsigned op_needs(msa_op op) {
  switch (op) {
    case MSA_OP_INDEX_TOPK: return kNeedDIdx;
    case MSA_OP_BLOCK_TOPK: return 0u;
    case MSA_OP_SPARSE_PREFILL: return kNeedD | kCsr;
    case MSA_OP_SPARSE_DECODE: return kNeedD | kDecode;
    case MSA_OP_DENSE_GQA: return kNeedD;
    case MSA_OP_INDEX_TOPK_FUSED: return kNeedDIdx | kOnly128;
  }
  return 0u;
}

msa_status hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

float resolve_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / sqrtf((float)d); }

// Workspace of msa_prefill_chunked: the index workspace of the most
// demanding chunk (its size follows each chunk's length and position on the
// fused path) and the sparse-prefill workspace of a full chunk (one
// sequence, `chunk` queries).
size_t chunked_ws_bytes(const Dims& d, int chunk, size_t* prefill_off) {
  Dims c = d;
  c.batch = 1;
  size_t idx = 0;
  for (int t0 = 0; t0 < std::max(d.n_q, 1); t0 += chunk) {
    c.n_q = std::min(chunk, std::max(d.n_q, 1) - t0);
    c.pos0 = d.pos0 + t0;
    idx = std::max(idx, index_ws_bytes(c));
  }
  idx = msa::align_up(idx, 256);
  c.n_q = chunk;
  c.pos0 = d.pos0;
  if (prefill_off) *prefill_off = idx;
  return idx + prefill_ws_bytes(c);
}

}  // namespace

extern "C" {

size_t msa_workspace_size(msa_op op, const msa_dims* dims) {
  if (op < MSA_OP_INDEX_TOPK || op > MSA_OP_INDEX_TOPK_FUSED) return 0;
  if (check_dims(dims, op_needs(op)) != MSA_OK) return 0;
  const Dims d = to_dims(*dims);
  switch (op) {
    case MSA_OP_INDEX_TOPK: return index_ws_bytes(d);
    case MSA_OP_BLOCK_TOPK: return 0;
    case MSA_OP_SPARSE_PREFILL: return prefill_ws_bytes(d);
    case MSA_OP_SPARSE_DECODE: return decode_ws_bytes(d);
    case MSA_OP_DENSE_GQA: return d.n_q == 1 ? msa::dense_decode_ws_layout(index128(d)).total : 0;
    case MSA_OP_INDEX_TOPK_FUSED: return msa::index_topk_fused_applies(d) ? msa::index_topk_fused_ws_bytes(d) : 0;
  }
  return 0;
}

const char* msa_status_str(msa_status s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_NULL: return "MSA_ERR_NULL: a required pointer is NULL";
    case MSA_ERR_SHAPE: return "MSA_ERR_SHAPE: inconsistent sizes";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: sizes outside what this build implements";
    case MSA_ERR_ALIGN: return "MSA_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE: workspace missing or too small";
    case MSA_ERR_HIP: return "MSA_ERR_HIP: a kernel launch failed";
    case MSA_ERR_TOO_LARGE: return "MSA_ERR_TOO_LARGE: the call needs more than the library's static scratch";
  }
  return "unknown msa_status";
}

msa_status msa_index_topk(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx, int32_t* blk_idx,
                          void* workspace, size_t workspace_bytes, msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_INDEX_TOPK));
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if (!q_idx || !k_idx || !blk_idx) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(blk_idx)) return MSA_ERR_ALIGN;
  const Dims d = to_dims(*dims);
  const size_t need = index_ws_bytes(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MSA_ERR_WORKSPACE;
  if (workspace && misaligned(workspace)) return MSA_ERR_ALIGN;
  return hip_status(run_index_topk(d, q_idx, k_idx, blk_idx, workspace, static_cast<hipStream_t>(stream)));
}

msa_status msa_index_topk_noalloc(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx,
                                  int32_t* blk_idx, msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_INDEX_TOPK));
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if (!q_idx || !k_idx || !blk_idx) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(blk_idx)) return MSA_ERR_ALIGN;
  const Dims d = to_dims(*dims);
  if (index_ws_bytes(d) > msa::kScratchBytes) return MSA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (msa::scratch_for_current_device(&ws) != hipSuccess) return MSA_ERR_HIP;
  return hip_status(run_index_topk(d, q_idx, k_idx, blk_idx, ws, static_cast<hipStream_t>(stream)));
}

msa_status msa_index_topk_fused(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx,
                                int32_t* blk_idx, void* workspace, size_t workspace_bytes, msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_INDEX_TOPK_FUSED));
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  const Dims d = to_dims(*dims);
  if (!msa::index_topk_fused_applies(d)) return MSA_ERR_UNSUPPORTED;
  if (!q_idx || !k_idx || !blk_idx) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(blk_idx)) return MSA_ERR_ALIGN;
  const size_t need = msa::index_topk_fused_ws_bytes(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MSA_ERR_WORKSPACE;
  if (workspace && misaligned(workspace)) return MSA_ERR_ALIGN;
  return hip_status(msa::launch_index_topk_fused(d, q_idx, k_idx, blk_idx, workspace,
                                                 static_cast<hipStream_t>(stream)));
}

msa_status msa_index_scores(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx, float* bscore,
                            msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_INDEX_TOPK) | kOnly128);
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if (!q_idx || !k_idx || !bscore) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(bscore)) return MSA_ERR_ALIGN;
  return hip_status(msa::launch_index_scores(to_dims(*dims), q_idx, k_idx, bscore, static_cast<hipStream_t>(stream)));
}

msa_status msa_block_topk(const msa_dims* dims, const float* bscore, int32_t* blk_idx, msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_BLOCK_TOPK));
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if (!bscore || !blk_idx) return MSA_ERR_NULL;
  if (misaligned(bscore) || misaligned(blk_idx)) return MSA_ERR_ALIGN;
  return hip_status(msa::launch_block_topk(to_dims(*dims), bscore, blk_idx, static_cast<hipStream_t>(stream)));
}

msa_status msa_sparse_prefill(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* blk_idx, float scale, uint16_t* out, float* lse, void* workspace,
                              size_t workspace_bytes, msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_SPARSE_PREFILL));
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if (!q || !k || !v || !blk_idx || !out) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(blk_idx) || misaligned(out) ||
      (lse && misaligned(lse)))
    return MSA_ERR_ALIGN;
  const Dims d = to_dims(*dims);
  if (!workspace) return MSA_ERR_WORKSPACE;
  const float sc = resolve_scale(scale, d.d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (workspace_bytes >= prefill_ws_bytes(d)) {
    if (misaligned(workspace)) return MSA_ERR_ALIGN;
    return hip_status(run_sparse(d, false, q, k, v, blk_idx, sc, out, lse, workspace, s));
  }
  // A smaller workspace: each sequence's queries in the largest chunks whose
  // workspace fits (every query's output depends only on its own selection,
  // so the chunks are independent; each re-stages the blocks it selects).
  const int cq = prefill_chunk_fitting(d, workspace_bytes);
  if (cq < 1) return MSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return MSA_ERR_ALIGN;
  return for_query_chunks(d, cq, [&](const Dims& c, int64_t row, int64_t kv_off) {
    return hip_status(run_sparse(c, false, q + row * d.h_q * d.d, k + kv_off, v + kv_off,
                                 blk_idx + row * d.h_kv * d.topk, sc, out + row * d.h_q * d.d,
                                 lse ? lse + row * d.h_q : nullptr, workspace, s));
  });
}

msa_status msa_sparse_prefill_target(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const int32_t* blk_idx, const float* bscore, float idx_scale, float scale,
                                     uint16_t* out, float* lse, float* target, float* kl, void* workspace,
                                     size_t workspace_bytes, msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_SPARSE_PREFILL) | kOnly128);
  if (st != MSA_OK) return st;
  if (!std::isfinite(idx_scale)) return MSA_ERR_SHAPE;
  if (empty(*dims)) return MSA_OK;
  if (!q || !k || !v || !blk_idx || !bscore || !out || !target || !kl) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(blk_idx) || misaligned(bscore) ||
      misaligned(out) || misaligned(target) || misaligned(kl) || (lse && misaligned(lse)))
    return MSA_ERR_ALIGN;
  const Dims d = to_dims(*dims);
  if (!workspace) return MSA_ERR_WORKSPACE;
  const float sc = resolve_scale(scale, d.d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (workspace_bytes >= prefill_ws_bytes(d)) {      // 128-token blocks: the sparse prefill's own layout
    if (misaligned(workspace)) return MSA_ERR_ALIGN;
    return hip_status(msa::launch_sparse_prefill_target(d, q, k, v, blk_idx, sc, bscore, idx_scale, out, lse,
                                                        target, kl, workspace, s));
  }
  // A smaller workspace: query chunks, as msa_sparse_prefill (every row's
  // target and KL depend only on its own partial results and pooled scores).
  const int cq = prefill_chunk_fitting(d, workspace_bytes);
  if (cq < 1) return MSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return MSA_ERR_ALIGN;
  return for_query_chunks(d, cq, [&](const Dims& c, int64_t row, int64_t kv_off) {
    return hip_status(msa::launch_sparse_prefill_target(
        c, q + row * d.h_q * d.d, k + kv_off, v + kv_off, blk_idx + row * d.h_kv * d.topk, sc,
        bscore + row * d.h_kv * d.nblk(), idx_scale, out + row * d.h_q * d.d, lse ? lse + row * d.h_q : nullptr,
        target + row * d.h_kv * d.topk, kl + row * d.h_kv, workspace, s));
  });
}

msa_status msa_sparse_prefill_backward(const msa_dims* dims, const uint16_t* q, const uint16_t* k,
                                       const uint16_t* v, const int32_t* blk_idx, const uint16_t* out,
                                       const float* lse, const uint16_t* dout, float scale, uint16_t* dq,
                                       uint16_t* dk, uint16_t* dv, void* workspace, size_t workspace_bytes,
                                       msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_SPARSE_PREFILL) | kOnly128);
  if (st != MSA_OK) return st;
  // The kernel forms addresses from 32-bit byte strides of q/dout rows and of dq partials.
  if ((int64_t)dims->h_q * dims->topk * dims->d >= (int64_t(1) << 31)) return MSA_ERR_UNSUPPORTED;
  if (dims->batch == 0 || dims->n_kv == 0) return MSA_OK;
  if (!k || !v || !dk || !dv) return MSA_ERR_NULL;
  if (dims->n_q > 0 && (!q || !blk_idx || !out || !lse || !dout || !dq)) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(blk_idx) || misaligned(out) ||
      misaligned(lse) || misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv))
    return MSA_ERR_ALIGN;
  const Dims d = to_dims(*dims);
  const size_t need = msa::prefill_ws_layout(d).total;
  if (!workspace || workspace_bytes < need) return MSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return MSA_ERR_ALIGN;
  return hip_status(msa::launch_sparse_prefill_backward(d, q, k, v, blk_idx, out, lse, dout,
                                                        resolve_scale(scale, d.d), dq, dk, dv, workspace,
                                                        static_cast<hipStream_t>(stream)));
}

msa_status msa_index_backward(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx,
                              const int32_t* blk_idx, const float* bscore, const float* target, const float* dkl,
                              float idx_scale, float* dq_idx, float* dk_idx, void* workspace, size_t workspace_bytes,
                              msa_stream stream) {
  msa_status st = check_dims(dims, kNeedDIdx | kCsr | kOnly128);
  if (st != MSA_OK) return st;
  if (dims->h_kv > 128) return MSA_ERR_UNSUPPORTED;
  if (!std::isfinite(idx_scale)) return MSA_ERR_SHAPE;
  if (dims->batch == 0) return MSA_OK;
  if (!k_idx || !dk_idx) return MSA_ERR_NULL;
  if (dims->n_q > 0 && (!q_idx || !blk_idx || !bscore || !target || !dkl || !dq_idx)) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(blk_idx) || misaligned(bscore) || misaligned(target) ||
      misaligned(dkl) || misaligned(dq_idx) || misaligned(dk_idx))
    return MSA_ERR_ALIGN;
  const Dims d = to_dims(*dims);
  const size_t need = msa::prefill_ws_layout(d).total;
  if (!workspace || workspace_bytes < need) return MSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return MSA_ERR_ALIGN;
  return hip_status(msa::launch_index_backward(d, q_idx, k_idx, blk_idx, bscore, target, dkl, idx_scale, dq_idx,
                                               dk_idx, workspace, static_cast<hipStream_t>(stream)));
}

msa_status msa_sparse_decode(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int32_t* blk_idx, float scale, uint16_t* out, float* lse, void* workspace,
                             size_t workspace_bytes, msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_SPARSE_DECODE));
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if (!q || !k || !v || !blk_idx || !out) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(blk_idx) || misaligned(out) ||
      (lse && misaligned(lse)))
    return MSA_ERR_ALIGN;
  const Dims d = to_dims(*dims);
  if (!workspace || workspace_bytes < decode_ws_bytes(d)) return MSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return MSA_ERR_ALIGN;
  return hip_status(run_sparse(d, true, q, k, v, blk_idx, resolve_scale(scale, d.d), out, lse, workspace,
                               static_cast<hipStream_t>(stream)));
}

size_t msa_prefill_chunked_workspace_size(const msa_dims* dims, int32_t chunk) {
  if (check_dims(dims, kNeedD | kNeedDIdx | kCsr) != MSA_OK || chunk < 1) return 0;
  return chunked_ws_bytes(to_dims(*dims), std::min<int>(chunk, std::max(dims->n_q, 1)), nullptr);
}

msa_status msa_prefill_chunked(const msa_dims* dims, int32_t chunk, const uint16_t* q_idx, const uint16_t* k_idx,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v, float scale,
                               int32_t* blk_idx, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                               msa_stream stream) {
  msa_status st = check_dims(dims, kNeedD | kNeedDIdx | kCsr);
  if (st != MSA_OK) return st;
  if (chunk < 1) return MSA_ERR_SHAPE;
  if (empty(*dims)) return MSA_OK;
  if (!q_idx || !k_idx || !q || !k || !v || !blk_idx || !out) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(q) || misaligned(k) || misaligned(v) ||
      misaligned(blk_idx) || misaligned(out) || (lse && misaligned(lse)))
    return MSA_ERR_ALIGN;
  const Dims d = to_dims(*dims);
  const int cq = std::min(chunk, d.n_q);
  size_t pre_off = 0;
  if (!workspace || workspace_bytes < chunked_ws_bytes(d, cq, &pre_off)) return MSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return MSA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float sc = resolve_scale(scale, d.d);
  void* pws = static_cast<char*>(workspace) + pre_off;
  for (int b = 0; b < d.batch; ++b) {
    for (int t0 = 0; t0 < d.n_q; t0 += cq) {
      Dims c = d;
      c.batch = 1;
      c.n_q = std::min(cq, d.n_q - t0);
      c.pos0 = d.pos0 + t0;
      const int64_t row = (int64_t)b * d.n_q + t0;      // first (sequence, query) row of the chunk
      const uint16_t* ci = q_idx + row * d.h_kv * d.d_idx;
      const uint16_t* ck = k_idx + (int64_t)b * d.n_kv * d.d_idx;
      const uint16_t* cqp = q + row * d.h_q * d.d;
      const int64_t kv_off = (int64_t)b * d.n_kv * d.h_kv * d.d;
      int32_t* cb = blk_idx + row * d.h_kv * d.topk;
      uint16_t* co = out + row * d.h_q * d.d;
      float* cl = lse ? lse + row * d.h_q : nullptr;
      st = hip_status(run_index_topk(c, ci, ck, cb, workspace, s));
      if (st == MSA_OK) st = hip_status(run_sparse(c, false, cqp, k + kv_off, v + kv_off, cb, sc, co, cl, pws, s));
      if (st != MSA_OK) return st;
    }
  }
  return MSA_OK;
}

msa_status msa_index_topk_varlen(const msa_dims* dims, const int32_t* seq_len, const uint16_t* q_idx,
                                 const uint16_t* k_idx, int32_t* blk_idx, void* workspace, size_t workspace_bytes,
                                 msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_INDEX_TOPK) | kDecode);
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if ((int64_t)dims->n_q * dims->h_kv > 16) return MSA_ERR_UNSUPPORTED;
  if (!seq_len || !q_idx || !k_idx || !blk_idx) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(blk_idx)) return MSA_ERR_ALIGN;
  Dims d = to_dims(*dims);
  d.seq_len = seq_len;
  if (!workspace || workspace_bytes < index_ws_bytes(d)) return MSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return MSA_ERR_ALIGN;
  return hip_status(run_index_topk(d, q_idx, k_idx, blk_idx, workspace, static_cast<hipStream_t>(stream)));
}

msa_status msa_sparse_decode_varlen(const msa_dims* dims, const int32_t* seq_len, const uint16_t* q,
                                    const uint16_t* k, const uint16_t* v, const int32_t* blk_idx, float scale,
                                    uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                    msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_SPARSE_DECODE));
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if (!seq_len || !q || !k || !v || !blk_idx || !out) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(blk_idx) || misaligned(out) ||
      (lse && misaligned(lse)))
    return MSA_ERR_ALIGN;
  Dims d = to_dims(*dims);
  d.seq_len = seq_len;
  if (!workspace || workspace_bytes < decode_ws_bytes(d)) return MSA_ERR_WORKSPACE;
  if (misaligned(workspace)) return MSA_ERR_ALIGN;
  return hip_status(run_sparse(d, true, q, k, v, blk_idx, resolve_scale(scale, d.d), out, lse, workspace,
                               static_cast<hipStream_t>(stream)));
}

msa_status msa_dense_gqa(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v, float scale,
                         uint16_t* out, float* lse, void* workspace, size_t workspace_bytes, msa_stream stream) {
  msa_status st = check_dims(dims, op_needs(MSA_OP_DENSE_GQA));
  if (st != MSA_OK) return st;
  if (empty(*dims)) return MSA_OK;
  if (!q || !k || !v || !out) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || (lse && misaligned(lse)))
    return MSA_ERR_ALIGN;
  const Dims d = index128(to_dims(*dims));          // the selection block plays no part
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float sc = resolve_scale(scale, d.d);
  if (d.n_q == 1) {
    const size_t need = msa::dense_decode_ws_layout(d).total;
    if (!workspace || workspace_bytes < need) return MSA_ERR_WORKSPACE;
    if (misaligned(workspace)) return MSA_ERR_ALIGN;
    return hip_status(msa::launch_dense_decode(d, q, k, v, sc, out, lse, workspace, s));
  }
  return hip_status(msa::launch_dense_prefill(d, q, k, v, sc, out, lse, s));
}

}  // extern "C"
