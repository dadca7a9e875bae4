// Index branch, step 3: exponential-free top-k over the pooled block scores with
// the query's own block always kept (lumi-systems summary: exponential-free
// top-k; lefilia.fr article: k blocks per query, local block always included).
//
// Per (query, group) row with local block jl = (pos0 + t) / 128:
//   * jl + 1 <= k: all blocks 0..jl, then -1 padding;
//   * otherwise jl plus the k-1 best blocks among 0..jl-1, best meaning larger
//     pooled score, ties to the lower block index; written in ascending order.
//
// The selection itself is msa_select.h's wave_select.
#include "launch.h"
#include "msa_device.h"
#include "msa_select.h"

namespace msa {
namespace {

constexpr int kRowsPerWg = 4;

// Rows of up to 64*V candidates: one wave per kRowsPerWave consecutive
// (query, group) rows, the next row's scores loaded while the current row is
// selected.  Each wave holds only as many scores per lane as its own longest
// row needs (causal prefill rows grow with the token, so most waves need far
// fewer than the launch's longest row).
constexpr int kRowsPerWave = 8;

template <int V>
__device__ __forceinline__ void topk_rows_body(const float* __restrict__ bscore, int32_t* __restrict__ blk,
                                               int64_t row0, int64_t row_end, int rb, int rt, int rg, int n_q,
                                               int pos0, int h_kv, int nblk, int topk, int n_kv,
                                               const int* __restrict__ seq_len, int lb, uint32_t* ck, int32_t* ci) {
  const int lane = lane_id();
  const int kk = topk - 1;
  auto step = [&](int& b, int& t, int& g) {
    if (++g == h_kv) {
      g = 0;
      if (++t == n_q) {
        t = 0;
        ++b;
      }
    }
  };
  // Local block of a row; its candidates are blocks 0 .. jl-1 (none when the row keeps all its blocks).
  auto local_block = [&](int b, int t) { return (seq_pos0(seq_len, b, pos0, n_q, n_kv) + t) >> lb; };
  auto load = [&](int64_t row, int jl, float (&f)[V]) {
    const float* sc = bscore + row * nblk;
    const int n = jl + 1 <= topk ? 0 : jl;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = i * 64 + lane;
      f[i] = sc[min(e, max(n - 1, 0))];                // clamped: every load is in the row
    }
  };
  float cur[V], nxt[V];
  int jl_next = local_block(rb, rt);
  load(row0, jl_next, cur);
#pragma unroll 1
  for (int64_t row = row0; row < row_end; ++row) {
    const int jl = jl_next;
    if (row + 1 < row_end) {                           // wave-uniform; the last row has no successor to look up
      step(rb, rt, rg);
      jl_next = local_block(rb, rt);
      load(row + 1, jl_next, nxt);
    }
    int32_t* out = blk + row * topk;
    if (jl + 1 <= topk) {
      for (int i = lane; i < topk; i += 64) out[i] = (i <= jl) ? i : -1;
    } else {
      if (lane == 0) out[kk] = jl;                     // the local block is the largest index
      if (kk > 0) {
        const int n = jl;                              // candidates 0..jl-1, n > kk
        uint32_t key[V];
#pragma unroll
        for (int i = 0; i < V; ++i) key[i] = (i * 64 + lane < n) ? order_key(cur[i]) : 0u;   // 0: below every key
        wave_select<V>(key, kk, ck, ci, [&](int pos, uint32_t, int e) { out[pos] = e; });
      }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) cur[i] = nxt[i];
  }
}

template <int V, bool WIDTHS>
__global__ __launch_bounds__(kRowsPerWg * 64) void block_topk_rows(const float* __restrict__ bscore,
                                                                   int32_t* __restrict__ blk, int n_q, int pos0,
                                                                   int h_kv, int nblk, int topk, int64_t nrows,
                                                                   int n_kv, const int* __restrict__ seq_len,
                                                                   int lb) {
  __shared__ uint32_t ck[kRowsPerWg][64];
  __shared__ int32_t ci[kRowsPerWg][64];
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * kRowsPerWg + wave) * kRowsPerWave;
  if (row0 >= nrows) return;
  const int64_t row_end = min(row0 + (int64_t)kRowsPerWave, nrows);
  // (sequence, token, group) of the wave's first row (wave-uniform; rows are
  // (b * n_q + t) * h_kv + g), and the most candidates any of its rows has.
  int rb, rt, rg;
  {
    const int64_t bt = row0 / h_kv;
    rg = (int)(row0 - bt * h_kv);
    rb = (int)(bt / n_q);
    rt = (int)(bt - (int64_t)rb * n_q);
  }
  if constexpr (!WIDTHS) {                             // every row of the launch needs the full width
    topk_rows_body<V>(bscore, blk, row0, row_end, rb, rt, rg, n_q, pos0, h_kv, nblk, topk, n_kv, seq_len, lb,
                      ck[wave], ci[wave]);
    return;
  }
  // Stepped row by row from the first row's (b, t, g), as the body does: no
  // 64-bit division per row.
  int need = 0;
  {
    int b = rb, t = rt, g = rg;
    for (int64_t row = row0; row < row_end; ++row) {
      const int jl = (seq_pos0(seq_len, b, pos0, n_q, n_kv) + t) >> lb;
      need = max(need, jl + 1 <= topk ? 0 : jl);
      if (++g == h_kv) {
        g = 0;
        if (++t == n_q) {
          t = 0;
          ++b;
        }
      }
    }
  }
  need = __builtin_amdgcn_readfirstlane(need);
#define MSA_TOPK_ROWS(VV)                                                                                      \
  topk_rows_body<VV>(bscore, blk, row0, row_end, rb, rt, rg, n_q, pos0, h_kv, nblk, topk, n_kv, seq_len, lb, \
                     ck[wave], ci[wave])
  if (V >= 2 && need <= 64) {
    MSA_TOPK_ROWS(1);
  } else if constexpr (V >= 4) {
    if (need <= 128) {
      MSA_TOPK_ROWS(2);
    } else if (V >= 8 && need <= 256) {
      MSA_TOPK_ROWS((V >= 8 ? 4 : V));
    } else if (V >= 16 && need <= 512) {
      MSA_TOPK_ROWS((V >= 16 ? 8 : V));
    } else {
      MSA_TOPK_ROWS(V);
    }
  } else {
    MSA_TOPK_ROWS(V);
  }
#undef MSA_TOPK_ROWS
}

// Long rows, or few rows: a workgroup of NW waves per row.  Wave w selects the
// exact top-kk of its contiguous slice [w*n/NW, (w+1)*n/NW) into LDS; the
// slices are in block order, so wave 0's exact top-kk over the (at most NW*kk)
// survivors, ties broken by position, is the row's answer.
template <int V, int NW>
__global__ __launch_bounds__(NW * 64) void block_topk_wg(const float* __restrict__ bscore,
                                                         int32_t* __restrict__ blk, int n_q, int pos0, int h_kv,
                                                         int nblk, int topk, int n_kv,
                                                         const int* __restrict__ seq_len, int lb) {
  constexpr int CV = (NW * 63 + 63) / 64;              // survivor slots per lane in the final round
  __shared__ uint32_t ck[NW][64];
  __shared__ int32_t ci[NW][64];
  __shared__ uint32_t cand_k[NW][64];
  __shared__ int32_t cand_i[NW][64];
  __shared__ int cand_n[NW];
  __shared__ uint32_t cat_k[CV * 64];
  __shared__ int32_t cat_i[CV * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;
  const int64_t bt = row / h_kv;
  const int jl = (seq_pos0(seq_len, (int)(bt / n_q), pos0, n_q, n_kv) + (int)(bt % n_q)) >> lb;
  int32_t* out = blk + row * topk;
  if (jl + 1 <= topk) {                                // whole workgroup leaves together
    for (int i = threadIdx.x; i < topk; i += NW * 64) out[i] = (i <= jl) ? i : -1;
    return;
  }
  const int kk = topk - 1;
  if (threadIdx.x == 0) out[kk] = jl;
  if (kk == 0) return;
  const float* sc = bscore + row * nblk;
  const int n = jl;
  const int q0 = (int)((int64_t)n * wave / NW), q1 = (int)((int64_t)n * (wave + 1) / NW);
  const int nq = q1 - q0;
  if (nq <= kk) {                                      // the whole slice survives
    for (int e = lane; e < nq; e += 64) {
      cand_k[wave][e] = order_key(sc[q0 + e]);
      cand_i[wave][e] = q0 + e;
    }
    if (lane == 0) cand_n[wave] = nq;
  } else {
    // Loads clamped into the slice (nq > kk >= 1 here) so none is behind a
    // branch: all V are in flight at once, then the tail is masked.
    float f[V];
#pragma unroll
    for (int i = 0; i < V; ++i) f[i] = sc[q0 + min(i * 64 + lane, nq - 1)];
    uint32_t key[V];
#pragma unroll
    for (int i = 0; i < V; ++i) key[i] = (i * 64 + lane < nq) ? order_key(f[i]) : 0u;
    wave_select<V>(key, kk, ck[wave], ci[wave], [&](int pos, uint32_t k, int e) {
      cand_k[wave][pos] = k;
      cand_i[wave][pos] = q0 + e;
    });
    if (lane == 0) cand_n[wave] = kk;
  }
  __syncthreads();
  // Concatenate the slices' survivors in block order into cat_*.
  int start = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) start += cand_n[w];
    total += cand_n[w];
  }
  for (int e = lane; e < cand_n[wave]; e += 64) {
    cat_k[start + e] = cand_k[wave][e];
    cat_i[start + e] = cand_i[wave][e];
  }
  __syncthreads();
  if (wave != 0) return;
  // At most NW * (topk - 1) <= NW * 63 candidates.
  uint32_t key[CV];
#pragma unroll
  for (int i = 0; i < CV; ++i) {
    const int c = i * 64 + lane;
    key[i] = c < total ? cat_k[c] : 0u;
  }
  wave_select<CV>(key, kk, ck[0], ci[0], [&](int pos, uint32_t, int c) { out[pos] = cat_i[c]; });
}

template <int V>
hipError_t launch_v(const Dims& d, const float* bscore, int32_t* blk, hipStream_t stream) {
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_kv;
  const int64_t per_wg = (int64_t)kRowsPerWg * kRowsPerWave;
  const int64_t wgs = (nrows + per_wg - 1) / per_wg;
  // Per-wave widths pay off when the rows' candidate counts span several
  // widths (a causal prefill from position 0: 0.85 against 0.91 ms at 128K);
  // when every row needs the launch's width (1,023 candidates in every row:
  // 0.91 against 0.96 ms) the plain kernel is faster.
  const int lb = block_shift(d);
  const int jl_lo = d.seq_len ? 0 : d.pos0 >> lb;
  const int n_lo = jl_lo + 1 <= d.topk ? 0 : jl_lo;   // candidates of the shortest row
  int w_lo = 1;
  while (64 * w_lo < n_lo) w_lo *= 2;
  const bool widths = w_lo < V;
  auto kern = widths ? block_topk_rows<V, true> : block_topk_rows<V, false>;
  {
    LaunchTimer timer("block_topk_rows", stream);
    hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kRowsPerWg * 64), 0, stream, bscore, blk,
                       d.n_q, d.pos0, d.h_kv, d.nblk(), d.topk, nrows, d.n_kv, d.seq_len, block_shift(d));
  }
  return hipGetLastError();
}

template <int V, int NW>
hipError_t launch_wg(const Dims& d, const float* bscore, int32_t* blk, hipStream_t stream) {
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_kv;
  {
    LaunchTimer timer("block_topk_wg", stream);
    hipLaunchKernelGGL((block_topk_wg<V, NW>), dim3((unsigned)nrows), dim3(NW * 64), 0, stream, bscore, blk, d.n_q,
                       d.pos0, d.h_kv, d.nblk(), d.topk, d.n_kv, d.seq_len, block_shift(d));
  }
  return hipGetLastError();
}

// A workgroup of NW waves per row, each wave holding V candidates per lane.
template <int NW>
hipError_t launch_wg_v(const Dims& d, int jl_max, const float* bscore, int32_t* blk, hipStream_t stream) {
  const int per_lane = ((jl_max + NW - 1) / NW + 63) / 64;
  if (per_lane <= 2 && NW >= 8) return launch_wg<2, NW>(d, bscore, blk, stream);
  if (per_lane <= 4) return launch_wg<4, NW>(d, bscore, blk, stream);
  if (per_lane <= 8) return launch_wg<8, NW>(d, bscore, blk, stream);
  if (per_lane <= 16) return launch_wg<16, NW>(d, bscore, blk, stream);
  return launch_wg<32, NW>(d, bscore, blk, stream);
}

}  // namespace

hipError_t launch_block_topk(const Dims& d, const float* bscore, int32_t* blk, hipStream_t stream) {
  const int jl_max = (d.seq_len ? d.n_kv - 1 : d.pos0 + d.n_q - 1) >> block_shift(d);   // most candidates of a row
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_kv;
  // Few rows (decode): a workgroup per row, its waves splitting the row, so the
  // launch still has a few thousand waves loading scores.
  const int64_t slots = 4LL * device_cu_count();       // one wave per SIMD
  if (nrows * 4 < slots * 4 && jl_max > 256) {
    if (nrows * 16 <= slots * 4 || jl_max > 4096) return launch_wg_v<16>(d, jl_max, bscore, blk, stream);
    return launch_wg_v<8>(d, jl_max, bscore, blk, stream);
  }
  const int per_lane = (jl_max + 63) / 64;
  if (per_lane <= 1) return launch_v<1>(d, bscore, blk, stream);
  if (per_lane <= 2) return launch_v<2>(d, bscore, blk, stream);
  if (per_lane <= 4) return launch_v<4>(d, bscore, blk, stream);
  if (per_lane <= 8) return launch_v<8>(d, bscore, blk, stream);
  if (per_lane <= 16) return launch_v<16>(d, bscore, blk, stream);
  // longer rows (more than 1,024 candidates), and many of them: a workgroup of
  // 4 waves per row (measured at 8,192 queries of a 1M context: 0.94 ms against
  // 1.36 ms with 8 waves of 16 scores per lane)
  return launch_wg_v<4>(d, jl_max, bscore, blk, stream);   // the C-ABI caps nblk at 8192
}

// ------------------------------------------------- 256-token blocks -------
//
// A block of 256 tokens is two blocks of 128: its pooled score is the larger
// of the two 128-token pooled scores (the second one only when it holds a
// causal token), so the top-k over 256-token blocks runs on these maxima, and
// a selected 256-token block j stands for the 128-token blocks 2j and 2j + 1
// in the main branch (a 128-token block past the query is skipped there).

namespace {

__global__ __launch_bounds__(256) void pool_block_pairs(const float* __restrict__ p128, float* __restrict__ p256,
                                                        int64_t nrows, int n_q, int pos0, int h_kv, int nblk128,
                                                        int nblk256, int n_kv, const int* __restrict__ seq_len) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nrows * nblk256) return;
  const int64_t row = i / nblk256;
  const int j = (int)(i % nblk256);
  const int64_t bt = row / h_kv;
  const int jl128 = (seq_pos0(seq_len, (int)(bt / n_q), pos0, n_q, n_kv) + (int)(bt % n_q)) / kBlock;
  const float* src = p128 + row * nblk128;
  float v = -INFINITY;
  if (2 * j <= jl128) v = src[2 * j];
  if (2 * j + 1 <= jl128) v = vmax(v, src[2 * j + 1]);
  p256[i] = v;
}

__global__ __launch_bounds__(256) void expand_block_pairs(const int32_t* __restrict__ blk256,
                                                          int32_t* __restrict__ blk128, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int j = blk256[i];
  int2 o;
  o.x = j >= 0 ? 2 * j : -1;
  o.y = j >= 0 ? 2 * j + 1 : -1;
  *reinterpret_cast<int2*>(blk128 + 2 * i) = o;
}

}  // namespace

hipError_t launch_pool_block_pairs(const Dims& d, const float* p128, float* p256, hipStream_t stream) {
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_kv;
  const int nblk128 = (d.n_kv + kBlock - 1) / kBlock, nblk256 = (d.n_kv + 2 * kBlock - 1) / (2 * kBlock);
  const int64_t n = nrows * nblk256;
  if (n == 0) return hipSuccess;
  LaunchTimer timer("pool_block_pairs", stream);
  hipLaunchKernelGGL(pool_block_pairs, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p128, p256, nrows,
                     d.n_q, d.pos0, d.h_kv, nblk128, nblk256, d.n_kv, d.seq_len);
  return hipGetLastError();
}

hipError_t launch_expand_block_pairs(const Dims& d, const int32_t* blk256, int32_t* blk128, hipStream_t stream) {
  const int64_t n = (int64_t)d.batch * d.n_q * d.h_kv * d.topk;
  if (n == 0) return hipSuccess;
  LaunchTimer timer("expand_block_pairs", stream);
  hipLaunchKernelGGL(expand_block_pairs, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, blk256, blk128, n);
  return hipGetLastError();
}

}  // namespace msa
