// Index branch, step 3: exponential-free top-k over the pooled block scores with
// the query's own block always kept (lumi-systems summary: exponential-free
// top-k; lefilia.fr article: k blocks per query, local block always included).
//
// Per (query, group) row with local block jl = (pos0 + t) / 128:
//   * jl + 1 <= k: all blocks 0..jl, then -1 padding;
//   * otherwise jl plus the k-1 best blocks among 0..jl-1, best meaning larger
//     pooled score, ties to the lower block index; written in ascending order.
//
// One wave per row; the row's scores live in registers (element e = 64*i + lane
// sits in slot i of lane `lane`, so slot-major / lane-minor order is block
// order).  Scores are mapped to order-preserving unsigned keys.  No exponential,
// no sort:
//   1. T0 = (k-1)-th largest of the 64 per-lane maxima.  At least k-1 elements
//      are >= T0, so the true threshold T is >= T0 and every selected block has
//      key >= T0.
//   2. If fewer than k-1 keys are > T0, then T = T0: keep all keys > T0 and the
//      lowest-index keys == T0 (two ballots per slot).
//   3. Else, if at most 64 keys are > T0, compact them into LDS in block order,
//      one per lane, and select exactly among them (bitwise threshold search
//      over one key per lane, ties by lane order = block order).
//   4. Else (adversarial rows only) bitwise threshold search over all keys.
// Each bitwise search finds the largest T with count(key >= T) >= k-1 by
// fixing bits from the top, counting with wave ballots.
#include "launch.h"
#include "msa_device.h"

namespace msa {
namespace {

constexpr int kRowsPerWg = 4;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);        // -0 + 0 = +0: -0 ties with +0
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);   // negative: ~u, else u | sign; finite keys >= 0x007fffff
}

// Largest T with #{lanes : x >= T} >= kk  (= the kk-th largest x).
__device__ __forceinline__ uint32_t kth_largest_wave(uint32_t x, int kk) {
  uint32_t T = 0u;
#pragma unroll 4
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    if (__popcll(ballot(x >= c)) >= kk) T = c;
  }
  return T;
}

template <int V>
__device__ __forceinline__ uint32_t kth_largest_all(const uint32_t (&key)[V], int kk) {
  uint32_t T = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) cnt += __popcll(ballot(key[i] >= c));
    if (cnt >= kk) T = c;
  }
  return T;
}

// Exact top-kk of the keys a wave holds (element e = 64*i + lane, key 0 =
// absent), ties to the lower element; sink(pos, key, e) receives the kk
// winners in ascending element order, pos = 0..kk-1.  Needs kk <= #present.
// cbuf: this wave's 64-entry LDS compaction buffer.
template <int V, typename Sink>
__device__ __forceinline__ void wave_select(const uint32_t (&key)[V], int kk, uint32_t* ck, int32_t* ci,
                                            Sink sink) {
  const int lane = lane_id();
  auto emit_threshold = [&](uint32_t T, int need) {
    int base = 0, eqbase = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const bool gt = key[i] > T, eq = key[i] == T;
      const uint64_t eqm = ballot(eq);
      const int er = eqbase + lanes_below(eqm);
      eqbase += __popcll(eqm);
      const bool sel = gt || (eq && er < need);
      const uint64_t sm = ballot(sel);
      if (sel) sink(base + lanes_below(sm), key[i], i * 64 + lane);
      base += __popcll(sm);
    }
  };
  uint32_t lm = 0u;
#pragma unroll
  for (int i = 0; i < V; ++i) lm = max(lm, key[i]);
  const uint32_t T0 = kth_largest_wave(lm, kk);
  int c_gt = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) c_gt += __popcll(ballot(key[i] > T0));
  if (c_gt < kk) {                                     // case 2: threshold is T0
    emit_threshold(T0, kk - c_gt);
    return;
  }
  if (c_gt <= 64) {                                    // case 3: compact the keys > T0
    int base = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const bool gt = key[i] > T0;
      const uint64_t m = ballot(gt);
      if (gt) {
        const int pos = base + lanes_below(m);
        ck[pos] = key[i];
        ci[pos] = i * 64 + lane;
      }
      base += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t my = lane < c_gt ? ck[lane] : 0u;
    const int32_t myi = lane < c_gt ? ci[lane] : 0;
    const uint32_t T = kth_largest_wave(my, kk);
    const int n_gt = __popcll(ballot(my > T));
    const uint64_t eqm = ballot(my == T);
    const bool sel = my > T || (my == T && lanes_below(eqm) < kk - n_gt);
    const uint64_t sm = ballot(sel);
    if (sel) sink(lanes_below(sm), my, myi);
    return;
  }
  // case 4
  const uint32_t T = kth_largest_all<V>(key, kk);
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) n_gt += __popcll(ballot(key[i] > T));
  emit_threshold(T, kk - n_gt);
}

// Rows of up to 64*V candidates: one wave per kRowsPerWave consecutive
// (query, group) rows, the next row's scores loaded while the current row is
// selected.
constexpr int kRowsPerWave = 8;
template <int V>
__global__ __launch_bounds__(kRowsPerWg * 64) void block_topk_rows(const float* __restrict__ bscore,
                                                                   int32_t* __restrict__ blk, int n_q, int pos0,
                                                                   int h_kv, int nblk, int topk, int64_t nrows,
                                                                   int n_kv, const int* __restrict__ seq_len,
                                                                   int lb) {
  __shared__ uint32_t ck[kRowsPerWg][64];
  __shared__ int32_t ci[kRowsPerWg][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * kRowsPerWg + wave) * kRowsPerWave;
  if (row0 >= nrows) return;
  const int64_t row_end = min(row0 + (int64_t)kRowsPerWave, nrows);
  const int kk = topk - 1;
  // (sequence, token) of a row, found once for the wave's first row and then
  // stepped row by row (wave-uniform; rows are (b * n_q + t) * h_kv + g).
  int rb, rt, rg;
  {
    const int64_t bt = row0 / h_kv;
    rg = (int)(row0 - bt * h_kv);
    rb = (int)(bt / n_q);
    rt = (int)(bt - (int64_t)rb * n_q);
  }
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
        wave_select<V>(key, kk, ck[wave], ci[wave], [&](int pos, uint32_t, int e) { out[pos] = e; });
      }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) cur[i] = nxt[i];
  }
}

// Long rows (up to 256*V candidates): a workgroup per row.  Wave w selects the
// exact top-kk of its contiguous quarter [w*n/4, (w+1)*n/4) into LDS; the
// quarters are in block order, so wave 0's exact top-kk over the (at most 4*kk)
// survivors, ties broken by position, is the row's answer.
constexpr int kWgWaves = 4;
template <int V>
__global__ __launch_bounds__(kWgWaves * 64) void block_topk_wg(const float* __restrict__ bscore,
                                                               int32_t* __restrict__ blk, int n_q, int pos0,
                                                               int h_kv, int nblk, int topk, int n_kv,
                                                               const int* __restrict__ seq_len, int lb) {
  __shared__ uint32_t ck[kWgWaves][64];
  __shared__ int32_t ci[kWgWaves][64];
  __shared__ uint32_t cand_k[kWgWaves][64];
  __shared__ int32_t cand_i[kWgWaves][64];
  __shared__ int cand_n[kWgWaves];
  __shared__ uint32_t cat_k[kWgWaves * 64];
  __shared__ int32_t cat_i[kWgWaves * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;
  const int64_t bt = row / h_kv;
  const int jl = (seq_pos0(seq_len, (int)(bt / n_q), pos0, n_q, n_kv) + (int)(bt % n_q)) >> lb;
  int32_t* out = blk + row * topk;
  if (jl + 1 <= topk) {                                // whole workgroup leaves together
    for (int i = threadIdx.x; i < topk; i += kWgWaves * 64) out[i] = (i <= jl) ? i : -1;
    return;
  }
  const int kk = topk - 1;
  if (threadIdx.x == 0) out[kk] = jl;
  if (kk == 0) return;
  const float* sc = bscore + row * nblk;
  const int n = jl;
  const int q0 = (int)((int64_t)n * wave / kWgWaves), q1 = (int)((int64_t)n * (wave + 1) / kWgWaves);
  const int nq = q1 - q0;
  if (nq <= kk) {                                      // the whole quarter survives
    for (int e = lane; e < nq; e += 64) {
      cand_k[wave][e] = order_key(sc[q0 + e]);
      cand_i[wave][e] = q0 + e;
    }
    if (lane == 0) cand_n[wave] = nq;
  } else {
    uint32_t key[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = i * 64 + lane;
      key[i] = (e < nq) ? order_key(sc[q0 + e]) : 0u;
    }
    wave_select<V>(key, kk, ck[wave], ci[wave], [&](int pos, uint32_t k, int e) {
      cand_k[wave][pos] = k;
      cand_i[wave][pos] = q0 + e;
    });
    if (lane == 0) cand_n[wave] = kk;
  }
  __syncthreads();
  // Concatenate the quarters' survivors in block order into cat_*.
  int start = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWgWaves; ++w) {
    if (w < wave) start += cand_n[w];
    total += cand_n[w];
  }
  for (int e = lane; e < cand_n[wave]; e += 64) {
    cat_k[start + e] = cand_k[wave][e];
    cat_i[start + e] = cand_i[wave][e];
  }
  __syncthreads();
  if (wave != 0) return;
  // At most kWgWaves * (topk - 1) <= 4 * 63 candidates.
  uint32_t key[kWgWaves];
#pragma unroll
  for (int i = 0; i < kWgWaves; ++i) {
    const int c = i * 64 + lane;
    key[i] = c < total ? cat_k[c] : 0u;
  }
  wave_select<kWgWaves>(key, kk, ck[0], ci[0], [&](int pos, uint32_t, int c) { out[pos] = cat_i[c]; });
}

template <int V>
hipError_t launch_v(const Dims& d, const float* bscore, int32_t* blk, hipStream_t stream) {
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_kv;
  const int64_t per_wg = (int64_t)kRowsPerWg * kRowsPerWave;
  const int64_t wgs = (nrows + per_wg - 1) / per_wg;
  {
    LaunchTimer timer("block_topk_rows", stream);
    hipLaunchKernelGGL(block_topk_rows<V>, dim3((unsigned)wgs), dim3(kRowsPerWg * 64), 0, stream, bscore, blk,
                       d.n_q, d.pos0, d.h_kv, d.nblk(), d.topk, nrows, d.n_kv, d.seq_len, block_shift(d));
  }
  return hipGetLastError();
}

template <int V>
hipError_t launch_wg(const Dims& d, const float* bscore, int32_t* blk, hipStream_t stream) {
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_kv;
  {
    LaunchTimer timer("block_topk_wg", stream);
    hipLaunchKernelGGL(block_topk_wg<V>, dim3((unsigned)nrows), dim3(kWgWaves * 64), 0, stream, bscore, blk, d.n_q,
                       d.pos0, d.h_kv, d.nblk(), d.topk, d.n_kv, d.seq_len, block_shift(d));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_topk(const Dims& d, const float* bscore, int32_t* blk, hipStream_t stream) {
  const int jl_max = (d.seq_len ? d.n_kv - 1 : d.pos0 + d.n_q - 1) >> block_shift(d);   // most candidates of a row
  const int per_lane = (jl_max + 63) / 64;
  if (per_lane <= 1) return launch_v<1>(d, bscore, blk, stream);
  if (per_lane <= 2) return launch_v<2>(d, bscore, blk, stream);
  if (per_lane <= 4) return launch_v<4>(d, bscore, blk, stream);
  if (per_lane <= 8) return launch_v<8>(d, bscore, blk, stream);
  if (per_lane <= 16) return launch_v<16>(d, bscore, blk, stream);
  if (per_lane <= 32) return launch_v<32>(d, bscore, blk, stream);
  // longer rows: a workgroup per row, a quarter row per wave
  const int per_lane_q = ((jl_max + kWgWaves - 1) / kWgWaves + 63) / 64;
  if (per_lane_q <= 16) return launch_wg<16>(d, bscore, blk, stream);
  return launch_wg<32>(d, bscore, blk, stream);         // the C-ABI caps nblk at 8192
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
