// Index branch, step 1 and 2: token scores q_idx . k_idx over every causal token,
// max-pooled per 128-token KV block (yhxrc.cn article, section "第一步：索引分支":
// one index query per GQA group, one index key per token shared by all heads,
// dot-product scores, block max-pooling).
//
// Output: bscore[b][t][g][j] (fp32, row stride nblk) for every j <= (pos0+t)/128.
// Entries j > (pos0+t)/128 are not written.  The pooled value of the query's
// own block covers only its causal tokens s <= pos0 + t.
//
// Two kernels:
//   * index_scores_tiled: many query rows (prefill).  The n_q*h_kv index queries
//     of a sequence form the rows of a matrix; a workgroup keeps 1024 of them in
//     registers as MFMA B operands and streams key blocks through LDS, so each
//     128-key block is fetched once per 1024 (token, group) rows.  The max over
//     a block's 128 keys is a reduction inside the score accumulators of a lane
//     plus two cross-lane steps, fused right after the MFMAs: scores never reach
//     memory, only the pooled block maxima do.
//   * index_scores_skinny: at most 16 query rows per sequence (decode).  Pure
//     index-key streaming: every wave pulls its key blocks straight from HBM into
//     MFMA A operands (no LDS round trip), bound by HBM bandwidth.
#include <algorithm>
#include <climits>
#include <atomic>
#include <cmath>

#include "launch.h"
#include "msa_device.h"
#include "msa_select.h"

namespace msa {
namespace {

constexpr int kTiledWaves = 8;
constexpr int kTiledColsPerWave = 128;                   // 4 MFMA column tiles of 32
constexpr int kTiledRows = kTiledWaves * kTiledColsPerWave;
constexpr int kFlush = 16;                               // pooled blocks buffered per row in LDS

template <int DI>
struct IndexSmem {
  static constexpr int S = DI + 8;                      // padded key row stride (elements)
  static constexpr int OS = kFlush + 1;                 // padded pooled-row stride (floats)
  uint16_t k[2][kBlock * S];                            // double-buffered key block
  float o[kTiledRows * OS];                             // pooled maxima awaiting write-out (per-wave rows)
};

// Scores of one 128-key block against this wave's 128 columns, reduced to the
// per-lane partial max rm[ct] over the 64 keys this lane's rows cover.  Work
// runs in 16 units (32-key tile kt, 32-column tile ct) of 8 chained MFMAs; the
// max-reduction of unit u-1 is issued after the MFMAs of unit u so the vector
// ALUs run while the matrix pipe is busy.  MASK adds the causal test (only the
// blocks reaching past some column's position need it).
template <int DI, bool MASK>
__device__ __forceinline__ void score_block(const uint16_t* __restrict__ kt_lds, const u32x4 (&qb)[4][DI / 16],
                                            int key0, const int (&plim)[4], float (&rm)[4]) {
  constexpr int KC = DI / 16;
  constexpr int S = DI + 8;
  const int lane = lane_id();
  const int half = lane >> 5, r32 = lane & 31;
  f32x16 acc[2];
  auto reduce = [&](const f32x16& a, int u) {
    const int kt = u >> 2, ct = u & 3;
    float m = rm[ct];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float x = a[v];
      if (MASK && (key0 + kt * 32 + 8 * (v >> 2) + 4 * half + (v & 3)) > plim[ct]) x = -INFINITY;
      m = vmax(m, x);
    }
    rm[ct] = m;
  };
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    u32x4 a[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      a[kc] = *reinterpret_cast<const u32x4*>(kt_lds + (kt * 32 + r32) * S + kc * 16 + half * 8);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int u = kt * 4 + ct;
      f32x16& cur = acc[u & 1];
      cur = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) cur = mfma_32x32x16(a[kc], qb[ct][kc], cur);
      if (u > 0) reduce(acc[(u - 1) & 1], u - 1);
    }
  }
  reduce(acc[1], 15);
}

// Number of KV blocks row tile t of a sequence needs: blocks 0 .. the block of
// the tile's last token.
__device__ __host__ __forceinline__ int tile_blocks(int t, int64_t nrows, int h_kv, int pos0) {
  const int64_t end = (int64_t)(t + 1) * kTiledRows;
  const int64_t last_row = (end < nrows ? end : nrows) - 1;
  return (pos0 + (int)(last_row / h_kv)) / kBlock + 1;
}

// One segment: row tile `tile` of sequence b against key blocks [jb, je).
// Double-buffered key staging through LDS with one barrier per block; pooled
// maxima collect in LDS per wave and go out in groups of kFlush blocks.
template <int DI>
__device__ __forceinline__ void tiled_segment(IndexSmem<DI>& sm, const uint16_t* __restrict__ q_idx,
                                              const uint16_t* __restrict__ k_idx, float* __restrict__ bscore, int b,
                                              int tile, int jb, int je, int n_kv, int pos0, int h_kv, int nblk,
                                              int64_t nrows) {
  constexpr int KC = DI / 16;                            // 16-wide contraction chunks
  constexpr int NT = kTiledWaves * 64;
  using Smem = IndexSmem<DI>;
  const int64_t r0 = (int64_t)tile * kTiledRows;
  const int64_t r_end = min(r0 + (int64_t)kTiledRows, nrows);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // wave index is uniform
  const int half = lane >> 5, r32 = lane & 31;

  // This wave's columns: rows rw0 + 32*ct + r32.
  const int64_t rw0 = r0 + (int64_t)wave * kTiledColsPerWave;
  const bool wave_live = rw0 < r_end;
  const int tw0 = wave_live ? (int)(rw0 / h_kv) : 0;
  const int tw1 = wave_live ? (int)((min(rw0 + kTiledColsPerWave, r_end) - 1) / h_kv) : 0;
  const int jw_max = (pos0 + tw1) / kBlock;              // last block any column of the wave needs
  const int jw_mask = (pos0 + tw0 + 1) / kBlock;         // first block reaching past the earliest column

  u32x4 qb[4][KC];
  int plim[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int64_t r = rw0 + ct * 32 + r32;
    const bool valid = wave_live && r < r_end;
    plim[ct] = valid ? pos0 + (int)(r / h_kv) : -1;      // -1: column never written
    const uint16_t* qr = q_idx + ((int64_t)b * nrows + r) * DI;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qb[ct][kc] = valid ? ld16(qr + kc * 16 + half * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  float* const orow = sm.o + (wave * kTiledColsPerWave + r32) * Smem::OS;   // + ct*32*OS

  // Key block staging: item i of this thread is key row key0 + i * KSTEP.
  constexpr int CHUNKS = kBlock * DI / 8;
  constexpr int ITEMS = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile staging must divide evenly");
  constexpr int KSTEP = NT / (DI / 8);
  const uint16_t* kseq = k_idx + (int64_t)b * n_kv * DI;
  const int skey0 = tid / (DI / 8);
  const int goff0 = skey0 * DI + (tid % (DI / 8)) * 8;
  const int loff0 = skey0 * Smem::S + (tid % (DI / 8)) * 8;
  u32x4 pre[ITEMS];
  auto fetch = [&](int j) {
    const uint16_t* kb = kseq + (int64_t)j * kBlock * DI + goff0;
    const int lim = n_kv - j * kBlock - skey0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      pre[i] = (i * KSTEP < lim) ? ld16(kb + i * KSTEP * DI) : u32x4{0u, 0u, 0u, 0u};
  };
  auto stash = [&](uint16_t* t) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) st16(t + loff0 + i * KSTEP * Smem::S, pre[i]);
  };

  fetch(jb);
  stash(sm.k[0]);
  __syncthreads();

  int jf = jb;                                           // first block of the group being buffered
  for (int j = jb; j < je; ++j) {
    const int cur = (j - jb) & 1;
    if (j + 1 < je) fetch(j + 1);
    const bool live = wave_live && j <= jw_max;
    if (live) {
      float rm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (j >= jw_mask)
        score_block<DI, true>(sm.k[cur], qb, j * kBlock, plim, rm);
      else
        score_block<DI, false>(sm.k[cur], qb, j * kBlock, plim, rm);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const float m = vmax(rm[ct], shfl_xor_f(rm[ct], 32)) + 0.0f;   // + 0 turns -0 into +0
        if (half == 0) orow[ct * 32 * Smem::OS + (j - jf)] = m;
      }
    }
    // The next key block goes to LDS before any pooled stores are issued, so
    // the wait for its loads never includes the stores of a write-out.
    if (j + 1 < je) stash(sm.k[cur ^ 1]);
    // Write out a full group (or the last one) row-contiguously: lane l takes
    // entry jf + (l & 15) of rows 4i + (l >> 4), so each store instruction
    // covers 4 rows x 16 consecutive blocks (four 64-byte runs) instead of 64
    // rows x 4 bytes.  Blocks past a row's own, and rows past the tile, are
    // skipped; the per-row test is needed only once the group reaches the
    // wave's earliest own block.
    if (live && (j - jf == kFlush - 1 || j == je - 1 || j == jw_max)) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int n = j - jf + 1;
      const int e = lane & 15, rsub = lane >> 4;
      const int nrw = (int)min((int64_t)kTiledColsPerWave, r_end - rw0);
      const bool all_causal = j <= (pos0 + tw0) / kBlock;
      // Wave-uniform bases with 32-bit byte offsets (a wave's rows span at
      // most 128 x 8192 entries); each pass issues its 4 LDS reads before its
      // 4 stores.
      const float* ow = sm.o + wave * kTiledColsPerWave * Smem::OS;
      char* gw = reinterpret_cast<char*>(bscore + ((int64_t)b * nrows + rw0) * nblk + jf);
      if (e < n) {
#pragma unroll 1
        for (int i0 = 0; i0 < kTiledColsPerWave / 4; i0 += 4) {
          float v[4];
          bool ok[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = 4 * (i0 + u) + rsub;
            ok[u] = c < nrw && (all_causal || jf + e <= (pos0 + ((int)rw0 + c) / h_kv) / kBlock);   // rows < 2^25
            v[u] = ow[c * Smem::OS + e];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t off = (uint32_t)((4 * (i0 + u) + rsub) * nblk + e) * 4u;
            if (ok[u]) *reinterpret_cast<float*>(gw + off) = v[u];
          }
        }
      }
      jf = j + 1;
    }
    __syncthreads();
  }
}

// Work decomposition.  Row tile t of a sequence needs blocks 0 .. ~t, so tile
// t is paired with tile T-1-t: every pair needs nearly the same number of
// block iterations.  Each pair's iterations (the long tile's blocks, then the
// short tile's) are cut into `pieces` equal ranges, one workgroup each, so all
// workgroups carry equal work whatever XCD and CU they land on.  A range spans
// at most the two tiles of its pair.
template <int DI>
__global__ __launch_bounds__(kTiledWaves * 64) void index_scores_tiled(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, float* __restrict__ bscore,
    int n_q, int n_kv, int pos0, int h_kv, int nblk, int tiles, int pairs, int pieces) {
  __shared__ IndexSmem<DI> sm;
  const int64_t nrows = (int64_t)n_q * h_kv;
  const int w = blockIdx.x;
  const int k = w % pieces;
  const int p = (w / pieces) % pairs;
  const int b = w / (pieces * pairs);
  const int ta = tiles - 1 - p, tb = p;                  // long tile, short tile (ta == tb: unpaired middle)
  const int na = tile_blocks(ta, nrows, h_kv, pos0);
  const int nb = ta != tb ? tile_blocks(tb, nrows, h_kv, pos0) : 0;
  const int total = na + nb;                             // <= 2 * 8192 blocks, so total * pieces fits an int
  const int lo = total * k / pieces, hi = total * (k + 1) / pieces;
#pragma nounroll
  for (int seg = 0; seg < 2; ++seg) {
    const int tile = __builtin_amdgcn_readfirstlane(seg == 0 ? ta : tb);
    const int jb = __builtin_amdgcn_readfirstlane(seg == 0 ? lo : max(lo, na) - na);
    const int je = __builtin_amdgcn_readfirstlane(seg == 0 ? min(hi, na) : hi - na);
    if (jb < je) tiled_segment<DI>(sm, q_idx, k_idx, bscore, b, tile, jb, je, n_kv, pos0, h_kv, nblk, nrows);
  }
}

// ---------------------------------------------------------------------------
// Index scores, block max-pool and top-k fused (k <= 16), for prefill-shaped
// calls: the pooled scores never leave the chip.  A workgroup keeps, in LDS,
// every one of its 1,024 rows' best k-1 blocks seen so far (the score's order
// key and 0xffff - block) and, per lane, the row's current worst kept key; as
// the key blocks stream by in increasing order, a block whose pooled score
// beats a row's worst kept score (strictly, so that among equal scores the
// earlier, lower block stays) replaces that worst entry.  When one workgroup
// sweeps a whole row tile, its lists are the selection and it writes blk_idx
// itself.  Otherwise each workgroup writes its rows' survivors, in block
// order, to the workspace (survivor lists [batch][row][piece][16]: 15 entries,
// then the count), and topk_merge_pieces selects each row's k-1 best among the
// survivors of the (at most kFusedPiecesMax) workgroups that swept its tile,
// adds the local block and writes the row ascending (yhxrc.cn article,
// "第一步：索引分支"; lumi-systems summary: exponential-free top-k).
constexpr int kFusedKk = 15;                             // k - 1 <= 15
constexpr int kFusedPiecesMax = 16;
constexpr int kFusedSlots = 256;                         // workgroup slots the piece count is chosen for
constexpr int kCandStride = 16;                          // survivors + count per (row, piece)

template <int DI>
struct IndexTopkSmem {
  static constexpr int S = DI + 8;
  uint16_t k[2][kBlock * S];                             // double-buffered key block
  uint32_t cs[kTiledRows * kFusedKk];                    // kept scores as order keys, [row][entry]
  uint16_t cj[kTiledRows * kFusedKk];                    // 0xffff - their blocks
};

// Piece k of a row tile's pair swept (and wrote survivor lists for) the tile
// when its range of the pair's block iterations meets the tile's blocks: the
// long tile's [0, na), then the short tile's [na, na + nb).  With more pieces
// than iterations some ranges are empty.
struct TilePieces {
  int total, na;
  bool long_tile;
  __device__ __forceinline__ bool covers(int k, int pieces) const {
    const int lo = total * k / pieces, hi = total * (k + 1) / pieces;
    return lo < hi && (long_tile ? lo < na : hi > na);
  }
};
__device__ __forceinline__ TilePieces tile_pieces(int tile, int tiles, int64_t nrows, int h_kv, int pos0) {
  const int p = tile < tiles - 1 - tile ? tile : tiles - 1 - tile;
  const int ta = tiles - 1 - p, tb = p;
  const int na = tile_blocks(ta, nrows, h_kv, pos0);
  const int nb = ta != tb ? tile_blocks(tb, nrows, h_kv, pos0) : 0;
  return TilePieces{na + nb, na, tile == ta};
}

// One segment: row tile `tile` of sequence b against key blocks [jb, je),
// scored as in tiled_segment, each block's pooled score offered to the row's
// kept list instead of being stored.
template <int DI>
__device__ __forceinline__ void tiled_segment_topk(IndexTopkSmem<DI>& sm, const uint16_t* __restrict__ q_idx,
                                                   const uint16_t* __restrict__ k_idx, float* __restrict__ cand_s,
                                                   int* __restrict__ cand_j, int32_t* __restrict__ blk, int b,
                                                   int tile, int jb, int je, int n_kv, int pos0, int h_kv,
                                                   int64_t nrows, int pieces, int piece, int kk) {
  constexpr int KC = DI / 16;
  constexpr int NT = kTiledWaves * 64;
  using Smem = IndexTopkSmem<DI>;
  const int64_t r0 = (int64_t)tile * kTiledRows;
  const int64_t r_end = min(r0 + (int64_t)kTiledRows, nrows);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, r32 = lane & 31;
  const int64_t rw0 = r0 + (int64_t)wave * kTiledColsPerWave;
  const bool wave_live = rw0 < r_end;
  const int tw0 = wave_live ? (int)(rw0 / h_kv) : 0;
  const int tw1 = wave_live ? (int)((min(rw0 + kTiledColsPerWave, r_end) - 1) / h_kv) : 0;
  const int jw_max = (pos0 + tw1) / kBlock;
  const int jw_mask = (pos0 + tw0 + 1) / kBlock;

  u32x4 qb[4][KC];
  int plim[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int64_t r = rw0 + ct * 32 + r32;
    const bool valid = wave_live && r < r_end;
    plim[ct] = valid ? pos0 + (int)(r / h_kv) : -1;
    const uint16_t* qr = q_idx + ((int64_t)b * nrows + r) * DI;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qb[ct][kc] = valid ? ld16(qr + kc * 16 + half * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  // This lane keeps the lists of rows ct = 2 half and 2 half + 1 of its column
  // r32: per row the kept count and the entry of the worst kept score (packed
  // count | entry << 8) and that score's order key.  A row's candidates are its
  // blocks j < jl = plim / 128 (none for a row past the tile, plim = -1).
  int meta[2] = {0, 0};
  uint32_t worst[2] = {0u, 0u};                        // order key of the worst kept score
  // Selected by value (not by an index into plim) so that no private array
  // is indexed by the lane's half.
  const int pl0 = half ? plim[2] : plim[0], pl1 = half ? plim[3] : plim[1];
  const int jlr[2] = {pl0 >= 0 ? pl0 / kBlock : -1, pl1 >= 0 ? pl1 / kBlock : -1};
  auto row_jl = [&](int u) { return jlr[u]; };
  // Empty slots hold the largest key, so the scan for the worst entry never
  // picks a slot past k-1.
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    uint32_t* rs = sm.cs + (wave * kTiledColsPerWave + r32 + (2 * half + u) * 32) * kFusedKk;
#pragma unroll
    for (int e = 0; e < kFusedKk; ++e) rs[e] = 0xffffffffu;
  }
  const int lrow0 = wave * kTiledColsPerWave + r32;      // + ct * 32: this lane's rows in the workgroup

  constexpr int CHUNKS = kBlock * DI / 8;
  constexpr int ITEMS = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile staging must divide evenly");
  constexpr int KSTEP = NT / (DI / 8);
  const uint16_t* kseq = k_idx + (int64_t)b * n_kv * DI;
  const int skey0 = tid / (DI / 8);
  const int goff0 = skey0 * DI + (tid % (DI / 8)) * 8;
  const int loff0 = skey0 * Smem::S + (tid % (DI / 8)) * 8;
  u32x4 pre[ITEMS];
  auto fetch = [&](int j) {
    const uint16_t* kb = kseq + (int64_t)j * kBlock * DI + goff0;
    const int lim = n_kv - j * kBlock - skey0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      pre[i] = (i * KSTEP < lim) ? ld16(kb + i * KSTEP * DI) : u32x4{0u, 0u, 0u, 0u};
  };
  auto stash = [&](uint16_t* t) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) st16(t + loff0 + i * KSTEP * Smem::S, pre[i]);
  };

  fetch(jb);
  stash(sm.k[0]);
  __syncthreads();

  for (int j = jb; j < je; ++j) {
    const int cur = (j - jb) & 1;
    if (j + 1 < je) fetch(j + 1);
    if (wave_live && j <= jw_max) {
      float rm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (j >= jw_mask)
        score_block<DI, true>(sm.k[cur], qb, j * kBlock, plim, rm);
      else
        score_block<DI, false>(sm.k[cur], qb, j * kBlock, plim, rm);
      // The two rows this lane keeps, as values (+ 0 turns -0 into +0).
      const float m0 = vmax(rm[0], shfl_xor_f(rm[0], 32)) + 0.0f, m1 = vmax(rm[1], shfl_xor_f(rm[1], 32)) + 0.0f;
      const float m2 = vmax(rm[2], shfl_xor_f(rm[2], 32)) + 0.0f, m3 = vmax(rm[3], shfl_xor_f(rm[3], 32)) + 0.0f;
      const float mrow[2] = {half ? m2 : m0, half ? m3 : m1};
      // Offer the block to the lane's two rows.  A lane that takes it into
      // one row goes through the insertion once with that row's state; only
      // lanes that take it into both rows go through it a second time, so a
      // wave pays two passes only when some lane needs both.
      const uint32_t mk0 = order_key(mrow[0]), mk1 = order_key(mrow[1]);
      const bool t0 = j < row_jl(0) && ((meta[0] & 0xff) < kk || mk0 > worst[0]);
      const bool t1 = j < row_jl(1) && ((meta[1] & 0xff) < kk || mk1 > worst[1]);
      // Insert key mk into the row held at LDS row `lrow` with state (m, w).
      auto insert = [&](int lrow, uint32_t mk, int& m, uint32_t& w) {
        uint32_t* rs = sm.cs + lrow * kFusedKk;
        uint16_t* rj = sm.cj + lrow * kFusedKk;
        const int cnt = m & 0xff;
        const int at = cnt < kk ? cnt : m >> 8;
        rs[at] = mk;
        rj[at] = (uint16_t)(0xffff - j);
        const int nc = min(cnt + 1, kk);
        m = nc;
        if (nc == kk) {
          // The worst kept entry (lowest score, then highest block) is the
          // smallest of the 64-bit keys (score key, 0xffff - block, slot);
          // all 15 slots are read at once.
          uint32_t ks[kFusedKk], ib[kFusedKk];
#pragma unroll
          for (int e = 0; e < kFusedKk; ++e) {
            ks[e] = rs[e];
            ib[e] = rj[e];
          }
          uint64_t best = ~0ull;
#pragma unroll
          for (int e = 0; e < kFusedKk; ++e) {
            const uint64_t key = ((uint64_t)ks[e] << 32) | ((ib[e] << 4) | (uint32_t)e);
            best = key < best ? key : best;
          }
          w = (uint32_t)(best >> 32);
          m = nc | ((int)(best & 15u) << 8);
        }
      };
      if (t0 || t1) {
        // Row 0 if it takes the block, else row 1 (state selected by value).
        int m = t0 ? meta[0] : meta[1];
        uint32_t w = t0 ? worst[0] : worst[1];
        insert(lrow0 + (2 * half + (t0 ? 0 : 1)) * 32, t0 ? mk0 : mk1, m, w);
        meta[0] = t0 ? m : meta[0];
        worst[0] = t0 ? w : worst[0];
        meta[1] = t0 ? meta[1] : m;
        worst[1] = t0 ? worst[1] : w;
      }
      if (t0 && t1) insert(lrow0 + (2 * half + 1) * 32, mk1, meta[1], worst[1]);
    }
    if (j + 1 < je) stash(sm.k[cur ^ 1]);
    __syncthreads();
  }
  // Each kept list goes out in block order: entry e's place is the number of
  // kept blocks below its own (blocks are distinct).  With one piece per tile
  // the segment has offered every candidate block j < jl of its rows, so the
  // list is the row's selection: it goes straight to blk_idx, followed by the
  // local block and -1 padding (a row with jl <= k-1 keeps all of 0 .. jl-1).
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int jl = row_jl(u);
    if (jl < 0) continue;
    const int cnt = meta[u] & 0xff;
    const int64_t r = rw0 + (2 * half + u) * 32 + r32;
    const int64_t at = (((int64_t)b * nrows + r) * pieces + piece) * kCandStride;
    const int topk = kk + 1;
    int32_t* out = blk + ((int64_t)b * nrows + r) * topk;
    const uint32_t* rs = sm.cs + (lrow0 + (2 * half + u) * 32) * kFusedKk;
    const uint16_t* rj = sm.cj + (lrow0 + (2 * half + u) * 32) * kFusedKk;
    int bjs[kFusedKk];
#pragma unroll
    for (int e = 0; e < kFusedKk; ++e) bjs[e] = e < cnt ? 0xffff - (int)rj[e] : INT_MAX;
#pragma unroll
    for (int e = 0; e < kFusedKk; ++e) {
      if (e < cnt) {
        int rank = 0;
#pragma unroll
        for (int f = 0; f < kFusedKk; ++f) rank += bjs[f] < bjs[e] ? 1 : 0;
        if (pieces == 1) {
          out[rank] = bjs[e];
        } else {
          const uint32_t k = rs[e];                      // back from the order key to the score
          cand_s[at + rank] = __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
          cand_j[at + rank] = bjs[e];
        }
      }
    }
    if (pieces == 1) {
      out[cnt] = jl;
      for (int i = cnt + 1; i < topk; ++i) out[i] = -1;
    } else {
      cand_j[at + kCandStride - 1] = cnt;
    }
  }
  __syncthreads();                                       // the lists are reused by the next segment
}

// The same decomposition as index_scores_tiled (tile pairs cut into equal
// pieces), with the piece count chosen for kFusedSlots slots and capped at
// kFusedPiecesMax so that the survivor workspace follows from the sizes alone.
template <int DI>
__global__ __launch_bounds__(kTiledWaves * 64) void index_topk_tiled(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, float* __restrict__ cand_s,
    int* __restrict__ cand_j, int32_t* __restrict__ blk, int n_q, int n_kv, int pos0, int h_kv, int tiles, int pairs,
    int pieces, int kk) {
  __shared__ IndexTopkSmem<DI> sm;
  const int64_t nrows = (int64_t)n_q * h_kv;
  const int w = blockIdx.x;
  const int k = w % pieces;
  const int p = (w / pieces) % pairs;
  const int b = w / (pieces * pairs);
  const int ta = tiles - 1 - p, tb = p;
  const int na = tile_blocks(ta, nrows, h_kv, pos0);
  const int nb = ta != tb ? tile_blocks(tb, nrows, h_kv, pos0) : 0;
  const int total = na + nb;
  const int lo = total * k / pieces, hi = total * (k + 1) / pieces;
#pragma nounroll
  for (int seg = 0; seg < 2; ++seg) {
    const int tile = __builtin_amdgcn_readfirstlane(seg == 0 ? ta : tb);
    const int jb = __builtin_amdgcn_readfirstlane(seg == 0 ? lo : max(lo, na) - na);
    const int je = __builtin_amdgcn_readfirstlane(seg == 0 ? min(hi, na) : hi - na);
    if (jb < je)
      tiled_segment_topk<DI>(sm, q_idx, k_idx, cand_s, cand_j, blk, b, tile, jb, je, n_kv, pos0, h_kv, nrows, pieces,
                             k, kk);
  }
}

// Each row's k-1 best among the survivor lists of the pieces that swept its
// tile (in piece order, each list in block order: position order is block
// order, so ties still go to the lower block), then the local block; one wave
// per row, rows ascending.
// V = slots per lane for the survivors: pieces * 15 <= 64 V.  A row whose
// survivors number exactly k-1 (one piece held all its candidates) takes them
// all, already in block order.
constexpr int kMergeRowsPerWg = 4;
template <int V>
__global__ __launch_bounds__(kMergeRowsPerWg * 64) void topk_merge_pieces(
    const float* __restrict__ cand_s, const int* __restrict__ cand_j, int32_t* __restrict__ blk, int64_t nrows_all,
    int n_q, int pos0, int h_kv, int topk, int tiles, int pieces) {
  __shared__ uint32_t ck[kMergeRowsPerWg][64];
  __shared__ int32_t ci[kMergeRowsPerWg][64];
  __shared__ uint32_t gk[kMergeRowsPerWg][V * 64];
  __shared__ int32_t gj[kMergeRowsPerWg][V * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kMergeRowsPerWg + wave;   // (b * n_q + t) * h_kv + g
  if (row >= nrows_all) return;
  const int64_t nrows = (int64_t)n_q * h_kv;
  const int64_t r = row % nrows;                        // row within its sequence
  const int t = (int)(r / h_kv);
  const int jl = (pos0 + t) / kBlock;
  int32_t* out = blk + row * topk;
  if (jl + 1 <= topk) {
    for (int i = lane; i < topk; i += 64) out[i] = (i <= jl) ? i : -1;
    return;
  }
  const int kk = topk - 1;
  if (lane == 0) out[kk] = jl;
  if (kk == 0) return;
  const TilePieces tp = tile_pieces((int)(r / kTiledRows), tiles, nrows, h_kv, pos0);
  int total = 0;
  for (int k = 0; k < pieces; ++k) {
    if (!tp.covers(k, pieces)) continue;
    const int64_t at = (row * pieces + k) * kCandStride;
    const int n = cand_j[at + kCandStride - 1];
    if (lane < n) {
      gk[wave][total + lane] = order_key(cand_s[at + lane]);
      gj[wave][total + lane] = cand_j[at + lane];
    }
    total += n;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (total == kk) {
    if (lane < kk) out[lane] = gj[wave][lane];
    return;
  }
  uint32_t key[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    key[i] = e < total ? gk[wave][e] : 0u;
  }
  wave_select<V>(key, kk, ck[wave], ci[wave], [&](int pos, uint32_t, int e) { out[pos] = gj[wave][e]; });
}

// Decode-shaped calls: at most 16 (token, group) rows per sequence.  One key
// block per wave: the scan is a pure HBM stream, and many short-lived waves
// keep more of it in flight than fewer waves walking several blocks each
// (measured at 1M tokens x 8 sequences: 0.364 ms against 0.385 ms at 4 blocks
// per wave).
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyBlocksPerWave = 1;

template <int DI>
__global__ __launch_bounds__(kSkinnyWaves * 64) void index_scores_skinny(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, float* __restrict__ bscore,
    int n_q, int n_kv, int pos0, int h_kv, int nblk, const int* __restrict__ seq_len) {
  constexpr int CC = DI / 32;
  const int b = blockIdx.y;
  const int nrows = n_q * h_kv;                         // <= 16
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, cl = lane & 15;
  pos0 = seq_pos0(seq_len, b, pos0, n_q, n_kv);
  const int jmax = (pos0 + n_q - 1) / kBlock;
  const int jw = (blockIdx.x * kSkinnyWaves + wave) * kSkinnyBlocksPerWave;
  if (jw > jmax) return;

  const bool cvalid = cl < nrows;
  const int plim = pos0 + (cvalid ? cl / h_kv : 0);
  float* orow = bscore + ((int64_t)b * nrows + (cvalid ? cl : 0)) * nblk;
  u32x4 qb[CC];
  const uint16_t* qr = q_idx + ((int64_t)b * nrows + cl) * DI;
#pragma unroll
  for (int cc = 0; cc < CC; ++cc) qb[cc] = cvalid ? ld16(qr + cc * 32 + q * 8) : u32x4{0u, 0u, 0u, 0u};
  const uint16_t* kseq = k_idx + (int64_t)b * n_kv * DI;

  const int je = min(jw + kSkinnyBlocksPerWave, jmax + 1);
  for (int j = jw; j < je; ++j) {
    u32x4 a[8][CC];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const int s = j * kBlock + kt * 16 + cl;
#pragma unroll
      for (int cc = 0; cc < CC; ++cc)
        a[kt][cc] = (s < n_kv) ? ld16(kseq + (int64_t)s * DI + cc * 32 + q * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    float rm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) acc = mfma_16x16x32(a[kt][cc], qb[cc], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[r];
        if ((j * kBlock + kt * 16 + q * 4 + r) > plim) v = -INFINITY;
        rm = vmax(rm, v);
      }
    }
    rm = colgroup_max(rm) + 0.0f;
    if (q == 0 && cvalid && j * kBlock <= plim) orow[j] = rm;
  }
}


// Pieces per tile pair.  Workgroups carry equal work, so the launch runs in
// ceil(W / slots) rounds of whole workgroups; the choice trades the idle part
// of the last round against the fixed cost of each piece (query operand load
// and pipeline fill, about kPieceCost block iterations).  At most kcap pieces.
int choose_pieces(int64_t units, double pair_iters, int64_t slots, int kcap = 1024) {
  constexpr double kPieceCost = 4.0;
  const int kmax = (int)std::max<double>(1.0, std::min<double>((double)kcap, pair_iters));
  int best = 1;
  double best_score = -1.0;
  for (int k = 1; k <= kmax; ++k) {
    const double w = (double)units * k;
    const double rounds = std::ceil(w / (double)slots);
    const double fill = w / (rounds * (double)slots);
    const double len = pair_iters / k;
    const double score = fill * len / (len + kPieceCost);
    if (score > best_score + 1e-9) {
      best_score = score;
      best = k;
    }
  }
  return best;
}

template <int DI>
hipError_t launch_index_scores_t(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, float* bscore,
                                 hipStream_t stream) {
  const int nblk = d.nblk();
  const int64_t nrows = (int64_t)d.n_q * d.h_kv;
  if (nrows <= 16) {
    const int jmax = d.seq_len ? (d.n_kv - 1) / kBlock : (d.pos0 + d.n_q - 1) / kBlock;
    const int per_wg = kSkinnyWaves * kSkinnyBlocksPerWave;
    dim3 grid((jmax + per_wg) / per_wg, d.batch);
    {
      LaunchTimer timer("index_scores_skinny", stream);
      hipLaunchKernelGGL(index_scores_skinny<DI>, grid, dim3(kSkinnyWaves * 64), 0, stream, q_idx, k_idx, bscore,
                         d.n_q, d.n_kv, d.pos0, d.h_kv, nblk, d.seq_len);
    }
  } else {
    const int64_t tiles = (nrows + kTiledRows - 1) / kTiledRows;
    const int64_t pairs = (tiles + 1) / 2;
    int64_t iters = 0;                                   // block iterations over all tiles of a sequence
    for (int64_t t = 0; t < tiles; ++t) iters += tile_blocks((int)t, nrows, d.h_kv, d.pos0);
    const int64_t slots = (int64_t)device_cu_count();    // one resident workgroup per CU (LDS-bound)
    const int pieces = choose_pieces(pairs * d.batch, (double)iters / pairs, slots);
    dim3 grid((unsigned)(d.batch * pairs * pieces));
    {
      LaunchTimer timer("index_scores_tiled", stream);
      hipLaunchKernelGGL(index_scores_tiled<DI>, grid, dim3(kTiledWaves * 64), 0, stream, q_idx, k_idx, bscore,
                         d.n_q, d.n_kv, d.pos0, d.h_kv, nblk, (int)tiles, (int)pairs, pieces);
    }
  }
  return hipGetLastError();
}

// Pieces per tile pair on the fused path: chosen for kFusedSlots workgroup
// slots (not the device's count) and at most kFusedPiecesMax, so that the
// survivor workspace follows from the sizes alone.
int fused_pieces(const Dims& d) {
  const int64_t nrows = (int64_t)d.n_q * d.h_kv;
  const int64_t tiles = (nrows + kTiledRows - 1) / kTiledRows;
  const int64_t pairs = (tiles + 1) / 2;
  int64_t iters = 0;
  for (int64_t t = 0; t < tiles; ++t) iters += tile_blocks((int)t, nrows, d.h_kv, d.pos0);
  return choose_pieces(pairs * d.batch, (double)iters / pairs, kFusedSlots, kFusedPiecesMax);
}

template <int DI>
hipError_t launch_index_topk_fused_t(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, int32_t* blk,
                                     void* ws, hipStream_t stream) {
  const int64_t nrows = (int64_t)d.n_q * d.h_kv;
  const int64_t tiles = (nrows + kTiledRows - 1) / kTiledRows;
  const int64_t pairs = (tiles + 1) / 2;
  const int pieces = fused_pieces(d);
  // One piece per tile writes blk_idx directly and needs no workspace.
  const size_t n = pieces > 1 ? (size_t)d.batch * nrows * pieces * kCandStride : 0;
  float* cand_s = pieces > 1 ? static_cast<float*>(ws) : nullptr;
  int* cand_j = pieces > 1 ? reinterpret_cast<int*>(static_cast<char*>(ws) + align_up(n * sizeof(float), 256))
                           : nullptr;
  {
    LaunchTimer timer("index_topk_tiled", stream);
    hipLaunchKernelGGL(index_topk_tiled<DI>, dim3((unsigned)(d.batch * pairs * pieces)), dim3(kTiledWaves * 64), 0,
                       stream, q_idx, k_idx, cand_s, cand_j, blk, d.n_q, d.n_kv, d.pos0, d.h_kv, (int)tiles,
                       (int)pairs, pieces, d.topk - 1);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pieces == 1) return e;
  const int64_t rows_all = (int64_t)d.batch * nrows;
  {
    LaunchTimer timer("topk_merge_pieces", stream);
    const dim3 grid((unsigned)((rows_all + kMergeRowsPerWg - 1) / kMergeRowsPerWg)), wg(kMergeRowsPerWg * 64);
    const int survivors = pieces * kFusedKk;
    if (survivors <= 64)
      hipLaunchKernelGGL(topk_merge_pieces<1>, grid, wg, 0, stream, cand_s, cand_j, blk, rows_all, d.n_q, d.pos0,
                         d.h_kv, d.topk, (int)tiles, pieces);
    else if (survivors <= 128)
      hipLaunchKernelGGL(topk_merge_pieces<2>, grid, wg, 0, stream, cand_s, cand_j, blk, rows_all, d.n_q, d.pos0,
                         d.h_kv, d.topk, (int)tiles, pieces);
    else
      hipLaunchKernelGGL(topk_merge_pieces<4>, grid, wg, 0, stream, cand_s, cand_j, blk, rows_all, d.n_q, d.pos0,
                         d.h_kv, d.topk, (int)tiles, pieces);
  }
  return hipGetLastError();
}

}  // namespace

bool index_topk_fused_applies(const Dims& d) {
  return d.block == 128 && !d.seq_len && d.topk - 1 <= kFusedKk && (int64_t)d.n_q * d.h_kv > 16;
}

size_t index_topk_fused_ws_bytes(const Dims& d) {
  const int pieces = fused_pieces(d);
  if (pieces == 1) return 0;
  const size_t n = (size_t)d.batch * d.n_q * d.h_kv * pieces * kCandStride;
  return align_up(n * sizeof(float), 256) + align_up(n * sizeof(int), 256);
}

hipError_t launch_index_topk_fused(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, int32_t* blk,
                                   void* ws, hipStream_t stream) {
  if (d.d_idx == 128) return launch_index_topk_fused_t<128>(d, q_idx, k_idx, blk, ws, stream);
  return launch_index_topk_fused_t<64>(d, q_idx, k_idx, blk, ws, stream);
}

hipError_t launch_index_scores(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, float* bscore,
                               hipStream_t stream) {
  if (d.d_idx == 128) return launch_index_scores_t<128>(d, q_idx, k_idx, bscore, stream);
  return launch_index_scores_t<64>(d, q_idx, k_idx, bscore, stream);
}

}  // namespace msa
