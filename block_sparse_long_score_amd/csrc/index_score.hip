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
#include "launch.h"
#include "msa_device.h"

namespace msa {
namespace {

constexpr int kTiledWaves = 8;
constexpr int kTiledColsPerWave = 128;                   // 8 MFMA column tiles
constexpr int kTiledRows = kTiledWaves * kTiledColsPerWave;

template <int DI>
struct KeyTile {
  static constexpr int S = DI + 8;                      // padded row stride
  uint16_t k[kBlock * S];
};

template <int DI>
__global__ __launch_bounds__(kTiledWaves * 64) void index_scores_tiled(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, float* __restrict__ bscore,
    int n_q, int n_kv, int pos0, int h_kv, int nblk, int blocks_per_chunk) {
  constexpr int CC = DI / 32;                            // 32-wide contraction chunks
  constexpr int NT = kTiledWaves * 64;
  __shared__ KeyTile<DI> tiles[2];

  const int b = blockIdx.z;
  const int64_t nrows = (int64_t)n_q * h_kv;
  const int64_t r0 = (int64_t)blockIdx.y * kTiledRows;
  const int64_t r_end = min(r0 + (int64_t)kTiledRows, nrows);
  const int t_last = (int)((r_end - 1) / h_kv);
  const int jmax = (pos0 + t_last) / kBlock;
  const int jb = blockIdx.x * blocks_per_chunk;
  if (jb > jmax) return;
  const int je = min(jb + blocks_per_chunk, jmax + 1);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, cl = lane & 15;

  // This wave's columns.
  const int64_t rw0 = r0 + (int64_t)wave * kTiledColsPerWave;
  const bool wave_live = rw0 < r_end;
  const int tw0 = wave_live ? (int)(rw0 / h_kv) : 0;
  const int tw1 = wave_live ? (int)((min(rw0 + kTiledColsPerWave, r_end) - 1) / h_kv) : 0;
  const int jw_max = (pos0 + tw1) / kBlock;              // last block any column of the wave needs

  u32x4 qb[8][CC];
  int plim[8];
  bool cvalid[8];
  float* orow[8];
  const uint16_t* kseq = k_idx + (int64_t)b * n_kv * DI;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const int64_t r = rw0 + ct * 16 + cl;
    cvalid[ct] = wave_live && r < r_end;
    const int t = cvalid[ct] ? (int)(r / h_kv) : 0;
    plim[ct] = pos0 + t;
    orow[ct] = bscore + ((int64_t)b * nrows + (cvalid[ct] ? r : 0)) * nblk;
    const uint16_t* qr = q_idx + ((int64_t)b * nrows + r) * DI;
#pragma unroll
    for (int cc = 0; cc < CC; ++cc)
      qb[ct][cc] = cvalid[ct] ? ld16(qr + cc * 32 + q * 8) : u32x4{0u, 0u, 0u, 0u};
  }

  // Key block staging: each thread moves ITEMS 16-byte chunks.
  constexpr int CHUNKS = kBlock * DI / 8;
  constexpr int ITEMS = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile staging must divide evenly");
  u32x4 pre[ITEMS];
  auto fetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int w = tid + i * NT;
      const int key = w / (DI / 8), dc = w % (DI / 8);
      const int s = j * kBlock + key;
      pre[i] = (s < n_kv) ? ld16(kseq + (int64_t)s * DI + dc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stash = [&](KeyTile<DI>& t) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int w = tid + i * NT;
      const int key = w / (DI / 8), dc = w % (DI / 8);
      st16(&t.k[key * KeyTile<DI>::S + dc * 8], pre[i]);
    }
  };

  fetch(jb);
  stash(tiles[0]);
  __syncthreads();

  float wbuf[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) wbuf[ct] = 0.f;

  for (int j = jb; j < je; ++j) {
    const int cur = (j - jb) & 1;
    if (j + 1 < je) fetch(j + 1);
    if (wave_live && j <= jw_max) {
      const KeyTile<DI>& t = tiles[cur];
      const bool need_mask = (j * kBlock + kBlock - 1) > (pos0 + tw0);
      float rm[8];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) rm[ct] = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        f32x4 acc[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < CC; ++cc) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&t.k[(kt * 16 + cl) * KeyTile<DI>::S + cc * 32 + q * 8]);
#pragma unroll
          for (int ct = 0; ct < 8; ++ct) acc[ct] = mfma_16x16x32(a, qb[ct][cc], acc[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = acc[ct][r];
            if (need_mask && (j * kBlock + kt * 16 + q * 4 + r) > plim[ct]) v = -INFINITY;
            rm[ct] = fmaxf(rm[ct], v);
          }
      }
      // Lane group q buffers block jb + 4n + q; every fourth block (or at the
      // end) the four groups write four consecutive blocks of each row.
      const int slot = (j - jb) & 3;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const float m = colgroup_max(rm[ct]) + 0.0f;     // + 0 turns -0 into +0
        if (slot == q) wbuf[ct] = m;
      }
      if (slot == 3 || j == je - 1 || j == jw_max) {
        const int jj = j - slot + q;
        if (jj <= j) {
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
            if (cvalid[ct] && jj * kBlock <= plim[ct]) orow[ct][jj] = wbuf[ct];
        }
      }
    }
    if (j + 1 < je) stash(tiles[cur ^ 1]);
    __syncthreads();
  }
}

// Decode-shaped calls: at most 16 (token, group) rows per sequence.
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyBlocksPerWave = 4;

template <int DI>
__global__ __launch_bounds__(kSkinnyWaves * 64) void index_scores_skinny(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, float* __restrict__ bscore,
    int n_q, int n_kv, int pos0, int h_kv, int nblk) {
  constexpr int CC = DI / 32;
  const int b = blockIdx.y;
  const int nrows = n_q * h_kv;                         // <= 16
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, cl = lane & 15;
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
        rm = fmaxf(rm, v);
      }
    }
    rm = colgroup_max(rm) + 0.0f;
    if (q == 0 && cvalid && j * kBlock <= plim) orow[j] = rm;
  }
}

template <int DI>
hipError_t launch_index_scores_t(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, float* bscore,
                                 hipStream_t stream) {
  const int nblk = d.nblk();
  const int64_t nrows = (int64_t)d.n_q * d.h_kv;
  if (nrows <= 16) {
    const int jmax = (d.pos0 + d.n_q - 1) / kBlock;
    const int per_wg = kSkinnyWaves * kSkinnyBlocksPerWave;
    dim3 grid((jmax + per_wg) / per_wg, d.batch);
    hipLaunchKernelGGL(index_scores_skinny<DI>, grid, dim3(kSkinnyWaves * 64), 0, stream, q_idx, k_idx, bscore,
                       d.n_q, d.n_kv, d.pos0, d.h_kv, nblk);
  } else {
    const int jmax = (d.pos0 + d.n_q - 1) / kBlock;
    const int bpc = jmax >= 512 ? 32 : (jmax >= 128 ? 16 : 4);
    const int64_t tiles = (nrows + kTiledRows - 1) / kTiledRows;
    dim3 grid((jmax + bpc) / bpc, (unsigned)tiles, d.batch);
    hipLaunchKernelGGL(index_scores_tiled<DI>, grid, dim3(kTiledWaves * 64), 0, stream, q_idx, k_idx, bscore,
                       d.n_q, d.n_kv, d.pos0, d.h_kv, nblk, bpc);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, float* bscore,
                               hipStream_t stream) {
  if (d.d_idx == 128) return launch_index_scores_t<128>(d, q_idx, k_idx, bscore, stream);
  return launch_index_scores_t<64>(d, q_idx, k_idx, bscore, stream);
}

}  // namespace msa
