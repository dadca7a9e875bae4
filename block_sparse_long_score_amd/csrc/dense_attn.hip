// Dense causal GQA attention, the comparator MSA is measured against: every
// query head attends to every token s <= its position (hamidun.com news,
// "Como o MSA funciona": the all-to-all attention of standard GQA; Notion notes
// "Minimax-sparse-Attention", "what is MHA, MQA, GQA?": each group of query
// heads shares one K/V head).
//
// Prefill: a workgroup owns 256 (token x group-head) columns of one K/V head,
// keeps their queries in registers and streams the head's 128-token K/V blocks
// through double-buffered LDS with online softmax (flash-attention order), so
// each K/V block is read once per 256 columns; query tiles are paired so every
// workgroup carries the same number of block iterations.
// Decode: the keys are split into chunks of kChunkBlocks blocks; one wave per
// (sequence, group, chunk) streams its chunk from HBM, and the per-chunk
// partials are merged with log-sum-exp weights.
#include <climits>

#include "launch.h"
#include "msa_device.h"

namespace msa {
namespace {

constexpr int kThreads = 256;                          // decode
constexpr int kChunkBlocks = 16;
constexpr int kColsPerWg = 256;                        // prefill: 8 waves x 32 (token, group head) columns

// Prefill.  A workgroup owns 256 (token x group head) columns of one K/V head
// (TQ = 256 / G tokens), keeps their queries in registers and sweeps the
// head's 128-token K/V blocks 0 .. the last token's block with online softmax
// (flash-attention order).  Blocks are double-buffered in LDS: block j + 1 is
// written from registers while block j is in use and block j + 2 is loaded,
// with one barrier per block.  Query tile t needs ~t blocks, so tile t is paired
// with tile T-1-t and one workgroup runs the pair: equal work per workgroup.
template <int D, int LOG2G>
__global__ __launch_bounds__(kKvThreads, 1) void dense_prefill(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               uint16_t* __restrict__ out, float* __restrict__ lse,
                                                               int n_q, int n_kv, int pos0, int h_q, int h_kv,
                                                               int tiles, float sl2) {
  constexpr int G = 1 << LOG2G;
  constexpr int TQ = kColsPerWg >> LOG2G;               // tokens per tile
  __shared__ KVTile<D> tile[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4;
  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t row_stride = (int64_t)h_kv * D;
  const int64_t head0 = ((int64_t)b * n_kv * h_kv + g) * D;
  KVPrefetch<D> pf;

#pragma unroll 1
  for (int seg = 0; seg < 2; ++seg) {
    const int ti = seg == 0 ? tiles - 1 - p : p;
    if (seg == 1 && ti == tiles - 1 - p) break;          // unpaired middle tile
    const int t0 = ti * TQ;
    const int t_last = min(t0 + TQ, n_q) - 1;
    const int jmax = (pos0 + t_last) / kBlock;
    const int twmin = t0 + ((wave * 32) >> LOG2G);
    const int twmax = min(t0 + ((wave * 32 + 31) >> LOG2G), n_q - 1);
    const bool wave_live = twmin < n_q;
    const int jw = wave_live ? (pos0 + twmax) / kBlock : -1;

    const uint16_t* qrow[2];
    int plim[2];
    bool valid[2];
    int64_t orow[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int c = wave * 32 + ct * 16 + (lane & 15);
      const int tt = t0 + (c >> LOG2G), hh = c & (G - 1);
      valid[ct] = tt < n_q;
      orow[ct] = ((int64_t)b * n_q + tt) * h_q + g * G + hh;
      qrow[ct] = valid[ct] ? q + orow[ct] * D : nullptr;
      plim[ct] = valid[ct] ? pos0 + tt : INT_MAX;
    }
    u32x4 qb[2][D / 32];
    load_q_operand<D>(qb, qrow);

    float mref[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
    f32x4 acc[2][D / 32][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int pp = 0; pp < D / 32; ++pp)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[ct][pp][h] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (seg == 1) __syncthreads();                     // the first tile's last block is no longer read
    pf.fetch_buf(k + head0, v + head0, row_stride, 0, n_kv, tid);
    pf.stash(tile[0], tid);
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j <= jmax; ++j) {
      const KVTile<D>& tl = tile[j & 1];
      // Block j + 1's loads are issued after the scores of block j (the
      // kernel's register peak) and are in flight during its P*V.
      const bool live = j <= jw;
      float m_old[2] = {mref[0], mref[1]};
      float bmax[2], bsum[2];
      u32x4 pb[2][4];
      if (live) {
        const bool need_mask = (j * kBlock + kBlock - 1) > (pos0 + twmin);
        block_scores_softmax<D>(tl, qb, sl2, j * kBlock, plim, need_mask, bmax, bsum, pb, mref, true);
      }
      if (j + 1 <= jmax) pf.fetch_buf(k + head0, v + head0, row_stride, (j + 1) * kBlock, n_kv, tid);
      if (live) {
        float alpha[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          alpha[ct] = __builtin_amdgcn_exp2f(m_old[ct] - mref[ct]);   // 0 on the first block
          lrun[ct] = lrun[ct] * alpha[ct] + bsum[ct];
        }
        // The accumulators are rescaled only when some column's running max
        // moved: otherwise every factor is exactly 1.
        if (ballot(m_old[0] != mref[0] || m_old[1] != mref[1])) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int pp = 0; pp < D / 32; ++pp)
#pragma unroll
              for (int h = 0; h < 2; ++h) acc[ct][pp][h] *= alpha[ct];
        }
        block_pv<D>(tl, pb, acc);
      }
      if (j + 1 <= jmax) pf.stash(tile[(j + 1) & 1], tid);   // read last in block j - 1, before the barrier
      __syncthreads();
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      if (!valid[ct]) continue;
      const float inv = 1.f / lrun[ct];
      uint16_t* dst = out + orow[ct] * D;
#pragma unroll
      for (int pp = 0; pp < D / 32; ++pp) {
        const f32x4 a0 = acc[ct][pp][0], a1 = acc[ct][pp][1];
        u32x4 o = {pack_bf16x2(a0[0] * inv, a0[1] * inv), pack_bf16x2(a0[2] * inv, a0[3] * inv),
                   pack_bf16x2(a1[0] * inv, a1[1] * inv), pack_bf16x2(a1[2] * inv, a1[3] * inv)};
        st16(dst + 32 * pp + 8 * q4, o);
      }
      if (lse && q4 == 0) lse[orow[ct]] = (mref[ct] + __log2f(lrun[ct])) * kLn2;
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void dense_decode_chunks(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ part_o, float* __restrict__ part_ml, int n_kv, int pos0, int h_q, int h_kv, int nsplit,
    int64_t units, float sl2) {
  __shared__ float pt[kThreads / 64][kBlock * 16 + 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t unit = (int64_t)blockIdx.x * (kThreads / 64) + wave;   // (b, g, chunk)
  if (unit >= units) return;
  const int split = (int)(unit % nsplit);
  const int64_t bg = unit / nsplit;
  const int g = (int)(bg % h_kv), b = (int)(bg / h_kv);
  const int jl = pos0 / kBlock;
  const int jb = split * kChunkBlocks;
  if (jb > jl) return;
  const int je = min(jb + kChunkBlocks, jl + 1);
  const int64_t head0 = ((int64_t)b * n_kv * h_kv + g) * D;
  decode_attend<D, G>(q + ((int64_t)b * h_q + g * G) * D, k + head0, v + head0, (int64_t)h_kv * D, n_kv, pos0, jb,
                      je, sl2, pt[wave], part_o + unit * G * D, part_ml + unit * G * 2);
}

template <int D, int LOG2G>
hipError_t prefill_t(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v, float sl2,
                     uint16_t* out, float* lse, hipStream_t stream) {
  constexpr int TQ = kColsPerWg >> LOG2G;
  const int tiles = (d.n_q + TQ - 1) / TQ;
  dim3 grid((tiles + 1) / 2, d.h_kv, d.batch);
  {
    LaunchTimer timer("dense_prefill", stream);
    hipLaunchKernelGGL((dense_prefill<D, LOG2G>), grid, dim3(kKvThreads), 0, stream, q, k, v, out, lse, d.n_q,
                       d.n_kv, d.pos0, d.h_q, d.h_kv, tiles, sl2);
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t decode_t(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v, float sl2,
                    uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  const DecodeWs L = dense_decode_ws_layout(d);
  char* base = static_cast<char*>(ws);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(base + L.part_o);
  float* part_ml = reinterpret_cast<float*>(base + L.part_ml);
  const int64_t units = (int64_t)d.batch * d.h_kv * L.nslot;
  {
    LaunchTimer timer("dense_decode_chunks", stream);
    hipLaunchKernelGGL((dense_decode_chunks<D, G>), dim3((unsigned)((units + 3) / 4)), dim3(kThreads), 0, stream, q,
                       k, v, part_o, part_ml, d.n_kv, d.pos0, d.h_q, d.h_kv, L.nslot, units, sl2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(d, part_o, part_ml, nullptr, out, lse, L.nslot, kChunkBlocks, stream);
}

template <int D>
hipError_t prefill_by_group(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v, float sl2,
                            uint16_t* out, float* lse, hipStream_t s) {
  switch (d.group()) {
    case 1: return prefill_t<D, 0>(d, q, k, v, sl2, out, lse, s);
    case 2: return prefill_t<D, 1>(d, q, k, v, sl2, out, lse, s);
    case 4: return prefill_t<D, 2>(d, q, k, v, sl2, out, lse, s);
    case 8: return prefill_t<D, 3>(d, q, k, v, sl2, out, lse, s);
    default: return prefill_t<D, 4>(d, q, k, v, sl2, out, lse, s);
  }
}

template <int D>
hipError_t decode_by_group(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v, float sl2,
                           uint16_t* out, float* lse, void* ws, hipStream_t s) {
  switch (d.group()) {
    case 1: return decode_t<D, 1>(d, q, k, v, sl2, out, lse, ws, s);
    case 2: return decode_t<D, 2>(d, q, k, v, sl2, out, lse, ws, s);
    case 4: return decode_t<D, 4>(d, q, k, v, sl2, out, lse, ws, s);
    case 8: return decode_t<D, 8>(d, q, k, v, sl2, out, lse, ws, s);
    default: return decode_t<D, 16>(d, q, k, v, sl2, out, lse, ws, s);
  }
}

}  // namespace

DecodeWs dense_decode_ws_layout(const Dims& d) {
  DecodeWs L{};
  L.nslot = (d.nblk() + kChunkBlocks - 1) / kChunkBlocks;
  const size_t units = (size_t)d.batch * d.h_kv * L.nslot * d.group();
  size_t o = 0;
  L.part_o = o;
  o = align_up(o + units * d.d * 2, 256);
  L.part_ml = o;
  o = align_up(o + units * 2 * sizeof(float), 256);
  L.total = o;
  return L;
}

hipError_t launch_dense_prefill(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                float scale, uint16_t* out, float* lse, hipStream_t stream) {
  const float sl2 = scale * kLog2e;
  if (d.d == 128) return prefill_by_group<128>(d, q, k, v, sl2, out, lse, stream);
  return prefill_by_group<64>(d, q, k, v, sl2, out, lse, stream);
}

hipError_t launch_dense_decode(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               float scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  const float sl2 = scale * kLog2e;
  if (d.d == 128) return decode_by_group<128>(d, q, k, v, sl2, out, lse, ws, stream);
  return decode_by_group<64>(d, q, k, v, sl2, out, lse, ws, stream);
}

}  // namespace msa
