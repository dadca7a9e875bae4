// Main branch: exact softmax attention of every query head of a GQA group over
// only the blocks its index branch selected (hamidun.com news, "Como o MSA
// funciona": exact attention on the selected blocks only; yhxrc.cn article,
// "第二步：稀疏分支": all heads of a group share the group's selection and the
// attention formula runs unchanged on the real K/V; lefilia.fr article: k blocks
// of 128 tokens per query).
//
// Prefill is KV-outer (lumi-systems summary names a KV-outer sparse attention
// kernel): the selection blk_idx[b][t][g][slot] is inverted into per-(b, g,
// block) lists of (t, slot); one workgroup stages a 128-token K/V block of one
// K/V head in LDS once and runs every (query token x group head) column that
// selected it through MFMA, writing one partial (o, m, l) per
// (t, g, slot, head): o unnormalised (sum of exp2(logit2 - m) * v, bf16), m
// and l.  A merge kernel then combines the <= k partials of each (t, head)
// with log-sum-exp weights.  Every partial is computed from its own
// column only, so the order of a list never changes a result bit.
//
// Decode streams the <= k selected blocks of each (sequence, group) straight
// from HBM, one wave per block, and merges the same way.
#include <algorithm>
#include <climits>

#include "launch.h"
#include "msa_device.h"

namespace msa {
namespace {

int64_t prefill_entries_max(const Dims& d) { return (int64_t)d.batch * d.n_q * d.h_kv * d.topk; }

// ---------------------------------------------------------------- CSR --------
//
// The selection is inverted per (b, g, token chunk): one workgroup counts, in
// an LDS histogram over the blocks, how often each block was selected by the
// chunk's tokens, and later places the chunk's entries through LDS cursors.
// Global memory sees one count per (chunk, list) instead of one atomic per
// selection, and each list comes out ordered by token chunk.

constexpr int kCsrThreads = 256;
constexpr int kCsrMaxBlocks = 8192;                    // nblk <= 8192 (n_kv <= 1M)
constexpr int kCsrTargetChunks = 4096;
constexpr int kCsrMinTokens = 64;

// Token chunks per (b, g): enough to fill the chip with the one-wave fill
// kernel, each of at least kCsrMinTokens tokens.
int csr_chunks(const Dims& d) {
  const int64_t bg = (int64_t)d.batch * d.h_kv;
  if (bg <= 0 || d.n_q <= 0) return 1;
  int64_t c = (kCsrTargetChunks + bg - 1) / bg;
  c = std::max<int64_t>(1, std::min<int64_t>(c, (d.n_q + kCsrMinTokens - 1) / kCsrMinTokens));
  const int64_t tc = (d.n_q + c - 1) / c;
  return (int)((d.n_q + tc - 1) / tc);
}

// Selected, causal block of entry (t, slot) or -1.
__device__ __forceinline__ int entry_block(const int32_t* __restrict__ blk, int64_t row, int slot, int topk, int t,
                                           int pos0) {
  const int j = blk[row * topk + slot];
  return (j >= 0 && j <= (pos0 + t) / kBlock) ? j : -1;
}

// ccnt[(b, g, c)][j] = number of tokens of chunk c (of sequence b, group g)
// that selected block j.
__global__ __launch_bounds__(kCsrThreads) void csr_count_chunks(const int32_t* __restrict__ blk,
                                                                int* __restrict__ ccnt, int n_q, int h_kv, int topk,
                                                                int nblk, int pos0, int tc, int chunks) {
  __shared__ int hist[kCsrMaxBlocks];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t0 = c * tc, t1 = min(n_q, t0 + tc);
  for (int j = threadIdx.x; j < nblk; j += kCsrThreads) hist[j] = 0;
  __syncthreads();
  const int n = (t1 - t0) * topk;
  for (int k = threadIdx.x; k < n; k += kCsrThreads) {
    const int t = t0 + k / topk, slot = k % topk;
    const int j = entry_block(blk, ((int64_t)b * n_q + t) * h_kv + g, slot, topk, t, pos0);
    if (j >= 0) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  int* dst = ccnt + (((int64_t)b * h_kv + g) * chunks + c) * nblk;
  for (int j = threadIdx.x; j < nblk; j += kCsrThreads) dst[j] = hist[j];
}

// Per list (b, g, j): ccnt over the chunks becomes its exclusive prefix, and
// cnt[list] the list's size.
__global__ void csr_chunk_scan(int* __restrict__ ccnt, int* __restrict__ cnt, int lists, int chunks, int nblk) {
  const int list = blockIdx.x * blockDim.x + threadIdx.x;
  if (list >= lists) return;
  const int bg = list / nblk, j = list % nblk;
  int* col = ccnt + (int64_t)bg * chunks * nblk + j;
  int run = 0;
  for (int c0 = 0; c0 < chunks; c0 += 8) {             // eight loads in flight
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = c0 + i < chunks ? col[(int64_t)(c0 + i) * nblk] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (c0 + i < chunks) col[(int64_t)(c0 + i) * nblk] = run;
      run += v[i];
    }
  }
  cnt[list] = run;
}

// One workgroup: exclusive scan of the list sizes; off[lists] = all entries.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void csr_scan(const int* __restrict__ cnt, int* __restrict__ off,
                                                        int lists) {
  __shared__ int s_e[kScanThreads];
  const int tid = threadIdx.x;
  const int per = (lists + kScanThreads - 1) / kScanThreads;
  const int lo = min(lists, tid * per), hi = min(lists, lo + per);
  int se = 0;
  for (int i = lo; i < hi; ++i) se += cnt[i];
  s_e[tid] = se;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {         // inclusive Hillis-Steele scan
    const int ae = tid >= o ? s_e[tid - o] : 0;
    __syncthreads();
    s_e[tid] += ae;
    __syncthreads();
  }
  int re = s_e[tid] - se;                              // exclusive prefix of this thread's range
  for (int i = lo; i < hi; ++i) {
    off[i] = re;
    re += cnt[i];
  }
  if (tid == kScanThreads - 1) off[lists] = s_e[tid];
}

// Unordered fill, for callers whose results do not depend on the order inside
// a list (the forward: every partial comes from its own column): entries of
// chunk c go to off[list] + (prefix of earlier chunks) + a rank taken from an
// LDS cursor.
__global__ __launch_bounds__(kCsrThreads) void csr_fill_any(const int32_t* __restrict__ blk,
                                                            const int* __restrict__ off,
                                                            const int* __restrict__ ccnt,
                                                            int* __restrict__ entries, int n_q, int h_kv, int topk,
                                                            int nblk, int pos0, int tc, int chunks) {
  __shared__ int cur[kCsrMaxBlocks];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t0 = c * tc, t1 = min(n_q, t0 + tc);
  const int* pre = ccnt + (((int64_t)b * h_kv + g) * chunks + c) * nblk;
  const int* loff = off + ((int64_t)b * h_kv + g) * nblk;
  for (int j = threadIdx.x; j < nblk; j += kCsrThreads) cur[j] = loff[j] + pre[j];
  __syncthreads();
  const int n = (t1 - t0) * topk;
  for (int k = threadIdx.x; k < n; k += kCsrThreads) {
    const int t = t0 + k / topk, slot = k % topk;
    const int j = entry_block(blk, ((int64_t)b * n_q + t) * h_kv + g, slot, topk, t, pos0);
    if (j >= 0) entries[atomicAdd(&cur[j], 1)] = (t << kSlotBits) | slot;
  }
}

// Entries of chunk c go to off[list] + (prefix of earlier chunks) + their rank
// among the chunk's entries of that list in (token, slot) order.  One wave per
// chunk: its lanes take the chunk's items in rounds of 64 (64 / T tokens, T =
// topk rounded up to a power of two, lane = token * T + slot); an entry's
// position is the list cursor plus the number of the round's entries before it
// with the same block, and the round's last such entry advances the cursor.
// A single wave's LDS operations complete in issue order, so no barrier is
// needed; the selections of four rounds are loaded together.  Every list is therefore ordered by token and slot whatever the
// scheduling, so a kernel that accumulates over a list in list order gives the
// same bits on every run.
constexpr int kFillThreads = 64;
constexpr int kFillBatch = 4;
__global__ __launch_bounds__(kFillThreads) void csr_fill_chunks(const int32_t* __restrict__ blk,
                                                                const int* __restrict__ off,
                                                                const int* __restrict__ ccnt,
                                                                int* __restrict__ entries, int n_q, int h_kv,
                                                                int topk, int nblk, int pos0, int tc, int chunks) {
  extern __shared__ int cur[];                         // [nblk]
  __shared__ __attribute__((aligned(16))) int sel[kFillThreads];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int t0 = c * tc, t1 = min(n_q, t0 + tc);
  const int* pre = ccnt + (((int64_t)b * h_kv + g) * chunks + c) * nblk;
  const int* loff = off + ((int64_t)b * h_kv + g) * nblk;
  for (int j = lane; j < nblk; j += kFillThreads) cur[j] = loff[j] + pre[j];
  int T = 1;
  while (T < topk) T <<= 1;
  const int tpr = kFillThreads / T, tl = lane / T, slot = lane % T;
  auto load_j = [&](int tb) {
    const int t = tb + tl;
    return (t < t1 && slot < topk) ? entry_block(blk, ((int64_t)b * n_q + t) * h_kv + g, slot, topk, t, pos0) : -1;
  };
  // Rounds go in batches of kFillBatch whose selections are loaded together:
  // one wait per batch (the wait also covers the batch's entry stores).
  for (int tb0 = t0; tb0 < t1; tb0 += kFillBatch * tpr) {
    int jb[kFillBatch];
#pragma unroll
    for (int r = 0; r < kFillBatch; ++r) jb[r] = load_j(tb0 + r * tpr);
#pragma unroll
    for (int r = 0; r < kFillBatch; ++r) {
      const int tb = tb0 + r * tpr, j = jb[r];
      sel[lane] = j;
      int rank = 0;
      bool last = true;
#pragma unroll
      for (int q = 0; q < kFillThreads / 4; ++q) {
        const int4 r4 = reinterpret_cast<const int4*>(sel)[q];
        const int v[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool same = v[e] == j;
          rank += (same && 4 * q + e < lane) ? 1 : 0;
          last = last && !(same && 4 * q + e > lane);
        }
      }
      if (j >= 0) {
        const int pos = cur[j] + rank;
        entries[pos] = ((tb + tl) << kSlotBits) | slot;   // slot < 64, t < 2^25
      }
      __builtin_amdgcn_wave_barrier();
      if (j >= 0 && last) cur[j] += rank + 1;          // after every lane has read its cursor
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// --------------------------------------------------------- KV-outer ---------
//
// Persistent: one 8-wave workgroup per CU takes an equal, contiguous range of
// the list entries (lists are consecutive in `entries`, in (b, g, block)
// order), so it walks a few dozen lists one after the other.  A list's K/V
// block is staged in LDS once for the whole segment of the list the range
// covers; the next list's block is loaded into registers while the current
// segment computes and is written to the other LDS buffer before the switch.
// Within a segment, waves take 32-column groups (column = entry x group head)
// round-robin and load the next group's queries and entries while computing.

// The list holding entry e: the first list L' > L whose range ends past e
// (off is nondecreasing; empty lists are stepped over 64 at a time).
__device__ __forceinline__ int next_list(const int* __restrict__ off, int lists, int L, int e) {
  for (int base = L + 1;; base += 64) {
    const int cand = base + lane_id();
    const uint64_t m = ballot(cand < lists && off[cand + 1] > e);
    if (m) return base + __builtin_ctzll(m);
  }
}

template <int D, int LOG2G>
__global__ __launch_bounds__(kKvThreads, 1) void sparse_kv_outer(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int* __restrict__ off, const int* __restrict__ entries, uint16_t* __restrict__ part_o,
    float* __restrict__ part_ml, int64_t sink_row, int n_q, int n_kv, int pos0, int h_q, int h_kv, int nblk,
    int topk, int lists, float sl2) {
  constexpr int G = 1 << LOG2G;
  constexpr int NW = kKvThreads / 64;
  __shared__ KVTile<D> tile[2];
  const int tid = threadIdx.x, lane = tid & 63, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int total = off[lists];
  const int lo = (int)((int64_t)total * blockIdx.x / gridDim.x);
  const int hi = (int)((int64_t)total * (blockIdx.x + 1) / gridDim.x);
  if (lo >= hi) return;
  int L;                                               // list holding entry lo: last L with off[L] <= lo
  {
    int a = 0, z = lists - 1;
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (off[mid] <= lo) a = mid; else z = mid - 1;
    }
    L = a;
    while (off[L + 1] <= lo) ++L;                      // step over empty lists sharing the offset
  }
  const int64_t row_stride = (int64_t)h_kv * D;
  auto block_base = [&](int list, const uint16_t* base) {
    const int bg = list / nblk;
    return base + ((int64_t)(bg / h_kv) * n_kv * h_kv + bg % h_kv) * D;
  };
  KVPrefetch<D> pf;
  pf.fetch(block_base(L, k), block_base(L, v), row_stride, (L % nblk) * kBlock, n_kv, tid);
  pf.stash(tile[0], tid);
  __syncthreads();
  int buf = 0;
  int seg_end = min(hi, off[L + 1]);
  int Ln = seg_end < hi ? next_list(off, lists, L, seg_end) : -1;
  if (Ln >= 0) pf.fetch(block_base(Ln, k), block_base(Ln, v), row_stride, (Ln % nblk) * kBlock, n_kv, tid);

  // Column (token, head) bookkeeping of one 32-column group.  Columns past a
  // segment's end read a clamped entry and write their partial to the sink
  // row, so that no load or store of the loop sits behind a per-lane branch:
  // the compiler then counts outstanding memory operations exactly, and the
  // wait for a group's entries or queries never includes the partial stores
  // issued after them.
  struct Cols {
    const uint16_t* qrow[2];
    int plim[2];
    int64_t prow[2];
    bool mask_any;
  };
#pragma unroll 1
  for (;;) {
    const int j = L % nblk, bg = L / nblk;
    const int g = bg % h_kv, b = bg / h_kv;
    const int s0 = j * kBlock;
    const int ea = max(lo, off[L]), eb = seg_end;      // this segment's entries
    const int ngroups = (((eb - ea) << LOG2G) + 31) >> 5;
    auto entry_of = [&](int cg, int ct) { return ea + ((cg * 32 + ct * 16 + (lane & 15)) >> LOG2G); };
    auto load_entries = [&](int cg, int (&en)[2]) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) en[ct] = entries[min(entry_of(cg, ct), eb - 1)];
    };
    auto describe = [&](int cg, const int (&en)[2], Cols& c) {
      c.mask_any = false;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bool valid = entry_of(cg, ct) < eb;
        const int hh = (cg * 32 + ct * 16 + (lane & 15)) & (G - 1);
        const int t = entry_token(en[ct]), slot = entry_slot(en[ct]);
        const int p = pos0 + t;
        c.qrow[ct] = q + (((int64_t)b * n_q + t) * h_q + g * G + hh) * D;
        c.plim[ct] = valid ? p : INT_MAX;
        c.prow[ct] = valid ? ((((int64_t)b * n_q + t) * h_kv + g) * topk + slot) * G + hh : sink_row + hh;
        c.mask_any |= valid && (p < s0 + kBlock - 1);
      }
    };
    const KVTile<D>& tl = tile[buf];
    auto load_q = [&](const Cols& c, u32x4 (&qv)[2][D / 32]) {   // unconditional: every qrow is a real row
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int cc = 0; cc < D / 32; ++cc) qv[ct][cc] = ld16(c.qrow[ct] + cc * 32 + q4 * 8);
    };
    Cols cur_c, nxt_c;
    u32x4 qb[2][D / 32], qn[2][D / 32];
    int en1[2];
    int cg = wave;
    if (cg < ngroups) {
      int en0[2];
      load_entries(cg, en0);
      describe(cg, en0, cur_c);
      load_q(cur_c, qb);
      load_entries(min(cg + NW, ngroups - 1), en1);
    }
    // Drain the memory counters once per segment: the loop header then sees
    // only the loop's own outstanding operations, and the compiler can wait
    // for each prefetch by count instead of draining every iteration.
    __builtin_amdgcn_s_waitcnt(0);
    // Straight-line body: the prefetches of the last iterations re-read the
    // segment's last group (clamped) and are not used.
#pragma unroll 1
    for (; cg < ngroups; cg += NW) {
      const int cn = min(cg + NW, ngroups - 1);
      describe(cn, en1, nxt_c);                        // queries of the next group (entries loaded a group ago)
      load_q(nxt_c, qn);
      const bool need_mask = ballot(cur_c.mask_any) != 0ull;
      float bmax[2], bsum[2], mref[2] = {0.f, 0.f};
      u32x4 pb[2][4];
      block_scores_softmax<D>(tl, qb, sl2, s0, cur_c.plim, need_mask, bmax, bsum, pb, mref, false);
      f32x4 acc[2][D / 32][2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int pp = 0; pp < D / 32; ++pp)
#pragma unroll
          for (int h = 0; h < 2; ++h) acc[ct][pp][h] = f32x4{0.f, 0.f, 0.f, 0.f};
      block_pv<D>(tl, pb, acc);
      // Entries of the group after next, issued before this group's stores.
      load_entries(min(cg + 2 * NW, ngroups - 1), en1);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        uint16_t* dst = part_o + cur_c.prow[ct] * D;
#pragma unroll
        for (int pp = 0; pp < D / 32; ++pp) {
          const f32x4 a0 = acc[ct][pp][0], a1 = acc[ct][pp][1];
          u32x4 o = {pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]), pack_bf16x2(a1[0], a1[1]),
                     pack_bf16x2(a1[2], a1[3])};
          st16(dst + 32 * pp + 8 * q4, o);
        }
        // (m, l) is replicated over the column's four lane groups; all store it.
        *reinterpret_cast<float2*>(part_ml + 2 * cur_c.prow[ct]) = make_float2(bmax[ct], bsum[ct]);
      }
      cur_c = nxt_c;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int cc = 0; cc < D / 32; ++cc) qb[ct][cc] = qn[ct][cc];
    }
    if (Ln < 0) break;
    // The other buffer was last read before the previous switch's barrier.
    pf.stash(tile[buf ^ 1], tid);
    __syncthreads();
    buf ^= 1;
    L = Ln;
    seg_end = min(hi, off[L + 1]);
    Ln = seg_end < hi ? next_list(off, lists, L, seg_end) : -1;
    if (Ln >= 0) pf.fetch(block_base(Ln, k), block_base(Ln, v), row_stride, (Ln % nblk) * kBlock, n_kv, tid);
  }
}

// ------------------------------------------------------------ decode -------
//
// One workgroup of four waves per (sequence, group, run of four selection
// slots), one wave per selected block.  A wave requests its query heads and
// the block's 128 keys at once, forms S^T = K Q^T on MFMA, then requests the
// 128 values (into the key registers, now free) while the softmax runs, and
// accumulates P V on the vector ALUs; at about 210 registers two waves fit per
// SIMD, so one workgroup's loads overlap another's arithmetic.  The four
// waves' results are merged in LDS into one partial (o unnormalised, m, l) per
// head, so the merge kernel combines ceil(topk / 4) partials per (sequence,
// head).  (Splitting a block over two waves measured slower at 64 sequences x
// 256K: 145 against 113 us.)

constexpr int kDecSlots = 4;                           // selection slots per workgroup
constexpr int kDecWavesPerBlock = 1;
constexpr int kDecWaves = kDecWavesPerBlock * kDecSlots;
constexpr int kDecKeys = kBlock / kDecWavesPerBlock;   // keys per wave

template <int D, int G>
__global__ __launch_bounds__(kDecWaves * 64) void sparse_decode_blocks(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ blk, uint16_t* __restrict__ part_o, float* __restrict__ part_ml, int n_kv, int pos0,
    int h_q, int h_kv, int topk, int nsub, float sl2, const int* __restrict__ seq_len) {
  constexpr int CC = D / 32;                           // 32-wide contraction chunks of a key
  constexpr int KT = kDecKeys / 16;                    // 16-key MFMA tiles per wave
  constexpr int LPR = D / 8;                           // lanes per V row (16-byte pieces)
  constexpr int KPI = 64 / LPR;                        // keys per V load instruction
  constexpr int VI = kDecKeys / KPI;                   // V loads per lane
  __shared__ float pt[kDecWaves][kDecKeys * 16];       // P[key][head] per wave
  __shared__ float so[kDecWaves][G * D];               // each wave's unnormalised o
  __shared__ float sml[kDecWaves][2 * G];              // each wave's (m, l) per head
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t unit = blockIdx.x;                     // (b, g, run of four slots)
  const int sub = (int)(unit % nsub);
  const int64_t bg = unit / nsub;
  const int g = (int)(bg % h_kv), b = (int)(bg / h_kv);
  const int p = seq_pos0(seq_len, b, pos0, 1, n_kv);
  const int slot = sub * kDecSlots + wave / kDecWavesPerBlock;
  const int j = __builtin_amdgcn_readfirstlane(slot < topk ? blk[bg * topk + slot] : -1);
  const int s0 = j * kBlock + (wave % kDecWavesPerBlock) * kDecKeys;   // this wave's first key
  const int col = lane & 15, q4 = lane >> 4;
  const int kg = lane / LPR, dl = lane % LPR;
  // wave-uniform: a selected, causal block whose part holds a visible key
  if (j >= 0 && j <= p / kBlock && s0 <= p) {
    const int64_t rs = (int64_t)h_kv * D;
    const int64_t head0 = ((int64_t)b * n_kv * h_kv + g) * D;
    const uint16_t* kb = k + head0;
    const uint16_t* vb = v + head0;
    const uint16_t* qh = q + ((int64_t)b * h_q + g * G) * D;
    u32x4 qb[CC], a[KT][CC], vv[VI];
#pragma unroll
    for (int cc = 0; cc < CC; ++cc) qb[cc] = (col < G) ? ld16(qh + col * D + cc * 32 + q4 * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int s = s0 + kt * 16 + col;
#pragma unroll
      for (int cc = 0; cc < CC; ++cc)
        a[kt][cc] = (s < n_kv) ? ld16(kb + (int64_t)s * rs + cc * 32 + q4 * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 sc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) sc[kt] = mfma_16x16x32(a[kt][cc], qb[cc], sc[kt]);
    }
    // The values are requested once the keys are consumed and arrive while
    // the softmax runs.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int it = 0; it < VI; ++it) {
      const int s = s0 + it * KPI + kg;
      vv[it] = (s < n_kv) ? ld16(vb + (int64_t)s * rs + dl * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = (s0 + kt * 16 + q4 * 4 + r > p) ? -INFINITY : sc[kt][r] * sl2;
        sc[kt][r] = x;
        mx = vmax(mx, x);
      }
    mx = colgroup_max(mx);                             // finite: key s0 <= p is visible
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(sc[kt][r] - mx);
        sum += e;
        if (col < G) pt[wave][(kt * 16 + q4 * 4 + r) * 16 + col] = e;
      }
    sum = colgroup_sum(sum);
    if (q4 == 0 && col < G) {
      sml[wave][col] = mx;
      sml[wave][G + col] = sum;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P V: lane (kg, dl) owns d = 8 dl .. 8 dl + 7 for keys kg, kg + KPI, ...
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int it = 0; it < VI; ++it) {
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_to_f32(vv[it][e] & 0xffffu);
        vf[2 * e + 1] = bf16_to_f32(vv[it][e] >> 16);
      }
      const float* prow = &pt[wave][(it * KPI + kg) * 16];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pr = prow[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[h][e];
#pragma unroll
        for (int m = LPR; m < 64; m <<= 1) x += shfl_xor_f(x, m);
        acc[h][e] = x;
      }
    if (kg == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        *reinterpret_cast<f32x4*>(&so[wave][h * D + dl * 8]) = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
        *reinterpret_cast<f32x4*>(&so[wave][h * D + dl * 8 + 4]) = f32x4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
      }
    }
  } else {                                             // padding, a block past the query, or an all-future part
    if (lane < G) {
      sml[wave][lane] = -INFINITY;
      sml[wave][G + lane] = 0.f;
    }
  }
  __syncthreads();
  // Merge the waves: thread t takes elements t, t + 64 kDecWaves, ... of [G][D].
  for (int e = threadIdx.x; e < G * D; e += kDecWaves * 64) {
    const int h = e / D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = vmax(M, sml[w][h]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float m = sml[w][h];
      if (m != -INFINITY) {                            // only waves that attended keys wrote so[w]
        const float wt = __builtin_amdgcn_exp2f(m - M);
        L = fmaf(wt, sml[w][G + h], L);
        o = fmaf(wt, so[w][e], o);
      }
    }
    part_o[unit * G * D + e] = (uint16_t)(pack_bf16x2(o, 0.f) & 0xffffu);
    if (e % D == 0) *reinterpret_cast<float2*>(part_ml + 2 * (unit * G + h)) = make_float2(M, L);
  }
}

// ------------------------------------------------------------- merge --------

// Slot s of a row takes part when it holds a result: for the sparse prefill
// when blk[.., s] is a block index in [0, jl]; for split dense decode (blk ==
// nullptr, per > 0) when s * per <= jl; for sparse decode (blk == nullptr, per
// == 0) when its m is finite.  With M the largest partial max and
// w_s = exp2(m_s - M):
// out = sum_s w_s o_s / sum_s w_s l_s  (o_s unnormalised), lse = ln2 (M + log2 L).
template <int D>
__global__ __launch_bounds__(256) void merge_partials(const uint16_t* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      const int32_t* __restrict__ blk, uint16_t* __restrict__ out,
                                                      float* __restrict__ lse, int64_t nrows, int n_q, int pos0,
                                                      int h_q, int G, int nslot, int per, int n_kv,
                                                      const int* __restrict__ seq_len) {
  constexpr int TPR = D / 8;                           // threads per (token, head) row
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;   // (b * n_q + t) * h_q + h
  if (row >= nrows) return;
  const int dl = threadIdx.x % TPR;
  const int h = (int)(row % h_q);
  const int64_t bt = row / h_q;
  const int t = (int)(bt % n_q);
  const int g = h / G, hh = h % G;
  const int h_kv = h_q / G;
  const int jl = (seq_pos0(seq_len, (int)(bt / n_q), pos0, n_q, n_kv) + t) / kBlock;
  const int64_t unit0 = (bt * h_kv + g) * nslot;
  const int32_t* brow = blk ? blk + unit0 : nullptr;
  // One pass with a running maximum: slots go in batches of 8, each thread
  // keeping 8 (m, l) pairs and 8 16-byte loads of o in flight.  Every slot is
  // loaded (address clamped into the row) and dead ones are dropped with
  // selects only: their memory may hold anything, and the branch-per-slot form
  // of such a loop was miscompiled by the gfx950 toolchain (wrong sums for
  // rows with dead slots).
  float M = -INFINITY, L = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < nslot; s0 += 8) {
    u32x4 o[8];
    float mv[8], lv[8];
    bool on[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = min(s0 + i, nslot - 1);
      const int j = brow ? brow[s] : s * per;
      const int64_t pr = (unit0 + s) * G + hh;
      const float2 ml = *reinterpret_cast<const float2*>(part_ml + 2 * pr);
      mv[i] = ml.x;
      lv[i] = ml.y;
      on[i] = (s0 + i < nslot) && j >= 0 && j <= jl && (brow || per > 0 || ml.x != -INFINITY);
      o[i] = ld16(part_o + pr * D + dl * 8);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) bm = on[i] ? vmax(bm, mv[i]) : bm;
    const float Mn = vmax(M, bm);
    // Mn = -inf only while every slot so far is dead; then nothing is added.
    const float scale = Mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(M - Mn);
    L *= scale;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= scale;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float w = on[i] ? __builtin_amdgcn_exp2f(mv[i] - Mn) : 0.f;
      L = fmaf(w, on[i] ? lv[i] : 0.f, L);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t ov = on[i] ? o[i][e] : 0u;
        acc[2 * e] = fmaf(w, bf16_to_f32(ov & 0xffffu), acc[2 * e]);
        acc[2 * e + 1] = fmaf(w, bf16_to_f32(ov >> 16), acc[2 * e + 1]);
      }
    }
    M = Mn;
  }
  const float inv = 1.f / L;
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  st16(out + row * D + dl * 8, r);
  if (lse && dl == 0) lse[row] = (M + __log2f(L)) * kLn2;
}

template <int D>
hipError_t launch_merge_t(const Dims& d, const uint16_t* part_o, const float* part_ml, const int32_t* blk,
                          uint16_t* out, float* lse, int nslot, int per, hipStream_t stream) {
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_q;
  const int rows_per_wg = 256 / (D / 8);
  const int64_t wgs = (nrows + rows_per_wg - 1) / rows_per_wg;
  {
    LaunchTimer timer("merge_partials", stream);
    hipLaunchKernelGGL(merge_partials<D>, dim3((unsigned)wgs), dim3(256), 0, stream, part_o, part_ml, blk, out, lse,
                       nrows, d.n_q, d.pos0, d.h_q, d.group(), nslot, per, d.n_kv, d.seq_len);
  }
  return hipGetLastError();
}

// ------------------------------------------------- index-branch target ------

// Notion notes "Minimax-sparse-Attention", "KL Loss Alignment": the main
// branch's attention distribution over blocks is the target the index branch
// imitates.  For one (b, t, g) row, R lanes hold its slots.  Head h's mass on
// slot s is w_hs / L_h with w_hs = exp2(m_hs - M_h) l_hs, M_h the largest
// partial maximum and L_h = sum_s w_hs, read from the sparse prefill's
// partials (m in log2 units, l the partial normaliser); the target is the mean
// over the group's G heads.  The index distribution is a softmax of
// idx_scale * bscore over the same live slots, and kl = sum_s target_s
// (ln target_s - ln index_s), 0 ln 0 = 0.  A slot is live when blk holds a
// block in [0, jl]; dead slots get target 0 and take no part.
template <int G, int R>
__global__ __launch_bounds__(256) void block_target_kl(const float* __restrict__ part_ml,
                                                       const int32_t* __restrict__ blk,
                                                       const float* __restrict__ bscore, float* __restrict__ target,
                                                       float* __restrict__ kl, int64_t nrows, int n_q, int h_kv,
                                                       int pos0, int topk, int nblk, float idx_sl2) {
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / R;   // (b * n_q + t) * h_kv + g
  const int s = threadIdx.x % R;
  const int64_t rr = row < nrows ? row : nrows - 1;      // idle lanes of the last wave read a real row
  const int t = (int)((rr / h_kv) % n_q);
  const int jl = (pos0 + t) / kBlock;
  const int sc = min(s, topk - 1);
  const int j = blk[rr * topk + sc];
  const bool on = s < topk && j >= 0 && j <= jl;
  const auto fmax = [](float x, float y) { return vmax(x, y); };
  const auto fadd = [](float x, float y) { return x + y; };
  // (m, l) of the G heads of this slot: 8 G contiguous bytes
  float mv[G], lv[G];
  const float* ml = part_ml + (rr * topk + sc) * G * 2;
  if constexpr (G == 1) {
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    const f32x2 v = *reinterpret_cast<const f32x2*>(ml);
    mv[0] = v[0];
    lv[0] = v[1];
  } else {
#pragma unroll
    for (int h = 0; h < G; h += 2) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(ml + 2 * h);
      mv[h] = v[0];
      lv[h] = v[1];
      mv[h + 1] = v[2];
      lv[h + 1] = v[3];
    }
  }
  const float a = on ? bscore[rr * nblk + (on ? j : 0)] * idx_sl2 : -INFINITY;   // log2 units
  float mass = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = on ? mv[h] : -INFINITY;
    const float M = row_reduce<R>(m, fmax);
    const float w = on ? __builtin_amdgcn_exp2f(m - M) * lv[h] : 0.f;
    const float L = row_reduce<R>(w, fadd);
    mass += L > 0.f ? w / L : 0.f;
  }
  const float tg = mass * (1.f / G);
  const float A = row_reduce<R>(a, fmax);
  const float e = on ? __builtin_amdgcn_exp2f(a - A) : 0.f;
  const float Z = row_reduce<R>(e, fadd);
  const float term = (on && tg > 0.f) ? tg * (__log2f(tg) - (a - A - __log2f(Z))) : 0.f;
  const float k2 = row_reduce<R>(term, fadd);
  if (row < nrows) {
    if (s < topk) target[row * topk + s] = on ? tg : 0.f;
    if (s == 0) kl[row] = k2 * kLn2;
  }
}

template <int G>
hipError_t launch_target_t(const Dims& d, const float* part_ml, const int32_t* blk, const float* bscore,
                           float idx_scale, float* target, float* kl, hipStream_t stream) {
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_kv;
  const int R = d.topk > 32 ? 64 : d.topk > 16 ? 32 : 16;
  const int64_t wgs = (nrows * R + 255) / 256;
  LaunchTimer timer("block_target_kl", stream);
  if (R == 16)
    hipLaunchKernelGGL((block_target_kl<G, 16>), dim3((unsigned)wgs), dim3(256), 0, stream, part_ml, blk, bscore,
                       target, kl, nrows, d.n_q, d.h_kv, d.pos0, d.topk, d.nblk(), idx_scale * kLog2e);
  else if (R == 32)
    hipLaunchKernelGGL((block_target_kl<G, 32>), dim3((unsigned)wgs), dim3(256), 0, stream, part_ml, blk, bscore,
                       target, kl, nrows, d.n_q, d.h_kv, d.pos0, d.topk, d.nblk(), idx_scale * kLog2e);
  else
    hipLaunchKernelGGL((block_target_kl<G, 64>), dim3((unsigned)wgs), dim3(256), 0, stream, part_ml, blk, bscore,
                       target, kl, nrows, d.n_q, d.h_kv, d.pos0, d.topk, d.nblk(), idx_scale * kLog2e);
  return hipGetLastError();
}

template <int D, int LOG2G>
hipError_t launch_prefill_t(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* blk, float sl2, uint16_t* out, float* lse, void* ws,
                            hipStream_t stream) {
  const PrefillWs L = prefill_ws_layout(d);
  char* base = static_cast<char*>(ws);
  const int* off = reinterpret_cast<const int*>(base + L.off);
  const int* entries = reinterpret_cast<const int*>(base + L.entries);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(base + L.part_o);
  float* part_ml = reinterpret_cast<float*>(base + L.part_ml);
  const int nblk = d.nblk();
  const int lists = (int)L.lists;
  hipError_t e = launch_csr(d, blk, ws, stream, false);   // partials do not depend on list order
  if (e != hipSuccess) return e;
  {
    LaunchTimer timer("sparse_kv_outer", stream);
    hipLaunchKernelGGL((sparse_kv_outer<D, LOG2G>), dim3((unsigned)device_cu_count()), dim3(kKvThreads), 0, stream,
                       q, k, v, off, entries, part_o, part_ml, L.entries_max * d.group(), d.n_q, d.n_kv, d.pos0,
                       d.h_q, d.h_kv, nblk, d.topk, lists, sl2);
  }
  return launch_merge_t<D>(d, part_o, part_ml, blk, out, lse, d.topk, 1, stream);
}

template <int D, int G>
hipError_t launch_decode_t(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* blk, float sl2, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
  const DecodeWs L = sparse_decode_ws_layout(d);
  char* base = static_cast<char*>(ws);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(base + L.part_o);
  float* part_ml = reinterpret_cast<float*>(base + L.part_ml);
  const int64_t wgs = (int64_t)d.batch * d.h_kv * L.nslot;
  {
    LaunchTimer timer("sparse_decode_blocks", stream);
    hipLaunchKernelGGL((sparse_decode_blocks<D, G>), dim3((unsigned)wgs), dim3(kDecWaves * 64), 0, stream, q, k, v,
                       blk, part_o, part_ml, d.n_kv, d.pos0, d.h_q, d.h_kv, d.topk, L.nslot, sl2, d.seq_len);
  }
  // One partial per run of four slots; a run without a selected causal block has m = -inf.
  return launch_merge_t<D>(d, part_o, part_ml, nullptr, out, lse, L.nslot, 0, stream);
}

template <int D>
hipError_t prefill_by_group(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* blk, float sl2, uint16_t* out, float* lse, void* ws, hipStream_t s) {
  switch (d.group()) {
    case 1: return launch_prefill_t<D, 0>(d, q, k, v, blk, sl2, out, lse, ws, s);
    case 2: return launch_prefill_t<D, 1>(d, q, k, v, blk, sl2, out, lse, ws, s);
    case 4: return launch_prefill_t<D, 2>(d, q, k, v, blk, sl2, out, lse, ws, s);
    case 8: return launch_prefill_t<D, 3>(d, q, k, v, blk, sl2, out, lse, ws, s);
    default: return launch_prefill_t<D, 4>(d, q, k, v, blk, sl2, out, lse, ws, s);
  }
}

template <int D>
hipError_t decode_by_group(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* blk, float sl2, uint16_t* out, float* lse, void* ws, hipStream_t s) {
  switch (d.group()) {
    case 1: return launch_decode_t<D, 1>(d, q, k, v, blk, sl2, out, lse, ws, s);
    case 2: return launch_decode_t<D, 2>(d, q, k, v, blk, sl2, out, lse, ws, s);
    case 4: return launch_decode_t<D, 4>(d, q, k, v, blk, sl2, out, lse, ws, s);
    case 8: return launch_decode_t<D, 8>(d, q, k, v, blk, sl2, out, lse, ws, s);
    default: return launch_decode_t<D, 16>(d, q, k, v, blk, sl2, out, lse, ws, s);
  }
}

}  // namespace

hipError_t launch_csr(const Dims& d, const int32_t* blk, void* ws, hipStream_t stream, bool ordered) {
  const PrefillWs L = prefill_ws_layout(d);
  char* base = static_cast<char*>(ws);
  int* cnt = reinterpret_cast<int*>(base + L.cnt);
  int* off = reinterpret_cast<int*>(base + L.off);
  int* ccnt = reinterpret_cast<int*>(base + L.ccnt);
  int* entries = reinterpret_cast<int*>(base + L.entries);
  const int nblk = d.nblk();
  const int lists = (int)L.lists;
  const int chunks = (int)L.chunks;
  const int tc = (d.n_q + chunks - 1) / chunks;
  const dim3 cgrid((unsigned)chunks, (unsigned)d.h_kv, (unsigned)d.batch);
  {
    LaunchTimer timer("csr_count_chunks", stream);
    hipLaunchKernelGGL(csr_count_chunks, cgrid, dim3(kCsrThreads), 0, stream, blk, ccnt, d.n_q, d.h_kv, d.topk, nblk,
                       d.pos0, tc, chunks);
  }
  {
    LaunchTimer timer("csr_chunk_scan", stream);
    hipLaunchKernelGGL(csr_chunk_scan, dim3((unsigned)((lists + 255) / 256)), dim3(256), 0, stream, ccnt, cnt, lists,
                       chunks, nblk);
  }
  {
    LaunchTimer timer("csr_scan", stream);
    hipLaunchKernelGGL(csr_scan, dim3(1), dim3(kScanThreads), 0, stream, cnt, off, lists);
  }
  if (ordered) {
    LaunchTimer timer("csr_fill_chunks", stream);
    hipLaunchKernelGGL(csr_fill_chunks, cgrid, dim3(kFillThreads), (unsigned)(nblk * sizeof(int)), stream, blk, off,
                       ccnt, entries, d.n_q, d.h_kv, d.topk, nblk, d.pos0, tc, chunks);
  } else {
    LaunchTimer timer("csr_fill_any", stream);
    hipLaunchKernelGGL(csr_fill_any, cgrid, dim3(kCsrThreads), 0, stream, blk, off, ccnt, entries, d.n_q, d.h_kv,
                       d.topk, nblk, d.pos0, tc, chunks);
  }
  return hipGetLastError();
}

PrefillWs prefill_ws_layout(const Dims& d) {
  PrefillWs L{};
  L.lists = (int64_t)d.batch * d.h_kv * d.nblk();
  L.entries_max = prefill_entries_max(d);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  L.cnt = take(sizeof(int) * L.lists);
  L.off = take(sizeof(int) * (L.lists + 1));
  L.chunks = csr_chunks(d);
  L.ccnt = take(sizeof(int) * (size_t)L.lists * L.chunks);
  L.entries = take(sizeof(int) * L.entries_max);
  // partials per (entry, head), plus one sink row of G heads for idle columns
  L.part_o = take((size_t)(L.entries_max + 1) * d.group() * d.d * 2);
  L.part_ml = take((size_t)(L.entries_max + 1) * d.group() * 2 * sizeof(float));
  L.counter = take(sizeof(int));                       // work-item counter of persistent kernels
  L.total = o;
  return L;
}

DecodeWs sparse_decode_ws_layout(const Dims& d) {
  DecodeWs L{};
  L.nslot = (d.topk + kDecSlots - 1) / kDecSlots;      // one partial per run of four selection slots
  const size_t units = (size_t)d.batch * d.h_kv * d.topk * d.group();
  size_t o = 0;
  L.part_o = o;
  o = align_up(o + units * d.d * 2, 256);
  L.part_ml = o;
  o = align_up(o + units * 2 * sizeof(float), 256);
  L.total = o;
  return L;
}

hipError_t launch_sparse_prefill(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* blk, float scale, uint16_t* out, float* lse, void* ws,
                                 hipStream_t stream) {
  const float sl2 = scale * kLog2e;
  if (d.d == 128) return prefill_by_group<128>(d, q, k, v, blk, sl2, out, lse, ws, stream);
  return prefill_by_group<64>(d, q, k, v, blk, sl2, out, lse, ws, stream);
}

hipError_t launch_sparse_prefill_target(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const int32_t* blk, float scale, const float* bscore, float idx_scale,
                                        uint16_t* out, float* lse, float* target, float* kl, void* ws,
                                        hipStream_t stream) {
  hipError_t e = launch_sparse_prefill(d, q, k, v, blk, scale, out, lse, ws, stream);
  if (e != hipSuccess) return e;
  const float* part_ml = reinterpret_cast<const float*>(static_cast<const char*>(ws) + prefill_ws_layout(d).part_ml);
  switch (d.group()) {
    case 1: return launch_target_t<1>(d, part_ml, blk, bscore, idx_scale, target, kl, stream);
    case 2: return launch_target_t<2>(d, part_ml, blk, bscore, idx_scale, target, kl, stream);
    case 4: return launch_target_t<4>(d, part_ml, blk, bscore, idx_scale, target, kl, stream);
    case 8: return launch_target_t<8>(d, part_ml, blk, bscore, idx_scale, target, kl, stream);
    default: return launch_target_t<16>(d, part_ml, blk, bscore, idx_scale, target, kl, stream);
  }
}

hipError_t launch_sparse_decode(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* blk, float scale, uint16_t* out, float* lse, void* ws,
                                hipStream_t stream) {
  const float sl2 = scale * kLog2e;
  if (d.d == 128) return decode_by_group<128>(d, q, k, v, blk, sl2, out, lse, ws, stream);
  return decode_by_group<64>(d, q, k, v, blk, sl2, out, lse, ws, stream);
}

hipError_t launch_merge(const Dims& d, const uint16_t* part_o, const float* part_ml, const int32_t* blk,
                        uint16_t* out, float* lse, int nslot, int per, hipStream_t stream) {
  if (d.d == 128) return launch_merge_t<128>(d, part_o, part_ml, blk, out, lse, nslot, per, stream);
  return launch_merge_t<64>(d, part_o, part_ml, blk, out, lse, nslot, per, stream);
}

}  // namespace msa
