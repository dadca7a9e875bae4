// Index branch, backward: gradient of the KL alignment loss with respect to the
// index queries and keys (Notion notes "Minimax-sparse-Attention": "KL Loss
// Alignment" trains the index branch to imitate the main branch's attention
// distribution; "Detached Gradients": the target is a constant and nothing
// flows into the main branch).  For a (b, t, g) row with live slots s:
//   a_s = idx_scale * pooled[j_s],  index = softmax(a),
//   coef_s = dkl[row] * idx_scale * (index_s - target_s),
// and the pooled score is a max over the block's causal tokens, so the
// gradient goes to its argmax token s* (the lowest position among equal
// maxima):  dq_idx[row] += coef_s k_idx[s*],  dk_idx[s*] += coef_s q_idx[row].
//
// Kernels: the per-row coefficients; a KV-outer pass over (b, block) work
// items that recomputes the scores of every entry of the block's lists (all
// groups share the index key) by MFMA, takes each entry's argmax and
// accumulates dk_idx for the block's keys on MFMA in registers, group by group
// in list order; and a per-row gather for dq_idx.  A causal prefill's earliest
// blocks are chosen by most later queries, so their lists hold several times
// the average work of a CU: such a block is cut into up to kIbMaxPieces pieces
// of consecutive column groups, the first writing dk_idx and the others a
// partial that index_dk_combine adds in piece order.  The pass is persistent
// (one workgroup per CU taking items from a counter, earliest blocks first):
// launching one workgroup per item left CUs idle for tens of microseconds
// between items.  Every sum runs in a fixed order, so results are
// deterministic without atomics on the data.
#include "launch.h"
#include "msa_device.h"

namespace msa {
namespace {

constexpr int kIbThreads = 512;
constexpr int kIbCols = 32;                            // entries per group
// A block whose lists hold many column groups is split into up to
// kIbMaxPieces workgroups of at least kIbPieceGroups groups each (a causal
// prefill's earliest blocks are chosen by most later queries: their lists are
// several times the average work per CU).
constexpr int kIbMaxPieces = 8;
constexpr int kIbPieceGroups = 128;

// Max / min over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48): each gfx950 permlane swap exchanges halves between its two
// operands, so op(result[0], result[1]) with the same value in both combines
// every lane with its partner 16 (then 32) lanes away.
__device__ __forceinline__ float rows_max(float v) {
  const int x = __builtin_bit_cast(int, v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = vmax(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  const int y = __builtin_bit_cast(int, v);
  const auto c = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return vmax(__builtin_bit_cast(float, (int)c[0]), __builtin_bit_cast(float, (int)c[1]));
}
__device__ __forceinline__ int rows_min(int v) {
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min((int)a[0], (int)a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min((int)c[0], (int)c[1]);
}

// coef[row][s] for the live slots, 0 for the others; R lanes per row.
template <int R>
__global__ __launch_bounds__(256) void index_kl_coef(const int32_t* __restrict__ blk,
                                                     const float* __restrict__ bscore,
                                                     const float* __restrict__ target,
                                                     const float* __restrict__ dkl, float* __restrict__ coef,
                                                     int64_t nrows, int n_q, int h_kv, int pos0, int topk, int nblk,
                                                     float idx_scale) {
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / R;   // (b * n_q + t) * h_kv + g
  const int s = threadIdx.x % R;
  const int64_t rr = row < nrows ? row : nrows - 1;
  const int t = (int)((rr / h_kv) % n_q);
  const int jl = (pos0 + t) / kBlock;
  const int sc = min(s, topk - 1);
  const int j = blk[rr * topk + sc];
  const bool on = s < topk && j >= 0 && j <= jl;
  const auto fmax = [](float x, float y) { return vmax(x, y); };
  const auto fadd = [](float x, float y) { return x + y; };
  const float sl2 = idx_scale * kLog2e;
  const float a = on ? bscore[rr * nblk + (on ? j : 0)] * sl2 : -INFINITY;
  const float A = row_reduce<R>(a, fmax);
  const float e = on ? __builtin_amdgcn_exp2f(a - A) : 0.f;
  const float Z = row_reduce<R>(e, fadd);
  const float tg = target[rr * topk + sc];
  const float c = on ? dkl[rr] * idx_scale * (e / Z - tg) : 0.f;
  if (row < nrows && s < topk) coef[row * topk + s] = c;
}

constexpr int kIbMaxLists = 128;                       // h_kv <= 128

template <int DI>
struct IbLds {
  union {
    uint16_t k[kBlock * DI];                           // the block's index keys, while loaded
    struct {
      // q rows and coefficients by group parity: the dk phase of one group
      // reads them while faster waves already stage the next group.
      uint16_t qr[2][kIbCols * DI];                    // [entry][d] index queries, qd_off
      float coef[2][kIbCols];
      int plim[kIbCols];                               // last visible position, -1 for an empty column
      // ((b * n_q + t) * h_kv + g) * topk + slot, -1 if empty; by group parity
      // (wave 0 publishes a group's argmax while faster waves stage the next).
      int slot_row[2][kIbCols];
      float wmax[8][kIbCols];                          // each wave's max per column
      int wkey[8][kIbCols];                            // and the lowest key in the block that has it
      // Per wave, per column: the coefficient as hi | mid << 16 and
      // lo | key << 16 (three bf16 terms; key -1 when the column has none).
      uint32_t whm[8][kIbCols], wlk[8][kIbCols];
    } g;
  };
  int lstart[kIbMaxLists];                             // flat column where group g's list starts
  int lbase[kIbMaxLists];                              // its first entry
  int item;                                            // the work item being processed
};

// One column group in flight: this thread's 16-byte chunk of its column's
// index query, the column's coefficient, last visible position and slot row,
// and the entry (value and group) that this buffer loads next.
struct IbStage {
  u32x4 q;
  float coef;
  int plim, srow, en_next, g_next;
};

// Bits of the bf16 nearest to x (round to nearest even).
__device__ __forceinline__ uint32_t bf16_rn(float x) { return pack_bf16x2(x, 0.f) & 0xffffu; }

// Column groups of the (b, block) lists of all groups, and the pieces they
// are split into (1 .. npmax).
__device__ __forceinline__ int ib_pieces(int ngroups, int npmax) {
  return max(1, min(npmax, ngroups / kIbPieceGroups));
}

// One work item: piece `piece` of the (b, block) lists jb = block * batch + b.
template <int DI>
__device__ __forceinline__ void ib_item(
    IbLds<DI>& sm, const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const int* __restrict__ off, const int* __restrict__ entries, const float* __restrict__ coef,
    int* __restrict__ amax_out, int sink, float* __restrict__ dk_idx, float* __restrict__ dk_part, int npmax,
    int batch, int n_q, int n_kv, int pos0, int h_kv, int nblk, int topk, int jb, int piece) {
  constexpr int DC = DI / 8;
  constexpr int DT = DI / 16;                          // 16-wide d tiles of dk_idx
  constexpr int NST = kIbCols * DC;                    // staging threads (one chunk each)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m16 = lane & 15, q4 = lane >> 4;
  const int j = jb / batch, b = jb % batch;
  const int s0 = j * kBlock;
  // Columns of the block's lists (uniform loads), and this workgroup's share.
  int ncols = 0;
  for (int g = 0; g < h_kv; ++g) {
    const int list = (b * h_kv + g) * nblk + j;
    ncols += off[list + 1] - off[list];
  }
  const int ngroups_all = (ncols + kIbCols - 1) / kIbCols;
  const int npieces = ib_pieces(ngroups_all, npmax);
  if (piece >= npieces) return;                        // workgroup-uniform: nothing of this block is left
  const int per = (ngroups_all + npieces - 1) / npieces;
  const int grp0 = piece * per;
  const int ngroups = max(0, min(ngroups_all, grp0 + per) - grp0);
  const uint16_t* kb = k_idx + (int64_t)b * n_kv * DI;

  for (int it = tid; it < kBlock * DC; it += kIbThreads) {
    const int key = it / DC, ch = it % DC, s = s0 + key;
    st16(&sm.k[rt_off<DI>(key, ch)], s < n_kv ? ld16(kb + (int64_t)s * DI + ch * 8) : u32x4{0u, 0u, 0u, 0u});
  }
  if (tid == 0) {                                      // the block's lists of all groups, back to back
    int run = 0;
    for (int g = 0; g < h_kv; ++g) {
      const int list = (b * h_kv + g) * nblk + j;
      sm.lstart[g] = run;
      sm.lbase[g] = off[list];
      run += off[list + 1] - off[list];
    }
  }
  __syncthreads();
  // A operands of S^T: row (MFMA m) = this lane's key, contraction slots
  // 8*q4 + i = d 32*c + 8*q4 + i.
  const int mykey = 16 * w + m16;
  u32x4 kop[DI / 32];
#pragma unroll
  for (int c = 0; c < DI / 32; ++c) kop[c] = ld16(&sm.k[rt_off<DI>(mykey, 4 * c + q4)]);
  __syncthreads();                                     // the LDS now holds entry groups
  // dk_idx of this wave's 16 keys: lane holds keys 16*w + 4*q4 + r, d 16*dt + m16.
  f32x4 dka[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dka[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (ngroups > 0) {
    // Staging role: column scol of each group, chunk sch of its query.
    // Threads beyond NST (d_idx = 64) mirror the first NST.
    const int st_id = tid % NST, scol = st_id / DC, sch = st_id % DC;
    // Transposing-read offsets of the dk products (B operand: column n = d
    // 16*dt + m16, contraction slot 8*q4 + i <-> column 4*q4 + i (i < 4) or
    // 16 + 4*q4 + i - 4 (i >= 4)): rows 4*q4 + (m16 >> 2) and 16 + ..., chunk
    // 2*dt + ((m16 & 3) >> 1), element 4*(m16 & 1).
    const int tr_r1 = 4 * q4 + (m16 >> 2), tr_r2 = tr_r1 + 16;
    const int tr_row1 = tr_r1 * DI, tr_row2 = tr_r2 * DI;
    const int tr_x1 = qd_swz<DI>(tr_r1) ^ ((m16 & 3) >> 1), tr_x2 = qd_swz<DI>(tr_r2) ^ ((m16 & 3) >> 1);
    const int tr_e = 4 * (m16 & 1);
    // Flat column f -> (entry value, group); f is clamped to a real column,
    // so no load of the loop sits behind a branch.
    // Groups are numbered from this piece's first one (grp0).
    const int cend = min(ncols, (grp0 + ngroups) * kIbCols);   // this piece's columns end here
    auto entry_at = [&](int grp, int& gout) {
      const int f = min((grp0 + grp) * kIbCols + scol, cend - 1);
      int lo = 0, hi = h_kv;                           // largest g with lstart[g] <= f
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sm.lstart[mid] <= f) lo = mid;
        else hi = mid;
      }
      gout = lo;
      return entries[sm.lbase[lo] + f - sm.lstart[lo]];
    };
    auto fetch = [&](IbStage& st, int grp, int en, int gc) {
      const int t = entry_token(en);
      const bool live = (grp0 + grp) * kIbCols + scol < cend;
      const int64_t qrow = ((int64_t)b * n_q + t) * h_kv + gc;
      const int sr = (int)(qrow * topk + entry_slot(en));
      st.q = ld16(q_idx + qrow * DI + sch * 8);
      st.coef = coef[sr];
      st.plim = live ? pos0 + t : -1;
      st.srow = live ? sr : -1;
    };
    IbStage sx, sy;
    {
      int g0, g1, g2, g3;
      const int en0 = entry_at(0, g0), en1 = entry_at(1, g1);
      fetch(sx, 0, en0, g0);
      fetch(sy, 1, en1, g1);
      sx.en_next = entry_at(2, g2);
      sx.g_next = g2;
      sy.en_next = entry_at(3, g3);
      sy.g_next = g3;
    }
    auto step = [&](IbStage& st, int grp) {
      const int par = grp & 1;
      // Every thread of a column writes the same per-column values.
      st16(&sm.g.qr[par][qd_off<DI>(scol, sch)], st.q);
      sm.g.coef[par][scol] = st.coef;
      sm.g.plim[scol] = st.plim;
      sm.g.slot_row[par][scol] = st.srow;
      __syncthreads();
      {
        const int en = st.en_next, gn = st.g_next;
        fetch(st, grp + 2, en, gn);
        int g4;
        st.en_next = entry_at(grp + 4, g4);
        st.g_next = g4;
      }
      // S^T for this wave's 16 keys with the key as the MFMA row (the resident
      // key operand serves as A): lane holds keys 16*w + 4*q4 + r of column
      // 16*ct + m16.
      f32x4 sacc[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DI / 32; ++c)
          sacc[ct] = mfma_16x16x32(kop[c], ld16(&sm.g.qr[par][qd_off<DI>(16 * ct + m16, 4 * c + q4)]), sacc[ct]);
      }
      // Per column: the wave's max over its 16 keys (4 in the lane, then over
      // the lane's four rows) and the lowest key that has it.
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int col = 16 * ct + m16;
        const int lim = sm.g.plim[col] - (s0 + 16 * w + 4 * q4);   // key r visible when r <= lim
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = r <= lim ? sacc[ct][r] : -INFINITY;
        const float m = rows_max(vmax(vmax(v[0], v[1]), vmax(v[2], v[3])));
        const int r0 = v[0] == m ? 0 : v[1] == m ? 1 : v[2] == m ? 2 : 3;
        const int kk = rows_min(m > -INFINITY && v[r0] == m ? 16 * w + 4 * q4 + r0 : 1 << 20);
        if (q4 == 0) {
          sm.g.wmax[w][col] = m;
          sm.g.wkey[w][col] = kk;
        }
      }
      __syncthreads();
      // Across waves (ascending key ranges): the first wave that reaches the
      // column's maximum holds its lowest argmax.  Every wave derives it for
      // column lane & 31 (lanes l and l + 32 agree), so no barrier follows;
      // wave 0 publishes it, its upper half storing to the sink slot.
      const int colm = lane & 31;
      float best = -INFINITY;
      int key = -1;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) {
        const float m = sm.g.wmax[ww][colm];
        key = m > best ? sm.g.wkey[ww][colm] : key;
        best = vmax(best, m);
      }
      const int sr = sm.g.slot_row[par][colm];
      key = sr < 0 ? -1 : key;
      if (w == 0) amax_out[(lane < 32 && sr >= 0) ? sr : sink] = key < 0 ? -1 : s0 + key;
      // dk_idx[key] += coef q for each column, as one product per group: A
      // (this wave's 16 keys x the 32 columns) holds a column's coefficient in
      // its argmax key's row and 0 elsewhere, B is the column's index query.
      // The fp32 coefficient is split exactly enough into three bf16 terms
      // (hi + mid + lo within 2^-27 of it), and bf16 x bf16 products are exact
      // in fp32, so the sum keeps fp32 accuracy.  Each wave writes its own
      // copy of the per-column values (no barrier: one wave's LDS operations
      // complete in order).
      {
        const float cf = sm.g.coef[par][colm];
        const uint32_t hi = bf16_rn(cf);
        const float r1 = cf - bf16_to_f32(hi);
        const uint32_t mid = bf16_rn(r1);
        const uint32_t lo = bf16_rn(r1 - bf16_to_f32(mid));
        if (lane < kIbCols) {
          sm.g.whm[w][colm] = hi | (mid << 16);
          sm.g.wlk[w][colm] = lo | ((uint32_t)key << 16);
        }
      }
      const u32x4 hm0 = *reinterpret_cast<const u32x4*>(&sm.g.whm[w][4 * q4]);
      const u32x4 hm1 = *reinterpret_cast<const u32x4*>(&sm.g.whm[w][16 + 4 * q4]);
      const u32x4 lk0 = *reinterpret_cast<const u32x4*>(&sm.g.wlk[w][4 * q4]);
      const u32x4 lk1 = *reinterpret_cast<const u32x4*>(&sm.g.wlk[w][16 + 4 * q4]);
      // Slot pair (2p, 2p + 1) of the A operands: columns of hm/lk elements
      // 2p', 2p' + 1 of the first (p < 2) or second (p >= 2) half.
      u32x4 ahi, amid, alo;
      const uint32_t me = (uint32_t)mykey;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const u32x4& hm = p < 2 ? hm0 : hm1;
        const u32x4& lk = p < 2 ? lk0 : lk1;
        const int e0 = 2 * (p & 1), e1 = e0 + 1;
        const uint32_t mask = ((lk[e0] >> 16) == me ? 0x0000ffffu : 0u) | ((lk[e1] >> 16) == me ? 0xffff0000u : 0u);
        ahi[p] = ((hm[e0] & 0xffffu) | (hm[e1] << 16)) & mask;
        amid[p] = ((hm[e0] >> 16) | (hm[e1] & 0xffff0000u)) & mask;
        alo[p] = ((lk[e0] & 0xffffu) | (lk[e1] << 16)) & mask;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int o1 = tr_row1 + 8 * ((2 * dt) ^ tr_x1) + tr_e;
        const int o2 = tr_row2 + 8 * ((2 * dt) ^ tr_x2) + tr_e;
        const u32x2 qlo = ld_tr16(&sm.g.qr[par][o1]), qhi = ld_tr16(&sm.g.qr[par][o2]);
        const u32x4 qb = {qlo[0], qlo[1], qhi[0], qhi[1]};
        dka[dt] = mfma_16x16x32(ahi, qb, dka[dt]);
        dka[dt] = mfma_16x16x32(amid, qb, dka[dt]);
        dka[dt] = mfma_16x16x32(alo, qb, dka[dt]);
      }
    };
    __builtin_amdgcn_s_waitcnt(0);                     // drain the prologue (exact waits in the loop)
    for (int grp = 0; grp < ngroups; grp += 2) {
      step(sx, grp);
      step(sy, grp + 1);
    }
  }
  // Rows 16*w + 4*q4 + r, d 16*dt + m16: piece 0 into dk_idx, the others into
  // their partial slot (summed in piece order by index_dk_combine).
  if (piece == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = s0 + 16 * w + 4 * q4 + r;
      if (s >= n_kv) continue;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dk_idx[((int64_t)b * n_kv + s) * DI + 16 * dt + m16] = dka[dt][r];
    }
  } else {
    float* dst = dk_part + ((((int64_t)(piece - 1) * batch + b) * nblk + j) * kBlock) * DI;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dst[(16 * w + 4 * q4 + r) * DI + 16 * dt + m16] = dka[dt][r];
  }
}

// Persistent: one workgroup per CU takes work items (block, piece) in order,
// earliest blocks first, from a counter that the launch zeroes beforehand
// (one vector atomic per item, broadcast through LDS).  Every wave of a
// workgroup sees the same item, so all leave the loop together once the
// items run out.
template <int DI>
__global__ __launch_bounds__(kIbThreads, 1) void index_bwd_kv(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const int* __restrict__ off,
    const int* __restrict__ entries, const float* __restrict__ coef, int* __restrict__ amax_out, int sink,
    float* __restrict__ dk_idx, float* __restrict__ dk_part, int npmax, int batch, int n_q, int n_kv, int pos0,
    int h_kv, int nblk, int topk, int* __restrict__ counter, const int* __restrict__ items) {
  __shared__ IbLds<DI> sm;
  const int nitems = items[0];
  for (;;) {
    if (threadIdx.x == 0) sm.item = atomicAdd(counter, 1);
    __syncthreads();
    const int v = sm.item;
    if (v >= nitems) break;
    const int it = items[1 + v];
    ib_item<DI>(sm, q_idx, k_idx, off, entries, coef, amax_out, sink, dk_idx, dk_part, npmax, batch, n_q, n_kv,
                pos0, h_kv, nblk, topk, it / npmax, it % npmax);
    __syncthreads();                                   // the next item reuses the LDS
  }
}

// The work items of index_bwd_kv: for every (b, block) in order (earliest
// blocks first) its pieces jb * npmax + p, p < npieces, after the count in
// items[0]; also zeroes the item counter.  One workgroup: each thread takes
// a contiguous run of blocks, and a scan over the threads places them.
constexpr int kPlanThreads = 1024;
__global__ __launch_bounds__(kPlanThreads) void ib_plan(const int* __restrict__ off, int* __restrict__ counter,
                                                          int* __restrict__ items, int npmax, int batch, int h_kv,
                                                          int nblk) {
  __shared__ int part[kPlanThreads];
  const int tid = threadIdx.x;
  const int nb = batch * nblk;
  const int per = (nb + kPlanThreads - 1) / kPlanThreads;
  const int jb0 = min(nb, tid * per), jb1 = min(nb, jb0 + per);
  auto pieces = [&](int jb) {
    const int j = jb / batch, b = jb % batch;
    int ncols = 0;
    for (int g = 0; g < h_kv; ++g) {
      const int list = (b * h_kv + g) * nblk + j;
      ncols += off[list + 1] - off[list];
    }
    return ib_pieces((ncols + kIbCols - 1) / kIbCols, npmax);
  };
  int mine = 0;
  for (int jb = jb0; jb < jb1; ++jb) mine += pieces(jb);
  part[tid] = mine;
  __syncthreads();
  for (int d = 1; d < kPlanThreads; d <<= 1) {         // inclusive scan
    const int x = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int at = part[tid] - mine;
  for (int jb = jb0; jb < jb1; ++jb) {
    const int np = pieces(jb);
    for (int p = 0; p < np; ++p) items[1 + at + p] = jb * npmax + p;
    at += np;
  }
  if (tid == kPlanThreads - 1) items[0] = part[tid];
  if (tid == 0) *counter = 0;
}

// dk_idx of a split block += its pieces 1 .. npieces - 1, in piece order.
// One workgroup per (b, block); blocks with one piece return at once.
template <int DI>
__global__ __launch_bounds__(256) void index_dk_combine(const int* __restrict__ off,
                                                        const float* __restrict__ dk_part,
                                                        float* __restrict__ dk_idx, int npmax, int batch,
                                                        int n_kv, int h_kv, int nblk) {
  const int j = blockIdx.x / batch, b = blockIdx.x % batch;
  int ncols = 0;
  for (int g = 0; g < h_kv; ++g) {
    const int list = (b * h_kv + g) * nblk + j;
    ncols += off[list + 1] - off[list];
  }
  const int npieces = ib_pieces((ncols + kIbCols - 1) / kIbCols, npmax);
  if (npieces == 1) return;
  const int s0 = j * kBlock;
  const int keys = min(kBlock, n_kv - s0);
  for (int i = threadIdx.x; i < keys * (DI / 4); i += 256) {
    const int key = i / (DI / 4), d4 = i % (DI / 4);
    f32x4* dst = reinterpret_cast<f32x4*>(dk_idx + ((int64_t)b * n_kv + s0 + key) * DI) + d4;
    f32x4 acc = *dst;
    for (int p = 1; p < npieces; ++p)
      acc += *(reinterpret_cast<const f32x4*>(
                  dk_part + ((((int64_t)(p - 1) * batch + b) * nblk + j) * kBlock + key) * DI) + d4);
    *dst = acc;
  }
}

// dq_idx[row] = sum over the live slots of coef * k_idx[argmax]; DI / 8
// threads per row, 8 values each.
template <int DI>
__global__ __launch_bounds__(256) void index_dq_gather(const float* __restrict__ coef,
                                                       const int* __restrict__ amax,
                                                       const uint16_t* __restrict__ k_idx,
                                                       float* __restrict__ dq_idx, int64_t nrows, int n_q,
                                                       int h_kv, int n_kv, int topk) {
  constexpr int TPR = DI / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= nrows) return;
  const int dl = threadIdx.x % TPR;
  const int b = (int)(row / ((int64_t)n_q * h_kv));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < topk; ++s) {
    const float cf = coef[row * topk + s];
    // Dead slots carry coef 0 and an unwritten argmax: clamp the address.
    const int pos = amax[row * topk + s];
    const int ps = min(max(pos, 0), n_kv - 1);
    const u32x4 kv = ld16(k_idx + ((int64_t)b * n_kv + ps) * DI + dl * 8);
    const float c = pos >= 0 ? cf : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(c, bf16_to_f32(kv[e] & 0xffffu), acc[2 * e]);
      acc[2 * e + 1] = fmaf(c, bf16_to_f32(kv[e] >> 16), acc[2 * e + 1]);
    }
  }
  float* dst = dq_idx + row * DI + dl * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = acc[e];
}

template <int DI>
hipError_t launch_index_bwd_t(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, const int32_t* blk,
                              const float* bscore, const float* target, const float* dkl, float idx_scale,
                              float* dq_idx, float* dk_idx, void* ws, hipStream_t stream) {
  const PrefillWs L = prefill_ws_layout(d);
  char* base = static_cast<char*>(ws);
  const int* off = reinterpret_cast<const int*>(base + L.off);
  const int* entries = reinterpret_cast<const int*>(base + L.entries);
  float* coef = reinterpret_cast<float*>(base + L.part_ml);
  int* amax = reinterpret_cast<int*>(base + L.part_o);
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_kv;
  if (nrows > 0) {
    const int R = d.topk > 32 ? 64 : d.topk > 16 ? 32 : 16;
    const int64_t wgs = (nrows * R + 255) / 256;
    LaunchTimer timer("index_kl_coef", stream);
    if (R == 16)
      hipLaunchKernelGGL(index_kl_coef<16>, dim3((unsigned)wgs), dim3(256), 0, stream, blk, bscore, target, dkl,
                         coef, nrows, d.n_q, d.h_kv, d.pos0, d.topk, d.nblk(), idx_scale);
    else if (R == 32)
      hipLaunchKernelGGL(index_kl_coef<32>, dim3((unsigned)wgs), dim3(256), 0, stream, blk, bscore, target, dkl,
                         coef, nrows, d.n_q, d.h_kv, d.pos0, d.topk, d.nblk(), idx_scale);
    else
      hipLaunchKernelGGL(index_kl_coef<64>, dim3((unsigned)wgs), dim3(256), 0, stream, blk, bscore, target, dkl,
                         coef, nrows, d.n_q, d.h_kv, d.pos0, d.topk, d.nblk(), idx_scale);
  }
  hipError_t e = launch_csr(d, blk, ws, stream, true);    // sums run in list order
  if (e != hipSuccess) return e;
  // Partial dk_idx of split blocks: after the argmax slots in the partial
  // region, as many pieces per block as fit (at most kIbMaxPieces).
  const size_t amax_bytes = align_up(sizeof(int) * (size_t)(nrows * d.topk + 1), 256);
  const size_t region = (size_t)(L.entries_max + 1) * d.group() * d.d * 2;
  const size_t per_piece = (size_t)d.batch * d.nblk() * kBlock * DI * sizeof(float);
  int npmax = kIbMaxPieces;
  auto items_size = [&](int np) { return align_up(sizeof(int) * (1 + (size_t)d.batch * d.nblk() * np), 256); };
  while (npmax > 1 && amax_bytes + 256 + items_size(npmax) + (size_t)(npmax - 1) * per_piece > region) npmax /= 2;
  const size_t items_bytes = items_size(npmax);
  int* counter = reinterpret_cast<int*>(base + L.part_o + amax_bytes);
  int* items = reinterpret_cast<int*>(base + L.part_o + amax_bytes + 256);
  float* dk_part = reinterpret_cast<float*>(base + L.part_o + amax_bytes + 256 + items_bytes);
  const int nitems_max = d.batch * d.nblk() * npmax;
  {
    LaunchTimer timer("ib_plan", stream);
    hipLaunchKernelGGL(ib_plan, dim3(1), dim3(kPlanThreads), 0, stream, off, counter, items, npmax, d.batch, d.h_kv,
                       d.nblk());
  }
  {
    LaunchTimer timer("index_bwd_kv", stream);
    hipLaunchKernelGGL(index_bwd_kv<DI>, dim3((unsigned)min(device_cu_count(), nitems_max)), dim3(kIbThreads), 0,
                       stream, q_idx, k_idx, off, entries, coef, amax, (int)(nrows * d.topk), dk_idx, dk_part, npmax,
                       d.batch, d.n_q, d.n_kv, d.pos0, d.h_kv, d.nblk(), d.topk, counter, items);
  }
  if (npmax > 1) {
    LaunchTimer timer("index_dk_combine", stream);
    hipLaunchKernelGGL(index_dk_combine<DI>, dim3((unsigned)(d.batch * d.nblk())), dim3(256), 0, stream, off,
                       dk_part, dk_idx, npmax, d.batch, d.n_kv, d.h_kv, d.nblk());
  }
  if (nrows > 0) {
    constexpr int TPR = DI / 8;
    const int64_t wgs = (nrows + 256 / TPR - 1) / (256 / TPR);
    LaunchTimer timer("index_dq_gather", stream);
    hipLaunchKernelGGL(index_dq_gather<DI>, dim3((unsigned)wgs), dim3(256), 0, stream, coef, amax, k_idx, dq_idx,
                       nrows, d.n_q, d.h_kv, d.n_kv, d.topk);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_backward(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, const int32_t* blk,
                                 const float* bscore, const float* target, const float* dkl, float idx_scale,
                                 float* dq_idx, float* dk_idx, void* ws, hipStream_t stream) {
  if (d.d_idx == 128)
    return launch_index_bwd_t<128>(d, q_idx, k_idx, blk, bscore, target, dkl, idx_scale, dq_idx, dk_idx, ws, stream);
  return launch_index_bwd_t<64>(d, q_idx, k_idx, blk, bscore, target, dkl, idx_scale, dq_idx, dk_idx, ws, stream);
}

}  // namespace msa
