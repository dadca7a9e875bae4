// Main branch, backward: gradients of the selected-block softmax attention with
// respect to q, k and v for a fixed selection (the selection is discrete and
// carries no gradient; Notion notes "Minimax-sparse-Attention", "Detached
// Gradients").  With P the softmax weights of a (query, head) over its visible
// keys, D = rowsum(dout * out):
//   dv[s] = sum P dout,   dP = dout . v[s],   dS = P (dP - D),
//   dq    = scale sum_s dS k[s],   dk[s] = scale sum dS q.
//
// KV-outer, like the forward (lumi-systems summary: KV-outer sparse attention):
// one workgroup at a time per (b, g, block) list of the CSR inversion (a
// persistent workgroup per CU takes the lists in order).  Its eight waves
// each own 16 keys of the block: they keep those keys' K and V rows as MFMA
// operands in registers, and their dk / dv rows as fp32 accumulators for the
// whole list, so every key gradient is summed inside one workgroup in a fixed
// order (no atomics).  For each group of 32 (entry x group head) columns the
// columns' q and dout rows are staged in LDS row-major; each wave computes S^T
// and dP^T for its keys, P and dS, and adds P * dout and dS * q into its rows,
// reading the q and dout operands of those two products from the same
// row-major tiles with transposing LDS reads.  dS goes through LDS so that each wave can then form
// one 16-wide d slice of dq over all 128 keys of the block; dq leaves as one
// bf16 partial per (t, g, slot, head), summed per (t, head) by a second kernel.
#include "launch.h"
#include "msa_device.h"

namespace msa {
namespace {

constexpr int kBwdThreads = 512;
constexpr int kBwdCols = 32;                           // (entry x head) columns per group

// dS tile [key][column]: 4-column (8-byte) chunk c of row key at
// c ^ ((key >> 1) & 6).  The writes (lane: key 16*w + m16, chunk 4*ct + q4) and
// the transposing reads of dq (lane: key 32*kc + 8*q4 + (m16 >> 2) (+ 4),
// chunk 4*ct + (m16 & 3)) then each reach 32 distinct bank pairs per half-wave.
__device__ __forceinline__ int ds_off(int key, int chunk) {
  return key * kBwdCols + 4 * (chunk ^ ((key >> 1) & 6));
}

template <int D>
struct BwdLds {
  union {
    struct {
      uint16_t k[kBlock * D];
      uint16_t v[kBlock * D];
    } kv;                                              // the block, while its operands are loaded
    struct {
      uint16_t qr[kBwdCols * D], dor[kBwdCols * D];    // [column][d], qd_off
      uint16_t ds[kBlock * kBwdCols];                  // [key][column], ds_off
      // Read as 16-byte vectors of 4 consecutive columns.
      alignas(16) float lse2[kBwdCols];
      alignas(16) float dcol[kBwdCols];
      alignas(16) int plim[kBwdCols];                  // last visible key position, -1 for an empty column
      // Element offset of each column's partial dq row (the sink when empty),
      // by group parity: the dq phase of one group reads it while faster waves
      // already stage the next group.  An offset from the kernel argument, not
      // an address: a pointer rebuilt from an integer would make the stores
      // flat ones, which also count against the LDS wait counter.
      uint64_t prow[2][kBwdCols];
    } g;
  };
  int item;                                            // the list being processed
};

__device__ __forceinline__ uint32_t bf16_bits(float x) { return pack_bf16x2(x, 0.f) & 0xffffu; }

// D = rowsum(dout * out) per (b, t, head) row, from the forward's bf16 output.
template <int D>
__global__ __launch_bounds__(256) void bwd_row_dot(const uint16_t* __restrict__ out,
                                                   const uint16_t* __restrict__ dout, float* __restrict__ dcol,
                                                   int64_t nrows) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int64_t rr = row < nrows ? row : nrows - 1;
  const int dl = threadIdx.x % TPR;
  const u32x4 a = ld16(out + rr * D + dl * 8), c = ld16(dout + rr * D + dl * 8);
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sum = fmaf(bf16_to_f32(a[e] & 0xffffu), bf16_to_f32(c[e] & 0xffffu), sum);
    sum = fmaf(bf16_to_f32(a[e] >> 16), bf16_to_f32(c[e] >> 16), sum);
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) sum += shfl_xor_f(sum, m);
  if (row < nrows && dl == 0) dcol[row] = sum;
}

// Registers of the next column group: this thread's staging tile (2 columns x
// one 16-byte chunk of q or dout), the values of its meta column (tid & 31),
// and the entries of the group after it (the 2 staging columns and the meta
// column).
struct BwdStage {
  u32x4 v[2];
  uint64_t prow;                                       // element offset of the column's dq partial row in part_dq
  float lse2, dcol;
  int plim;
  int en[2], men;
};

// One (b, g, block) list; `item` numbers the lists block-major.
template <int D, int LOG2G>
__device__ __forceinline__ void bwd_list(
    BwdLds<D>& sm, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dcol,
    const int* __restrict__ off, const int* __restrict__ entries, uint16_t* __restrict__ part_dq,
    int64_t sink_off, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int batch, int n_q, int n_kv, int pos0,
    int h_q, int h_kv, int nblk, int topk, float sl2, float scale, int item) {
  constexpr int G = 1 << LOG2G;
  constexpr int DC = D / 8;                            // 16-byte chunks per row
  constexpr int DT = D / 16;                           // 16-wide d tiles
  constexpr int NDT = DT / 4;                          // d tiles of dq per wave (one column tile)
  constexpr int NST = 2 * 16 * DC;                     // staging threads: 2-column tiles of q and dout
  // The thread index passes through an empty asm so that what derives from it
  // is recomputed per list instead of being held across the whole loop.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, w = tid >> 6;
  const int m16 = lane & 15, q4 = lane >> 4;
  // Block index outermost, so the earliest blocks (candidates for the most
  // queries) start first.
  const int bgs = batch * h_kv;
  const int j = item / bgs, bg = item % bgs;
  const int g = bg % h_kv, b = bg / h_kv;
  const int list = bg * nblk + j;
  const int e0 = off[list], e1 = off[list + 1];
  const int ncols = (e1 - e0) << LOG2G;
  const int s0 = j * kBlock;
  const int64_t rs = (int64_t)h_kv * D;
  const uint16_t* kb = k + ((int64_t)b * n_kv * h_kv + g) * D;
  const uint16_t* vb = v + ((int64_t)b * n_kv * h_kv + g) * D;

  for (int it = tid; it < kBlock * DC; it += kBwdThreads) {
    const int key = it / DC, ch = it % DC, s = s0 + key;
    const u32x4 z = {0u, 0u, 0u, 0u};
    st16(&sm.kv.k[rt_off<D>(key, ch)], s < n_kv ? ld16(kb + s * rs + ch * 8) : z);
    st16(&sm.kv.v[rt_off<D>(key, ch)], s < n_kv ? ld16(vb + s * rs + ch * 8) : z);
  }
  __syncthreads();
  // B operands of S^T and dP^T: column (MFMA n) = this lane's key, contraction
  // slots 8*q4 + i = d 32*c + 8*q4 + i.
  const int mykey = 16 * w + m16;
  u32x4 kop[D / 32], vop[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    kop[c] = ld16(&sm.kv.k[rt_off<D>(mykey, 4 * c + q4)]);
    vop[c] = ld16(&sm.kv.v[rt_off<D>(mykey, 4 * c + q4)]);
  }
  // dq: wave w forms column tile w >> 2 for d tiles dt0 .. dt0 + NDT - 1, so
  // each dS operand it reads feeds NDT products.  A operands: row (MFMA m) =
  // d 16*(dt0 + n) + m16, contraction slots = keys 32*kc + 8*q4 + i.
  const int dct = w >> 2, dt0 = (w & 3) * NDT;
  u32x4 ktop[NDT][4];
#pragma unroll
  for (int n = 0; n < NDT; ++n) {
    const int d = 16 * (dt0 + n) + m16;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 32 * kc + 8 * q4 + 2 * i;
        const uint32_t lo = sm.kv.k[rt_off<D>(key, d >> 3) + (d & 7)];
        const uint32_t hi = sm.kv.k[rt_off<D>(key + 1, d >> 3) + (d & 7)];
        ktop[n][kc][i] = lo | (hi << 16);
      }
  }
  __syncthreads();                                     // the LDS now holds column groups

  f32x4 dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dka[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dva[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int ngroups = (ncols + kBwdCols - 1) / kBwdCols;
  if (ngroups > 0) {
    const int skey = s0 + mykey;
    // Transposing-read offsets: rows 4*q4 + (m16 >> 2) and 16 + ..., chunk
    // 2*dt + ((m16 & 3) >> 1) (so chunk ^ qd_swz = 2*dt ^ x), element 4*(m16 & 1).
    const int tr_r1 = 4 * q4 + (m16 >> 2), tr_r2 = tr_r1 + 16;
    const int tr_row1 = tr_r1 * D, tr_row2 = tr_r2 * D;
    const int tr_x1 = qd_swz<D>(tr_r1) ^ ((m16 & 3) >> 1), tr_x2 = qd_swz<D>(tr_r2) ^ ((m16 & 3) >> 1);
    const int tr_e = 4 * (m16 & 1);
    // Staging role: tensor `which` (q or dout), columns 2*scp and 2*scp + 1,
    // chunk sch (d = 128: every thread; d = 64: threads beyond NST mirror the
    // first NST and write nothing); every thread also carries the meta values
    // of column tid & 31.
    const int st_id = tid % NST, which = st_id / (16 * DC), scp = (st_id % (16 * DC)) / DC, sch = st_id % DC;
    const int mcol = tid & 31;
    const uint16_t* src = which ? dout : q;
    // Addresses are 32 x 32 -> 64-bit products of the token row T = b * n_q + t
    // (< 2^31) and byte strides (< 2^32, checked on the host) onto per-lane
    // bases.
    const uint32_t tok0 = (uint32_t)b * (uint32_t)n_q;
    const int* ent = entries + e0;
    const uint32_t q_tok_bytes = (uint32_t)h_q * (D * 2);
    const uint32_t pr_tok_elems = (uint32_t)h_q * (uint32_t)topk * D;
    const char* src_lane = reinterpret_cast<const char*>(src) + ((size_t)g * G * D + sch * 8) * 2;
    const uint32_t pdq_g = (uint32_t)(g * topk * G * D);
    const float* lse_g = lse + g * G;
    const float* dcol_g = dcol + g * G;
    // Every load of the loop reads a real row (the column index is clamped), so
    // the loop body has no memory operation behind a branch and the compiler's
    // wait counts stay exact across iterations; columns past the list end are
    // masked through plim = -1 and their dq goes to the sink row.
    auto entry_at = [&](int grp, int col) {
      const uint32_t gc = (uint32_t)min(grp * kBwdCols + col, ncols - 1);
      return ent[gc >> LOG2G];
    };
    auto fetch = [&](BwdStage& st, int grp) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint32_t hh = (uint32_t)min(grp * kBwdCols + 2 * scp + kk, ncols - 1) & (G - 1);
        const uint32_t T = tok0 + (uint32_t)entry_token(st.en[kk]);
        st.v[kk] = ld16(src_lane + hh * (D * 2) + (uint64_t)T * q_tok_bytes);
      }
      const int gc = grp * kBwdCols + mcol;
      const uint32_t hh = (uint32_t)min(gc, ncols - 1) & (G - 1);
      const int t = entry_token(st.men);
      const uint32_t T = tok0 + (uint32_t)t;
      const uint64_t row = (uint64_t)T * (uint32_t)h_q + hh;
      st.lse2 = lse_g[row] * kLog2e;
      st.dcol = dcol_g[row];
      // Selects by mask, not a ternary: a branch here would make the
      // compiler's wait counts at the loop head conservative.
      const uint64_t live = -(uint64_t)(gc < ncols);
      const uint64_t pa = (uint64_t)T * pr_tok_elems + (pdq_g + ((uint32_t)entry_slot(st.men) * G + hh) * D);
      st.plim = (int)(((uint32_t)(pos0 + t) & (uint32_t)live) | ~(uint32_t)live);
      st.prow = (pa & live) | ((uint64_t)sink_off & ~live);
    };
    auto load_entries = [&](BwdStage& st, int grp) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) st.en[kk] = entry_at(grp, 2 * scp + kk);
      st.men = entry_at(grp, mcol);
    };
    BwdStage st;
    load_entries(st, 0);
    fetch(st, 0);
    load_entries(st, 1);
    // Drain the prologue's loads: the wait counts at the loop head are the
    // merge of the entry and back-edge states, and an empty entry state keeps
    // them those of the loop itself.
    __builtin_amdgcn_s_waitcnt(0);
    for (int grp = 0; grp < ngroups; ++grp) {
      if (tid < NST) {                                 // wave-uniform
        uint16_t* rt = which ? sm.g.dor : sm.g.qr;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) st16(&rt[qd_off<D>(2 * scp + kk, sch)], st.v[kk]);
      }
      if (w == 0) {                                    // wave-uniform; lanes l and l + 32 agree
        sm.g.plim[mcol] = st.plim;
        sm.g.lse2[mcol] = st.lse2;
        sm.g.dcol[mcol] = st.dcol;
        sm.g.prow[grp & 1][mcol] = st.prow;
      }
      __syncthreads();
      // The next group's rows, and the entries of the group after it.
      fetch(st, grp + 1);
      load_entries(st, grp + 2);
      // S^T and dP^T for this wave's 16 keys and the 32 columns: lane holds
      // column 16*ct + 4*q4 + r, key mykey.
      f32x4 sacc[2], dpacc[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        dpacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          sacc[ct] = mfma_16x16x32(ld16(&sm.g.qr[qd_off<D>(16 * ct + m16, 4 * c + q4)]), kop[c], sacc[ct]);
          dpacc[ct] = mfma_16x16x32(ld16(&sm.g.dor[qd_off<D>(16 * ct + m16, 4 * c + q4)]), vop[c], dpacc[ct]);
        }
      }
      float p[2][4], ds[2][4];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int c0 = 16 * ct + 4 * q4;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.g.lse2[c0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.g.dcol[c0]);
        const u32x4 m4 = *reinterpret_cast<const u32x4*>(&sm.g.plim[c0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = fmaf(sacc[ct][r], sl2, -l4[r]);
          const float pv = __builtin_amdgcn_exp2f(skey <= (int)m4[r] ? x : -INFINITY);
          p[ct][r] = pv;
          ds[ct][r] = pv * (dpacc[ct][r] - d4[r]);
        }
      }
      // A operands (row = this lane's key) with contraction slot 8*q4 + i <->
      // column 4*q4 + i (i < 4) or 16 + 4*q4 + i - 4 (i >= 4).
      const u32x4 pa = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                        pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
      const u32x4 dsa = {pack_bf16x2(ds[0][0], ds[0][1]), pack_bf16x2(ds[0][2], ds[0][3]),
                         pack_bf16x2(ds[1][0], ds[1][1]), pack_bf16x2(ds[1][2], ds[1][3])};
      // B operands (column n = d 16*dt + m16, the same contraction slots):
      // transposing reads of rows 4*q4 + (m16 >> 2) and 16 + 4*q4 + (m16 >> 2)
      // at d 16*dt + 4*(m16 & 3); lane m16 then holds columns 4*q4 .. 4*q4 + 3
      // (and 16 + ...) of its d.
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int o1 = tr_row1 + 8 * ((2 * dt) ^ tr_x1) + tr_e;
        const int o2 = tr_row2 + 8 * ((2 * dt) ^ tr_x2) + tr_e;
        const u32x2 dlo = ld_tr16(&sm.g.dor[o1]), dhi = ld_tr16(&sm.g.dor[o2]);
        dva[dt] = mfma_16x16x32(pa, u32x4{dlo[0], dlo[1], dhi[0], dhi[1]}, dva[dt]);
        const u32x2 qlo = ld_tr16(&sm.g.qr[o1]), qhi = ld_tr16(&sm.g.qr[o2]);
        dka[dt] = mfma_16x16x32(dsa, u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, dka[dt]);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        *reinterpret_cast<u32x2*>(&sm.g.ds[ds_off(mykey, 4 * ct + q4)]) = u32x2{dsa[2 * ct], dsa[2 * ct + 1]};
      __syncthreads();

      // dq slice: rows d 16*(dt0 + n) + 4*q4 + r of column 16*dct + m16.
      {
        f32x4 acc[NDT];
#pragma unroll
        for (int n = 0; n < NDT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        // B operand (column n = 16*dct + m16, contraction slots = keys
        // 32*kc + 8*q4 + i) by two transposing reads of keys +0..3 and +4..7.
        const int dkey = 8 * q4 + (m16 >> 2), dch = 4 * dct + (m16 & 3);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const u32x2 lo = ld_tr16(&sm.g.ds[ds_off(32 * kc + dkey, dch)]);
          const u32x2 hi = ld_tr16(&sm.g.ds[ds_off(32 * kc + dkey + 4, dch)]);
          const u32x4 bop = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int n = 0; n < NDT; ++n) acc[n] = mfma_16x16x32(ktop[n][kc], bop, acc[n]);
        }
        const uint64_t prow = sm.g.prow[grp & 1][16 * dct + m16];
#pragma unroll
        for (int n = 0; n < NDT; ++n) {
          u32x2 o;
          o[0] = pack_bf16x2(acc[n][0], acc[n][1]);
          o[1] = pack_bf16x2(acc[n][2], acc[n][3]);
          *reinterpret_cast<u32x2*>(part_dq + prow + 16 * (dt0 + n) + 4 * q4) = o;
        }
      }
    }
  }
  // Rows 16*w + 4*q4 + r, d 16*dt + m16.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = s0 + 16 * w + 4 * q4 + r;
    if (s >= n_kv) continue;
    const int64_t base = ((int64_t)b * n_kv + s) * rs + (int64_t)g * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dk[base + 16 * dt + m16] = (uint16_t)bf16_bits(dka[dt][r] * scale);
      dv[base + 16 * dt + m16] = (uint16_t)bf16_bits(dva[dt][r]);
    }
  }
}

// Persistent: one workgroup per CU takes the lists in order from a counter
// that the launch zeroes beforehand (one vector atomic per list, broadcast
// through LDS); launching one workgroup per list left CUs idle between
// workgroups.  Every wave of a workgroup sees the same item, so all leave the
// loop together.
template <int D, int LOG2G>
__global__ __launch_bounds__(kBwdThreads, 1) void sparse_bwd_kv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dcol,
    const int* __restrict__ off, const int* __restrict__ entries, uint16_t* __restrict__ part_dq,
    int64_t sink_off, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int batch, int n_q, int n_kv, int pos0,
    int h_q, int h_kv, int nblk, int topk, float sl2, float scale, int* __restrict__ counter, int nlists) {
  __shared__ BwdLds<D> sm;
  for (;;) {
    if (threadIdx.x == 0) sm.item = atomicAdd(counter, 1);
    __syncthreads();
    const int item = sm.item;
    if (item >= nlists) break;
    bwd_list<D, LOG2G>(sm, q, k, v, dout, lse, dcol, off, entries, part_dq, sink_off, dk, dv, batch, n_q, n_kv, pos0,
                       h_q, h_kv, nblk, topk, sl2, scale, item);
    __syncthreads();                                   // the next list reuses the LDS
  }
}

__global__ void bwd_counter_reset(int* counter) { *counter = 0; }

// dq[t, h] = scale * (sum over the live slots of the row's partials): the
// partials hold sum dS k unscaled, so the scale costs one multiply per
// element here instead of one per partial element.  Every slot is loaded from
// an in-row address and dead ones are dropped with selects.
template <int D, int G>
__global__ __launch_bounds__(256) void sum_dq_partials(const uint16_t* __restrict__ part_dq,
                                                       const int32_t* __restrict__ blk, uint16_t* __restrict__ dq,
                                                       int64_t nrows, int n_q, int pos0, int h_q, int topk,
                                                       float scale) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;   // (b * n_q + t) * h_q + h
  if (row >= nrows) return;
  const int dl = threadIdx.x % TPR;
  const int h = (int)(row % h_q);
  const int64_t bt = row / h_q;
  const int t = (int)(bt % n_q);
  const int g = h / G, hh = h % G, h_kv = h_q / G;
  const int jl = (pos0 + t) / kBlock;
  const int64_t unit0 = (bt * h_kv + g) * topk;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < topk; s0 += 8) {
    u32x4 o[8];
    bool on[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = min(s0 + i, topk - 1);
      const int jb = blk[unit0 + s];
      on[i] = (s0 + i < topk) && jb >= 0 && jb <= jl;
      o[i] = ld16(part_dq + ((unit0 + s) * G + hh) * D + dl * 8);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t ov = on[i] ? o[i][e] : 0u;
        acc[2 * e] += bf16_to_f32(ov & 0xffffu);
        acc[2 * e + 1] += bf16_to_f32(ov >> 16);
      }
  }
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * scale, acc[2 * e + 1] * scale);
  st16(dq + row * D + dl * 8, r);
}

template <int D, int LOG2G>
hipError_t launch_bwd_t(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* blk, const uint16_t* out, const float* lse, const uint16_t* dout,
                        float scale, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, hipStream_t stream) {
  constexpr int G = 1 << LOG2G;
  constexpr int TPR = D / 8;
  const PrefillWs L = prefill_ws_layout(d);
  char* base = static_cast<char*>(ws);
  const int* off = reinterpret_cast<const int*>(base + L.off);
  const int* entries = reinterpret_cast<const int*>(base + L.entries);
  uint16_t* part_dq = reinterpret_cast<uint16_t*>(base + L.part_o);
  float* dcol = reinterpret_cast<float*>(base + L.part_ml);
  const int64_t nrows = (int64_t)d.batch * d.n_q * d.h_q;
  const int64_t row_wgs = (nrows + 256 / TPR - 1) / (256 / TPR);
  if (nrows > 0) {
    LaunchTimer timer("bwd_row_dot", stream);
    hipLaunchKernelGGL(bwd_row_dot<D>, dim3((unsigned)row_wgs), dim3(256), 0, stream, out, dout, dcol, nrows);
  }
  hipError_t e = launch_csr(d, blk, ws, stream, true);    // sums run in list order
  if (e != hipSuccess) return e;
  int* counter = reinterpret_cast<int*>(base + L.counter);
  hipLaunchKernelGGL(bwd_counter_reset, dim3(1), dim3(1), 0, stream, counter);
  {
    LaunchTimer timer("sparse_bwd_kv", stream);
    hipLaunchKernelGGL((sparse_bwd_kv<D, LOG2G>), dim3((unsigned)std::min<int64_t>(device_cu_count(), L.lists)),
                       dim3(kBwdThreads), 0, stream, q, k, v, dout, lse, dcol, off, entries, part_dq,
                       L.entries_max * G * D, dk, dv, d.batch, d.n_q, d.n_kv, d.pos0, d.h_q, d.h_kv, d.nblk(), d.topk,
                       scale * kLog2e, scale, counter, (int)L.lists);
  }
  if (nrows > 0) {
    LaunchTimer timer("sum_dq_partials", stream);
    hipLaunchKernelGGL((sum_dq_partials<D, G>), dim3((unsigned)row_wgs), dim3(256), 0, stream, part_dq, blk, dq,
                       nrows, d.n_q, d.pos0, d.h_q, d.topk, scale);
  }
  return hipGetLastError();
}

template <int D>
hipError_t bwd_by_group(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* blk,
                        const uint16_t* out, const float* lse, const uint16_t* dout, float scale, uint16_t* dq,
                        uint16_t* dk, uint16_t* dv, void* ws, hipStream_t s) {
  switch (d.group()) {
    case 1: return launch_bwd_t<D, 0>(d, q, k, v, blk, out, lse, dout, scale, dq, dk, dv, ws, s);
    case 2: return launch_bwd_t<D, 1>(d, q, k, v, blk, out, lse, dout, scale, dq, dk, dv, ws, s);
    case 4: return launch_bwd_t<D, 2>(d, q, k, v, blk, out, lse, dout, scale, dq, dk, dv, ws, s);
    case 8: return launch_bwd_t<D, 3>(d, q, k, v, blk, out, lse, dout, scale, dq, dk, dv, ws, s);
    default: return launch_bwd_t<D, 4>(d, q, k, v, blk, out, lse, dout, scale, dq, dk, dv, ws, s);
  }
}

}  // namespace

hipError_t launch_sparse_prefill_backward(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                          const int32_t* blk, const uint16_t* out, const float* lse,
                                          const uint16_t* dout, float scale, uint16_t* dq, uint16_t* dk,
                                          uint16_t* dv, void* ws, hipStream_t stream) {
  if (d.d == 128) return bwd_by_group<128>(d, q, k, v, blk, out, lse, dout, scale, dq, dk, dv, ws, stream);
  return bwd_by_group<64>(d, q, k, v, blk, out, lse, dout, scale, dq, dk, dv, ws, stream);
}

}  // namespace msa
