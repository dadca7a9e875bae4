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
// Three kernels: the per-row coefficients; a KV-outer pass, one workgroup per
// (b, block), that recomputes the scores of every entry of the block's lists
// (all groups share the index key) by MFMA, takes each entry's argmax and
// accumulates dk_idx for the block's keys in LDS in list order (deterministic,
// no atomics); and a per-row gather for dq_idx.
#include "launch.h"
#include "msa_device.h"

namespace msa {
namespace {

constexpr int kIbThreads = 512;
constexpr int kIbCols = 32;                            // entries per group

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
  float dk[kBlock * DI];                               // dk_idx of the block's keys
  union {
    uint16_t k[kBlock * DI];                           // the block's index keys, while loaded
    struct {
      // q rows and coefficients by group parity: the dk phase of one group
      // reads them while faster waves already stage the next group.
      uint16_t qr[2][kIbCols * DI];                    // [entry][d] index queries
      float coef[2][kIbCols];
      int plim[kIbCols];                               // last visible position, -1 for an empty column
      // ((b * n_q + t) * h_kv + g) * topk + slot, -1 if empty; by group parity
      // (wave 0 publishes a group's argmax while faster waves stage the next).
      int slot_row[2][kIbCols];
      float wmax[8][kIbCols];                          // each wave's max per column
      int wkey[8][kIbCols];                            // and the lowest key in the block that has it
    } g;
  };
  int lstart[kIbMaxLists + 1];                         // flat column where group g's list starts
  int lbase[kIbMaxLists];                              // its first entry
};

// One column group in flight: this thread's 16-byte chunk of its column's
// index query, the column's coefficient, last visible position and slot row,
// and the entry (value and group) that this buffer loads next.
struct IbStage {
  u32x4 q;
  float coef;
  int plim, srow, en_next, g_next;
};

template <int DI>
__global__ __launch_bounds__(kIbThreads, 1) void index_bwd_kv(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const int* __restrict__ off,
    const int* __restrict__ entries, const float* __restrict__ coef, int* __restrict__ amax_out, int sink,
    float* __restrict__ dk_idx, int batch, int n_q, int n_kv, int pos0, int h_kv, int nblk, int topk) {
  constexpr int DC = DI / 8;
  constexpr int NST = kIbCols * DC;                    // staging threads (one chunk each)
  __shared__ IbLds<DI> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m16 = lane & 15, q4 = lane >> 4;
  const int j = blockIdx.x / batch, b = blockIdx.x % batch;   // early blocks (most entries) first
  const int s0 = j * kBlock;
  const uint16_t* kb = k_idx + (int64_t)b * n_kv * DI;

  for (int i = tid; i < kBlock * DI; i += kIbThreads) sm.dk[i] = 0.f;
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
    sm.lstart[h_kv] = run;
  }
  __syncthreads();
  // B operands of S^T: column (MFMA n) = this lane's key, contraction slots
  // 8*q4 + i = d 32*c + 8*q4 + i.
  const int mykey = 16 * w + m16;
  u32x4 kop[DI / 32];
#pragma unroll
  for (int c = 0; c < DI / 32; ++c) kop[c] = ld16(&sm.k[rt_off<DI>(mykey, 4 * c + q4)]);
  const int ncols = sm.lstart[h_kv];
  __syncthreads();                                     // the LDS now holds entry groups
  const int skey = s0 + mykey;
  const int ngroups = (ncols + kIbCols - 1) / kIbCols;

  if (ngroups > 0) {
    // Staging role: column scol of each group, chunk sch of its query.
    // Threads beyond NST (d_idx = 64) mirror the first NST.
    const int st_id = tid % NST, scol = st_id / DC, sch = st_id % DC;
    // Flat column f -> (entry value, group); f is clamped to a real column,
    // so no load of the loop sits behind a branch.
    auto entry_at = [&](int grp, int& gout) {
      const int f = min(grp * kIbCols + scol, ncols - 1);
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
      const bool live = grp * kIbCols + scol < ncols;
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
    const auto fmax = [](float x, float y) { return vmax(x, y); };
    auto step = [&](IbStage& st, int grp) {
      const int par = grp & 1;
      // Every thread of a column writes the same per-column values.
      st16(&sm.g.qr[par][rt_off<DI>(scol, sch)], st.q);
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
          sacc[ct] = mfma_16x16x32(kop[c], ld16(&sm.g.qr[par][rt_off<DI>(16 * ct + m16, 4 * c + q4)]), sacc[ct]);
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
      // dk_idx rows of this wave's keys, columns in list order: a ballot over
      // the 32 argmax keys picks this wave's columns.
      {
        uint64_t hits = ballot(lane < kIbCols && key >= 0 && (key >> 4) == w);
        while (hits) {
          const int col = __builtin_ctzll(hits);
          hits &= hits - 1;
          const int kc = __builtin_amdgcn_readlane(key, col);
          const float cf = sm.g.coef[par][col];
#pragma unroll
          for (int d0 = 0; d0 < DI; d0 += 64) {
            const int d = d0 + lane;
            const float qv = bf16_to_f32(sm.g.qr[par][rt_off<DI>(col, d >> 3) + (d & 7)]);
            sm.dk[kc * DI + d] = fmaf(cf, qv, sm.dk[kc * DI + d]);
          }
        }
      }
    };
    __builtin_amdgcn_s_waitcnt(0);                     // drain the prologue (exact waits in the loop)
    for (int grp = 0; grp < ngroups; grp += 2) {
      step(sx, grp);
      step(sy, grp + 1);
    }
  }
  __syncthreads();
  for (int i = tid; i < kBlock * DI; i += kIbThreads) {
    const int s = s0 + i / DI;
    if (s < n_kv) dk_idx[((int64_t)b * n_kv + s) * DI + (i % DI)] = sm.dk[i];
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
  {
    LaunchTimer timer("index_bwd_kv", stream);
    hipLaunchKernelGGL(index_bwd_kv<DI>, dim3((unsigned)(d.batch * d.nblk())), dim3(kIbThreads), 0, stream, q_idx,
                       k_idx, off, entries, coef, amax, (int)(nrows * d.topk), dk_idx, d.batch, d.n_q, d.n_kv,
                       d.pos0, d.h_kv, d.nblk(), d.topk);
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
