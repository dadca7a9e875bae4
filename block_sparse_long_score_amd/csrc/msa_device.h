// Device-side building blocks shared by the MSA kernels (gfx950 / CDNA4).
//
// Conventions used by every kernel in this library:
//   * bf16 values travel as uint16_t bit patterns; arithmetic is fp32.
//   * MFMA: v_mfma_f32_16x16x32_bf16.  For one 16x16 output tile D = A * B:
//       lane l supplies A[row = l % 16][k = 8*(l/16) .. 8*(l/16)+7]
//       lane l supplies B[k = 8*(l/16) .. +7][col = l % 16]
//       lane l receives D[row = 4*(l/16) + r][col = l % 16], r = 0..3.
//     The contraction is a sum, so any assignment of contraction indices to
//     the 32 (lane-group, element) slots works as long as A and B agree; the
//     attention kernels use that freedom to feed softmax probabilities straight
//     from the score accumulators into the P*V product.
//   * Scores are computed transposed, S^T = K * Q^T: keys are MFMA rows and
//     query columns are MFMA columns, so a per-query reduction over keys is a
//     reduction inside a lane plus two cross-lane steps (xor 16, xor 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBlock = 128;   // KV block size B (tokens); the only size supported

// A CSR entry packs (query token t, selection slot): t << kSlotBits | slot.
constexpr int kSlotBits = 6;  // topk <= 64
__device__ __forceinline__ int entry_token(int en) { return en >> kSlotBits; }
__device__ __forceinline__ int entry_slot(int en) { return en & ((1 << kSlotBits) - 1); }

__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: lane l supplies A[row = l % 32][k = 8*(l/32) .. +7]
// and B[k = 8*(l/32) .. +7][col = l % 32]; accumulator element v of lane l is
// D[row = 8*(v/4) + 4*(l/32) + v%4][col = l % 32].
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 pair, packed low|high: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Position of sequence b's first query: pos0, or with per-sequence lengths
// seq_len[b] - n_q, the length clamped into [n_q, n_kv] so that every access
// stays inside the cache whatever the array holds.
__device__ __forceinline__ int seq_pos0(const int* __restrict__ seq_len, int b, int pos0, int n_q, int n_kv) {
  if (!seq_len) return pos0;
  return min(max(seq_len[b], n_q), n_kv) - n_q;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) {
  return __shfl_xor(v, m, 64);
}

// IEEE-754 maximum (NaN-propagating).  Lowers to v_maximum3_f32 on gfx950
// without the canonicalising v_max_f32 x, x, x that fmaxf needs on every MFMA
// result; inputs here are finite or -inf, so the NaN rule never matters.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max over the four lane groups (l/16) that share a column.
__device__ __forceinline__ float colgroup_max(float v) {
  v = vmax(v, shfl_xor_f(v, 16));
  v = vmax(v, shfl_xor_f(v, 32));
  return v;
}

__device__ __forceinline__ float colgroup_sum(float v) {
  v += shfl_xor_f(v, 16);
  v += shfl_xor_f(v, 32);
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Reductions over the R lanes of a row: DPP moves inside each row of 16 lanes
// (swap neighbours, swap pairs, mirror within 8, mirror within 16; after each
// step every lane holds the reduction of its group), then one cross-row swap
// when R >= 32 (and a second one when R == 64).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

template <int R, typename Op>
__device__ __forceinline__ float row_reduce(float v, Op op) {
  v = op(v, dpp_f<0xb1>(v));                           // quad_perm [1,0,3,2]
  v = op(v, dpp_f<0x4e>(v));                           // quad_perm [2,3,0,1]
  v = op(v, dpp_f<0x141>(v));                          // row_half_mirror
  v = op(v, dpp_f<0x140>(v));                          // row_mirror
  if constexpr (R >= 32) v = op(v, shfl_xor_f(v, 16));
  if constexpr (R == 64) v = op(v, shfl_xor_f(v, 32));
  return v;
}

// [row][d] tiles in LDS (rows of D bf16): 16-byte chunk c of row r sits at
// c ^ row_swz(r), so 16 consecutive rows read at the same chunk hit 16
// different bank groups.
template <int D>
__device__ __forceinline__ int row_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int rt_off(int r, int chunk) { return r * D + 8 * (chunk ^ row_swz<D>(r)); }

// Row-major [column][d] tiles of query-side rows (q, dout, index queries) read
// both as MFMA rows and, transposed, as contraction rows: 16-byte chunk c of
// row r sits at c ^ qd_swz(r).  The LDS has 64 four-byte banks; an 8-byte read (the
// transposing one included) serves lanes 0-31 in one cycle and 32-63 in the
// next, a 16-byte read serves in each cycle the 16 lanes with the same lane
// index mod 4 (measured with the bank-conflict counter).  Two reads use these
// tiles.  The S^T / dP^T operands: lane (q4, m16) reads row 16*ct + m16 at
// chunk 4*c + q4, so for rows with equal bits 0-1, bits 2-3 of qd_swz must be a
// bijection of row bits 2-3.  The dV / dK operands (transposing reads): lane
// (q4, m16) reads row 4*q4 + (m16 >> 2) (+ 16) at chunk 2*dt + ((m16 & 3) >> 1),
// so for rows with equal bit 3, bits 1-3 of qd_swz must be a bijection of row
// bits 0-2.  With s0 = r3, s1 = r0, s2 = r1 ^ r2, s3 = r2 ^ r3 (d = 128) both
// hold, and neither read has a bank conflict.  For d = 64 (rows of 128 bytes,
// the row parity picks the half of the banks) the transposing reads are free of
// conflicts and the S^T / dP^T reads conflict 2-way, as with any swizzle.
template <int D>
__device__ __forceinline__ int qd_swz(int r) {
  if (D == 128)
    return ((r >> 3) & 1) | ((r & 1) << 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 3);
  return ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}
template <int D>
__device__ __forceinline__ int qd_off(int r, int chunk) { return r * D + 8 * (chunk ^ qd_swz<D>(r)); }

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element i & 3 of the 8 bytes that lane 4r + (i >> 2)
// addresses, as its element r (r = 0..3).
__device__ __forceinline__ u32x2 ld_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}



// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// One KV block of one K/V head staged in LDS, rows 16-byte aligned and
// unpadded; 16-byte chunks are XOR-swizzled per row (chunk c of row r sits at
// c ^ tile_swz(r)) so that every staging write and operand read below touches
// each bank the minimum number of times.
//   k  : [128 keys][D]       row-major.
//   vt : [D][128 keys]       V transposed (d-major): the P*V operand of 8
//                            consecutive keys at a fixed d is one chunk.
// Key order inside the score tiles: MFMA row m of key tile kt holds key
//   kt_key(kt, m) = 32*(kt/2) + 8*(m/4) + 4*(kt%2) + m%4,
// so lane group q of a column ends up with keys 32*kc + 8*q + [0, 8) in the two
// tiles 2*kc, 2*kc+1 -- exactly one chunk of a vt row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kt_key(int kt, int m) { return 32 * (kt >> 1) + 8 * (m >> 2) + 4 * (kt & 1) + (m & 3); }
__device__ __forceinline__ int tile_swz(int r) { return (((r >> 3) & 3) << 2) | (r & 3); }

template <int D>
struct KVTile {
  static constexpr int DC = D / 8;          // 16-byte chunks per K row
  uint16_t k[kBlock * D];
  uint16_t vt[D * kBlock];
  __device__ __forceinline__ const uint16_t* k_chunk(int row, int c) const {
    return &k[row * D + 8 * (c ^ (tile_swz(row) & (DC - 1)))];
  }
  __device__ __forceinline__ const uint16_t* vt_chunk(int d, int c) const {
    return &vt[d * kBlock + 8 * (c ^ tile_swz(d))];
  }
};

// Staging of one K/V block by a 512-thread workgroup through registers, so the
// next block's loads can be in flight while the current block is used.
constexpr int kKvThreads = 512;
// Third word of a buffer descriptor: raw 32-bit data, no swizzle or stride.
constexpr int kBufferWord3 = 0x00020000;

// Registers of one K/V block in flight: K as 16-byte chunks, V as 4-key x
// 8-dim tiles that are transposed into the vt rows when written to LDS.
// V tile w covers keys 4*kq .. 4*kq + 3 and dims 8*dg .. 8*dg + 7; each group
// of 16 consecutive threads takes 4 key quads x 4 dim groups, so its loads
// read 64-byte runs of 4 rows and its transposed 8-byte writes (rows
// 8*dg + e) reach 16 different 8-byte slots of the 64 banks (16 dim groups
// of one key quad, the plain order, hit only 4).
template <int D>
struct KVPrefetch {
  static constexpr int DC = D / 8;
  static constexpr int KI = kBlock * DC / kKvThreads;            // K chunks per thread
  static constexpr int VQ = (kBlock / 4) * DC;                    // V tiles per block
  static constexpr int VI = (VQ + kKvThreads - 1) / kKvThreads;   // V tiles per thread
  static_assert(KI * kKvThreads == kBlock * DC, "K staging must divide evenly");
  static_assert(DC % 4 == 0 && VQ % 16 == 0, "V tiles go in groups of 4 key quads x 4 dim groups");
  u32x4 kr[KI];
  u32x4 vr[VI][4];

  __device__ __forceinline__ static void v_tile(int w, int& kq, int& dg) {
    const int g = w >> 4, l = w & 15;
    kq = (g / (DC / 4)) * 4 + (l >> 2);
    dg = (g % (DC / 4)) * 4 + (l & 3);
  }

  __device__ __forceinline__ void fetch(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                        int64_t rs, int s0, int n_kv, int tid) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int w = tid + i * kKvThreads, key = w / DC, dc = w % DC;
      const int s = s0 + key;
      kr[i] = s < n_kv ? ld16(kb + (int64_t)s * rs + dc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int w = tid + i * kKvThreads;
      int kq, dg;
      v_tile(w, kq, dg);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = s0 + 4 * kq + r;
        vr[i][r] = (w < VQ && s < n_kv) ? ld16(vb + (int64_t)s * rs + dg * 8) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // Loads through buffer descriptors (scalar base, one 32-bit vector offset
  // per thread, no 64-bit vector arithmetic).  A descriptor covers only keys
  // below n_kv, and the hardware returns zeros for a load whose vector offset
  // is past its range, so a partial last block and a block past the end (no
  // key in range, no memory touched) need no branch.  The range check does
  // not see the scalar offset, so each group of rows a thread loads with one
  // vector offset gets a descriptor of its own, based at the group's first
  // row.  Key rows are at least D elements apart, so a 16-byte piece of a row
  // is either wholly inside a range or wholly past it.
  //   rsrc(base, rs, first, stride_rows, n_kv): rows first + stride_rows * m
  //   of the block are in range for m * stride_rows <= n_kv - 1 - first.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int64_t rs, int first,
                                                                     int n_kv) {
    const int rows = n_kv - first;                                     // keys at or after `first`
    const int bytes = rows > 0 ? (rows - 1) * (int)rs * 2 + D * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + (int64_t)first * rs), (short)0, bytes,
                                             kBufferWord3);
  }

  __device__ __forceinline__ void fetch_k_buf(const uint16_t* __restrict__ kb, int64_t rs, int s0, int n_kv,
                                              int tid) {
    static_assert(kKvThreads % DC == 0, "a thread's K chunks are whole key rows apart");
    const uint32_t rsb = (uint32_t)rs * 2u;                        // key row stride in bytes
    const uint32_t koff = (uint32_t)(tid / DC) * rsb + (uint32_t)(tid % DC) * 16u;
    const int lim = min(n_kv, s0 + kBlock);                        // keys of this block below n_kv
#pragma unroll
    for (int i = 0; i < KI; ++i)
      kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rows_rsrc(kb, rs, s0 + i * (kKvThreads / DC), lim), koff, 0, 0));
  }

  __device__ __forceinline__ void fetch_v_buf(const uint16_t* __restrict__ vb, int64_t rs, int s0, int n_kv,
                                              int tid) {
    const uint32_t rsb = (uint32_t)rs * 2u;
    const int lim = min(n_kv, s0 + kBlock);
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int w = tid + i * kKvThreads;
      int kq, dg;
      v_tile(w, kq, dg);
      const uint32_t voff = (uint32_t)(4 * kq) * rsb + (uint32_t)dg * 16u;   // row 4 kq of the group
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        if (VI * kKvThreads == VQ || w < VQ)
          vr[i][rr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rows_rsrc(vb, rs, s0 + rr, lim), voff, 0, 0));
        else
          vr[i][rr] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // A block whose 128 keys are all below n_kv: one descriptor per tensor, the
  // row steps in the scalar offset (nothing to range-check).
  __device__ __forceinline__ void fetch_full(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                             int64_t rs, int s0, int tid) {
    const uint32_t rsb = (uint32_t)rs * 2u;
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kb, rs, s0, s0 + kBlock);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vb, rs, s0, s0 + kBlock);
    const uint32_t koff = (uint32_t)(tid / DC) * rsb + (uint32_t)(tid % DC) * 16u;
#pragma unroll
    for (int i = 0; i < KI; ++i)
      kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, i * (kKvThreads / DC) * rsb, 0));
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int w = tid + i * kKvThreads;
      int kq, dg;
      v_tile(w, kq, dg);
      const uint32_t voff = (uint32_t)(4 * kq) * rsb + (uint32_t)dg * 16u;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        if (VI * kKvThreads == VQ || w < VQ)
          vr[i][rr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, rr * rsb, 0));
        else
          vr[i][rr] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void fetch_buf(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                            int64_t rs, int s0, int n_kv, int tid) {
    if (s0 + kBlock <= n_kv) {
      fetch_full(kb, vb, rs, s0, tid);
    } else {
      fetch_k_buf(kb, rs, s0, n_kv, tid);
      fetch_v_buf(vb, rs, s0, n_kv, tid);
    }
  }

  __device__ __forceinline__ void stash(KVTile<D>& t, int tid) const {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int w = tid + i * kKvThreads, key = w / DC, dc = w % DC;
      st16(&t.k[key * D + 8 * (dc ^ (tile_swz(key) & (DC - 1)))], kr[i]);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int w = tid + i * kKvThreads;
      if (w >= VQ) continue;
      int kq, dg;
      v_tile(w, kq, dg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int word = e >> 1, sh = (e & 1) * 16, d = dg * 8 + e;
        u32x2 o;
        o[0] = ((vr[i][0][word] >> sh) & 0xffffu) | (((vr[i][1][word] >> sh) & 0xffffu) << 16);
        o[1] = ((vr[i][2][word] >> sh) & 0xffffu) | (((vr[i][3][word] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(&t.vt[d * kBlock + 8 * ((kq >> 1) ^ tile_swz(d)) + 4 * (kq & 1)]) = o;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Attention of up to 32 query columns (two 16-column MFMA tiles) against the
// staged block, for one wave.
//
// qrow[ct]      : pointer to the D-vector of this lane's column in tile ct
//                 (column = l % 16), or nullptr for an empty column (reads 0).
// plim[ct]      : last visible absolute key position for this lane's column;
//                 keys s0 + key > plim are masked.
// need_mask     : wave-uniform; false when every key of the block is visible
//                 to every column.
// block_scores_softmax returns, per lane and tile ct (replicated over the four
// lane groups of a column): bmax = block max of the scaled logits in log2
// units, mref = the max the exponentials were taken against (bmax, or for
// online softmax max(previous mref, bmax)), bsum = sum of exp2(logit2 - mref).
// block_pv then accumulates the unnormalised P*V.
// ---------------------------------------------------------------------------

template <int D>
__device__ __forceinline__ void load_q_operand(u32x4 (&qb)[2][D / 32], const uint16_t* const (&qrow)[2]) {
  const int q = lane_id() >> 4;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc)
      qb[ct][cc] = qrow[ct] ? ld16(qrow[ct] + cc * 32 + q * 8) : u32x4{0u, 0u, 0u, 0u};
}

// Computes S^T for the block and its block-local softmax pieces.  Writes the
// probabilities (bf16, already laid out as the B operand of the P*V MFMA) into
// pb and returns the block max / sum per column.
template <int D>
__device__ __forceinline__ void block_scores_softmax(const KVTile<D>& t, const u32x4 (&qb)[2][D / 32],
                                                     float sl2, int s0, const int (&plim)[2], bool need_mask,
                                                     float (&bmax)[2], float (&bsum)[2],
                                                     u32x4 (&pb)[2][4], float (&mref)[2], bool use_mref) {
  const int lane = lane_id();
  const int col = lane & 15, q = lane >> 4;
  (void)col;
  f32x4 s[8][2];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) s[kt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(t.k_chunk(kt_key(kt, lane & 15), 4 * cc + q));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) s[kt][ct] = mfma_16x16x32(a, qb[ct][cc], s[kt][ct]);
    }
    // keep the LDS operand reads of later key tiles from being hoisted (register pressure)
    if (kt & 1) __builtin_amdgcn_sched_barrier(0);
  }
  // Causal mask (only blocks that reach past some column's position).
  if (need_mask) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int kt = 0; kt < 8; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (s0 + kt_key(kt, 4 * q + r) > plim[ct]) s[kt][ct][r] = -INFINITY;
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    // The max of the raw scores times sl2 > 0 is the max of the rounded scaled
    // scores (rounding is monotone), so one FMA per score forms the exponent.
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = vmax(mx, s[kt][ct][r]);
    mx = colgroup_max(mx) * sl2;
    bmax[ct] = mx;
    // Reference max for the exponentials: the block max, or (online softmax)
    // the caller's running max merged with it.
    const float mr = use_mref ? vmax(mref[ct], mx) : mx;
    mref[ct] = mr;
    float sum = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      float p[8];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[2 * kc + hlf][ct][r], sl2, -mr));
          p[hlf * 4 + r] = e;
          sum += e;
        }
      pb[ct][kc] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                         pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    }
    bsum[ct] = colgroup_sum(sum);
  }
}

// acc[ct][pp][half] += V^T * P^T for the block.  acc rows are permuted so that
// lane group q ends up holding d = 32*pp + 8*q + 4*half + r; the contraction
// slots of lane group q are keys 32*kc + 8*q + [0, 8) on both operands.
template <int D>
__device__ __forceinline__ void block_pv(const KVTile<D>& t, const u32x4 (&pb)[2][4],
                                         f32x4 (&acc)[2][D / 32][2]) {
  const int lane = lane_id();
  const int m = lane & 15, q = lane >> 4;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int pp = 0; pp < D / 32; ++pp)
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int d = 32 * pp + 8 * (m >> 2) + 4 * hlf + (m & 3);
        const u32x4 a = *reinterpret_cast<const u32x4*>(t.vt_chunk(d, 4 * kc + q));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[ct][pp][hlf] = mfma_16x16x32(a, pb[ct][kc], acc[ct][pp][hlf]);
      }
  }
}


// ---------------------------------------------------------------------------
// Decode-shaped attention: the G <= 16 query heads of one (sequence, group)
// against blocks [j_begin, j_end) of that group's K/V, with online softmax
// across the blocks.  One wave, no LDS staging of K/V: K streams from HBM
// straight into MFMA A operands (S^T = K * Q^T, heads are the columns), V
// streams with 16-byte loads into a VALU accumulation.  pt is this wave's LDS
// scratch of kBlock * 16 + 16 floats (probabilities and per-head rescales).
//
// Writes the unnormalised partial o = sum exp2(logit2 - m2) * v (bf16, [G][D])
// and (m2, l) per head, where m2 is the running max of the scaled logits in
// log2 units and l the sum of exp2(logit2 - m2).  Keys past plim (the query position) are masked.
// ---------------------------------------------------------------------------
template <int D, int G>
__device__ __forceinline__ void decode_attend(const uint16_t* __restrict__ qheads,
                                              const uint16_t* __restrict__ kbase,
                                              const uint16_t* __restrict__ vbase, int64_t row_stride,
                                              int n_kv, int plim, int j_begin, int j_end, float sl2,
                                              float* pt, uint16_t* __restrict__ out_o,
                                              float* __restrict__ out_ml) {
  constexpr int CC = D / 32;
  constexpr int LPR = D / 8;          // lanes per V row (16-byte pieces)
  constexpr int KPI = 64 / LPR;       // keys per V load instruction
  const int lane = lane_id();
  const int col = lane & 15, q = lane >> 4;
  const int kg = lane / LPR, dl = lane % LPR;
  float* alpha_s = pt + kBlock * 16;

  u32x4 qb[CC];
#pragma unroll
  for (int cc = 0; cc < CC; ++cc)
    qb[cc] = (col < G) ? ld16(qheads + col * D + cc * 32 + q * 8) : u32x4{0u, 0u, 0u, 0u};

  float m_run = -INFINITY, l_run = 0.f;                 // this lane's column
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  for (int j = j_begin; j < j_end; ++j) {
    const int s0 = j * kBlock;
    u32x4 a[8][CC];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const int s = s0 + kt * 16 + col;
#pragma unroll
      for (int cc = 0; cc < CC; ++cc)
        a[kt][cc] = (s < n_kv) ? ld16(kbase + (int64_t)s * row_stride + cc * 32 + q * 8)
                               : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 sc[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < CC; ++cc) sc[kt] = mfma_16x16x32(a[kt][cc], qb[cc], sc[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[kt][r] * sl2;
        if (s0 + kt * 16 + q * 4 + r > plim) v = -INFINITY;
        sc[kt][r] = v;
        mx = vmax(mx, v);
      }
    mx = colgroup_max(mx);
    const float m_new = vmax(m_run, mx);               // finite: the first block has key s0 <= plim
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(sc[kt][r] - m_new);
        sum += e;
        if (col < G) pt[(kt * 16 + q * 4 + r) * 16 + col] = e;
      }
    sum = colgroup_sum(sum);
    l_run = l_run * alpha + sum;
    m_run = m_new;
    if (q == 0 && col < G) alpha_s[col] = alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // P * V on the vector ALUs: lane (kg, dl) owns d = 8*dl .. 8*dl+7 for keys
    // kg, kg + KPI, ...
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = alpha_s[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al;
    }
#pragma unroll 4
    for (int it = 0; it < kBlock / KPI; ++it) {
      const int key = it * KPI + kg;
      const int s = s0 + key;
      u32x4 vv = {0u, 0u, 0u, 0u};
      if (s < n_kv) vv = ld16(vbase + (int64_t)s * row_stride + dl * 8);
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_to_f32(vv[e] & 0xffffu);
        vf[2 * e + 1] = bf16_to_f32(vv[e] >> 16);
      }
      const float* prow = pt + key * 16;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pr = prow[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Sum the partial P*V over the key groups; lanes of group kg = 0 write.
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
#pragma unroll
      for (int m = LPR; m < 64; m <<= 1) v += shfl_xor_f(v, m);
      acc[h][e] = v;
    }
  }
  // (m, l) of head h lives in lanes with col == h; share them through LDS.
  if (q == 0 && col < G) {
    alpha_s[col] = l_run;
    pt[col] = m_run;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (kg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[h][2 * e], acc[h][2 * e + 1]);
      st16(out_o + h * D + dl * 8, o);
    }
  }
  if (lane < G) {
    out_ml[2 * lane] = pt[lane];
    out_ml[2 * lane + 1] = alpha_s[lane];
  }
}

}  // namespace msa
