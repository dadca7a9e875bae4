// Exact wave-level top-k selection without sorting or exponentials
// (lumi-systems summary: exponential-free top-k), shared by the top-k kernels
// and the decode index scan.  Scores become order-preserving unsigned keys;
// 64-lane ballots find thresholds bit by bit; ties go to the lower element.
//
// A wave holds a row's scores in registers (element e = 64*i + lane
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
#pragma once

#include "msa_device.h"

namespace msa {

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

}  // namespace msa
