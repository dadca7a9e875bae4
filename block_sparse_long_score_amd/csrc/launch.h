// Internal host-side interface between the C-ABI layer and the kernel files.
// Every launcher assumes its arguments were validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Kernel timing hook (msa_profile_begin / msa_profile_end): constructed right
// before a launch, destroyed right after it; records a HIP event pair around
// the launch on its stream while recording is on, and does nothing otherwise.
class LaunchTimer {
 public:
  LaunchTimer(const char* name, hipStream_t stream);
  ~LaunchTimer();
  LaunchTimer(const LaunchTimer&) = delete;
  LaunchTimer& operator=(const LaunchTimer&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

// Compute units of the current device (cached per device id; 256 if the query fails).
int device_cu_count();

struct Dims {
  int batch, n_q, n_kv, pos0, h_q, h_kv, d, d_idx, block, topk;
  // Variable-length decode: per-sequence lengths (device array of `batch`
  // int32) or nullptr.  With it, sequence b holds seq_len[b] tokens of its
  // n_kv-token cache and its n_q queries sit at seq_len[b] - n_q ...; pos0 is
  // not used.
  const int* seq_len = nullptr;
  int nblk() const { return (n_kv + block - 1) / block; }
  int group() const { return h_q / h_kv; }
};

// Sparse-prefill workspace: CSR inversion of the block selection plus the
// per-(query, group, slot) partial softmax results.  Offsets in bytes.
struct PrefillWs {
  size_t cnt, off, ccnt, entries, part_o, part_ml, counter, total;
  int64_t lists, chunks, entries_max;
};
PrefillWs prefill_ws_layout(const Dims& d);
// Builds the per-(b, g, block) lists of (t, slot) entries in the workspace;
// `ordered`: each list sorted by (t, slot), for kernels that sum over a list.
hipError_t launch_csr(const Dims& d, const int32_t* blk, void* ws, hipStream_t stream, bool ordered);

// Decode / dense-decode partials.
struct DecodeWs {
  size_t part_o, part_ml, total;
  int nslot;
};
DecodeWs sparse_decode_ws_layout(const Dims& d);
DecodeWs dense_decode_ws_layout(const Dims& d);

hipError_t launch_index_scores(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, float* bscore,
                               hipStream_t stream);
hipError_t launch_block_topk(const Dims& d, const float* bscore, int32_t* blk_idx, hipStream_t stream);
// Index branch with the top-k fused into the tiled scorer (128-token blocks,
// k <= 16, more than 16 (token, group) rows per sequence): no pooled scores in
// memory; `ws` holds index_topk_fused_ws_bytes(d) bytes of per-row survivor
// lists.
bool index_topk_fused_applies(const Dims& d);
size_t index_topk_fused_ws_bytes(const Dims& d);
hipError_t launch_index_topk_fused(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, int32_t* blk_idx,
                                   void* ws, hipStream_t stream);
// log2 of the selection block size (128 or 256).
inline int block_shift(const Dims& d) { return d.block == 256 ? 8 : 7; }
// 256-token blocks from 128-token ones: pooled scores of pairs (rows of the
// 256-token dims d), and a 256-token selection expanded into 128-token blocks
// (2 * topk per row, ascending, -1 padded).
hipError_t launch_pool_block_pairs(const Dims& d, const float* p128, float* p256, hipStream_t stream);
hipError_t launch_expand_block_pairs(const Dims& d, const int32_t* blk256, int32_t* blk128, hipStream_t stream);
hipError_t launch_sparse_prefill(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* blk_idx, float scale, uint16_t* out, float* lse, void* ws,
                                 hipStream_t stream);
// msa_sparse_prefill, then the index-branch target and its KL from the partials.
hipError_t launch_sparse_prefill_target(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const int32_t* blk, float scale, const float* bscore, float idx_scale,
                                        uint16_t* out, float* lse, float* target, float* kl, void* ws,
                                        hipStream_t stream);
// Gradients of msa_sparse_prefill: dq, dk, dv from dout, the forward's output
// and lse; same workspace layout (partial dq in part_o, row dots in part_ml).
hipError_t launch_sparse_prefill_backward(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                          const int32_t* blk, const uint16_t* out, const float* lse,
                                          const uint16_t* dout, float scale, uint16_t* dq, uint16_t* dk,
                                          uint16_t* dv, void* ws, hipStream_t stream);
// Gradient of the KL alignment loss w.r.t. q_idx and k_idx (fp32 outputs).
hipError_t launch_index_backward(const Dims& d, const uint16_t* q_idx, const uint16_t* k_idx, const int32_t* blk,
                                 const float* bscore, const float* target, const float* dkl, float idx_scale,
                                 float* dq_idx, float* dk_idx, void* ws, hipStream_t stream);
hipError_t launch_sparse_decode(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* blk_idx, float scale, uint16_t* out, float* lse, void* ws,
                                hipStream_t stream);
hipError_t launch_dense_prefill(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                float scale, uint16_t* out, float* lse, hipStream_t stream);
hipError_t launch_merge(const Dims& d, const uint16_t* part_o, const float* part_ml, const int32_t* blk,
                        uint16_t* out, float* lse, int nslot, int per, hipStream_t stream);
hipError_t launch_dense_decode(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               float scale, uint16_t* out, float* lse, void* ws, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The library's own device scratch (msa_index_topk_noalloc): kScratchBytes per
// device, in the code object; its device address on the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_for_current_device(void** ptr);

}  // namespace msa
