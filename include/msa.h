/*
 * msa.h - C ABI of the MiniMax Sparse Attention (MSA) forward path for AMD
 * MI355X (gfx950).
 *
 * The method (as described on the pages this library follows):
 *   - Built on grouped-query attention: h_q query heads in h_kv consecutive
 *     groups, each group sharing one K/V head (Notion notes
 *     "Minimax-sparse-Attention", "what is MHA, MQA, GQA?").
 *   - Index branch: one index query per (token, group), one index key per token
 *     shared by all heads; token score = dot product; scores max-pooled per
 *     KV block; top-k blocks kept per (query, group) (yhxrc.cn article, section
 *     "第一步：索引分支"; hamidun.com news, "Como o MSA funciona"), with no
 *     exponential in the selection (lumi-systems news summary), k = 16 blocks of
 *     128 tokens and the query's own block always included (lefilia.fr
 *     article).
 *   - Main branch: exact softmax attention, on the real K/V, of every head of a
 *     group over only that group's selected blocks (yhxrc.cn article,
 *     "第二步：稀疏分支"; lefilia.fr article).
 *   - The index branch is a separate upstream step whose only output is the
 *     block selection (yhxrc.cn article, "三個刻意的減法", third point), hence
 *     the split between msa_index_topk and msa_sparse_prefill/decode.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, row-major, last dimension
 *     contiguous, 16-byte aligned.  bf16 tensors are passed as uint16_t bit
 *     patterns.  The caller owns every buffer (inputs, outputs, workspace); the
 *     library never allocates, frees or synchronises and keeps no pointer after
 *     returning.  Work is enqueued on `stream` (a hipStream_t, NULL = the null
 *     stream); buffers must stay valid until the stream has passed the work.
 *   - Query i of a call sits at absolute position p = pos0 + i of its
 *     sequence; keys/values/index keys of positions 0 .. n_kv-1 are cached.
 *     Causality is per token: a query sees keys s <= p.
 *   - Block j covers tokens [j*block, min((j+1)*block, n_kv)); the local block
 *     of a query is p / block.  nblk = ceil(n_kv / block).
 *   - Every argument check runs on the host before any HIP call and returns a
 *     status; no exception crosses the ABI.  MSA_ERR_HIP reports a launch
 *     failure; faults inside kernels surface at the caller's next
 *     synchronisation.  Inputs are never written.  Same inputs, same outputs,
 *     bit for bit (no floating-point atomics).  Functions keep no state
 *     between calls and are thread-safe, with two documented exceptions:
 *     msa_index_topk_noalloc (one shared scratch array per GPU) and the
 *     kernel-timing hook (msa_profile_begin / msa_profile_end).
 *   - Supported: block 128 or 256; 1 <= topk <= 64 (<= 32 with block 256);
 *     d, d_idx in {64, 128};
 *     h_q / h_kv in {1, 2, 4, 8, 16}; n_kv <= 1,048,576; pos0 + n_q <= n_kv;
 *     batch * n_q * h_kv * topk < 2^31 (2 * topk with block 256);
 *     n_q * h_kv <= 2^25.  batch == 0 or n_q == 0 is a no-op.
 *   - Block 256 (yhxrc.cn article, "社區沖擊與深層信號": block size and
 *     selection may have to be re-tuned for far longer contexts): a block
 *     of 256 tokens is two of 128, its pooled score the larger of theirs, so
 *     the same pooled scores, selections and outputs follow as with a plain
 *     256-token max-pool; the main branch runs on the two 128-token halves of
 *     each selected block.  msa_index_scores, msa_sparse_prefill_target and
 *     both backward calls take block 128 only (MSA_ERR_UNSUPPORTED).  With
 *     block 256 the index workspace holds the 256-token pooled scores at
 *     offset 0 followed by the 128-token ones, and the sparse workspaces begin
 *     with the expanded 128-token selection.
 *   - NaN or infinite inputs give undefined (but memory-safe) results.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct msa_dims {
  int32_t batch; /* sequences */
  int32_t n_q;   /* query tokens per sequence in this call */
  int32_t n_kv;  /* cached tokens per sequence */
  int32_t pos0;  /* absolute position of query 0 */
  int32_t h_q;   /* query heads */
  int32_t h_kv;  /* K/V heads = GQA groups */
  int32_t d;     /* head dimension of Q, K, V */
  int32_t d_idx; /* dimension of index queries / keys */
  int32_t block; /* KV block size in tokens (128) */
  int32_t topk;  /* blocks selected per (query, group), local block included */
} msa_dims;

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_NULL = 1,        /* a required pointer (or dims) is NULL */
  MSA_ERR_SHAPE = 2,       /* inconsistent sizes: negative, h_q % h_kv, pos0 + n_q > n_kv, decode n_q != 1 */
  MSA_ERR_UNSUPPORTED = 3, /* sizes this build does not implement (see the list above) */
  MSA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  MSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than msa_workspace_size() */
  MSA_ERR_HIP = 6,         /* a kernel launch failed */
  MSA_ERR_TOO_LARGE = 7    /* msa_index_topk_noalloc: more than the library's static scratch */
} msa_status;

typedef enum msa_op {
  MSA_OP_INDEX_TOPK = 0,
  MSA_OP_SPARSE_PREFILL = 1,
  MSA_OP_SPARSE_DECODE = 2,
  MSA_OP_DENSE_GQA = 3,
  MSA_OP_BLOCK_TOPK = 4,
  MSA_OP_INDEX_TOPK_FUSED = 5
} msa_op;

typedef void* msa_stream; /* hipStream_t */

/* Workspace bytes `op` needs for `dims` (0 if it needs none).  Returns 0 for
 * dims the op rejects as well; call the op to get the status. */
size_t msa_workspace_size(msa_op op, const msa_dims* dims);

/* Static, human-readable name of a status. */
const char* msa_status_str(msa_status status);

/* Index branch: scores, block max-pool, top-k with the local block forced.
 * (yhxrc.cn article, "第一步：索引分支"; lumi-systems summary; lefilia.fr.)
 *   q_idx   [batch][n_q][h_kv][d_idx]  bf16   one index query per token and group
 *   k_idx   [batch][n_kv][d_idx]       bf16   one index key per cached token
 *   blk_idx [batch][n_q][h_kv][topk]   int32  out: selected blocks, ascending;
 *           all blocks 0..jl when jl + 1 <= topk (then -1 padding), else jl
 *           plus the topk-1 earlier blocks with the largest pooled score, ties
 *           to the lower block index.
 *   workspace >= msa_workspace_size(MSA_OP_INDEX_TOPK), which may be 0 (then
 *           workspace may be NULL).  Calls with 128-token blocks, topk <= 16
 *           and more than 16 (token, group) rows per sequence run the top-k
 *           fused into the scoring kernel (as msa_index_topk_fused below: no
 *           pooled scores in memory) and leave the workspace's contents
 *           unspecified.  Every other call leaves, at offset 0, the pooled
 *           block scores bscore[batch][n_q][h_kv][nblk] (fp32): entry j <= jl
 *           is max over tokens s of block j with s <= p of q_idx . k_idx[s];
 *           entries j > jl are unspecified.  msa_index_scores gives the pooled
 *           scores of any call (a caller that needs them, as the training
 *           calls below do, runs msa_index_scores + msa_block_topk: one
 *           scoring pass for both).
 * Scores accumulate in fp32; with integer-valued index inputs of magnitude
 * <= 3 and d_idx <= 128 they are exact. */
msa_status msa_index_topk(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx,
                          int32_t* blk_idx, void* workspace, size_t workspace_bytes, msa_stream stream);

/* The index branch with the top-k fused into the scoring kernel, so that the
 * pooled block scores never reach memory (yhxrc.cn article, "第一步：索引分支":
 * scores, block max-pool and top-k as one step; lumi-systems summary: the
 * selection uses no exponential).  msa_index_topk takes this path by itself
 * whenever it applies; this entry point guarantees it (MSA_ERR_UNSUPPORTED
 * otherwise).  Same arguments and the same blk_idx as msa_index_topk, bit for
 * bit:
 *   workspace >= msa_workspace_size(MSA_OP_INDEX_TOPK_FUSED): per (token,
 *           group) row, P lists of up to 15 surviving blocks, where P = 1..16
 *           workgroups sweep each 1,024-row tile (chosen from the sizes alone):
 *           batch * n_q * h_kv * P * 128 bytes, and none when P = 1 (the
 *           workgroup then writes blk_idx itself; workspace may be NULL).  Its
 *           contents on return are unspecified.  At 131,072 tokens x 8 groups
 *           P = 1, against 4 GiB of pooled scores on the unfused path.
 * Each sweeping workgroup keeps every row's best k - 1 blocks so far in LDS as
 * the key blocks stream by (a later block replaces the worst kept one only
 * with a strictly larger score, so ties keep the lower block); with P > 1 a
 * second kernel selects each row's k - 1 best among its P lists and adds the
 * local block.
 *   - MSA_ERR_UNSUPPORTED for block 256, topk > 16, or n_q * h_kv <= 16 (a
 *     decode-shaped call, whose pooled scores are small); msa_workspace_size
 *     then returns 0. */
msa_status msa_index_topk_fused(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx,
                                int32_t* blk_idx, void* workspace, size_t workspace_bytes, msa_stream stream);

/* msa_index_topk without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid allocation.  Same arguments (minus the
 * workspace), same checks and the same blk_idx, bit for bit.  What
 * msa_index_topk keeps in its workspace (pooled scores, or survivor lists on
 * the fused path) goes to a scratch array of 64 MiB that the library keeps in
 * its code object: every GPU the library runs on holds its own copy from the
 * first use until the process ends.  The call itself allocates nothing.
 *   - Returns MSA_ERR_TOO_LARGE when the call needs more than 64 MiB, i.e.
 *     msa_workspace_size(MSA_OP_INDEX_TOPK, dims) > 64 << 20 (for example
 *     batch * n_q * h_kv * nblk > 16,777,216 pooled scores with 128-token
 *     blocks and topk > 16).
 *   - Every call on one GPU uses that GPU's single array, which keeps the last
 *     call's contents: calls whose work overlaps on one GPU (other streams,
 *     other threads) race and give undefined results.  Calls ordered on one
 *     stream are safe.
 *   - The first call on a device looks up the array's device address
 *     (MSA_ERR_HIP if that fails). */
msa_status msa_index_topk_noalloc(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx,
                                  int32_t* blk_idx, msa_stream stream);

/* Scoring and block max-pool alone (the first half of msa_index_topk), for
 * callers that want the pooled scores themselves.
 *   bscore [batch][n_q][h_kv][nblk] fp32 out, as msa_index_topk documents for
 *          its workspace (entries j > jl unspecified). */
msa_status msa_index_scores(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx, float* bscore,
                            msa_stream stream);

/* The top-k step alone, on pooled scores in the layout msa_index_scores writes
 * (lumi-systems summary: exponential-free top-k).
 *   bscore  [batch][n_q][h_kv][nblk] fp32 (only entries j < jl are read)
 *   blk_idx [batch][n_q][h_kv][topk] int32 out, as for msa_index_topk. */
msa_status msa_block_topk(const msa_dims* dims, const float* bscore, int32_t* blk_idx, msa_stream stream);

/* Main branch, prefill: for every head h of group g = h / (h_q / h_kv),
 *   out[b][t][h] = softmax over visible keys s of (scale * q[b][t][h] . k[b][s][g]) applied to v[b][s][g],
 * where s is visible when block(s) is in blk_idx[b][t][g] and s <= p
 * (yhxrc.cn article, "第二步：稀疏分支"; hamidun.com, "Como o MSA funciona").
 *   q   [batch][n_q][h_q][d]   bf16
 *   k,v [batch][n_kv][h_kv][d] bf16
 *   blk_idx [batch][n_q][h_kv][topk] int32 from msa_index_topk, or any
 *           selection of distinct blocks j <= jl (entries < 0 or > jl are
 *           skipped); at least one valid entry per row.
 *   scale   softmax scale; <= 0 means 1/sqrt(d)
 *   out [batch][n_q][h_q][d] bf16 (fp32 accumulation, round-to-nearest-even)
 *   lse [batch][n_q][h_q] fp32 natural-log normaliser of the scaled logits, or NULL
 *   workspace: msa_workspace_size(MSA_OP_SPARSE_PREFILL, dims) bytes run the
 *           call in one pass.  A smaller workspace is accepted as long as it
 *           holds the workspace of one query of one sequence
 *           (msa_workspace_size(MSA_OP_SPARSE_PREFILL) of dims with batch = 1,
 *           n_q = 1): the call then takes each sequence's queries in the
 *           largest chunks whose workspace fits, one after another on the
 *           stream (the same outputs bit for bit; each chunk re-reads the
 *           K/V blocks it selects).  Below that: MSA_ERR_WORKSPACE. */
msa_status msa_sparse_prefill(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* blk_idx, float scale, uint16_t* out, float* lse, void* workspace,
                              size_t workspace_bytes, msa_stream stream);

/* Index-branch training target, forward only (Notion notes
 * "Minimax-sparse-Attention", "KL Loss Alignment" and "Detached Gradients":
 * the main branch's attention distribution is what the index branch is
 * trained to imitate through a KL divergence, and no gradient passes between
 * the branches).  Runs msa_sparse_prefill (same outputs, same workspace) and
 * then, for every (b, t, g) row and from the same partial results:
 *   target[b][t][g][s] = mean over the group's heads h of the share of head h's
 *            softmax weight that falls in block blk_idx[b][t][g][s]
 *            (fp32; each row sums to 1 over its live slots; 0 at padding);
 *   kl[b][t][g] = sum_s target_s * (ln target_s - ln index_s) in nats, where
 *            index_s = softmax over the live slots of idx_scale * bscore at
 *            the selected block (0 ln 0 = 0).
 * A slot is live when it holds a block in [0, jl].  The target is a plain
 * value: nothing here computes or carries gradients.
 *   bscore   [batch][n_q][h_kv][nblk] fp32 pooled index scores, as written by
 *            msa_index_scores (or at offset 0 of msa_index_topk's workspace);
 *            only entries at live selected blocks are read.
 *   idx_scale finite temperature of the index softmax (MSA_ERR_SHAPE if not
 *            finite; the pages name none).
 *   target   [batch][n_q][h_kv][topk] fp32, kl [batch][n_q][h_kv] fp32, outputs.
 * Workspace: msa_workspace_size(MSA_OP_SPARSE_PREFILL, dims) for one pass; as for
 * msa_sparse_prefill, anything down to one query's workspace runs the call in
 * query chunks with the same outputs. */
msa_status msa_sparse_prefill_target(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const int32_t* blk_idx, const float* bscore, float idx_scale, float scale,
                                     uint16_t* out, float* lse, float* target, float* kl, void* workspace,
                                     size_t workspace_bytes, msa_stream stream);

/* Main branch, backward: gradients of msa_sparse_prefill's output with
 * respect to q, k and v for the given selection (the selection is discrete
 * and carries no gradient; Notion notes "Minimax-sparse-Attention",
 * "Detached Gradients").  With P the softmax weights of a (query, head) over
 * its visible keys and D = sum_d dout * out:
 *   dv[s] = sum P dout,  dS = P (dout . v[s] - D),  dq = scale sum_s dS k[s],
 *   dk[s] = scale sum dS q  (sums over the (query, head) pairs that see s).
 *   q, k, v, blk_idx, scale   as given to msa_sparse_prefill;
 *   out, lse  that call's outputs (lse is required here);
 *   dout      [batch][n_q][h_q][d] bf16, the gradient of the loss w.r.t. out;
 *   dq        [batch][n_q][h_q][d] bf16, output;
 *   dk, dv    [batch][n_kv][h_kv][d] bf16, outputs, fully written (0 for keys
 *             no query saw, and for every key when n_q == 0).
 * Every key gradient is summed in one fixed order inside one workgroup, so the
 * results are deterministic.  block == 128 and h_q * topk * d < 2^31
 * (MSA_ERR_UNSUPPORTED otherwise).  Workspace: msa_workspace_size(
 * MSA_OP_SPARSE_PREFILL, dims); do not share one workspace between this call
 * and a forward call in flight on another stream. */
msa_status msa_sparse_prefill_backward(const msa_dims* dims, const uint16_t* q, const uint16_t* k,
                                       const uint16_t* v, const int32_t* blk_idx, const uint16_t* out,
                                       const float* lse, const uint16_t* dout, float scale, uint16_t* dq,
                                       uint16_t* dk, uint16_t* dv, void* workspace, size_t workspace_bytes,
                                       msa_stream stream);

/* Index branch, backward: gradient of sum_rows dkl[row] * KL(target ||
 * index distribution) with respect to q_idx and k_idx (Notion notes
 * "Minimax-sparse-Attention": "KL Loss Alignment" trains the index branch to
 * imitate the main branch's attention distribution; "Detached Gradients": the
 * target is a constant and no gradient reaches the main branch).  With the
 * selection fixed and, per (b, t, g) row and live slot s,
 *   coef_s = dkl[row] * idx_scale * (softmax_s(idx_scale * bscore[j_s]) - target_s),
 *   dq_idx[row] = sum_s coef_s k_idx[s*],   dk_idx[s*] += coef_s q_idx[row],
 * where s* is the position of the largest causal token score in block j_s
 * (the lowest position among equal maxima): the block max-pool passes its
 * gradient to that token alone.  The argmax is taken on scores recomputed
 * with the index scorer's arithmetic (bf16 products, fp32 sums).
 *   q_idx, k_idx, blk_idx   as for msa_index_topk / msa_sparse_prefill_target;
 *   bscore  [batch][n_q][h_kv][nblk] fp32 pooled index scores (read at the
 *           live selected blocks);
 *   target  [batch][n_q][h_kv][topk] fp32, msa_sparse_prefill_target's output;
 *   dkl     [batch][n_q][h_kv] fp32, the loss gradient w.r.t. each row's KL;
 *   idx_scale  as given to msa_sparse_prefill_target (finite);
 *   dq_idx  [batch][n_q][h_kv][d_idx] fp32, output;
 *   dk_idx  [batch][n_kv][d_idx] fp32, output, fully written (0 for keys that
 *           are no row's argmax).
 * Deterministic (every sum in a fixed order).  h_kv <= 128
 * (MSA_ERR_UNSUPPORTED otherwise).  Workspace:
 * msa_workspace_size(MSA_OP_SPARSE_PREFILL, dims). */
msa_status msa_index_backward(const msa_dims* dims, const uint16_t* q_idx, const uint16_t* k_idx,
                              const int32_t* blk_idx, const float* bscore, const float* target, const float* dkl,
                              float idx_scale, float* dq_idx, float* dk_idx, void* workspace, size_t workspace_bytes,
                              msa_stream stream);

/* Main branch, decode: msa_sparse_prefill with n_q == 1; each of the batch
 * sequences has its own cache of n_kv tokens and its query at p = pos0
 * (normally n_kv - 1).  Streams only the selected blocks (lefilia.fr: a fixed
 * budget of topk * 128 key-value tokens per query whatever the context).
 *   q [batch][1][h_q][d], blk_idx [batch][1][h_kv][topk], out [batch][1][h_q][d]. */
msa_status msa_sparse_decode(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int32_t* blk_idx, float scale, uint16_t* out, float* lse, void* workspace,
                             size_t workspace_bytes, msa_stream stream);

/* Whole-sequence prefill in chunks of `chunk` query tokens: for each sequence
 * and each chunk of its n_q queries (positions pos0 + t0 .. pos0 + t0 + chunk - 1,
 * the last chunk possibly shorter) the index branch (scores, block max-pool,
 * top-k) and the main branch (sparse attention) run on that chunk alone
 * against the sequence's n_kv-token cache, as a serving system extends a
 * context chunk by chunk (lefilia.fr article: 1M-token contexts; yhxrc.cn
 * article, "第一步：索引分支" and "第二步：稀疏分支").  Every query row's
 * result depends only on its own row, so the outputs equal those of
 * msa_index_topk followed by msa_sparse_prefill on the whole call, while the
 * workspace holds one chunk's index workspace (the largest over the chunks)
 * and partials: a 1,048,576-token prefill in chunks of 8,192 queries (64 heads)
 * runs in about 2.2 GiB, where one-shot sparse-prefill partials alone would
 * take 264 GiB.
 *   q_idx, k_idx, q, k, v, blk_idx, out, lse   as for msa_index_topk and
 *            msa_sparse_prefill (blk_idx is an output here, lse may be NULL)
 *   chunk    >= 1 query tokens per chunk (MSA_ERR_SHAPE otherwise)
 *   workspace >= msa_prefill_chunked_workspace_size(dims, chunk); reused by
 *            every chunk, in stream order. */
size_t msa_prefill_chunked_workspace_size(const msa_dims* dims, int32_t chunk);
msa_status msa_prefill_chunked(const msa_dims* dims, int32_t chunk, const uint16_t* q_idx, const uint16_t* k_idx,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v, float scale,
                               int32_t* blk_idx, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                               msa_stream stream);

/* Variable-length decode (a batch of sequences of different lengths in one
 * call): as msa_index_topk / msa_sparse_decode with n_q == 1, except that
 * sequence b holds seq_len[b] tokens of its n_kv-token cache (k_idx, k, v keep
 * the [batch][n_kv]... layout, n_kv being the capacity) and its query sits at
 * p = seq_len[b] - 1; dims->pos0 is not used (it must still satisfy
 * pos0 + 1 <= n_kv).  Blocks, the local block and the -1 padding follow from
 * each sequence's own p; pooled-score rows in the index workspace are valid up
 * to each sequence's local block.
 *   seq_len  [batch] int32 device array, each in [1, n_kv]; the kernels clamp
 *            values outside that range into it (no access leaves the cache),
 *            the results for such a sequence are then those of the clamped
 *            length.
 * Same workspaces as msa_index_topk and msa_sparse_decode.  The index step
 * supports n_q * h_kv <= 16 (MSA_ERR_UNSUPPORTED otherwise). */
msa_status msa_index_topk_varlen(const msa_dims* dims, const int32_t* seq_len, const uint16_t* q_idx,
                                 const uint16_t* k_idx, int32_t* blk_idx, void* workspace, size_t workspace_bytes,
                                 msa_stream stream);
msa_status msa_sparse_decode_varlen(const msa_dims* dims, const int32_t* seq_len, const uint16_t* q,
                                    const uint16_t* k, const uint16_t* v, const int32_t* blk_idx, float scale,
                                    uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                    msa_stream stream);

/* Dense causal GQA, the comparator: as msa_sparse_prefill with every s <= p
 * visible (hamidun.com, "Como o MSA funciona": standard GQA attends every
 * key).  n_q == 1 takes a split-key decode path that needs workspace; n_q > 1
 * needs none (workspace may then be NULL). */
msa_status msa_dense_gqa(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v, float scale,
                         uint16_t* out, float* lse, void* workspace, size_t workspace_bytes, msa_stream stream);


/* Kernel timing (a profiling aid, not part of the computation).  Between
 * msa_profile_begin and msa_profile_end every kernel the library launches is
 * bracketed by two HIP events recorded on the launch's own stream, so each
 * duration is that kernel's execution on the device.  msa_profile_end waits
 * for the recorded events, sums the durations per kernel name, stops
 * recording and releases the events.  msa_profile_begin creates a pool of
 * 4096 HIP events on the host (no device memory; more are created if a run
 * records over 2048 launches) and returns MSA_ERR_HIP if it cannot; recording
 * adds two event records to the stream per launch, so leave it off outside
 * measurements.  Launches from several threads are recorded safely, also while
 * another thread calls msa_profile_begin or msa_profile_end (the event pool is
 * guarded by a mutex); two begin/end calls must not overlap each other.
 *   out       array of `capacity` entries, filled with the kernels in order of
 *             decreasing total time (may be NULL when capacity is 0)
 *   count     out: number of distinct kernels recorded (may exceed capacity)
 * Returns MSA_ERR_NULL for a NULL count, MSA_ERR_HIP if an event call fails
 * (recording is stopped and the events released either way). */
typedef struct {
  char name[64];      /* kernel function name, without template arguments */
  int32_t launches;   /* launches recorded */
  double total_ms;    /* summed device time */
} msa_kernel_time;

msa_status msa_profile_begin(void);
msa_status msa_profile_end(msa_kernel_time* out, int32_t capacity, int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
