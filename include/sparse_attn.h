/*
 * sparse_attn.h — C ABI of the MI355X (gfx950) gated sparse attention hot path.
 *
 * The path, per query token: a lightweight multi-head indexer scores every
 * causal history position, a per-token Top-K keeps K positions, and exact
 * softmax attention over only those K KV rows (shared by all query heads) is
 * scaled by a sigmoid output gate.
 *
 * Pages cited (by title):
 *   [HAT] "Hybrid Attention Architectures: Engineering Trade-offs from Linear
 *          Attention to Gated Sparse Attention"
 *   [EVO] "Evolution of Hybrid Attention in Open-Source LLMs: From Linear to
 *          Gated Sparse Attention"
 *   [F2S] "From Full Attention to Sparsity: The Evolution of Hybrid Attention
 *          Architectures in Large Language Models"
 *   [SAD] "Sparse Attention and Hybrid Attention Architecture Design in Large
 *          Language Models"
 *   [SEL] "Hybrid Attention Architecture Evolution in LLMs: From Full
 *          Attention to Sparse Selection"
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless marked (host).  Tensors are dense
 *     row-major; base pointers are 16-byte aligned.
 *   - Every call is asynchronous on `stream` (a hipStream_t); the library
 *     never allocates, frees or synchronises, so it is reentrant.  The caller
 *     owns every buffer, including workspaces sized by the *_workspace_size
 *     queries.  The one exception to "the caller owns every buffer" is
 *     sparse_gated_attn_fwd_noalloc, whose scratch is a static device array
 *     of the library (see there).
 *   - Argument errors are detected on the host before any launch and return
 *     SA_EINVAL (bad value / NULL / shape) or SA_EUNSUPPORTED (a valid request
 *     the library has no kernel for); nothing is launched then.  A failed
 *     launch returns SA_ELAUNCH.  Device-side data (page ids, index values,
 *     lengths inside q_start / ctx_len) is trusted and not range-checked.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *sa_stream_t; /* a hipStream_t; NULL is the default stream */

typedef enum {
    SA_F32 = 0,
    SA_BF16 = 1,
    SA_FP8_E4M3 = 2 /* OCP e4m3fn: bias 7, max 448, NaN = S.1111.111, no infinity */
} sa_dtype;

typedef enum {
    SA_OK = 0,
    SA_EINVAL = -1,
    SA_EUNSUPPORTED = -2,
    SA_EWORKSPACE = -3,
    SA_ELAUNCH = -4
} sa_status;

/*
 * Ragged batch over a paged cache.  [HAT §5 item 4] asks for varying lengths
 * within a batch; [F2S "Engineering Considerations" item 1] for variable-length
 * Top-K and paged cache management.  Prefill passes an identity page table.
 *
 * Query token j of sequence b (global token q_start[b] + j) sits at position
 *     pos = ctx_len[b] - (q_start[b+1] - q_start[b]) + j,
 * i.e. the new tokens are the last positions of the cache, already appended.
 * Its causal candidates are the n = pos + 1 positions 0..pos (self-inclusive).
 * Logical position s of sequence b lives at physical cache row
 *     page_table[b * max_pages + s / page_size] * page_size + s % page_size.
 * Decode is the case of one new token per sequence.  A sequence may have no
 * new tokens (q_start[b+1] == q_start[b]); it then takes part only through its
 * cached pages.  A batch with T = 0 is valid: every entry point that takes a
 * batch checks it and returns SA_OK without launching anything (workspace
 * sizes are 0), except sparse_block_pool, which pools the cached pages as for
 * any other batch.
 */
typedef struct {
    int32_t num_seqs;          /* (host) B >= 1 */
    int32_t total_q;           /* (host) T = q_start[B] >= 0 */
    int32_t max_q;             /* (host) max_b (q_start[b+1] - q_start[b]); >= 1, or 0 when T = 0 */
    int32_t max_ctx;           /* (host) max_b ctx_len[b]; sizes grids and bounds score rows */
    int32_t page_size;         /* (host) tokens per page: power of two, 16..4096 */
    int32_t max_pages;         /* (host) row stride of page_table, >= ceil(max_ctx / page_size) */
    const int32_t *q_start;    /* [B+1] nondecreasing prefix offsets, q_start[0] = 0 */
    const int32_t *ctx_len;    /* [B] cache length after the new tokens; >= the sequence's new tokens */
    const int32_t *page_table; /* [B, max_pages] physical page ids */
} sa_batch;

/*
 * a1 — indexer scores.  [HAT §3.1, §3.3]: a lightweight relevance score of
 * each query against every history position, before selection.
 * [F2S "Fine-Grained Sparse Attention: Indexer Plus Top-K"]: few heads, low
 * dims, content only (no positional encoding), scores of shape [n, n].
 * The form is the DSA-style reading (the pages print no formula):
 *     scores[i, s] = sum_h w[i,h] * max(0, q_idx[i,h,:] . k_idx[s,:])
 * for s in [0, n_i); one k_idx row per position is shared by all heads.
 * fp8: the dot of the decoded e4m3fn codes is multiplied by
 * q_scale[i] * k_scale[s]; both scales must be >= 0.
 *
 *   q_idx      [T, n_heads, head_dim] in dtype
 *   q_scale    [T] fp32 (fp8 only, else NULL)
 *   weights    [T, n_heads] fp32
 *   k_idx_cache   [num_pages, page_size, head_dim] in dtype
 *   k_scale_cache [num_pages, page_size] fp32 (fp8 only, else NULL)
 *   scores     [T, ld_scores] fp32; row i gets entries [0, n_i) and nothing
 *              else is written.  ld_scores >= max_ctx and a multiple of 4.
 * Supported (dtype, n_heads, head_dim): f32 with head_dim 32; bf16 with
 * head_dim 64 or 128; fp8 with head_dim 128; n_heads in {4, 8, 16, 32, 64}.
 * Any other shape returns SA_EUNSUPPORTED.  Weights may be of any finite
 * magnitude: where the fp8 epilogue multiplies in fp16, each token's weights
 * are scaled by a power of two that keeps them in fp16's normal range and the
 * factor is given back in fp32.  Scores are finite for finite inputs whose
 * exact scores are within fp32 range.
 */
sa_status sparse_indexer_scores(const sa_batch *batch, sa_dtype dtype,
                                const void *q_idx, int32_t n_heads, int32_t head_dim,
                                const float *q_scale, const float *weights,
                                const void *k_idx_cache, const float *k_scale_cache,
                                float *scores, int64_t ld_scores, sa_stream_t stream);

/*
 * a2 — per-token Top-K.  [HAT §3.1]: keep the K highest-scoring positions;
 * [F2S "Fine-Grained Sparse Attention: Indexer Plus Top-K"]: indices of
 * shape [n, K]; [HAT §5 item 4]: fewer candidates than K are padded.
 * [EVO] §5 item 3 warns against approximate Top-K: this one is exact.
 *
 * Row i (token i) selects from scores[i, 0..n_i): if n_i <= k all n_i
 * positions, else the k positions with the largest scores, ties broken
 * toward the lower position (+0 and -0 compare equal).  indices[i, :] holds
 * the min(k, n_i) selected positions in ascending order, then -1.
 * Scores must be finite.  1 <= k <= 4096.
 *   workspace: >= sparse_topk_workspace_size(batch, k) bytes (may be 0 bytes;
 *   then workspace may be NULL), 16-byte aligned.  Results are deterministic.
 */
size_t sparse_topk_workspace_size(const sa_batch *batch, int32_t k);
sa_status sparse_topk(const sa_batch *batch, const float *scores, int64_t ld_scores,
                      int32_t k, int32_t *indices, void *workspace, size_t workspace_bytes,
                      sa_stream_t stream);

/*
 * a3-a5 — gather, exact sparse attention, sigmoid output gate.
 * [HAT §3.3]: exact attention over kv_history[idx], then the gate scales it.
 * [F2S "Fine-Grained Sparse Attention: Indexer Plus Top-K", pseudocode]:
 * attention(q, gather(k, idx), gather(v, idx)) and g = sigmoid(...).
 * [SEL §3.2]: standard attention over the selected set.
 * [SAD §4 "Output gating"]: per-channel or per-head scaling of the output.
 * [SAD §2]: query heads share one KV head; a latent row may serve as K and V.
 *
 * For token i, head h, over the valid entries s_j of indices[i, :] (values
 * < 0 are padding and are skipped):
 *     z_j = softmax_scale * q[i,h,:] . K[s_j, 0:d_qk]
 *     o   = sum_j softmax(z)_j * V[s_j, 0:d_v]
 *     out[i,h,c] = o[c] * sigmoid(G),  G = gate_logits[i,h,c] (per channel)
 *                                      or gate_logits[i,h]   (per head)
 *     lse[i,h]   = max_j z_j + log(sum_j exp(z_j - max_j z_j))
 * A row with no valid entry gives out = 0 and lse = -inf.
 *
 *   q            [T, n_q_heads, d_qk] in dtype (SA_F32 or SA_BF16)
 *   k_cache      [num_pages, page_size, kv_row_stride]: K row = first d_qk elements
 *   v_cache      [num_pages, page_size, kv_row_stride]: V row = first d_v elements;
 *                may equal k_cache (latent layout, d_v <= d_qk)
 *   indices      [T, k] int32 positions (as produced by sparse_topk); padding
 *                (< 0) may sit anywhere in a row.  Valid entries must lie in
 *                [0, ctx_len[b]) of the token's sequence: they are not checked,
 *                and one past the sequence's pages reads outside its page table.
 *   gate_logits  [T, n_q_heads, d_v] if gate_per_channel else [T, n_q_heads], in dtype
 *   out          [T, n_q_heads, d_v] in dtype (bf16 rounded to nearest even)
 *   lse          [T, n_q_heads] fp32, or NULL
 * Supported: SA_F32 with d_qk = d_v in {32, 64, 128}; SA_BF16 with
 * (d_qk, d_v) = (128, 128), separate or shared caches, or (576, 512) with
 * v_cache == k_cache (latent layout); n_q_heads a multiple of 16 (bf16) or
 * any (f32); 1 <= k <= 65536.
 */
size_t sparse_gated_attn_workspace_size(const sa_batch *batch, int32_t n_q_heads, int32_t d_v, int32_t k);
sa_status sparse_gated_attn_fwd(const sa_batch *batch, sa_dtype dtype,
                                const void *q, int32_t n_q_heads, int32_t d_qk,
                                const void *k_cache, const void *v_cache, int32_t d_v,
                                int64_t kv_row_stride,
                                const int32_t *indices, int32_t k,
                                const void *gate_logits, int32_t gate_per_channel,
                                float softmax_scale, void *out, float *lse,
                                void *workspace, size_t workspace_bytes, sa_stream_t stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sparse_gated_attn_fwd with
 * the same arguments, results and errors, minus the workspace.  Where the
 * index list is split over workgroups (decode, few tokens), the partial
 * results go to a static device array of SA_NOALLOC_SCRATCH_BYTES per GPU,
 * which the library holds from its first use on that GPU until the process
 * ends.  The call allocates nothing: no hipMalloc, no hipFree, no allocating
 * library routine.  The stream must belong to the current device.
 *   - A batch whose partials need more than SA_NOALLOC_SCRATCH_BYTES (the
 *     bytes sparse_gated_attn_workspace_size reports) returns SA_EWORKSPACE
 *     before anything is launched; sparse_gated_attn_fwd with a caller
 *     workspace serves it.
 *   - Every call on one GPU shares that GPU's array, and the array keeps the
 *     last call's contents (the kernels write every partial before reading
 *     it, so nothing needs clearing).  Calls that overlap in time on one GPU
 *     (two streams, or two host threads) race on the array and must be
 *     serialised by the caller.
 */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
sa_status sparse_gated_attn_fwd_noalloc(const sa_batch *batch, sa_dtype dtype,
                                        const void *q, int32_t n_q_heads, int32_t d_qk,
                                        const void *k_cache, const void *v_cache, int32_t d_v,
                                        int64_t kv_row_stride,
                                        const int32_t *indices, int32_t k,
                                        const void *gate_logits, int32_t gate_per_channel,
                                        float softmax_scale, void *out, float *lse,
                                        sa_stream_t stream);

/*
 * Block-level selection, the pages' second variant.  [SEL §3.2] pseudocode:
 * pool the keys by block, score the blocks with the queries, keep the top-k
 * blocks, gather them, exact attention within them; [SAD §3]: block sparsity
 * with top-k routing, query-to-block relevance at block granularity; [SEL
 * §4.1-4.2]: the effective length becomes k*b, and block sparsity is the form
 * that most easily turns into real speed-ups.
 *
 * Readings (the pages fix none): a block is one page of the paged cache
 * (b = page_size); its pooled key is the mean of its K rows; the query heads
 * share one selection (they share a KV head, [SAD §2]), so the score of block
 * j for token i is  S[i, j] = (sum_h q[i,h,:]) . kbar_j  over the candidate
 * blocks j <= pos(i) / page_size.  The flow, all on `stream`:
 *   sparse_block_pool   -> kbar        [num_pages, d_qk] fp32, row = physical page
 *   sparse_block_scores -> S           [T, ld] fp32, row i: entries [0, pos_i / page_size + 1)
 *   sparse_block_topk   -> block ids   [T, kb] (a2's rule on block rows: ascending, then -1)
 *   sparse_block_expand -> positions   [T, kb * page_size] (the causal positions of the
 *                                       selected blocks, ascending, then -1)
 *   sparse_gated_attn_fwd over those positions with k = kb * page_size.
 *
 * sparse_block_pool: for every sequence b and block j < ceil(ctx_len[b] /
 *   page_size), kbar[page_table[b, j], :] = mean of the block's rows s <
 *   ctx_len[b] of k_cache (first d_qk elements, dtype SA_F32 or SA_BF16),
 *   summed in fp32.  Pages no sequence uses are not written.
 *   Rows of whole 16-byte units, at most 4 KB (d_qk <= 2048 bf16, 1024 f32).
 * sparse_block_scores: needs a workspace of sparse_block_scores_workspace_size
 *   bytes (T * d_qk fp32); d_qk a multiple of 32, rows of at most 4 KB;
 *   ld_scores >= the most blocks of any sequence.  Products accumulate in fp32
 *   (MFMA).
 * sparse_block_topk: 1 <= kb <= 4096; workspace as sparse_topk's.
 * sparse_block_expand: kb * page_size <= 65536.
 */
sa_status sparse_block_pool(const sa_batch *batch, sa_dtype dtype, const void *k_cache, int32_t d_qk,
                            int64_t kv_row_stride, float *k_blocks, sa_stream_t stream);
size_t sparse_block_scores_workspace_size(const sa_batch *batch, int32_t d_qk);
sa_status sparse_block_scores(const sa_batch *batch, sa_dtype dtype, const void *q, int32_t n_q_heads,
                              int32_t d_qk, const float *k_blocks, float *scores, int64_t ld_scores,
                              void *workspace, size_t workspace_bytes, sa_stream_t stream);
size_t sparse_block_topk_workspace_size(const sa_batch *batch, int32_t kb);
sa_status sparse_block_topk(const sa_batch *batch, const float *scores, int64_t ld_scores, int32_t kb,
                            int32_t *block_idx, void *workspace, size_t workspace_bytes, sa_stream_t stream);
sa_status sparse_block_expand(const sa_batch *batch, const int32_t *block_idx, int32_t kb, int32_t *indices,
                              sa_stream_t stream);

/*
 * Backward over fixed indices (training).  [HAT §3.3]: exact attention over
 * kv_history[idx], scaled by the gate; [HAT §3.2]: the gate is a continuous
 * path for the gradient; [F2S "Fine-Grained Sparse Attention: Indexer Plus
 * Top-K"]: the indices come from a Top-K, which passes no gradient, so only
 * the attention and the gate are differentiated.  For the forward of
 * sparse_gated_attn_fwd (its output `out` and log-sum-exp `lse` are inputs
 * here) and an upstream gradient d_out:
 *     d_gate = d_out * out * (1 - g)               (per channel; summed over c per head)
 *     do = d_out * g,  D = d_out . out,  dP_j = do . V_j,  dS_j = P_j (dP_j - D),
 *     P_j = exp(softmax_scale * q . K_j - lse)
 *     d_q = softmax_scale * sum_j dS_j K_j                      (written)
 *     d_k_cache[row(s_j)] += softmax_scale * dS_j q             (added)
 *     d_v_cache[row(s_j)] += P_j do                             (added)
 * summed over every (token, head, slot) that selected the row; a position
 * repeated in one row counts once per slot, as in the forward.  The caller
 * zeroes d_k_cache and d_v_cache ([num_pages, page_size, kv_row_stride]
 * fp32; the same array when v_cache == k_cache).  d_q is [T, n_q_heads,
 * d_qk] fp32, d_gate fp32 shaped like the gate.  P, dS and do enter the
 * MFMAs rounded to bf16; sums are fp32.  The rows are merged with float
 * atomics (once per 256-token chunk and key for d_qk = d_v in {64, 128} with
 * 16, 32 or 64 heads; once per slot otherwise), so the last bits of d_k/d_v
 * vary between runs.  Valid positions are < ctx_len of the token's sequence.
 * Supported: SA_BF16; d_qk = d_v in {64, 128}, separate or shared caches, or
 * (576, 512) with v_cache == k_cache (latent layout); n_q_heads a multiple of
 * 16 up to 256; 1 <= k <= 65536.
 * sparse_gated_attn_bwd_workspace_size: bytes of device workspace (do, Q^T
 * and do^T copies, D, and for the first group of shapes a position bitmap, a
 * byte per slot and a byte per token); 0 for an empty batch.  The workspace is 256-byte aligned
 * (SA_EINVAL otherwise); fewer bytes than reported: SA_EWORKSPACE.
 */
size_t sparse_gated_attn_bwd_workspace_size(const sa_batch *batch, int32_t n_q_heads, int32_t d_qk, int32_t d_v,
                                            int32_t k);
sa_status sparse_gated_attn_bwd(const sa_batch *batch, sa_dtype dtype, const void *q, int32_t n_q_heads,
                                int32_t d_qk, const void *k_cache, const void *v_cache, int32_t d_v,
                                int64_t kv_row_stride, const int32_t *indices, int32_t k, const void *gate_logits,
                                int32_t gate_per_channel, float softmax_scale, const void *out, const float *lse,
                                const void *d_out, float *d_q, float *d_k_cache, float *d_v_cache, float *d_gate,
                                void *workspace, size_t workspace_bytes, sa_stream_t stream);

/*
 * Branch fusion with a sliding-window local branch.  [SAD §3] pseudocode: a
 * sparse branch, a sliding-window branch so that nearby context is never
 * lost, and y = g * sparse_out + (1 - g) * local_out with g = sigmoid(...);
 * [SAD §4] "branch fusion gating".  Readings: the local branch is exact causal
 * attention over positions max(0, pos(i) - window + 1) .. pos(i) with the
 * same q, K, V and softmax scale; G is per head or per channel.
 * The flow, all on `stream`:
 *   o_sparse = sparse_gated_attn_fwd over the Top-K indices, and
 *   o_local  = sparse_gated_attn_fwd over sparse_window_indices(window),
 *              both with a per-head gate of +inf (sigmoid(+inf) = 1: ungated);
 *   out      = sparse_branch_fuse(o_sparse, o_local, G).
 *
 * sparse_window_indices: indices [T, window] = the window's positions,
 *   ascending, then -1 (rows shorter than the window).  1 <= window <= 65536.
 * sparse_branch_fuse: out = g * o_sparse + (1 - g) * o_local, g = sigmoid(G),
 *   elementwise over rows x d_v (rows = T * n_q_heads), in fp32, rounded to
 *   dtype (bf16 to nearest even).  gate_logits is [rows, d_v] when
 *   gate_per_channel, else [rows]; d_v a multiple of 8; 16-byte aligned.
 *   rows = 0 returns SA_OK and launches nothing.
 */
sa_status sparse_window_indices(const sa_batch *batch, int32_t window, int32_t *indices, sa_stream_t stream);
sa_status sparse_branch_fuse(sa_dtype dtype, int64_t rows, int32_t d_v, const void *o_sparse, const void *o_local,
                             const void *gate_logits, int32_t gate_per_channel, void *out, sa_stream_t stream);

/*
 * Branch fusion with the mix inside the attention epilogue ([SAD §3]
 * pseudocode, y = g * sparse + (1 - g) * local; [SAD §4] branch fusion
 * gating).  Attention of q over the index list (the local branch, e.g.
 * positions from sparse_window_indices), then, where the output is formed,
 *     out[i,h,c] = g * other[i,h,c] + (1 - g) * o[c],  g = sigmoid(G)
 * with o the normalised attention in fp32 (it is not rounded before the mix)
 * and G per channel or per head as in sparse_gated_attn_fwd.  `other` is the
 * other branch's output [T, n_q_heads, d_v] in dtype, typically
 * sparse_gated_attn_fwd of the sparse branch with a per-head gate of +inf
 * (sigmoid 1: ungated); 16-byte aligned, and it must not overlap `out`
 * (other NULL, unaligned or equal to out: SA_EINVAL).  This replaces the
 * local branch's own output and sparse_branch_fuse: one pass fewer over three
 * [T, H, d_v] tensors, and the local branch is not rounded before the mix.
 * Shapes, workspace (sparse_gated_attn_workspace_size), lse (of the local
 * branch) and the other errors as sparse_gated_attn_fwd.
 */
sa_status sparse_attn_fuse_fwd(const sa_batch *batch, sa_dtype dtype,
                               const void *q, int32_t n_q_heads, int32_t d_qk,
                               const void *k_cache, const void *v_cache, int32_t d_v,
                               int64_t kv_row_stride,
                               const int32_t *indices, int32_t k,
                               const void *gate_logits, int32_t gate_per_channel,
                               float softmax_scale, const void *other, void *out, float *lse,
                               void *workspace, size_t workspace_bytes, sa_stream_t stream);

/*
 * Cache append (the step before the path): writes the new tokens' rows into
 * the paged caches.  [HAT §5 item 2]: the cache organisation decides indexing
 * efficiency; [F2S "Engineering Considerations" item 1]: paged cache
 * management is on the critical path; [HAT §5 item 3]: low-precision ranges
 * need care in the indexer.
 *
 * Query token i (position pos(i) of its sequence, the sa_batch rule, i.e. the
 * cache already counts it in ctx_len) goes to physical row
 *     r = page_table[b * max_pages + pos / page_size] * page_size + pos % page_size:
 *     k_cache[r, 0:d_qk] = k_new[i, :]
 *     v_cache[r, 0:d_v]  = v_new[i, :]      (v_new NULL: latent layout, V is the
 *                                            first d_v elements of the K row)
 *     k_idx_cache[r, :]  = k_idx_new[i, :]  (idx_dtype == src_dtype: copied), or
 *     fp8 (idx_dtype SA_FP8_E4M3): k_scale_cache[r] = s = max_d |k_idx_new[i, d]| / 448
 *         and k_idx_cache[r, d] = e4m3fn(k_idx_new[i, d] / s), nearest even,
 *         saturating at +-448, both operations in fp32; a zero row gives s = 0
 *         and codes 0.  This is the format sparse_indexer_scores reads.
 * Other rows are not touched.  Positions of one call must be distinct rows.
 *
 *   k_new, v_new   [T, d_qk], [T, d_v] in kv_dtype (SA_F32 or SA_BF16)
 *   k_cache, v_cache  as in sparse_gated_attn_fwd (kv_row_stride elements per row)
 *   k_idx_new      [T, d_i] in src_dtype (SA_F32 or SA_BF16); finite values
 *   k_idx_cache    [num_pages, page_size, d_i] in idx_dtype
 *   k_scale_cache  [num_pages, page_size] fp32 (fp8 only, else ignored)
 * Requires d_qk, d_v and kv_row_stride rows of whole 16-byte units (K and V
 * rows of at most 4 KB), d_i even and <= 1024, 16-byte aligned base pointers.
 */
sa_status sparse_cache_append(const sa_batch *batch, sa_dtype kv_dtype, const void *k_new, int32_t d_qk,
                              const void *v_new, int32_t d_v, void *k_cache, void *v_cache, int64_t kv_row_stride,
                              sa_dtype src_dtype, const void *k_idx_new, int32_t d_i, sa_dtype idx_dtype,
                              void *k_idx_cache, float *k_scale_cache, sa_stream_t stream);

/*
 * fp8 quantisation of the rows of x [rows, cols] (src_dtype SA_F32 or
 * SA_BF16, finite values), by the rule of sparse_cache_append: scales[r] =
 * max|x[r, :]| / 448, codes[r, c] = e4m3fn(x[r, c] / scales[r]).  For the
 * indexer queries, rows = T and cols = n_heads * head_dim give q_idx and
 * q_scale.  cols a multiple of 8; x 16-byte and codes 8-byte aligned.
 * rows = 0 returns SA_OK and launches nothing.
 */
sa_status sparse_quantize_fp8_rows(sa_dtype src_dtype, const void *x, int64_t rows, int32_t cols,
                                   uint8_t *codes, float *scales, sa_stream_t stream);

/* Static description of a status code; never NULL. */
const char *sa_status_string(sa_status s);

/* ABI version of this header (incremented on incompatible changes). */
int32_t sa_abi_version(void);

#define SA_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
