// extern "C" entry points of libsparse_attn.so: argument validation on the
// host, then kernel launches on the caller's stream.  No allocation and no
// synchronisation; the only global state is the per-device address of the
// static scratch array of the no-allocation attention entry point.  The
// operations and their citations are documented in sparse_attn.h.
#include "sparse_attn.h"

#include <mutex>

#include "launch.h"
#include "sa_device.h"

// Scratch of sparse_gated_attn_fwd_noalloc: split-attention partials for
// callers that cannot allocate.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code this name is only a stand-in for
// the symbol: kernels get the device address from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void *p) { return (((uintptr_t)p) & 15u) == 0; }

int log2_exact(int x)
{
    if (x <= 0 || (x & (x - 1)))
        return -1;
    int s = 0;
    while ((1 << s) < x)
        ++s;
    return s;
}

// A valid batch with no query tokens (T = 0): the entry points return SA_OK
// without launching anything.  Never returned to a caller.
constexpr sa_status kEmptyBatch = (sa_status)1;

sa_status make_batch(const sa_batch *in, sa::Batch *out)
{
    if (!in || in->num_seqs < 1 || in->total_q < 0 || in->max_ctx < 1 || in->max_pages < 1)
        return SA_EINVAL;
    if (in->total_q > 0 ? in->max_q < 1 : in->max_q != 0)
        return SA_EINVAL;
    if (!in->q_start || !in->ctx_len || !in->page_table)
        return SA_EINVAL;
    const int shift = log2_exact(in->page_size);
    if (shift < 4 || shift > 12)
        return SA_EINVAL;
    if ((int64_t)in->max_pages * in->page_size < in->max_ctx)
        return SA_EINVAL;
    if (in->max_q > in->total_q)
        return SA_EINVAL;
    out->num_seqs = in->num_seqs;
    out->total_q = in->total_q;
    out->max_q = in->max_q;
    out->max_ctx = in->max_ctx;
    out->page_shift = shift;
    out->max_pages = in->max_pages;
    out->q_start = in->q_start;
    out->ctx_len = in->ctx_len;
    out->page_table = in->page_table;
    return in->total_q == 0 ? kEmptyBatch : SA_OK;
}

sa_status launched(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ELAUNCH; }

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

sa_status scratch_of_current_device(hipStream_t stream, void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return SA_ELAUNCH;
    if (stream) {
        int sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess)
            return SA_EINVAL;
        if (sdev != dev)                 // the stream must belong to the current device
            return SA_EINVAL;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return SA_ELAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SA_OK;
}

} // namespace

extern "C" {

sa_status sparse_indexer_scores(const sa_batch *batch, sa_dtype dtype, const void *q_idx, int32_t n_heads,
                                int32_t head_dim, const float *q_scale, const float *weights,
                                const void *k_idx_cache, const float *k_scale_cache, float *scores,
                                int64_t ld_scores, sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (dtype != SA_F32 && dtype != SA_BF16 && dtype != SA_FP8_E4M3)
        return SA_EINVAL;
    if (!q_idx || !weights || !k_idx_cache || !scores || n_heads < 1 || head_dim < 1)
        return SA_EINVAL;
    if (dtype == SA_FP8_E4M3 && (!q_scale || !k_scale_cache))
        return SA_EINVAL;
    if (ld_scores < bt.max_ctx || (ld_scores & 3))
        return SA_EINVAL;
    if (!aligned16(q_idx) || !aligned16(k_idx_cache) || !aligned16(scores))
        return SA_EINVAL;
    if (!sa::indexer_supported((int)dtype, n_heads, head_dim))
        return SA_EUNSUPPORTED;
    return launched(sa::launch_indexer((int)dtype, n_heads, head_dim, bt, q_idx, q_scale, weights, k_idx_cache,
                                       k_scale_cache, scores, ld_scores, (hipStream_t)stream));
}

size_t sparse_topk_workspace_size(const sa_batch *batch, int32_t k)
{
    sa::Batch bt;
    if (make_batch(batch, &bt) != SA_OK || k < 1)
        return 0;
    return sa::topk_plan(bt.total_q, bt.max_ctx, k).ws_bytes;
}

sa_status sparse_topk(const sa_batch *batch, const float *scores, int64_t ld_scores, int32_t k, int32_t *indices,
                      void *workspace, size_t workspace_bytes, sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (!scores || !indices || k < 1)
        return SA_EINVAL;
    if (k > 4096)
        return SA_EUNSUPPORTED;
    if (ld_scores < bt.max_ctx || (ld_scores & 3) || !aligned16(scores))
        return SA_EINVAL;
    const sa::TopkPlan plan = sa::topk_plan(bt.total_q, bt.max_ctx, k);
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
        return SA_EWORKSPACE;
    if (plan.chunked && bt.total_q > 65535)
        return SA_EUNSUPPORTED;
    return launched(sa::launch_topk(bt, plan, scores, ld_scores, k, indices, workspace, (hipStream_t)stream));
}

size_t sparse_gated_attn_workspace_size(const sa_batch *batch, int32_t n_q_heads, int32_t d_v, int32_t k)
{
    sa::Batch bt;
    if (make_batch(batch, &bt) != SA_OK || n_q_heads < 1 || d_v < 1 || k < 1)
        return 0;
    return sa::attn_plan(bt.total_q, n_q_heads, d_v, k).ws_bytes;
}

static sa_status attn_fwd_checked(const sa_batch *batch, sa_dtype dtype, const void *q, int32_t n_q_heads,
                                  int32_t d_qk, const void *k_cache, const void *v_cache, int32_t d_v,
                                  int64_t kv_row_stride, const int32_t *indices, int32_t k, const void *gate_logits,
                                  int32_t gate_per_channel, float softmax_scale, void *out, float *lse,
                                  void *workspace, size_t workspace_bytes, bool static_scratch, sa_stream_t stream,
                                  const void *mix = nullptr)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (dtype != SA_F32 && dtype != SA_BF16)
        return SA_EINVAL;
    if (!q || !k_cache || !v_cache || !indices || !gate_logits || !out)
        return SA_EINVAL;
    if (n_q_heads < 1 || d_qk < 1 || d_v < 1 || k < 1 || k > 65536)
        return SA_EINVAL;
    if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
        return SA_EINVAL;
    if (kv_row_stride < d_qk || kv_row_stride < d_v)
        return SA_EINVAL;
    const int esz = dtype == SA_BF16 ? 2 : 4;
    if ((kv_row_stride * esz) % 16 || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(out) || !aligned16(gate_logits))
        return SA_EINVAL;
    if (k_cache == v_cache && d_v > d_qk)
        return SA_EINVAL;
    if (mix && (!aligned16(mix) || mix == out))
        return SA_EINVAL;
    if (!sa::attn_supported((int)dtype, n_q_heads, d_qk, d_v) ||
        !sa::attn_supported_layout((int)dtype, d_qk, d_v, k_cache == v_cache))
        return SA_EUNSUPPORTED;
    const sa::AttnPlan plan = sa::attn_plan(bt.total_q, n_q_heads, d_v, k);
    if (static_scratch) {
        if (plan.ws_bytes > SA_NOALLOC_SCRATCH_BYTES)
            return SA_EWORKSPACE;
        if (plan.ws_bytes > 0) {
            st = scratch_of_current_device((hipStream_t)stream, &workspace);
            if (st != SA_OK)
                return st;
        }
    } else if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes || !aligned16(workspace))) {
        return SA_EWORKSPACE;
    }
    return launched(sa::launch_attn((int)dtype, bt, plan, q, n_q_heads, d_qk, k_cache, v_cache, d_v, kv_row_stride,
                                    indices, k, gate_logits, gate_per_channel ? 1 : 0, softmax_scale, out, lse,
                                    workspace, (hipStream_t)stream, mix));
}

sa_status sparse_gated_attn_fwd(const sa_batch *batch, sa_dtype dtype, const void *q, int32_t n_q_heads,
                                int32_t d_qk, const void *k_cache, const void *v_cache, int32_t d_v,
                                int64_t kv_row_stride, const int32_t *indices, int32_t k, const void *gate_logits,
                                int32_t gate_per_channel, float softmax_scale, void *out, float *lse,
                                void *workspace, size_t workspace_bytes, sa_stream_t stream)
{
    return attn_fwd_checked(batch, dtype, q, n_q_heads, d_qk, k_cache, v_cache, d_v, kv_row_stride, indices, k,
                            gate_logits, gate_per_channel, softmax_scale, out, lse, workspace, workspace_bytes,
                            false, stream);
}

sa_status sparse_attn_fuse_fwd(const sa_batch *batch, sa_dtype dtype, const void *q, int32_t n_q_heads, int32_t d_qk,
                               const void *k_cache, const void *v_cache, int32_t d_v, int64_t kv_row_stride,
                               const int32_t *indices, int32_t k, const void *gate_logits, int32_t gate_per_channel,
                               float softmax_scale, const void *other, void *out, float *lse, void *workspace,
                               size_t workspace_bytes, sa_stream_t stream)
{
    if (!other)
        return SA_EINVAL;
    return attn_fwd_checked(batch, dtype, q, n_q_heads, d_qk, k_cache, v_cache, d_v, kv_row_stride, indices, k,
                            gate_logits, gate_per_channel, softmax_scale, out, lse, workspace, workspace_bytes,
                            false, stream, other);
}

sa_status sparse_gated_attn_fwd_noalloc(const sa_batch *batch, sa_dtype dtype, const void *q, int32_t n_q_heads,
                                        int32_t d_qk, const void *k_cache, const void *v_cache, int32_t d_v,
                                        int64_t kv_row_stride, const int32_t *indices, int32_t k,
                                        const void *gate_logits, int32_t gate_per_channel, float softmax_scale,
                                        void *out, float *lse, sa_stream_t stream)
{
    return attn_fwd_checked(batch, dtype, q, n_q_heads, d_qk, k_cache, v_cache, d_v, kv_row_stride, indices, k,
                            gate_logits, gate_per_channel, softmax_scale, out, lse, nullptr, 0, true, stream);
}

sa_status sparse_block_pool(const sa_batch *batch, sa_dtype dtype, const void *k_cache, int32_t d_qk,
                            int64_t kv_row_stride, float *k_blocks, sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK && st != kEmptyBatch)      // pooling depends on the cached pages only
        return st;
    if (dtype != SA_F32 && dtype != SA_BF16)
        return SA_EINVAL;
    const int esz = dtype == SA_BF16 ? 2 : 4;
    if (!k_cache || !k_blocks || d_qk < 1 || kv_row_stride < d_qk || (d_qk * esz) % 16 ||
        (kv_row_stride * esz) % 16)
        return SA_EINVAL;
    if (!aligned16(k_cache) || !aligned16(k_blocks))
        return SA_EINVAL;
    if (d_qk * esz > 4096)
        return SA_EUNSUPPORTED;
    return launched(sa::launch_block_pool(bt, (int)dtype, k_cache, d_qk, kv_row_stride, k_blocks,
                                          (hipStream_t)stream));
}

size_t sparse_block_scores_workspace_size(const sa_batch *batch, int32_t d_qk)
{
    sa::Batch bt;
    if (make_batch(batch, &bt) != SA_OK || d_qk < 1)
        return 0;
    return (size_t)bt.total_q * (size_t)d_qk * 4u;
}

sa_status sparse_block_scores(const sa_batch *batch, sa_dtype dtype, const void *q, int32_t n_q_heads,
                              int32_t d_qk, const float *k_blocks, float *scores, int64_t ld_scores,
                              void *workspace, size_t workspace_bytes, sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (dtype != SA_F32 && dtype != SA_BF16)
        return SA_EINVAL;
    if (!q || !k_blocks || !scores || n_q_heads < 1 || d_qk < 32 || (d_qk % 32))
        return SA_EINVAL;
    if (d_qk * (dtype == SA_BF16 ? 2 : 4) > 4096)
        return SA_EUNSUPPORTED;
    const int64_t max_blocks = (bt.max_ctx + (1 << bt.page_shift) - 1) >> bt.page_shift;
    if (ld_scores < max_blocks)
        return SA_EINVAL;
    if (!aligned16(q) || !aligned16(k_blocks) || !aligned16(scores))
        return SA_EINVAL;
    const size_t need = (size_t)bt.total_q * (size_t)d_qk * 4u;
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return SA_EWORKSPACE;
    return launched(sa::launch_block_scores(bt, (int)dtype, q, n_q_heads, d_qk, k_blocks, scores, ld_scores,
                                            (float *)workspace, (hipStream_t)stream));
}

// A batch whose rows are block rows: lengths (pos >> page_shift) + 1, the
// longest ceil(max_ctx / page_size).
static sa::TopkPlan block_topk_plan(const sa::Batch &bt, int32_t kb)
{
    const int max_blocks = (bt.max_ctx + (1 << bt.page_shift) - 1) >> bt.page_shift;
    return sa::topk_plan(bt.total_q, max_blocks, kb);
}

size_t sparse_block_topk_workspace_size(const sa_batch *batch, int32_t kb)
{
    sa::Batch bt;
    if (make_batch(batch, &bt) != SA_OK || kb < 1)
        return 0;
    return block_topk_plan(bt, kb).ws_bytes;
}

sa_status sparse_block_topk(const sa_batch *batch, const float *scores, int64_t ld_scores, int32_t kb,
                            int32_t *block_idx, void *workspace, size_t workspace_bytes, sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (!scores || !block_idx || kb < 1)
        return SA_EINVAL;
    if (kb > 4096)
        return SA_EUNSUPPORTED;
    const int64_t max_blocks = (bt.max_ctx + (1 << bt.page_shift) - 1) >> bt.page_shift;
    if (ld_scores < max_blocks || (ld_scores & 3) || !aligned16(scores))
        return SA_EINVAL;
    const sa::TopkPlan plan = block_topk_plan(bt, kb);
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
        return SA_EWORKSPACE;
    if (plan.chunked && bt.total_q > 65535)
        return SA_EUNSUPPORTED;
    return launched(sa::launch_topk(bt, plan, scores, ld_scores, kb, block_idx, workspace, (hipStream_t)stream,
                                    bt.page_shift));
}

sa_status sparse_block_expand(const sa_batch *batch, const int32_t *block_idx, int32_t kb, int32_t *indices,
                              sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (!block_idx || !indices || kb < 1 || ((int64_t)kb << bt.page_shift) > 65536)
        return SA_EINVAL;
    return launched(sa::launch_block_expand(bt, block_idx, kb, indices, (hipStream_t)stream));
}

size_t sparse_gated_attn_bwd_workspace_size(const sa_batch *batch, int32_t n_q_heads, int32_t d_qk, int32_t d_v,
                                            int32_t k)
{
    sa::Batch bt;
    if (make_batch(batch, &bt) != SA_OK || n_q_heads < 1 || d_qk < 1 || d_v < 1 || k < 1)
        return 0;
    return sa::attn_bwd_ws_bytes(bt.total_q, bt.max_ctx, n_q_heads, d_qk, d_v, k);
}

sa_status sparse_gated_attn_bwd(const sa_batch *batch, sa_dtype dtype, const void *q, int32_t n_q_heads,
                                int32_t d_qk, const void *k_cache, const void *v_cache, int32_t d_v,
                                int64_t kv_row_stride, const int32_t *indices, int32_t k, const void *gate_logits,
                                int32_t gate_per_channel, float softmax_scale, const void *out, const float *lse,
                                const void *d_out, float *d_q, float *d_k_cache, float *d_v_cache, float *d_gate,
                                void *workspace, size_t workspace_bytes, sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (dtype != SA_F32 && dtype != SA_BF16)
        return SA_EINVAL;
    if (!q || !k_cache || !v_cache || !indices || !gate_logits || !out || !lse || !d_out || !d_q || !d_k_cache ||
        !d_v_cache || !d_gate)
        return SA_EINVAL;
    if (n_q_heads < 1 || d_qk < 1 || d_v < 1 || k < 1 || k > 65536 || kv_row_stride < d_qk || kv_row_stride < d_v)
        return SA_EINVAL;
    if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
        return SA_EINVAL;
    if ((kv_row_stride * 2) % 16 || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(d_out) ||
        !aligned16(out) || !aligned16(d_q))
        return SA_EINVAL;
    if ((k_cache == v_cache) != (d_k_cache == d_v_cache))
        return SA_EINVAL;
    if (!sa::attn_bwd_supported((int)dtype, n_q_heads, d_qk, d_v))
        return SA_EUNSUPPORTED;
    if (sa::attn_bwd_needs_shared(d_qk, d_v) && k_cache != v_cache)
        return SA_EUNSUPPORTED;
    const size_t need = sa::attn_bwd_ws_bytes(bt.total_q, bt.max_ctx, n_q_heads, d_qk, d_v, k);
    if (workspace_bytes < need || (need && !workspace))
        return SA_EWORKSPACE;
    if (workspace && ((uintptr_t)workspace & 255))
        return SA_EINVAL;
    return launched(sa::launch_attn_bwd(bt, n_q_heads, d_qk, d_v, q, k_cache, v_cache, kv_row_stride, indices, k,
                                        gate_logits, gate_per_channel ? 1 : 0, softmax_scale, out, lse, d_out, d_q,
                                        d_k_cache, d_v_cache, d_gate, workspace, (hipStream_t)stream));
}

sa_status sparse_window_indices(const sa_batch *batch, int32_t window, int32_t *indices, sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (!indices || window < 1 || window > 65536)
        return SA_EINVAL;
    return launched(sa::launch_window_indices(bt, window, indices, (hipStream_t)stream));
}

sa_status sparse_branch_fuse(sa_dtype dtype, int64_t rows, int32_t d_v, const void *o_sparse, const void *o_local,
                             const void *gate_logits, int32_t gate_per_channel, void *out, sa_stream_t stream)
{
    if (dtype != SA_F32 && dtype != SA_BF16)
        return SA_EINVAL;
    if (rows == 0)
        return SA_OK;
    if (!o_sparse || !o_local || !gate_logits || !out || rows < 1 || d_v < 8 || (d_v % 8))
        return SA_EINVAL;
    if (!aligned16(o_sparse) || !aligned16(o_local) || !aligned16(out) ||
        (gate_per_channel && !aligned16(gate_logits)))
        return SA_EINVAL;
    return launched(sa::launch_branch_fuse((int)dtype, rows, d_v, o_sparse, o_local, gate_logits,
                                           gate_per_channel ? 1 : 0, out, (hipStream_t)stream));
}

sa_status sparse_cache_append(const sa_batch *batch, sa_dtype kv_dtype, const void *k_new, int32_t d_qk,
                              const void *v_new, int32_t d_v, void *k_cache, void *v_cache, int64_t kv_row_stride,
                              sa_dtype src_dtype, const void *k_idx_new, int32_t d_i, sa_dtype idx_dtype,
                              void *k_idx_cache, float *k_scale_cache, sa_stream_t stream)
{
    sa::Batch bt;
    sa_status st = make_batch(batch, &bt);
    if (st != SA_OK)
        return st == kEmptyBatch ? SA_OK : st;
    if (kv_dtype != SA_F32 && kv_dtype != SA_BF16)
        return SA_EINVAL;
    if (src_dtype != SA_F32 && src_dtype != SA_BF16)
        return SA_EINVAL;
    if (idx_dtype != src_dtype && idx_dtype != SA_FP8_E4M3)
        return SA_EINVAL;
    if (!k_new || !k_cache || !k_idx_new || !k_idx_cache || (v_new && !v_cache))
        return SA_EINVAL;
    if (idx_dtype == SA_FP8_E4M3 && !k_scale_cache)
        return SA_EINVAL;
    if (d_qk < 1 || d_i < 2 || (d_i & 1) || (v_new && d_v < 1))
        return SA_EINVAL;
    if (kv_row_stride < d_qk || (v_new && kv_row_stride < d_v))
        return SA_EINVAL;
    const int esz = kv_dtype == SA_BF16 ? 2 : 4;
    if ((d_qk * esz) % 16 || (v_new && (d_v * esz) % 16) || (kv_row_stride * esz) % 16)
        return SA_EINVAL;
    if (!aligned16(k_new) || !aligned16(k_cache) || (v_new && (!aligned16(v_new) || !aligned16(v_cache))))
        return SA_EINVAL;
    if (!aligned16(k_idx_new) || !aligned16(k_idx_cache))
        return SA_EINVAL;
    if (d_i > 2 * 64 * 8 || d_qk * esz > 4096 || (v_new && d_v * esz > 4096))
        return SA_EUNSUPPORTED;
    return launched(sa::launch_cache_append(bt, esz, k_new, d_qk, v_new, d_v, k_cache, v_cache, kv_row_stride,
                                            src_dtype == SA_F32 ? 1 : 0, k_idx_new, d_i,
                                            idx_dtype == SA_FP8_E4M3 ? 1 : 0, k_idx_cache, k_scale_cache,
                                            (hipStream_t)stream));
}

sa_status sparse_quantize_fp8_rows(sa_dtype src_dtype, const void *x, int64_t rows, int32_t cols, uint8_t *codes,
                                   float *scales, sa_stream_t stream)
{
    if (src_dtype != SA_F32 && src_dtype != SA_BF16)
        return SA_EINVAL;
    if (rows == 0)
        return SA_OK;
    if (!x || !codes || !scales || rows < 1 || rows > 0x7fffffff || cols < 8 || (cols & 7))
        return SA_EINVAL;
    if (!aligned16(x) || (((uintptr_t)codes) & 7u))
        return SA_EINVAL;
    return launched(sa::launch_quantize_rows(x, src_dtype == SA_F32 ? 1 : 0, rows, cols, codes, scales,
                                             (hipStream_t)stream));
}

const char *sa_status_string(sa_status s)
{
    switch (s) {
    case SA_OK: return "ok";
    case SA_EINVAL: return "invalid argument";
    case SA_EUNSUPPORTED: return "unsupported shape or dtype";
    case SA_EWORKSPACE: return "workspace missing, too small or misaligned";
    case SA_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

int32_t sa_abi_version(void) { return SA_ABI_VERSION; }

} // extern "C"
