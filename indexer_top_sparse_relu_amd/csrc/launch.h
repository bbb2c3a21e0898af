// Internal launchers shared by the kernel sources and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

struct Batch;

// a1
int indexer_supported(int dtype, int H, int D);
hipError_t launch_indexer(int dtype, int H, int D, const Batch &bt, const void *q_idx, const float *q_scale,
                          const float *w, const void *k_idx, const float *k_scale, float *scores, int64_t ld,
                          hipStream_t st);

// a2
struct TopkPlan {
    int chunked;      // 1: per-chunk selection followed by a merge pass
    int chunk;        // chunk length (positions) when chunked
    int n_chunks;     // chunks per row when chunked
    int group;        // chunk lists per first-level merge (n_chunks: one merge level)
    size_t ws_bytes;  // workspace the plan needs
    int thr;          // chunked by a per-row sampled threshold (compaction, then one finish per row)
    int reg;          // slots per thread when every row is held in registers (16), else 0
};
TopkPlan topk_plan(int total_q, int max_ctx, int k);
// len_shift 0: row i holds the pos_i + 1 position scores; len_shift > 0: the
// (pos_i >> len_shift) + 1 scores of its candidate blocks
hipError_t launch_topk(const Batch &bt, const TopkPlan &plan, const float *scores, int64_t ld, int k,
                       int32_t *indices, void *ws, hipStream_t st, int len_shift = 0);

// a3-a5
struct AttnPlan {
    int n_split;      // workgroups per (token, head group) along the index list
    size_t ws_bytes;
};
AttnPlan attn_plan(int total_q, int Hq, int d_v, int k);
int attn_supported(int dtype, int Hq, int d_qk, int d_v);
int attn_supported_layout(int dtype, int d_qk, int d_v, int aliased);
hipError_t launch_attn(int dtype, const Batch &bt, const AttnPlan &plan, const void *q, int Hq, int d_qk,
                       const void *k_cache, const void *v_cache, int d_v, int64_t row_stride,
                       const int32_t *indices, int k, const void *gate, int per_channel, float scale,
                       void *out, float *lse, void *ws, hipStream_t st, const void *mix = nullptr);

// block-level selection
hipError_t launch_block_pool(const Batch &bt, int dtype, const void *k_cache, int d_qk, int64_t row_stride,
                             float *k_blocks, hipStream_t st);
hipError_t launch_block_scores(const Batch &bt, int dtype, const void *q, int Hq, int d_qk, const float *k_blocks,
                               float *scores, int64_t ld, float *qbar, hipStream_t st);
hipError_t launch_block_expand(const Batch &bt, const int32_t *blk, int kb, int32_t *indices, hipStream_t st);

// backward over fixed indices
int attn_bwd_supported(int dtype, int Hq, int d_qk, int d_v);
int attn_bwd_needs_shared(int d_qk, int d_v);
size_t attn_bwd_ws_bytes(int T, int max_ctx, int Hq, int d_qk, int d_v, int K);
// key-major dK, dV (d = 64 or 128; 16, 32 or 64 heads), from the backward's workspace
hipError_t launch_attn_bwd_kv(const Batch &bt, int Hq, int d, bool shared, const void *q, const void *kc,
                              const void *vc, int64_t rs, float scale, const float *lse, const uint16_t *dO,
                              const float *Dh, const uint32_t *bits, int W, float *dk, float *dv, hipStream_t st);
hipError_t launch_attn_bwd(const Batch &bt, int Hq, int d_qk, int d_v, const void *q, const void *kc,
                           const void *vc, int64_t rs, const int32_t *idx, int K, const void *gate, int per_channel,
                           float scale, const void *y, const float *lse, const void *dy, float *dq, float *dk,
                           float *dv, float *dgate, void *ws, hipStream_t st);

// branch fusion with a local branch
hipError_t launch_window_indices(const Batch &bt, int w, int32_t *indices, hipStream_t st);
hipError_t launch_branch_fuse(int dtype, int64_t rows, int dv, const void *a, const void *b, const void *gate,
                              int per_channel, void *y, hipStream_t st);

// cache append + fp8 quantisation
hipError_t launch_cache_append(const Batch &bt, int kv_esz, const void *k_new, int d_qk, const void *v_new, int d_v,
                               void *k_cache, void *v_cache, int64_t row_stride, int src_f32, const void *kidx_new,
                               int d_i, int fp8, void *kidx_cache, float *kscale_cache, hipStream_t st);
hipError_t launch_quantize_rows(const void *x, int src_f32, int64_t rows, int cols, uint8_t *codes, float *scales,
                                hipStream_t st);

} // namespace sa
