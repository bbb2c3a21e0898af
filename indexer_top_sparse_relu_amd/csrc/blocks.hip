// Block-level selection (gfx950): pooled block keys, block scores and the
// expansion of the selected blocks to positions.  The Top-K over block scores
// is the a2 kernel with block row lengths, and the attention is a3-a5
// unchanged, over the expanded index list.
//
// Pages (by title):
//   [SEL] "Hybrid Attention Architecture Evolution in LLMs: From Full
//          Attention to Sparse Selection", §3.2 (pseudocode: pool the keys by
//          block, score the blocks, keep the top-k blocks, gather them, exact
//          attention) and §4.1-4.2 (effective length k*b; block sparsity is
//          the form that turns into real speed-ups).
//   [SAD] "Sparse Attention and Hybrid Attention Architecture Design in Large
//          Language Models", §3 (block sparsity with top-k routing: relevance
//          between queries and key blocks at block granularity) and §2 (query
//          heads share a KV head).
//
// Readings: a block is one page of the paged cache, its pooled key the mean of
// its K rows, and the block score of token i sums its query heads' dots,
// S[i, j] = (sum_h q[i,h,:]) . kbar_j, over the blocks that start at or
// before pos(i) (one selection shared by the heads of the KV head).
#include "launch.h"
#include "sa_device.h"

namespace sa {

constexpr int kBlkThreads = 256;
constexpr int kBlkTok = 32;          // tokens per score tile (MFMA rows)
constexpr int kBlkCols = 128;        // blocks per score tile (4 waves x 32 MFMA columns)

__device__ __forceinline__ float load_elem(const uint8_t *base, int f32, int64_t i)
{
    return f32 ? ((const float *)base)[i] : __uint_as_float((uint32_t)((const uint16_t *)base)[i] << 16);
}

constexpr int kSumChunks = 4;       // 16-byte chunks per lane and row: rows of up to 4 KB

// Column sums (fp32) of nrows rows of `dims` elements (bf16 or f32), row r at
// base + r * row_bytes_stride, into out[0, dims) of LDS.  Wave w takes rows
// w, w + 4, ...; a lane takes 16-byte chunks lane, lane + 64, ... of each
// row, so every load is a coalesced 16-byte access; the four waves' partial
// sums meet in LDS.
__device__ void sum_rows(const uint8_t *__restrict__ base, int64_t row_bytes_stride, int nrows, int dims, int f32,
                         float *part /* LDS [4][dims] */, float *out /* LDS [dims] */)
{
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int per = f32 ? 4 : 8;                    // elements per 16-byte chunk
    const int nch = dims / per;
    float acc[kSumChunks][8];
#pragma unroll
    for (int k = 0; k < kSumChunks; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[k][e] = 0.0f;
#pragma unroll 4
    for (int r = wv; r < nrows; r += 4) {
        const uint8_t *row = base + r * row_bytes_stride;
#pragma unroll
        for (int k = 0; k < kSumChunks; ++k) {
            const int c = lane + 64 * k;
            if (c < nch) {
                const u32x4 w = *(const u32x4 *)(row + 16 * c);
                if (f32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[k][e] += __uint_as_float(w[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[k][2 * e] += __uint_as_float(w[e] << 16);
                        acc[k][2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kSumChunks; ++k) {
        const int c = lane + 64 * k;
        if (c < nch) {
            if (f32) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    part[wv * dims + c * 4 + e] = acc[k][e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    part[wv * dims + c * 8 + e] = acc[k][e];
            }
        }
    }
    __syncthreads();
    for (int d = threadIdx.x; d < dims; d += kBlkThreads)
        out[d] = (part[d] + part[dims + d]) + (part[2 * dims + d] + part[3 * dims + d]);
    __syncthreads();
}

// LDS of sum_rows: 4 partial rows and the sums, 5 * dims floats, sized at
// launch so that short rows leave room for more workgroups per CU.
__device__ __forceinline__ float *sum_lds()
{
    extern __shared__ __align__(16) float blk_lds[];
    return blk_lds;
}

// One workgroup per (block j, sequence b): the mean of the block's valid K
// rows (fp32 sums), written at k_blocks[page].
__global__ __launch_bounds__(kBlkThreads) void block_pool_kernel(Batch bt, const uint8_t *__restrict__ k_cache,
                                                                 int f32, int d_qk, int64_t row_stride,
                                                                 float *__restrict__ k_blocks)
{
    float *part = sum_lds(), *sums = part + 4 * d_qk;
    const int j = blockIdx.x, b = blockIdx.y;
    const int ps = 1 << bt.page_shift;
    const int L = bt.ctx_len[b];
    if (j >= ((L + ps - 1) >> bt.page_shift))
        return;
    const int64_t page = bt.page_table[(int64_t)b * bt.max_pages + j];
    const int len = min(ps, L - j * ps);
    const int esz = f32 ? 4 : 2;
    sum_rows(k_cache + page * ps * row_stride * esz, row_stride * esz, len, d_qk, f32, part, sums);
    for (int d = threadIdx.x; d < d_qk; d += kBlkThreads)
        k_blocks[page * d_qk + d] = sums[d] / (float)len;
}

// qbar[i, :] = sum over the query heads of q[i, h, :] (fp32); one workgroup
// per token.
__global__ __launch_bounds__(kBlkThreads) void qbar_kernel(const uint8_t *__restrict__ q, int f32, int Hq, int d_qk,
                                                           float *__restrict__ qbar)
{
    float *part = sum_lds(), *sums = part + 4 * d_qk;
    const int64_t i = blockIdx.x;
    const int esz = f32 ? 4 : 2;
    sum_rows(q + i * Hq * d_qk * esz, (int64_t)d_qk * esz, Hq, d_qk, f32, part, sums);
    for (int d = threadIdx.x; d < d_qk; d += kBlkThreads)
        qbar[i * d_qk + d] = sums[d];
}

// Block scores on fp32 MFMA (32x32x2): a workgroup takes 32 consecutive tokens
// of one sequence and 128 blocks (32 per wave).  Each 32-dim chunk of the token
// rows (A) and the block rows (B) goes into LDS by direct loads of whole
// 128-byte row pieces (8 rows per load instruction), double-buffered; lane (row
// l % 32, half h) then reads dims 16h .. 16h+15 of its rows with four 16-byte
// LDS reads.  Chunk c of row r sits at slot c ^ ((r >> 1) & 7), so the 16 lanes
// of a read phase hit distinct banks.  Tokens past the tile and blocks past the
// sequence read row 0 and are not stored.  (Loaded straight into the MFMA
// layout, every load instruction touched 32 rows: the address unit's cost.)
constexpr int kBsRows = kBlkTok + kBlkCols;     // LDS rows of 128 bytes per chunk
constexpr int kBsLoads = kBsRows / 8 / 4;       // direct loads per wave per chunk
static_assert(kBsRows % 32 == 0, "whole load instructions per wave");

__global__ __launch_bounds__(kBlkThreads) void block_scores_kernel(Batch bt, const float *__restrict__ qbar, int d_qk,
                                                                   const float *__restrict__ k_blocks,
                                                                   float *__restrict__ scores, int64_t ld,
                                                                   int n_tiles_max)
{
    __shared__ __align__(16) uint8_t lbuf[2][kBsRows * 128];
    int tile = blockIdx.x;
    if (tile >= n_tiles_max)
        return;
    int b = 0;
    for (; b < bt.num_seqs; ++b) {
        const int nq = bt.q_start[b + 1] - bt.q_start[b];
        const int nt = (nq + kBlkTok - 1) / kBlkTok;
        if (tile < nt)
            break;
        tile -= nt;
    }
    if (b >= bt.num_seqs)
        return;
    const int q0 = bt.q_start[b], nq = bt.q_start[b + 1] - q0;
    const int tok0 = q0 + tile * kBlkTok;
    const int ntok = min(kBlkTok, nq - tile * kBlkTok);
    const int pos0 = bt.ctx_len[b] - nq + tile * kBlkTok;        // position of token tok0
    const int nb_max = ((pos0 + ntok - 1) >> bt.page_shift) + 1;  // candidate blocks of the tile's last token
    const int jg0 = blockIdx.y * kBlkCols;
    if (jg0 >= nb_max)
        return;                             // the whole workgroup
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, hf = lane >> 5;
    // load i of this wave covers LDS rows 8u .. 8u+7, u = wv + 4i: lane l brings the
    // 16 bytes of physical slot l & 7 of row 8u + (l >> 3), i.e. its logical chunk
    // (l & 7) ^ ((row >> 1) & 7); rows 0..31 are the tile's tokens, rows 32.. its blocks
    const float *src[kBsLoads];
#pragma unroll
    for (int i = 0; i < kBsLoads; ++i) {
        const int row = 8 * (wv + 4 * i) + (lane >> 3);
        const int lc = (lane & 7) ^ ((row >> 1) & 7);
        const float *rp;
        if (row < kBlkTok) {
            rp = qbar + (int64_t)(tok0 + (row < ntok ? row : 0)) * d_qk;
        } else {
            const int j = jg0 + row - kBlkTok;
            rp = k_blocks + (int64_t)bt.page_table[(int64_t)b * bt.max_pages + (j < nb_max ? j : 0)] * d_qk;
        }
        src[i] = rp + 4 * lc;
    }
    auto issue = [&](int c, int buf) {
#pragma unroll
        for (int i = 0; i < kBsLoads; ++i)
            dma_b128(src[i] + 32 * c, (const lds_u8 *)&lbuf[buf][(wv + 4 * i) * 1024]);
    };
    const int ra = col, rb = kBlkTok + wv * 32 + col;
    auto ld4 = [&](int buf, int row, int q) {
        const int slot = (4 * hf + q) ^ ((row >> 1) & 7);
        return *(const __attribute__((address_space(3))) f32x4 *)&lbuf[buf][row * 128 + 16 * slot];
    };
    const int nch = d_qk / 32;
    f32x16 acc = f32x16{};
    issue(0, 0);
    for (int c = 0; c < nch; ++c) {
        const int cur = c & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // this wave's loads of chunk c
        __syncthreads();                    // every wave's loads of chunk c; buffer cur ^ 1 is free
        if (c + 1 < nch)
            issue(c + 1, cur ^ 1);
        f32x4 a[4], bb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            a[q] = ld4(cur, ra, q);
            bb[q] = ld4(cur, rb, q);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m >> 2][m & 3], bb[m >> 2][m & 3], acc, 0, 0, 0);
    }
    // output: lane holds block column jg0 + 32wv + col, token rows 8*(i/4) + 4*hf + i%4
    const int j = jg0 + wv * 32 + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * hf + (i & 3);
        if (r < ntok && j <= ((pos0 + r) >> bt.page_shift))
            scores[(int64_t)(tok0 + r) * ld + j] = acc[i];
    }
}

// One wave per token: slot e of its kb * page_size index row is position
// blk*page_size + t of selected block k = e / page_size (t = e % page_size),
// or -1 past the token's position or for an empty block slot.  The Top-K
// lists blocks in ascending order with empty slots last, and only the block
// holding pos(i) can be cut, so the rows come out as ascending positions
// followed by -1.
__global__ __launch_bounds__(kBlkThreads) void block_expand_kernel(Batch bt, const int32_t *__restrict__ blk, int kb,
                                                                   int32_t *__restrict__ out)
{
    const int tok = blockIdx.x * (kBlkThreads / 64) + (threadIdx.x >> 6);
    if (tok >= bt.total_q)
        return;
    const int lane = threadIdx.x & 63;
    const int b = seq_of_token(bt, tok);
    const int pos = pos_of_token(bt, b, tok);
    const int sh = bt.page_shift;
    const int width = kb << sh;
    for (int e = lane; e < width; e += 64) {
        const int j = blk[(int64_t)tok * kb + (e >> sh)];
        const int p = (j << sh) + (e & ((1 << sh) - 1));
        out[(int64_t)tok * width + e] = (j >= 0 && p <= pos) ? p : -1;
    }
}

hipError_t launch_block_pool(const Batch &bt, int dtype, const void *k_cache, int d_qk, int64_t row_stride,
                             float *k_blocks, hipStream_t st)
{
    const int max_blocks = (bt.max_ctx + (1 << bt.page_shift) - 1) >> bt.page_shift;
    hipLaunchKernelGGL(block_pool_kernel, dim3(max_blocks, bt.num_seqs), dim3(kBlkThreads), 5 * d_qk * 4, st, bt,
                       (const uint8_t *)k_cache, dtype == 0 ? 1 : 0, d_qk, row_stride, k_blocks);
    return hipGetLastError();
}

hipError_t launch_block_scores(const Batch &bt, int dtype, const void *q, int Hq, int d_qk, const float *k_blocks,
                               float *scores, int64_t ld, float *qbar, hipStream_t st)
{
    hipLaunchKernelGGL(qbar_kernel, dim3(bt.total_q), dim3(kBlkThreads), 5 * d_qk * 4, st, (const uint8_t *)q,
                       dtype == 0 ? 1 : 0, Hq, d_qk, qbar);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int max_blocks = (bt.max_ctx + (1 << bt.page_shift) - 1) >> bt.page_shift;
    const int n_tiles_max = (bt.total_q + kBlkTok - 1) / kBlkTok + bt.num_seqs - 1;
    hipLaunchKernelGGL(block_scores_kernel, dim3(n_tiles_max, (max_blocks + kBlkCols - 1) / kBlkCols),
                       dim3(kBlkThreads), 0, st, bt, qbar, d_qk, k_blocks, scores, ld, n_tiles_max);
    return hipGetLastError();
}

hipError_t launch_block_expand(const Batch &bt, const int32_t *blk, int kb, int32_t *indices, hipStream_t st)
{
    const int per = kBlkThreads / 64;
    hipLaunchKernelGGL(block_expand_kernel, dim3((bt.total_q + per - 1) / per), dim3(kBlkThreads), 0, st, bt, blk,
                       kb, indices);
    return hipGetLastError();
}

} // namespace sa
