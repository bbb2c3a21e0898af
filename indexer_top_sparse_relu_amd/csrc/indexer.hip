// a1 — indexer scores on MFMA (gfx950).
//
// Pages (by title):
//   [HAT] "Hybrid Attention Architectures: Engineering Trade-offs from Linear
//          Attention to Gated Sparse Attention", §3.1 and §3.3: a lightweight
//          relevance score of the query against every history position.
//   [F2S] "From Full Attention to Sparsity: The Evolution of Hybrid Attention
//          Architectures in Large Language Models", "Fine-Grained Sparse
//          Attention: Indexer Plus Top-K": few heads, low dims, content only,
//          one score per (query, position).
// Form (the DSA-style reading; the pages print no formula):
//   I[i,s] = sum_h w[i,h] * max(0, q[i,h,:] . k[s,:])   (fp8: dot * q_scale[i] * k_scale[s])
//
// The contraction q k^T runs on 32x32 MFMA tiles whose rows are (token, head)
// pairs and whose columns are key positions.  A lane of a 32x32 output holds
// 16 rows of one column, so the head reduction is mostly in-lane: ReLU and the
// w-FMA per element, then one cross-half add.  Positive scales factor out of
// the ReLU, so fp8 scales are applied once per (token, key).
//
// Two kernels:
//   indexer_tile_kernel — prefill: a workgroup owns TQ tokens of one sequence
//     and a chunk of keys; 64-key tiles are gathered through the page table
//     into LDS (double-buffered) and shared by all TQ tokens.  Workgroups are
//     mapped so that every key chunk stays on one XCD (its L2).
//   indexer_token_kernel — decode: one token per workgroup row, keys split over
//     workgroups and waves, key rows streamed straight from HBM into MFMA
//     operands (no reuse to stage for).
#include "sa_device.h"
#include "launch.h"

namespace sa {

// Per-dtype MFMA step.  ELEM bytes per element, KS contraction elements per
// instruction, LB bytes one lane supplies per instruction.
template <int DT> struct IdxT;
template <> struct IdxT<0> {
    static constexpr int ELEM = 4, KS = 2, LB = 4;
    typedef float Op;
    static __device__ __forceinline__ Op load(const uint8_t *p) { return *(const float *)p; }
    static __device__ __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) { return mma32_f32(a, b, c); }
};
template <> struct IdxT<1> {
    static constexpr int ELEM = 2, KS = 16, LB = 16;
    typedef bf16x8 Op;
    static __device__ __forceinline__ Op load(const uint8_t *p) { return *(const bf16x8 *)p; }
    static __device__ __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) { return mma32_bf16(a, b, c); }
};
template <> struct IdxT<2> {
    static constexpr int ELEM = 1, KS = 64, LB = 32;
    typedef i32x8 Op;
    static __device__ __forceinline__ Op load(const uint8_t *p) { return *(const i32x8 *)p; }
    static __device__ __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) { return mma32_fp8(a, b, c); }
};

// Rows per wave = 32*MT; tokens per wave = 32*MT/H.
template <int H> struct IdxShape {
    static constexpr int MT = H <= 8 ? 1 : (H <= 32 ? 2 : H / 16);
    static constexpr int TPW = 32 * MT / H;
};

constexpr int kIdxWaves = 4;
constexpr int kIdxTileKeys = 64;

// ------------------------------------------------------------------ prefill
template <int DT, int H, int D>
__global__ __launch_bounds__(256) void indexer_tile_kernel(
    Batch bt, const uint8_t *__restrict__ q_idx, const float *__restrict__ q_scale,
    const float *__restrict__ w, const uint8_t *__restrict__ k_idx, const float *__restrict__ k_scale,
    float *__restrict__ scores, int64_t ld, int key_chunk, int n_chunks, int n_tiles_max)
{
    typedef IdxT<DT> X;
    constexpr int MT = IdxShape<H>::MT, TPW = IdxShape<H>::TPW;
    constexpr int TQ = kIdxWaves * TPW;
    constexpr int RB = D * X::ELEM;              // bytes per key row
    constexpr int RBP = RB + 16;                 // padded LDS row (bank spread)
    constexpr int NKS = D / X::KS;               // MFMA steps along d
    constexpr bool FP8 = DT == 2;
    static_assert(RB % 32 == 0, "row bytes");
    __shared__ __align__(16) uint8_t lds_k[2][kIdxTileKeys * RBP];
    __shared__ float lds_ks[2][kIdxTileKeys];

    // ---- workgroup -> (token tile, key chunk): chunk c always runs on XCD c % 8
    const int bid = blockIdx.x;
    const int xcd = bid & 7, j = bid >> 3;
    const int cpx = (n_chunks - xcd + 7) >> 3;   // chunks owned by this XCD
    if (cpx <= 0)
        return;
    const int chunk = xcd + 8 * (j % cpx);
    int tile = j / cpx;
    if (tile >= n_tiles_max)
        return;
    int b = 0;
    for (; b < bt.num_seqs; ++b) {
        int nq = bt.q_start[b + 1] - bt.q_start[b];
        int nt = (nq + TQ - 1) / TQ;
        if (tile < nt)
            break;
        tile -= nt;
    }
    if (b >= bt.num_seqs)
        return;
    const int q0 = bt.q_start[b];
    const int nq = bt.q_start[b + 1] - q0;
    const int tok0 = q0 + tile * TQ;
    const int ntok = min(TQ, nq - tile * TQ);
    const int pos0 = bt.ctx_len[b] - nq + tile * TQ;      // position of token tok0
    const int kb0 = chunk * key_chunk;
    const int kb1 = min(kb0 + key_chunk, pos0 + ntok);    // last token sees pos0+ntok-1
    if (kb0 >= kb1)
        return;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int half = lane >> 5, col = lane & 31;

    // ---- A operands (this wave's tokens x heads) and weights, kept in registers
    typename X::Op a[MT][NKS];
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int R = mt * 32 + col;              // operand row of this lane
        const int tl = wv * TPW + R / H, h = R % H;
        const bool ok = tl < ntok;
        const uint8_t *src = q_idx + ((int64_t)(tok0 + (ok ? tl : 0)) * H + h) * RB;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            typename X::Op v = X::load(src + ks * X::KS * X::ELEM + half * X::LB);
            a[mt][ks] = ok ? v : typename X::Op{};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int Ro = mt * 32 + mfma32_row(i, lane);
            const int to = wv * TPW + Ro / H;
            wr[mt][i] = to < ntok ? w[(int64_t)(tok0 + to) * H + Ro % H] : 0.0f;
        }
    }
    float qs[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tl = wv * TPW + t;
        qs[t] = (FP8 && tl < ntok) ? q_scale[tok0 + tl] : 1.0f;
    }

    // ---- key tile staging: thread -> (key, 32-byte part)
    constexpr int PARTS = RB / 32;
    constexpr int LOADS = (kIdxTileKeys * PARTS + 255) / 256;
    i32x4 stage[LOADS][2];
    float stage_ks = 0.0f;
    auto gload = [&](int t0) {
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int e = tid + u * 256;
            const int kk = e / PARTS, p = e % PARTS;
            const int s = t0 + kk;
            if (kk < kIdxTileKeys && s < kb1) {
                const i32x4 *src = (const i32x4 *)(k_idx + phys_row(bt, b, s) * RB + p * 32);
                stage[u][0] = src[0];
                stage[u][1] = src[1];
            } else {
                stage[u][0] = i32x4{0, 0, 0, 0};
                stage[u][1] = i32x4{0, 0, 0, 0};
            }
        }
        if (FP8 && tid < kIdxTileKeys) {
            const int s = t0 + tid;
            stage_ks = s < kb1 ? k_scale[phys_row(bt, b, s)] : 0.0f;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
            const int e = tid + u * 256;
            const int kk = e / PARTS, p = e % PARTS;
            if (kk < kIdxTileKeys) {
                i32x4 *dst = (i32x4 *)(&lds_k[buf][kk * RBP + p * 32]);
                dst[0] = stage[u][0];
                dst[1] = stage[u][1];
            }
        }
        if (FP8 && tid < kIdxTileKeys)
            lds_ks[buf][tid] = stage_ks;
    };

    const int ntiles = (kb1 - kb0 + kIdxTileKeys - 1) / kIdxTileKeys;
    gload(kb0);
    lstore(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        const int t0 = kb0 + it * kIdxTileKeys;
        if (it + 1 < ntiles)
            gload(t0 + kIdxTileKeys);
#pragma unroll
        for (int nt = 0; nt < kIdxTileKeys / 32; ++nt) {
            f32x16 c[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                c[mt] = f32x16{};
            const uint8_t *brow = &lds_k[buf][(nt * 32 + col) * RBP + half * X::LB];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                typename X::Op bop = X::load(brow + ks * X::KS * X::ELEM);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    c[mt] = X::mma(a[mt][ks], bop, c[mt]);
            }
            // epilogue: ReLU, head weights, head sum
            const int s = t0 + nt * 32 + col;
            const float ks_s = FP8 ? lds_ks[buf][nt * 32 + col] : 1.0f;
            if constexpr (H >= 8) {
                float acc[TPW];
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    acc[t] = 0.0f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[(mt * 32 + 8 * (i >> 2)) / H] =
                            fmaf(wr[mt][i], fmaxf(c[mt][i], 0.0f), acc[(mt * 32 + 8 * (i >> 2)) / H]);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    acc[t] += shfl_xor(acc[t], 32);
                // lanes of half 0 write even wave-tokens, half 1 odd ones
#pragma unroll
                for (int t0w = 0; t0w < TPW; t0w += 2) {
                    const int t1 = t0w + 1 < TPW ? t0w + 1 : t0w;
                    const float v = half ? acc[t1] * qs[t1] : acc[t0w] * qs[t0w];
                    const int tl = wv * TPW + t0w + half;
                    if (t0w + half < TPW && tl < ntok && s <= pos0 + tl && s < kb1)
                        scores[(int64_t)(tok0 + tl) * ld + s] = v * ks_s;
                }
            } else {
                // H == 4: a lane's register group g holds rows 8g+4*half..+3, one whole token
                static_assert(H == 4, "n_heads");
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float acc = 0.0f;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc = fmaf(wr[mt][4 * g + r], fmaxf(c[mt][4 * g + r], 0.0f), acc);
                        const int te = mt * 8 + 2 * g;         // even token of the pair
                        const float qv = half ? qs[te + 1] : qs[te];
                        const int tl = wv * TPW + te + half;
                        if (tl < ntok && s <= pos0 + tl && s < kb1)
                            scores[(int64_t)(tok0 + tl) * ld + s] = acc * qv * ks_s;
                    }
            }
        }
        if (it + 1 < ntiles)
            lstore(buf ^ 1);
        __syncthreads();
    }
}

// ------------------------------------------------------------------- decode
// One token per blockIdx.y; blockIdx.x = key chunk.  Wave wv takes 32-key
// tiles wv, wv+4, ... of the chunk; each lane streams its key's bytes from
// HBM directly into the B operand.
template <int DT, int H, int D>
__global__ __launch_bounds__(256) void indexer_token_kernel(
    Batch bt, const uint8_t *__restrict__ q_idx, const float *__restrict__ q_scale,
    const float *__restrict__ w, const uint8_t *__restrict__ k_idx, const float *__restrict__ k_scale,
    float *__restrict__ scores, int64_t ld, int key_chunk)
{
    typedef IdxT<DT> X;
    constexpr int MT = (H + 31) / 32;
    constexpr int RB = D * X::ELEM;
    constexpr int NKS = D / X::KS;
    constexpr bool FP8 = DT == 2;

    const int tok = blockIdx.y;
    const int b = seq_of_token(bt, tok);
    const int pos = pos_of_token(bt, b, tok);
    const int kb0 = blockIdx.x * key_chunk;
    const int kb1 = min(kb0 + key_chunk, pos + 1);
    if (kb0 >= kb1)
        return;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int half = lane >> 5, col = lane & 31;

    typename X::Op a[MT][NKS];
    float wr[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int h = mt * 32 + col;
        const bool ok = h < H;
        const uint8_t *src = q_idx + ((int64_t)tok * H + (ok ? h : 0)) * RB;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            typename X::Op v = X::load(src + ks * X::KS * X::ELEM + half * X::LB);
            a[mt][ks] = ok ? v : typename X::Op{};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int ho = mt * 32 + mfma32_row(i, lane);
            wr[mt][i] = ho < H ? w[(int64_t)tok * H + ho] : 0.0f;
        }
    }
    const float qs = FP8 ? q_scale[tok] : 1.0f;

    const int ntiles = (kb1 - kb0 + 31) / 32;
    // two operand slots, software-pipelined; the loop is unrolled by two so
    // every register array index is a compile-time constant
    typename X::Op b0[NKS], b1[NKS];
    float ks0 = 0.0f, ks1 = 0.0f;
    auto gload = [&](typename X::Op (&bo)[NKS], float &ksv, int t) {
        const int s = kb0 + t * 32 + col;
        if (s < kb1) {
            const int64_t pr = phys_row(bt, b, s);
            const uint8_t *src = k_idx + pr * RB + half * X::LB;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                bo[ks] = X::load(src + ks * X::KS * X::ELEM);
            ksv = FP8 ? k_scale[pr] : 1.0f;
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                bo[ks] = typename X::Op{};
            ksv = 0.0f;
        }
    };
    auto compute = [&](typename X::Op (&bo)[NKS], float ksv, int t) {
        f32x16 c[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            c[mt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                c[mt] = X::mma(a[mt][ks], bo[ks], c[mt]);
        }
        float acc = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (mt * 32 + 8 * (i >> 2) < H)
                    acc = fmaf(wr[mt][i], fmaxf(c[mt][i], 0.0f), acc);
        acc += shfl_xor(acc, 32);
        const int s = kb0 + t * 32 + col;
        if (half == 0 && s < kb1)
            scores[(int64_t)tok * ld + s] = acc * qs * ksv;
    };
    constexpr int W = kIdxWaves;
    int t = wv;
    if (t < ntiles)
        gload(b0, ks0, t);
    for (; t < ntiles; t += 2 * W) {
        if (t + W < ntiles)
            gload(b1, ks1, t + W);
        compute(b0, ks0, t);
        if (t + 2 * W < ntiles)
            gload(b0, ks0, t + 2 * W);
        if (t + W < ntiles)
            compute(b1, ks1, t + W);
    }
}

// ------------------------------------------------------------------ launch
template <int DT, int H, int D>
static hipError_t launch_indexer_t(const Batch &bt, const void *q_idx, const float *q_scale, const float *w,
                                   const void *k_idx, const float *k_scale, float *scores, int64_t ld,
                                   hipStream_t st)
{
    if (bt.max_q >= 8) {
        constexpr int TQ = kIdxWaves * IdxShape<H>::TPW;
        // key chunks: a multiple of 8 (one set per XCD) once the context is long
        int n_chunks = bt.max_ctx > 8192 ? 8 * ((bt.max_ctx + 8 * 8192 - 1) / (8 * 8192)) : 1;
        int key_chunk = (bt.max_ctx + n_chunks - 1) / n_chunks;
        key_chunk = (key_chunk + kIdxTileKeys - 1) / kIdxTileKeys * kIdxTileKeys;
        n_chunks = (bt.max_ctx + key_chunk - 1) / key_chunk;
        const int n_tiles_max = (bt.total_q + TQ - 1) / TQ + bt.num_seqs - 1;
        const int cpx_max = (n_chunks + 7) / 8;
        const int64_t grid = 8LL * cpx_max * n_tiles_max;
        if (grid > 0x7fffffff)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((indexer_tile_kernel<DT, H, D>), dim3((unsigned)grid), dim3(256), 0, st, bt,
                           (const uint8_t *)q_idx, q_scale, w, (const uint8_t *)k_idx, k_scale, scores, ld,
                           key_chunk, n_chunks, n_tiles_max);
    } else {
        // enough workgroups to cover the GPU even for a handful of sequences
        int key_chunk = 2048;
        const int64_t want = 2048;
        while (key_chunk > 256 && (int64_t)bt.total_q * ((bt.max_ctx + key_chunk - 1) / key_chunk) < want)
            key_chunk >>= 1;
        const int n_chunks = (bt.max_ctx + key_chunk - 1) / key_chunk;
        if (bt.total_q > 65535)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((indexer_token_kernel<DT, H, D>), dim3(n_chunks, bt.total_q), dim3(256), 0, st, bt,
                           (const uint8_t *)q_idx, q_scale, w, (const uint8_t *)k_idx, k_scale, scores, ld,
                           key_chunk);
    }
    return hipGetLastError();
}

template <int DT, int D>
static int dispatch_heads(int H, const Batch &bt, const void *q_idx, const float *q_scale, const float *w,
                          const void *k_idx, const float *k_scale, float *scores, int64_t ld, hipStream_t st,
                          hipError_t *err)
{
    switch (H) {
    case 4: *err = launch_indexer_t<DT, 4, D>(bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st); return 1;
    case 8: *err = launch_indexer_t<DT, 8, D>(bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st); return 1;
    case 16: *err = launch_indexer_t<DT, 16, D>(bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st); return 1;
    case 32: *err = launch_indexer_t<DT, 32, D>(bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st); return 1;
    case 64: *err = launch_indexer_t<DT, 64, D>(bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st); return 1;
    default: return 0;
    }
}

int indexer_supported(int dtype, int H, int D)
{
    if (H != 4 && H != 8 && H != 16 && H != 32 && H != 64)
        return 0;
    return (dtype == 0 && D == 32) || (dtype == 1 && (D == 64 || D == 128)) || (dtype == 2 && D == 128);
}

hipError_t launch_indexer(int dtype, int H, int D, const Batch &bt, const void *q_idx, const float *q_scale,
                          const float *w, const void *k_idx, const float *k_scale, float *scores, int64_t ld,
                          hipStream_t st)
{
    hipError_t err = hipErrorInvalidValue;
    int ok = 0;
    if (dtype == 0 && D == 32)
        ok = dispatch_heads<0, 32>(H, bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st, &err);
    else if (dtype == 1 && D == 64)
        ok = dispatch_heads<1, 64>(H, bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st, &err);
    else if (dtype == 1 && D == 128)
        ok = dispatch_heads<1, 128>(H, bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st, &err);
    else if (dtype == 2 && D == 128)
        ok = dispatch_heads<2, 128>(H, bt, q_idx, q_scale, w, k_idx, k_scale, scores, ld, st, &err);
    return ok ? err : hipErrorInvalidValue;
}

} // namespace sa
