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
// the ReLU, so fp8 scales are applied once per (token, key).  The fp8 path runs
// the epilogue on packed fp16 pairs (convert, ReLU, dot2 with fp32
// accumulation: 1.5 VALU instructions per element instead of 2): the MFMA's
// own block scales shrink every dot by 2^-10 so it always fits fp16, and the
// factor is given back once per score.  Each term then carries a relative
// rounding of at most 2^-10 (dot) and 2^-11 (weight) before the fp32 sum.
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
    static __device__ __forceinline__ f32x16 mma(Op a, Op b, f32x16 c) { return mma32_fp8_s10(a, b, c); }
};
// fp8 MFMAs of the packed-fp16 epilogue return dots scaled by 2^-10 (UNSCALE
// gives it back per score); with at least 8 heads the fp8 epilogue runs on
// packed fp16 pairs.  The linear-term path (fp32 epilogue) takes the products
// unscaled.
template <int DT> struct IdxEpi {
    static constexpr bool F16 = DT == 2;
    static constexpr float UNSCALE = DT == 2 ? 1024.0f : 1.0f;
};

// Rows per wave = 32*MT; tokens per wave = 32*MT/H.
template <int H> struct IdxShape {
    static constexpr int MT = H <= 8 ? 1 : (H <= 32 ? 2 : H / 16);
    static constexpr int TPW = 32 * MT / H;
};

constexpr int kIdxWaves = 4;
constexpr int kIdxTileKeys = 64;
constexpr int kIdxLinTileKeys = 128;   // key tile of the fp8 linear-term path
constexpr int kIdxMaxChunk = 17408;    // keys per prefill workgroup, at most
constexpr int kIdxChunkTarget = 17408; // prefill chunks: this many keys or fewer, eight at a time
constexpr int kIdxTokChunk = 2048;     // keys per decode workgroup, at most

typedef __attribute__((address_space(3))) float lds_f32;


// ------------------------------------------------------------------ prefill
template <int DT, int H, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void indexer_tile_kernel(
    Batch bt, const uint8_t *__restrict__ q_idx, const float *__restrict__ q_scale,
    const float *__restrict__ w, const uint8_t *__restrict__ k_idx, const float *__restrict__ k_scale,
    float *__restrict__ scores, int64_t ld, int key_chunk, int n_chunks, int n_tiles_max, int rotate,
    int last_open)
{
    typedef IdxT<DT> X;
    constexpr int MT = IdxShape<H>::MT, TPW = IdxShape<H>::TPW;
    constexpr int TQ = kIdxWaves * TPW;
    constexpr int RB = D * X::ELEM;              // bytes per key row
    constexpr int RBP = RB + 16;                 // padded LDS row (bank spread)
    constexpr int NKS = D / X::KS;               // MFMA steps along d
    constexpr bool FP8 = DT == 2;
    static_assert(RB % 32 == 0, "row bytes");
    // fp8 with >= 16 heads: the linear part of the ReLU runs on the MFMA (see below)
    constexpr bool LIN = (DT == 2) && (H >= 16) && (MT % 2 == 0) && (D == 128);
    __shared__ __align__(16) uint8_t lds_k[2][LIN ? 16 : kIdxTileKeys * RBP];
    __shared__ float lds_ks[2][LIN ? 1 : kIdxTileKeys];
    __shared__ __align__(16) uint8_t lkr0[LIN ? kIdxLinTileKeys * 128 : 16];
    __shared__ __align__(16) uint8_t lkr1[LIN ? kIdxLinTileKeys * 128 : 16];
    __shared__ __align__(16) uint8_t lkr2[LIN ? kIdxLinTileKeys * 128 : 16];
    __shared__ float lksr[LIN ? 3 * kIdxWaves * kIdxLinTileKeys : 1];
    __shared__ int lpt[kIdxMaxChunk / 16 + 2];
    constexpr int LTS = 128 + 16;                // padded term row (bank spread, as RBP)
    constexpr int TROWS = TPW == 2 ? 16 : 32;  // used rows of a wave's term tile
    __shared__ __align__(16) uint8_t lterm[LIN ? kIdxWaves * TROWS * LTS : 16];
    __shared__ int lscl[LIN ? kIdxWaves * 32 : 1];

    // ---- workgroup -> (token tile, key chunk).  Consecutive workgroups go to
    // consecutive XCDs.  Without rotation chunk c always runs on XCD c % 8, so
    // its k^I rows stay in one L2.  With rotation (all keys fit in one L2, and
    // n_chunks is a multiple of 8) token tile t puts chunk c on XCD (c - t) % 8,
    // so that causal prefill, where early tiles see only the first chunks,
    // spreads its work evenly over the XCDs.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, j = bid >> 3;
    int chunk, tile;
    if (rotate) {
        const int cpx = n_chunks >> 3;
        tile = j / cpx;
        chunk = ((xcd + tile) & 7) + 8 * (j % cpx);
    } else {
        const int cpx = (n_chunks - xcd + 7) >> 3;   // chunks owned by this XCD
        if (cpx <= 0)
            return;
        chunk = xcd + 8 * (j % cpx);
        tile = j / cpx;
    }
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
    // last token sees pos0+ntok-1; an open last chunk runs to it
    const int kb1 = (last_open && chunk == n_chunks - 1) ? pos0 + ntok : min(kb0 + key_chunk, pos0 + ntok);
    if (kb0 >= kb1)
        return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int half = lane >> 5, col = lane & 31;

    // ---- A operands (this wave's tokens x heads) and weights, kept in registers
    constexpr bool F16E = IdxEpi<DT>::F16 && H >= 8 && !LIN;
    typename X::Op a[MT][NKS];
    float wr[MT][F16E ? 1 : 16];
    float wt[MT][F16E ? 16 : 1];
    f16x2 wp[MT][F16E ? 8 : 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int R = mt * 32 + col;              // operand row of this lane
        const int tl = wv * TPW + R / H, h = R % H;
        // Rows of tokens past the tile's end read the tile's first token: their
        // products are finite, only ever summed into their own token (whose
        // weights are zero), and never stored.
        const uint8_t *src = q_idx + ((int64_t)(tok0 + (tl < ntok ? tl : 0)) * H + h) * RB;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            a[mt][ks] = X::load(src + ks * X::KS * X::ELEM + half * X::LB);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int Ro = mt * 32 + mfma32_row(i, lane);
            const int to = wv * TPW + Ro / H;
            // unconditional load (clamped token), then select: no branch per weight
            const float wl = w[(int64_t)(tok0 + min(to, ntok - 1)) * H + Ro % H];
            const float wv_ = to < ntok ? wl : 0.0f;
            if constexpr (F16E)
                wt[mt][i] = wv_;
            else
                wr[mt][i] = wv_;
        }
    }
    // fp16 weights: each token's weights are scaled by a power of two that puts
    // their largest magnitude in [2^14, 2^15) (no overflow, no subnormals for
    // 28 binades below it); the factor is given back through the score scale
    int wsh[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        wsh[t] = 0;
    if constexpr (F16E) {
        float tmax[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            tmax[t] = 0.0f;
        // with H >= 8 the token of register i is the same in both lane halves
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                tmax[(mt * 32 + 8 * (i >> 2)) / H] = fmaxf(tmax[(mt * 32 + 8 * (i >> 2)) / H], fabsf(wt[mt][i]));
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            wsh[t] = f16_weight_shift(fmaxf(tmax[t], __shfl_xor(tmax[t], 32, 64)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                wp[mt][i >> 1][i & 1] = (_Float16)ldexpf(wt[mt][i], wsh[(mt * 32 + 8 * (i >> 2)) / H]);
    }
    if constexpr (LIN) {
        // opaque from here on, so the selects above are not redone inside the key loop
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                asm volatile("" : "+v"(wr[mt][i]));
    }
    float qs[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tl = wv * TPW + t;
        qs[t] = ldexpf(((FP8 && tl < ntok) ? q_scale[tok0 + tl] : 1.0f) * (LIN ? 1.0f : IdxEpi<DT>::UNSCALE), -wsh[t]);
    }

    // Physical page of every page the chunk touches, staged once in LDS, so a
    // tile's key loads never wait on a page-table load.
    const int pshift = bt.page_shift, pmask = (1 << pshift) - 1;
    const int pg0 = kb0 >> pshift;
    {
        const int npg = ((kb1 - 1) >> pshift) - pg0 + 1;
        for (int i = tid; i < npg; i += 256)
            lpt[i] = bt.page_table[(int64_t)b * bt.max_pages + pg0 + i];
    }
    auto krow = [&](int s) -> int64_t { return ((int64_t)lpt[(s >> pshift) - pg0] << pshift) + (s & pmask); };

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
                const i32x4 *src = (const i32x4 *)(k_idx + krow(s) * RB + p * 32);
                stage[u][0] = src[0];
                stage[u][1] = src[1];
            } else {
                stage[u][0] = i32x4{0, 0, 0, 0};
                stage[u][1] = i32x4{0, 0, 0, 0};
            }
        }
        if (FP8 && tid < kIdxTileKeys) {
            const int s = t0 + tid;
            stage_ks = s < kb1 ? k_scale[krow(s)] : 0.0f;
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
    if constexpr (!LIN) {
        __syncthreads();                         // the staged page ids
        gload(kb0);
        lstore(0);
        __syncthreads();
    }

    if constexpr (LIN) {
        // w * ReLU(x) = (w x + w |x|) / 2.  The w |x| sum is one FMA per element
        // (|x| is a free source modifier); the linear sum over heads,
        // sum_h w_h (q_h . k) = (sum_h w_h q_h) . k, runs on the MFMA as extra A
        // rows: the weighted query qbar is split into 8 fp8 terms, term t scaled
        // by 2^e_t, and each row's 2^e_t is applied by the MFMA's per-row block
        // scale.  Eight terms carry qbar to full fp32 precision.
        // Four tokens per wave: the 32-row term tile is a 32x32x64 MFMA A
        // operand, token tt's term t at row 8*(2*(tt/2) + t/4) + 4*(tt%2) + t%4,
        // so in the 32x32 output the terms of token tt land in the lanes of half
        // tt%2 (registers 0-7 for tt < 2, 8-15 for tt >= 2): the lanes that write
        // that token's scores.  Two tokens per wave: the 16 term rows (row
        // 8*tt + t) are a 16x16x128 MFMA A operand, half the MFMA work of a
        // 32-row tile; see the key loop for how its output reaches the writers.
        uint8_t *myterm = lterm + wv * TROWS * LTS;
        int *myscl = lscl + wv * 32;
        for (int e = lane; e < TROWS * LTS / 16; e += 64)
            ((i32x4 *)myterm)[e] = i32x4{0, 0, 0, 0};
        if (lane < 32)
            myscl[lane] = 127;
        for (int tt = 0; tt < TPW; ++tt) {
            const int tl = wv * TPW + tt;
            if (tl >= ntok)
                break;
            const int tok = tok0 + tl;
            // qbar at dims 2*lane, 2*lane+1: the H loads are all issued before
            // the first use, so the sum waits for one memory round trip
            const uint8_t *qp = q_idx + (int64_t)tok * H * 128 + 2 * lane;
            const float *wt = w + (int64_t)tok * H;
            int pq[H];
#pragma unroll
            for (int h = 0; h < H; ++h)
                pq[h] = *(const uint16_t *)(qp + h * 128);
            float r0 = 0.0f, r1 = 0.0f;
#pragma unroll
            for (int h = 0; h < H; ++h) {
                r0 = fmaf(wt[h], __builtin_amdgcn_cvt_f32_fp8(pq[h], 0), r0);
                r1 = fmaf(wt[h], __builtin_amdgcn_cvt_f32_fp8(pq[h], 1), r1);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float mx = wave_max(fmaxf(fabsf(r0), fabsf(r1)));
                const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFF) - 127;   // floor(log2 mx)
                const int e = ex - 7;                                             // mx * 2^-e < 256
                if (mx > 0.0f && ex > -100) {
                    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(r0, -e), ldexpf(r1, -e), 0, false);
                    r0 -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(pk, 0), e);
                    r1 -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(pk, 1), e);
                    const int row = TPW == 2 ? 8 * tt + t : 8 * (2 * (tt >> 1) + (t >> 2)) + 4 * (tt & 1) + (t & 3);
                    *(uint16_t *)(myterm + row * LTS + 2 * lane) = (uint16_t)pk;
                    if (lane == 0)
                        myscl[row] = e + 127;                  // 2^e (B unscaled)
                }
            }
        }
        __syncthreads();
        const int sal = myscl[TPW == 2 ? (lane & 15) : col];
        const uint8_t *arow = TPW == 2 ? myterm + (lane & 15) * LTS + (lane >> 4) * 32 : myterm + col * LTS + half * X::LB;

        // Key tiles: a ring of KST stages of LT = 128 rows x 128 bytes, filled by
        // direct global->LDS loads (no registers).  The 16-byte chunk c of row r
        // sits at chunk position c ^ ((r >> 1) & 7): the B-operand reads (16 rows
        // of one chunk per LDS phase) then hit 16 distinct bank groups.  Wave wv
        // loads the 1 KB blocks wv + 4m, m = 0..3 (8 rows each), and its own copy
        // of the tile's 128 key scales (two loads of 64).  Positions past the
        // chunk are clamped to its last key, so every tile, also one past the
        // end, is a full, in-bounds load.
        constexpr int KST = 3;
        constexpr int LT = kIdxLinTileKeys;
        constexpr int NB = LT / 8 / kIdxWaves;          // 1 KB row blocks per wave per tile
        constexpr int NS = LT / 64;                     // key-scale loads per wave per tile
        const int ntiles = (kb1 - kb0 + LT - 1) / LT;
        auto stage = [&](int st) -> lds_u8 * {
            return st == 0 ? (lds_u8 *)lkr0 : st == 1 ? (lds_u8 *)lkr1 : (lds_u8 *)lkr2;
        };
        lds_f32 *const LKS = (lds_f32 *)lksr;
        // The lane's key positions of tile tt (NB rows of the key tile, NS key
        // scales) and their physical pages.  The pages are read from LDS one
        // tile ahead of the loads, inside the previous tile's MFMA work, so the
        // issue itself waits on nothing.  A row-block load covers one 8-row group
        // (8-aligned, so inside one page: pages hold a power of two >= 16 rows): its
        // page is wave-uniform and kept in a scalar register, and the address is a
        // scalar page base plus a 32-bit lane offset.  Positions past the chunk are
        // clamped to its last key, which lies in the group's own page or, for a
        // group wholly past it, in the page all of its rows are clamped to.
        struct Pg { int p[NB + NS]; };
        auto krow_of = [&](int m, int ln) { return (kIdxWaves * m + wv) * 8 + (ln >> 3); };
        auto kpos = [&](int tt, int ln, int which) {
            const int t0 = kb0 + tt * LT;
            const int r = which < NB ? krow_of(which, ln) : 64 * (which - NB) + ln;
            return min(t0 + r, kb1 - 1);
        };
        // The row blocks' pages come from one LDS read (lane w reads block w's) and
        // reach scalar registers by lane reads, so the wave waits on a single LDS
        // round trip for them.
        auto pages = [&](int tt, int ln) {
            Pg g;
            const int t0 = kb0 + tt * LT;
            const int wl = min(ln, NB - 1);
            const int pw = lpt[(min(t0 + 8 * (kIdxWaves * wl + wv), kb1 - 1) >> pshift) - pg0];
#pragma unroll
            for (int w = 0; w < NB + NS; ++w) {
                if (w < NB)
                    g.p[w] = __builtin_amdgcn_readlane(pw, w);
                else
                    g.p[w] = lpt[(kpos(tt, ln, w) >> pshift) - pg0];
            }
            return g;
        };
        // load w of tile tt: row block w (w < NB) or key-scale load w - NB
        auto issue_part = [&](int tt, int ln, const Pg &pg, int w) {
            const int st = tt % KST;
            const uint32_t inpage = (uint32_t)(kpos(tt, ln, w) & pmask);
            if (w < NB) {
                const int r = krow_of(w, ln);
                const uint8_t *sb = k_idx + ((uint64_t)(uint32_t)pg.p[w] << (pshift + 7));
                dma_b128_sv(sb, (inpage << 7) + (uint32_t)(((ln & 7) ^ ((r >> 1) & 7)) * 16),
                            stage(st) + (kIdxWaves * w + wv) * 1024);
            } else {
                dma_b32(k_scale + (((int64_t)pg.p[w] << pshift) + inpage),
                        (const lds_u8 *)(LKS + (st * kIdxWaves + wv) * LT + 64 * (w - NB)));
            }
        };
        auto issue = [&](int tt, int ln, const Pg &pg) {
#pragma unroll
            for (int w = 0; w < NB + NS; ++w)
                issue_part(tt, ln, pg, w);
        };

        // Scores go out through a buffer resource spanning this wave's token rows:
        // a masked lane gets an offset past the end, which the hardware drops, so
        // every store instruction issues and the memory-op count per tile is fixed.
        const int wt0 = min(wv * TPW, ntok - 1);
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            scores + (int64_t)(tok0 + wt0) * ld, 0, (int)(TPW * ld * 4), 0x00020000);

        constexpr int MH = MT / 2, TH = TPW / 2;
        // Per half gh of the M-tiles, loop-invariant: the lane's score limit (it writes
        // position s when s < lim, i.e. s <= pos(token) and s < kb1; 0 when it writes
        // nothing), its token row's byte offset in the buffer, and half its token's scale.
        int lim[2];
        uint32_t rowoff[2];
        float qh[2];
        // With one token per half (two per wave) the limit is wave-uniform: each
        // token gets a buffer resource of exactly its lim scores, so the range
        // check drops positions past it and the other half's lanes carry an
        // offset past the end; a store then needs one address operation.
        __amdgpu_buffer_rsrc_t srt[2];
#pragma unroll
        for (int gh = 0; gh < 2; ++gh) {
            const int tw = TH == 1 ? 0 : half;
            const int tl = wv * TPW + gh * TH + tw;
            const bool writes = (TH > 1 || half == gh) && tl < ntok;
            lim[gh] = writes ? min(kb1, pos0 + tl + 1) : 0;
            rowoff[gh] = writes ? (uint32_t)((int64_t)(tl - wt0) * ld * 4) : 0u;
            qh[gh] = 0.5f * ((TH > 1 && half) ? qs[gh * TH + TH - 1] : qs[gh * TH]);
            if constexpr (TH == 1) {
                const int tu = wv * TPW + gh;                       // wave-uniform
                const int lu = tu < ntok ? min(kb1, pos0 + tu + 1) : 0;
                srt[gh] = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)(tok0 + min(tu, ntok - 1)) * ld, 0,
                                                            4 * lu, 0x00020000);
                rowoff[gh] = half == gh ? 0u : 0x80000000u;
            }
        }
        auto epi = [&](const f32x16 (&c)[MH], int gh, int s, float ks_s, float L) {
            float acc[TH];
#pragma unroll
            for (int t = 0; t < TH; ++t)
                acc[t] = 0.0f;
#pragma unroll
            for (int m = 0; m < MH; ++m) {
                const int mt = gh * MH + m;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = (mt * 32 + 8 * (i >> 2)) / H - gh * TH;
                    acc[t] = fmaf(wr[mt][i], fabsf(c[m][i]), acc[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < TH; ++t)
                acc[t] = sum_halves(acc[t]);
            // writer of token gh*TH + t is the half t%2 (TH == 2) or half gh (TH == 1)
            const float a = (TH > 1 && half) ? acc[TH - 1] : acc[0];
            if constexpr (TH == 1) {
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((a + L) * qh[gh] * ks_s), srt[gh],
                                                      rowoff[gh] + 4u * (uint32_t)s, 0, 0);
            } else {
                const uint32_t off = s < lim[gh] ? rowoff[gh] + 4u * (uint32_t)s : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((a + L) * qh[gh] * ks_s), srs, off, 0, 0);
            }
        };
        f32x16 c0[MH], c1[MH];
        int s_prev = 0;
        float ks_prev = 0.0f, L_prev = 0.0f;
        issue(0, lane, pages(0, lane));
        issue(1, lane, pages(1, lane));
        Pg pg_next = pages(2, lane);
        // memory operations per wave: NL loads per tile, NST score stores per
        // tile iteration (one fewer in the first)
        constexpr int NL = NB + NS, NST = 2 * (LT / 32);
        for (int it = 0; it < ntiles; ++it) {
            // Tile it was issued two iterations back; since then came the next
            // tile's loads and the stores of up to two iterations, which may stay
            // in flight.
            if (it == 0)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");
            else if (it == 1)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL + NST - 1) : "memory");
            else if (it == 2)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NST - 1 + NL + NST) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NST + NL + NST) : "memory");
            __syncthreads();
            const int ln = opaque(lane);
            issue(it + 2, ln, pg_next);
            const int st = it % KST;
            const int t0 = kb0 + it * LT;
            // B operands of N-tile nt (the key rows and, with two tokens per
            // wave, the 16-key halves for the linear-term MFMAs), read from LDS
            // one N-tile ahead, under the previous N-tile's epilogue
            struct Bt {
                typename X::Op bop[NKS];
            };
            auto load_b = [&](int nt) {
                Bt b;
                const int r = nt * 32 + (ln & 31);
                const lds_u8 *brow = stage(st) + r * 128;
                const int f = (r >> 1) & 7, hf = ln >> 5;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int c = 2 * hf + 4 * ks;
                    const i32x4 lo = *(const __attribute__((address_space(3))) i32x4 *)(brow + 16 * (c ^ f));
                    const i32x4 hi = *(const __attribute__((address_space(3))) i32x4 *)(brow + 16 * ((c + 1) ^ f));
                    b.bop[ks] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
                return b;
            };
            auto load_bq = [&](int nt, int w2) {
                const int rq = nt * 32 + 16 * w2 + (ln & 15);
                const lds_u8 *bq = stage(st) + rq * 128;
                const int fq = (rq >> 1) & 7, c = 2 * (ln >> 4);
                const i32x4 lo = *(const __attribute__((address_space(3))) i32x4 *)(bq + 16 * (c ^ fq));
                const i32x4 hi = *(const __attribute__((address_space(3))) i32x4 *)(bq + 16 * ((c + 1) ^ fq));
                return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            };
            Bt cur = load_b(0);
#pragma unroll
            for (int nt = 0; nt < LT / 32; ++nt) {
                const int r = nt * 32 + (ln & 31);
                const typename X::Op *bop = cur.bop;
                const int s = t0 + r;
                const float ks_s = LKS[(st * kIdxWaves + wv) * LT + r];
                // linear term first, reduced to one value per lane right away
                float La = 0.0f, Lb = 0.0f;
                if constexpr (TPW == 2) {
                    // Two 16x16x128 MFMAs, keys 0-15 (P) and 16-31 (Q) of the
                    // N-tile.  Output lane l holds key l%16 and term rows
                    // 4*(l/16)..+3, so lane row g (16 lanes) holds token g/2's
                    // terms 4*(g%2)..+3.  After summing its 4 registers, a lane
                    // needs its partner l^16: v_permlane16_swap(P, Q) gives
                    // (P row0, Q row0, P row2, Q row2) and (P row1, Q row1, P row3,
                    // Q row3), whose sum is token g/2's linear term for key l%32,
                    // in the lanes that write it.
                    const i32x8 at = *(const i32x8 *)arow;
                    f32x4 pq[2];
#pragma unroll
                    for (int w2 = 0; w2 < 2; ++w2)
                        pq[w2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(at, load_bq(nt, w2), f32x4{}, 0,
                                                                                  0, 0, sal, 0, 127);
                    const float sp = (pq[0][0] + pq[0][1]) + (pq[0][2] + pq[0][3]);
                    const float sq = (pq[1][0] + pq[1][1]) + (pq[1][2] + pq[1][3]);
                    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(sp), __float_as_uint(sq), false, false);
                    La = __uint_as_float(x[0]) + __uint_as_float(x[1]);
                } else {
                    f32x16 cl = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        cl = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            *(const i32x8 *)(arow + ks * X::KS), bop[ks], cl, 0, 0, 0, sal, 0, 127);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        La += cl[i];
                        if (TPW == 4)
                            Lb += cl[8 + i];
                    }
                }
#pragma unroll
                for (int m = 0; m < MH; ++m) {
                    c0[m] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        c0[m] = mma32_fp8_plain(a[m][ks], bop[ks], c0[m]);
                }
                if (it > 0 || nt > 0)
                    epi(c1, 1, s_prev, ks_prev, L_prev);
#pragma unroll
                for (int m = 0; m < MH; ++m) {
                    c1[m] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        c1[m] = mma32_fp8_plain(a[MH + m][ks], bop[ks], c1[m]);
                }
                if (nt + 1 < LT / 32)
                    cur = load_b(nt + 1);
                epi(c0, 0, s, ks_s, La);
                if (nt == 0)
                    pg_next = pages(it + 3, ln);
                s_prev = s;
                ks_prev = ks_s;
                L_prev = TPW == 4 ? Lb : La;
            }
        }
        if (ntiles > 0)
            epi(c1, 1, s_prev, ks_prev, L_prev);
        // the ring's last two tiles were loaded past the end: drain them before
        // the workgroup's LDS is released
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }

    if constexpr (H >= 8 && MT % 2 == 0) {
        // Ping-pong over the two halves of the wave's M-tiles (G0 = first MT/2,
        // G1 = the rest; each holds whole tokens): the MFMAs of one half run
        // while the VALU epilogue of the other half (of this or the previous
        // 32-key N-tile) runs, with no extra accumulator registers.
        constexpr int MH = MT / 2, TH = TPW / 2;
        // Scores leave through a buffer resource over this wave's token rows; a
        // masked lane gets an offset past the end, which the hardware drops.
        // With no branch around the stores the compiler counts them exactly, and
        // the wait for the next tile's loads leaves this tile's stores in flight.
        const int wt0 = min(wv * TPW, ntok - 1);
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            scores + (int64_t)(tok0 + wt0) * ld, 0, (int)(TPW * ld * 4), 0x00020000);
        auto epi = [&](const f32x16 (&c)[MH], int gh, int s, float ks_s) {
            float acc[TH];
#pragma unroll
            for (int t = 0; t < TH; ++t)
                acc[t] = 0.0f;
#pragma unroll
            for (int m = 0; m < MH; ++m) {
                const int mt = gh * MH + m;
                if constexpr (F16E) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int t = (mt * 32 + 8 * (j >> 1)) / H - gh * TH;
                        acc[t] = relu_dot2(c[m][2 * j], c[m][2 * j + 1], wp[mt][j], acc[t]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = (mt * 32 + 8 * (i >> 2)) / H - gh * TH;
                        acc[t] = fmaf(wr[mt][i], fmaxf(c[m][i], 0.0f), acc[t]);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < TH; ++t)
                acc[t] = sum_halves(acc[t]);
            // one token per half: lanes of half 0 write it; two: half h writes token h
#pragma unroll
            for (int t0w = 0; t0w < TH; t0w += 2) {
                const int t1 = t0w + 1 < TH ? t0w + 1 : t0w;
                const int tw = t0w + (TH > 1 ? half : 0);
                const float v = (TH > 1 && half) ? acc[t1] * qs[gh * TH + t1] : acc[t0w] * qs[gh * TH + t0w];
                const int tl = wv * TPW + gh * TH + tw;
                const bool ok = (TH > 1 || half == 0) && tw < TH && tl < ntok && s <= pos0 + tl && s < kb1;
                const uint32_t off = ok ? (uint32_t)(((int64_t)(tl - wt0) * ld + s) * 4) : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v * ks_s), srs, off, 0, 0);
            }
        };
        f32x16 c0[MH], c1[MH];
        int s_prev = 0;
        float ks_prev = 0.0f;
        for (int it = 0; it < ntiles; ++it) {
            const int buf = it & 1;
            const int t0 = kb0 + it * kIdxTileKeys;
            if (it + 1 < ntiles)
                gload(t0 + kIdxTileKeys);
#pragma unroll
            for (int nt = 0; nt < kIdxTileKeys / 32; ++nt) {
                const uint8_t *brow = &lds_k[buf][(nt * 32 + col) * RBP + half * X::LB];
                typename X::Op bop[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    bop[ks] = X::load(brow + ks * X::KS * X::ELEM);
                const int s = t0 + nt * 32 + col;
                const float ks_s = FP8 ? lds_ks[buf][nt * 32 + col] : 1.0f;
#pragma unroll
                for (int m = 0; m < MH; ++m) {
                    c0[m] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        c0[m] = X::mma(a[m][ks], bop[ks], c0[m]);
                }
                if (it > 0 || nt > 0)
                    epi(c1, 1, s_prev, ks_prev);
#pragma unroll
                for (int m = 0; m < MH; ++m) {
                    c1[m] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        c1[m] = X::mma(a[MH + m][ks], bop[ks], c1[m]);
                }
                epi(c0, 0, s, ks_s);
                s_prev = s;
                ks_prev = ks_s;
            }
            if (it + 1 < ntiles)
                lstore(buf ^ 1);
            __syncthreads();
        }
        if (ntiles > 0)
            epi(c1, 1, s_prev, ks_prev);
        return;
    }

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
                for (int mt = 0; mt < MT; ++mt) {
                    if constexpr (F16E) {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            acc[(mt * 32 + 8 * (j >> 1)) / H] = relu_dot2(
                                c[mt][2 * j], c[mt][2 * j + 1], wp[mt][j], acc[(mt * 32 + 8 * (j >> 1)) / H]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            acc[(mt * 32 + 8 * (i >> 2)) / H] =
                                fmaf(wr[mt][i], fmaxf(c[mt][i], 0.0f), acc[(mt * 32 + 8 * (i >> 2)) / H]);
                    }
                }
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    acc[t] = sum_halves(acc[t]);
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

    constexpr bool F16E = IdxEpi<DT>::F16 && H >= 8;
    typename X::Op a[MT][NKS];
    float wr[MT][F16E ? 1 : 16];
    float wt[MT][F16E ? 16 : 1];
    f16x2 wp[MT][F16E ? 8 : 1];
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
            const float wv_ = ho < H ? w[(int64_t)tok * H + ho] : 0.0f;
            if constexpr (F16E)
                wt[mt][i] = wv_;
            else
                wr[mt][i] = wv_;
        }
    }
    // fp16 weights: scaled by the power of two that puts the token's largest
    // |w| in [2^14, 2^15), given back through the score scale (a lane half
    // holds every register's head of its half; the other half the rest)
    int wsh = 0;
    if constexpr (F16E) {
        float m = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                m = fmaxf(m, fabsf(wt[mt][i]));
        wsh = f16_weight_shift(fmaxf(m, __shfl_xor(m, 32, 64)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                wp[mt][i >> 1][i & 1] = (_Float16)ldexpf(wt[mt][i], wsh);
    }
    const float qs = ldexpf((FP8 ? q_scale[tok] : 1.0f) * IdxEpi<DT>::UNSCALE, -wsh);

    // Physical page of every page the chunk touches, staged once in LDS: a
    // key load then waits on an LDS read, not on a page-table load (a global
    // load would have to drain every key load issued before it).
    __shared__ int lpt[kIdxTokChunk / 16 + 2];
    const int pshift = bt.page_shift, pmask = (1 << pshift) - 1;
    const int pg0 = kb0 >> pshift;
    {
        const int npg = ((kb1 - 1) >> pshift) - pg0 + 1;
        for (int i = tid; i < npg; i += 256)
            lpt[i] = bt.page_table[(int64_t)b * bt.max_pages + pg0 + i];
    }
    __syncthreads();

    const int ntiles = (kb1 - kb0 + 31) / 32;
    // operand slots, software-pipelined; the loop is unrolled by the slot count
    // so every register array index is a compile-time constant.  Loads have no
    // branch: a key past the chunk rereads its last key (never stored), and a
    // tile past the end rereads the last tile, so the compiler's waits count
    // the loads in flight exactly.
    typename X::Op b0[NKS], b1[NKS], b2[NKS];
    float ks0 = 0.0f, ks1 = 0.0f, ks2 = 0.0f;
    auto gload = [&](typename X::Op (&bo)[NKS], float &ksv, int t) {
        const int s = min(kb0 + min(t, ntiles - 1) * 32 + col, kb1 - 1);
        const int64_t pr = ((int64_t)lpt[(s >> pshift) - pg0] << pshift) + (s & pmask);
        const uint8_t *src = k_idx + pr * RB + half * X::LB;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            bo[ks] = X::load(src + ks * X::KS * X::ELEM);
        ksv = FP8 ? k_scale[pr] : 1.0f;
    };
    // scores leave through a buffer resource over the token's score row
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)tok * ld, 0,
                                                                         (int)(ld * 4), 0x00020000);
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
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (F16E) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (mt * 32 + 8 * (j >> 1) < H)
                        acc = relu_dot2(c[mt][2 * j], c[mt][2 * j + 1], wp[mt][j], acc);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (mt * 32 + 8 * (i >> 2) < H)
                        acc = fmaf(wr[mt][i], fmaxf(c[mt][i], 0.0f), acc);
            }
        }
        acc = sum_halves(acc);
        // a masked lane (or a tile past the end) stores past the resource's end,
        // which the hardware drops
        const int s = kb0 + t * 32 + col;
        const uint32_t off = (half == 0 && s < kb1) ? (uint32_t)s * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc * qs * ksv), srs, off, 0, 0);
    };
    constexpr int W = kIdxWaves;
    int t = wv;
    if constexpr (FP8) {
        // fp8 (the long-context layout): three slots in flight
        gload(b0, ks0, t);
        gload(b1, ks1, t + W);
        for (; t < ntiles; t += 3 * W) {
            gload(b2, ks2, t + 2 * W);
            compute(b0, ks0, t);
            gload(b0, ks0, t + 3 * W);
            if (t + W < ntiles)
                compute(b1, ks1, t + W);
            gload(b1, ks1, t + 4 * W);
            if (t + 2 * W < ntiles)
                compute(b2, ks2, t + 2 * W);
        }
    } else {
        // two slots: the third costs a wave per SIMD of occupancy here
        gload(b0, ks0, t);
        for (; t < ntiles; t += 2 * W) {
            gload(b1, ks1, t + W);
            compute(b0, ks0, t);
            gload(b0, ks0, t + 2 * W);
            if (t + W < ntiles)
                compute(b1, ks1, t + W);
        }
    }
    // the last loads of the ring are never used: let them land before the wave ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Decode with 128-byte key rows (fp8 x 128, bf16 x 64, f32 x 32): the same
// work split and epilogue as indexer_token_kernel, but each wave gathers its
// 32-key tiles into its own LDS ring by direct loads that cover whole rows
// (8 rows x 128 bytes per load instruction) and reads the MFMA operands from
// there.  On gfx950 the address unit's cost grows with the cache lines one
// load instruction touches: loading the operand layout directly (32 keys x 32
// bytes per instruction) gathers about 2.5x slower.  The ring holds four
// tiles (three in flight); the loads are issued from asm with exact vmcnt
// waits, and keys past the chunk re-read its last key, so every tile issues
// the same loads.  Chunk c of row r sits at position c ^ ((r >> 1) & 7): the
// operand reads (32 rows of one chunk) hit distinct bank groups.
template <int DT, int H, int D>
__global__ __launch_bounds__(256) void indexer_token_lds_kernel(
    Batch bt, const uint8_t *__restrict__ q_idx, const float *__restrict__ q_scale,
    const float *__restrict__ w, const uint8_t *__restrict__ k_idx, const float *__restrict__ k_scale,
    float *__restrict__ scores, int64_t ld, int key_chunk)
{
    typedef IdxT<DT> X;
    constexpr int MT = (H + 31) / 32;
    constexpr int RB = D * X::ELEM;
    constexpr int NKS = D / X::KS;
    constexpr bool FP8 = DT == 2;
    constexpr int R = 4;                          // tiles in a wave's ring
    constexpr int TBY = 32 * RB;                  // bytes of one 32-key tile
    constexpr int NPT = TBY / 1024 + (FP8 ? 1 : 0);   // direct loads per tile per wave
    static_assert(RB == 128, "128-byte key rows");
    __shared__ __align__(16) uint8_t lkt[kIdxWaves * R * TBY];
    __shared__ float lks[kIdxWaves * R * 64];
    __shared__ int lpt[kIdxTokChunk / 16 + 2];

    const int tok = blockIdx.y;
    const int b = seq_of_token(bt, tok);
    const int pos = pos_of_token(bt, b, tok);
    const int kb0 = blockIdx.x * key_chunk;
    const int kb1 = min(kb0 + key_chunk, pos + 1);
    if (kb0 >= kb1)
        return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;

    constexpr bool F16E = IdxEpi<DT>::F16 && H >= 8;
    typename X::Op a[MT][NKS];
    float wr[MT][F16E ? 1 : 16];
    float wt[MT][F16E ? 16 : 1];
    f16x2 wp[MT][F16E ? 8 : 1];
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
            const float wv_ = ho < H ? w[(int64_t)tok * H + ho] : 0.0f;
            if constexpr (F16E)
                wt[mt][i] = wv_;
            else
                wr[mt][i] = wv_;
        }
    }
    int wsh = 0;
    if constexpr (F16E) {
        float m = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                m = fmaxf(m, fabsf(wt[mt][i]));
        wsh = f16_weight_shift(fmaxf(m, __shfl_xor(m, 32, 64)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                wp[mt][i >> 1][i & 1] = (_Float16)ldexpf(wt[mt][i], wsh);
    }
    const float qs = ldexpf((FP8 ? q_scale[tok] : 1.0f) * IdxEpi<DT>::UNSCALE, -wsh);

    const int pshift = bt.page_shift, pmask = (1 << pshift) - 1;
    const int pg0 = kb0 >> pshift;
    {
        const int npg = ((kb1 - 1) >> pshift) - pg0 + 1;
        for (int i = tid; i < npg; i += 256)
            lpt[i] = bt.page_table[(int64_t)b * bt.max_pages + pg0 + i];
    }
    __syncthreads();
    // the operand loads of the prologue land before the loop (their registers
    // are not waited on inside it, where the asm tile loads are in flight)
    __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0)

    // this wave's tiles: t = wv, wv + 4, ...; local tile m is global tile wv + 4m
    const int ntiles = (kb1 - kb0 + 31) / 32;
    const int nm = (ntiles - wv + kIdxWaves - 1) / kIdxWaves;
    lds_u8 *const ring = (lds_u8 *)lkt + wv * R * TBY;
    lds_u8 *const ksr = (lds_u8 *)lks + wv * R * 64 * 4;
    auto physical = [&](int s) -> int64_t {
        return ((int64_t)lpt[(s >> pshift) - pg0] << pshift) + (s & pmask);
    };
    auto issue = [&](int m, int ln) {
        const int t0 = kb0 + (wv + kIdxWaves * m) * 32;
        lds_u8 *dst = ring + (m % R) * TBY;
#pragma unroll
        for (int j = 0; j < TBY / 1024; ++j) {
            const int row = 8 * j + (ln >> 3);
            const int s = min(t0 + row, kb1 - 1);
            dma_b128(k_idx + physical(s) * RB + 16 * ((ln & 7) ^ ((row >> 1) & 7)), dst + j * 1024);
        }
        if constexpr (FP8) {
            const int s = min(t0 + (ln & 31), kb1 - 1);
            dma_b32(k_scale + physical(s), ksr + (m % R) * 256);
        }
    };
    // B operand of k-step ks: bytes ks*KS*ELEM + half*LB .. +LB of key row col
    const int f = (col >> 1) & 7;
    auto bload = [&](int m, typename X::Op (&bo)[NKS]) {
        const lds_u8 *row = ring + (m % R) * TBY + col * 128;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int by = ks * X::KS * X::ELEM + half * X::LB;
            if constexpr (X::LB == 32) {
                const int c = by >> 4;
                const i32x4 lo = *(const __attribute__((address_space(3))) i32x4 *)(row + 16 * (c ^ f));
                const i32x4 hi = *(const __attribute__((address_space(3))) i32x4 *)(row + 16 * ((c + 1) ^ f));
                bo[ks] = __builtin_bit_cast(typename X::Op, i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
            } else {
                const int c = by >> 4;
                bo[ks] = *(const __attribute__((address_space(3))) typename X::Op *)(row + 16 * (c ^ f) + (by & 15));
            }
        }
    };
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)tok * ld, 0,
                                                                         (int)(ld * 4), 0x00020000);
#pragma unroll
    for (int m = 0; m < R - 1; ++m)
        issue(m, lane);
    static_assert(R == 4, "wait counts below");
    for (int m = 0; m < nm; ++m) {
        // Tile m's loads were followed by those of tiles m+1 and m+2 and by the
        // score stores of the iterations since (vmcnt counts stores too): none
        // before iteration 1, then one, two, and from iteration 3 on three.
        if (m == 0)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NPT) : "memory");
        else if (m == 1)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NPT + 1) : "memory");
        else if (m == 2)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NPT + 2) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NPT + 3) : "memory");
        const int ln = opaque(lane);
        issue(m + R - 1, ln);           // into the buffer of tile m-1, read last iteration
        typename X::Op bo[NKS];
        bload(m, bo);
        const float ksv = FP8 ? *(const __attribute__((address_space(3))) float *)(ksr + (m % R) * 256 + 4 * col)
                              : 1.0f;
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
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (F16E) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (mt * 32 + 8 * (j >> 1) < H)
                        acc = relu_dot2(c[mt][2 * j], c[mt][2 * j + 1], wp[mt][j], acc);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (mt * 32 + 8 * (i >> 2) < H)
                        acc = fmaf(wr[mt][i], fmaxf(c[mt][i], 0.0f), acc);
            }
        }
        acc = sum_halves(acc);
        const int s = kb0 + (wv + kIdxWaves * m) * 32 + col;
        const uint32_t off = (half == 0 && s < kb1) ? (uint32_t)s * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc * qs * ksv), srs, off, 0, 0);
    }
    // the ring's last loads land before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------ launch
template <int DT, int H, int D>
static hipError_t launch_indexer_t(const Batch &bt, const void *q_idx, const float *q_scale, const float *w,
                                   const void *k_idx, const float *k_scale, float *scores, int64_t ld,
                                   hipStream_t st)
{
    if (bt.max_q >= 8) {
        constexpr int TQ = kIdxWaves * IdxShape<H>::TPW;
        // key chunks: a multiple of 8, since chunk c runs on XCD c % 8 (fewer
        // chunks would leave XCDs idle); short contexts give short chunks
        int n_chunks = 8 * ((bt.max_ctx + 8 * kIdxChunkTarget - 1) / (8 * kIdxChunkTarget));
        int key_chunk = (bt.max_ctx + n_chunks - 1) / n_chunks;
        key_chunk = (key_chunk + kIdxTileKeys - 1) / kIdxTileKeys * kIdxTileKeys;
        n_chunks = (bt.max_ctx + key_chunk - 1) / key_chunk;
        if (key_chunk > kIdxMaxChunk || ld * 4 * IdxShape<H>::TPW >= (1LL << 31))
            return hipErrorInvalidValue;
        const int n_tiles_max = (bt.total_q + TQ - 1) / TQ + bt.num_seqs - 1;
        const int cpx_max = (n_chunks + 7) / 8;
        const int64_t grid = 8LL * cpx_max * n_tiles_max;
        if (grid > 0x7fffffff)
            return hipErrorInvalidValue;
        // rotate the chunk -> XCD map when every chunk's keys fit in one L2 together
        const int64_t key_bytes = (int64_t)n_chunks * key_chunk * D * IdxT<DT>::ELEM;
        const int rotate = n_chunks % 8 == 0 && key_bytes <= (2 << 20);
        // Without rotation chunk c runs on XCD c % 8, and equal chunks of max_ctx keys
        // give the last one less causal work (its tokens stop at their own positions):
        // at 4096 new tokens on 131072 cached ones it has 88% of the others' pairs, and
        // its XCD idles for the rest.  Chunks sized on the mean causal limit of the
        // longest query run, with the last chunk open to each token's limit, even that
        // out, as long as the longer last chunk's pages fit the staged page table.
        int last_open = 0;
        if (!rotate && n_chunks % 8 == 0 && n_chunks > 1) {
            int kc = (bt.max_ctx - bt.max_q / 2 + n_chunks - 1) / n_chunks;
            kc = (kc + kIdxTileKeys - 1) / kIdxTileKeys * kIdxTileKeys;
            const int last_len = bt.max_ctx - (n_chunks - 1) * kc;
            if (kc < key_chunk && (last_len >> bt.page_shift) + 2 <= kIdxMaxChunk / 16 + 2) {
                key_chunk = kc;
                last_open = 1;
            }
        }
        hipLaunchKernelGGL((indexer_tile_kernel<DT, H, D>), dim3((unsigned)grid), dim3(256), 0, st, bt,
                           (const uint8_t *)q_idx, q_scale, w, (const uint8_t *)k_idx, k_scale, scores, ld,
                           key_chunk, n_chunks, n_tiles_max, rotate, last_open);
    } else {
        // enough workgroups to cover the GPU even for a handful of sequences
        int key_chunk = kIdxTokChunk;
        const int64_t want = 2048;
        while (key_chunk > 256 && (int64_t)bt.total_q * ((bt.max_ctx + key_chunk - 1) / key_chunk) < want)
            key_chunk >>= 1;
        const int n_chunks = (bt.max_ctx + key_chunk - 1) / key_chunk;
        if (bt.total_q > 65535 || ld * 4 >= (1LL << 31))
            return hipErrorInvalidValue;
        if constexpr (D * IdxT<DT>::ELEM == 128)
            hipLaunchKernelGGL((indexer_token_lds_kernel<DT, H, D>), dim3(n_chunks, bt.total_q), dim3(256), 0, st,
                               bt, (const uint8_t *)q_idx, q_scale, w, (const uint8_t *)k_idx, k_scale, scores, ld,
                               key_chunk);
        else
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
