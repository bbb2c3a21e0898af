// Backward of the gated sparse attention over fixed indices (gfx950).
//
// Pages (by title):
//   [HAT] "Hybrid Attention Architectures: Engineering Trade-offs from Linear
//          Attention to Gated Sparse Attention", §3.2 (the gate as a
//          continuous path for the gradient) and §3.3 (exact attention over
//          kv_history[idx], scaled by the gate).
//   [F2S] "From Full Attention to Sparsity: The Evolution of Hybrid Attention
//          Architectures in Large Language Models", "Fine-Grained Sparse
//          Attention: Indexer Plus Top-K": the indices come from a Top-K, which
//          passes no gradient; the attention and the gate do.
//
// For token i, head h, over the valid entries s_j of idx[i, :] (forward:
// P_j = softmax(scale q.K_j), o = sum_j P_j V_j, y = o * g, g = sigmoid(G)):
//     dG = dy * y * (1 - g)      (= dy * o * g * (1 - g); summed over c per head)
//     do = dy * g,   D = do . o = dy . y,   dP_j = do . V_j,   dS_j = P_j (dP_j - D)
//     dq = scale * sum_j dS_j K_j,   dK[row(s_j)] += scale * dS_j q,   dV[row(s_j)] += P_j do
// P comes back from the forward's log-sum-exp and D from its output y, so no
// forward pass is repeated.  P, dS and do enter the MFMAs rounded to bf16;
// every sum is fp32.
//
// Kernels, in launch order:
//   attn_bwd_prep_kernel   per token: do (bf16), D, dG, and the transposed
//                          copies Q^T [d][h] and do^T [d][h] that the
//                          contractions over heads read.
//   attn_bwd_mask_kernel   per token (key-major layouts): the selected
//                          positions as a bitmap over the sequence, and a flag
//                          on every slot whose position an earlier slot of the
//                          row already holds.
//   attn_bwd_dq_kernel     per (token, head group), over the index list:
//                          S^T and dP^T again, P from lse, dS, and
//                          dq^T += K^T dS^T with K^T read by the LDS transpose
//                          load.  In scatter mode it also sums each slot's
//                          dK / dV over the group's heads and adds them to the
//                          cache rows with float atomics: every slot (latent
//                          layout) or only the flagged repeats.
//   attn_bwd_kv_kernel     (attn_bwd_kv.hip) key-major, per (sequence, 128 key positions,
//                          chunk of the sequence's tokens): each wave keeps
//                          32 keys' K and V operands in registers and their
//                          dK, dV in accumulators, and walks the chunk's
//                          tokens that selected any of the block's keys
//                          (their Q, do, Q^T, do^T staged in an LDS ring by
//                          direct loads).  One float atomic per (chunk, key,
//                          element) merges the chunks: about 1/16 of the
//                          per-slot scatter at the prefill shapes.
#include "launch.h"
#include "sa_device.h"

namespace sa {

constexpr float kBLog2e = 1.4426950408889634f;
constexpr int kBwdTK = 64;              // slots per LDS tile of the query-major kernel
constexpr int kBwdChunk = 1024;         // slots whose rows one pass resolves up front
constexpr int kPrepMaxH = 256;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_b;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_b;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2_b;

// ------------------------------------------------------------------ prep
// One workgroup per token.  Each thread takes runs of 8 channels of one head
// (16-byte loads and stores): do = bf16(dy g), the gate gradient, and D_h =
// dy . y, summed over the DV / 8 runs of a head (a power of two <= 64, on
// consecutive lanes) by a fixed xor-shuffle tree, so the sums do not depend on
// timing.  Q^T and do^T (read by the per-slot merge) go out through an LDS tile
// 32 columns at a time, for every row when trep is NULL, else only for rows
// whose index list repeats a position.
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(
    int H, int DQK, int DV, const uint16_t *__restrict__ q, const uint16_t *__restrict__ gate, int per_channel,
    const uint16_t *__restrict__ y, const uint16_t *__restrict__ dy, uint16_t *__restrict__ dO,
    uint16_t *__restrict__ QT, uint16_t *__restrict__ dOT, float *__restrict__ Dh, float *__restrict__ dgate,
    const uint8_t *__restrict__ trep)
{
    __shared__ uint16_t tile[kPrepMaxH][34];
    const int tok = blockIdx.x, tid = threadIdx.x;
    const int rph = DV >> 3;                // runs per head
    for (int r = tid; r < H * rph; r += 256) {
        const int h = r / rph, c0 = (r - h * rph) * 8;
        const int64_t o = ((int64_t)tok * H + h) * DV + c0;
        const u32x4 dyv = *(const u32x4 *)(dy + o), yv = *(const u32x4 *)(y + o);
        u32x4 gv;
        if (per_channel) {
            gv = *(const u32x4 *)(gate + o);
        } else {
            const uint32_t g1 = gate[(int64_t)tok * H + h];
            gv = u32x4{g1 | (g1 << 16), g1 | (g1 << 16), g1 | (g1 << 16), g1 | (g1 << 16)};
        }
        float ds = 0.0f, gs = 0.0f, dg[8];
        uint32_t ov[4];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int sh = 16 * (k & 1);
            const float dyc = bf16_bits_to_f32((uint16_t)(dyv[k >> 1] >> sh));
            const float yc = bf16_bits_to_f32((uint16_t)(yv[k >> 1] >> sh));
            const float g = 1.0f / (1.0f + __expf(-bf16_bits_to_f32((uint16_t)(gv[k >> 1] >> sh))));
            ds += dyc * yc;
            dg[k] = dyc * yc * (1.0f - g);
            gs += dg[k];
            const uint32_t b = f32_to_bf16_bits(dyc * g);
            ov[k >> 1] = (k & 1) ? (ov[k >> 1] | (b << 16)) : b;
        }
        *(u32x4 *)(dO + o) = u32x4{ov[0], ov[1], ov[2], ov[3]};
        if (per_channel) {
            *(f32x4 *)(dgate + o) = f32x4{dg[0], dg[1], dg[2], dg[3]};
            *(f32x4 *)(dgate + o + 4) = f32x4{dg[4], dg[5], dg[6], dg[7]};
        }
        // the head's runs are rph consecutive lanes, rph-aligned (64 % rph == 0)
        for (int m = rph >> 1; m >= 1; m >>= 1) {
            ds += __shfl_xor(ds, m, 64);
            gs += __shfl_xor(gs, m, 64);
        }
        if (c0 == 0) {
            Dh[(int64_t)tok * H + h] = ds;
            if (!per_channel)
                dgate[(int64_t)tok * H + h] = gs;
        }
    }
    if (trep != nullptr && trep[tok] == 0)
        return;
    const int cmax = DQK > DV ? DQK : DV;
    for (int c0 = 0; c0 < cmax; c0 += 32) {
        if (c0 < DQK) {
            for (int e = tid; e < H * 32; e += 256) {
                const int h = e >> 5, x = e & 31;
                tile[h][x] = c0 + x < DQK ? q[((int64_t)tok * H + h) * DQK + c0 + x] : (uint16_t)0;
            }
            __syncthreads();
            for (int e = tid; e < H * 32; e += 256) {
                const int x = e / H, h = e - x * H;
                if (c0 + x < DQK)
                    QT[((int64_t)tok * DQK + c0 + x) * H + h] = tile[h][x];
            }
            __syncthreads();
        }
        if (c0 < DV) {
            for (int e = tid; e < H * 32; e += 256) {
                const int h = e >> 5, x = e & 31, c = c0 + x;
                uint16_t v = 0;
                if (c < DV) {
                    const int64_t o = ((int64_t)tok * H + h) * DV + c;
                    const float G = bf16_bits_to_f32(per_channel ? gate[o] : gate[(int64_t)tok * H + h]);
                    const float g = 1.0f / (1.0f + __expf(-G));
                    v = f32_to_bf16_bits(bf16_bits_to_f32(dy[o]) * g);
                }
                tile[h][x] = v;
            }
            __syncthreads();
            for (int e = tid; e < H * 32; e += 256) {
                const int x = e / H, h = e - x * H;
                if (c0 + x < DV)
                    dOT[((int64_t)tok * DV + c0 + x) * H + h] = tile[h][x];
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------------ mask
// One workgroup per token: a cleared bitmap row gets one bit per valid slot.
// The slot whose atomic finds its bit already set repeats a position and is
// flagged (its contribution goes through the per-slot merge).  Rows of up to
// kMaskLdsWords words are built in LDS and written out whole; longer ones with
// global atomics.  trep[tok] tells whether the row flagged any slot, so that the
// pass merging the repeats skips the other rows at once.
constexpr int kMaskLdsWords = 8192;

__global__ __launch_bounds__(256) void attn_bwd_mask_kernel(const int32_t *__restrict__ idx, int K, int W,
                                                           int max_ctx, uint32_t *__restrict__ bits,
                                                           uint8_t *__restrict__ flags, uint8_t *__restrict__ trep)
{
    __shared__ uint32_t lb[kMaskLdsWords];
    const int tok = blockIdx.x;
    uint32_t *row = bits + (int64_t)tok * W;
    const bool in_lds = W <= kMaskLdsWords;
    for (int w = threadIdx.x; w < W; w += 256) {
        if (in_lds)
            lb[w] = 0u;
        else
            row[w] = 0u;
    }
    __syncthreads();            // (the barrier waits for the cleared words: only this workgroup touches the row)
    bool mine = false;
    for (int j = threadIdx.x; j < K; j += 256) {
        const int s = idx[(int64_t)tok * K + j];
        uint8_t rep = 0;
        if (s >= 0 && s < max_ctx) {
            const uint32_t bit = 1u << (s & 31);
            const uint32_t old = in_lds ? atomicOr(&lb[s >> 5], bit) : atomicOr(&row[s >> 5], bit);
            rep = (old & bit) ? 1 : 0;
        }
        mine = mine || rep;
        flags[(int64_t)tok * K + j] = rep;
    }
    const int any = __syncthreads_or(mine);     // also the barrier before an LDS row is written out
    if (threadIdx.x == 0)
        trep[tok] = any ? 1 : 0;
    if (in_lds) {
        for (int w = threadIdx.x; w < W; w += 256)
            row[w] = lb[w];
    }
}

// ------------------------------------------------------------------ dq
// One workgroup per (token, 16*NW heads), a wave per 16 heads, 64-slot tiles
// gathered by direct loads into two LDS buffers (the layout of the forward's
// kernel: 8-row blocks of 8 sixteen-byte chunks, chunks XOR-swizzled by row).
// Per 32-slot half tile on 16x16x32 bf16 MFMA: S^T = K Q^T and dP^T = V do^T
// (a lane owns one head's column, keys 4g..4g+3 and 16+4g..16+4g+3 in its
// registers), P = exp(scale S - lse), dS = P (dP - D), and dq^T += K^T dS^T
// with the K^T operand read by ds_read_b64_tr_b16 from the row-major tile, in
// the key order the registers hold.
__device__ __forceinline__ int bswz(int r) { return r & 7; }

template <int DQK, int DV, bool MLA, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(
    Batch bt, const uint16_t *__restrict__ q, int Hq, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, int64_t rs, const int32_t *__restrict__ idx, int K, float scale,
    const float *__restrict__ lse, const uint16_t *__restrict__ dO, const float *__restrict__ Dh,
    float *__restrict__ dq, int mode, const uint8_t *__restrict__ flags, const uint8_t *__restrict__ trep,
    const uint16_t *__restrict__ QT, const uint16_t *__restrict__ dOT, float *__restrict__ dk, float *__restrict__ dv)
{
    constexpr int NT = NW * 64;
    constexpr int NKQ = DQK / 32;           // k-steps over d_qk
    constexpr int NKV = DV / 32;            // k-steps over d_v
    constexpr int NMQ = DQK / 16;           // 16-dim tiles of dq
    constexpr int KCH = DQK / 8, VCH = DV / 8;
    constexpr int KCB = KCH / 8, VCB = VCH / 8;
    constexpr int VROWB = MLA ? KCB : VCB;
    constexpr int KCHUNKS = kBwdTK * KCH, VCHUNKS = MLA ? 0 : kBwdTK * VCH;
    constexpr int HW = 16 * NW;             // heads of the workgroup
    constexpr int HWP = HW < 32 ? 32 : HW;  // padded to the k-step of the head contraction
    constexpr int XS = HWP + 8;             // row of the scatter operands (bank spread)
    static_assert(DQK % 64 == 0 && DV % 32 == 0 && KCH % 8 == 0 && VCH % 8 == 0, "dims");
    static_assert(kBwdTK % (8 * NW) == 0, "whole 8-row groups per wave");
    __shared__ __align__(16) uint8_t lk0[KCHUNKS * 16];
    __shared__ __align__(16) uint8_t lk1[KCHUNKS * 16];
    __shared__ __align__(16) uint8_t lv0[(MLA ? 16 : VCHUNKS * 16)];
    __shared__ __align__(16) uint8_t lv1[(MLA ? 16 : VCHUNKS * 16)];
    __shared__ int32_t prow[kBwdChunk];
    __shared__ __align__(16) __bf16 xds[32][XS];     // scatter: scale*dS^T [key][head]
    __shared__ __align__(16) __bf16 xp[32][XS];      // scatter: P^T [key][head]
    __shared__ int32_t xrow[32];

    const int tok = blockIdx.x, hg = blockIdx.y;
    if (mode == 3 && trep[tok] == 0)
        return;                             // repeats only, and this row has none
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int hl = wv * 16 + n;             // head within the workgroup
    const int h = hg * HW + hl;
    const int b = seq_of_token(bt, tok);
    const int32_t *irow = idx + (int64_t)tok * K;
    const float sl2 = scale * kBLog2e;
    const float L = lse[(int64_t)tok * Hq + h];
    const bool live = L != -INFINITY;       // a head with no valid key has no gradient
    const float L2 = live ? L * kBLog2e : 0.0f;
    const float Dv = Dh[(int64_t)tok * Hq + h];

    bf16x8 qop[NKQ], dop[NKV];
    {
        const uint16_t *qp = q + ((int64_t)tok * Hq + h) * DQK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < NKQ; ++ks)
            qop[ks] = *(const bf16x8 *)(qp + 32 * ks);
        const uint16_t *dp = dO + ((int64_t)tok * Hq + h) * DV + 8 * g;
#pragma unroll
        for (int ks = 0; ks < NKV; ++ks)
            dop[ks] = *(const bf16x8 *)(dp + 32 * ks);
    }
    f32x4 dqa[NMQ];
#pragma unroll
    for (int mt = 0; mt < NMQ; ++mt)
        dqa[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (mode != 0) {
        for (int e = tid; e < 32 * XS; e += NT) {
            (&xds[0][0])[e] = (__bf16)0.0f;
            (&xp[0][0])[e] = (__bf16)0.0f;
        }
    }
    const int row0 = (int)phys_row(bt, b, 0);
    lds_u8 *const LK0 = (lds_u8 *)lk0, *const LK1 = (lds_u8 *)lk1;
    lds_u8 *const LV0 = (lds_u8 *)lv0, *const LV1 = (lds_u8 *)lv1;
    constexpr int RG = kBwdTK / 8;

    static_assert(kBwdChunk / kBwdTK <= 32, "a bit per tile of a pass");
    __shared__ uint32_t lfm;
    for (int c0 = 0; c0 < K; c0 += kBwdChunk) {
        const int nslots = min(kBwdChunk, K - c0);
        const int ntiles = (nslots + kBwdTK - 1) / kBwdTK;
        __syncthreads();                    // the previous chunk's rows and tiles are done with
        // the tiles this pass visits (bit t: tile t): all of them, or in mode 3 only
        // those holding a flagged repeat
        uint32_t fm = ntiles >= 32 ? 0xFFFFFFFFu : (1u << ntiles) - 1u;
        if (mode == 3) {
            uint32_t m = 0u;
            for (int j = tid; j < nslots; j += NT)
                if (flags[(int64_t)tok * K + c0 + j])
                    m |= 1u << (j / kBwdTK);
            if (tid == 0)
                lfm = 0u;
            __syncthreads();
            if (m)
                atomicOr(&lfm, m);
            __syncthreads();
            fm = lfm;
            if (fm == 0u)
                continue;
        }
        for (int j = tid; j < nslots; j += NT) {
            const int s = irow[c0 + j];
            prow[j] = s >= 0 ? (int)phys_row(bt, b, s) : -1 - row0;
        }
        __syncthreads();
        auto issue = [&](int t, lds_u8 *dk_, lds_u8 *dv_, int ln) {
#pragma unroll
            for (int rg = wv; rg < RG; rg += NW) {
                const int r = 8 * rg + (ln >> 3);
                const int slot = t * kBwdTK + r;
                int pr = prow[slot < nslots ? slot : 0];
                pr = pr >= 0 ? pr : -1 - pr;
                const int cpos = (ln & 7) ^ bswz(r);
                const uint16_t *ksrc = kc + (int64_t)pr * rs + cpos * 8;
#pragma unroll
                for (int cb = 0; cb < KCB; ++cb)
                    __builtin_amdgcn_global_load_lds(ksrc + cb * 64, (lds_void *)(dk_ + (rg * KCB + cb) * 1024), 16,
                                                     0, 0);
                if (!MLA) {
                    const uint16_t *vsrc = vc + (int64_t)pr * rs + cpos * 8;
#pragma unroll
                    for (int cb = 0; cb < VCB; ++cb)
                        __builtin_amdgcn_global_load_lds(vsrc + cb * 64, (lds_void *)(dv_ + (rg * VCB + cb) * 1024),
                                                         16, 0, 0);
                }
            }
        };
        const int nvisit = __popc(fm);
        int tcur = fm ? __builtin_ctz(fm) : 0;
        uint32_t rest = fm & (fm - 1u);
        if (nvisit > 0)
            issue(tcur, LK0, LV0, lane);
        for (int it = 0; it < nvisit; ++it) {
            const int t = tcur;
            const int tnext = rest ? __builtin_ctz(rest) : -1;
            tcur = tnext;
            rest &= rest - 1u;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            const bool odd = it & 1;
            const int ln = opaque(lane);
            const int myslot = t * kBwdTK + ln;
            const bool myvalid = myslot < nslots && prow[myslot < nslots ? myslot : 0] >= 0;
            const uint64_t vmask = __ballot(myvalid);
            // scatter this tile: every valid slot (mode 1) or the flagged repeats (modes 2
            // and 3); every wave forms the same mask
            bool sc_me = false;
            if (mode == 1)
                sc_me = myvalid;
            else if (mode >= 2 && myvalid)
                sc_me = flags[(int64_t)tok * K + c0 + myslot] != 0;
            const uint64_t scmask = __ballot(sc_me);
            const bool scatter = scmask != 0;
            lds_u8 *tk = odd ? LK1 : LK0;
            lds_u8 *tv = MLA ? tk : (odd ? LV1 : LV0);
            if (tnext >= 0) {
                if (odd)
                    issue(tnext, LK0, LV0, ln);
                else
                    issue(tnext, LK1, LV1, ln);
            }
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const int rb = 32 * kh;
                const int lk = lane;
                const int g_ = lk >> 4, n_ = lk & 15;
                // ---- S^T = K Q^T and dP^T = V do^T for keys rb..rb+15 (s0, p0) and rb+16..rb+31
                f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0, d0 = s0, d1 = s0;
                {
                    const int r0 = rb + n_, r1 = rb + 16 + n_;
                    lds_u8 *k0 = tk + (r0 >> 3) * KCB * 1024 + (r0 & 7) * 128;
                    lds_u8 *k1 = tk + (r1 >> 3) * KCB * 1024 + (r1 & 7) * 128;
                    lds_u8 *v0 = tv + (r0 >> 3) * VROWB * 1024 + (r0 & 7) * 128;
                    lds_u8 *v1 = tv + (r1 >> 3) * VROWB * 1024 + (r1 & 7) * 128;
                    auto lda = [&](lds_u8 *row, int r, int ks) {
                        return *(lds_bf16x8_b *)(row + 1024 * (ks >> 1) + 16 * ((4 * (ks & 1) + g_) ^ bswz(r)));
                    };
#pragma unroll
                    for (int ks = 0; ks < NKQ; ++ks) {
                        s0 = mma16_bf16(lda(k0, r0, ks), qop[ks], s0);
                        s1 = mma16_bf16(lda(k1, r1, ks), qop[ks], s1);
                    }
#pragma unroll
                    for (int ks = 0; ks < NKV; ++ks) {
                        d0 = mma16_bf16(lda(v0, r0, ks), dop[ks], d0);
                        d1 = mma16_bf16(lda(v1, r1, ks), dop[ks], d1);
                    }
                }
                // ---- P and dS for keys rb+4g+i (first four) and rb+16+4g+i
                float pv[8], dsv[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool va = live && ((vmask >> (rb + 4 * g_ + i)) & 1);
                    const bool vb = live && ((vmask >> (rb + 16 + 4 * g_ + i)) & 1);
                    pv[i] = va ? __builtin_amdgcn_exp2f(fmaf(s0[i], sl2, -L2)) : 0.0f;
                    pv[4 + i] = vb ? __builtin_amdgcn_exp2f(fmaf(s1[i], sl2, -L2)) : 0.0f;
                    dsv[i] = pv[i] * (d0[i] - Dv);
                    dsv[4 + i] = pv[4 + i] * (d1[i] - Dv);
                }
                bf16x8 dsop;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    dsop[i] = (__bf16)dsv[i];
                // ---- dq^T += K^T dS^T; the transpose load gives lane (dim i, group g)
                // the dims of keys rb+4g..+3 (first load) and rb+16+4g..+3 (second)
                {
                    const int jj = lk & 15;
                    const int ra_ = rb + 4 * g_ + (jj >> 2), rc_ = ra_ + 16;
                    const int cc = jj & 3, hh = cc >> 1;
                    const int fa = bswz(ra_), fc = bswz(rc_);
                    lds_u8 *ka = tk + (ra_ >> 3) * KCB * 1024 + (ra_ & 7) * 128 + (cc & 1) * 8;
                    lds_u8 *kb = tk + (rc_ >> 3) * KCB * 1024 + (rc_ & 7) * 128 + (cc & 1) * 8;
                    auto ldk = [&](lds_u8 *v, int f, int mt) {
                        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                            (lds_bf16x4_b *)(v + 1024 * (mt >> 2) + 16 * ((2 * (mt & 3) + hh) ^ f)));
                    };
#pragma unroll
                    for (int mt = 0; mt < NMQ; ++mt) {
                        const bf16x4 la = ldk(ka, fa, mt), lc = ldk(kb, fc, mt);
                        const bf16x8 kop = {la[0], la[1], la[2], la[3], lc[0], lc[1], lc[2], lc[3]};
                        dqa[mt] = mma16_bf16(kop, dsop, dqa[mt]);
                    }
                }
                // ---- scatter: sum each slot's dK, dV over the workgroup's heads
                if (scatter) {
                    // this half tile's rows and operands: P^T and scale*dS^T, zero where not scattered
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int kl = (i < 4 ? 4 * g_ + i : 16 + 4 * g_ + (i - 4));
                        const bool on = (scmask >> (rb + kl)) & 1;
                        xp[kl][hl] = (__bf16)(on ? pv[i] : 0.0f);
                        xds[kl][hl] = (__bf16)(on ? scale * dsv[i] : 0.0f);
                    }
                    if (tid < 32) {
                        const int slot = t * kBwdTK + rb + tid;
                        xrow[tid] = ((scmask >> (rb + tid)) & 1) ? prow[slot] : -1;
                    }
                    __syncthreads();
                    constexpr int NDQ = DQK / 16;
                    constexpr int HK = HWP / 32;
                    const uint16_t *qtr = QT + (int64_t)tok * DQK * Hq + hg * HW + 8 * g_;
                    const uint16_t *dotr = dOT + (int64_t)tok * DV * Hq + hg * HW + 8 * g_;
                    for (int dt = wv; dt < NDQ; dt += NW) {
                        const int d = 16 * dt + n_;
                        bf16x8 bq[HK], bo[HK];
#pragma unroll
                        for (int kk = 0; kk < HK; ++kk) {
                            const bool hv = 32 * kk + 8 * g_ < HW;
                            bq[kk] = hv ? *(const bf16x8 *)(qtr + (int64_t)d * Hq + 32 * kk) : bf16x8{};
                            bo[kk] = (hv && d < DV) ? *(const bf16x8 *)(dotr + (int64_t)d * Hq + 32 * kk) : bf16x8{};
                        }
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt) {
                            f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = ak;
#pragma unroll
                            for (int kk = 0; kk < HK; ++kk) {
                                const bf16x8 a1 = *(const lds_bf16x8_b *)&xds[16 * mt + n_][32 * kk + 8 * g_];
                                ak = mma16_bf16(a1, bq[kk], ak);
                                if (16 * dt < DV) {
                                    const bf16x8 a2 = *(const lds_bf16x8_b *)&xp[16 * mt + n_][32 * kk + 8 * g_];
                                    av = mma16_bf16(a2, bo[kk], av);
                                }
                            }
                            // lane: dim d, keys 16mt + 4g + i
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int pr = xrow[16 * mt + 4 * g_ + i];
                                if (pr >= 0) {
                                    if (MLA) {
                                        unsafeAtomicAdd(dk + (int64_t)pr * rs + d, ak[i] + av[i]);
                                    } else {
                                        unsafeAtomicAdd(dk + (int64_t)pr * rs + d, ak[i]);
                                        if (16 * dt < DV)
                                            unsafeAtomicAdd(dv + (int64_t)pr * rs + d, av[i]);
                                    }
                                }
                            }
                        }
                    }
                    __syncthreads();
                }
            }
        }
    }
    if (mode == 3)
        return;                             // d_q comes from attn_bwd_dq32_kernel
    // ---- dq out: lane holds head h, dims 16mt + 4g + i
    float *dqp = dq + ((int64_t)tok * Hq + h) * DQK + 4 * g;
#pragma unroll
    for (int mt = 0; mt < NMQ; ++mt)
        *(f32x4 *)(dqp + 16 * mt) = dqa[mt] * scale;
}

// ------------------------------------------------------------------ dq, 32 heads per wave
// d_qk = d_v = 128, a multiple of 32 query heads, lists of at most kDq32MaxK slots:
// one wave per (token, 32 heads), the four waves of a workgroup independent
// (consecutive tokens, no workgroup barrier), on 32x32x16 bf16 MFMA.  The gather
// is the forward MQA kernel's: each load instruction covers four whole rows, into
// VGPRs two tiles ahead (row offsets read one tile before that), then into the
// wave's LDS tiles, blocks of 8 rows x 8 sixteen-byte chunks at position
// (c & 7) ^ g(r).  Per 32-key tile:
//   - S^T = K Q^T and dP^T = V do^T, two interleaved chains of 8 MFMAs (asm, so
//     that their accumulators stay in VGPRs while dq^T holds AGPRs); a lane holds
//     one head's column, keys 8(i >> 2) + 4hq + (i & 3) in register i;
//   - P = 2^(S scale log2 e - lse log2 e), zero for slots outside the list, and
//     dS = P (dP - D);
//   - dq^T += K^T dS^T (8 MFMAs): K^T by transpose loads of the row-major K tile,
//     dS^T the lane's own registers, in the key order the loads deliver.
// d_q = scale dq^T leaves as whole 16-byte runs.  The flagged repeats' dK, dV are
// merged by attn_bwd_dq_kernel in its repeats-only mode.
constexpr int kDq32MaxK = 2048;

__device__ __forceinline__ int dq32_g(int r) { return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1); }

template <bool SHARED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_bwd_dq32_kernel(
    Batch bt, const uint16_t *__restrict__ q, int Hq, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, int64_t rs, const int32_t *__restrict__ idx, int K, float scale,
    const float *__restrict__ lse, const uint16_t *__restrict__ dO, const float *__restrict__ Dh,
    float *__restrict__ dq, int n_units)
{
    constexpr int D = 128;
    constexpr int NW = 4;
    constexpr int NKQ = D / 16;             // k-steps of the S^T and dP^T chains
    constexpr int NDT = D / 32;             // 32-dim tiles of dq^T
    constexpr int KCB = D / 64;             // 8-chunk blocks per row
    constexpr int TK = 32;                  // keys per tile
    constexpr int TB = TK * D * 2;          // bytes of one K (or V) tile in LDS
    constexpr int RPI = 64 / (D / 8);       // rows per load instruction
    constexpr int NI = TK / RPI;            // load instructions per tile and cache
    constexpr int NT = SHARED ? 1 : 2;      // LDS tiles per wave (K, V)
    constexpr int MAXT = kDq32MaxK / TK + 3;   // a list's tiles, two loaded past its end, one more read
    static_assert(RPI == 4, "four rows per load instruction");
    __shared__ __align__(16) uint8_t ltile[NW * NT * TB];
    __shared__ uint64_t loff[NW * MAXT * TK];  // byte offset of each slot's cache row
    __shared__ uint32_t lmask[NW * MAXT];     // valid slots of each tile, one bit per key

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int unit = blockIdx.x * NW + wv;
    if (unit >= n_units)
        return;
    const int HG = Hq >> 5;
    const int hg = unit % HG, tok = unit / HG;
    const int col = lane & 31, hq = lane >> 5;
    const int h = hg * 32 + col;
    const int b = seq_of_token(bt, tok);
    const int32_t *irow = idx + (int64_t)tok * K;
    lds_u8 *const tk = (lds_u8 *)ltile + wv * NT * TB;
    lds_u8 *const tv = SHARED ? tk : tk + TB;
    uint64_t *const off = loff + wv * MAXT * TK;
    uint32_t *const msk = lmask + wv * MAXT;

    // this lane's head: lse (a head with no valid key has lse = -inf and no gradient:
    // its terms are 2^-inf = 0) and D = dy . y
    const float L = lse[(int64_t)tok * Hq + h];
    const float L2 = L != -INFINITY ? L * kBLog2e : INFINITY;
    const float Dv = Dh[(int64_t)tok * Hq + h];
    const float sl2 = scale * kBLog2e;
    // B operands Q^T and do^T: head h, dims 16ks + 8hq .. +7
    bf16x8 qop[NKQ], dop[NKQ];
    {
        const uint16_t *qp = q + ((int64_t)tok * Hq + h) * D + 8 * hq;
        const uint16_t *dp = dO + ((int64_t)tok * Hq + h) * D + 8 * hq;
#pragma unroll
        for (int ks = 0; ks < NKQ; ++ks) {
            qop[ks] = *(const bf16x8 *)(qp + 16 * ks);
            dop[ks] = *(const bf16x8 *)(dp + 16 * ks);
        }
    }
    // every slot's index, then every page-table entry (two round trips); slots past
    // the list or holding -1 keep position 0's row (in bounds, masked)
    int ntiles = 0;
    {
        const uint64_t rsb = (uint64_t)rs * 2;
        const int64_t row0 = phys_row(bt, b, 0);
        constexpr int PS = kDq32MaxK / 64 + 2;
        int sv[PS];
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            const int j = lane + 64 * u;
            sv[u] = j < K ? irow[j] : -1;
        }
        int pg[PS];
#pragma unroll
        for (int u = 0; u < PS; ++u)
            pg[u] = bt.page_table[(int64_t)b * bt.max_pages + ((sv[u] >= 0 ? sv[u] : 0) >> bt.page_shift)];
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            const int j = lane + 64 * u;
            const int64_t pr = sv[u] >= 0 ? ((int64_t)pg[u] << bt.page_shift) + (sv[u] & ((1 << bt.page_shift) - 1))
                                          : row0;
            if (j < MAXT * TK)
                off[j] = (uint64_t)pr * rsb;
            const uint64_t vb = __ballot(sv[u] >= 0);
            const uint32_t lo = (uint32_t)vb, hi = (uint32_t)(vb >> 32);
            if (lo)
                ntiles = 2 * u + 1;
            if (hi)
                ntiles = 2 * u + 2;
            if (lane == 0 && 2 * u < MAXT) {
                msk[2 * u] = lo;
                if (2 * u + 1 < MAXT)
                    msk[2 * u + 1] = hi;
            }
        }
    }

    // ---- the gather: instruction i, lane l -> tile row RPI*i + l / (D/8), chunk l % (D/8)
    struct Stage {
        i32x4 k[NI];
        i32x4 v[SHARED ? 1 : NI];
    };
    struct Offs {
        uint64_t o[NI];
    };
    const int lrow = lane / (D / 8), lch = lane % (D / 8);
    const uint8_t *const kbase = (const uint8_t *)kc + 16 * lch;
    const uint8_t *const vbase = (const uint8_t *)vc + 16 * lch;
    auto read_offs = [&](int t) {
        Offs r;
        const uint64_t *o = off + t * TK + lrow;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            r.o[i] = o[RPI * i];
        return r;
    };
    auto load_stage = [&](const Offs &of) {
        Stage st;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            st.k[i] = *(const i32x4 *)(kbase + of.o[i]);
            if constexpr (!SHARED)
                st.v[i] = *(const i32x4 *)(vbase + of.o[i]);
        }
        return st;
    };
    // LDS position of chunk c of tile row r = RPI*i + lrow: block (i >> 1) * KCB + c / 8,
    // row 4(i & 1) + lrow of the block, position (c & 7) ^ g(r), g(r) = 4(lrow >> 1) + (i & 3)
    lds_u8 *wbase[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        wbase[c] = tk + (lch >> 3) * 1024 + lrow * 128 + 16 * (((lch & 7) ^ (4 * (lrow >> 1))) ^ c);
    auto put_stage = [&](const Stage &st) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int cst = (i >> 1) * KCB * 1024 + (i & 1) * 512;
            *(__attribute__((address_space(3))) i32x4 *)(wbase[i & 3] + cst) = st.k[i];
            if constexpr (!SHARED)
                *(__attribute__((address_space(3))) i32x4 *)(wbase[i & 3] + (tv - tk) + cst) = st.v[i];
        }
    };
    // A operands of the chains: row cl, chunk 2ks + hl of the K (or V) tile
    const int cl = lane & 31, hl = lane >> 5;
    lds_u8 *kb[4];
    {
        lds_u8 *krow = tk + (cl >> 3) * KCB * 1024 + (cl & 7) * 128;
        const int gh = hl ^ dq32_g(cl);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            kb[m] = krow + 16 * ((2 * m) ^ gh);
    }
    // K^T transpose-load bases (group G = lane / 16, i = lane % 16 reads row
    // 16j + 8sec + 4hl + (i >> 2), dims 32dt + 16(G & 1) + 4(i & 3) .. +3)
    lds_u8 *ktb[2][2];
    {
        const int G = lane >> 4, i16 = lane & 15;
        lds_u8 *trow = tk + (4 * hl + (i16 >> 2)) * 128 + 8 * (i16 & 1) + 16 * (((i16 & 3) >> 1) ^ hl);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int sc = 0; sc < 2; ++sc)
                ktb[a][sc] = trow + 64 * (a ^ ((i16 >> 3) & 1)) + 32 * ((G & 1) ^ sc);
    }
    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_q;

    f32x16 dqa[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        dqa[dt] = f32x16{};
    Stage s0 = load_stage(read_offs(0)), s1 = load_stage(read_offs(1));
    Offs on = read_offs(2);
    auto step = [&](int t, Stage &st) {
        put_stage(st);
        asm volatile("" ::: "memory");      // the tile's writes precede its reads
        st = load_stage(on);                // tile t + 2
        on = read_offs(t + 3);
        // ---- S^T = K Q^T and dP^T = V do^T, interleaved.  The compiler inserts no wait
        // states around asm, and with the register file full it copies operands back
        // from AGPRs (VALU writes) right before an MFMA: each MFMA is preceded by the
        // wait states such a write needs, and the last one followed by those a VALU
        // read of its result needs.
        f32x16 sa, pa;
        {
            constexpr int QD = 3;
            auto lda = [&](int ks) { return *(lds_bf16x8_q *)(kb[ks & 3] + 1024 * (ks >> 2)); };
            auto ldv = [&](int ks) { return *(lds_bf16x8_q *)(kb[ks & 3] + (tv - tk) + 1024 * (ks >> 2)); };
            bf16x8 ka[QD], va[QD];
#pragma unroll
            for (int d = 0; d < QD; ++d) {
                ka[d] = lda(d);
                if constexpr (!SHARED)
                    va[d] = ldv(d);
            }
#pragma unroll
            for (int ks = 0; ks < NKQ; ++ks) {
                const bf16x8 &kv = ka[ks % QD];
                const bf16x8 &vv = SHARED ? ka[ks % QD] : va[ks % QD];
                if (ks == 0) {
                    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sa) : "v"(kv), "v"(qop[ks]));
                    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(pa) : "v"(vv), "v"(dop[ks]));
                } else if (ks + 1 < NKQ) {
                    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sa) : "v"(kv), "v"(qop[ks]));
                    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(pa) : "v"(vv), "v"(dop[ks]));
                } else {
                    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sa) : "v"(kv), "v"(qop[ks]));
                    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
                                 "s_nop 7\n\ts_nop 7\n\ts_nop 3"
                                 : "+v"(pa) : "v"(vv), "v"(dop[ks]));
                }
                if (ks + QD < NKQ) {
                    ka[ks % QD] = lda(ks + QD);
                    if constexpr (!SHARED)
                        va[ks % QD] = ldv(ks + QD);
                }
            }
        }
        // ---- the first K^T operands, read before the dS terms whose VALU work
        // covers their LDS latency
        auto ldt = [&](int dt, int j, int sec) {
            return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4_b *)(ktb[dt & 1][sec] + (2 * j + sec) * KCB * 1024 + (dt >> 1) * 1024));
        };
        auto tstep = [](int u) { return 2 * (u % NDT) + u / NDT; };
        auto ldt8 = [&](int stp) {
            const bf16x4 lo = ldt(stp >> 1, stp & 1, 0), hi = ldt(stp >> 1, stp & 1, 1);
            return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        constexpr int PD = 4;
        bf16x8 kt[PD];
#pragma unroll
        for (int d = 0; d < PD; ++d)
            kt[d] = ldt8(tstep(d));
        // ---- P and dS for keys 8(i >> 2) + 4hq + (i & 3)
        const uint32_t vmask = __builtin_amdgcn_readfirstlane(msk[t]);
        bf16x8 dso[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool on_ = (vmask >> (8 * (i >> 2) + 4 * hq + (i & 3))) & 1u;
            const float p = on_ ? __builtin_amdgcn_exp2f(fmaf(sa[i], sl2, -L2)) : 0.0f;
            dso[i >> 3][i & 7] = (__bf16)(p * (pa[i] - Dv));
        }
        // ---- dq^T += K^T dS^T: step u covers dim tile u % NDT and k-half u / NDT
#pragma unroll
        for (int u = 0; u < 2 * NDT; ++u) {
            dqa[u % NDT] = mma32_bf16(kt[u % PD], dso[u / NDT], dqa[u % NDT]);
            if (u + PD < 2 * NDT)
                kt[u % PD] = ldt8(tstep(u + PD));
        }
        asm volatile("" ::: "memory");      // the tile's reads precede the next tile's writes
    };
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(t, s0);
        step(t + 1, s1);
    }
    if (t < ntiles)
        step(t, s0);
    // ---- d_q: lane holds head h, dims 32dt + 8g + 4hq + {0..3} of tile dt
    float *dqp = dq + ((int64_t)tok * Hq + h) * D + 4 * hq;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *(f32x4 *)(dqp + 32 * dt + 8 * g) =
                f32x4{dqa[dt][4 * g], dqa[dt][4 * g + 1], dqa[dt][4 * g + 2], dqa[dt][4 * g + 3]} * scale;
}

// ------------------------------------------------------------------ host side
static bool kv_shape(int Hq, int d_qk, int d_v)
{
    return d_qk == d_v && (d_qk == 64 || d_qk == 128) && (Hq == 16 || Hq == 32 || Hq == 64);
}

int attn_bwd_supported(int dtype, int Hq, int d_qk, int d_v)
{
    if (dtype != 1 || Hq < 16 || Hq % 16 || Hq > kPrepMaxH)
        return 0;
    return (d_qk == d_v && (d_qk == 64 || d_qk == 128)) || (d_qk == 576 && d_v == 512);
}

int attn_bwd_needs_shared(int d_qk, int d_v)
{
    return d_qk == 576 && d_v == 512;
}

struct BwdLayout {
    size_t dO, QT, dOT, Dh, bits, flags, trep, total;
    int W;
    bool km;
};

static size_t up256(size_t x) { return (x + 255) / 256 * 256; }

static BwdLayout bwd_layout(int T, int max_ctx, int Hq, int d_qk, int d_v, int K)
{
    BwdLayout L{};
    L.km = kv_shape(Hq, d_qk, d_v);
    L.W = (max_ctx + 31) / 32;
    size_t o = 0;
    L.dO = o;
    o += up256((size_t)T * Hq * d_v * 2);
    L.QT = o;
    o += up256((size_t)T * Hq * d_qk * 2);
    L.dOT = o;
    o += up256((size_t)T * Hq * d_v * 2);
    L.Dh = o;
    o += up256((size_t)T * Hq * 4);
    if (L.km) {
        L.bits = o;
        o += up256((size_t)T * L.W * 4);
        L.flags = o;
        o += up256((size_t)T * K);
        L.trep = o;
        o += up256((size_t)T);
    }
    L.total = o;
    return L;
}

size_t attn_bwd_ws_bytes(int T, int max_ctx, int Hq, int d_qk, int d_v, int K)
{
    return T > 0 ? bwd_layout(T, max_ctx, Hq, d_qk, d_v, K).total : 0;
}

static int bwd_waves(int Hq, int d_qk)
{
    const int cap = d_qk == 576 ? 4 : 8;
    for (int nw = cap; nw > 1; nw >>= 1)
        if (Hq % (16 * nw) == 0)
            return nw;
    return 1;
}

hipError_t launch_attn_bwd(const Batch &bt, int Hq, int d_qk, int d_v, const void *q, const void *kc,
                           const void *vc, int64_t rs, const int32_t *idx, int K, const void *gate, int per_channel,
                           float scale, const void *y, const float *lse, const void *dy, float *dq, float *dk,
                           float *dv, float *dgate, void *ws, hipStream_t st)
{
    const int T = bt.total_q;
    const BwdLayout L = bwd_layout(T, bt.max_ctx, Hq, d_qk, d_v, K);
    uint8_t *w = (uint8_t *)ws;
    uint16_t *dO = (uint16_t *)(w + L.dO), *QT = (uint16_t *)(w + L.QT), *dOT = (uint16_t *)(w + L.dOT);
    float *Dh = (float *)(w + L.Dh);
    uint32_t *bits = L.km ? (uint32_t *)(w + L.bits) : nullptr;
    uint8_t *flags = L.km ? (uint8_t *)(w + L.flags) : nullptr;
    uint8_t *trep = L.km ? (uint8_t *)(w + L.trep) : nullptr;
    const bool shared = kc == vc;

    // d_q on one wave per 32 heads where the shape allows; the query-major kernel then
    // only merges the flagged repeats' dK, dV (mode 3), and needs Q^T, do^T only for
    // the rows with repeats
    const bool dq32 = L.km && d_qk == 128 && d_v == 128 && Hq % 32 == 0 && K <= kDq32MaxK;
    if (L.km)
        hipLaunchKernelGGL(attn_bwd_mask_kernel, dim3(T), dim3(256), 0, st, idx, K, L.W, bt.max_ctx, bits, flags,
                           trep);
    hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3(T), dim3(256), 0, st, Hq, d_qk, d_v, (const uint16_t *)q,
                       (const uint16_t *)gate, per_channel, (const uint16_t *)y, (const uint16_t *)dy, dO, QT, dOT,
                       Dh, dgate, dq32 ? (const uint8_t *)trep : nullptr);
    if (dq32) {
        const int64_t units = (int64_t)T * (Hq / 32);
        if (units > 0x7fffffffLL)
            return hipErrorInvalidValue;
        const dim3 g32((unsigned)((units + 3) / 4));
        if (shared)
            hipLaunchKernelGGL((attn_bwd_dq32_kernel<true>), g32, dim3(256), 0, st, bt, (const uint16_t *)q, Hq,
                               (const uint16_t *)kc, (const uint16_t *)vc, rs, idx, K, scale, lse, dO, Dh, dq,
                               (int)units);
        else
            hipLaunchKernelGGL((attn_bwd_dq32_kernel<false>), g32, dim3(256), 0, st, bt, (const uint16_t *)q, Hq,
                               (const uint16_t *)kc, (const uint16_t *)vc, rs, idx, K, scale, lse, dO, Dh, dq,
                               (int)units);
    }
    const int nw = bwd_waves(Hq, d_qk);
    const int mode = L.km ? (dq32 ? 3 : 2) : 1;
    const dim3 grid(T, Hq / (16 * nw));
#define SA_DQ(DQ, DV_, MLA_, NW_)                                                                                 \
    hipLaunchKernelGGL((attn_bwd_dq_kernel<DQ, DV_, MLA_, NW_>), grid, dim3(NW_ * 64), 0, st, bt,                \
                       (const uint16_t *)q, Hq, (const uint16_t *)kc, (const uint16_t *)vc, rs, idx, K, scale, lse, \
                       dO, Dh, dq, mode, flags, trep, QT, dOT, dk, dv)
#define SA_DQ_NW(DQ, DV_, MLA_)                    \
    switch (nw) {                                  \
    case 8: SA_DQ(DQ, DV_, MLA_, 8); break;        \
    case 4: SA_DQ(DQ, DV_, MLA_, 4); break;        \
    case 2: SA_DQ(DQ, DV_, MLA_, 2); break;        \
    default: SA_DQ(DQ, DV_, MLA_, 1); break;       \
    }
    if (d_qk == 576) {
        switch (nw) {
        case 4: SA_DQ(576, 512, true, 4); break;
        case 2: SA_DQ(576, 512, true, 2); break;
        default: SA_DQ(576, 512, true, 1); break;
        }
    } else if (d_qk == 128 && shared) {
        SA_DQ_NW(128, 128, true)
    } else if (d_qk == 128) {
        SA_DQ_NW(128, 128, false)
    } else if (shared) {
        SA_DQ_NW(64, 64, true)
    } else {
        SA_DQ_NW(64, 64, false)
    }
#undef SA_DQ_NW
#undef SA_DQ
    if (L.km) {
        const hipError_t e = launch_attn_bwd_kv(bt, Hq, d_qk, shared, q, kc, vc, rs, scale, lse, dO, Dh, bits, L.W,
                                                dk, dv, st);
        if (e != hipSuccess)
            return e;
    }
    return hipGetLastError();
}

} // namespace sa
