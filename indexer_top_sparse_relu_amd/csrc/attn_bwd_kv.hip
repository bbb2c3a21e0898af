// Key-major dK, dV of the sparse attention backward: the kernel and its launch.
// Built on its own with MFMA accumulators in VGPRs (the compiler's S and dP
// chains then leave the AGPRs to the dK, dV accumulators, which the asm MFMAs
// below pin there), where the d_q kernels keep theirs in AGPRs.
//
// Pages: "Hybrid Attention Architectures: Engineering Trade-offs ..." §3.2 (the
// gate as a gradient path), §3.3; "From Full Attention to Sparsity ...",
// "Fine-Grained Sparse Attention: Indexer Plus Top-K" (the Top-K passes no
// gradient: only the attention over the fixed index lists is differentiated).
#include "launch.h"
#include "sa_device.h"

namespace sa {

constexpr float kBLog2e = 1.4426950408889634f;
constexpr int kKvKeys = 128;            // key positions per key-major workgroup
constexpr int kKvTokens = 256;          // tokens per key-major chunk

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_b;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_b;

// ------------------------------------------------------------------ dK, dV (key-major)
// Workgroup = (sequence b, key positions p0 .. p0+127, tokens t0 .. t0+255 of
// b); wave w owns keys p0+32w .. +31, their K and V operands in registers and
// their dK, dV in accumulators.  On 32x32x16 bf16 MFMA per token i that
// selected any of the block's keys:
//   S = Q_i K^T and dP = do_i V^T (heads x keys: a lane owns one key's column,
//   its registers the heads 8(r>>2) + 4(lane>>5) + (r&3));
//   P and scale*dS where the token selected the key;
//   dV += P^T do_i and dK += (scale dS)^T Q_i.  The head contraction takes the
//   registers in that order: lane (dim d, half) needs heads 16ks + 4half .. +3
//   and 16ks + 8 + 4half .. +3 of column d, which two LDS transpose loads read
//   straight from the row-major Q_i / do_i (no transposed copy is staged).
// Staged per token in an LDS ring by direct loads (1 KB each, spread over the
// waves): Q_i and do_i, rows of 16-byte chunks XOR-swizzled by row, and
// lse_i, D_i.
// dK / dV accumulation held in AGPRs.  Written as asm so that the loop-carried
// accumulators stay in the AGPR half of the register file: left to the compiler
// they live in VGPRs between tokens and are copied over before every MFMA.  The
// compiler does not insert wait states around asm, so each MFMA is preceded by
// enough for operands a VALU instruction (or an accumulator write) has just
// produced; the dependent MFMAs of one accumulator chain back to back (same
// opcode), and the caller pads the final reads of the accumulators.
__device__ __forceinline__ void mma32_acc_agpr(f32x16 &acc, const bf16x8 &a, const bf16x8 &b)
{
    asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <int D, int H>
struct KvShape {
    static constexpr int MT = H >= 32 ? H / 32 : 1;     // 32-head tiles of S
    static constexpr int QB = H * D * 2;                 // bytes of Q_i (and of do_i)
    static constexpr int SB = 2 * QB + 512;              // + lse and D (256 bytes each)
    static constexpr int R = 4 * SB <= 100 * 1024 ? 4 : (3 * SB <= 100 * 1024 ? 3 : 2);
    static constexpr int NPW = 2 * QB / 1024 / 4 + 1;   // direct loads per wave per token
};

template <int D, int H, bool SHARED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_bwd_kv_kernel(
    Batch bt, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    int64_t rs, float scale, const float *__restrict__ lse, const uint16_t *__restrict__ dO,
    const float *__restrict__ Dh, const uint32_t *__restrict__ bits, int W, int nkb, int ntc,
    float *__restrict__ dk, float *__restrict__ dv)
{
    typedef KvShape<D, H> S_;
    constexpr int MT = S_::MT, QB = S_::QB, SB = S_::SB, R = S_::R, NPW = S_::NPW;
    constexpr int KS = D / 16;              // k-steps over d
    constexpr int NTD = D / 32;             // 32-dim tiles of dK, dV
    constexpr int HKS = H / 16;             // k-steps over heads
    constexpr int RC = 2 * D / 16;          // 16-byte chunks per row of Q_i, do_i
    // Row r's logical chunk c sits at c ^ swz(r).  Two reads must hit distinct banks
    // (64 four-byte banks, 256 bytes per bank period, rows of 2D bytes):
    //   - a 128-bit operand read: 16 lanes, 16 consecutive rows (mod 16), one chunk;
    //   - a 64-bit transpose read: 32 lanes, rows 4m .. 4m+3 x chunks 4n .. 4n+3, each
    //     half a chunk.
    // d = 128 (one row per bank period): swz swaps the two 2-bit halves of r mod 16, so
    // that the 4 rows of a transpose read differ in position bits 2-3 and its 4 chunks in
    // bits 0-1.  d = 64 (two rows per period, told apart by r & 1): swz takes bit 1 of r
    // to position bit 2 and bits 2-3 of r to position bits 0-1.  (Plain c ^ (r mod 16)
    // put the 16 row-chunk pairs of a transpose read on 4 positions: 4-way conflicts.)
    static_assert(D == 64 || D == 128, "swizzle for 64 or 128 dims");
    auto swz = [](int r) {
        return D == 128 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    };
    constexpr int NB = 2 * QB / 1024;       // 1 KB loads per token
    static_assert(H % 16 == 0 && D % 32 == 0 && QB % 1024 == 0 && NB % 4 == 0 && RC <= 16, "shape");
    static_assert(kKvKeys == 32 * 4 && kKvKeys <= 256 && kKvTokens <= 256, "one wave per 32 keys, a thread per token");
    __shared__ __align__(16) uint8_t stage[R * SB];
    __shared__ int32_t ltok[kKvTokens];
    __shared__ uint32_t lwd[kKvTokens][kKvKeys / 32];
    __shared__ int32_t lrow[kKvKeys];
    __shared__ int32_t lcount[4];

    // Workgroup i runs on XCD i % 8.  A group is one (sequence, token chunk); its nkb
    // key blocks go to one XCD back to back, so the workgroups that XCD runs at
    // once stream the same tokens and share them through its L2.  Groups are dealt
    // to the XCDs in a snake order (0..7, 7..0, ...) to even out their work.
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int kg = j / nkb, kb = j - kg * nkb;
    const int grp = 8 * kg + ((kg & 1) ? 7 - xcd : xcd);
    if (grp >= bt.num_seqs * ntc)
        return;
    const int b = grp / ntc, tc = grp - b * ntc;
    const int ctx = bt.ctx_len[b];
    const int p0 = kb * kKvKeys;
    const int q0 = bt.q_start[b], nq = bt.q_start[b + 1] - q0;
    const int t0 = tc * kKvTokens;
    if (p0 >= ctx || t0 >= nq)
        return;
    const int t1 = min(nq, t0 + kKvTokens);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hf = lane >> 5;

    // ---- the chunk's tokens that selected any of the block's keys, in order
    {
        constexpr int NWD = kKvKeys / 32;
        const int t = t0 + tid;
        uint32_t wd[NWD];
        bool act = false;
#pragma unroll
        for (int w = 0; w < NWD; ++w) {
            wd[w] = 0u;
            if (tid < kKvTokens && t < t1 && (p0 >> 5) + w < W)
                wd[w] = bits[(int64_t)(q0 + t) * W + (p0 >> 5) + w];
            act |= wd[w] != 0u;
        }
        const uint64_t bal = __ballot(act);
        if (lane == 0)
            lcount[tid >> 6] = __popcll(bal);
        if (tid < kKvKeys) {
            const int p = p0 + tid;
            lrow[tid] = p < ctx ? (int)phys_row(bt, b, p) : -1;
        }
        __syncthreads();
        int base = 0;
        for (int w = 0; w < (tid >> 6); ++w)
            base += lcount[w];
        if (act) {
            const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
            ltok[pos] = q0 + t;
#pragma unroll
            for (int w = 0; w < NWD; ++w)
                lwd[pos][w] = wd[w];
        }
        __syncthreads();
    }
    const int nact = lcount[0] + lcount[1] + lcount[2] + lcount[3];
    if (nact == 0)
        return;

    // ---- this wave's keys: K and V operands (B of S and dP: key = lane & 31, dims 16kk + 8hf ..)
    bf16x8 kop[KS], vop[SHARED ? 1 : KS];
    {
        const int r = lrow[32 * wv + col];
        const int64_t pr = r >= 0 ? r : 0;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            kop[kk] = r >= 0 ? *(const bf16x8 *)(kc + pr * rs + 16 * kk + 8 * hf) : bf16x8{};
            if (!SHARED)
                vop[kk] = r >= 0 ? *(const bf16x8 *)(vc + pr * rs + 16 * kk + 8 * hf) : bf16x8{};
        }
    }
    f32x16 ak[NTD], av[NTD];
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt) {
        ak[nt] = f32x16{};
        av[nt] = f32x16{};
    }
    // the compiler does not count the asm loads: the operand loads above land first
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // ---- staging: token m's 1 KB blocks of Q_i and do_i go to ring slot m % R;
    // wave w issues blocks w, w+4, ... and one 256-byte load (wave 1: D, the
    // others lse; only wave 0's lse copy is read)
    auto issue = [&](int m, int ln) {
        const int tk = ltok[m < nact ? m : nact - 1];
        lds_u8 *dst = (lds_u8 *)stage + (m % R) * SB;
#pragma unroll
        for (int jb = 0; jb < NB / 4; ++jb) {
            const int kb_ = wv + 4 * jb;
            const int op = kb_ / (QB / 1024);                        // 0 Q, 1 do
            const int off = (kb_ % (QB / 1024)) * 1024 + 16 * ln;    // this lane's position in the operand
            const int r = off / (2 * D), p = (off % (2 * D)) / 16;
            const int c = p ^ swz(r);
            const uint16_t *src = (op == 0 ? q : dO) + (int64_t)tk * H * D + r * D + 8 * c;
            dma_b128(src, dst + kb_ * 1024);
        }
        const int hh = ln < H ? ln : 0;
        dma_b32((wv == 1 ? Dh : lse) + (int64_t)tk * H + hh, dst + 2 * QB + (wv == 1 ? 256 : 0));
    };
#pragma unroll
    for (int m = 0; m < R - 1; ++m)
        issue(m, lane);
    const float sl2 = scale * kBLog2e;
    const int G = lane >> 4, i16 = lane & 15;
    for (int m = 0; m < nact; ++m) {
        // token m's loads were followed by those of tokens m+1 .. m+R-2
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((R - 2) * NPW) : "memory");
        __syncthreads();
        const int ln = opaque(lane);
        issue(m + R - 1, ln);
        const uint32_t wd = lwd[m][wv];
        if (wd == 0u)
            continue;
        const lds_u8 *st = (const lds_u8 *)stage + (m % R) * SB;
        const lds_u8 *sQ = st, *sO = st + QB;
        const float *sL = (const float *)(st + 2 * QB), *sD = (const float *)(st + 2 * QB + 256);
        // ---- S and dP (heads x keys), then P and scale*dS packed as A operands of the
        // head contractions: k-step ks covers heads 16ks .. 16ks+15 in the register order
        // of head tile ks/2
        const bool sel = ((wd >> col) & 1u) != 0u;
        bf16x8 pa[HKS], da[HKS];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int hr = 32 * mt + col;                   // A row: head
            const bool hv = hr < H;
            const lds_u8 *qrow = sQ + (hv ? hr : 0) * 2 * D;
            const lds_u8 *orow = sO + (hv ? hr : 0) * 2 * D;
            // S and dP, two interleaved chains (this file is built with MFMA
            // accumulators in VGPRs, where the terms below read them, so dK and dV
            // keep the AGPRs to themselves); the A operands (rows of Q_i and do_i) are
            // read QD k-steps ahead
            constexpr int QD = 3;
            auto lda = [&](const lds_u8 *row, int kk) {
                const bf16x8 v = *(const lds_bf16x8_b *)(row + 16 * ((2 * kk + hf) ^ swz(hr)));
                return hv ? v : bf16x8{};
            };
            bf16x8 aq[QD], ao[QD];
#pragma unroll
            for (int d = 0; d < QD; ++d) {
                aq[d] = lda(qrow, d);
                ao[d] = lda(orow, d);
            }
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                s = mma32_bf16(aq[kk % QD], kop[kk], s);
                dp = mma32_bf16(ao[kk % QD], SHARED ? kop[kk] : vop[kk], dp);
                if (kk + QD < KS) {
                    aq[kk % QD] = lda(qrow, kk + QD);
                    ao[kk % QD] = lda(orow, kk + QD);
                }
            }
            // this lane's heads 32mt + 8jj + 4hf + (0..3): lse and D four at a time
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4 *)(sL + 32 * mt + 8 * jj + 4 * hf);
                const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4 *)(sD + 32 * mt + 8 * jj + 4 * hf);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int i = 4 * jj + qq;
                    const int hh = 32 * mt + mfma32_row(i, lane);
                    const bool on = sel && (H >= 32 || hh < H);
                    const float e = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -l4[qq] * kBLog2e));
                    const float p = on ? e : 0.0f;
                    const float ds = (scale * p) * (dp[i] - d4[qq]);
                    const int ks = 2 * mt + (i >> 3);
                    if (ks < HKS) {
                        pa[ks][i & 7] = (__bf16)p;
                        da[ks][i & 7] = (__bf16)ds;
                    }
                }
            }
        }
        // ---- dV += P^T do and dK += (scale dS)^T Q.  Transpose loads: the 16 lanes of
        // group G supply rows (heads) base + (i16 >> 2), dims blk + 4(i16 & 3) .. +3,
        // and each receives dim blk + i16 of the four heads.  The B operands of step
        // u = (nt, ks) are read one step ahead.
        const int hb = 4 * (G >> 1) + (i16 >> 2);
        auto ldb = [&](int u, bf16x8 &bq, bf16x8 &bo) {
            const int nt = u / HKS, ks = u % HKS;
            const int d0 = 32 * nt + 16 * (G & 1) + 4 * (i16 & 3);
            const int cd = d0 >> 3, cb = 2 * (d0 & 7);
            const int ra = 16 * ks + hb, rb2 = ra + 8;
            const lds_u8 *qa = sQ + ra * 2 * D + 16 * (cd ^ swz(ra)) + cb;
            const lds_u8 *qb = sQ + rb2 * 2 * D + 16 * (cd ^ swz(rb2)) + cb;
            const lds_u8 *oa = sO + ra * 2 * D + 16 * (cd ^ swz(ra)) + cb;
            const lds_u8 *ob = sO + rb2 * 2 * D + 16 * (cd ^ swz(rb2)) + cb;
            const bf16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b *)qa);
            const bf16x4 q2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b *)qb);
            const bf16x4 o1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b *)oa);
            const bf16x4 o2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_b *)ob);
            bq = bf16x8{q1[0], q1[1], q1[2], q1[3], q2[0], q2[1], q2[2], q2[3]};
            bo = bf16x8{o1[0], o1[1], o1[2], o1[3], o2[0], o2[1], o2[2], o2[3]};
        };
        constexpr int NU = NTD * HKS;
        bf16x8 nq, no;
        ldb(0, nq, no);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const bf16x8 bq = nq, bo = no;
            if (u + 1 < NU)
                ldb(u + 1, nq, no);
            mma32_acc_agpr(av[u / HKS], pa[u % HKS], bo);
            mma32_acc_agpr(ak[u / HKS], da[u % HKS], bq);
        }
    }
    // the ring's last loads land before the workgroup's LDS is released, and the
    // last MFMAs finish before their accumulators are read
    asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    // ---- merge into the gradient rows: lane holds dim 32nt + col, keys mfma32_row(i)
#pragma unroll
    for (int nt = 0; nt < NTD; ++nt) {
        const int d = 32 * nt + col;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = lrow[32 * wv + mfma32_row(i, lane)];
            if (r >= 0) {
                if (SHARED) {
                    unsafeAtomicAdd(dk + (int64_t)r * rs + d, ak[nt][i] + av[nt][i]);
                } else {
                    unsafeAtomicAdd(dk + (int64_t)r * rs + d, ak[nt][i]);
                    unsafeAtomicAdd(dv + (int64_t)r * rs + d, av[nt][i]);
                }
            }
        }
    }
}


hipError_t launch_attn_bwd_kv(const Batch &bt, int Hq, int d, bool shared, const void *q, const void *kc,
                              const void *vc, int64_t rs, float scale, const float *lse, const uint16_t *dO,
                              const float *Dh, const uint32_t *bits, int W, float *dk, float *dv, hipStream_t st)
{
    const int nkb = (bt.max_ctx + kKvKeys - 1) / kKvKeys;
    const int ntc = (bt.max_q + kKvTokens - 1) / kKvTokens;
    const int64_t items = 8LL * (((int64_t)bt.num_seqs * ntc + 7) / 8) * nkb;
    if (items > 0x7fffffff)
        return hipErrorInvalidValue;
    if (items == 0)
        return hipSuccess;
#define SA_KV(DD, HH, SH)                                                                                         \
    hipLaunchKernelGGL((attn_bwd_kv_kernel<DD, HH, SH>), dim3((unsigned)items), dim3(256), 0, st, bt,            \
                       (const uint16_t *)q, (const uint16_t *)kc, (const uint16_t *)vc, rs, scale, lse, dO, Dh,   \
                       bits, W, nkb, ntc, dk, dv)
#define SA_KV_H(DD, SH)                                    \
    if (Hq == 16) SA_KV(DD, 16, SH);                       \
    else if (Hq == 32) SA_KV(DD, 32, SH);                  \
    else SA_KV(DD, 64, SH);
    if (d == 128) {
        if (shared) { SA_KV_H(128, true) } else { SA_KV_H(128, false) }
    } else {
        if (shared) { SA_KV_H(64, true) } else { SA_KV_H(64, false) }
    }
#undef SA_KV_H
#undef SA_KV
    return hipGetLastError();
}

} // namespace sa
