// Backward of the gated sparse attention over fixed indices (gfx950).
//
// Pages (by title):
//   [HAT] "Hybrid Attention Architectures: Engineering Trade-offs from Linear
//          Attention to Gated Sparse Attention", §3.3: exact attention over
//          kv_history[idx], scaled by the gate.
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
// P comes back from the forward's log-sum-exp, D and dG from its output y, so
// no forward pass is repeated.
//
// One workgroup per token, all its heads, 32 keys per tile, bf16 MFMA
// (16x16x32) with fp32 accumulation.  Every operand of every contraction is
// kept in LDS in the layout that makes its MFMA fragment one 16-byte read:
// Q and dO row-major and transposed, the key tile row-major and transposed,
// P^T, dS and dS^T per tile.  dq accumulates in registers over the tiles; the
// tile's dK and dV (summed over the heads by the MFMA) are added to the fp32
// gradient rows with hardware float atomics, one per (token, key, element).
#include "launch.h"
#include "sa_device.h"

namespace sa {

constexpr int kBwdThreads = 256;
constexpr int kBwdTK = 32;              // keys per tile

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

template <int D, int H>
__global__ __launch_bounds__(kBwdThreads) void attn_bwd_kernel(
    Batch bt, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    int64_t rs, const int32_t *__restrict__ idx, int K, const uint16_t *__restrict__ gate, int per_channel,
    float scale, const uint16_t *__restrict__ y, const float *__restrict__ lse, const uint16_t *__restrict__ dy,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dvv, float *__restrict__ dgate)
{
    constexpr int HP = H < 32 ? 32 : H;     // heads padded to the MFMA k-step of the head contractions
    constexpr int DP = D + 8;               // padded rows (bank spread)
    constexpr int HPP = HP + 8;
    constexpr int TKP = kBwdTK + 8;
    __shared__ __align__(16) __bf16 Qs[H][DP];
    __shared__ __align__(16) __bf16 QT[D][HPP];
    __shared__ __align__(16) __bf16 dOs[H][DP];
    __shared__ __align__(16) __bf16 dOT[D][HPP];
    __shared__ __align__(16) __bf16 Ks[kBwdTK][DP];
    __shared__ __align__(16) __bf16 KT[D][TKP];
    __shared__ __align__(16) __bf16 Vs[kBwdTK][DP];
    __shared__ __align__(16) __bf16 PT[kBwdTK][HPP];
    __shared__ __align__(16) __bf16 dS[H][TKP];
    __shared__ __align__(16) __bf16 dST[kBwdTK][HPP];
    __shared__ float lse_s[H], Dh[H];
    __shared__ int64_t rows[kBwdTK];

    const int tok = blockIdx.x;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    const int b = seq_of_token(bt, tok);
    const int64_t row0 = phys_row(bt, b, 0);
    const int32_t *irow = idx + (int64_t)tok * K;

    // ---- per token: Q, dO = dy * g (both layouts), D_h = dy . y, the gate gradient
    for (int e = tid; e < H * D; e += kBwdThreads) {
        const int h = e / D, d = e % D;
        const __bf16 qv = __builtin_bit_cast(__bf16, q[((int64_t)tok * H + h) * D + d]);
        Qs[h][d] = qv;
        QT[d][h] = qv;
    }
    for (int e = tid; e < (HP - H) * D; e += kBwdThreads)
        QT[e % D][H + e / D] = (__bf16)0.0f;
    for (int h = wv; h < H; h += kBwdThreads / 64) {
        float dsum = 0.0f, gsum = 0.0f;
        for (int c = lane; c < D; c += 64) {
            const int64_t o = ((int64_t)tok * H + h) * D + c;
            const float G = bf16_bits_to_f32(per_channel ? gate[o] : gate[(int64_t)tok * H + h]);
            const float g = 1.0f / (1.0f + __expf(-G));
            const float dyc = bf16_bits_to_f32(dy[o]), yc = bf16_bits_to_f32(y[o]);
            const __bf16 dov = (__bf16)(dyc * g);
            dOs[h][c] = dov;
            dOT[c][h] = dov;
            dsum += dyc * yc;
            const float dg = dyc * yc * (1.0f - g);
            if (per_channel)
                dgate[o] = dg;
            else
                gsum += dg;
        }
        dsum = wave_sum(dsum);
        if (!per_channel)
            gsum = wave_sum(gsum);
        if (lane == 0) {
            Dh[h] = dsum;
            lse_s[h] = lse[(int64_t)tok * H + h];
            if (!per_channel)
                dgate[(int64_t)tok * H + h] = gsum;
        }
    }
    for (int e = tid; e < (HP - H) * D; e += kBwdThreads)
        dOT[e % D][H + e / D] = (__bf16)0.0f;
    for (int e = tid; e < kBwdTK * (HP - H); e += kBwdThreads) {
        PT[e / (HP - H)][H + e % (HP - H)] = (__bf16)0.0f;
        dST[e / (HP - H)][H + e % (HP - H)] = (__bf16)0.0f;
    }

    // dq tiles owned by this wave: (head tile, dim tile) pairs t = wv + 4u
    constexpr int NQT = (H / 16) * (D / 16);
    constexpr int QPW = (NQT + 3) / 4;
    f32x4 dqa[QPW];
#pragma unroll
    for (int u = 0; u < QPW; ++u)
        dqa[u] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (K + kBwdTK - 1) / kBwdTK;
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();                    // the previous tile's LDS is free
        // ---- gather the tile's K and V rows (invalid keys read row 0 and are masked)
        if (tid < kBwdTK) {
            const int j = t * kBwdTK + tid;
            const int s = j < K ? irow[j] : -1;
            rows[tid] = s >= 0 ? phys_row(bt, b, s) : -1;
        }
        __syncthreads();
        for (int e = tid; e < kBwdTK * (D / 8); e += kBwdThreads) {
            const int r = e / (D / 8), c8 = e % (D / 8);
            const int64_t pr = rows[r] >= 0 ? rows[r] : row0;
            const bf16x8 kv = *(const bf16x8 *)(kc + pr * rs + 8 * c8);
            const bf16x8 vv = *(const bf16x8 *)(vc + pr * rs + 8 * c8);
            *(lds_bf16x8_t *)&Ks[r][8 * c8] = kv;
            *(lds_bf16x8_t *)&Vs[r][8 * c8] = vv;
#pragma unroll
            for (int x = 0; x < 8; ++x)
                KT[8 * c8 + x][r] = kv[x];
        }
        __syncthreads();

        // ---- S = Q K^T and dP = dO V^T per (head tile, key tile); P, dS to LDS
        constexpr int NST = (H / 16) * 2;
        for (int st = wv; st < NST; st += 4) {
            const int m0 = 16 * (st >> 1), n0 = 16 * (st & 1);
            f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const int d0 = 32 * ks + 8 * grp;
                s = mma16_bf16(*(const lds_bf16x8_t *)&Qs[m0 + col][d0], *(const lds_bf16x8_t *)&Ks[n0 + col][d0], s);
                dp = mma16_bf16(*(const lds_bf16x8_t *)&dOs[m0 + col][d0], *(const lds_bf16x8_t *)&Vs[n0 + col][d0],
                                dp);
            }
            // lane: key n0 + col, heads m0 + 4 grp + i
            const int key = n0 + col;
            const bool valid = rows[key] >= 0;
            float pv[4], dsv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = m0 + 4 * grp + i;
                const float L = lse_s[h];
                const float p = (valid && L != -INFINITY) ? __expf(scale * s[i] - L) : 0.0f;
                pv[i] = p;
                dsv[i] = p * (dp[i] - Dh[h]) * scale;
                dS[h][key] = (__bf16)dsv[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                PT[key][m0 + 4 * grp + i] = (__bf16)pv[i];
                dST[key][m0 + 4 * grp + i] = (__bf16)dsv[i];
            }
        }
        __syncthreads();

        // ---- dq += dS K  (k-step: the tile's 32 keys)
#pragma unroll
        for (int u = 0; u < QPW; ++u) {
            const int qt = wv + 4 * u;
            if (qt < NQT) {
                const int m0 = 16 * (qt / (D / 16)), n0 = 16 * (qt % (D / 16));
                dqa[u] = mma16_bf16(*(const lds_bf16x8_t *)&dS[m0 + col][8 * grp],
                                    *(const lds_bf16x8_t *)&KT[n0 + col][8 * grp], dqa[u]);
            }
        }
        // ---- dK = dS^T Q and dV = P^T dO per (key tile, dim tile), added to the rows
        constexpr int NKT = 2 * (D / 16);
        for (int kt = wv; kt < NKT; kt += 4) {
            const int m0 = 16 * (kt / (D / 16)), n0 = 16 * (kt % (D / 16));
            f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < HP / 32; ++ks) {
                const int h0 = 32 * ks + 8 * grp;
                ak = mma16_bf16(*(const lds_bf16x8_t *)&dST[m0 + col][h0], *(const lds_bf16x8_t *)&QT[n0 + col][h0],
                                ak);
                av = mma16_bf16(*(const lds_bf16x8_t *)&PT[m0 + col][h0], *(const lds_bf16x8_t *)&dOT[n0 + col][h0],
                                av);
            }
            // lane: dim n0 + col, keys m0 + 4 grp + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t pr = rows[m0 + 4 * grp + i];
                if (pr >= 0) {
                    unsafeAtomicAdd(dk + pr * rs + n0 + col, ak[i]);
                    unsafeAtomicAdd(dvv + pr * rs + n0 + col, av[i]);
                }
            }
        }
    }
    // ---- dq out: lane holds dim n0 + col, heads m0 + 4 grp + i
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        const int qt = wv + 4 * u;
        if (qt < NQT) {
            const int m0 = 16 * (qt / (D / 16)), n0 = 16 * (qt % (D / 16));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dq[((int64_t)tok * H + m0 + 4 * grp + i) * D + n0 + col] = dqa[u][i];
        }
    }
}

int attn_bwd_supported(int dtype, int Hq, int d_qk, int d_v)
{
    return dtype == 1 && d_qk == d_v && (d_qk == 64 || d_qk == 128) && (Hq == 16 || Hq == 32 || Hq == 64);
}

hipError_t launch_attn_bwd(const Batch &bt, int Hq, int D, const void *q, const void *kc, const void *vc,
                           int64_t rs, const int32_t *idx, int K, const void *gate, int per_channel, float scale,
                           const void *y, const float *lse, const void *dy, float *dq, float *dk, float *dv,
                           float *dgate, hipStream_t st)
{
#define SA_BWD(DD, HH)                                                                                          \
    hipLaunchKernelGGL((attn_bwd_kernel<DD, HH>), dim3(bt.total_q), dim3(kBwdThreads), 0, st, bt,              \
                       (const uint16_t *)q, (const uint16_t *)kc, (const uint16_t *)vc, rs, idx, K,            \
                       (const uint16_t *)gate, per_channel, scale, (const uint16_t *)y, lse, (const uint16_t *)dy, \
                       dq, dk, dv, dgate)
    if (D == 64 && Hq == 16) SA_BWD(64, 16);
    else if (D == 64 && Hq == 32) SA_BWD(64, 32);
    else if (D == 64 && Hq == 64) SA_BWD(64, 64);
    else if (D == 128 && Hq == 16) SA_BWD(128, 16);
    else if (D == 128 && Hq == 32) SA_BWD(128, 32);
    else if (D == 128 && Hq == 64) SA_BWD(128, 64);
    else
        return hipErrorInvalidValue;
#undef SA_BWD
    return hipGetLastError();
}

} // namespace sa
