// a3-a5 — gather, exact sparse attention and sigmoid output gate (gfx950).
//
// Pages (by title):
//   [HAT] "Hybrid Attention Architectures: Engineering Trade-offs from Linear
//          Attention to Gated Sparse Attention", §3.3: exact attention over
//          kv_history[idx], then the gate scales the output; §3.2: the gate is
//          a learnable scaling coefficient of the attention output.
//   [F2S] "From Full Attention to Sparsity: The Evolution of Hybrid Attention
//          Architectures in Large Language Models", "Fine-Grained Sparse
//          Attention: Indexer Plus Top-K", pseudocode: attention(q, gather(k,
//          idx), gather(v, idx)) and g = sigmoid(...).
//   [SEL] "Hybrid Attention Architecture Evolution in LLMs: From Full
//          Attention to Sparse Selection", §3.2: standard attention over the
//          selected set; §4.2: the gather itself costs memory traffic.
//   [SAD] "Sparse Attention and Hybrid Attention Architecture Design in Large
//          Language Models", §2 (query heads share a KV head; a latent row can
//          hold K and V) and §4 "Output gating" (per-channel or per-head).
//
// bf16 kernel.  A workgroup owns one token, a group of 16*NW query heads (16
// per wave) and a contiguous range of that token's index list.  Per 32-key
// tile it gathers the selected K rows through the page table into LDS
// (row-major) and V rows into LDS transposed (dim-major, keys in pairs per
// dword), then on 16x16x32 bf16 MFMA computes S^T = K Q^T (keys x heads, so a
// lane owns one head's column and the softmax is mostly in-lane), the online
// softmax in fp32, and O^T += V^T P^T.  The K-tile operand order inside a lane
// (keys 4g..4g+3 of the first 16, then of the second 16) is matched by the V^T
// operand, so P feeds the second MFMA straight from registers.  The epilogue
// divides by the softmax sum, multiplies by sigmoid(gate) and rounds to bf16;
// with a split index list it writes (O, max, sum) partials that a combine
// kernel merges by log-sum-exp.
#include "sa_device.h"
#include "launch.h"

namespace sa {

constexpr int kTK = 32;                 // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DQK, int DV, bool MLA, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(
    Batch bt, const uint16_t *__restrict__ q, int Hq, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, int64_t rs, const int32_t *__restrict__ idx, int K,
    const uint16_t *__restrict__ gate, int per_channel, float scale_log2, uint16_t *__restrict__ out,
    float *__restrict__ lse, float *__restrict__ part, int n_split, int split_len)
{
    constexpr int NT = NW * 64;
    constexpr int NKQ = DQK / 32;           // MFMA steps over d_qk
    constexpr int NMO = DV / 16;            // 16-dim tiles of O
    constexpr int KROW = DQK + 8;           // padded K row in LDS (bf16)
    constexpr int VROW = kTK + 4;           // padded V^T row in LDS (bf16)
    constexpr int KCH = DQK / 8;            // 16-byte chunks per K row
    constexpr int VCH = DV / 8;             // 16-byte chunks per V row
    static_assert(DQK % 32 == 0 && DV % 16 == 0, "dims");
    __shared__ __align__(16) uint16_t lk[kTK * KROW];
    __shared__ __align__(16) uint16_t lv[DV * VROW];
    __shared__ int64_t lrow[kTK];           // physical rows of the tile (-1: empty slot)

    const int tok = blockIdx.x;
    const int hg = blockIdx.y;               // head group
    const int sp = blockIdx.z;               // split of the index list
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int h = hg * (16 * NW) + wv * 16 + n;   // this lane's head (column of S^T and O^T)
    const int b = seq_of_token(bt, tok);
    const int j0 = sp * split_len;
    const int j1 = min(K, j0 + split_len);
    const int32_t *irow = idx + (int64_t)tok * K;

    // Q^T operand: head h, dims 32*ks + 8*g .. +7
    bf16x8 qop[NKQ];
    {
        const uint16_t *qp = q + ((int64_t)tok * Hq + h) * DQK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < NKQ; ++ks)
            qop[ks] = *(const bf16x8 *)(qp + 32 * ks);
    }
    f32x4 o[NMO];
#pragma unroll
    for (int mt = 0; mt < NMO; ++mt)
        o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    // gather tasks: (key pair, 16-byte chunk); K chunks first, then separate V chunks
    constexpr int KT = (kTK / 2) * KCH;
    constexpr int VT = MLA ? 0 : (kTK / 2) * VCH;
    constexpr int TASKS = (KT + VT + NT - 1) / NT;

    for (int t0 = j0; t0 < j1; t0 += kTK) {
        if (tid < kTK) {
            const int j = t0 + tid;
            const int s = j < j1 ? irow[j] : -1;
            lrow[tid] = s >= 0 ? phys_row(bt, b, s) : -1;
        }
        __syncthreads();
        // ---- gather the tile into LDS
#pragma unroll
        for (int u = 0; u < TASKS; ++u) {
            const int e = tid + u * NT;
            if (e < KT + VT) {
                const bool isk = e < KT;
                const int e2 = isk ? e : e - KT;
                const int nch = isk ? KCH : VCH;
                const int kp = e2 / nch, ch = e2 % nch;
                const int64_t r0 = lrow[2 * kp], r1 = lrow[2 * kp + 1];
                const uint16_t *base = isk ? kc : vc;
                i32x4 x0 = i32x4{0, 0, 0, 0}, x1 = i32x4{0, 0, 0, 0};
                if (r0 >= 0)
                    x0 = *(const i32x4 *)(base + r0 * rs + ch * 8);
                if (r1 >= 0)
                    x1 = *(const i32x4 *)(base + r1 * rs + ch * 8);
                if (isk) {
                    *(i32x4 *)(&lk[(2 * kp) * KROW + ch * 8]) = x0;
                    *(i32x4 *)(&lk[(2 * kp + 1) * KROW + ch * 8]) = x1;
                }
                if ((MLA && isk && ch < VCH) || !isk) {
                    // V^T: dword (V[2kp][d], V[2kp+1][d]) at lv[d][2kp]
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2) {
                        const uint32_t a = (uint32_t)x0[q2], c = (uint32_t)x1[q2];
                        const int d = ch * 8 + 2 * q2;
                        *(uint32_t *)(&lv[d * VROW + 2 * kp]) = (a & 0xFFFFu) | (c << 16);
                        *(uint32_t *)(&lv[(d + 1) * VROW + 2 * kp]) = (a >> 16) | (c & 0xFFFF0000u);
                    }
                }
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T for keys 0-15 and 16-31 of the tile
        f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
        {
            const uint16_t *k0 = &lk[n * KROW + 8 * g];
            const uint16_t *k1 = &lk[(16 + n) * KROW + 8 * g];
#pragma unroll
            for (int ks = 0; ks < NKQ; ++ks) {
                s0 = mma16_bf16(*(const bf16x8 *)(k0 + 32 * ks), qop[ks], s0);
                s1 = mma16_bf16(*(const bf16x8 *)(k1 + 32 * ks), qop[ks], s1);
            }
        }
        // lane holds keys 4g+i (s0) and 16+4g+i (s1) of head h
        float z[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = lrow[4 * g + i] >= 0 ? s0[i] * scale_log2 : -INFINITY;
            z[4 + i] = lrow[16 + 4 * g + i] >= 0 ? s1[i] * scale_log2 : -INFINITY;
        }
        float mt_ = z[0];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            mt_ = fmaxf(mt_, z[i]);
        mt_ = fmaxf(mt_, shfl_xor(mt_, 16));
        mt_ = fmaxf(mt_, shfl_xor(mt_, 32));
        const float m_new = fmaxf(m_run, mt_);
        const float base = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = exp2f(m_run - base);          // 0 when m_run = -inf
        float p[8], psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = exp2f(z[i] - base);
            psum += p[i];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        bf16x8 pop;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            pop[i] = (__bf16)p[i];
        // ---- O^T = alpha O^T + V^T P^T
        {
            const uint16_t *vp = &lv[n * VROW + 4 * g];
#pragma unroll
            for (int mt = 0; mt < NMO; ++mt) {
                const uint16_t *vr = vp + (16 * mt) * VROW;
                const bf16x4 lo4 = *(const bf16x4 *)(vr);
                const bf16x4 hi4 = *(const bf16x4 *)(vr + 16);
                bf16x8 vop;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vop[i] = lo4[i];
                    vop[4 + i] = hi4[i];
                }
                o[mt] *= alpha;
                o[mt] = mma16_bf16(vop, pop, o[mt]);
            }
        }
        __syncthreads();
    }

    // ---- epilogue
    float l_tot = l_run;
    l_tot += shfl_xor(l_tot, 16);
    l_tot += shfl_xor(l_tot, 32);
    if (n_split == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        float gh = 0.0f;
        if (!per_channel)
            gh = sigmoidf_(bf16_bits_to_f32(gate[(int64_t)tok * Hq + h]));
        uint16_t *op = out + ((int64_t)tok * Hq + h) * DV + 4 * g;
        const uint16_t *gp = gate + ((int64_t)tok * Hq + h) * DV + 4 * g;
#pragma unroll
        for (int mt = 0; mt < NMO; ++mt) {
            uint16_t r[4];
            uint2 gv = per_channel ? *(const uint2 *)(gp + 16 * mt) : uint2{0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t gw = i < 2 ? gv.x : gv.y;
                const float gi = per_channel ? sigmoidf_(bf16_bits_to_f32((uint16_t)(gw >> (16 * (i & 1))))) : gh;
                r[i] = f32_to_bf16_bits(o[mt][i] * inv * gi);
            }
            *(uint2 *)(op + 16 * mt) = uint2{(uint32_t)r[0] | ((uint32_t)r[1] << 16),
                                            (uint32_t)r[2] | ((uint32_t)r[3] << 16)};
        }
        if (lse && g == 0)
            lse[(int64_t)tok * Hq + h] = l_tot > 0.0f ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
    } else {
        // partial: [tok][split][head] x (DV values, max (log2 units), sum, 2 pad)
        float *pp = part + (((int64_t)tok * n_split + sp) * Hq + h) * (DV + 4);
#pragma unroll
        for (int mt = 0; mt < NMO; ++mt)
            *(f32x4 *)(pp + 16 * mt + 4 * g) = o[mt];
        if (g == 0) {
            pp[DV] = m_run;
            pp[DV + 1] = l_tot;
        }
    }
}

// Merge split partials by log-sum-exp, then gate; one block per (token, head).
__global__ __launch_bounds__(128) void attn_combine_kernel(int Hq, int DV, int n_split, const float *__restrict__ part,
                                                          const void *__restrict__ gate, int per_channel, int is_bf16,
                                                          void *__restrict__ out, float *__restrict__ lse)
{
    const int tok = blockIdx.x, h = blockIdx.y;
    const float *pp = part + ((int64_t)tok * n_split * Hq + h) * (DV + 4);
    const int64_t sstride = (int64_t)Hq * (DV + 4);
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s)
        M = fmaxf(M, pp[s * sstride + DV]);
    const float base = M == -INFINITY ? 0.0f : M;
    float L = 0.0f;
    for (int s = 0; s < n_split; ++s)
        L += pp[s * sstride + DV + 1] * exp2f(pp[s * sstride + DV] - base);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int64_t ob = ((int64_t)tok * Hq + h) * DV;
    for (int c = threadIdx.x; c < DV; c += blockDim.x) {
        float acc = 0.0f;
        for (int s = 0; s < n_split; ++s)
            acc += pp[s * sstride + c] * exp2f(pp[s * sstride + DV] - base);
        float gl;
        const int64_t gi = per_channel ? ob + c : (int64_t)tok * Hq + h;
        if (is_bf16)
            gl = bf16_bits_to_f32(((const uint16_t *)gate)[gi]);
        else
            gl = ((const float *)gate)[gi];
        const float y = acc * inv * sigmoidf_(gl);
        if (is_bf16)
            ((uint16_t *)out)[ob + c] = f32_to_bf16_bits(y);
        else
            ((float *)out)[ob + c] = y;
    }
    if (lse && threadIdx.x == 0)
        lse[(int64_t)tok * Hq + h] = L > 0.0f ? M * kLn2 + __logf(L) : -INFINITY;
}

// fp32 path: one wave per (token, head); 64 index slots per step, one slot per
// lane for the logits, then the lanes own output dims for P V.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(Batch bt, const float *__restrict__ q, int Hq,
                                                      const float *__restrict__ kc, const float *__restrict__ vc,
                                                      int64_t rs, const int32_t *__restrict__ idx, int K,
                                                      const float *__restrict__ gate, int per_channel,
                                                      float scale_log2, float *__restrict__ out,
                                                      float *__restrict__ lse, float *__restrict__ part,
                                                      int n_split, int split_len)
{
    constexpr int PER = (D + 63) / 64;
    const int tok = blockIdx.x, h = blockIdx.y, sp = blockIdx.z, lane = threadIdx.x;
    const int b = seq_of_token(bt, tok);
    const int j0 = sp * split_len, j1 = min(K, j0 + split_len);
    const float *qp = q + ((int64_t)tok * Hq + h) * D;
    float o[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u)
        o[u] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    for (int t0 = j0; t0 < j1; t0 += 64) {
        const int j = t0 + lane;
        const int s = j < j1 ? idx[(int64_t)tok * K + j] : -1;
        const int64_t r = s >= 0 ? phys_row(bt, b, s) : -1;
        float z = -INFINITY;
        if (r >= 0) {
            float dot = 0.0f;
            const float *kp = kc + r * rs;
            for (int d = 0; d < D; ++d)
                dot = fmaf(qp[d], kp[d], dot);
            z = dot * scale_log2;
        }
        const float m_new = fmaxf(m_run, wave_max(z));
        const float base = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = exp2f(m_run - base);
        const float p = exp2f(z - base);
        l_run = l_run * alpha + wave_sum(p);
        m_run = m_new;
#pragma unroll
        for (int u = 0; u < PER; ++u)
            o[u] *= alpha;
        for (int jj = 0; jj < 64; ++jj) {
            const float pj = __shfl(p, jj, 64);
            const int64_t rj = __shfl(r, jj, 64);
            if (rj >= 0) {
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int c = lane + 64 * u;
                    if (c < D)
                        o[u] = fmaf(pj, vc[rj * rs + c], o[u]);
                }
            }
        }
    }
    if (n_split == 1) {
        const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = lane + 64 * u;
            if (c < D) {
                const float gl = per_channel ? gate[((int64_t)tok * Hq + h) * D + c] : gate[(int64_t)tok * Hq + h];
                out[((int64_t)tok * Hq + h) * D + c] = o[u] * inv * sigmoidf_(gl);
            }
        }
        if (lse && lane == 0)
            lse[(int64_t)tok * Hq + h] = l_run > 0.0f ? m_run * kLn2 + __logf(l_run) : -INFINITY;
    } else {
        float *pp = part + (((int64_t)tok * n_split + sp) * Hq + h) * (D + 4);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = lane + 64 * u;
            if (c < D)
                pp[c] = o[u];
        }
        if (lane == 0) {
            pp[D] = m_run;
            pp[D + 1] = l_run;
        }
    }
}

// ------------------------------------------------------------------ launch
static int bf16_waves(int Hq)
{
    const int g16 = Hq / 16;
    for (int nw = 8; nw >= 1; nw >>= 1)
        if (g16 % nw == 0)
            return nw;
    return 1;
}

int attn_supported(int dtype, int Hq, int d_qk, int d_v)
{
    if (Hq < 1)
        return 0;
    if (dtype == 0)
        return d_qk == d_v && (d_qk == 32 || d_qk == 64 || d_qk == 128);
    if (dtype == 1)
        return Hq % 16 == 0 && ((d_qk == 128 && d_v == 128) || (d_qk == 576 && d_v == 512));
    return 0;
}

AttnPlan attn_plan(int total_q, int Hq, int d_v, int k)
{
    AttnPlan p{1, 0};
    const int groups = Hq % 16 == 0 ? (Hq / 16) / bf16_waves(Hq) : Hq;
    const int64_t wgs = (int64_t)total_q * groups;
    if (wgs < 512) {
        int ns = (int)((512 + wgs - 1) / wgs);
        ns = min(ns, max(1, k / 128));
        ns = min(ns, 16);
        if (ns > 1) {
            p.n_split = ns;
            p.ws_bytes = (size_t)total_q * ns * Hq * (d_v + 4) * sizeof(float);
        }
    }
    return p;
}

template <int DQK, int DV, bool MLA>
static hipError_t launch_bf16(const Batch &bt, const AttnPlan &pl, const void *q, int Hq, const void *kc,
                              const void *vc, int64_t rs, const int32_t *idx, int K, const void *gate, int pc,
                              float sl2, void *out, float *lse, float *part, int split_len, hipStream_t st)
{
    const int nw = bf16_waves(Hq);
    const dim3 grid(bt.total_q, Hq / (16 * nw), pl.n_split);
#define SA_LAUNCH_NW(NW)                                                                                        \
    hipLaunchKernelGGL((attn_bf16_kernel<DQK, DV, MLA, NW>), grid, dim3(NW * 64), 0, st, bt, (const uint16_t *)q, \
                       Hq, (const uint16_t *)kc, (const uint16_t *)vc, rs, idx, K, (const uint16_t *)gate, pc, sl2, \
                       (uint16_t *)out, lse, part, pl.n_split, split_len)
    switch (nw) {
    case 8: SA_LAUNCH_NW(8); break;
    case 4: SA_LAUNCH_NW(4); break;
    case 2: SA_LAUNCH_NW(2); break;
    default: SA_LAUNCH_NW(1); break;
    }
#undef SA_LAUNCH_NW
    return hipGetLastError();
}

hipError_t launch_attn(int dtype, const Batch &bt, const AttnPlan &pl, const void *q, int Hq, int d_qk,
                       const void *k_cache, const void *v_cache, int d_v, int64_t row_stride,
                       const int32_t *indices, int k, const void *gate, int per_channel, float scale, void *out,
                       float *lse, void *ws, hipStream_t st)
{
    if (bt.total_q > 0x7fffffff || pl.n_split > 65535)
        return hipErrorInvalidValue;
    const float sl2 = scale * kLog2e;
    const int split_len = (k + pl.n_split - 1) / pl.n_split;
    float *part = (float *)ws;
    hipError_t e = hipErrorInvalidValue;
    if (dtype == 1) {
        const bool mla = (k_cache == v_cache) && d_v <= d_qk;
        if (d_qk == 128 && d_v == 128 && !mla)
            e = launch_bf16<128, 128, false>(bt, pl, q, Hq, k_cache, v_cache, row_stride, indices, k, gate,
                                             per_channel, sl2, out, lse, part, split_len, st);
        else if (d_qk == 128 && d_v == 128 && mla)
            e = launch_bf16<128, 128, true>(bt, pl, q, Hq, k_cache, v_cache, row_stride, indices, k, gate,
                                            per_channel, sl2, out, lse, part, split_len, st);
        else if (d_qk == 576 && d_v == 512 && mla)
            e = launch_bf16<576, 512, true>(bt, pl, q, Hq, k_cache, v_cache, row_stride, indices, k, gate,
                                            per_channel, sl2, out, lse, part, split_len, st);
        else if (d_qk == 576 && d_v == 512)
            e = launch_bf16<576, 512, false>(bt, pl, q, Hq, k_cache, v_cache, row_stride, indices, k, gate,
                                             per_channel, sl2, out, lse, part, split_len, st);
    } else if (dtype == 0) {
        const dim3 grid(bt.total_q, Hq, pl.n_split);
#define SA_LAUNCH_F32(D)                                                                                         \
    hipLaunchKernelGGL((attn_f32_kernel<D>), grid, dim3(64), 0, st, bt, (const float *)q, Hq,                     \
                       (const float *)k_cache, (const float *)v_cache, row_stride, indices, k, (const float *)gate, \
                       per_channel, sl2, (float *)out, lse, part, pl.n_split, split_len)
        if (d_qk == 32) SA_LAUNCH_F32(32);
        else if (d_qk == 64) SA_LAUNCH_F32(64);
        else SA_LAUNCH_F32(128);
#undef SA_LAUNCH_F32
        e = hipGetLastError();
    }
    if (e != hipSuccess || pl.n_split == 1)
        return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(bt.total_q, Hq), dim3(128), 0, st, Hq, d_v, pl.n_split,
                       part, gate, per_channel, dtype == 1 ? 1 : 0, out, lse);
    return hipGetLastError();
}

} // namespace sa
