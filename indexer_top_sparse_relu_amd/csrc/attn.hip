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
// per wave) and a contiguous range of that token's index list.  At start it
// resolves every slot of its range to a physical cache row (page table) in
// LDS.  The selected rows are then gathered 64 at a time straight from global
// memory into LDS (global_load_lds, no registers), double-buffered so the next
// tile's gather runs under the current tile's math.  The tile is stored in
// blocks of 8 rows x 8 sixteen-byte chunks (1 KB, exactly one wave-wide load),
// with the chunks of each row XOR-swizzled by the row index, which spreads both
// operand reads over the LDS banks.  Per 32-key half tile, on 16x16x32 bf16
// MFMA: S^T = K Q^T (keys x heads: a lane owns one head's column, so the
// softmax is mostly in-lane), the online softmax in fp32, and O^T += V^T P^T
// with the V^T operand read by the LDS transpose load (ds_read_b64_tr_b16)
// directly from the row-major tile, so no transposed copy of V is made (for
// the latent layout V is the first d_v elements of the same rows).  The key
// order inside a lane's P registers (keys 4g..4g+3, then 16+4g..16+4g+3) is
// the order the transpose load delivers V in.  The epilogue divides by the
// softmax sum, multiplies by sigmoid(gate) and rounds to bf16; with a split
// index list it writes (O, max, sum) partials that a combine kernel merges by
// log-sum-exp.
#include <type_traits>

#include "sa_device.h"
#include "launch.h"

namespace sa {

constexpr int kTK = 64;                 // keys per LDS tile
constexpr int kMaxSplit = 2048;         // index slots one workgroup resolves up front
constexpr int kMaxCombine = 64;         // splits one combine workgroup merges (one lane each)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Swizzle of tile row r: logical chunk c of the row sits at chunk position
// (c & ~7) | ((c & 7) ^ f(r)) of its 8-chunk block, f(r) = r & 7.  A K-operand
// read (16 rows, one logical chunk each) and a V transpose read (8 rows, one
// chunk pair each) then hit distinct LDS banks; this was measured on gfx950
// with the bank-conflict counter for every read of the tile at its real LDS
// offsets (the bank of an address also depends on bits above the 256-byte
// bank span, so a plain modulo model does not predict it).
__device__ __forceinline__ int swzf(int r) { return r & 7; }

// The epilogue's output from the normalised attention x = o / l and the gate g:
// the gated output x * g or, given the other branch's output a of a two-branch
// layer, the branch mix g * a + (1 - g) * x = x + g * (a - x), in fp32.
__device__ __forceinline__ float gated(float x, float g, const void *mix, float a)
{
    return mix ? fmaf(g, a - x, x) : x * g;
}

template <int DQK, int DV, bool MLA, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(
    Batch bt, const uint16_t *__restrict__ q, int Hq, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, int64_t rs, const int32_t *__restrict__ idx, int K,
    const uint16_t *__restrict__ gate, int per_channel, float scale_log2, uint16_t *__restrict__ out,
    float *__restrict__ lse, float *__restrict__ part, int n_split, int split_len, const uint16_t *__restrict__ mix)
{
    constexpr int NT = NW * 64;
    constexpr int NKQ = DQK / 32;           // MFMA steps over d_qk
    constexpr int NMO = DV / 16;            // 16-dim tiles of O
    constexpr int KCH = DQK / 8;            // 16-byte chunks per K row
    constexpr int VCH = DV / 8;             // 16-byte chunks per V row
    constexpr int KCHUNKS = kTK * KCH, VCHUNKS = MLA ? 0 : kTK * VCH;
    constexpr int KCB = KCH / 8, VCB = VCH / 8;     // 8-chunk blocks per row
    constexpr int VROWB = MLA ? KCB : VCB;          // blocks per row of the buffer V is read from
    static_assert(DQK % 64 == 0 && DV % 16 == 0 && KCH % 8 == 0 && VCH % 8 == 0, "dims");
    static_assert(kTK % (8 * NW) == 0, "whole 8-row groups per wave");
    __shared__ __align__(16) uint8_t lk0[KCHUNKS * 16];
    __shared__ __align__(16) uint8_t lk1[KCHUNKS * 16];
    __shared__ __align__(16) uint8_t lv0[(MLA ? 16 : VCHUNKS * 16)];
    __shared__ __align__(16) uint8_t lv1[(MLA ? 16 : VCHUNKS * 16)];
    __shared__ int32_t prow[kMaxSplit];     // physical row of each slot; -1 - row0 when empty

    const int tok = blockIdx.x;
    const int hg = blockIdx.y;               // head group
    const int sp = blockIdx.z;               // split of the index list
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int h = hg * (16 * NW) + wv * 16 + n;   // this lane's head (column of S^T and O^T)
    const int b = seq_of_token(bt, tok);
    const int j0 = sp * split_len;
    const int j1 = min(K, j0 + split_len);
    const int nslots = max(0, j1 - j0);
    const int32_t *irow = idx + (int64_t)tok * K + j0;

    // ---- resolve slots to physical rows; empty slots point at position 0 (a real row)
    {
        const int row0 = (int)phys_row(bt, b, 0);
        for (int j = tid; j < nslots; j += NT) {
            const int s = irow[j];
            prow[j] = s >= 0 ? (int)phys_row(bt, b, s) : -1 - row0;
        }
    }

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
    __syncthreads();

    const int ntiles = (nslots + kTK - 1) / kTK;
    // Direct loads of one tile: block (rg, cb) holds rows 8rg..8rg+7, logical chunks
    // 8cb..8cb+7; lane i of the wave that loads it fetches row 8rg + i/8, chunk
    // position i%8 (logical chunk (i%8) ^ f(row)).  Wave wv owns row groups wv,
    // wv+NW, ... so it resolves one physical row per group.
    constexpr int RG = kTK / 8;
    auto issue = [&](int t, lds_u8 *dk, lds_u8 *dv, int ln) {
#pragma unroll
        for (int rg = wv; rg < RG; rg += NW) {
            const int r = 8 * rg + (ln >> 3);
            const int slot = t * kTK + r;
            int pr = prow[slot < nslots ? slot : 0];
            pr = pr >= 0 ? pr : -1 - pr;
            const int cpos = (ln & 7) ^ swzf(r);
            const uint16_t *ksrc = kc + (int64_t)pr * rs + cpos * 8;
#pragma unroll
            for (int cb = 0; cb < KCB; ++cb)
                __builtin_amdgcn_global_load_lds(ksrc + cb * 64, (lds_void *)(dk + (rg * KCB + cb) * 1024), 16, 0, 0);
            if (!MLA) {
                const uint16_t *vsrc = vc + (int64_t)pr * rs + cpos * 8;
#pragma unroll
                for (int cb = 0; cb < VCB; ++cb)
                    __builtin_amdgcn_global_load_lds(vsrc + cb * 64, (lds_void *)(dv + (rg * VCB + cb) * 1024), 16, 0, 0);
            }
        }
    };
    lds_u8 *const LK0 = (lds_u8 *)lk0, *const LK1 = (lds_u8 *)lk1;
    lds_u8 *const LV0 = (lds_u8 *)lv0, *const LV1 = (lds_u8 *)lv1;
    if (ntiles > 0)
        issue(0, LK0, LV0, lane);

    for (int t = 0; t < ntiles; ++t) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const bool odd = t & 1;
        const int ln = opaque(lane);
        // which of the tile's 64 slots hold a selected position (one bit per slot)
        const int myslot = t * kTK + ln;
        const uint64_t vmask = __ballot(myslot < nslots && prow[myslot < nslots ? myslot : 0] >= 0);
        lds_u8 *tk = odd ? LK1 : LK0;
        lds_u8 *tv = MLA ? tk : (odd ? LV1 : LV0);
        if (t + 1 < ntiles) {
            if (odd)
                issue(t + 1, LK0, LV0, ln);
            else
                issue(t + 1, LK1, LV1, ln);
        }
#pragma unroll 1
        for (int kh = 0; kh < 2; ++kh) {
            const int rb = 32 * kh;                       // first row of this half tile
            const int lk = opaque(lane);
            const int g = lk >> 4, n = lk & 15;
            // ---- S^T = K Q^T for keys rb..rb+15 and rb+16..rb+31.  Logical chunk
            // 4ks+g of row r: block ks/2, position 4(ks&1)+g xor f(r).  Operands
            // stream through a ring of QD steps so each MFMA waits only for its own.
            f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
            {
                constexpr int QD = 2;
                const int r0 = rb + n, r1 = rb + 16 + n;
                lds_u8 *k0 = tk + (r0 >> 3) * KCB * 1024 + (r0 & 7) * 128;
                lds_u8 *k1 = tk + (r1 >> 3) * KCB * 1024 + (r1 & 7) * 128;
                lds_u8 *k0e = k0 + 16 * (g ^ swzf(r0)), *k0o = k0 + 16 * ((4 + g) ^ swzf(r0));
                lds_u8 *k1e = k1 + 16 * (g ^ swzf(r1)), *k1o = k1 + 16 * ((4 + g) ^ swzf(r1));
                auto lda = [&](lds_u8 *e, lds_u8 *o_, int ks) {
                    return *(lds_bf16x8 *)(((ks & 1) ? o_ : e) + 1024 * (ks >> 1));
                };
                bf16x8 ra[QD], rb_[QD];
#pragma unroll
                for (int d = 0; d < QD; ++d) {
                    ra[d] = lda(k0e, k0o, d);
                    rb_[d] = lda(k1e, k1o, d);
                }
#pragma unroll
                for (int ks = 0; ks < NKQ; ++ks) {
                    s0 = mma16_bf16(ra[ks % QD], qop[ks], s0);
                    s1 = mma16_bf16(rb_[ks % QD], qop[ks], s1);
                    if (ks + QD < NKQ) {
                        ra[ks % QD] = lda(k0e, k0o, ks + QD);
                        rb_[ks % QD] = lda(k1e, k1o, ks + QD);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // ---- V^T operand ring: the transpose load gives lane (dim i, group g) the
            // dims of keys rb+4g..+3 (first load) and rb+16+4g..+3 (second load).
            // Logical chunk 2mt+hh of row r: block mt/4, position (2(mt&3)+hh) xor f(r).
            constexpr int PD = 3;
            const int jj = lk & 15;
            const int ra_ = rb + 4 * g + (jj >> 2), rc_ = ra_ + 16;
            const int cc = jj & 3, hh = cc >> 1;
            const int fa = swzf(ra_), fc = swzf(rc_);
            lds_u8 *va = tv + (ra_ >> 3) * VROWB * 1024 + (ra_ & 7) * 128 + (cc & 1) * 8;
            lds_u8 *vc2 = tv + (rc_ >> 3) * VROWB * 1024 + (rc_ & 7) * 128 + (cc & 1) * 8;
            auto ldv = [&](lds_u8 *v, int f, int mt) {
                return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4 *)(v + 1024 * (mt >> 2) + 16 * ((2 * (mt & 3) + hh) ^ f)));
            };
            bf16x4 la[PD], lc[PD];
#pragma unroll
            for (int d = 0; d < PD; ++d) {
                la[d] = ldv(va, fa, d);
                lc[d] = ldv(vc2, fc, d);
            }
            // ---- online softmax (log2 domain).  The running max is raised lazily:
            // only when some head of the wave grows by more than 2^8 are O and the
            // sum rescaled; otherwise probabilities use the stale max (<= 2^8).
            float z[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[i] = ((vmask >> (rb + 4 * g + i)) & 1) ? s0[i] * scale_log2 : -INFINITY;
                z[4 + i] = ((vmask >> (rb + 16 + 4 * g + i)) & 1) ? s1[i] * scale_log2 : -INFINITY;
            }
            float mt_ = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
            mt_ = fmaxf(mt_, shfl_xor(mt_, 16));
            mt_ = fmaxf(mt_, shfl_xor(mt_, 32));
            if (__any(mt_ > m_run + 8.0f)) {
                const float m_new = fmaxf(m_run, mt_);
                const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int mt = 0; mt < NMO; ++mt)
                    o[mt] *= alpha;
                m_run = m_new;
            }
            const float base = m_run == -INFINITY ? 0.0f : m_run;
            bf16x8 pop;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pi = __builtin_amdgcn_exp2f(z[i] - base);
                l_run += pi;
                pop[i] = (__bf16)pi;
            }
            // ---- O^T += V^T P^T
#pragma unroll
            for (int mt = 0; mt < NMO; ++mt) {
                bf16x8 vop;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vop[i] = la[mt % PD][i];
                    vop[4 + i] = lc[mt % PD][i];
                }
                o[mt] = mma16_bf16(vop, pop, o[mt]);
                if (mt + PD < NMO) {
                    la[mt % PD] = ldv(va, fa, mt + PD);
                    lc[mt % PD] = ldv(vc2, fc, mt + PD);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
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
        const uint16_t *ap = mix + ((int64_t)tok * Hq + h) * DV + 4 * g;
#pragma unroll
        for (int mt = 0; mt < NMO; ++mt) {
            uint16_t r[4];
            uint2 gv = per_channel ? *(const uint2 *)(gp + 16 * mt) : uint2{0u, 0u};
            uint2 av = mix ? *(const uint2 *)(ap + 16 * mt) : uint2{0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t gw = i < 2 ? gv.x : gv.y;
                const float gl = bf16_bits_to_f32((uint16_t)(gw >> (16 * (i & 1))));
                const float gi = per_channel ? __builtin_amdgcn_rcpf(1.0f + __expf(-gl)) : gh;
                const float a = bf16_bits_to_f32((uint16_t)((i < 2 ? av.x : av.y) >> (16 * (i & 1))));
                r[i] = f32_to_bf16_bits(gated(o[mt][i] * inv, gi, mix, a));
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

// Latent-layout kernel (d_qk = 576, d_v = 512, V = the first 512 dims of each
// gathered row) on 32x32x16 bf16 MFMA: 4 waves x 32 query heads per
// workgroup, one wave per SIMD.  Compared with 16 heads per wave on 16x16
// tiles, every LDS operand read feeds twice the MACs, so the tile reads per
// flop halve; Q^T stays in 144 VGPRs and the 16 O^T tiles (512 dims x 32
// heads) accumulate in the AGPR half of the register file.
// Per 32-key sub-tile: S^T = K Q^T (36 MFMAs; a lane holds one head's column
// and 16 keys), the online softmax, then O^T += V^T P^T (2 x 16 MFMAs).  The
// P^T operand is the lane's own S registers: in step j, lane half hq supplies
// keys 16j + 4hq + {0..3} and 16j + 8 + 4hq + {0..3}, the order in which two
// transpose loads of V deliver them.
// Tile layout: 64 rows x 72 sixteen-byte chunks, blocks of 8 rows x 8 chunks;
// chunk c of row r sits at block position (c & 7) ^ g(r), g(r) = 4*r[1] +
// 2*r[3] + r[2].  On gfx950 a 128-bit LDS read is served in four phases of 16
// lanes grouped by (lane bit 5, lane bit 3 ^ lane bit 4) and a transpose read
// in two phases of 32 lanes (bit 5), over 64 four-byte banks; under that
// (measured) rule g makes both the K reads (32 rows of one chunk per wave
// half) and the V reads (4 rows x 4 chunks per phase) conflict-free.
__device__ __forceinline__ int swzg(int r) { return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1); }

template <int DQK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_mla_kernel(
    Batch bt, const uint16_t *__restrict__ q, int Hq, const uint16_t *__restrict__ kc, int64_t rs,
    const int32_t *__restrict__ idx, int K, const uint16_t *__restrict__ gate, int per_channel, float scale_log2,
    uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part, int n_split, int split_len,
    const uint16_t *__restrict__ mix)
{
    constexpr int NW = 4;
    constexpr int NKQ = DQK / 16;           // MFMA k-steps over d_qk
    constexpr int NDT = DV / 32;            // 32-dim tiles of O^T
    constexpr int KCH = DQK / 8;            // 16-byte chunks per row
    constexpr int KCB = KCH / 8;            // 8-chunk blocks per row
    constexpr int TK = 32;                  // keys per tile (one 32x32 S^T tile)
    constexpr int KCHUNKS = TK * KCH;
    static_assert(DQK % 64 == 0 && DV % 32 == 0 && DV <= DQK, "dims");
    // a ring of four tiles: the gather of tile t+3 is issued while tile t is used
    // (one array: after the last tile it also stages the gated output rows)
    __shared__ __align__(16) uint8_t lkr[4 * KCHUNKS * 16];
    __shared__ int32_t prow[kMaxSplit];

    const int tok = blockIdx.x, hg = blockIdx.y, sp = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, hq = lane >> 5;
    const int h = hg * (32 * NW) + wv * 32 + col;
    const int b = seq_of_token(bt, tok);
    const int j0 = sp * split_len;
    const int j1 = min(K, j0 + split_len);
    const int nslots = max(0, j1 - j0);
    const int32_t *irow = idx + (int64_t)tok * K + j0;
    // Q^T operand: head h, dims 16ks + 8hq .. +7.  Issued first, so that its
    // loads overlap the slot resolution below; the rare rerun loads it again.
    struct QOp {
        bf16x8 v[NKQ];
    };
    auto load_q = [&]() {
        QOp r;
        const uint16_t *qp = q + ((int64_t)tok * Hq + h) * DQK + 8 * hq;
#pragma unroll
        for (int ks = 0; ks < NKQ; ++ks)
            r.v[ks] = *(const bf16x8 *)(qp + 16 * ks);
        return r;
    };
    const QOp q0 = load_q();
    const int row0 = (int)phys_row(bt, b, 0);      // a valid row of this sequence
    {
        // every slot's index, then every page-table entry: two memory round
        // trips in all (reads past the list re-read slot 0 and are dropped)
        constexpr int PS = kMaxSplit / (64 * NW);
        int sv[PS];
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            const int j = tid + 64 * NW * u;
            sv[u] = irow[j < nslots ? j : 0];
        }
        int pg[PS];
#pragma unroll
        for (int u = 0; u < PS; ++u)
            pg[u] = bt.page_table[(int64_t)b * bt.max_pages + ((sv[u] >= 0 ? sv[u] : 0) >> bt.page_shift)];
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            const int j = tid + 64 * NW * u;
            const int pr = (pg[u] << bt.page_shift) + (sv[u] & ((1 << bt.page_shift) - 1));
            if (j < nslots)
                prow[j] = sv[u] >= 0 ? pr : -1 - row0;
        }
    }
    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        o[dt] = f32x16{};
    // Softmax reference (log2 units) of this lane's head: fixed at the maximum of
    // its first valid keys and never moved, so O is never rescaled inside the
    // loop and later keys need no maximum at all.  Terms relative to it are exact
    // in fp32/bf16 while none exceeds 2^64; a sum above that (or a non-finite
    // result) sends the workgroup through a rerun: one pass for the exact
    // maximum, one with it as the reference (all terms then <= 1).
    // l_run sums the terms of keys 0..15 of each tile, l_run2 those of keys
    // 16..31 (two independent add chains)
    float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.0f, l_run2 = 0.0f;
    bool over = false;
    __syncthreads();

    const int ntiles = (nslots + TK - 1) / TK;
    constexpr int RG = TK / 8;
    static_assert(RG == NW, "one 8-row group per wave");
    // gather of tile t: wave wv loads row group wv (8 rows, KCB blocks of 1 KB):
    // exactly KCB direct loads per wave per tile; src_of gives this lane's
    // source (block 0) and the wave's LDS destination is dk + wv * KCB * 1024
    auto src_of = [&](int t, int ln) -> const uint16_t * {
        const int r = 8 * wv + (ln >> 3);
        const int slot = t * TK + r;
        const int raw = prow[slot < nslots ? slot : 0];
        int pr = slot < nslots ? raw : row0;      // (prow is unset when the list is empty)
        pr = pr >= 0 ? pr : -1 - pr;
        const int cpos = (ln & 7) ^ swzg(r);
        return kc + (int64_t)pr * rs + cpos * 8;
    };
    // slot-validity entry of key (ln & 31) of tile t (-1 past the list)
    auto vm_val = [&](int t, int ln) {
        const int sl = t * TK + (ln & 31);
        const int v = prow[sl < nslots ? sl : 0];
        return sl < nslots ? v : -1;
    };
    auto issue = [&](int t, lds_u8 *dk, int ln) {
        const uint16_t *ksrc = src_of(t, ln);
#pragma unroll
        for (int cb = 0; cb < KCB; ++cb)
            dma_b128(ksrc + cb * 64, dk + (wv * KCB + cb) * 1024);
    };
    auto buf = [&](int t) -> lds_u8 * {
        return (lds_u8 *)lkr + (t & 3) * (KCHUNKS * 16);
    };
    // One pass over the index list.  mode 0: reference from the first valid
    // keys, accumulate into oa; mode 1: exact maximum only (m_true), no P V;
    // mode 2: reference m_ref as given, accumulate into oa.
    auto run = [&](f32x16 (&oa)[NDT], const int mode, const QOp &qo) {
    const bf16x8 *qop = qo.v;
    bool have_ref = false;      // mode 0: the reference has been set from some valid key
    // Every pass issues exactly KCB loads per wave for each of the tiles
    // 0 .. ntiles+2: past the end of the list src_of falls back to a valid row
    // of the sequence and the data lands in a ring buffer nobody reads.  The
    // waits below are then one constant, and no load sits behind a branch.
#pragma unroll
    for (int t = 0; t < 3; ++t)
        issue(t, buf(t), lane);
    // One wait the compiler can see for the Q loads (and the first tiles).  Its
    // own tracking does not count the asm tile loads, and without this it would
    // keep the Q loads pending into the loop and wait on them before every MFMA
    // of the S chain, which in hardware also drains the tile loads in flight.
    __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0), expcnt and lgkmcnt unconstrained

    // The next tile's key mask entry and the source of the loads of tile t+4
    // are read from LDS inside the S chain of tile t, where the MFMAs cover the
    // read latency, and used one iteration later.
    int vm_cur = vm_val(0, lane);
    const uint16_t *src_cur = src_of(3, lane);
    for (int t = 0; t < ntiles; ++t) {
        // Tile t's loads were followed by those of tiles t+1 and t+2, KCB per
        // wave each, and by no other memory operation of this loop.
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * KCB) : "memory");
        __syncthreads();            // tile t complete; the buffer of tile t-1 is free
        const int ln = opaque(lane);
        const uint64_t vmask = __ballot(vm_cur >= 0);
        lds_u8 *tk = buf(t);
        // Tile t+3's loads are spread over the S chain (one per 4 MFMAs): issued
        // together, the four waves' loads back up the memory pipeline and each
        // wave stalls at issue with its MFMAs idle.
        const uint16_t *nsrc = src_cur;
        lds_u8 *ndk = buf(t + 3) + wv * KCB * 1024;
        static_assert(4 * (KCB - 1) < NKQ, "one tile load per 4 S-chain MFMAs");
        {
            constexpr int kh = 0;
            const int lk = opaque(lane);
            const int cl = lk & 31, hl = lk >> 5;
            // ---- S^T = K Q^T: A = K row r = 32kh + cl, chunk c = 2ks + hl.  With
            // (c & 7) ^ g(r) = 2(ks & 3) ^ (hl ^ g(r)) and c >> 3 = ks >> 2, every
            // read is one of four lane bases plus a constant offset.
            f32x16 s;
            {
                constexpr int QD = 6;
                const int r = 32 * kh + cl;
                lds_u8 *krow = tk + (r >> 3) * KCB * 1024 + (r & 7) * 128;
                const int gh = hl ^ swzg(r);
                lds_u8 *kb[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    kb[m] = krow + 16 * ((2 * m) ^ gh);
                auto lda = [&](int ks) { return *(lds_bf16x8 *)(kb[ks & 3] + 1024 * (ks >> 2)); };
                bf16x8 ka[QD];
#pragma unroll
                for (int d = 0; d < QD; ++d)
                    ka[d] = lda(d);
                // The S chain is written as asm so that its accumulator stays in
                // VGPRs: the AGPR half of the register file holds exactly the 256 O
                // accumulators.  Dependent MFMAs of one opcode chain back to back;
                // the last one is followed by the wait states a VALU read of its
                // result needs.
                // NSC independent chains (k-steps ks = c mod NSC) keep the MFMA pipe
                // busy with one wave per SIMD; summed at the end
                constexpr int NSC = 1;
                f32x16 sc[NSC];
#pragma unroll
                for (int ks = 0; ks < NKQ; ++ks) {
                    const int c = ks % NSC;
                    if (ks < NSC)
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                                     : "=&v"(sc[c]) : "v"(ka[ks % QD]), "v"(qop[ks]));
                    else if (ks + NSC < NKQ)
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                                     : "+v"(sc[c]) : "v"(ka[ks % QD]), "v"(qop[ks]));
                    else if (ks + 1 < NKQ)
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                                     : "+v"(sc[c]) : "v"(ka[ks % QD]), "v"(qop[ks]));
                    else
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
                                     "s_nop 7\n\ts_nop 7\n\ts_nop 3"
                                     : "+v"(sc[c]) : "v"(ka[ks % QD]), "v"(qop[ks]));
                    if (ks + QD < NKQ)
                        ka[ks % QD] = lda(ks + QD);
                    if (ks % 4 == 0 && ks / 4 < KCB)
                        dma_b128(nsrc + (ks / 4) * 64, ndk + (ks / 4) * 1024);
                    if (ks == NKQ - 12)
                        vm_cur = vm_val(t + 1, ln);
                    if (ks == NKQ - 8)
                        src_cur = src_of(t + 4, ln);
                }
                s = sc[0];
#pragma unroll
                for (int c = 1; c < NSC; ++c)
                    s += sc[c];
            }
            // ---- softmax terms against the head's reference (log2 units)
            const bool full = (uint32_t)(vmask >> (32 * kh)) == 0xFFFFFFFFu;
            auto valid = [&](int i) {
                return full || ((vmask >> (32 * kh + 8 * (i >> 2) + 4 * hl + (i & 3))) & 1);
            };
            // (have_ref and the key mask are wave-uniform: every head of the wave
            // sees the same keys, so this is a scalar branch taken once in mode 0)
            if (mode == 1 || (mode == 0 && !have_ref)) {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    mx = fmaxf(mx, valid(i) ? s[i] * scale_log2 : -INFINITY);
                mx = max_halves(mx);
                if (mode == 1) {
                    m_true = fmaxf(m_true, mx);
                } else {
                    m_ref = mx;
                    have_ref = (uint32_t)(vmask >> (32 * kh)) != 0u;
                }
            }
            if (mode != 1) {
                // ---- V^T operand ring: group G = lane / 16, i = lane % 16 reads row
                // r = 32kh + 16j + 8sec + 4hl + (i >> 2) (sec = second half of the
                // k-run), dims 32dt + 16(G & 1) + 4(i & 3) .. +3, i.e. chunk
                // c = 4dt + 2(G & 1) + (i & 3) / 2.  Here g(r) = 4 i[3] + 2 sec + hl,
                // so (c & 7) ^ g(r) splits into bits that depend on (dt & 1, sec) and
                // on the lane only: four lane bases plus constant offsets.
                constexpr int PD = 5;
                const int G = lk >> 4, i16 = lk & 15;
                lds_u8 *vrow = tk + kh * 4 * KCB * 1024 + (4 * hl + (i16 >> 2)) * 128 + 8 * (i16 & 1) +
                               16 * (((i16 & 3) >> 1) ^ hl);
                lds_u8 *vb[2][2];
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int sc = 0; sc < 2; ++sc)
                        vb[a][sc] = vrow + 64 * (a ^ ((i16 >> 3) & 1)) + 32 * ((G & 1) ^ sc);
                auto ldv = [&](int dt, int j, int sec) {
                    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4 *)(vb[dt & 1][sec] + (2 * j + sec) * KCB * 1024 + (dt >> 1) * 1024));
                };
                // PV step u covers dim tile u % NDT and k-half u / NDT (dim tile
                // fastest, so consecutive MFMAs never share an accumulator)
                auto vstep = [](int u) { return 2 * (u % NDT) + u / NDT; };
                auto ldv8 = [&](int step) {          // step = 2*dt + j
                    const bf16x4 lo = ldv(step >> 1, step & 1, 0), hi = ldv(step >> 1, step & 1, 1);
                    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                };
                bf16x8 va[PD];
#pragma unroll
                for (int d = 0; d < PD; ++d)
                    va[d] = ldv8(vstep(d));
                const float base = m_ref == -INFINITY ? 0.0f : m_ref;
                bf16x8 pop[2];
                auto pterm = [&](int i) {
                    const float pi = __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -base));
                    l_run += pi;
                    pop[i >> 3][i & 7] = (__bf16)pi;
                };
                // ---- O^T += V^T P^T.  The first NDT steps use keys 0..15 only
                // (pop[0]); the terms of keys 16..31 are computed between those
                // MFMAs, where VALU work hides behind the matrix pipe, as a
                // three-stage pipeline (step u: fma of key 16+u, exp of key 15+u,
                // sum and bf16 of key 14+u), so that no VALU op in a step waits
                // on another and the next MFMA issues on time.  Keys outside the
                // list get a logit of -inf (a term of exactly 0) up front, so every
                // tile runs the same straight-line code.
                static_assert(NDT >= 10, "keys 16..31 are ready before their first PV step");
                if (!full) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        s[i] = valid(i) ? s[i] : -INFINITY;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    pterm(i);
                float arg[8], ex[8];
#pragma unroll
                for (int u = 0; u < 2 * NDT; ++u) {
                    oa[u % NDT] = mma32_bf16(va[u % PD], pop[u / NDT], oa[u % NDT]);
                    if (u + PD < 2 * NDT)
                        va[u % PD] = ldv8(vstep(u + PD));
                    if (u < 8)
                        arg[u] = fmaf(s[8 + u], scale_log2, -base);
                    if (u >= 1 && u < 9)
                        ex[u - 1] = __builtin_amdgcn_exp2f(arg[u - 1]);
                    if (u >= 2 && u < 10) {
                        l_run2 += ex[u - 2];
                        pop[1][u - 2] = (__bf16)ex[u - 2];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    // the loads past the end of the list land before the ring is reused
    __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0)
    };

    // ---- epilogue: lane holds head h, dims 32dt + 8g + 4hq + {0..3} of tile dt
    auto store = [&](const f32x16 (&oa)[NDT]) {
    const float l_lane = l_run + l_run2;
    float l_tot = sum_halves(l_lane);
    float probe = 0.0f;                 // turns NaN if any result is not finite
    if (n_split == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        float gh = 0.0f;
        if (!per_channel)
            gh = sigmoidf_(bf16_bits_to_f32(gate[(int64_t)tok * Hq + h]));
        // The wave's 32 output rows (heads wv*32 .. +31, DV bf16 each) leave
        // through LDS as whole rows (16-byte stores); straight from the O^T
        // layout every access would be 8 bytes per lane, 64 rows apart.
        constexpr int ROWB = 2 * DV + 16;
        static_assert(4 * 32 * ROWB <= 4 * KCHUNKS * 16 && DV * 2 == 64 * 16, "output staging");
        lds_u8 *stg = (lds_u8 *)lkr + wv * 32 * ROWB;
        const int64_t row0 = (int64_t)tok * Hq + hg * (32 * NW) + wv * 32;
        __syncthreads();                        // every wave is done with the tile ring
        if (mix) {
            // Branch mix: the other branch's rows are read as well, so the
            // columns go in two halves.  Row j of the staging area holds the
            // half's gate values (bytes 0..DV) and the other branch's (DV..2DV),
            // both brought in by direct loads (lanes 0-31 and 32-63 of each
            // load); y replaces the gate values in place and leaves as whole
            // half rows.
            constexpr int HALF = NDT / 2;
            static_assert(NDT % 2 == 0, "halves");
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const uint16_t *src = (hq ? mix : gate) + row0 * DV + hf * (DV / 2) + 8 * col;
                if (hq || per_channel) {
#pragma unroll 8
                    for (int j = 0; j < 32; ++j)
                        dma_b128(src + j * DV, stg + j * ROWB);
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this half's rows are in LDS
                lds_u8 *mh = stg + col * ROWB + 8 * hq;
#pragma unroll
                for (int dt = 0; dt < HALF; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        lds_u8 *p = mh + 2 * (32 * dt + 8 * g);
                        const u32x2 av = *(const lds_u32x2 *)(p + DV);
                        const u32x2 w = per_channel ? *(const lds_u32x2 *)p : u32x2{0u, 0u};
                        float y[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int sh = 16 * (i & 1);
                            float gi = gh;
                            if (per_channel)
                                gi = __builtin_amdgcn_rcpf(
                                    1.0f + __expf(-bf16_bits_to_f32((uint16_t)((i < 2 ? w.x : w.y) >> sh))));
                            const float a = bf16_bits_to_f32((uint16_t)((i < 2 ? av.x : av.y) >> sh));
                            y[i] = gated(oa[HALF * hf + dt][4 * g + i] * inv, gi, mix, a);
                            probe = fmaf(y[i], 0.0f, probe);
                        }
                        const bf16x2 lo = {(__bf16)y[0], (__bf16)y[1]}, hi = {(__bf16)y[2], (__bf16)y[3]};
                        *(lds_u32x2 *)p = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                    }
                __builtin_amdgcn_wave_barrier();
                // two half rows per store instruction
                uint16_t *oh = out + row0 * DV + hf * (DV / 2) + 8 * col;
#pragma unroll 8
                for (int j = 0; j < 32; j += 2)
                    *(u32x4 *)(oh + (j + hq) * DV) = *(const lds_u32x4 *)(stg + (j + hq) * ROWB + 16 * col);
                // the stores' reads of the staging area are done before the
                // next half's loads land there
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            }
        } else {
            // row j at stg + j*ROWB: the gate rows arrive there by direct loads
            // (contiguous in memory), each lane forms y = o/l * gate for its
            // 4 x 4 x NDT elements in place, and whole rows leave
            if (per_channel) {
                const uint16_t *gsrc = gate + row0 * DV + 8 * lane;
#pragma unroll 8
                for (int j = 0; j < 32; ++j)
                    dma_b128(gsrc + j * DV, stg + j * ROWB);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the gate rows are in LDS
            lds_u8 *mine = stg + col * ROWB + 8 * hq;
            auto put4 = [&](int dt, int g, const float (&gi)[4]) {
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // (inv * gate first: with o * inv shared by both gate forms the
                    // compiler would compute all of them up front)
                    y[i] = oa[dt][4 * g + i] * (inv * gi[i]);
                    probe = fmaf(y[i], 0.0f, probe);
                }
                // bf16 round-to-nearest-even, two values per convert instruction
                const bf16x2 lo = {(__bf16)y[0], (__bf16)y[1]}, hi = {(__bf16)y[2], (__bf16)y[3]};
                *(lds_u32x2 *)(mine + 2 * (32 * dt + 8 * g)) =
                    u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            };
            if (per_channel) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const u32x2 w = *(const lds_u32x2 *)(mine + 2 * (32 * dt + 8 * g));
                        float gi[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = bf16_bits_to_f32((uint16_t)((i < 2 ? w.x : w.y) >> (16 * (i & 1))));
                            gi[i] = __builtin_amdgcn_rcpf(1.0f + __expf(-x));
                        }
                        put4(dt, g, gi);
                    }
            } else {
                const float gi[4] = {gh, gh, gh, gh};
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        put4(dt, g, gi);
            }
            __builtin_amdgcn_wave_barrier();
            uint16_t *orow = out + row0 * DV + 8 * lane;
#pragma unroll 8
            for (int j = 0; j < 32; ++j)
                *(u32x4 *)(orow + j * DV) = *(const lds_u32x4 *)(stg + j * ROWB + 16 * lane);
        }
        if (lse && hq == 0)
            lse[(int64_t)tok * Hq + h] = l_tot > 0.0f ? m_ref * kLn2 + __logf(l_tot) : -INFINITY;
    } else {
        float *pp = part + (((int64_t)tok * n_split + sp) * Hq + h) * (DV + 4) + 4 * hq;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v4 = f32x4{oa[dt][4 * g], oa[dt][4 * g + 1], oa[dt][4 * g + 2], oa[dt][4 * g + 3]};
                probe = fmaf(v4[0] + v4[1] + v4[2] + v4[3], 0.0f, probe);
                *(f32x4 *)(pp + 32 * dt + 8 * g) = v4;
            }
        if (hq == 0) {
            pp[DV] = m_ref;
            pp[DV + 1] = l_tot;
        }
    }
    return !(l_tot <= 0x1p64f) || probe != 0.0f;
    };

    run(o, 0, q0);
    over = store(o);
    if (__syncthreads_or(over)) {
        // rare: some head's terms outgrew 2^64 relative to its first keys; find
        // the exact maximum, then rerun with it as the reference (terms <= 1).
        // The max-only pass does not touch o; o is cleared only after it, so no
        // second accumulator array is ever live.
        run(o, 1, load_q());
        __syncthreads();
        m_ref = m_true;
        l_run = 0.0f;
        l_run2 = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            o[dt] = f32x16{};
        run(o, 2, load_q());
        store(o);
    }
}

// MQA kernel (d_qk = d_v = D = 128, 32 query heads per unit, separate K and V
// caches or one shared row) on 32x32x16 bf16 MFMA.  A unit is one (token,
// group of 32 heads, split of the index list) and belongs to one wave; the
// four waves of a workgroup are independent units (consecutive tokens), so the
// kernel has no workgroup barrier.  Each wave resolves its slots to physical
// rows in its own LDS area.  Per 32-key tile:
//   - the gather: each load instruction covers four whole rows (16 lanes x 16
//     bytes per 256-byte row).  On gfx950 the address unit's cost grows with
//     the cache lines an instruction touches: this pattern gathers about 2.5x
//     faster than loading the MFMA operand layout directly (32 rows x 32
//     bytes per instruction).  The rows land in VGPRs, two tiles ahead (every
//     load is compiler-tracked, so its waits are exact), and are written to
//     the wave's LDS tiles (K, and V unless the row is shared);
//   - S^T = K Q^T (8 MFMAs, K from LDS, Q^T in VGPRs, a lane holds one head's
//     column), softmax terms against a fixed per-head reference as in the
//     latent kernel (exact rerun when a term outgrows 2^64), O^T += V^T P^T
//     (8 MFMAs, V^T by transpose loads).
// The LDS tiles use the latent kernel's layout and swizzle (blocks of 8 rows x
// 8 sixteen-byte chunks, position (c & 7) ^ g(r)), under which its K reads and
// V transpose reads are conflict-free.
template <int D, bool SHARED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_mqa_kernel(
    Batch bt, const uint16_t *__restrict__ q, int Hq, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, int64_t rs, const int32_t *__restrict__ idx, int K,
    const uint16_t *__restrict__ gate, int per_channel, float scale_log2, uint16_t *__restrict__ out,
    float *__restrict__ lse, float *__restrict__ part, int n_split, int split_len, int n_units,
    const uint16_t *__restrict__ mix)
{
    constexpr int NW = 4;
    constexpr int NKQ = D / 16;             // S-chain k-steps
    constexpr int NDT = D / 32;             // 32-dim tiles of O^T
    constexpr int KCB = D / 64;             // 8-chunk blocks per row
    constexpr int TK = 32;                  // keys per tile
    constexpr int TB = TK * D * 2;          // bytes of one K (or V) tile in LDS
    constexpr int RPI = 64 / (D / 8);       // rows per load instruction (16-byte chunks per row: D / 8)
    constexpr int NI = TK / RPI;            // load instructions per tile and cache
    constexpr int NT = SHARED ? 1 : 2;      // LDS tiles per wave (K, V)
    static_assert(D % 64 == 0 && NKQ % 4 == 0 && 64 % (D / 8) == 0, "dims");
    constexpr int MAXT = kMaxSplit / TK + 3;   // tiles of a list, the two loaded past its end, and one more
                                               // whose offsets are read (not used) after the last step
    __shared__ __align__(16) uint8_t ltile[NW * NT * TB];
    __shared__ uint64_t loff[NW * MAXT * TK];  // byte offset of each slot's cache row
    __shared__ uint32_t lmask[NW * MAXT];     // valid slots of each tile, one bit per key

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // units in reverse: in causal prefill the last tokens have the longest lists,
    // so they start first and the short lists of the first tokens fill the tail
    const int unit = n_units - 1 - (blockIdx.x * NW + wv);
    if (unit < 0)
        return;
    const int HG = Hq >> 5;
    const int sp = unit % n_split;
    const int rest = unit / n_split;
    const int hg = rest % HG, tok = rest / HG;
    const int col = lane & 31, hq = lane >> 5;
    const int h = hg * 32 + col;
    const int b = seq_of_token(bt, tok);
    const int j0 = sp * split_len;
    const int j1 = min(K, j0 + split_len);
    const int nslots = max(0, j1 - j0);
    const int32_t *irow = idx + (int64_t)tok * K + j0;
    lds_u8 *const tk = (lds_u8 *)ltile + wv * NT * TB;
    lds_u8 *const tv = SHARED ? tk : tk + TB;
    uint64_t *const off = loff + wv * MAXT * TK;
    uint32_t *const msk = lmask + wv * MAXT;

    // Q^T operand: head h, dims 16ks + 8hq .. +7
    struct QOp {
        bf16x8 v[NKQ];
    };
    auto load_q = [&]() {
        QOp r;
        const uint16_t *qp = q + ((int64_t)tok * Hq + h) * D + 8 * hq;
#pragma unroll
        for (int ks = 0; ks < NKQ; ++ks)
            r.v[ks] = *(const bf16x8 *)(qp + 16 * ks);
        return r;
    };
    const QOp q0 = load_q();
    // leading tiles with every key valid, and the tiles up to the last valid key
    // (lists from sparse_topk hold their valid positions first, then -1, so all
    // but the last of their tiles are full; any other list takes the masked step
    // from its first tile with a missing key on)
    int nfull = 0, ntiles = 0;
    {
        // every slot's index, then every page-table entry (two round trips); each
        // slot keeps the byte offset of its cache row, and slots past the list or
        // holding padding keep position 0's row (a valid row: their loads are in
        // bounds, their keys are masked)
        const uint64_t rsb = (uint64_t)rs * 2;
        const int64_t row0 = phys_row(bt, b, 0);
        constexpr int PS = kMaxSplit / 64 + 2;
        int sv[PS];
#pragma unroll
        for (int u = 0; u < PS; ++u) {
            const int j = lane + 64 * u;
            sv[u] = j < nslots ? irow[j] : -1;
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
            if (nfull == 2 * u && lo == 0xFFFFFFFFu)
                nfull = 2 * u + 1 + (hi == 0xFFFFFFFFu);
            if (lo)
                ntiles = 2 * u + 1;
            if (hi)
                ntiles = 2 * u + 2;
            if (lane == 0 && 2 * u < MAXT) {
                msk[2 * u] = (uint32_t)vb;
                if (2 * u + 1 < MAXT)
                    msk[2 * u + 1] = (uint32_t)(vb >> 32);
            }
        }
    }
    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        o[dt] = f32x16{};
    float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.0f;

    // one tile's gather: instruction i, lane l -> tile row RPI*i + l / (D/8), chunk l % (D/8)
    struct Stage {
        i32x4 k[NI];
        i32x4 v[SHARED ? 1 : NI];
    };
    const int lrow = lane / (D / 8), lch = lane % (D / 8);
    const uint8_t *const kbase = (const uint8_t *)kc + 16 * lch;
    const uint8_t *const vbase = (const uint8_t *)vc + 16 * lch;
    // the byte offsets of this lane's rows of tile t, read from LDS one tile
    // before its loads are issued, so that the issue waits on no LDS read
    struct Offs {
        uint64_t o[NI];
    };
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
            const uint64_t ob = of.o[i];
            st.k[i] = *(const i32x4 *)(kbase + ob);
            if constexpr (!SHARED)
                st.v[i] = *(const i32x4 *)(vbase + ob);
        }
        return st;
    };
    // LDS position of chunk c of tile row r: block (r / 8) * KCB + c / 8, row r % 8
    // of the block, position (c % 8) ^ g(r).  With r = RPI*i + lrow (RPI = 4),
    // g(r) = 4*(lrow / 2) + (i % 4), so four lane bases plus constants cover it.
    static_assert(RPI == 4, "four rows per load instruction");
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
    // S^T A operand (K row cl, chunk 2ks + hl) and V^T transpose-load bases
    const int cl = lane & 31, hl = lane >> 5;
    lds_u8 *kb[4];
    {
        lds_u8 *krow = tk + (cl >> 3) * KCB * 1024 + (cl & 7) * 128;
        const int gh = hl ^ swzg(cl);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            kb[m] = krow + 16 * ((2 * m) ^ gh);
    }
    lds_u8 *vb[2][2];
    {
        const int G = lane >> 4, i16 = lane & 15;
        lds_u8 *vrow = tv + (4 * hl + (i16 >> 2)) * 128 + 8 * (i16 & 1) + 16 * (((i16 & 3) >> 1) ^ hl);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int sc = 0; sc < 2; ++sc)
                vb[a][sc] = vrow + 64 * (a ^ ((i16 >> 3) & 1)) + 32 * ((G & 1) ^ sc);
    }

    // One pass over the index list.  mode 0: reference from the first valid
    // keys, accumulate; mode 1: exact maximum only (m_true); mode 2: reference
    // m_ref as given, accumulate.
    // The reference is taken from the first tile with a valid key (tile 0 for a
    // list from sparse_topk) and the leading full tiles need no key mask, so the
    // steady-state tile step carries neither: `first` and `partial` are
    // compile-time flags, and later tiles test the wave-uniform have_ref only
    // until some tile has set the reference.
    auto run = [&](f32x16 (&oa)[NDT], const int mode, const QOp &qo) {
        const bf16x8 *qop = qo.v;
        bool have_ref = false;      // mode 0: the reference has been set from some valid key
        // two stages in registers: tile t is written to LDS while t+1 is in flight,
        // then the stage is reloaded with tile t+2
        Stage s0 = load_stage(read_offs(0)), s1 = load_stage(read_offs(1));
        Offs on = read_offs(2);
        auto step = [&](int t, Stage &st, auto first_c, auto partial_c) {
            constexpr bool FIRST = decltype(first_c)::value, PARTIAL = decltype(partial_c)::value;
            put_stage(st);
            asm volatile("" ::: "memory");      // the tile's writes precede its reads
            st = load_stage(on);                // tile t + 2
            on = read_offs(t + 3);
            // ---- S^T = K Q^T: A = K row cl, chunk 2ks + hl
            // (written as asm so that the accumulator stays in VGPRs, where the
            // softmax reads it; the AGPRs hold O.  The last MFMA is followed by the
            // wait states a VALU read of its result needs.)
            f32x16 s;
            {
                constexpr int QD = 4;
                auto lda = [&](int ks) { return *(lds_bf16x8 *)(kb[ks & 3] + 1024 * (ks >> 2)); };
                bf16x8 ka[QD];
#pragma unroll
                for (int d = 0; d < QD; ++d)
                    ka[d] = lda(d);
#pragma unroll
                for (int ks = 0; ks < NKQ; ++ks) {
                    if (ks == 0)
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                                     : "=&v"(s) : "v"(ka[ks % QD]), "v"(qop[ks]));
                    else if (ks + 1 < NKQ)
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                                     : "+v"(s) : "v"(ka[ks % QD]), "v"(qop[ks]));
                    else
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
                                     "s_nop 7\n\ts_nop 7\n\ts_nop 3"
                                     : "+v"(s) : "v"(ka[ks % QD]), "v"(qop[ks]));
                    if (ks + QD < NKQ)
                        ka[ks % QD] = lda(ks + QD);
                }
            }
            // logits in log2 units; keys outside the list get -inf (a term of 0)
            const uint32_t vmask = PARTIAL ? __builtin_amdgcn_readfirstlane(msk[t]) : 0xFFFFFFFFu;
            if constexpr (PARTIAL) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    s[i] = ((vmask >> (8 * (i >> 2) + 4 * hl + (i & 3))) & 1) ? s[i] : -INFINITY;
            }
            if (mode == 1 || (mode == 0 && (FIRST || !have_ref))) {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    mx = fmaxf(mx, s[i] * scale_log2);
                mx = max_halves(mx);
                if (mode == 1) {
                    m_true = fmaxf(m_true, mx);
                } else {
                    m_ref = mx;
                    have_ref = vmask != 0u;
                }
            }
            if (mode != 1) {
                // ---- O^T += V^T P^T (transpose loads; the latent kernel's V^T mapping).
                // The first V^T operands are read before the softmax terms, whose
                // VALU work covers their LDS latency.
                auto ldv = [&](int dt, int j, int sec) {
                    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4 *)(vb[dt & 1][sec] + (2 * j + sec) * KCB * 1024 + (dt >> 1) * 1024));
                };
                auto vstep = [](int u) { return 2 * (u % NDT) + u / NDT; };
                auto ldv8 = [&](int stp) {
                    const bf16x4 lo = ldv(stp >> 1, stp & 1, 0), hi = ldv(stp >> 1, stp & 1, 1);
                    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                };
                constexpr int PD = 4;
                bf16x8 va[PD];
#pragma unroll
                for (int d = 0; d < PD; ++d)
                    va[d] = ldv8(vstep(d));
                const float base = m_ref == -INFINITY ? 0.0f : m_ref;
                bf16x8 pop[2];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pi = __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -base));
                    l_run += pi;
                    pop[i >> 3][i & 7] = (__bf16)pi;
                }
#pragma unroll
                for (int u = 0; u < 2 * NDT; ++u) {
                    oa[u % NDT] = mma32_bf16(va[u % PD], pop[u / NDT], oa[u % NDT]);
                    if (u + PD < 2 * NDT)
                        va[u % PD] = ldv8(vstep(u + PD));
                }
            }
            asm volatile("" ::: "memory");      // the tile's reads precede the next tile's writes
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        if (ntiles == 0)
            return;
        // tile 0 (stage s0), then the full tiles in pairs (s1, s0), then the tail
        if (nfull == 0)
            step(0, s0, T_{}, T_{});
        else
            step(0, s0, T_{}, F_{});
        int t = 1;
        for (; t + 1 < nfull; t += 2) {
            step(t, s1, F_{}, F_{});
            step(t + 1, s0, F_{}, F_{});
        }
        if (t < nfull) {
            step(t, s1, F_{}, F_{});
            ++t;
        }
        for (; t < ntiles; ++t) {       // tiles with some key missing
            if (t & 1)
                step(t, s1, F_{}, T_{});
            else
                step(t, s0, F_{}, T_{});
        }
    };

    // ---- epilogue: lane holds head h, dims 32dt + 8g + 4hq + {0..3} of tile dt
    auto store = [&](const f32x16 (&oa)[NDT]) {
        float l_tot = sum_halves(l_run);
        float probe = 0.0f;                 // turns NaN if any result is not finite
        if (n_split == 1) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            const int64_t orow = ((int64_t)tok * Hq + h) * D;
            u32x2 aw[NDT][4];           // the other branch's output (branch mix only)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    aw[dt][g] = mix ? *(const u32x2 *)(mix + orow + 32 * dt + 8 * g + 4 * hq) : u32x2{0u, 0u};
            auto a_of = [&](int dt, int g, int i) {
                return bf16_bits_to_f32((uint16_t)((i < 2 ? aw[dt][g].x : aw[dt][g].y) >> (16 * (i & 1))));
            };
            if (per_channel) {
                u32x2 gw[NDT][4];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        gw[dt][g] = *(const u32x2 *)(gate + orow + 32 * dt + 8 * g + 4 * hq);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float y[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t w = i < 2 ? gw[dt][g].x : gw[dt][g].y;
                            const float x = bf16_bits_to_f32((uint16_t)(w >> (16 * (i & 1))));
                            const float gi = __builtin_amdgcn_rcpf(1.0f + __expf(-x));
                            y[i] = gated(oa[dt][4 * g + i] * inv, gi, mix, a_of(dt, g, i));
                            probe = fmaf(y[i], 0.0f, probe);
                        }
                        const bf16x2 lo = {(__bf16)y[0], (__bf16)y[1]}, hi = {(__bf16)y[2], (__bf16)y[3]};
                        *(u32x2 *)(out + orow + 32 * dt + 8 * g + 4 * hq) =
                            u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                    }
            } else {
                const float gi = sigmoidf_(bf16_bits_to_f32(gate[(int64_t)tok * Hq + h]));
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float y[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            y[i] = gated(oa[dt][4 * g + i] * inv, gi, mix, a_of(dt, g, i));
                            probe = fmaf(y[i], 0.0f, probe);
                        }
                        const bf16x2 lo = {(__bf16)y[0], (__bf16)y[1]}, hi = {(__bf16)y[2], (__bf16)y[3]};
                        *(u32x2 *)(out + orow + 32 * dt + 8 * g + 4 * hq) =
                            u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                    }
            }
            if (lse && hq == 0)
                lse[(int64_t)tok * Hq + h] = l_tot > 0.0f ? m_ref * kLn2 + __logf(l_tot) : -INFINITY;
        } else {
            float *pp = part + (((int64_t)tok * n_split + sp) * Hq + h) * (D + 4) + 4 * hq;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 v4 = f32x4{oa[dt][4 * g], oa[dt][4 * g + 1], oa[dt][4 * g + 2], oa[dt][4 * g + 3]};
                    probe = fmaf(v4[0] + v4[1] + v4[2] + v4[3], 0.0f, probe);
                    *(f32x4 *)(pp + 32 * dt + 8 * g) = v4;
                }
            if (hq == 0) {
                pp[D] = m_ref;
                pp[D + 1] = l_tot;
            }
        }
        return !(l_tot <= 0x1p64f) || probe != 0.0f;
    };

    run(o, 0, q0);
    const bool over = store(o);
    if (__ballot(over) != 0) {
        // rare: some head's terms outgrew 2^64 relative to its first keys; find
        // the exact maximum, then rerun with it as the reference (terms <= 1)
        run(o, 1, load_q());
        m_ref = m_true;
        l_run = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            o[dt] = f32x16{};
        run(o, 2, load_q());
        store(o);
    }
}

// Merge split partials by log-sum-exp, then gate; one block per (token, head).
__global__ __launch_bounds__(128) void attn_combine_kernel(int Hq, int DV, int n_split, const float *__restrict__ part,
                                                          const void *__restrict__ gate, int per_channel, int is_bf16,
                                                          void *__restrict__ out, float *__restrict__ lse,
                                                          const void *__restrict__ mix)
{
    const int tok = blockIdx.x, h = blockIdx.y;
    const float *pp = part + ((int64_t)tok * n_split * Hq + h) * (DV + 4);
    const int64_t sstride = (int64_t)Hq * (DV + 4);
    // wave 0, one lane per split: the splits' (max, sum) pairs are loaded at
    // once, and each split's weight 2^(m_s - M) is kept in LDS
    __shared__ float wsh[kMaxCombine];
    __shared__ float ml[2];
    if (threadIdx.x < 64) {
        const int s = threadIdx.x;
        const float m = s < n_split ? pp[s * sstride + DV] : -INFINITY;
        const float l = s < n_split ? pp[s * sstride + DV + 1] : 0.0f;
        const float Mw = wave_max(m);
        const float w = s < n_split ? exp2f(m - (Mw == -INFINITY ? 0.0f : Mw)) : 0.0f;
        const float Lw = wave_sum(l * w);
        if (s < n_split)
            wsh[s] = w;
        if (s == 0) {
            ml[0] = Mw;
            ml[1] = Lw;
        }
    }
    __syncthreads();
    const float M = ml[0], L = ml[1];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int64_t ob = ((int64_t)tok * Hq + h) * DV;
    for (int c = threadIdx.x; c < DV; c += blockDim.x) {
        float acc = 0.0f;
#pragma unroll 8
        for (int s = 0; s < n_split; ++s)
            acc += pp[s * sstride + c] * wsh[s];
        float gl;
        const int64_t gi = per_channel ? ob + c : (int64_t)tok * Hq + h;
        if (is_bf16)
            gl = bf16_bits_to_f32(((const uint16_t *)gate)[gi]);
        else
            gl = ((const float *)gate)[gi];
        float a = 0.0f;
        if (mix)
            a = is_bf16 ? bf16_bits_to_f32(((const uint16_t *)mix)[ob + c]) : ((const float *)mix)[ob + c];
        const float y = gated(acc * inv, sigmoidf_(gl), mix, a);
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
                                                      int n_split, int split_len, const float *__restrict__ mix)
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
                const int64_t oi = ((int64_t)tok * Hq + h) * D + c;
                out[oi] = gated(o[u] * inv, sigmoidf_(gl), mix, mix ? mix[oi] : 0.0f);
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

int attn_supported_layout(int dtype, int d_qk, int d_v, int aliased)
{
    // two double-buffered 576-wide tiles do not fit the 160 KB LDS: latent layout only
    if (dtype == 1 && d_qk == 576 && d_v == 512)
        return aliased;
    return 1;
}

AttnPlan attn_plan(int total_q, int Hq, int d_v, int k)
{
    AttnPlan p{1, 0};
    const int groups = Hq % 16 == 0 ? (Hq / 16) / bf16_waves(Hq) : Hq;
    const int64_t wgs = (int64_t)total_q * groups;
    int ns = 1;
    if (wgs < 512) {
        // at most 8 splits: each split writes a partial of d_v + 4 floats per head,
        // which the combine reads back (16 decode tokens x 128 latent heads: 0.061
        // ms with 8 splits, 0.072 with 16, 0.079 with 4)
        ns = (int)((512 + wgs - 1) / wgs);
        ns = min(ns, max(1, k / 128));
        ns = min(ns, 8);
    }
    ns = max(ns, (k + kMaxSplit - 1) / kMaxSplit);     // a workgroup resolves at most kMaxSplit slots
    if (ns > 1) {
        p.n_split = ns;
        p.ws_bytes = (size_t)total_q * ns * Hq * (d_v + 4) * sizeof(float);
    }
    return p;
}

template <int DQK, int DV, bool MLA>
static hipError_t launch_bf16(const Batch &bt, const AttnPlan &pl, const void *q, int Hq, const void *kc,
                              const void *vc, int64_t rs, const int32_t *idx, int K, const void *gate, int pc,
                              float sl2, void *out, float *lse, float *part, int split_len, const void *mix,
                              hipStream_t st)
{
    const int nw = bf16_waves(Hq);
    const dim3 grid(bt.total_q, Hq / (16 * nw), pl.n_split);
#define SA_LAUNCH_NW(NW)                                                                                        \
    hipLaunchKernelGGL((attn_bf16_kernel<DQK, DV, MLA, NW>), grid, dim3(NW * 64), 0, st, bt, (const uint16_t *)q, \
                       Hq, (const uint16_t *)kc, (const uint16_t *)vc, rs, idx, K, (const uint16_t *)gate, pc, sl2, \
                       (uint16_t *)out, lse, part, pl.n_split, split_len, (const uint16_t *)(pl.n_split == 1 ? mix : nullptr))
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
                       float *lse, void *ws, hipStream_t st, const void *mix)
{
    if (bt.total_q > 0x7fffffff || pl.n_split > 65535)
        return hipErrorInvalidValue;
    const float sl2 = scale * kLog2e;
    const int split_len = (k + pl.n_split - 1) / pl.n_split;
    float *part = (float *)ws;
    // the branch mix is applied where the output is formed: by the attention
    // kernel itself, or by the combine kernel when the list is split
    const void *kmix = pl.n_split == 1 ? mix : nullptr;
    hipError_t e = hipErrorInvalidValue;
    if (dtype == 1) {
        const bool mla = (k_cache == v_cache) && d_v <= d_qk;
        if (d_qk == 128 && d_v == 128 && Hq % 32 == 0 && pl.n_split == 1) {
            // one wave per (token, 32 heads); split lists (decode, few tokens) take
            // attn_bf16_kernel, measured faster there (its workgroups hold 16*NW
            // heads of a token, and each split is short)
            const int64_t units = (int64_t)bt.total_q * (Hq / 32) * pl.n_split;
            if (units > 0x7fffffffLL)
                return hipErrorInvalidValue;
            const dim3 grid((unsigned)((units + 3) / 4));
#define SA_LAUNCH_MQA(SH)                                                                                       \
    hipLaunchKernelGGL((attn_mqa_kernel<128, SH>), grid, dim3(256), 0, st, bt, (const uint16_t *)q, Hq,           \
                       (const uint16_t *)k_cache, (const uint16_t *)v_cache, row_stride, indices, k,              \
                       (const uint16_t *)gate, per_channel, sl2, (uint16_t *)out, lse, part, pl.n_split, split_len, \
                       (int)units, (const uint16_t *)kmix)
            if (mla)
                SA_LAUNCH_MQA(true);
            else
                SA_LAUNCH_MQA(false);
#undef SA_LAUNCH_MQA
            e = hipGetLastError();
        } else if (d_qk == 128 && d_v == 128 && !mla)
            e = launch_bf16<128, 128, false>(bt, pl, q, Hq, k_cache, v_cache, row_stride, indices, k, gate,
                                             per_channel, sl2, out, lse, part, split_len, mix, st);
        else if (d_qk == 128 && d_v == 128 && mla)
            e = launch_bf16<128, 128, true>(bt, pl, q, Hq, k_cache, v_cache, row_stride, indices, k, gate,
                                            per_channel, sl2, out, lse, part, split_len, mix, st);
        else if (d_qk == 576 && d_v == 512 && mla && Hq % 128 == 0) {
            hipLaunchKernelGGL((attn_mla_kernel<576, 512>), dim3(bt.total_q, Hq / 128, pl.n_split), dim3(256), 0, st,
                               bt, (const uint16_t *)q, Hq, (const uint16_t *)k_cache, row_stride, indices, k,
                               (const uint16_t *)gate, per_channel, sl2, (uint16_t *)out, lse, part, pl.n_split,
                               split_len, (const uint16_t *)kmix);
            e = hipGetLastError();
        } else if (d_qk == 576 && d_v == 512 && mla)
            e = launch_bf16<576, 512, true>(bt, pl, q, Hq, k_cache, v_cache, row_stride, indices, k, gate,
                                            per_channel, sl2, out, lse, part, split_len, mix, st);
    } else if (dtype == 0) {
        const dim3 grid(bt.total_q, Hq, pl.n_split);
#define SA_LAUNCH_F32(D)                                                                                         \
    hipLaunchKernelGGL((attn_f32_kernel<D>), grid, dim3(64), 0, st, bt, (const float *)q, Hq,                     \
                       (const float *)k_cache, (const float *)v_cache, row_stride, indices, k, (const float *)gate, \
                       per_channel, sl2, (float *)out, lse, part, pl.n_split, split_len, (const float *)kmix)
        if (d_qk == 32) SA_LAUNCH_F32(32);
        else if (d_qk == 64) SA_LAUNCH_F32(64);
        else SA_LAUNCH_F32(128);
#undef SA_LAUNCH_F32
        e = hipGetLastError();
    }
    if (e != hipSuccess || pl.n_split == 1)
        return e;
    if (pl.n_split > kMaxCombine)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_combine_kernel, dim3(bt.total_q, Hq), dim3(128), 0, st, Hq, d_v, pl.n_split,
                       part, gate, per_channel, dtype == 1 ? 1 : 0, out, lse, mix);
    return hipGetLastError();
}

} // namespace sa
