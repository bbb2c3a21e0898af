// a2 — exact per-token Top-K (gfx950).
//
// Pages (by title):
//   [HAT] "Hybrid Attention Architectures: Engineering Trade-offs from Linear
//          Attention to Gated Sparse Attention", §3.1 (keep the K highest-
//          scoring positions) and §5 item 4 (rows shorter than K are padded).
//   [F2S] "From Full Attention to Sparsity: The Evolution of Hybrid Attention
//          Architectures in Large Language Models", "Fine-Grained Sparse
//          Attention: Indexer Plus Top-K" (indices of shape [n, K]) and
//          "Engineering Considerations" item 1 (variable-length Top-K).
//   [EVO] "Evolution of Hybrid Attention in Open-Source LLMs: From Linear to
//          Gated Sparse Attention", §5 item 3: approximate Top-K breaks
//          train/inference consistency, so selection here is exact.
// Order: (score descending, position ascending); +0 and -0 compare equal.
//
// One workgroup (512 threads) selects from one segment of slots:
//   1. a strided sample (<= 4096 slots) gives a key window [lo, hi];
//   2. a pass over the segment counts slots above the window (registers) and
//      histograms the window into 4096 LDS bins; the bin holding the K-th key
//      narrows the window (a refinement pass repeats this when that bin is
//      still large, at most three times for 32-bit keys);
//   3. an order-preserving pass writes the slots above the window (sure
//      winners) and keeps the window's slots in LDS, both in slot order;
//   4. LDS histograms narrow the kept slots down to the exact K-th key; ties
//      at that key go to the lowest slots;
//   5. the two ascending runs are merged by co-rank and written.
// Keys are the order-preserving uint32 image of the fp32 score.
//
// Long rows first try a single-pass variant (select_topk_fast): a contiguous-
// run sample fixes a conservative threshold and one order-preserving pass
// keeps every slot at or above it in LDS, where step 4 finishes; when the
// kept count misses [K, kCap] the general steps 1-5 run instead (for the rows
// kernel: in a second launch, over the rows the first one marked).
//
// Rows up to a few hundred thousand slots take one workgroup each.  When there
// are too few rows to fill the GPU, each row is cut into chunks selected in
// parallel (stage 1: top-K per chunk, with scores), and a second pass selects
// from the concatenated per-chunk winners (stage 2).  The global top-K is a
// subset of the union of per-chunk top-Ks under the same total order, and the
// chunk lists are concatenated in position order, so slot order is position
// order in both stages.
#include <type_traits>

#include "sa_device.h"
#include "launch.h"

namespace sa {

constexpr int kTkThreads = 512;
static_assert(kTkThreads <= 1024, "misc holds per-wave slots for at most 16 waves");
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kBins = 4096;
constexpr int kCap = 4096;      // LDS slots for the window's candidates
constexpr int kSample = 4096;
constexpr int kSampleBig = 8192;   // single-pass sample on long segments
constexpr int kMaxK = 4096;

__device__ __forceinline__ uint32_t fkey(float v)
{
    uint32_t u = __float_as_uint(v);
    u = (u == 0x80000000u) ? 0u : u;                  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float kval(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int bitlen(uint32_t x) { return x ? 32 - __clz((int)x) : 0; }

struct TkSmem {
    uint32_t *hist;     // [kBins]
    uint32_t *ckey;     // [kCap]
    int32_t *cidx;      // [kCap]
    uint32_t *okey;     // [K]
    int32_t *oidx;      // [K]
    uint32_t *misc;     // [64]
};

// Inclusive scan over the 64 lanes of a wave in the VALU (DPP): shifts by 1,
// 2, 4, 8 within each row of 16 lanes (lanes with no source add 0), then the
// last lane of row 0 (resp. 1) is broadcast into rows 1 and 3 (resp. 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
#define SA_DPP_ADD(ctrl, rmask, bctl) \
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, ctrl, rmask, 0xF, bctl)
    SA_DPP_ADD(0x111, 0xF, true);      // row_shr:1
    SA_DPP_ADD(0x112, 0xF, true);      // row_shr:2
    SA_DPP_ADD(0x114, 0xF, true);      // row_shr:4
    SA_DPP_ADD(0x118, 0xF, true);      // row_shr:8
    SA_DPP_ADD(0x142, 0xA, false);     // row_bcast:15 into rows 1, 3
    SA_DPP_ADD(0x143, 0xC, false);     // row_bcast:31 into rows 2, 3
#undef SA_DPP_ADD
    return x;
}

// Exclusive block scan of v (512 threads); *total gets the block sum.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *misc, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63)
        misc[wv] = x;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
        uint32_t s = misc[w];
        off += (w < wv) ? s : 0u;
        tot += s;
    }
    total = tot;
    __syncthreads();
    return off + x - v;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t *misc)
{
    uint32_t t;
    block_scan(v, misc, t);
    return t;
}

// Minimum and maximum over the 64 lanes of a wave, in the VALU (DPP within
// rows of 16, then v_permlane16_swap and v_permlane32_swap across rows).
__device__ __forceinline__ void wave_minmax(uint32_t &mn, uint32_t &mx)
{
#define SA_DPP_MM(ctrl)                                                                                   \
    mn = min(mn, (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFF, (int)mn, ctrl, 0xF, 0xF, false));  \
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, ctrl, 0xF, 0xF, false))
    SA_DPP_MM(0xB1);                   // quad_perm [1,0,3,2]
    SA_DPP_MM(0x4E);                   // quad_perm [2,3,0,1]
    SA_DPP_MM(0x124);                  // row_ror:4
    SA_DPP_MM(0x128);                  // row_ror:8
#undef SA_DPP_MM
    auto a = __builtin_amdgcn_permlane16_swap(mn, mn, false, false);
    mn = min(a[0], a[1]);
    a = __builtin_amdgcn_permlane32_swap(mn, mn, false, false);
    mn = min(a[0], a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
    mx = max(b[0], b[1]);
    b = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
    mx = max(b[0], b[1]);
}

__device__ __forceinline__ void block_minmax(uint32_t &mn, uint32_t &mx, uint32_t *misc)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    wave_minmax(mn, mx);
    if (lane == 0) {
        misc[16 + wv] = mn;
        misc[32 + wv] = mx;
    }
    __syncthreads();
    mn = 0xFFFFFFFFu;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
        mn = min(mn, misc[16 + w]);
        mx = max(mx, misc[32 + w]);
    }
    __syncthreads();
}

// Bin b of hist[0, NB) with sum(hist[b+1..]) < need <= sum(hist[b..]);
// *gt = sum(hist[b+1..]).  Requires 1 <= need <= sum(hist).  Each thread owns
// NB / 512 consecutive bins.
template <int NB>
__device__ __forceinline__ void find_bin(const TkSmem &sm, uint32_t need, int &b_out, uint32_t &gt_out)
{
    constexpr int BT = NB / kTkThreads;
    static_assert(NB % kTkThreads == 0, "bins per thread");
    const int t = threadIdx.x;
    uint32_t h[BT], local = 0;
#pragma unroll
    for (int j = 0; j < BT; ++j) {
        h[j] = sm.hist[t * BT + j];
        local += h[j];
    }
    uint32_t total;
    const uint32_t excl = block_scan(local, sm.misc, total);
    const uint32_t above = total - excl - local;      // bins owned by higher threads
    if (need > above && need <= above + local) {
        uint32_t acc = above;
#pragma unroll
        for (int j = BT - 1; j >= 0; --j) {
            if (acc + h[j] >= need) {
                sm.misc[48] = (uint32_t)(t * BT + j);
                sm.misc[49] = acc;
                break;
            }
            acc += h[j];
        }
    }
    __syncthreads();
    b_out = (int)sm.misc[48];
    gt_out = sm.misc[49];
    __syncthreads();
}

// Steps 4-5 of a selection: the window's slots (ckey/cidx[0, C), in slot order)
// hold the remaining `need` winners; the sure winners are okey/oidx[0, above),
// in slot order.  Resolves the exact K-th key inside LDS (ties to the lowest
// slots), then merges the two ascending runs into gidx (and gval).
// direct (only with above == 0): the K selected slots go straight to gidx/gval
// in slot order, without the okey/oidx staging.  NB: histogram bins in sm.hist.
template <int NB>
__device__ void finish_select(uint32_t lo, uint32_t hi, uint32_t cnt, uint32_t above, uint32_t need, bool single,
                              int K, int32_t *__restrict__ gidx, float *__restrict__ gval, const TkSmem &sm,
                              bool direct = false)
{
    const int tid = threadIdx.x;
    // ---- 4. resolve the window inside LDS
    if (!single) {
        const int C = (int)min(cnt, (uint32_t)kCap);
        uint32_t wl = lo, wh = hi, needw = need;
        bool all_in = false;
        // each pass narrows a window of width W to at most W / NB (or stops)
        constexpr int LB = __builtin_ctz(NB);
        static_assert((NB & (NB - 1)) == 0, "power-of-two bins");
        for (int pass = 0; pass < (32 + LB - 1) / LB && wl != wh && !all_in; ++pass) {
            const int sh = max(0, bitlen(wh - wl) - LB);
            for (int b = tid; b < NB; b += kTkThreads)
                sm.hist[b] = 0u;
            __syncthreads();
            for (int c = tid; c < C; c += kTkThreads) {
                const uint32_t key = sm.ckey[c];
                if (key >= wl && key <= wh)
                    atomicAdd(&sm.hist[(key - wl) >> sh], 1u);
            }
            __syncthreads();
            int bsel;
            uint32_t gt;
            find_bin<NB>(sm, needw, bsel, gt);
            const uint32_t hb = sm.hist[bsel];
            needw -= gt;
            const uint64_t nlo = (uint64_t)wl + ((uint64_t)bsel << sh);
            wh = (uint32_t)min((uint64_t)wh, nlo + ((1ull << sh) - 1ull));
            wl = (uint32_t)nlo;
            all_in = (hb == needw);
            __syncthreads();
        }
        // ordered selection: keys above the window, then the first needw keys inside it
        uint32_t bsel_ = 0, bwin = 0;
        for (int c0 = 0; c0 < C; c0 += kTkThreads) {
            const int c = c0 + tid;
            const uint32_t key = c < C ? sm.ckey[c] : 0u;
            const bool inw = c < C && key >= wl && key <= wh;
            const bool abv = c < C && key > wh;
            uint32_t tot;
            const uint32_t ex = block_scan((inw ? 1u : 0u) | ((abv ? 1u : 0u) << 16), sm.misc, tot);
            const uint32_t rank_w = bwin + (ex & 0xFFFFu);
            const bool sel = abv || (inw && (all_in || rank_w < needw));
            uint32_t tot2;
            const uint32_t ps = bsel_ + block_scan(sel ? 1u : 0u, sm.misc, tot2);
            if (sel && above + ps < (uint32_t)K) {
                if (direct) {
                    gidx[ps] = sm.cidx[c];
                    if (gval)
                        gval[ps] = kval(key);
                } else {
                    sm.okey[above + ps] = key;
                    sm.oidx[above + ps] = sm.cidx[c];
                }
            }
            bwin += tot & 0xFFFFu;
            bsel_ += tot2;
        }
        __syncthreads();
        if (direct)
            return;
    }

    // ---- 5. merge the two ascending runs [0, above) and [above, K)
    {
        const int A = (int)above, Bn = K - (int)above;
        const int32_t *ra = sm.oidx, *rb = sm.oidx + A;
        for (int i = tid; i < K; i += kTkThreads) {
            const bool inA = i < A;
            const int32_t x = sm.oidx[i];
            const int32_t *other = inA ? rb : ra;
            int lo2 = 0, hi2 = inA ? Bn : A;         // count of `other` elements < x
            while (lo2 < hi2) {
                const int mid = (lo2 + hi2) >> 1;
                if (other[mid] < x)
                    lo2 = mid + 1;
                else
                    hi2 = mid;
            }
            const int p = (inA ? i : i - A) + lo2;
            gidx[p] = x;
            if (gval)
                gval[p] = kval(sm.okey[i]);
        }
    }
}

// One selection problem: n slots with values `vals`; positions are idx0 + j,
// or idxs[j] when idxs != nullptr (then slots with idxs[j] < 0 are empty).
// Writes K entries to gidx (and their scores to gval when non-null): the
// selected positions in ascending order, then -1 (score 0).
template <bool EXPLICIT>
__device__ void select_topk(const float *__restrict__ vals, const int32_t *__restrict__ idxs, int n, int idx0,
                            int K, int32_t *__restrict__ gidx, float *__restrict__ gval, const TkSmem &sm)
{
    const int tid = threadIdx.x;
    auto pos_of = [&](int j) -> int32_t { return EXPLICIT ? idxs[j] : idx0 + j; };
    auto valid = [&](int j) -> bool { return j < n && (!EXPLICIT || idxs[j] >= 0); };

    // ---- number of non-empty slots
    int nvalid = n;
    if (EXPLICIT) {
        uint32_t c = 0;
        for (int j = tid; j < n; j += kTkThreads)
            c += idxs[j] >= 0;
        nvalid = (int)block_sum(c, sm.misc);
    }

    if (nvalid <= K) {
        // everything is selected: slot order is ascending position order
        uint32_t base = 0;
        for (int j0 = 0; j0 < n; j0 += kTkThreads) {
            const int j = j0 + tid;
            const bool v = valid(j);
            uint32_t tot;
            const uint32_t p = base + block_scan(v ? 1u : 0u, sm.misc, tot);
            if (v) {
                gidx[p] = pos_of(j);
                if (gval)
                    gval[p] = vals[j];
            }
            base += tot;
        }
        for (int p = nvalid + tid; p < K; p += kTkThreads) {
            gidx[p] = -1;
            if (gval)
                gval[p] = 0.0f;
        }
        return;
    }

    // ---- 1. sample -> initial window
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    {
        const int S = n < kSample ? n : kSample;
        for (int k = tid; k < S; k += kTkThreads) {
            const int j = (int)(((int64_t)k * n) / S);
            if (valid(j)) {
                const uint32_t key = fkey(vals[j]);
                lo = min(lo, key);
                hi = max(hi, key);
            }
        }
        block_minmax(lo, hi, sm.misc);
        if (lo > hi) {
            lo = 0u;
            hi = 0xFFFFFFFFu;
        }
    }

    // ---- 2. histogram passes over the segment until the K-th key's bin is small
    uint32_t above = 0, cnt = 0;
    for (int iter = 0; iter < 12; ++iter) {
        const int sh = max(0, bitlen(hi - lo) - 12);
        for (int b = tid; b < kBins; b += kTkThreads)
            sm.hist[b] = 0u;
        __syncthreads();
        uint32_t ab = 0;
        const bool aligned = ((((uintptr_t)vals) & 15u) == 0);
        for (int j0 = tid * 4; j0 < n; j0 += kTkThreads * 4) {
            float v4[4];
            if (aligned && j0 + 3 < n) {
                const float4 f = *(const float4 *)(vals + j0);
                v4[0] = f.x; v4[1] = f.y; v4[2] = f.z; v4[3] = f.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v4[e] = (j0 + e < n) ? vals[j0 + e] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (!valid(j0 + e))
                    continue;
                const uint32_t key = fkey(v4[e]);
                if (key > hi)
                    ++ab;
                else if (key >= lo)
                    atomicAdd(&sm.hist[(key - lo) >> sh], 1u);
            }
        }
        above = block_sum(ab, sm.misc);          // also orders the histogram writes
        if (above >= (uint32_t)K) {              // the K-th key lies above the window
            lo = hi + 1u;
            hi = 0xFFFFFFFFu;
            continue;
        }
        const uint32_t need = (uint32_t)K - above;
        uint32_t wtot = 0;
        for (int b = tid; b < kBins; b += kTkThreads)
            wtot += sm.hist[b];
        wtot = block_sum(wtot, sm.misc);
        if (wtot < need) {                       // it lies below the window (lo > 0 here)
            hi = lo - 1u;
            lo = 0u;
            continue;
        }
        int bsel;
        uint32_t gt;
        find_bin<kBins>(sm, need, bsel, gt);
        cnt = sm.hist[bsel];
        const uint64_t nlo = (uint64_t)lo + ((uint64_t)bsel << sh);
        const uint64_t nhi = min((uint64_t)hi, nlo + ((1ull << sh) - 1ull));
        lo = (uint32_t)nlo;
        hi = (uint32_t)nhi;
        above += gt;
        __syncthreads();
        if (cnt <= (uint32_t)kCap || lo == hi)
            break;
    }
    const uint32_t need = (uint32_t)K - above;   // 1 <= need <= cnt
    const bool single = (lo == hi);

    // ---- 3. order-preserving pass: winners to okey/oidx[0, above); window slots kept
    {
        const bool aligned = ((((uintptr_t)vals) & 15u) == 0);
        uint32_t bw = 0, bc = 0;
        for (int j00 = 0; j00 < n; j00 += kTkThreads * 4) {
            const int j0 = j00 + tid * 4;
            float v4[4];
            if (aligned && j0 + 3 < n) {
                const float4 f = *(const float4 *)(vals + j0);
                v4[0] = f.x; v4[1] = f.y; v4[2] = f.z; v4[3] = f.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v4[e] = (j0 + e < n) ? vals[j0 + e] : 0.0f;
            }
            uint32_t kk[4];
            bool w4[4], c4[4];
            uint32_t nw = 0, nc = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool v = valid(j0 + e);
                kk[e] = fkey(v4[e]);
                w4[e] = v && kk[e] > hi;
                c4[e] = v && kk[e] >= lo && kk[e] <= hi;
                nw += w4[e];
                nc += c4[e];
            }
            uint32_t tot;
            const uint32_t ex = block_scan(nw | (nc << 16), sm.misc, tot);
            uint32_t pw = bw + (ex & 0xFFFFu), pc = bc + (ex >> 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (w4[e] && pw < (uint32_t)K) {
                    sm.okey[pw] = kk[e];
                    sm.oidx[pw] = pos_of(j0 + e);
                    ++pw;
                }
                if (c4[e]) {
                    if (single) {
                        if (pc < need) {
                            sm.okey[above + pc] = kk[e];
                            sm.oidx[above + pc] = pos_of(j0 + e);
                        }
                    } else if (pc < (uint32_t)kCap) {
                        sm.ckey[pc] = kk[e];
                        sm.cidx[pc] = pos_of(j0 + e);
                    }
                    ++pc;
                }
            }
            bw += tot & 0xFFFFu;
            bc += tot >> 16;
        }
        __syncthreads();
    }

    finish_select<kBins>(lo, hi, cnt, above, need, single, K, gidx, gval, sm);
}

// A key at most the rank-th largest of keys[0, cnt) (rank >= 1), within a
// factor 1/NB^2 of the keys' range above it: an NB-bin histogram over the keys'
// actual range [min, max] (so the bins, and their LDS atomics, spread out),
// then one over the bin holding that rank.  Returns the lower edge of the final
// bin.
template <int NB>
__device__ uint32_t lds_window_select(const uint32_t *keys, int cnt, uint32_t rank, const TkSmem &sm)
{
    constexpr int LB = __builtin_ctz(NB);
    const int tid = threadIdx.x;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int c = tid; c < cnt; c += kTkThreads) {
        mn = min(mn, keys[c]);
        mx = max(mx, keys[c]);
    }
    block_minmax(mn, mx, sm.misc);
    uint32_t lo = mn, span = mx - mn, need = rank;     // the window [lo, lo + span]
#pragma unroll 1
    for (int lv = 0; lv < 2; ++lv) {
        const int sh = max(0, bitlen(span) - LB);       // (span >> sh) < NB
        for (int b = tid; b < NB; b += kTkThreads)
            sm.hist[b] = 0u;
        __syncthreads();
        for (int c = tid; c < cnt; c += kTkThreads) {
            const uint32_t k = keys[c];
            if (k >= lo && k - lo <= span)
                atomicAdd(&sm.hist[(k - lo) >> sh], 1u);
        }
        __syncthreads();
        int b;
        uint32_t gt;
        find_bin<NB>(sm, need, b, gt);
        need -= gt;
        lo += (uint32_t)b << sh;
        if (sh == 0)
            break;
        span = (1u << sh) - 1u;                         // the chosen bin
    }
    return lo;
}

// Single-pass selection for long rows (slot j has position idx0 + j).  A
// sample of 64 (128 on long rows) runs of 64 consecutive slots, spread evenly
// over the row, gives a threshold: the sample key whose rank is the K-th key's
// expected rank in the sample plus about four standard deviations, so that the
// row's slots at or above it very likely number between K and kCap.  One
// order-preserving pass keeps exactly those slots in LDS (slot order); the
// exact K-th key and its ties are then resolved there and the K winners
// written out.  Returns false, having written nothing, when the kept count
// falls outside [K, kCap] (or a wave's share overflows its LDS region); the
// caller then runs the general selection, so the result never depends on the
// sample.  NB: histogram bins at sm.hist (the pair area is ckey, cidx and those
// bins); TD: wave steps of loads in flight.
template <int NB, int TD>
__device__ bool select_topk_fast(const float *__restrict__ vals, int n, bool pad4, int idx0, int K,
                                 int32_t *__restrict__ gidx, float *__restrict__ gval, const TkSmem &sm)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (n < kSample || n >= (1 << 25) || !pad4 || (((uintptr_t)vals) & 15u) != 0)
        return false;
    // the sample: 64 runs, or 128 on segments of at least 16 runs per wave
    // step (the K-th key's expected rank in it then doubles, so the same
    // relative margin keeps fewer slots)
    const bool big = n >= 4 * kSampleBig;
    const int S = big ? kSampleBig : kSample;
    const float rexp = (float)K * (float)S / (float)n;
    const int rlow = (int)(rexp + 4.0f * sqrtf(rexp) + 4.0f) + 1;
    if (rlow >= S)
        return false;

    // ---- 2. one pass, streamed per wave: wave w scans its own contiguous chunk
    // of the segment in slot order and appends the slots with key >= thr to its
    // own LDS region (RC slots); the regions, concatenated in wave order, hold
    // the kept slots in slot order.  The pass has no barrier: each wave keeps
    // TD steps of loads in flight, and its compaction is a lane prefix count
    // from ballots (no LDS traffic).  A region that overflows sends the
    // segment to the general path.
    constexpr int WST = 1024;                   // slots per wave step: 4 runs of 64 lanes x 4
    constexpr int PC = kCap + NB / 2;           // (key, index) pairs in ckey, cidx, hist
    constexpr int RC = PC / kTkWaves;           // region pairs per wave
    static_assert(PC % kTkThreads == 0, "concatenation: every thread moves PC / kTkThreads pairs");
    const int wchunk = (n + kTkWaves * WST - 1) / (kTkWaves * WST) * WST;
    const int c0 = min(n, wv * wchunk), c1 = min(n, c0 + wchunk);
    // every wave runs the same number of steps, a multiple of TD, so that the
    // loop has one path and the compiler's waits count TD steps in flight
    const int nsteps = (wchunk / WST + TD - 1) / TD * TD;
    // step s of this lane: slots c0 + s*WST + 256u + 4*lane + q, u, q = 0..3,
    // read as 16-byte loads without branches (so the compiler's waits can count
    // the loads in flight).  jmax is the group holding the chunk's last slot; a
    // group past it rereads it (a line already fetched) and its slots are
    // masked out below.  Reading that whole group needs the segment to be
    // readable up to a multiple of 4 slots (the caller's pad4 guarantee).
    const int jmax = ((c1 > c0 ? c1 : n) - 1) & ~3;
    auto load = [&](int s, float (&v)[16]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = min(c0 + s * WST + 256 * u + 4 * lane, jmax);
            const float4 f = *(const float4 *)(vals + j);
            v[4 * u] = f.x;
            v[4 * u + 1] = f.y;
            v[4 * u + 2] = f.z;
            v[4 * u + 3] = f.w;
        }
    };
    // the pass's first loads do not depend on the threshold: TD - 1 steps are
    // issued now, so that they arrive while the sample is selected
    float buf[TD][16];
#pragma unroll
    for (int d = 0; d < TD - 1; ++d)
        load(d, buf[d]);

    // ---- 1. sample -> threshold (the sample sits in the pair area)
    auto sample = [&](auto runs_c) {
        constexpr int RUNS = decltype(runs_c)::value;
        // all of the wave's runs in flight at once
        float sv[RUNS / kTkWaves];
#pragma unroll
        for (int i = 0; i < RUNS / kTkWaves; ++i) {
            const int r = wv + kTkWaves * i;
            // (32-bit: r * (n - 64) < 2^32 for n < 2^25; the division by a
            // constant is a multiply-high)
            sv[i] = vals[(int)(((uint32_t)r * (uint32_t)(n - 64)) / (uint32_t)(RUNS - 1)) + lane];
        }
#pragma unroll
        for (int i = 0; i < RUNS / kTkWaves; ++i)
            sm.ckey[(wv + kTkWaves * i) * 64 + lane] = fkey(sv[i]);
    };
    static_assert(kSampleBig <= 2 * kCap, "the sample fits in ckey and cidx");
    if (big)
        sample(std::integral_constant<int, kSampleBig / 64>{});
    else
        sample(std::integral_constant<int, kSample / 64>{});
    __syncthreads();
    // (a threshold a little below the exact sample key only keeps a few more
    // slots)
    const uint32_t thr = lds_window_select<NB>(sm.ckey, S, (uint32_t)rlow, sm);

    u32x2 *const pairs = (u32x2 *)sm.ckey;     // the pair area (ckey, cidx, hist)
    u32x2 *rgn = pairs + wv * RC;
    uint32_t wcount = 0;                        // kept slots of this wave so far
    auto keep = [&](int s, const float (&v)[16]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = c0 + s * WST + 256 * u + 4 * lane;
            uint32_t kk[4], m = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                kk[q] = fkey(v[4 * u + q]);
                if (j + q < c1 && kk[q] >= thr)
                    m |= 1u << q;
            }
            // exclusive prefix over lanes of the per-lane counts (0..4), bit-sliced
            const int c = __popc(m);
            const uint64_t b0 = __ballot(c & 1), b1 = __ballot(c & 2), b2 = __ballot(c & 4);
            if ((b0 | b1 | b2) == 0)
                continue;
            auto below = [](uint64_t b) {
                return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            };
            uint32_t p = wcount + below(b0) + 2u * below(b1) + 4u * below(b2);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if ((m >> q) & 1u) {
                    if (p < (uint32_t)RC)
                        rgn[p] = u32x2{kk[q], (uint32_t)(idx0 + j + q)};
                    ++p;
                }
            wcount += (uint32_t)(__popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2));
        }
    };
    load(TD - 1, buf[TD - 1]);
    for (int s0 = 0; s0 < nsteps; s0 += TD) {
#pragma unroll
        for (int d = 0; d < TD; ++d) {
            keep(s0 + d, buf[d]);
            load(s0 + d + TD, buf[d]);
        }
    }
    if (lane == 0)
        sm.misc[wv] = wcount;
    __syncthreads();
    uint32_t cnt[kTkWaves], pfx[kTkWaves], base = 0;
    bool ovf = false;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
        cnt[w] = sm.misc[w];
        pfx[w] = base;
        base += cnt[w];
        ovf |= cnt[w] > (uint32_t)RC;
    }
    if (ovf || base < (uint32_t)K || base > (uint32_t)kCap)
        return false;
    // concatenate the regions in wave order into ckey/cidx[0, base) (all reads,
    // then all writes: the pair area overlaps its destination)
    constexpr int PT = PC / kTkThreads;
    u32x2 pv[PT];
    int dst[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int g = tid + kTkThreads * i, w = g / RC, o = g - w * RC;
        dst[i] = -1;
#pragma unroll
        for (int x = 0; x < kTkWaves; ++x)
            if (x == w && (uint32_t)o < cnt[x])
                dst[i] = (int)pfx[x] + o;
        if (dst[i] >= 0)
            pv[i] = pairs[g];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PT; ++i)
        if (dst[i] >= 0) {
            sm.ckey[dst[i]] = pv[i].x;
            sm.cidx[dst[i]] = (int32_t)pv[i].y;
        }
    __syncthreads();
    // ---- 3. exact K-th key among the kept slots (all K winners are among them)
    // the window [thr, largest kept key] (no kept key is above it), so that the
    // finish's histograms spread over the keys' actual range
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
    for (int c = tid; c < (int)base; c += kTkThreads)
        kmx = max(kmx, sm.ckey[c]);
    block_minmax(kmn, kmx, sm.misc);
    finish_select<NB>(thr, kmx, base, 0u, (uint32_t)K, false, K, gidx, gval, sm, true);
    return true;
}

// Both layouts start with ckey, cidx, hist back to back: during its pass the
// single-pass selection uses those 2*kCap + kBins words as one area of
// (key, index) pairs.
__device__ __forceinline__ TkSmem tk_smem(int K)
{
    extern __shared__ __align__(16) uint32_t tk_lds[];
    TkSmem sm;
    sm.ckey = tk_lds;
    sm.cidx = (int32_t *)(sm.ckey + kCap);
    sm.hist = (uint32_t *)(sm.cidx + kCap);
    sm.okey = sm.hist + kBins;
    sm.oidx = (int32_t *)(sm.okey + ((K + 3) & ~3));
    sm.misc = (uint32_t *)(sm.oidx + ((K + 3) & ~3));
    return sm;
}

static size_t tk_smem_bytes(int K)
{
    return (size_t)(kBins + 2 * kCap + 2 * ((K + 3) & ~3) + 64) * 4;
}

// The single pass alone needs no output staging (its selection is written
// straight out): 48.25 KB, three workgroups per CU instead of two.  (With
// 1024-bin histograms, 36.25 KB, and two steps of loads in flight, four fit;
// measured at the benchmark that was 2% slower: the selects need one more
// histogram level and the pass has fewer loads in flight.)
__device__ __forceinline__ TkSmem tk_smem_fast()
{
    extern __shared__ __align__(16) uint32_t tk_lds[];
    TkSmem sm;
    sm.ckey = tk_lds;
    sm.cidx = (int32_t *)(sm.ckey + kCap);
    sm.hist = (uint32_t *)(sm.cidx + kCap);
    sm.misc = sm.hist + kBins;
    sm.okey = nullptr;
    sm.oidx = nullptr;
    return sm;
}

constexpr size_t kTkSmemFast = (size_t)(kBins + 2 * kCap + 64) * 4;
constexpr int32_t kTkPending = INT32_MIN;   // first output slot of a row left to the general path

// One workgroup per token row, in two launches: the single pass first (small
// LDS, more workgroups per CU); a row it cannot finish gets kTkPending in its
// first output slot and is selected by the general path in the second launch,
// whose workgroups return at once for every other row.
// A row's length: pos + 1 scores of positions (len_shift 0), or the
// (pos >> len_shift) + 1 scores of the blocks of 2^len_shift positions that
// start at or before pos.
__device__ __forceinline__ int row_length(const Batch &bt, int row, int len_shift)
{
    const int b = seq_of_token(bt, row);
    return (pos_of_token(bt, b, row) >> len_shift) + 1;
}

__global__ __launch_bounds__(kTkThreads) void topk_rows_fast_kernel(Batch bt, const float *__restrict__ scores,
                                                                    int64_t ld, int K, int32_t *__restrict__ out,
                                                                    int len_shift)
{
    // last rows first: the scores a preceding indexer wrote last may still be in the cache
    const int row = gridDim.x - 1 - blockIdx.x;
    const int n = row_length(bt, row, len_shift);
    const TkSmem sm = tk_smem_fast();
    const float *vals = scores + (int64_t)row * ld;
    int32_t *o = out + (int64_t)row * K;
    // rows start 16-byte aligned and can be read up to a multiple of 4 slots
    // when the row stride is a multiple of 4 floats
    if (!select_topk_fast<kBins, 3>(vals, n, (ld & 3) == 0, 0, K, o, nullptr, sm) && threadIdx.x == 0)
        o[0] = kTkPending;
}

// Fewer than 256 rows (the GPU is not filled either way): the single pass and,
// for a row it cannot finish, the general path in the same workgroup, which then
// holds the general path's LDS: one launch instead of two.
__global__ __launch_bounds__(kTkThreads) void topk_rows_one_kernel(Batch bt, const float *__restrict__ scores,
                                                                   int64_t ld, int K, int32_t *__restrict__ out,
                                                                   int len_shift)
{
    const int row = blockIdx.x;
    const int n = row_length(bt, row, len_shift);
    const TkSmem sm = tk_smem(K);
    const float *vals = scores + (int64_t)row * ld;
    int32_t *o = out + (int64_t)row * K;
    if (!select_topk_fast<kBins, 3>(vals, n, (ld & 3) == 0, 0, K, o, nullptr, sm))
        select_topk<false>(vals, nullptr, n, 0, K, o, nullptr, sm);
}

// Rows of up to 512 * PER slots, one workgroup each, in one launch: the row is
// loaded once into registers (thread t holds the 4-slot groups t, t + 512, ...,
// so every load is coalesced), the K-th largest key is found by three LDS
// histogram levels over its bits (12, 12 and 8), and the winners are written in
// slot order: one block scan per round of groups counts, before each thread,
// the keys above the K-th and the keys equal to it (ties go to the lowest
// positions).
template <int PER>
__global__ __launch_bounds__(kTkThreads) void topk_rows_reg_kernel(Batch bt, const float *__restrict__ scores,
                                                                   int64_t ld, int K, int32_t *__restrict__ out,
                                                                   int len_shift)
{
    static_assert(PER % 4 == 0, "4-slot groups");
    constexpr int G = PER / 4;                  // groups per thread
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t misc[64];
    TkSmem sm;
    sm.hist = hist;
    sm.misc = misc;
    // last rows first: in causal prefill they are the longest (the short rows fill
    // the tail), and the scores a preceding indexer wrote last may still be cached
    const int row = gridDim.x - 1 - blockIdx.x, tid = threadIdx.x;
    const int n = row_length(bt, row, len_shift);
    const float *vals = scores + (int64_t)row * ld;
    int32_t *o = out + (int64_t)row * K;
    if (n <= K) {
        // every slot is selected: position j goes to output j, the rest is -1
        for (int j = tid; j < K; j += kTkThreads)
            o[j] = j < n ? j : -1;
        return;
    }
    const bool v4 = (ld & 3) == 0 && (((uintptr_t)vals) & 15u) == 0;
    uint32_t key[G][4];
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int j = 4 * (tid + kTkThreads * u);
        float f[4];
        if (v4 && j + 3 < n) {
            const float4 x = *(const float4 *)(vals + j);
            f[0] = x.x;
            f[1] = x.y;
            f[2] = x.z;
            f[3] = x.w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                f[q] = j + q < n ? vals[j + q] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            key[u][q] = j + q < n ? fkey(f[q]) : 0u;      // 0: below every finite score's key
    }
    // ---- the K-th largest key, 12 + 12 + 8 bits
    uint32_t prefix = 0u, need = (uint32_t)K;
    const int shifts[3] = {20, 8, 0};
    const uint32_t masks[3] = {0xFFFu, 0xFFFu, 0xFFu};
#pragma unroll
    for (int lv = 0; lv < 3; ++lv) {
        const int sh = shifts[lv];
        for (int b = tid; b < kBins; b += kTkThreads)
            hist[b] = 0u;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < G; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = 4 * (tid + kTkThreads * u) + q;
                const uint32_t k = key[u][q];
                // keys whose bits above this level match the prefix found so far
                if (j < n && (lv == 0 || (k >> (sh + (lv == 1 ? 12 : 8))) == prefix))
                    atomicAdd(&hist[(k >> sh) & masks[lv]], 1u);
            }
        __syncthreads();
        int b;
        uint32_t gt;
        find_bin<kBins>(sm, need, b, gt);
        need -= gt;
        prefix = (prefix << (lv == 0 ? 12 : (lv == 1 ? 12 : 8))) | (uint32_t)b;
    }
    const uint32_t kth = prefix;                // the K-th largest key
    const uint32_t ties = need;                 // keys equal to it that are taken (lowest positions)
    // ---- winners in slot order
    uint32_t above_done = 0, ties_done = 0;     // before this group of slots, over the whole block
#pragma unroll
    for (int u = 0; u < G; ++u) {
        const int j = 4 * (tid + kTkThreads * u);
        uint32_t a = 0, e = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool ok = j + q < n;
            a += ok && key[u][q] > kth;
            e += ok && key[u][q] == kth;
        }
        uint32_t tot;
        const uint32_t ex = block_scan(a | (e << 16), misc, tot);
        uint32_t ab = above_done + (ex & 0xFFFFu), tb = ties_done + (ex >> 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (j + q >= n)
                continue;
            const uint32_t k = key[u][q];
            if (k > kth || (k == kth && tb < ties)) {
                o[ab + min(tb, ties)] = j + q;
            }
            ab += k > kth;
            tb += k == kth;
        }
        above_done += tot & 0xFFFFu;
        ties_done += tot >> 16;
    }
}

__global__ __launch_bounds__(kTkThreads) void topk_rows_kernel(Batch bt, const float *__restrict__ scores,
                                                               int64_t ld, int K, int32_t *__restrict__ out,
                                                               int len_shift)
{
    const int row = blockIdx.x;
    int32_t *o = out + (int64_t)row * K;
    if (o[0] != kTkPending)     // (read by every thread before any is written)
        return;
    const int n = row_length(bt, row, len_shift);
    const TkSmem sm = tk_smem(K);
    const float *vals = scores + (int64_t)row * ld;
    select_topk<false>(vals, nullptr, n, 0, K, o, nullptr, sm);
}

// Stage 1: blockIdx.x = chunk, blockIdx.y = row; per-chunk top-K with scores.
__global__ __launch_bounds__(kTkThreads) void topk_chunk_kernel(Batch bt, const float *__restrict__ scores,
                                                                int64_t ld, int K, int chunk, int64_t cand_ld,
                                                                int32_t *__restrict__ cidx, float *__restrict__ cval,
                                                                int len_shift)
{
    const int c = blockIdx.x, row = blockIdx.y;
    const int n = row_length(bt, row, len_shift);
    const int j0 = c * chunk;
    const int len = max(0, min(chunk, n - j0));
    const int64_t o = (int64_t)row * cand_ld + (int64_t)c * K;
    const TkSmem sm = tk_smem(K);
    const float *vals = scores + (int64_t)row * ld + j0;
    if (!select_topk_fast<kBins, 3>(vals, len, (ld & 3) == 0, j0, K, cidx + o, cval + o, sm))
        select_topk<false>(vals, nullptr, len, j0, K, cidx + o, cval + o, sm);
}

// Stage 2: blockIdx.y = row, blockIdx.x = group: the top K of the group's
// candidates [g*gc, min(n_cand, (g+1)*gc)) of the row, written at
// row*out_ld + g*K (values too when oval is set).  With many chunks a first
// level merges groups of chunk lists in parallel and a second level merges
// the group winners; both keep position order, so ties still go to the lower
// position.
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(int K, int n_cand, int gc, int64_t cand_ld,
                                                                const int32_t *__restrict__ cidx,
                                                                const float *__restrict__ cval, int64_t out_ld,
                                                                int32_t *__restrict__ oidx, float *__restrict__ oval)
{
    const int g = blockIdx.x, row = blockIdx.y;
    const int64_t o = (int64_t)row * cand_ld + (int64_t)g * gc;
    const int len = min(gc, n_cand - g * gc);
    const int64_t w = (int64_t)row * out_ld + (int64_t)g * K;
    select_topk<true>(cval + o, cidx + o, len, 0, K, oidx + w, oval ? oval + w : nullptr, tk_smem(K));
}

// ---------------------------------------------------------------- few long rows
// A row of up to millions of slots, with too few rows to fill the GPU: a
// threshold from a large sample of the row, a compaction of each chunk to the
// slots at or above it, and the exact selection among those in one workgroup
// per row.  As in the single-pass selection the threshold is the sample key
// whose rank is the K-th key's expected rank in the sample plus about four
// standard deviations, so that the kept slots very likely number between K
// and kCap; the result never depends on the sample: a row whose kept count
// falls outside [K, kCap] (or a chunk that keeps more than kThrCap slots) is
// selected from its scores by the single-workgroup path instead.
constexpr int kThrRuns = 512;           // sample: runs of 64 consecutive slots
constexpr int kThrSample = kThrRuns * 64;
constexpr int kThrCap = 1024;           // kept (key, position) pairs a chunk may write
constexpr int kThrWaveCap = kThrCap / kTkWaves;

// The sample's keys, streamed twice from memory (L2 the second time): the
// window of keys at or below the rlow-th largest, to 1/NB^2 of the keys' range.
__global__ __launch_bounds__(kTkThreads) void topk_thr_kernel(Batch bt, const float *__restrict__ scores,
                                                              int64_t ld, int K, uint32_t *__restrict__ thr,
                                                              int len_shift)
{
    const int row = blockIdx.x;
    const int n = row_length(bt, row, len_shift);
    const TkSmem sm = tk_smem_fast();
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const float rexp = (float)K * (float)kThrSample / (float)max(n, 1);
    const int rlow = (int)(rexp + 4.0f * sqrtf(rexp) + 4.0f) + 1;
    if (n < 4 * kThrSample || n >= (1 << 30) || rlow >= kThrSample) {
        if (tid == 0)
            thr[row] = 0u;              // not thresholded: the finish selects from the scores
        return;
    }
    const float *vals = scores + (int64_t)row * ld;
    // every run value of this lane loaded at once, kept as keys in registers
    constexpr int RPW = kThrRuns / kTkWaves;
    uint32_t kv[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = wv + kTkWaves * i;
        kv[i] = fkey(vals[(int64_t)r * (n - 64) / (kThrRuns - 1) + lane]);
    }
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        mn = min(mn, kv[i]);
        mx = max(mx, kv[i]);
    }
    block_minmax(mn, mx, sm.misc);
    uint32_t lo = mn, span = mx - mn, need = (uint32_t)rlow;
    constexpr int LB = __builtin_ctz(kBins);
#pragma unroll 1
    for (int lv = 0; lv < 2; ++lv) {
        const int sh = max(0, bitlen(span) - LB);
        for (int b = tid; b < kBins; b += kTkThreads)
            sm.hist[b] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RPW; ++i)
            if (kv[i] >= lo && kv[i] - lo <= span)
                atomicAdd(&sm.hist[(kv[i] - lo) >> sh], 1u);
        __syncthreads();
        int b;
        uint32_t gt;
        find_bin<kBins>(sm, need, b, gt);
        need -= gt;
        lo += (uint32_t)b << sh;
        if (sh == 0)
            break;
        span = (1u << sh) - 1u;
    }
    if (tid == 0)
        thr[row] = max(lo, 1u);
}

// One workgroup per (chunk, row): the chunk's slots with key >= thr, in slot
// order, as (key, position) pairs; count -1 when the row is not thresholded or
// the chunk keeps more than kThrCap.  Wave w scans its own contiguous share in
// steps of 256 slots with every load of the share in flight, compacts by lane
// prefix counts from ballots into its LDS region, and the regions leave in wave
// order.
__global__ __launch_bounds__(kTkThreads) void topk_thr_chunk_kernel(Batch bt, const float *__restrict__ scores,
                                                                    int64_t ld, int chunk, int n_chunks,
                                                                    const uint32_t *__restrict__ thr,
                                                                    int32_t *__restrict__ counts,
                                                                    u32x2 *__restrict__ pairs, int len_shift)
{
    const int c = blockIdx.x, row = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = row_length(bt, row, len_shift);
    const int j0 = c * chunk;
    const int len = max(0, min(chunk, n - j0));
    const uint32_t t = thr[row];
    int32_t *cnt = counts + (int64_t)row * n_chunks + c;
    if (t == 0u) {
        if (tid == 0)
            *cnt = -1;
        return;
    }
    __shared__ u32x2 rgn[kTkWaves][kThrWaveCap];
    __shared__ uint32_t wcnt[kTkWaves];
    const float *vals = scores + (int64_t)row * ld + j0;
    // wave shares of whole 256-slot steps; a slot past the chunk is masked, and
    // its load clamped to the chunk's last slot
    constexpr int STEP = 256, MAXS = 8;     // at most 8 steps per wave: chunks up to 16384 slots
    const int share = (len + kTkWaves * STEP - 1) / (kTkWaves * STEP) * STEP;
    const int s0 = wv * share;
    float v[MAXS][4];
    const bool v4 = (ld & 3) == 0;          // rows 16-byte aligned and readable to a multiple of 4 slots
#pragma unroll
    for (int st = 0; st < MAXS; ++st) {
        const int j = s0 + st * STEP + 4 * lane;
        const bool in = st * STEP < share && j < len;
        if (v4) {
            const float4 f = in ? *(const float4 *)(vals + j) : float4{0.f, 0.f, 0.f, 0.f};
            v[st][0] = f.x;
            v[st][1] = f.y;
            v[st][2] = f.z;
            v[st][3] = f.w;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[st][q] = (in && j + q < len) ? vals[j + q] : 0.0f;
        }
    }
    uint32_t wc = 0;
#pragma unroll
    for (int st = 0; st < MAXS; ++st) {
        if (st * STEP >= share)
            break;
        const int j = s0 + st * STEP + 4 * lane;
        uint32_t kk[4], m = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            kk[q] = fkey(v[st][q]);
            if (j + q < len && kk[q] >= t)
                m |= 1u << q;
        }
        const int cq = __popc(m);
        const uint64_t b0 = __ballot(cq & 1), b1 = __ballot(cq & 2), b2 = __ballot(cq & 4);
        if ((b0 | b1 | b2) == 0)
            continue;
        auto below = [](uint64_t b) {
            return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        };
        uint32_t p = wc + below(b0) + 2u * below(b1) + 4u * below(b2);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if ((m >> q) & 1u) {
                if (p < (uint32_t)kThrWaveCap)
                    rgn[wv][p] = u32x2{kk[q], (uint32_t)(j0 + j + q)};
                ++p;
            }
        wc += (uint32_t)(__popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2));
    }
    if (lane == 0)
        wcnt[wv] = wc;
    __syncthreads();
    uint32_t base = 0, total = 0;
    bool ovf = false;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
        const uint32_t x = wcnt[w];
        base += w < wv ? x : 0u;
        total += x;
        ovf |= x > (uint32_t)kThrWaveCap;
    }
    u32x2 *out = pairs + ((int64_t)row * n_chunks + c) * kThrCap;
    if (!ovf)
        for (uint32_t i = lane; i < wc; i += 64)
            out[base + i] = rgn[wv][i];
    if (tid == 0)
        *cnt = ovf ? -1 : (int32_t)total;
}

// One workgroup per row: the chunks' kept pairs, concatenated in chunk order
// (slot order), hold the row's top K when their count is in [K, kCap]; else the
// row is selected from its scores.
__global__ __launch_bounds__(kTkThreads) void topk_thr_finish_kernel(Batch bt, const float *__restrict__ scores,
                                                                     int64_t ld, int K, int n_chunks,
                                                                     const uint32_t *__restrict__ thr,
                                                                     const int32_t *__restrict__ counts,
                                                                     const u32x2 *__restrict__ pairs,
                                                                     int32_t *__restrict__ out, int len_shift)
{
    const int row = blockIdx.x, tid = threadIdx.x;
    const int n = row_length(bt, row, len_shift);
    const TkSmem sm = tk_smem(K);
    int32_t *o = out + (int64_t)row * K;
    const float *vals = scores + (int64_t)row * ld;
    const int32_t *cr = counts + (int64_t)row * n_chunks;
    // chunk counts (a thread per chunk): total, validity and each chunk's offset
    __shared__ uint32_t coff[kTkThreads + 1];
    const int32_t x = tid < n_chunks ? cr[tid] : 0;
    const uint32_t bad = __syncthreads_or(x < 0);
    uint32_t tot;
    const uint32_t ex = block_scan(x > 0 ? (uint32_t)x : 0u, sm.misc, tot);
    if (bad || tot < (uint32_t)K || tot > (uint32_t)kCap) {
        if (!select_topk_fast<kBins, 3>(vals, n, (ld & 3) == 0, 0, K, o, nullptr, sm))
            select_topk<false>(vals, nullptr, n, 0, K, o, nullptr, sm);
        return;
    }
    if (tid < n_chunks)
        coff[tid] = ex;
    if (tid == 0)
        coff[n_chunks] = tot;
    __syncthreads();
    // kept pair i sits in the last chunk whose offset is <= i
    uint32_t kmx = 0u;
    for (uint32_t i = tid; i < tot; i += kTkThreads) {
        int lo_ = 0, hi_ = n_chunks - 1;
        while (lo_ < hi_) {
            const int mid = (lo_ + hi_ + 1) >> 1;
            if (coff[mid] <= i)
                lo_ = mid;
            else
                hi_ = mid - 1;
        }
        const u32x2 pr = pairs[((int64_t)row * n_chunks + lo_) * kThrCap + (i - coff[lo_])];
        sm.ckey[i] = pr.x;
        sm.cidx[i] = (int32_t)pr.y;
        kmx = max(kmx, pr.x);
    }
    uint32_t kmn = 0xFFFFFFFFu;
    block_minmax(kmn, kmx, sm.misc);
    finish_select<kBins>(thr[row], kmx, tot, 0u, (uint32_t)K, false, K, o, nullptr, sm, true);
}

TopkPlan topk_plan(int total_q, int max_ctx, int k)
{
    TopkPlan p{0, 0, 1, 1, 0, 0, 0};
    // rows of up to 8192 slots: one launch, each row held in registers (8192
    // rows of up to 8192: 0.103 ms against 0.201 for the single pass and the
    // general path; 64 rows of 8K-32K at 64 slots per thread took 0.037 ms
    // against 0.029: too few workgroups)
    if (max_ctx <= 512 * 16) {
        p.reg = 16;
        return p;
    }
    // Few rows cannot fill 256 CUs: cut long rows into chunks.  Rows of up to
    // 64K positions are still faster whole, one workgroup each (64 rows of
    // 8K-32K: 0.024 ms against 0.043 chunked and merged).  With k <= kCap / 2
    // the chunks are compacted against a per-row sampled threshold (about 512
    // workgroups of up to 16384 slots); otherwise each chunk's top k is
    // selected (chunks >= 4 k) and the lists merged.
    if (total_q < 256 && max_ctx > 65536 && 2 * k <= kCap && max_ctx <= kTkThreads * 16384) {
        int chunk = (int)(((int64_t)max_ctx * total_q + 511) / 512);
        chunk = min(16384, max(4096, (chunk + 1023) / 1024 * 1024));
        p.chunked = 1;
        p.thr = 1;
        p.chunk = chunk;
        p.n_chunks = (max_ctx + chunk - 1) / chunk;
        p.group = p.n_chunks;
        const size_t a = ((size_t)total_q * 4 + 255) / 256 * 256;
        const size_t b = ((size_t)total_q * p.n_chunks * 4 + 255) / 256 * 256;
        p.ws_bytes = a + b + (size_t)total_q * p.n_chunks * kThrCap * 8;
        return p;
    }
    if (total_q < 256 && max_ctx > 65536) {
        const int want_chunks = (512 + total_q - 1) / total_q;
        int chunk = (max_ctx + want_chunks - 1) / want_chunks;
        chunk = max(chunk, max(4 * k, 8192));
        chunk = (chunk + 1023) / 1024 * 1024;
        const int n_chunks = (max_ctx + chunk - 1) / chunk;
        if (n_chunks > 1) {
            p.chunked = 1;
            p.chunk = chunk;
            p.n_chunks = n_chunks;
            // one merge workgroup per row over every chunk list leaves most CUs
            // idle when the lists are many: merge groups of about sqrt(n_chunks)
            // lists first
            int group = n_chunks;
            if (n_chunks >= 8) {
                group = 1;
                while (group * group < n_chunks)
                    ++group;
            }
            p.group = group;
            const int n_groups = (n_chunks + group - 1) / group;
            const int64_t cand_ld = ((int64_t)n_chunks * k + 63) / 64 * 64;
            const int64_t cand2_ld = n_groups > 1 ? ((int64_t)n_groups * k + 63) / 64 * 64 : 0;
            p.ws_bytes = (size_t)total_q * (size_t)(cand_ld + cand2_ld) * 8u;
        }
    }
    return p;
}

hipError_t launch_topk(const Batch &bt, const TopkPlan &plan, const float *scores, int64_t ld, int k,
                       int32_t *indices, void *ws, hipStream_t st, int len_shift)
{
    if (k < 1 || k > kMaxK)
        return hipErrorInvalidValue;
    const size_t smem = tk_smem_bytes(k);
    if (smem > 65536) {
        // above the default dynamic-LDS limit: raise it for the kernels this plan launches
        if (hipFuncSetAttribute((const void *)topk_rows_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)smem) != hipSuccess ||
            hipFuncSetAttribute((const void *)topk_rows_one_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)smem) != hipSuccess ||
            hipFuncSetAttribute((const void *)topk_chunk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)smem) != hipSuccess ||
            hipFuncSetAttribute((const void *)topk_merge_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)smem) != hipSuccess)
            return hipErrorInvalidValue;
    }
    if (plan.reg) {
        hipLaunchKernelGGL((topk_rows_reg_kernel<16>), dim3(bt.total_q), dim3(kTkThreads), 0, st, bt, scores, ld, k,
                           indices, len_shift);
        return hipGetLastError();
    }
    if (plan.thr) {
        if (bt.total_q > 65535)
            return hipErrorInvalidValue;
        if (smem > 65536 && hipFuncSetAttribute((const void *)topk_thr_finish_kernel,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
            return hipErrorInvalidValue;
        uint32_t *thr = (uint32_t *)ws;
        int32_t *counts = (int32_t *)((char *)ws + ((size_t)bt.total_q * 4 + 255) / 256 * 256);
        u32x2 *pairs = (u32x2 *)((char *)counts + ((size_t)bt.total_q * plan.n_chunks * 4 + 255) / 256 * 256);
        hipLaunchKernelGGL(topk_thr_kernel, dim3(bt.total_q), dim3(kTkThreads), kTkSmemFast, st, bt, scores, ld, k,
                           thr, len_shift);
        hipLaunchKernelGGL(topk_thr_chunk_kernel, dim3(plan.n_chunks, bt.total_q), dim3(kTkThreads), 0, st, bt,
                           scores, ld, plan.chunk, plan.n_chunks, (const uint32_t *)thr, counts, pairs, len_shift);
        hipLaunchKernelGGL(topk_thr_finish_kernel, dim3(bt.total_q), dim3(kTkThreads), smem, st, bt, scores, ld, k,
                           plan.n_chunks, (const uint32_t *)thr, (const int32_t *)counts, (const u32x2 *)pairs,
                           indices, len_shift);
        return hipGetLastError();
    }
    if (!plan.chunked && bt.total_q < 256) {
        hipLaunchKernelGGL(topk_rows_one_kernel, dim3(bt.total_q), dim3(kTkThreads), smem, st, bt, scores, ld, k,
                           indices, len_shift);
        return hipGetLastError();
    }
    if (!plan.chunked) {
        hipLaunchKernelGGL(topk_rows_fast_kernel, dim3(bt.total_q), dim3(kTkThreads), kTkSmemFast, st, bt, scores,
                           ld, k, indices, len_shift);
        hipLaunchKernelGGL(topk_rows_kernel, dim3(bt.total_q), dim3(kTkThreads), smem, st, bt, scores, ld, k,
                           indices, len_shift);
        return hipGetLastError();
    }
    const int64_t cand_ld = ((int64_t)plan.n_chunks * k + 63) / 64 * 64;
    int32_t *cidx = (int32_t *)ws;
    float *cval = (float *)((char *)ws + (size_t)bt.total_q * (size_t)cand_ld * 4u);
    if (bt.total_q > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(plan.n_chunks, bt.total_q), dim3(kTkThreads), smem, st, bt, scores,
                       ld, k, plan.chunk, cand_ld, cidx, cval, len_shift);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int n_cand = plan.n_chunks * k;
    const int n_groups = (plan.n_chunks + plan.group - 1) / plan.group;
    if (n_groups == 1) {
        hipLaunchKernelGGL(topk_merge_kernel, dim3(1, bt.total_q), dim3(kTkThreads), smem, st, k, n_cand, n_cand,
                           cand_ld, cidx, cval, (int64_t)k, indices, (float *)nullptr);
        return hipGetLastError();
    }
    // two levels: group winners (indices and values) after the chunk lists
    const int64_t cand2_ld = ((int64_t)n_groups * k + 63) / 64 * 64;
    int32_t *gidx = (int32_t *)((char *)ws + (size_t)bt.total_q * (size_t)cand_ld * 8u);
    float *gval = (float *)((char *)gidx + (size_t)bt.total_q * (size_t)cand2_ld * 4u);
    hipLaunchKernelGGL(topk_merge_kernel, dim3(n_groups, bt.total_q), dim3(kTkThreads), smem, st, k, n_cand,
                       plan.group * k, cand_ld, cidx, cval, cand2_ld, gidx, gval);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(1, bt.total_q), dim3(kTkThreads), smem, st, k, n_groups * k,
                       n_groups * k, cand2_ld, gidx, gval, (int64_t)k, indices, (float *)nullptr);
    return hipGetLastError();
}

} // namespace sa
