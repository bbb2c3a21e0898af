// Cache append and fp8 quantisation (gfx950): the step before the path.
//
// Pages (by title):
//   [HAT] "Hybrid Attention Architectures: Engineering Trade-offs from Linear
//          Attention to Gated Sparse Attention", §5 item 2 (cache organisation
//          decides indexing efficiency) and item 3 (the indexer is sensitive
//          to numeric range in low precision).
//   [F2S] "From Full Attention to Sparsity: The Evolution of Hybrid Attention
//          Architectures in Large Language Models", "Engineering
//          Considerations" item 1 (paged cache management is on the critical
//          path).
//
// Format (the pages fix none): an fp8 indexer key is a row of OCP e4m3fn
// codes plus one fp32 scale, s = max|x| / 448, code = e4m3fn(x / s) rounded
// to nearest even and saturated at +-448; a row of zeros gets s = 0 and
// codes 0.  The division is the IEEE single-precision one, so each code is
// decided in fp32.
//
// Both kernels are HBM-bound streams with no reuse: one wave per token row
// for the append (16-byte copies of the K / V rows, the key quantised in
// registers with a DPP maximum), one workgroup per row for the row
// quantiser (wide rows: the maximum goes through LDS).
#include "launch.h"
#include "sa_device.h"

namespace sa {

constexpr int kAppendWaves = 4;           // tokens per workgroup
constexpr int kQuantThreads = 256;

// Two e4m3fn codes (low byte: a) of values already divided by the scale.  The
// clamp makes the conversion saturate; v_cvt_pk_fp8_f32 rounds to nearest
// even.
__device__ __forceinline__ uint32_t fp8_pair(float a, float b)
{
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float2 load_pair(const void *src, int src_f32, int64_t pair)
{
    if (src_f32)
        return ((const float2 *)src)[pair];
    const uint32_t w = ((const uint32_t *)src)[pair];
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
}

// One wave per new token: its K row (and V row when separate) go to the
// physical row of its position, its indexer key is copied or quantised.
// Row byte counts are multiples of 16 and at most kRowPieces * 1 KB; d_i is
// even and at most 2 * 64 * 8.  The sources are read before the destination
// row is known (they do not depend on it), so the page-table lookup and the
// source loads share one memory round trip.
constexpr int kRowPieces = 4;
__global__ __launch_bounds__(64 * kAppendWaves) void cache_append_kernel(
    Batch bt, const uint8_t *__restrict__ k_new, int krow_bytes, const uint8_t *__restrict__ v_new, int vrow_bytes,
    uint8_t *__restrict__ k_cache, uint8_t *__restrict__ v_cache, int64_t stride_bytes, const void *__restrict__ kidx_new,
    int src_f32, int d_i, int fp8, uint8_t *__restrict__ kidx_cache, float *__restrict__ kscale_cache)
{
    const int lane = threadIdx.x & 63;
    const int tok = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
    if (tok >= bt.total_q)
        return;
    u32x4 kp[kRowPieces], vp[kRowPieces];
#pragma unroll
    for (int u = 0; u < kRowPieces; ++u) {
        const int o = 16 * lane + 1024 * u;
        if (o < krow_bytes)
            kp[u] = *(const u32x4 *)(k_new + (int64_t)tok * krow_bytes + o);
        if (v_new && o < vrow_bytes)
            vp[u] = *(const u32x4 *)(v_new + (int64_t)tok * vrow_bytes + o);
    }
    constexpr int PU = 8;                         // key pairs per lane, at most
    const int npair = d_i / 2;
    float2 x[PU];
    uint32_t cw[2 * PU];                          // same-dtype copy: 4-byte words
    const int words = src_f32 ? d_i : npair;
#pragma unroll
    for (int u = 0; u < PU; ++u) {
        const int p = lane + 64 * u;
        if (fp8) {
            x[u] = p < npair ? load_pair(kidx_new, src_f32, (int64_t)tok * npair + p) : make_float2(0.0f, 0.0f);
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int w = lane + 64 * (2 * u + h);
                cw[2 * u + h] = w < words ? ((const uint32_t *)kidx_new)[(int64_t)tok * words + w] : 0u;
            }
        }
    }

    const int b = seq_of_token(bt, tok);
    const int64_t row = phys_row(bt, b, pos_of_token(bt, b, tok));
#pragma unroll
    for (int u = 0; u < kRowPieces; ++u) {
        const int o = 16 * lane + 1024 * u;
        if (o < krow_bytes)
            *(u32x4 *)(k_cache + row * stride_bytes + o) = kp[u];
        if (v_new && o < vrow_bytes)
            *(u32x4 *)(v_cache + row * stride_bytes + o) = vp[u];
    }
    if (!fp8) {
        uint32_t *dst = (uint32_t *)kidx_cache + row * words;
#pragma unroll
        for (int u = 0; u < 2 * PU; ++u) {
            const int w = lane + 64 * u;
            if (w < words)
                dst[w] = cw[u];
        }
        return;
    }
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < PU; ++u)
        amax = fmaxf(amax, fmaxf(fabsf(x[u].x), fabsf(x[u].y)));
    amax = wave_max(amax);
    const float s = amax / 448.0f;
    uint16_t *dst = (uint16_t *)(kidx_cache + row * d_i);
#pragma unroll
    for (int u = 0; u < PU; ++u) {
        const int p = lane + 64 * u;
        if (p < npair)
            dst[p] = (uint16_t)(amax > 0.0f ? fp8_pair(x[u].x / s, x[u].y / s) : 0u);
    }
    if (lane == 0)
        kscale_cache[row] = s;
}

// One workgroup per row of x [rows, cols] (cols a multiple of 8): the row's
// maximum, then its codes, 8 per thread and step.  Rows of at most
// 8 * kQuantThreads * kQuantHeld elements stay in registers between the two
// steps (one read of the row); longer rows are read twice (the second time
// from the L2).
constexpr int kQuantHeld = 4;
__global__ __launch_bounds__(kQuantThreads) void quantize_rows_kernel(const void *__restrict__ x, int src_f32,
                                                                      int cols, uint8_t *__restrict__ codes,
                                                                      float *__restrict__ scales)
{
    __shared__ float wmax[kQuantThreads / 64];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    auto load8 = [&](int c, float (&v)[8]) {
        if (src_f32) {
            const f32x4 *p = (const f32x4 *)((const float *)x + r * cols + c);
            const f32x4 a = p[0], b = p[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = a[e];
                v[4 + e] = b[e];
            }
        } else {
            const u32x4 w = *(const u32x4 *)((const uint16_t *)x + r * cols + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = __uint_as_float(w[e] << 16);
                v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
        }
    };
    const bool held = cols <= 8 * kQuantThreads * kQuantHeld;
    float hv[kQuantHeld][8];
    float amax = 0.0f;
    if (held) {
#pragma unroll
        for (int u = 0; u < kQuantHeld; ++u) {
            const int c = 8 * tid + 8 * kQuantThreads * u;
            if (c < cols)
                load8(c, hv[u]);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    hv[u][e] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                amax = fmaxf(amax, fabsf(hv[u][e]));
        }
    } else {
        for (int c = 8 * tid; c < cols; c += 8 * kQuantThreads) {
            float v[8];
            load8(c, v);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                amax = fmaxf(amax, fabsf(v[e]));
        }
    }
    amax = wave_max(amax);
    if (lane == 0)
        wmax[tid >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kQuantThreads / 64; ++w)
        amax = fmaxf(amax, wmax[w]);
    const float s = amax / 448.0f;
    auto put8 = [&](int c, const float (&v)[8]) {
        u32x2 out = {0u, 0u};
        if (amax > 0.0f) {
            out.x = fp8_pair(v[0] / s, v[1] / s) | (fp8_pair(v[2] / s, v[3] / s) << 16);
            out.y = fp8_pair(v[4] / s, v[5] / s) | (fp8_pair(v[6] / s, v[7] / s) << 16);
        }
        *(u32x2 *)(codes + r * cols + c) = out;
    };
    if (held) {
#pragma unroll
        for (int u = 0; u < kQuantHeld; ++u) {
            const int c = 8 * tid + 8 * kQuantThreads * u;
            if (c < cols)
                put8(c, hv[u]);
        }
    } else {
        for (int c = 8 * tid; c < cols; c += 8 * kQuantThreads) {
            float v[8];
            load8(c, v);
            put8(c, v);
        }
    }
    if (tid == 0)
        scales[r] = s;
}

hipError_t launch_cache_append(const Batch &bt, int kv_esz, const void *k_new, int d_qk, const void *v_new, int d_v,
                               void *k_cache, void *v_cache, int64_t row_stride, int src_f32, const void *kidx_new,
                               int d_i, int fp8, void *kidx_cache, float *kscale_cache, hipStream_t st)
{
    const int grid = (bt.total_q + kAppendWaves - 1) / kAppendWaves;
    hipLaunchKernelGGL(cache_append_kernel, dim3(grid), dim3(64 * kAppendWaves), 0, st, bt,
                       (const uint8_t *)k_new, d_qk * kv_esz, (const uint8_t *)v_new, d_v * kv_esz,
                       (uint8_t *)k_cache, (uint8_t *)v_cache, row_stride * kv_esz, kidx_new, src_f32, d_i, fp8,
                       (uint8_t *)kidx_cache, kscale_cache);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const void *x, int src_f32, int64_t rows, int cols, uint8_t *codes, float *scales,
                                hipStream_t st)
{
    hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)rows), dim3(kQuantThreads), 0, st, x, src_f32, cols,
                       codes, scales);
    return hipGetLastError();
}

} // namespace sa
