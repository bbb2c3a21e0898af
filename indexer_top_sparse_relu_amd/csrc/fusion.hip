// Branch fusion with a sliding-window local branch (gfx950).
//
// Pages (by title):
//   [SAD] "Sparse Attention and Hybrid Attention Architecture Design in Large
//          Language Models", §3 (pseudocode: a sparse branch over the selected
//          blocks, a sliding-window branch so that nearby context is never
//          lost, and a gated fusion g * sparse + (1 - g) * local) and §4
//          (branch fusion gating).
//
// The local branch is the path's exact attention (a3-a5) over an index list of
// the last `window` positions, so only two small kernels are new: the window
// list, and the fusion y = g * a + (1 - g) * b, g = sigmoid(G), of the two
// ungated branch outputs (each branch runs with a per-head gate of +inf,
// whose sigmoid is exactly 1).  The fusion is a stream over the outputs:
// 16-byte loads and stores, fp32 arithmetic, round to nearest even for bf16.
#include "launch.h"
#include "sa_device.h"

namespace sa {

constexpr int kFuseThreads = 256;

// One wave per token: slot e holds position lo + e for lo = max(0, pos - w + 1)
// while that is <= pos, then -1.
__global__ __launch_bounds__(kFuseThreads) void window_indices_kernel(Batch bt, int w, int32_t *__restrict__ out)
{
    const int tok = blockIdx.x * (kFuseThreads / 64) + (threadIdx.x >> 6);
    if (tok >= bt.total_q)
        return;
    const int lane = threadIdx.x & 63;
    const int b = seq_of_token(bt, tok);
    const int pos = pos_of_token(bt, b, tok);
    const int lo = max(0, pos - w + 1);
    for (int e = lane; e < w; e += 64)
        out[(int64_t)tok * w + e] = lo + e <= pos ? lo + e : -1;
}

__device__ __forceinline__ float fuse1(float a, float b, float G)
{
    const float g = 1.0f / (1.0f + __expf(-G));
    return fmaf(g, a - b, b);
}

// y = g * a + (1 - g) * b over rows x d_v elements; 8 elements per thread and
// step (bf16: one 16-byte load per operand; f32: two).
template <bool BF16>
__global__ __launch_bounds__(kFuseThreads) void branch_fuse_kernel(int64_t rows, int dv, const void *__restrict__ a,
                                                                   const void *__restrict__ b,
                                                                   const void *__restrict__ gate, int per_channel,
                                                                   void *__restrict__ y)
{
    const int64_t n8 = rows * dv / 8;
    for (int64_t v = (int64_t)blockIdx.x * kFuseThreads + threadIdx.x; v < n8;
         v += (int64_t)gridDim.x * kFuseThreads) {
        const int64_t e0 = v * 8, row = e0 / dv;
        float av[8], bv[8], gv[8];
        if constexpr (BF16) {
            const u32x4 A = ((const u32x4 *)a)[v], Bv = ((const u32x4 *)b)[v];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                av[2 * k] = __uint_as_float(A[k] << 16);
                av[2 * k + 1] = __uint_as_float(A[k] & 0xFFFF0000u);
                bv[2 * k] = __uint_as_float(Bv[k] << 16);
                bv[2 * k + 1] = __uint_as_float(Bv[k] & 0xFFFF0000u);
            }
            if (per_channel) {
                const u32x4 G = ((const u32x4 *)gate)[v];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    gv[2 * k] = __uint_as_float(G[k] << 16);
                    gv[2 * k + 1] = __uint_as_float(G[k] & 0xFFFF0000u);
                }
            } else {
                const float g = __uint_as_float((uint32_t)((const uint16_t *)gate)[row] << 16);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    gv[k] = g;
            }
            u32x4 out;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bf16x2 p = {(__bf16)fuse1(av[2 * k], bv[2 * k], gv[2 * k]),
                                  (__bf16)fuse1(av[2 * k + 1], bv[2 * k + 1], gv[2 * k + 1])};
                out[k] = __builtin_bit_cast(uint32_t, p);
            }
            ((u32x4 *)y)[v] = out;
        } else {
            const f32x4 *A = (const f32x4 *)a + 2 * v, *Bp = (const f32x4 *)b + 2 * v;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 x = A[h], z = Bp[h];
                f32x4 G;
                if (per_channel)
                    G = ((const f32x4 *)gate)[2 * v + h];
                else
                    G = f32x4{1.0f, 1.0f, 1.0f, 1.0f} * ((const float *)gate)[row];
                f32x4 r;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    r[k] = fuse1(x[k], z[k], G[k]);
                ((f32x4 *)y)[2 * v + h] = r;
            }
        }
    }
}

hipError_t launch_window_indices(const Batch &bt, int w, int32_t *indices, hipStream_t st)
{
    const int per = kFuseThreads / 64;
    hipLaunchKernelGGL(window_indices_kernel, dim3((bt.total_q + per - 1) / per), dim3(kFuseThreads), 0, st, bt, w,
                       indices);
    return hipGetLastError();
}

hipError_t launch_branch_fuse(int dtype, int64_t rows, int dv, const void *a, const void *b, const void *gate,
                              int per_channel, void *y, hipStream_t st)
{
    const int64_t n8 = rows * dv / 8;
    const int64_t grid = min((n8 + kFuseThreads - 1) / kFuseThreads, (int64_t)256 * 64);
    if (dtype == 1)
        hipLaunchKernelGGL(branch_fuse_kernel<true>, dim3((unsigned)grid), dim3(kFuseThreads), 0, st, rows, dv, a, b,
                           gate, per_channel, y);
    else
        hipLaunchKernelGGL(branch_fuse_kernel<false>, dim3((unsigned)grid), dim3(kFuseThreads), 0, st, rows, dv, a,
                           b, gate, per_channel, y);
    return hipGetLastError();
}

} // namespace sa
