// Device-side helpers shared by the HIP kernels of the gated sparse attention
// path (gfx950 / CDNA4, wave64).  Host code never includes this file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Ragged batch over a paged cache, passed to kernels by value.  Query token j
// of sequence b sits at pos = ctx_len[b] - nq_b + j; position s of sequence b
// lives at physical row page_table[b*max_pages + s/page_size]*page_size +
// s%page_size (page_size is a power of two).
struct Batch {
    int32_t num_seqs;
    int32_t total_q;
    int32_t max_q;
    int32_t max_ctx;
    int32_t page_shift;
    int32_t max_pages;
    const int32_t *q_start;
    const int32_t *ctx_len;
    const int32_t *page_table;
};

// Largest b with q_start[b] <= tok: the sequence that owns token tok (empty
// sequences have q_start[b] == q_start[b+1] and are skipped by construction).
__device__ __forceinline__ int seq_of_token(const Batch &bt, int tok)
{
    int lo = 0, hi = bt.num_seqs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (bt.q_start[mid] <= tok)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Position of token tok, given its sequence b.
__device__ __forceinline__ int pos_of_token(const Batch &bt, int b, int tok)
{
    int q0 = bt.q_start[b];
    int nq = bt.q_start[b + 1] - q0;
    return bt.ctx_len[b] - nq + (tok - q0);
}

__device__ __forceinline__ int64_t phys_row(const Batch &bt, int b, int s)
{
    int page = bt.page_table[(int64_t)b * bt.max_pages + (s >> bt.page_shift)];
    return ((int64_t)page << bt.page_shift) + (s & ((1 << bt.page_shift) - 1));
}

// ---------------------------------------------------------------- MFMA tiles
// 32x32 output tile layout (all 32x32 MFMAs used here): lane l holds column
// l % 32; register i holds row 8*(i/4) + 4*(l/32) + i%4.
__device__ __forceinline__ int mfma32_row(int i, int lane)
{
    return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// 16x16 output tile layout: lane l holds column l % 16; register i holds row
// 4*(l/16) + i.
__device__ __forceinline__ int mfma16_row(int i, int lane)
{
    return 4 * (lane >> 4) + i;
}

// A/B operands: lane l supplies row (A) or column (B) l % 32 (32x32) or
// l % 16 (16x16), and a contiguous run of the contraction index selected by
// l / 32 (resp. l / 16).  A and B use the same run for the same lane group,
// so the product contracts matching elements whatever order the hardware
// walks inside a run.

__device__ __forceinline__ f32x16 mma32_f32(float a, float b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mma32_bf16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp8 (OCP e4m3fn) x fp8, 32x32x64, unit block scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x16 mma32_fp8(i32x8 a, i32x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The plain (unscaled) instruction: zero scale operands select it.
__device__ __forceinline__ f32x16 mma32_fp8_plain(i32x8 a, i32x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Same, with both block scales 2^-5 (E8M0 122): the product comes out scaled by
// 2^-10, which keeps any fp8 dot of length <= 128 (|dot| <= 128 * 448^2) inside
// the fp16 range for a packed-fp16 epilogue.
__device__ __forceinline__ f32x16 mma32_fp8_s10(i32x8 a, i32x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 122, 0, 122);
}

__device__ __forceinline__ f32x4 mma16_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float sigmoidf_(float x)
{
    return 1.0f / (1.0f + __expf(-x));
}

// ReLU of two fp32 values rounded (toward zero) to a packed fp16 pair, then
// acc + w.x with the fp16 products summed in fp32 (v_dot2_f32_f16).
__device__ __forceinline__ float relu_dot2(float x0, float x1, f16x2 w, float acc)
{
    f16x2 x = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0, x1));
    x = __builtin_elementwise_max(x, f16x2{(_Float16)0.0f, (_Float16)0.0f});
    return __builtin_amdgcn_fdot2(x, w, acc, false);
}

// Power-of-two exponent that moves m > 0 into [2^14, 2^15): fp16 weights scaled
// by it neither overflow nor go subnormal within 28 binades below m.
__device__ __forceinline__ int f16_weight_shift(float m)
{
    return m > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(m) : 0;
}

// A copy of v that the compiler cannot see through.  Lane-derived addresses
// computed from it inside a loop body are recomputed there (a few VALU ops)
// instead of being hoisted and kept live across the loop, where register
// pressure would spill them: a scratch reload waits on vmcnt, which also
// counts the loop's in-flight prefetches.
__device__ __forceinline__ int opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// ----------------------------------------------------------------- LDS DMA
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Direct global->LDS loads (global_load_lds): lane i's 16 (resp. 4) bytes land
// at lds + 16*i (resp. 4*i); lds is wave-uniform and goes through M0, which is
// saved and restored.  Written as asm so the compiler does not track them:
// its LDS-DMA tracking would put a full vmcnt wait in front of every LDS read
// while a prefetch into another buffer is in flight.  Completion is awaited explicitly with s_waitcnt vmcnt, and
// loads unknown to the compiler can only make its own waits stricter.
__device__ __forceinline__ void dma_b128(const void *src, const lds_u8 *lds)
{
    const uint32_t base = (uint32_t)(uintptr_t)lds;
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(src), "s"(base) : "memory");
}
__device__ __forceinline__ void dma_b32(const void *src, const lds_u8 *lds)
{
    const uint32_t base = (uint32_t)(uintptr_t)lds;
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dword %1, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(src), "s"(base) : "memory");
}

// The same with a wave-uniform base in scalar registers and a 32-bit per-lane
// byte offset (the saddr form): the address costs the lanes one 32-bit value.
__device__ __forceinline__ void dma_b128_sv(const void *sbase, uint32_t voff, const lds_u8 *lds)
{
    const uint32_t base = (uint32_t)(uintptr_t)lds;
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_nop 0\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(base) : "memory");
}

// ------------------------------------------------------------ wave helpers
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m)
{
    return __shfl_xor(v, m, kWave);
}

// x[l] + x[l ^ 32] and max(x[l], x[l ^ 32]) in every lane of a wave64, in the
// VALU: v_permlane32_swap exchanges the upper half of one register with the
// lower half of another, so two copies of x end up holding (lower, lower) and
// (upper, upper).  (A lane shuffle goes through the LDS crossbar and makes the
// wave wait for every LDS access in flight.)
__device__ __forceinline__ float sum_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum over the 64 lanes, all in the VALU: DPP within each row of 16
// lanes (pair swaps, then rotations by 4 and 8), v_permlane16_swap across the
// rows of each half, v_permlane32_swap across the halves.
__device__ __forceinline__ float wave_max(float v)
{
#define SA_DPP_MAX(ctrl) \
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false)))
    SA_DPP_MAX(0xB1);                  // quad_perm [1,0,3,2]
    SA_DPP_MAX(0x4E);                  // quad_perm [2,3,0,1]
    SA_DPP_MAX(0x124);                 // row_ror:4
    SA_DPP_MAX(0x128);                 // row_ror:8
#undef SA_DPP_MAX
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return max_halves(v);
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += shfl_xor(v, m);
    return v;
}

} // namespace sa
