// Device-side building blocks shared by the gfx950 kernels of the MXFP4
// LatentMoE layer: vector types, the bf16 matrix-core instruction, MXFP4
// decode, and bf16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace moe {

constexpr int kWave = 64;

// D = A * B + C on one 16x16 fp32 tile with K = 32 bf16 products.
// Operand lanes: lane L supplies row (L % 16) of A and column (L % 16) of B,
// 8 consecutive contraction elements of the lane group L / 16. Any mapping of
// contraction indices to (lane group, element) gives the same sum as long as A
// and B use the same one, so kernels choose the mapping that makes their loads
// contiguous. Result: lane L holds C[4 * (L / 16) + i][L % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A * B + C on one 32x32 fp32 tile with K = 16 bf16 products. Lane L
// supplies row (L % 32) of A and column (L % 32) of B, 8 consecutive
// contraction elements of the half L / 32 (same freedom of mapping as above).
// Result: lane L holds C[8 (v / 4) + 4 (L / 32) + v % 4][L % 32], v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// E8M0 scale code -> fp32 2^(s-127). Code 0 is the fp32 subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Decode 8 E2M1 codes (one dword: element 2i in the low nibble of byte i) and
// multiply by `scale` (a power of two), giving 8 bf16 values. Products of an
// E2M1 value and 2^n are exact in bf16 unless they leave its normal range.
__device__ __forceinline__ bf16x8 mx_decode8(uint32_t codes, float scale)
{
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ bf16 to_bf16(float f)
{
    return (bf16)f;
}

__device__ __forceinline__ float bf16_to_f32(bf16 b)
{
    return (float)b;
}

// Split an fp32 value into three bf16 parts whose exact sum is the value:
// hi keeps the top 8 significant bits (truncated), mid the next 8 of the
// remainder, lo the rest (at most 8 bits, so exact in bf16). Each product of
// a bf16 with a part is exact in fp32.
__device__ __forceinline__ void split3_bf16(float v, bf16 &hi, bf16 &mid, bf16 &lo)
{
    float h = __uint_as_float(__float_as_uint(v) & 0xffff0000u);
    float r1 = v - h;
    float m = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
    float r2 = r1 - m;
    hi = (bf16)h;
    mid = (bf16)m;
    lo = (bf16)r2;
}

// v ~ hi + mid, both rounded to nearest bf16: hi = bf16(v), mid = bf16(v - hi)
// (v - hi is exact in fp32), so |v - hi - mid| <= 2^-17 |v| (16 significant
// bits against fp32's 24).
__device__ __forceinline__ void split2_bf16(float v, bf16 &hi, bf16 &mid)
{
    hi = to_bf16(v);
    mid = to_bf16(v - (float)hi);
}

// Activation stages (the elementwise step between the two projections).
enum { ACT_NONE = 0, ACT_SILU_MUL = 1, ACT_GELU_TANH_MUL = 2 };

// g * u / (1 + exp(-z)) with the hardware exp2 and reciprocal (each within
// about 1 ulp); exp overflowing to inf gives 0, the limit.
__device__ __forceinline__ float gated_sigmoid(float g, float u, float z)
{
    const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
    return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// silu(g) * u = g * sigmoid(g) * u; gelu_tanh(g) * u =
// 0.5 g (1 + tanh(y)) u = g * sigmoid(2 y) * u with y = sqrt(2/pi) (g + 0.044715 g^3).
template <int ACT>
__device__ __forceinline__ float act_apply(float g, float u)
{
    if constexpr (ACT == ACT_SILU_MUL) {
        return gated_sigmoid(g, u, g);
    } else if constexpr (ACT == ACT_GELU_TANH_MUL) {
        const float y = 0.7978845608028654f * (g + 0.044715f * g * g * g);
        return gated_sigmoid(g, u, 2.0f * y);
    } else {
        return g;
    }
}

// Exclusive prefix sum over the threads of a workgroup of `nthreads`
// (a multiple of 64, at most 1024) threads: an inclusive scan inside each
// wavefront with lane shuffles, one exchange of the wave totals through LDS.
// `scratch` holds 16 ints of LDS; `total` receives the sum of all values.
// Every thread of the workgroup must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
    }
    if (lane == 63) scratch[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < nwaves; w++) {
        const int t = scratch[w];
        before += w < wave ? t : 0;
        all += t;
    }
    __syncthreads();  // scratch may be reused by the caller
    total = all;
    return before + inc - v;
}

// Work items of the grouped GEMMs: an expert's c rows in g = ceil(c / R)
// groups, either R rows each (the last one shorter) or, `balanced`, of
// nearly equal size (sizes differ by at most one), so that no group is a
// short tail that streams a whole weight tile for a few rows.
// Item = {expert | rows << 16, first row} (experts < 2^16, rows <= R).
__device__ __forceinline__ int2 plan_item(int e, int off_e, int c, int g, int i, int R,
                                          bool balanced)
{
    const int s = balanced ? (int)((int64_t)i * c / g) : i * R;
    const int t = balanced ? (int)((int64_t)(i + 1) * c / g) : min((i + 1) * R, c);
    return make_int2(e | ((t - s) << 16), off_e + s);
}

template <typename T>
__device__ __forceinline__ void store_out(T *p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<bf16>(bf16 *p, float v) { *p = to_bf16(v); }

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes per lane from `src` to LDS at `lds_base` (wave-uniform) + 16 lane
// (global_load_lds_dwordx4). The load counts in vmcnt like any vector load;
// callers wait explicitly (the compiler's own wait insertion would otherwise
// drain every such load before the next LDS read). M0 holds no compiler value
// in the kernels that use it, so clobbering it needs no save.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// The same for outputs that are read once, much later, by another kernel (the
// expert outputs Y before the combine): fp32 is stored with the non-temporal
// hint, which measured 6% faster in the combine that reads it back.
template <typename T>
__device__ __forceinline__ void store_out_once(T *p, float v)
{
    if constexpr (sizeof(T) == 4) __builtin_nontemporal_store(v, p);
    else store_out<T>(p, v);
}

}  // namespace moe
