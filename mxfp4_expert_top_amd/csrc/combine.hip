// Weighted unpermute / combine (P3 "Kimi K3 Day-0 适配剖析", section 四: the
// combine step gathers expert results back by weight; P2 "SGLang 0.5.17", section
// "MoE 稀疏激活": a weighted sum over the selected experts).
//
// out[t][m] = sum_{j < k, inv[t][j] >= 0} w[t][j] * y[inv[t][j]][m], summed in
// slot order j in fp32. A gather, not a scatter: every output element is
// written once, without atomics. Bandwidth-bound: one workgroup per token,
// 8 contiguous elements per thread per step.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <typename YT>
__device__ __forceinline__ void load8(const YT *p, float v[8]);
template <>
__device__ __forceinline__ void load8<float>(const float *p, float v[8])
{
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<bf16>(const bf16 *p, float v[8])
{
    const bf16x8 a = *(const bf16x8 *)p;
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = (float)a[i];
}

template <typename OT>
__device__ __forceinline__ void store8(OT *p, const float v[8]);
template <>
__device__ __forceinline__ void store8<float>(float *p, const float v[8])
{
    *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4 *)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ __forceinline__ void store8<bf16>(bf16 *p, const float v[8])
{
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] = to_bf16(v[i]);
    *(bf16x8 *)p = o;
}

template <typename YT, typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const YT *__restrict__ y, int64_t ldy,
                                                      const int32_t *__restrict__ inv,
                                                      const float *__restrict__ w, int d, int k,
                                                      OT *__restrict__ out, int64_t ldo)
{
    // blockIdx.x = token, blockIdx.y = a slice of 2048 columns; 8 columns per
    // thread. The token's local (row, weight) pairs are compacted in slot
    // order first, so the sum loop has no per-slot branch and its loads can
    // be issued ahead.
    const int t = blockIdx.x;
    __shared__ int32_t rows[MOE_MAX_TOPK_DEV];
    __shared__ float wts[MOE_MAX_TOPK_DEV];
    __shared__ int n_rows;
    if (threadIdx.x < 64) {
        const int j = threadIdx.x;
        const int r = j < k ? inv[(int64_t)t * k + j] : -1;
        const uint64_t valid = __ballot(r >= 0);
        const int slot = __popcll(valid & ((1ull << j) - 1ull));
        if (r >= 0) {
            rows[slot] = r;
            wts[slot] = w[(int64_t)t * k + j];
        }
        if (j == 0) n_rows = __popcll(valid);
    }
    __syncthreads();
    const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
    if (c >= d) return;
    const int n = n_rows;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int j = 0; j < n; j++) {
        float v[8];
        load8<YT>(y + (int64_t)rows[j] * ldy + c, v);
        const float wj = wts[j];
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] += wj * v[i];
    }
    store8<OT>(out + (int64_t)t * ldo + c, acc);
}

// The same gather over block-int16 expert outputs (the FP6X2 down
// projection's F6_OUT_Q16 rows: half the bytes of fp32). A thread's 8 columns
// lie in one 32-column block; value = q 2^(e - 126) / 32767, taken as
// q (w / 32767) 2^(e - 126) with the weight's factor formed once per row.
template <typename OT>
__global__ __launch_bounds__(256) void combine_q16_kernel(const int16_t *__restrict__ yq,
                                                          const uint8_t *__restrict__ ys,
                                                          int64_t ldy,
                                                          const int32_t *__restrict__ inv,
                                                          const float *__restrict__ w, int d,
                                                          int k, OT *__restrict__ out,
                                                          int64_t ldo)
{
    const int t = blockIdx.x;
    __shared__ int32_t rows[MOE_MAX_TOPK_DEV];
    __shared__ float wts[MOE_MAX_TOPK_DEV];
    __shared__ int n_rows;
    if (threadIdx.x < 64) {
        const int j = threadIdx.x;
        const int r = j < k ? inv[(int64_t)t * k + j] : -1;
        const uint64_t valid = __ballot(r >= 0);
        const int slot = __popcll(valid & ((1ull << j) - 1ull));
        if (r >= 0) {
            rows[slot] = r;
            wts[slot] = w[(int64_t)t * k + j];
        }
        if (j == 0) n_rows = __popcll(valid);
    }
    __syncthreads();
    const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
    if (c >= d) return;
    const int n = n_rows;
    const int64_t lds = ldy / 32;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int j = 0; j < n; j++) {
        const int64_t r = rows[j];
        // Y is read once: non-temporal loads (prefill combine 0.215 -> 0.196 ms,
        // long skewed 1.74 -> 1.67 ms; the fp32-Y combine measured slower so)
        const u32x4 q = __builtin_nontemporal_load((const u32x4 *)(yq + r * ldy + c));
        const float wx = ldexpf(wts[j] * (1.0f / 32767.0f), (int)ys[r * lds + c / 32] - 126);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            acc[2 * i] += wx * (float)(int16_t)(q[i] & 0xffffu);
            acc[2 * i + 1] += wx * (float)(int16_t)(q[i] >> 16);
        }
    }
    store8<OT>(out + (int64_t)t * ldo + c, acc);
}

hipError_t launch_combine_q16(const int16_t *yq, const uint8_t *ys, int64_t ldy,
                              const int32_t *inv, const float *w, int T, int d, int k,
                              void *out, int out_f32, int64_t ldo, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    if (d % 32 != 0 || ldy % 32 != 0) return hipErrorInvalidValue;
    dim3 grid(T, (d + 8 * 256 - 1) / (8 * 256)), block(256);
    if (out_f32)
        hipLaunchKernelGGL((combine_q16_kernel<float>), grid, block, 0, s, yq, ys, ldy, inv, w, d,
                           k, (float *)out, ldo);
    else
        hipLaunchKernelGGL((combine_q16_kernel<bf16>), grid, block, 0, s, yq, ys, ldy, inv, w, d,
                           k, (bf16 *)out, ldo);
    return hipGetLastError();
}

hipError_t launch_combine(const void *y, int y_f32, int64_t ldy, const int32_t *inv,
                          const float *w, int T, int d, int k, void *out, int out_f32,
                          int64_t ldo, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    dim3 grid(T, (d + 8 * 256 - 1) / (8 * 256)), block(256);
    if (y_f32 && out_f32)
        hipLaunchKernelGGL((combine_kernel<float, float>), grid, block, 0, s, (const float *)y,
                           ldy, inv, w, d, k, (float *)out, ldo);
    else if (y_f32)
        hipLaunchKernelGGL((combine_kernel<float, bf16>), grid, block, 0, s, (const float *)y,
                           ldy, inv, w, d, k, (bf16 *)out, ldo);
    else if (out_f32)
        hipLaunchKernelGGL((combine_kernel<bf16, float>), grid, block, 0, s, (const bf16 *)y, ldy,
                           inv, w, d, k, (float *)out, ldo);
    else
        hipLaunchKernelGGL((combine_kernel<bf16, bf16>), grid, block, 0, s, (const bf16 *)y, ldy,
                           inv, w, d, k, (bf16 *)out, ldo);
    return hipGetLastError();
}

}  // namespace moe
