// Load-time conversion of MXFP4 expert weights into the layout the GEMM
// kernels stream (P3 "Kimi K3 Day-0 适配剖析", section 三: the MXFP4 checkpoint
// is converted layer by layer at load time into a form the hardware runs
// efficiently; no offline copy). The conversion is a byte permutation: codes
// and scales are moved, never re-encoded.
//
// One matrix [N][K] (N % 16 == 0, K % 128 == 0), rb = N/16 row blocks of 16
// rows, nch = K/128 chunks of 128 contraction elements, nc4 = ceil(nch/4):
//
//   codes  [rb][nch][g][m][16 bytes]  = canonical codes of row 16 rb + m,
//                                       MX block 4 c + g (elements 128 c + 32 g ..)
//   scales [rb][nc4][g][m][cc]        = scale of row 16 rb + m, block
//                                       4 (4 c4 + cc) + g; 0 past the last chunk
//
// so lane L = 16 g + m of a wave reads 16 contiguous code bytes at L * 16 of a
// 1 KB block and one scale dword at L * 4 of a 256-byte block.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(256) void prepack_codes_kernel(const uint8_t *__restrict__ src,
                                                            uint8_t *__restrict__ dst,
                                                            int64_t n_rows, int K)
{
    // one thread per 16-byte block, destination-major
    const int nch = K / 128;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = n_rows * (K / 32);
    if (i >= total) return;
    const int lane = (int)(i % 64);
    const int64_t rest = i / 64;               // (rb, c)
    const int c = (int)(rest % nch);
    const int64_t rb = rest / nch;
    const int g = lane >> 4, m = lane & 15;
    const int64_t row = rb * 16 + m;
    const int blk = 4 * c + g;
    *(u32x4 *)(dst + i * 16) = *(const u32x4 *)(src + row * (K / 2) + blk * 16);
}

__global__ __launch_bounds__(256) void prepack_scales_kernel(const uint8_t *__restrict__ src,
                                                             uint8_t *__restrict__ dst,
                                                             int64_t n_rows, int K)
{
    // one thread per destination byte
    const int nch = K / 128, nc4 = (nch + 3) / 4;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (n_rows / 16) * nc4 * 256;
    if (i >= total) return;
    const int cc = (int)(i % 4);
    const int lane = (int)((i / 4) % 64);
    const int64_t rest = i / 256;              // (rb, c4)
    const int c4 = (int)(rest % nc4);
    const int64_t rb = rest / nc4;
    const int g = lane >> 4, m = lane & 15;
    const int c = 4 * c4 + cc;
    uint8_t v = 0;
    if (c < nch) v = src[(rb * 16 + m) * (K / 32) + 4 * c + g];
    dst[i] = v;
}

// ---------------------------------------------------------------------------
// fp32 -> MXFP4 on the device (P3 "Kimi K3 Day-0 适配剖析", section 三: the
// weights are quantised to MXFP4 online, when the model is loaded; OCP MX
// v1.0: one E8M0 scale per 32 elements, E2M1 elements). One thread per
// 32-element block:
//   amax = max |v|; all zero -> scale code 0 and codes 0;
//   else s = clamp(floor(log2 amax) - 2 + 127, 0, 254), with floor(log2)
//   read from the exponent bits (subnormals included);
//   q = v * 2^(127 - s) (a power of two: exact), |q| rounded to the nearest
//   E2M1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6} with ties to the even code and
//   |q| > 5 to 6; the sign bit of v gives bit 3 (so -0 and small negatives
//   that round to 0 keep their sign).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1_code(float q)
{
    const float a = fabsf(q);
    uint32_t m;
    if (a > 5.0f) m = 7;         // 6
    else if (a >= 3.5f) m = 6;   // 4 (3.5 ties to the even code)
    else if (a > 2.5f) m = 5;    // 3
    else if (a >= 1.75f) m = 4;  // 2 (1.75 up, 2.5 down: even)
    else if (a > 1.25f) m = 3;   // 1.5
    else if (a >= 0.75f) m = 2;  // 1 (0.75 up, 1.25 down: even)
    else if (a > 0.25f) m = 1;   // 0.5
    else m = 0;                  // 0 (0.25 down: even)
    return m | ((__float_as_uint(q) >> 28) & 8u);
}

__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const float *__restrict__ w,
                                                             int64_t nblocks,
                                                             uint8_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nblocks) return;
    const float4 *v4 = (const float4 *)(w + i * 32);
    float v[32];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const float4 t = v4[j];
        v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
    const uint32_t u = __float_as_uint(amax);
    const int ex = (int)((u >> 23) & 0xffu);
    const int e = ex ? ex - 127 : (31 - __clz((int)(u & 0x7fffffu))) - 149;  // floor(log2 amax)
    const int s = amax == 0.0f ? 0 : min(254, max(0, e - 2 + 127));
    const float inv = __uint_as_float((uint32_t)(254 - s) << 23);  // 2^(127 - s), s <= 253
    u32x4 out;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) word |= e2m1_code(v[8 * d + j] * inv) << (4 * j);
        out[d] = amax == 0.0f ? 0u : word;
    }
    *(u32x4 *)(codes + i * 16) = out;
    scales[i] = (uint8_t)s;
}

hipError_t launch_mxfp4_quantize(const float *w, int64_t N, int K, uint8_t *codes,
                                 uint8_t *scales, hipStream_t s)
{
    const int64_t nb = N * (K / 32);
    if (nb <= 0) return hipSuccess;
    hipLaunchKernelGGL(mxfp4_quantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s,
                       w, nb, codes, scales);
    return hipGetLastError();
}

size_t packed_scale_bytes(int64_t N, int K)
{
    const int nch = K / 128, nc4 = (nch + 3) / 4;
    return (size_t)(N / 16) * nc4 * 256;
}

hipError_t launch_prepack(const uint8_t *codes, const uint8_t *scales, int64_t n_rows, int K,
                          uint8_t *pcodes, uint8_t *pscales, hipStream_t s)
{
    const int64_t nb = n_rows * (K / 32);
    if (nb > 0) {
        hipLaunchKernelGGL(prepack_codes_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0,
                           s, codes, pcodes, n_rows, K);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t ns = (int64_t)packed_scale_bytes(n_rows, K);
    if (ns > 0) {
        hipLaunchKernelGGL(prepack_scales_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0,
                           s, scales, pscales, n_rows, K);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace moe
