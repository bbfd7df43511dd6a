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
