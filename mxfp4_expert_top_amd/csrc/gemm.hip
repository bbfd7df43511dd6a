// Grouped expert projections with MXFP4 weights on the gfx950 bf16 matrix
// cores (P2 "SGLang 0.5.17：Kimi K3 原生 MXFP4 推理架构解析", section "MXFP4
// 原生支持": dequantisation fused into the GEMM; P1 "从Kimi K3到MiniMax-H3",
// section 二/第一层: 4-bit weights combined with higher-precision activations,
// dequantise + multiply + accumulate in the kernel).
//
// MXFP4 codes go from HBM straight into registers, are decoded there with the
// scaled FP4->bf16 convert (exact: an E2M1 value times a power of two), and
// feed v_mfma_f32_16x16x32_bf16 with fp32 accumulation. No dequantised copy of
// a weight ever reaches memory.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int PLAN_HDR = 64;  // int32 slots before the work items
constexpr int ST_ROWS = 16;   // streaming schedule: permuted rows per group
constexpr int ST_NB = 64;     // streaming schedule: weight rows per workgroup

// ---------------------------------------------------------------------------
// Work plan: groups of up to R consecutive rows of one expert, expert-major.
// plan[0] = number of groups; items (expert, first row) from plan[PLAN_HDR].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void gemm_plan_kernel(const int32_t *__restrict__ off, int nl,
                                                         int R, int max_groups,
                                                         int32_t *__restrict__ plan)
{
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int per = (nl + 1023) / 1024;
    const int lo = tid * per, hi = min(lo + per, nl);
    int s = 0;
    for (int i = lo; i < hi; i++) s += (off[i + 1] - off[i] + R - 1) / R;
    part[tid] = s;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        int v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int pos = part[tid] - s;
    int2 *items = (int2 *)(plan + PLAN_HDR);
    for (int i = lo; i < hi; i++) {
        const int c = off[i + 1] - off[i];
        for (int r = 0; r < c; r += R, pos++)
            if (pos < max_groups) items[pos] = make_int2(i, off[i] + r);
    }
    if (tid == 1023) plan[0] = min(part[1023], max_groups);
}

// ---------------------------------------------------------------------------
// Weight-streaming schedule (few rows per expert: decode batches).
//
// Work item = (row group of <= 16 rows of expert e, 64 weight rows). Each of
// the 4 waves owns 16 weight rows and streams them over all of K; every
// weight byte is read once per row group. Lane L: token row m = L % 16 of
// the group (A operand), weight row L % 16 of the wave (B operand), lane
// group g = L / 16.
//
// Contraction mapping per 128-wide K chunk at kc: lane group g holds the
// 32 elements kc + 32 g .. +32, i.e. exactly one MX block, so one 16-byte
// code load and one scale byte per lane per matrix. MFMA step s (0..3) takes
// elements kc + 32 g + 8 s .. +8 of both operands.
//
// GLU (act != NONE): the wave streams the same 16 rows of both W1 (gate) and
// W2 (up); the two accumulators of a (token, n) pair sit in the same lane and
// register, so act(gate, up) is applied in registers.
// ---------------------------------------------------------------------------
template <int ACT, typename OutT>
__global__ __launch_bounds__(256) void gemm_stream_kernel(
    const bf16 *__restrict__ a, int64_t lda, const int32_t *__restrict__ a_rows,
    const uint8_t *__restrict__ w1c, const uint8_t *__restrict__ w1s,
    const uint8_t *__restrict__ w2c, const uint8_t *__restrict__ w2s,
    const int32_t *__restrict__ off, const int32_t *__restrict__ plan, int N, int K,
    OutT *__restrict__ out, int64_t ldo)
{
    constexpr bool GLU = ACT != ACT_NONE;
    const int n_groups = plan[0];
    const int2 *items = (const int2 *)(plan + PLAN_HDR);
    const int nblk = N / ST_NB;
    const int total = n_groups * nblk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t code_row = K / 2, scale_row = K / 32;

    for (int w = blockIdx.x; w < total; w += gridDim.x) {
        const int grp = w / nblk, nb = w - grp * nblk;
        const int2 it = items[grp];
        const int e = it.x, r0 = it.y;
        const int rend = min(r0 + ST_ROWS, off[e + 1]);
        const int r = r0 + m;
        const bool rv = r < rend;
        const int64_t arow = rv ? (a_rows ? (int64_t)a_rows[r] : (int64_t)r) : 0;
        const bf16 *ap = a + arow * lda + 32 * g;
        const int n = nb * ST_NB + wave * 16 + m;
        const int64_t wrow = (int64_t)e * N + n;
        const uint8_t *c1 = w1c + wrow * code_row + 16 * g;
        const uint8_t *s1 = w1s + wrow * scale_row;
        const uint8_t *c2 = GLU ? w2c + wrow * code_row + 16 * g : nullptr;
        const uint8_t *s2 = GLU ? w2s + wrow * scale_row : nullptr;

        f32x4 acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int kc = 0; kc < K; kc += 128) {
            const u32x4 q1 = *(const u32x4 *)(c1 + kc / 2);
            const float f1 = e8m0_to_f32((*(const uint32_t *)(s1 + kc / 32) >> (8 * g)) & 0xffu);
            u32x4 q2;
            float f2 = 0.f;
            if constexpr (GLU) {
                q2 = *(const u32x4 *)(c2 + kc / 2);
                f2 = e8m0_to_f32((*(const uint32_t *)(s2 + kc / 32) >> (8 * g)) & 0xffu);
            }
            bf16x8 af[4];
#pragma unroll
            for (int s = 0; s < 4; s++)
                af[s] = rv ? *(const bf16x8 *)(ap + kc + 8 * s) : bf16x8{};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                acc1 = mfma16x16x32(af[s], mx_decode8(q1[s], f1), acc1);
                if constexpr (GLU) acc2 = mfma16x16x32(af[s], mx_decode8(q2[s], f2), acc2);
            }
        }
        // lane holds C[4 g + i][m]: token row r0 + 4 g + i, output column n
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = r0 + 4 * g + i;
            if (row < rend) {
                float v = GLU ? act_apply<ACT>(acc1[i], acc2[i]) : acc1[i];
                store_out<OutT>(out + (int64_t)row * ldo + n, v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Standalone decode of an MXFP4 matrix to bf16 (8 elements per thread).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mxfp4_dequant_kernel(const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t N, int K,
                                                            bf16 *__restrict__ out)
{
    const int64_t per_row = K / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N * per_row) return;
    const int64_t n = i / per_row, c = i - n * per_row;
    const uint32_t q = *(const uint32_t *)(codes + n * (K / 2) + c * 4);
    const float f = e8m0_to_f32(scales[n * (K / 32) + c / 4]);
    *(bf16x8 *)(out + n * K + c * 8) = mx_decode8(q, f);
}

// ---------------------------------------------------------------------------
static int device_cus()
{
    static thread_local int dev_cached = -1, cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != dev_cached) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        dev_cached = dev;
    }
    return cus;
}

int resolve_mode(int mode, int num_local, int max_rows)
{
    (void)num_local;
    (void)max_rows;
    if (mode == 1 || mode == 2) return 1;
    return 1;
}

static int rows_per_group(int mode) { return mode == 2 ? 128 : ST_ROWS; }

static int max_groups_for(int num_local, int max_rows, int R)
{
    return (max_rows + R - 1) / R + num_local;
}

size_t gemm_plan_ws_bytes(int num_local, int max_rows, int R)
{
    size_t n = (size_t)PLAN_HDR + 2 * (size_t)max_groups_for(num_local, max_rows, R);
    return ((n * sizeof(int32_t)) + 255) & ~(size_t)255;
}

size_t grouped_gemm_ws_bytes(int num_local, int max_rows, int N, int mode)
{
    (void)N;
    const int md = resolve_mode(mode, num_local, max_rows);
    return gemm_plan_ws_bytes(num_local, max_rows, rows_per_group(md));
}

template <int ACT, typename OutT>
static hipError_t launch_stream(const bf16 *a, int64_t lda, const int32_t *a_rows,
                                const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                                const uint8_t *w2s, const int32_t *off, const int32_t *plan,
                                int max_groups, int N, int K, OutT *out, int64_t ldo,
                                hipStream_t s)
{
    const int64_t bound = (int64_t)max_groups * (N / ST_NB);
    const int64_t cap = (int64_t)device_cus() * 8;
    const int grid = (int)(bound < cap ? bound : cap);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_stream_kernel<ACT, OutT>), dim3(grid), dim3(256), 0, s, a, lda,
                       a_rows, w1c, w1s, w2c, w2s, off, plan, N, K, out, ldo);
    return hipGetLastError();
}

template <typename OutT>
static hipError_t dispatch_act(int act, const bf16 *a, int64_t lda, const int32_t *a_rows,
                               const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                               const uint8_t *w2s, const int32_t *off, const int32_t *plan,
                               int max_groups, int N, int K, OutT *out, int64_t ldo,
                               hipStream_t s)
{
    switch (act) {
    case ACT_NONE:
        return launch_stream<ACT_NONE, OutT>(a, lda, a_rows, w1c, w1s, w2c, w2s, off, plan,
                                             max_groups, N, K, out, ldo, s);
    case ACT_SILU_MUL:
        return launch_stream<ACT_SILU_MUL, OutT>(a, lda, a_rows, w1c, w1s, w2c, w2s, off, plan,
                                                 max_groups, N, K, out, ldo, s);
    case ACT_GELU_TANH_MUL:
        return launch_stream<ACT_GELU_TANH_MUL, OutT>(a, lda, a_rows, w1c, w1s, w2c, w2s, off,
                                                      plan, max_groups, N, K, out, ldo, s);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_plan(const int32_t *off, int num_local, int max_rows, int mode, void *ws,
                            hipStream_t s)
{
    const int R = rows_per_group(resolve_mode(mode, num_local, max_rows));
    hipLaunchKernelGGL(gemm_plan_kernel, dim3(1), dim3(1024), 0, s, off, num_local, R,
                       max_groups_for(num_local, max_rows, R), (int32_t *)ws);
    return hipGetLastError();
}

hipError_t launch_gemm_run(const bf16 *a, int64_t lda, const int32_t *a_rows, const uint8_t *w1c,
                           const uint8_t *w1s, const uint8_t *w2c, const uint8_t *w2s,
                           const int32_t *off, int num_local, int max_rows, int N, int K, int act,
                           void *out, int out_f32, int64_t ldo, int mode, const void *plan_ws,
                           hipStream_t s)
{
    const int md = resolve_mode(mode, num_local, max_rows);
    const int max_groups = max_groups_for(num_local, max_rows, rows_per_group(md));
    const int32_t *plan = (const int32_t *)plan_ws;
    if (out_f32)
        return dispatch_act<float>(act, a, lda, a_rows, w1c, w1s, w2c, w2s, off, plan, max_groups,
                                   N, K, (float *)out, ldo, s);
    return dispatch_act<bf16>(act, a, lda, a_rows, w1c, w1s, w2c, w2s, off, plan, max_groups, N,
                              K, (bf16 *)out, ldo, s);
}

hipError_t launch_grouped_gemm(const bf16 *a, int64_t lda, const int32_t *a_rows,
                               const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                               const uint8_t *w2s, const int32_t *off, int num_local,
                               int max_rows, int N, int K, int act, void *out, int out_f32,
                               int64_t ldo, int mode, void *ws, hipStream_t s)
{
    hipError_t e = launch_gemm_plan(off, num_local, max_rows, mode, ws, s);
    if (e != hipSuccess) return e;
    return launch_gemm_run(a, lda, a_rows, w1c, w1s, w2c, w2s, off, num_local, max_rows, N, K,
                           act, out, out_f32, ldo, mode, ws, s);
}

hipError_t launch_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t N, int K,
                                bf16 *out, hipStream_t s)
{
    const int64_t n = N * (K / 8);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(mxfp4_dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       codes, scales, N, K, out);
    return hipGetLastError();
}

}  // namespace moe
