// LoRA on the MXFP4 base: a low-rank increment B A on a frozen expert
// projection (P1 "从Kimi K3到MiniMax-H3" section 二, 第五层: LoRA keeps the
// large quantised base frozen and trains only the low-rank delta).
//
// For permuted row r of local expert e (rows off[e] .. off[e+1]-1):
//   t[r][j]  = scale * sum_k x_row(r)[k] * A_e[j][k]        (rank factor)
//   y[r][n] += sum_j t[r][j] * B_e[n][j]                     (the delta)
// with A_e [rank][K], B_e [N][rank] bf16 and y the fp32 output of the frozen
// projection. Both kernels are bandwidth-bound passes; the layer applies them
// between its unfused projections (the gate/up delta must land before the
// activation).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// The local expert whose row range holds row r: the last e with off[e] <= r.
__device__ __forceinline__ int expert_of_row(const int32_t *off, int nl, int r)
{
    int lo = 0, hi = nl;  // off[lo] <= r < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Rank factor. One wave takes RW consecutive permuted rows (RW = 64 / RK,
// RK the rank rounded up to 16, 32 or 64); lane l covers k = 512 c + 8 l .. + 8
// of chunk c. When the wave's rows belong to one expert (the common case)
// each A fragment it loads serves all RW rows; otherwise each row reads its
// expert's.
template <int RK, typename TOut>
__global__ __launch_bounds__(256) void lora_t_kernel(const bf16 *__restrict__ x, int64_t ldx,
                                                     const int32_t *__restrict__ x_rows,
                                                     const bf16 *__restrict__ la,
                                                     const int32_t *__restrict__ off, int nl,
                                                     int rank, int K, float scale,
                                                     TOut *__restrict__ t)
{
    constexpr int RW = 64 / RK;
    const int A = off[nl];
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6), lane = threadIdx.x & 63;
    const int r0 = wave * RW;
    if (r0 >= A) return;
    int64_t xrow[RW];
    const bf16 *arow[RW];
#pragma unroll
    for (int i = 0; i < RW; i++) {
        const int r = min(r0 + i, A - 1);
        xrow[i] = x_rows ? (int64_t)x_rows[r] : (int64_t)r;
        arow[i] = la + (int64_t)expert_of_row(off, nl, r) * rank * K;
    }
    // rows are grouped by expert, so a wave's rows usually share one
    const bool one_expert = arow[0] == arow[RW - 1];
    float acc[RW][RK];
#pragma unroll
    for (int i = 0; i < RW; i++)
#pragma unroll
        for (int j = 0; j < RK; j++) acc[i][j] = 0.f;
    for (int k = 8 * lane; k < K; k += 512) {
        float xv[RW][8];
#pragma unroll
        for (int i = 0; i < RW; i++) {
            const bf16x8 v = *(const bf16x8 *)(x + xrow[i] * ldx + k);
#pragma unroll
            for (int q = 0; q < 8; q++) xv[i][q] = (float)v[q];
        }
        if (one_expert) {
#pragma unroll
            for (int j = 0; j < RK; j++) {
                if (j < rank) {
                    const bf16x8 a = *(const bf16x8 *)(arow[0] + (int64_t)j * K + k);
#pragma unroll
                    for (int i = 0; i < RW; i++)
#pragma unroll
                        for (int q = 0; q < 8; q++) acc[i][j] += xv[i][q] * (float)a[q];
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < RK; j++) {
                if (j < rank) {
#pragma unroll
                    for (int i = 0; i < RW; i++) {
                        const bf16x8 a = *(const bf16x8 *)(arow[i] + (int64_t)j * K + k);
#pragma unroll
                        for (int q = 0; q < 8; q++) acc[i][j] += xv[i][q] * (float)a[q];
                    }
                }
            }
        }
    }
    // sum over the 64 lanes; lane 0 writes
#pragma unroll
    for (int i = 0; i < RW; i++) {
#pragma unroll
        for (int j = 0; j < RK; j++) {
            if (j < rank) {
                float v = acc[i][j];
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
                if (lane == 0 && r0 + i < A) store_out<TOut>(t + (int64_t)(r0 + i) * rank + j, scale * v);
            }
        }
    }
}

// Rank factors on the matrix cores, for the increment inside the GEMMs. Per
// expert the factor is a small dense product, t = scale * X_e A_e^T with X_e
// the expert's rows [rows][K] and A_e [rank][K], so it follows the GEMMs' own
// work plan: one workgroup per plan item (expert, first row, 16 to 256 rows),
// 32 rows per wave. Two adapters that read the same input (gate
// and up) are evaluated in one pass over it; their 2 rank output columns are
// covered by NT tiles of 32.
//
// Lane L: row (A operand) and adapter column (B operand) L % 32, half
// h = L / 32. For the 64-wide K chunk at kc, half h holds elements
// kc + 32 h .. + 32 of its row and of its column (64 contiguous bytes, four
// 16-byte loads) and MFMA step s (0..3) takes elements kc + 32 h + 8 s .. + 8
// of both, so every product x[k] A[j][k] enters exactly once. The loads of
// chunk c + 1 are issued before chunk c is consumed. Output rows hold the
// hi and lo bf16 parts of each factor (2 rank bf16 per row).
//
// Items of at most 32 rows (the streaming schedule's groups) leave a single
// wave per item, which cannot keep enough loads in flight to stream the
// adapter; there KS = 4 waves take a quarter of K each and add their partial
// tiles through LDS in wave order.
template <int NT, int KS>
__global__ __launch_bounds__(512) void lora_t_mfma_kernel(
    const bf16 *__restrict__ x, int64_t ldx, const int32_t *__restrict__ x_rows,
    const bf16 *__restrict__ a1, const bf16 *__restrict__ a2, int rank, int K, float scale,
    const int32_t *__restrict__ plan, int hdr, bf16 *__restrict__ t1, bf16 *__restrict__ t2)
{
    const int grp = blockIdx.x;
    if (grp >= plan[0]) return;
    const int2 it = ((const int2 *)(plan + hdr))[grp];
    const int e = it.x & 0xFFFF, rows = it.x >> 16;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
    const int rw = KS > 1 ? 0 : w;  // the wave's 32-row slice
    if (32 * rw >= rows) return;    // (KS > 1: rows <= 32, every wave stays)
    const int r0 = it.y + 32 * rw, nr = min(32, rows - 32 * rw);
    // the wave's contraction range, in units of 64
    const int n64 = K / 64, per = (n64 + KS - 1) / KS;
    const int kb = KS > 1 ? min(K, 64 * per * w) : 0, ke = KS > 1 ? min(K, 64 * per * (w + 1)) : K;
    const int prow = r0 + min(l32, nr - 1);
    const bf16 *xp = x + (x_rows ? (int64_t)x_rows[prow] : (int64_t)prow) * ldx + 32 * hf;
    const int ncol = a2 ? 2 * rank : rank;
    const bf16 *bp[NT];
    bool bon[NT];
#pragma unroll
    for (int g = 0; g < NT; g++) {
        const int c = 32 * g + l32;
        bon[g] = c < ncol;
        const bool second = bon[g] && c >= rank;
        bp[g] = (second ? a2 : a1) + ((int64_t)e * rank + (bon[g] ? c - (second ? rank : 0) : 0)) * K +
                32 * hf;
    }
    const bf16x8 zero = {};
    bf16x8 xa[2][4], bb[2][NT][4];
    auto load = [&](int buf, int kc) {
#pragma unroll
        for (int q = 0; q < 4; q++) xa[buf][q] = *(const bf16x8 *)(xp + kc + 8 * q);
#pragma unroll
        for (int g = 0; g < NT; g++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const bf16x8 v = *(const bf16x8 *)(bp[g] + kc + 8 * q);
                bb[buf][g][q] = bon[g] ? v : zero;
            }
    };
    f32x16 acc[NT];
#pragma unroll
    for (int g = 0; g < NT; g++) acc[g] = f32x16{};
    auto step = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
            for (int g = 0; g < NT; g++) acc[g] = mfma32x32x16(xa[buf][q], bb[buf][g][q], acc[g]);
    };
    if (kb < ke) {
        load(0, kb);
        for (int kc = kb; kc < ke; kc += 128) {
            if (kc + 64 < ke) load(1, kc + 64);
            step(0);
            if (kc + 128 < ke) load(0, kc + 128);
            if (kc + 64 < ke) step(1);
        }
    }
    if constexpr (KS > 1) {
        // wave 0 adds the other waves' partial tiles, in wave order
        __shared__ f32x16 part[KS - 1][NT][64];
        if (w > 0)
#pragma unroll
            for (int g = 0; g < NT; g++) part[w - 1][g][lane] = acc[g];
        __syncthreads();
        if (w > 0) return;
#pragma unroll
        for (int i = 0; i < KS - 1; i++)
#pragma unroll
            for (int g = 0; g < NT; g++) acc[g] += part[i][g][lane];
    }
    // lane holds C[8 (v / 4) + 4 h + v % 4][l32] of each column tile. Each
    // factor is stored as two bf16 parts, hi = bf16(v) at column c and
    // lo = bf16(v - hi) at column rank + c of a row of 2 rank: v - hi is exact
    // in fp32, and hi + lo matches v to 16 significant bits, so the
    // increment's MFMAs see the fp32 factor rather than one bf16 rounding.
#pragma unroll
    for (int g = 0; g < NT; g++) {
        const int c = 32 * g + l32;
        if (!bon[g]) continue;
        bf16 *tc = c < rank ? t1 + c : t2 + (c - rank);
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int rr = 8 * (v >> 2) + 4 * hf + (v & 3);
            if (rr < nr) {
                const float f = scale * acc[g][v];
                const bf16 hi = to_bf16(f);
                bf16 *dst = tc + (int64_t)(r0 + rr) * 2 * rank;
                dst[0] = hi;
                dst[rank] = to_bf16(f - (float)hi);
            }
        }
    }
}

// The delta. Block -> `rows` (1..64) consecutive permuted rows x 256
// columns, thread -> one column. The expert's B slice [256 columns][rank] is staged in LDS
// (coalesced) whenever the expert changes along the rows, then each row adds
// sum_j t[r][j] B[n][j] to y with coalesced fp32 read-modify-writes.
constexpr int LA_ROWS = 64, LA_COLS = 256, LA_LD = MOE_MAX_LORA_RANK + 2;  // rows: at most

__global__ __launch_bounds__(256) void lora_apply_kernel(const float *__restrict__ t,
                                                         const bf16 *__restrict__ lb,
                                                         const int32_t *__restrict__ off, int nl,
                                                         int rank, int N, int nchunks, int rows,
                                                         float *__restrict__ y, int64_t ldy)
{
    __shared__ bf16 bs[LA_COLS][LA_LD];
    const int A = off[nl];
    const int rb = (int)(blockIdx.x / nchunks) * rows, c0 = (int)(blockIdx.x % nchunks) * LA_COLS;
    if (rb >= A) return;
    const int tid = threadIdx.x, n = c0 + tid;
    const int r1 = min(rb + rows, A);
    int cur = -1;
    for (int r = rb; r < r1; r++) {
        const int e = expert_of_row(off, nl, r);  // the same for every thread
        if (e != cur) {
            __syncthreads();  // the previous slice is no longer read
            const bf16 *src = lb + ((int64_t)e * N + c0) * rank;
            for (int i = tid; i < LA_COLS * rank; i += 256) {
                const int c = i / rank, j = i - c * rank;
                bs[c][j] = c0 + c < N ? src[i] : (bf16)0.0f;
            }
            __syncthreads();
            cur = e;
        }
        if (n < N) {
            const float *tr = t + (int64_t)r * rank;
            float d = 0.f;
            for (int j = 0; j < rank; j++) d += tr[j] * (float)bs[tid][j];
            y[(int64_t)r * ldy + n] += d;
        }
    }
}

// h = act(g, u), fp32 in, bf16 out, 4 elements per thread.
template <int ACT>
__global__ __launch_bounds__(256) void glu_kernel(const float *__restrict__ g,
                                                  const float *__restrict__ u,
                                                  const int32_t *__restrict__ off, int nl, int I,
                                                  bf16 *__restrict__ h)
{
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= (int64_t)off[nl] * I) return;
    const float4 a = *(const float4 *)(g + i), b = *(const float4 *)(u + i);
    h[i] = to_bf16(act_apply<ACT>(a.x, b.x));
    h[i + 1] = to_bf16(act_apply<ACT>(a.y, b.y));
    h[i + 2] = to_bf16(act_apply<ACT>(a.z, b.z));
    h[i + 3] = to_bf16(act_apply<ACT>(a.w, b.w));
}

size_t lora_ws_bytes(int max_rows, int rank)
{
    return (((size_t)max_rows * rank * sizeof(float)) + 255) & ~(size_t)255;
}

hipError_t launch_lora_t(const bf16 *x, int64_t ldx, const int32_t *x_rows, const bf16 *la,
                         int rank, float scale, const int32_t *off, int nl, int max_rows, int K,
                         void *t, int t_bf16, hipStream_t s)
{
    if (max_rows <= 0) return hipSuccess;
    // rows per expert on average decide how many rows share an adapter slice:
    // few (small batches) -> one row per wave, so the grid still covers the chip
    const int mean = max(1, max_rows / max(1, nl));
    const int rk = mean < 4 ? 64 : rank <= 16 ? 16 : rank <= 32 ? 32 : 64;
    const int rw = 64 / rk;
    const int64_t waves = (max_rows + rw - 1) / rw;
    const dim3 gt((unsigned)((waves + 3) / 4)), b(256);
#define LT(R, T)                                                                                \
    hipLaunchKernelGGL((lora_t_kernel<R, T>), gt, b, 0, s, x, ldx, x_rows, la, off, nl, rank, K, \
                       scale, (T *)t)
    if (t_bf16) {
        if (rk == 16) LT(16, bf16);
        else if (rk == 32) LT(32, bf16);
        else LT(64, bf16);
    } else {
        if (rk == 16) LT(16, float);
        else if (rk == 32) LT(32, float);
        else LT(64, float);
    }
#undef LT
    return hipGetLastError();
}

hipError_t launch_lora_t_plan(const bf16 *x, int64_t ldx, const int32_t *x_rows, const bf16 *a1,
                              const bf16 *a2, int rank, int K, float scale,
                              const GemmPlanArgs &plan, bf16 *t1, bf16 *t2, hipStream_t s)
{
    if (plan.max_groups <= 0) return hipSuccess;
    const int R = plan.rows_per_group;
    if (K % 64 || rank % 16 || rank > MOE_MAX_LORA_RANK || R % 16 || (R > 32 && R % 32) || R <= 0 ||
        R > 256)
        return hipErrorInvalidValue;
    // more than 96 columns would not fit the registers: one pass per adapter
    if (a2 && 2 * rank > 96) {
        const hipError_t e = launch_lora_t_plan(x, ldx, x_rows, a1, nullptr, rank, K, scale, plan,
                                                t1, nullptr, s);
        if (e != hipSuccess) return e;
        return launch_lora_t_plan(x, ldx, x_rows, a2, nullptr, rank, K, scale, plan, t2, nullptr,
                                  s);
    }
    const int nt = ((a2 ? 2 : 1) * rank + 31) / 32;
    // one wave per 32 rows of a work item; items of at most 32 rows (the
    // streaming plan's 16-row groups) get four waves splitting K
    const bool ks = R <= 32;
    const dim3 grid((unsigned)plan.max_groups), block((unsigned)(ks ? 256 : R / 32 * 64));
#define LTP(NT, KS)                                                                           \
    hipLaunchKernelGGL((lora_t_mfma_kernel<NT, KS>), grid, block, 0, s, x, ldx, x_rows, a1, a2, \
                       rank, K, scale, plan.plan, plan.hdr, t1, t2)
    if (ks) {
        if (nt == 1) LTP(1, 4);
        else if (nt == 2) LTP(2, 4);
        else LTP(3, 4);
    } else {
        if (nt == 1) LTP(1, 1);
        else if (nt == 2) LTP(2, 1);
        else LTP(3, 1);
    }
#undef LTP
    return hipGetLastError();
}

hipError_t launch_lora(const bf16 *x, int64_t ldx, const int32_t *x_rows, const bf16 *la,
                       const bf16 *lb, int rank, float scale, const int32_t *off, int nl,
                       int max_rows, int N, int K, float *y, int64_t ldy, float *t,
                       hipStream_t s)
{
    if (max_rows <= 0) return hipSuccess;
    hipError_t e = launch_lora_t(x, ldx, x_rows, la, rank, scale, off, nl, max_rows, K, t, 0, s);
    if (e != hipSuccess) return e;
    const int mean = max(1, max_rows / max(1, nl));
    const dim3 b(256);
    const int nchunks = (N + LA_COLS - 1) / LA_COLS;
    int rows = 1;
    while (rows < mean && rows < LA_ROWS) rows *= 2;
    const int64_t rblocks = (max_rows + rows - 1) / rows;
    hipLaunchKernelGGL(lora_apply_kernel, dim3((unsigned)(rblocks * nchunks)), b, 0, s, t, lb,
                       off, nl, rank, N, nchunks, rows, y, ldy);
    return hipGetLastError();
}

hipError_t launch_glu(const float *g, const float *u, const int32_t *off, int nl, int max_rows,
                      int I, int act, bf16 *h, hipStream_t s)
{
    const int64_t n4 = (int64_t)max_rows * I / 4;
    if (n4 <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
    if (act == ACT_GELU_TANH_MUL)
        hipLaunchKernelGGL(glu_kernel<ACT_GELU_TANH_MUL>, grid, block, 0, s, g, u, off, nl, I, h);
    else
        hipLaunchKernelGGL(glu_kernel<ACT_SILU_MUL>, grid, block, 0, s, g, u, off, nl, I, h);
    return hipGetLastError();
}

}  // namespace moe
