// Routing kernels: router scores (a dense GEMM on the bf16 matrix cores with
// the fp32 router weights split into three exact bf16 parts), and a
// wavefront-per-token top-k select with softmax weights and the expert
// histogram.
//
// Sources: P2 "SGLang 0.5.17：Kimi K3 原生 MXFP4 推理架构解析", section
// "MoE 稀疏激活" (score every token against every expert, keep the best 16,
// weight the kept experts' outputs); P1 "从Kimi K3到MiniMax-H3", section 一
// (896 experts, 16 active, routing in the 3584-wide latent space).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Router scores: logits[t][e] = sum_i x[t][i] * W[e][i] + bias[e].
//
// W (fp32) = hi + mid + lo exactly, each part bf16, so every product with a
// bf16 token element is exact in fp32; the matrix cores accumulate in fp32.
// Workgroup tile: 64 tokens x 64 experts, 4 waves, each wave 16 tokens x 64
// experts (4 accumulator tiles). The W tile of one 128-wide K step is split
// once into LDS (3 parts) and shared by the 4 waves; token rows come straight
// from global memory (each row is read by one wave only).
//
// Contraction mapping inside a 128-wide K step: lane group g = L / 16 owns
// K offsets [32 g, 32 g + 32); MFMA step s (0..3) takes the 8 elements
// 32 g + 8 s .. +8, for both operands.
// ---------------------------------------------------------------------------
constexpr int RT_TOK = 64, RT_EXP = 64, RT_K = 128;

__global__ __launch_bounds__(256) void router_logits_kernel(
    const bf16 *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int d, int E, int k_per_split,
    int32_t *__restrict__ zero_counts)
{
    // the histogram the top-k kernel fills next starts from zero
    if (zero_counts && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
        for (int i = threadIdx.x; i < E; i += blockDim.x) zero_counts[i] = 0;
    // blockIdx.z selects a K range; with more than one range each writes its
    // partial sums to its own [T][E] plane (no bias) and the top-k kernel adds
    // the planes in order.
    const int kbeg = blockIdx.z * k_per_split, kend = kbeg + k_per_split;
    logits += (int64_t)blockIdx.z * T * E;
    if (gridDim.z > 1) bias = nullptr;
    // LDS: [part][expert][K] bf16, padded rows to spread banks.
    constexpr int LDK = RT_K + 8;
    __shared__ bf16 wpart[3][RT_EXP][LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * RT_TOK, e0 = blockIdx.y * RT_EXP;
    const int m = lane & 15, g = lane >> 4;
    const int tok = t0 + wave * 16 + m;
    const bool tok_ok = tok < T;
    const bf16 *xrow = x + (int64_t)(tok_ok ? tok : 0) * d;

    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; nb++) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = kbeg; k0 < kend; k0 += RT_K) {
        // Stage and split the W tile: 64 experts x 128 K fp32 = 8192 values,
        // 32 per thread as 8 float4 loads.
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 8; it++) {
            int idx4 = it * 256 + tid;         // float4 index inside the tile
            int er = idx4 / (RT_K / 4);        // expert row 0..63
            int kc = (idx4 % (RT_K / 4)) * 4;  // K offset
            int e = e0 + er;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < E) v = *(const float4 *)(w + (int64_t)e * d + k0 + kc);
            float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; c++) {
                bf16 h, md, lo;
                split3_bf16(vv[c], h, md, lo);
                wpart[0][er][kc + c] = h;
                wpart[1][er][kc + c] = md;
                wpart[2][er][kc + c] = lo;
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int kk = 32 * g + 8 * s;
            bf16x8 a = bf16x8{};
            if (tok_ok) a = *(const bf16x8 *)(xrow + k0 + kk);
#pragma unroll
            for (int nb = 0; nb < 4; nb++) {
                const int er = nb * 16 + m;
#pragma unroll
                for (int p = 0; p < 3; p++) {
                    bf16x8 b = *(const bf16x8 *)(&wpart[p][er][kk]);
                    acc[nb] = mfma16x16x32(a, b, acc[nb]);
                }
            }
        }
    }
    // C layout: lane holds C[4*g + i][m] for its 16x16 tile: token row
    // 4*g+i of the wave's 16, expert column m of n-block nb.
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
        const int e = e0 + nb * 16 + m;
        if (e >= E) continue;
        const float b = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = t0 + wave * 16 + 4 * g + i;
            if (t < T) logits[(int64_t)t * E + e] = acc[nb][i] + b;
        }
    }
}

// ---------------------------------------------------------------------------
// Router scores for larger batches: the fp32 weights are split once into
// three bf16 planes Wp[p][e][i] (hi, mid, lo; exact sum), then
//   logits[t][e] = sum_p sum_i x[t][i] * Wp[p][e][i]  (+ bias)
// is one bf16 GEMM over K' = 3 d on the 32x32x16 matrix cores. Workgroup
// tile 128 tokens x 128 experts, K step 64, both operands double-buffered in
// LDS, 4 waves of 64 x 64. blockIdx.y splits K' into planes of partial sums
// when the tile grid alone is too small for the chip.
// ---------------------------------------------------------------------------
constexpr int RG_BM = 128, RG_BN = 128, RG_BK = 64, RG_LD = RG_BK + 8;

__global__ __launch_bounds__(256) void split_router_kernel(const float *__restrict__ w,
                                                           int64_t n, bf16 *__restrict__ wp)
{
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    const float4 v = *(const float4 *)(w + i);
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; c++) {
        bf16 h, md, lo;
        split3_bf16(vv[c], h, md, lo);
        wp[i + c] = h;
        wp[n + i + c] = md;
        wp[2 * n + i + c] = lo;
    }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256, 2) void router_tile_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ wp, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int d, int E, int ksteps_per_split,
    int32_t *__restrict__ zero_counts)
{
    if (zero_counts && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < E; i += blockDim.x) zero_counts[i] = 0;
    __shared__ __attribute__((aligned(16))) bf16 As[2][RG_BM][RG_LD];
    __shared__ __attribute__((aligned(16))) bf16 Bs[2][RG_BN][RG_LD];
    const int n_nb = (E + RG_BN - 1) / RG_BN;
    const int mb = blockIdx.x / n_nb, nb = blockIdx.x - mb * n_nb;
    const int t0 = mb * RG_BM, e0 = nb * RG_BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int steps_d = d / RG_BK;
    const int kt0 = blockIdx.y * ksteps_per_split, kt1 = kt0 + ksteps_per_split;
    logits += (int64_t)blockIdx.y * T * E;
    if (gridDim.y > 1) bias = nullptr;

    // global -> LDS: thread -> row tid / 2, 64 bytes at column 32 * (tid % 2)
    const int lr = tid >> 1, lc = (tid & 1) * 32;
    const bf16 *xa = x + (int64_t)min(t0 + lr, T - 1) * d + lc;
    const int eb = min(e0 + lr, E - 1);
    u32x4 ra[4], rb[4];
    auto gload = [&](int kt) {
        const int p = kt / steps_d, k0 = (kt - p * steps_d) * RG_BK;
        const bf16 *wb = wp + ((int64_t)p * E + eb) * d + lc + k0;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            ra[c] = *(const u32x4 *)(xa + k0 + 8 * c);
            rb[c] = *(const u32x4 *)(wb + 8 * c);
        }
    };
    auto lstore = [&](int st) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            *(u32x4 *)(&As[st][lr][lc + 8 * c]) = ra[c];
            *(u32x4 *)(&Bs[st][lr][lc + 8 * c]) = rb[c];
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;
    const bool mt_on[2] = {t0 + wm * 64 < T, t0 + wm * 64 + 32 < T};

    gload(kt0);
    lstore(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; kt++) {
        const int st = (kt - kt0) & 1;
        if (kt + 1 < kt1) gload(kt + 1);
        if (mt_on[0]) {
#pragma unroll
            for (int s = 0; s < 4; s++) {
                bf16x8 b[2];
#pragma unroll
                for (int j = 0; j < 2; j++)
                    b[j] = *(const bf16x8 *)(&Bs[st][wn * 64 + 32 * j + l32][32 * h + 8 * s]);
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    if (!mt_on[i]) continue;
                    const bf16x8 a = *(const bf16x8 *)(&As[st][wm * 64 + 32 * i + l32][32 * h + 8 * s]);
#pragma unroll
                    for (int j = 0; j < 2; j++) acc[i][j] = mfma32x32x16(a, b[j], acc[i][j]);
                }
            }
        }
        if (kt + 1 < kt1) lstore(st ^ 1);
        __syncthreads();
    }
    // lane holds C[8 (v / 4) + 4 h + v % 4][l32] of each 32 x 32 tile
#pragma unroll
    for (int i = 0; i < 2; i++) {
        if (!mt_on[i]) continue;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int e = e0 + wn * 64 + 32 * j + l32;
            if (e >= E) continue;
            const float b = bias ? bias[e] : 0.f;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int t = t0 + wm * 64 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (t < T) logits[(int64_t)t * E + e] = acc[i][j][v] + b;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Top-k select, softmax, histogram: one wavefront per token.
//
// A score maps to a 64-bit key that orders (score desc, expert asc):
// the fp32 bits made monotone (with -0 folded onto +0) in the high word, the
// complemented expert id in the low word. k rounds of a wave-wide max pick
// the winners best first; the winning lane retires its element.
// ---------------------------------------------------------------------------
constexpr int TK_MAX_PER_LANE = MOE_MAX_EXPERTS_DEV / 64;

__device__ __forceinline__ uint64_t score_key(float v, int e)
{
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) == 0) u = 0;  // -0 == +0
    uint32_t mono = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)mono << 32) | (uint32_t)(~(uint32_t)e);
}

// The score a key was built from (exact; -0 comes back as +0, which changes
// neither the order nor exp(l - max)).
__device__ __forceinline__ float key_score(uint64_t key)
{
    uint32_t mono = (uint32_t)(key >> 32);
    uint32_t u = (mono & 0x80000000u) ? (mono & 0x7fffffffu) : ~mono;
    return __uint_as_float(u);
}

// One DPP step: v = max(v, v taken from the lane `ctrl` names); lanes the
// pattern leaves without a source keep their own value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v)
{
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const uint32_t olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false);
    const uint32_t ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > v ? o : v;
}

// Maximum over the 64 lanes, returned to every lane (wave-uniform). Within
// each row of 16 lanes: quad swaps, half-row and row mirrors; then rows are
// chained with the row broadcasts so lane 63 holds the maximum, which is read
// back as a scalar.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    v = dpp_max_step<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_step<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_step<0x141, 0xf>(v);  // row_half_mirror
    v = dpp_max_step<0x140, 0xf>(v);  // row_mirror
    v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int32_t *__restrict__ counts)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *l = logits + (int64_t)t * E;

    // all of the token's scores in flight at once (indices clamped, keys of
    // padding lanes zeroed afterwards)
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; i++) v[i] = l[min(i * 64 + lane, E - 1)];
    uint64_t key[NPL];
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPL; i++) {
        const int e = i * 64 + lane;
        key[i] = e < E ? score_key(v[i], e) : 0ull;  // 0 never wins over a real key
        best = key[i] > best ? key[i] : best;
    }

    float my_score = 0.f;
    int my_idx = 0;
    for (int j = 0; j < k; j++) {
        const uint64_t win = wave_max_u64(best);  // wave-uniform
        if (lane == j) {
            my_idx = (int)(~(uint32_t)win);
            my_score = key_score(win);
        }
        // retire the winner (exactly one element matches) and refresh maxima
        best = 0;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
            key[i] = key[i] == win ? 0ull : key[i];
            best = key[i] > best ? key[i] : best;
        }
    }
    const float top = __shfl(my_score, 0, 64);
    const float z = (lane < k) ? expf(my_score - top) : 0.f;
    float sum = 0.f;
    for (int j = 0; j < k; j++) sum += __shfl(z, j, 64);  // j order, as a plain loop
    if (lane < k) {
        topk_idx[(int64_t)t * k + lane] = my_idx;
        topk_w[(int64_t)t * k + lane] = z / sum;
        atomicAdd(&counts[my_idx], 1);
    }
}

// Router scores from split-K planes: logits = sum of the planes in order +
// bias. Four consecutive scores per thread, every plane's load issued before
// the sums.
__global__ __launch_bounds__(256) void sum_planes_kernel(const float *__restrict__ planes,
                                                         int n_planes, int64_t plane, int E,
                                                         const float *__restrict__ bias,
                                                         float *__restrict__ logits)
{
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= plane) return;
    float4 acc = *(const float4 *)(planes + i4);
    int p = 1;
    for (; p + 4 <= n_planes; p += 4) {
        const float4 a = *(const float4 *)(planes + p * plane + i4);
        const float4 b = *(const float4 *)(planes + (p + 1) * plane + i4);
        const float4 c = *(const float4 *)(planes + (p + 2) * plane + i4);
        const float4 d = *(const float4 *)(planes + (p + 3) * plane + i4);
        acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
        acc.x += b.x; acc.y += b.y; acc.z += b.z; acc.w += b.w;
        acc.x += c.x; acc.y += c.y; acc.z += c.z; acc.w += c.w;
        acc.x += d.x; acc.y += d.y; acc.z += d.z; acc.w += d.w;
    }
    for (; p < n_planes; p++) {
        const float4 a = *(const float4 *)(planes + p * plane + i4);
        acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
    }
    if (bias) {
        const int e = (int)(i4 % E);  // E % 4 == 0: the four scores share a row
        acc.x += bias[e]; acc.y += bias[e + 1]; acc.z += bias[e + 2]; acc.w += bias[e + 3];
    }
    *(float4 *)(logits + i4) = acc;
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v)
{
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n,
                       v);
    return hipGetLastError();
}

hipError_t launch_router_logits(const bf16 *x, const float *w, const float *bias, float *logits,
                                int T, int d, int E, int splits, int32_t *zero_counts,
                                hipStream_t s)
{
    dim3 grid((T + RT_TOK - 1) / RT_TOK, (E + RT_EXP - 1) / RT_EXP, splits);
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, s, x, w, bias, logits, T, d, E,
                       d / splits, zero_counts);
    return hipGetLastError();
}

hipError_t launch_sum_planes(const float *planes, int n_planes, const float *bias, float *logits,
                             int T, int E, hipStream_t s)
{
    const int64_t plane = (int64_t)T * E;
    const int64_t threads = plane / 4;
    if (threads <= 0) return hipSuccess;
    hipLaunchKernelGGL(sum_planes_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       planes, n_planes, plane, E, bias, logits);
    return hipGetLastError();
}

hipError_t launch_split_router(const float *w, int E, int d, bf16 *wp, hipStream_t s)
{
    const int64_t n = (int64_t)E * d;
    hipLaunchKernelGGL(split_router_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s,
                       w, n, wp);
    return hipGetLastError();
}

int router_tile_splits(int T, int d, int E, int target_blocks)
{
    const int tiles = ((T + RG_BM - 1) / RG_BM) * ((E + RG_BN - 1) / RG_BN);
    const int steps = 3 * (d / RG_BK);
    if (E % 4) return 1;
    int best = 1;
    for (int sp = 1; sp <= steps; sp++) {
        if (steps % sp) continue;
        if ((int64_t)tiles * sp > target_blocks) break;
        best = sp;
    }
    return best;
}

hipError_t launch_router_tile(const bf16 *x, const bf16 *wp, const float *bias, float *logits,
                              int T, int d, int E, int splits, int32_t *zero_counts,
                              hipStream_t s)
{
    const int tiles = ((T + RG_BM - 1) / RG_BM) * ((E + RG_BN - 1) / RG_BN);
    const int steps = 3 * (d / RG_BK);
    hipLaunchKernelGGL(router_tile_kernel, dim3(tiles, splits), dim3(256), 0, s, x, wp, bias,
                       logits, T, d, E, steps / splits, zero_counts);
    return hipGetLastError();
}

int router_splits(int T, int d, int E, int target_blocks)
{
    if (E % 4) return 1;  // the plane sum reads scores four at a time
    // Split K while the token x expert tiles alone leave the chip idle. Each
    // split is a whole number of 128-wide K steps.
    const int tiles = ((T + RT_TOK - 1) / RT_TOK) * ((E + RT_EXP - 1) / RT_EXP);
    const int steps = d / RT_K;
    int best = 1;
    for (int sp = 1; sp <= steps; sp++) {
        if (steps % sp) continue;
        if ((int64_t)tiles * sp > target_blocks) break;
        best = sp;
    }
    return best;
}

hipError_t launch_topk_softmax(const float *logits, int T, int E, int k, int32_t *idx, float *w,
                               int32_t *counts, hipStream_t s)
{
    dim3 grid((T + 3) / 4);
    const int npl = (E + 63) / 64;
#define TK_CASE(N)                                                                            \
    if (npl <= N) {                                                                           \
        hipLaunchKernelGGL(topk_softmax_kernel<N>, grid, dim3(256), 0, s, logits, T, E, k, idx, \
                           w, counts);                                                        \
        return hipGetLastError();                                                             \
    }
    TK_CASE(2)
    TK_CASE(4)
    TK_CASE(8)
    TK_CASE(14)
    TK_CASE(16)
    TK_CASE(TK_MAX_PER_LANE)
#undef TK_CASE
    return hipErrorInvalidValue;
}

}  // namespace moe
