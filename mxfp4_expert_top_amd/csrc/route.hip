// Routing kernels: router scores (a dense GEMM on the bf16 matrix cores with
// the fp32 router weights split into bf16 parts: three exact ones for the
// bandwidth-bound small batches, two for the MFMA-bound tiled router), and a
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
// Router scores for small batches (T <= 16 NT, NT <= 4): weight streaming.
//
// The fp32 router weights are the streamed operand. Lane (m, g) of a wave
// reads 8 consecutive K elements of expert e0 + m per 32-wide K step, splits
// them into the three exact bf16 parts in registers and multiplies each part
// against every token (NT tiles of 16 rows) on the 16x16x32 matrix cores.
// Workgroup = 16 experts x one K range (blockIdx.y) that its four waves split
// four ways; their partial tiles are added in LDS in wave order. With more
// than one K range each range writes a plane [T][E] of partial sums (no bias)
// and the top-k kernel adds the planes in order.
// ---------------------------------------------------------------------------
constexpr int RS_STEP = 32, RS_BATCH = 8;

template <int NT>
__global__ __launch_bounds__(256) void router_skinny_kernel(
    const bf16 *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ out, int T, int d, int E, int steps, int32_t *__restrict__ zero_counts)
{
    if (zero_counts && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < E; i += blockDim.x) zero_counts[i] = 0;
    __shared__ f32x4 red[4][NT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int e0 = blockIdx.x * 16;
    out += (int64_t)blockIdx.y * T * E;
    // this wave's K range: steps x 32 elements; the lane's 8 at offset 8 g
    const int64_t k0 = ((int64_t)blockIdx.y * 4 + wave) * steps * RS_STEP + 8 * g;
    const float *wp = w + (int64_t)min(e0 + m, E - 1) * d + k0;
    const bf16 *xp[NT];
#pragma unroll
    for (int i = 0; i < NT; i++) xp[i] = x + (int64_t)min(16 * i + m, T - 1) * d + k0;

    f32x4 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < steps; s0 += RS_BATCH) {
        // a batch of steps in flight at once (steps past the end repeat the
        // last one and are not used)
        float4 wa[RS_BATCH], wb[RS_BATCH];
        bf16x8 xa[RS_BATCH][NT];
#pragma unroll
        for (int b = 0; b < RS_BATCH; b++) {
            const int st = min(s0 + b, steps - 1) * RS_STEP;
            wa[b] = *(const float4 *)(wp + st);
            wb[b] = *(const float4 *)(wp + st + 4);
#pragma unroll
            for (int i = 0; i < NT; i++) xa[b][i] = *(const bf16x8 *)(xp[i] + st);
        }
#pragma unroll
        for (int b = 0; b < RS_BATCH; b++) {
            if (s0 + b < steps) {
                const float v[8] = {wa[b].x, wa[b].y, wa[b].z, wa[b].w,
                                    wb[b].x, wb[b].y, wb[b].z, wb[b].w};
                bf16x8 hi, mid, lo;
#pragma unroll
                for (int c = 0; c < 8; c++) {
                    bf16 h_, m_, l_;
                    split3_bf16(v[c], h_, m_, l_);
                    hi[c] = h_;
                    mid[c] = m_;
                    lo[c] = l_;
                }
#pragma unroll
                for (int i = 0; i < NT; i++) {
                    acc[i] = mfma16x16x32(xa[b][i], hi, acc[i]);
                    acc[i] = mfma16x16x32(xa[b][i], mid, acc[i]);
                    acc[i] = mfma16x16x32(xa[b][i], lo, acc[i]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NT; i++) red[wave][i][lane] = acc[i];
    __syncthreads();
    // lane l of tile i holds C[4 (l / 16) + q][l % 16]: token 16 i + 4 (l / 16) + q,
    // expert e0 + l % 16
    for (int j = threadIdx.x; j < NT * 64; j += 256) {
        const int i = j >> 6, l = j & 63;
        f32x4 r = red[0][i][l];
#pragma unroll
        for (int wv = 1; wv < 4; wv++) {
            const f32x4 o = red[wv][i][l];
            r[0] += o[0]; r[1] += o[1]; r[2] += o[2]; r[3] += o[3];
        }
        const int e = e0 + (l & 15);
        if (e >= E) continue;
        const float bb = bias ? bias[e] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int t = 16 * i + 4 * (l >> 4) + q;
            if (t < T) out[(int64_t)t * E + e] = r[q] + bb;
        }
    }
}

// ---------------------------------------------------------------------------
// Router scores for larger batches (the MFMA-bound case): the fp32 weights
// are split once into RG_P = 2 bf16 planes Wp[p][e][i] (hi, mid, each rounded
// to nearest; hi + mid holds 16 of fp32's 24 significant bits, within
// 2^-17 |w| of the weight), then
//   logits[t][e] = sum_i sum_p x[t][i] * Wp[p][e][i]  (+ bias)
// on the 32x32x16 matrix cores. A third plane would make every product exact
// for one more MFMA per fragment; the scores' own contract is
// |l - l_exact| <= 1e-4 max(1, |l|), and two planes leave an error of about
// 2^-17 / sqrt(3) of the rms of x w per term summed over d (~4e-6 on the
// workloads' scores), so the third plane is spent on nothing. Workgroup tile
// 256 tokens x 256 experts, K step 32 of d covering both planes: each token
// fragment read from LDS feeds both planes' MFMAs. 8 waves of 128 tokens x 64
// experts. blockIdx.y splits d into ranges whose partial sums go to separate
// planes when the tile grid alone is too small for the chip.
//
// Operands go from memory straight into a two-stage LDS ring with
// global_load_lds_dwordx4 (16 bytes per lane at the wave's LDS base + 16
// lane): step k + 1 is in flight while step k's MFMAs run, and one wait and
// barrier per step both publish step k + 1 and free step k's stage. A stage
// holds 256 token rows and 2 x 256 weight rows of 64 bytes (32 bf16), 48 KB;
// the 16-byte chunk c of row r sits at position c ^ ((r / 4) % 4), which
// keeps the 32-lane fragment reads free of bank conflicts without padding.
// 16 waves of 64 x 64 (RG_WAVES = 16) measured level with 8 waves.
// ---------------------------------------------------------------------------
constexpr int RG_BM = 256, RG_BN = 256, RG_BK = 32, RG_WAVES = 8, RG_THREADS = 64 * RG_WAVES;
constexpr int RG_P = 2;  // bf16 planes of the weights
constexpr int RG_TPW = RG_BM / (RG_WAVES / 4), RG_NI = RG_TPW / 32;  // tokens per wave, 32-row tiles
constexpr int RG_ROW = RG_BK * 2;                                 // bytes per LDS row
constexpr int RG_A_BYTES = RG_BM * RG_ROW;                        // 16 KB
constexpr int RG_STAGE = RG_A_BYTES + RG_P * RG_BN * RG_ROW;      // 48 KB
constexpr size_t RG_LDS = (size_t)2 * RG_STAGE;                   // 96 KB
// 1 KB DMA blocks (16 rows) per stage: 16 token blocks, 16 per weight plane;
// each wave moves an equal share of them
constexpr int RG_A_DMA = RG_BM / 16 / RG_WAVES, RG_B_DMA = RG_P * RG_BN / 16 / RG_WAVES;
static_assert(RG_A_DMA * RG_WAVES * 16 == RG_BM && RG_B_DMA * RG_WAVES * 16 == RG_P * RG_BN,
              "DMA blocks split evenly over the waves");

__device__ __forceinline__ int rg_swz(int r, int c) { return c ^ ((r >> 2) & 3); }

__global__ __launch_bounds__(256) void split_router_kernel(const float *__restrict__ w,
                                                           int64_t n, bf16 *__restrict__ wp)
{
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    const float4 v = *(const float4 *)(w + i);
    const float vv[4] = {v.x, v.y, v.z, v.w};
    // one 8-byte store per plane
    bf16x4 h, md;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        bf16 a, b;
        split2_bf16(vv[c], a, b);
        h[c] = a;
        md[c] = b;
    }
    *(bf16x4 *)(wp + i) = h;
    *(bf16x4 *)(wp + n + i) = md;
}

__global__ __launch_bounds__(RG_THREADS, 1) void router_tile_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ wp, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int d, int E, int ksteps_per_split,
    int32_t *__restrict__ zero_counts)
{
    if (zero_counts && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < E; i += blockDim.x) zero_counts[i] = 0;
    extern __shared__ __attribute__((aligned(16))) uint8_t rg_lds[];
    const int n_nb = (E + RG_BN - 1) / RG_BN;
    // XCD-aware order: XCD b % 8 takes a contiguous range of tiles, token
    // block major, so the expert blocks of a token block share one L2
    const int tiles = (T + RG_BM - 1) / RG_BM * n_nb;
    const int per_xcd = (tiles + 7) / 8;
    const int wi = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if ((int)(blockIdx.x / 8) >= per_xcd || wi >= tiles) return;
    const int mb = wi / n_nb, nb = wi - mb * n_nb;
    const int t0 = mb * RG_BM, e0 = nb * RG_BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases in M0
    const int wm = wave >> 2, wn = wave & 3;  // RG_TPW tokens x 64 experts per wave
    const int h = lane >> 5, l32 = lane & 31;
    const int kt0 = blockIdx.y * ksteps_per_split, kt1 = kt0 + ksteps_per_split;
    logits += (int64_t)blockIdx.y * T * E;
    if (gridDim.y > 1) bias = nullptr;

    // DMA sources. Within a 16-row block lane L fills LDS position L % 4 of
    // row L / 4, so it loads the chunk that position holds. Rows past T or E
    // repeat the last real row (their results are never stored).
    const int dr = lane >> 2, dc = rg_swz(dr, lane & 3);
    const bf16 *src[RG_A_DMA + RG_B_DMA];
#pragma unroll
    for (int i = 0; i < RG_A_DMA; i++) {
        const int r = 16 * (RG_A_DMA * wave + i) + dr;
        src[i] = x + (int64_t)min(t0 + r, T - 1) * d + 8 * dc;
    }
#pragma unroll
    for (int i = 0; i < RG_B_DMA; i++) {
        const int blk = RG_B_DMA * wave + i, p = blk >> 4, r = 16 * (blk & 15) + dr;
        src[RG_A_DMA + i] = wp + ((int64_t)p * E + min(e0 + r, E - 1)) * d + 8 * dc;
    }
    const uint32_t lds0 = lds_address(rg_lds);
    auto issue = [&](int kt, int st) {
        const int k0 = kt * RG_BK;
        const uint32_t base = lds0 + st * RG_STAGE;
#pragma unroll
        for (int i = 0; i < RG_A_DMA; i++)
            dma16(src[i] + k0, base + 1024 * (RG_A_DMA * wave + i));
#pragma unroll
        for (int i = 0; i < RG_B_DMA; i++)
            dma16(src[RG_A_DMA + i] + k0, base + RG_A_BYTES + 1024 * (RG_B_DMA * wave + i));
    };

    f32x16 acc[RG_NI][2];
#pragma unroll
    for (int i = 0; i < RG_NI; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;
    // the wave's tokens hold at least one real row and its 64 experts one real expert
    const bool on = t0 + wm * RG_TPW < T && e0 + wn * 64 < E;
    // fragment rows: token rows wm RG_TPW + 32 i + l32, expert rows wn 64 + 32 j + l32
    // (row / 4 % 4 is l32 / 4 % 4 for all of them)
    const int swz = (l32 >> 2) & 3;
    const int a_off = (wm * RG_TPW + l32) * RG_ROW, b_off = RG_A_BYTES + (wn * 64 + l32) * RG_ROW;

    issue(kt0, 0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    for (int kt = kt0; kt < kt1; kt++) {
        const int st = (kt - kt0) & 1;
        if (kt + 1 < kt1) issue(kt + 1, st ^ 1);
        if (on) {
            const uint8_t *S = rg_lds + st * RG_STAGE;
#pragma unroll
            for (int s = 0; s < 2; s++) {
                const int cpos = 16 * ((2 * s + h) ^ swz);
                bf16x8 a[RG_NI];
#pragma unroll
                for (int i = 0; i < RG_NI; i++)
                    a[i] = *(const bf16x8 *)(S + a_off + 32 * i * RG_ROW + cpos);
#pragma unroll
                for (int p = 0; p < RG_P; p++) {
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const bf16x8 b = *(const bf16x8 *)(S + b_off + (p * RG_BN + 32 * j) * RG_ROW +
                                                           cpos);
#pragma unroll
                        for (int i = 0; i < RG_NI; i++) acc[i][j] = mfma32x32x16(a[i], b, acc[i][j]);
                    }
                }
            }
        }
        // this wave's loads of step kt + 1 have landed and every wave is done
        // with stage st: publish the one, free the other
        asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // lane holds C[8 (v / 4) + 4 h + v % 4][l32] of each 32 x 32 tile
    if (!on) return;
#pragma unroll
    for (int i = 0; i < RG_NI; i++) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int e = e0 + wn * 64 + 32 * j + l32;
            if (e >= E) continue;
            const float bb = bias ? bias[e] : 0.f;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int t = t0 + wm * RG_TPW + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (t < T) logits[(int64_t)t * E + e] = acc[i][j][v] + bb;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Top-k select, softmax, histogram: one wavefront per token.
//
// A score maps to a 64-bit key that orders (score desc, expert asc): the fp32
// bits made monotone (with -0 folded onto +0) in the high word, the
// complemented expert id in the low word. Keys are distinct, so the k winners
// are the keys of rank 0..k-1, where a key's rank is the number of larger
// keys. A token's 14 keys per lane are too many to rank directly, so:
//   1. each lane's largest key is ranked among the 64 lane maxima; tau, the
//      maximum of rank k-1, is a lower bound of the winners (k lanes hold a
//      key >= tau);
//   2. the keys >= tau (usually about 20) are packed into LDS and ranked
//      among themselves: ranks 0..k-1 are the winners, best first.
// More than 64 candidates (only for unusual score patterns) take k rounds of
// a wave-wide maximum instead. Every step is a short fixed sequence: no
// chains of k or 32 dependent rounds.
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

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Number of the 64 keys in LDS that are larger than `mine`.
__device__ __forceinline__ int rank64(const uint64_t *s, uint64_t mine)
{
    int r = 0;
#pragma unroll
    for (int j = 0; j < 64; j++) r += s[j] > mine ? 1 : 0;
    return r;
}

// With n_planes > 1 the scores are first assembled from split-K planes of
// partial sums: plane 0 + plane 1 + ... in that order, then the bias, and
// written to `logits`; with one plane `src` already holds the final scores.
template <int NPL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float *__restrict__ src, int n_planes, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int E, int k, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int32_t *__restrict__ counts)
{
    // planes loaded per batch: 8 planes of 14 scores took 186 VGPRs (two waves
    // per SIMD, the top-k of 16 K tokens 40 us); with 2, 76 VGPRs and 25 us
    constexpr int PB = NPL <= 8 ? 8 : 2;
    __shared__ uint64_t s_key[4][64];
    __shared__ uint64_t s_ord[4][MOE_MAX_TOPK_DEV];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    // a wave past the last token repeats it and stores nothing (every wave
    // reaches the barriers)
    const bool t_ok = t < T;
    const int tt = t_ok ? t : T - 1;
    const int64_t plane = (int64_t)T * E;
    const float *l = src + (int64_t)tt * E;

    // the token's scores: one batch of loads per PB planes (indices clamped)
    float v[NPL];
    if (n_planes == 1) {
#pragma unroll
        for (int i = 0; i < NPL; i++) v[i] = l[min(i * 64 + lane, E - 1)];
    } else {
        for (int p = 0; p < n_planes; p += PB) {
            float u[PB][NPL];
#pragma unroll
            for (int q = 0; q < PB; q++)
#pragma unroll
                for (int i = 0; i < NPL; i++)
                    u[q][i] = l[min(p + q, n_planes - 1) * plane + min(i * 64 + lane, E - 1)];
#pragma unroll
            for (int i = 0; i < NPL; i++) v[i] = p == 0 ? u[0][i] : v[i] + u[0][i];
#pragma unroll
            for (int q = 1; q < PB; q++)
                if (p + q < n_planes)
#pragma unroll
                    for (int i = 0; i < NPL; i++) v[i] += u[q][i];
        }
        float *lo = logits + (int64_t)tt * E;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
            const int e = i * 64 + lane;
            if (e < E) {
                if (bias) v[i] += bias[e];
                if (t_ok) lo[e] = v[i];
            }
        }
    }
    uint64_t key[NPL];
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPL; i++) {
        const int e = i * 64 + lane;
        key[i] = e < E ? score_key(v[i], e) : 0ull;  // 0 ranks below every real key
        best = key[i] > best ? key[i] : best;
    }

    // candidates, one per lane (0 past the count)
    uint64_t cand = best;
    int ncand = 64;
    if constexpr (NPL > 1) {
        // E > 64: every lane holds a real key, so the 64 maxima are distinct
        s_key[wv][lane] = best;
        __syncthreads();
        const int r0 = rank64(s_key[wv], best);
        const uint64_t at = __ballot(r0 == k - 1);  // exactly one lane
        const uint64_t tau = readlane_u64(best, (int)__builtin_ctzll(at));
        __syncthreads();
        int base = 0;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
            const bool p = key[i] >= tau;
            const uint64_t msk = __ballot(p);
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                       (uint32_t)(msk >> 32),
                                       __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
            if (p && pos < 64) s_key[wv][pos] = key[i];
            base += __popcll(msk);
        }
        ncand = base;
        if (lane >= ncand) s_key[wv][lane] = 0ull;
        __syncthreads();
        cand = lane < ncand ? s_key[wv][lane] : 0ull;
    } else {
        s_key[wv][lane] = cand;
        __syncthreads();
    }
    // rank the candidates (zeros past the count rank below all of them)
    if (ncand <= 64) {
        const int r = rank64(s_key[wv], cand);
        if (lane < ncand && r < k) s_ord[wv][r] = cand;
    }
    __syncthreads();
    uint64_t my = 0;
    if (ncand <= 64) {
        if (lane < k) my = s_ord[wv][lane];
    } else {
        // k rounds of a wave-wide maximum; the winner's slot is retired
        for (int j = 0; j < k; j++) {
            const uint64_t win = wave_max_u64(best);
            if (lane == j) my = win;
            best = 0;
#pragma unroll
            for (int i = 0; i < NPL; i++) {
                key[i] = key[i] == win ? 0ull : key[i];
                best = key[i] > best ? key[i] : best;
            }
        }
    }
    const int my_idx = (int)(~(uint32_t)my);
    const float my_score = key_score(my);

    // softmax over the selected scores, summed best first
    const float top = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(my_score)));
    const float z = (lane < k) ? expf(my_score - top) : 0.f;
    float sum = 0.f;
    for (int j = 0; j < k; j++)
        sum += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(z), j));
    if (t_ok && lane < k) {
        topk_idx[(int64_t)t * k + lane] = my_idx;
        topk_w[(int64_t)t * k + lane] = z / sum;
        if (counts) atomicAdd(&counts[my_idx], 1);
    }
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
    const int steps = d / RG_BK;
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
    const int steps = d / RG_BK;
    hipError_t err = ensure_dynamic_lds((const void *)router_tile_kernel, (int)RG_LDS);
    if (err != hipSuccess) return err;
    // a grid of 8 * ceil(tiles / 8) blocks covers every tile in the XCD-aware order
    const unsigned G = (unsigned)((tiles + 7) / 8 * 8);
    hipLaunchKernelGGL(router_tile_kernel, dim3(G, splits), dim3(RG_THREADS), RG_LDS, s, x, wp,
                       bias, logits, T, d, E, steps / splits, zero_counts);
    return hipGetLastError();
}

int router_skinny_splits(int T, int d, int E, int target_blocks)
{
    (void)T;
    // K ranges of 4 x 32 x steps elements; the largest count whose grid
    // stays within target_blocks, at most 4 planes for the top-k kernel
    const int tiles = (E + 15) / 16;
    const int units = d / (4 * RS_STEP);
    int best = 1;
    for (int sp = 1; sp <= 4; sp++) {
        if (units % sp) continue;
        if ((int64_t)tiles * sp > target_blocks) break;
        best = sp;
    }
    return best;
}

hipError_t launch_router_skinny(const bf16 *x, const float *w, const float *bias, float *out,
                                int T, int d, int E, int splits, int32_t *zero_counts,
                                hipStream_t s)
{
    dim3 grid((E + 15) / 16, splits);
    const int steps = d / (4 * RS_STEP * splits);
    const float *b = splits > 1 ? nullptr : bias;
#define RS_CASE(N)                                                                          \
    if (T <= 16 * N) {                                                                      \
        hipLaunchKernelGGL(router_skinny_kernel<N>, grid, dim3(256), 0, s, x, w, b, out, T, \
                           d, E, steps, zero_counts);                                       \
        return hipGetLastError();                                                           \
    }
    RS_CASE(1)
    RS_CASE(2)
    RS_CASE(4)
#undef RS_CASE
    return hipErrorInvalidValue;
}

int router_splits(int T, int d, int E, int target_blocks)
{
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

hipError_t launch_topk_softmax(const float *src, int n_planes, const float *bias, float *logits,
                               int T, int E, int k, int32_t *idx, float *w, int32_t *counts,
                               hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    const int npl = (E + 63) / 64;
#define TK_CASE(N)                                                                        \
    if (npl <= N) {                                                                       \
        hipLaunchKernelGGL(topk_softmax_kernel<N>, grid, dim3(256), 0, s, src, n_planes,  \
                           bias, logits, T, E, k, idx, w, counts);                        \
        return hipGetLastError();                                                         \
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
