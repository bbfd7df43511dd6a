// The block-scaled precision mode (MX8): activations as MXFP8 (E4M3 elements,
// one E8M0 scale per 32) against MXFP4 weights on the gfx950 block-scaled
// matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4, which takes both
// operands and both scale sets as stored and runs at the 8-bit rate, twice
// the bf16 one, with no decode instructions.
//
// The formats are OCP Microscaling (MX) v1.0; the pages' layer (P1 section
// 二, 第一层: 4-bit weights meet higher-precision activations in hardware
// matrix kernels; P2 "MXFP4 原生支持": dequantisation fused into the GEMM)
// keeps bf16 activations, so MX8 is a separate accuracy contract: tokens and
// h are rounded to E4M3 before each projection.
//
//   mxfp8_quantize_kernel  bf16 or fp32 rows -> MXFP8 (codes [N][K], scales
//                          [N][K/32]); one thread per 32-element block
//   gemm_mx8_kernel        grouped projection, 256 x 256 tiles, MXFP8 rows x
//                          MXFP4 weights, fp32 accumulation
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// fp32 -> MXFP8. Per block: s = clamp(floor(log2 amax) - 8 + 127, 0, 254)
// (8 = emax of E4M3), q = v * 2^(127 - s) (exact), E4M3 code of q rounded to
// nearest-even with magnitudes from 448 up clamped to 448 (0x7E); an all-zero
// block gets scale 0 and codes 0; the sign bit comes from q, so -0 and
// negatives rounding to zero give 0x80.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_code(float q)
{
    const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
    const float a = fabsf(q);
    uint32_t mag;
    if (a >= 448.0f) {
        mag = 0x7Eu;
    } else if (a < 0.015625f) {
        // below 2^-6 the grid is k * 2^-9, k = 0..8 (k = 8 is the smallest
        // normal, whose code is also 8); the scaling is exact
        mag = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        // round the 23-bit fp32 mantissa to 3 bits, nearest-even; a carry
        // moves into the exponent field
        uint32_t b = __float_as_uint(a);
        b += 0x7FFFFu + ((b >> 20) & 1u);
        mag = ((((b >> 23) & 0xFFu) - 127u + 7u) << 3) | ((b >> 20) & 7u);
    }
    return sign | mag;
}

// The E8M0 scale code of a block with this amax, and 2^(127 - s): s =
// clamp(floor(log2 amax) - 8 + 127, 0, 254); an fp32-subnormal amax is below
// 2^-126 and clamps to 0. s <= 246 for finite input, so the exponent field of
// 2^(127 - s) is >= 8.
__device__ __forceinline__ int mxfp8_scale(float amax, float &inv)
{
    const int ex = (int)((__float_as_uint(amax) >> 23) & 0xffu);
    const int s = (amax == 0.0f || ex == 0) ? 0 : min(254, max(0, ex - 127 - 8 + 127));
    inv = __uint_as_float((uint32_t)(254 - s) << 23);
    return s;
}

// A DPP move of a float (all rows and banks, no bound control).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <typename InT>
__device__ __forceinline__ void load32(const InT *p, float v[32]);
template <>
__device__ __forceinline__ void load32<float>(const float *p, float v[32])
{
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const float4 t = ((const float4 *)p)[j];
        v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
    }
}
template <>
__device__ __forceinline__ void load32<bf16>(const bf16 *p, float v[32])
{
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const bf16x8 t = ((const bf16x8 *)p)[j];
#pragma unroll
        for (int i = 0; i < 8; i++) v[8 * j + i] = (float)t[i];
    }
}

// Rows n < min(N, *n_dev) (all N rows when n_dev is null: a device-side row
// count, so a buffer sized for the host bound is converted only as far as it
// holds rows); one thread per 32-element block, grid-stride.
template <typename InT>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const InT *__restrict__ v,
                                                             int64_t ldv, int64_t N, int K,
                                                             const int32_t *__restrict__ n_dev,
                                                             uint8_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales)
{
    const int nb = K / 32;
    const int64_t rows = n_dev ? min(N, (int64_t)max(*n_dev, 0)) : N;
    const int64_t total = rows * nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = i / nb;
        const int b = (int)(i - n * nb);
        float x[32];
        load32<InT>(v + n * ldv + 32 * b, x);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(x[j]));
        float inv;
        const int s = mxfp8_scale(amax, inv);
        uint8_t *c = codes + n * (int64_t)K + 32 * b;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            u32x4 w;
#pragma unroll
            for (int d = 0; d < 4; d++) {
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < 4; j++) word |= e4m3_code(x[16 * h + 4 * d + j] * inv) << (8 * j);
                w[d] = amax == 0.0f ? 0u : word;
            }
            *(u32x4 *)(c + 16 * h) = w;
        }
        scales[n * nb + b] = (uint8_t)s;
    }
}

hipError_t launch_mxfp8_quantize(const void *v, int v_f32, int64_t ldv, int64_t N, int K,
                                 uint8_t *codes, uint8_t *scales, hipStream_t s,
                                 const int32_t *n_dev)
{
    const int64_t nb = N * (K / 32);
    if (nb <= 0) return hipSuccess;
    // at most 16 K workgroups (64 per CU); larger inputs loop
    const dim3 grid((unsigned)std::min<int64_t>((nb + 255) / 256, 16384)), block(256);
    if (v_f32)
        hipLaunchKernelGGL(mxfp8_quantize_kernel<float>, grid, block, 0, s, (const float *)v, ldv,
                           N, K, n_dev, codes, scales);
    else
        hipLaunchKernelGGL(mxfp8_quantize_kernel<bf16>, grid, block, 0, s, (const bf16 *)v, ldv,
                           N, K, n_dev, codes, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped projection on the block-scaled matrix cores.
//
// Workgroup tile: BM (256 or 128) permuted rows of one expert x 256 weight
// rows, K step 64 (two MX blocks). 8 waves as 4 row quarters x 2 weight
// halves; quarter q owns row tile q of 32, and q + 4 in the 256-row tile
// (those holding rows of the group), each against the 4 weight tiles of 32 of
// its half; one 32 x 32 x 64 MFMA per (row tile, weight tile) per K step.
// The 128-row tile has twice the work items of half the size (one workgroup
// per CU either way: at 128 VGPRs, for two, the 128-row kernel spills). A GLU tile holds 128 W1 rows and the
// same 128 W2 rows (weight half ch: rows 64 ch .. 64 ch + 63 of each), so
// act(gate, up) is applied in registers.
//
// Operands, as the instruction takes them (lane L, l = L % 32, g = L / 32):
//   B (E2M1, 16 bytes): weight row l, K 32 g .. 32 g + 31 of the step, i.e.
//     MX block g, exactly the 16 stored code bytes (low nibble = even K);
//   A (E4M3, 32 bytes): row l, K 16 g .. 16 g + 15 in bytes 0-15 and
//     32 + 16 g .. 32 + 16 g + 15 in bytes 16-31;
//   scales: lane L gives the E8M0 scale of its row (A) or weight row (B)
//     for MX block g of the step.
// A rows sit in LDS at an 80-byte stride (64 code bytes + 16), so the 16
// lanes of a 16-byte read land on distinct banks; weights stay 4-bit in LDS.
//
// Pipeline: two LDS stages and two register stages, global loads two K steps
// ahead (the last steps repeat step nk - 1), one barrier per K step.
//
// Output: fp32 or bf16, or (OutT = uint8_t) MXFP8 with the quantiser's
// arithmetic: a weight tile's 32 columns are one MX block of the output row,
// held by the 32 lanes of a half-wave, so the block's amax is a 32-lane
// reduction; codes go to out [rows][ldo], scales to out_scales [rows][ldo/32].
// ---------------------------------------------------------------------------
constexpr int M8_BN = 256, M8_BK = 64, M8_THREADS = 512, M8_ALD = 80;

template <int ACT, typename OutT, bool PACKED, int BM>
__global__ __launch_bounds__(M8_THREADS, 1) void gemm_mx8_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, int64_t lda,
    const int32_t *__restrict__ a_rows, const uint8_t *__restrict__ w1c,
    const uint8_t *__restrict__ w1s, const uint8_t *__restrict__ w2c,
    const uint8_t *__restrict__ w2s, const int32_t *__restrict__ plan, int hdr, int N, int K,
    OutT *__restrict__ out, uint8_t *__restrict__ out_scales, int64_t ldo)
{
    constexpr bool GLU = ACT != ACT_NONE;
    constexpr bool QOUT = std::is_same<OutT, uint8_t>::value;
    constexpr int COLS = GLU ? M8_BN / 2 : M8_BN;
    constexpr int AJ = BM / 128;  // 16-byte A chunks per thread per K step
    __shared__ __attribute__((aligned(16))) uint8_t Aq[2][BM][M8_ALD];
    __shared__ uint8_t Asc[2][BM][2];
    __shared__ __attribute__((aligned(16))) uint8_t Bq[2][M8_BN][M8_BK / 2];
    __shared__ uint8_t Bsc[2][M8_BN][2];

    const int nblk = (N + COLS - 1) / COLS;
    const int total = plan[0] * nblk;
    // XCD-aware order: each XCD takes a contiguous run of work items, so the
    // column blocks of one row group share an L2
    const int per_xcd = (total + 7) / 8;
    const int local = blockIdx.x / 8;
    const int wi = (blockIdx.x % 8) * per_xcd + local;
    if (local >= per_xcd || wi >= total) return;
    const int grp = wi / nblk, nb = wi - grp * nblk;
    const int2 it = ((const int2 *)(plan + hdr))[grp];
    const int e = it.x & 0xffff, r0 = it.y, rend = r0 + (it.x >> 16);
    const int mrows = rend - r0;
    const int n0 = nb * COLS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ch = wave & 1, q = wave >> 1;

    // ---- global -> LDS assignment
    // A codes: 16-byte chunks c = tid + 512 j (j < AJ) of the BM x 64-byte
    // step, row c / 4, bytes 16 (c % 4); A scales: row tid / 2, block tid % 2,
    // for the first 2 BM threads
    const int64_t lds_ = lda / 32;
    const bool a_sc = BM == 256 || tid < 2 * BM;
    const uint8_t *ag[AJ];
#pragma unroll
    for (int j = 0; j < AJ; j++) {
        const int c = tid + 512 * j;
        const int rc = min(r0 + (c >> 2), rend - 1);
        const int64_t arow = a_rows ? (int64_t)a_rows[rc] : (int64_t)rc;
        ag[j] = ac + arow * lda + 16 * (c & 3);
    }
    const uint8_t *asg;
    {
        const int rc = min(r0 + min(tid >> 1, BM - 1), rend - 1);
        const int64_t arow = a_rows ? (int64_t)a_rows[rc] : (int64_t)rc;
        asg = as + arow * lds_ + (tid & 1);
    }
    // B: weight row tid / 2 of the tile, MX block tid % 2 of the step
    const int br = tid >> 1, bh = tid & 1;
    int wrow;
    const uint8_t *wcb, *wsb;
    if (GLU) {
        wrow = min(n0 + (br & 127), N - 1);
        wcb = br < 128 ? w1c : w2c;
        wsb = br < 128 ? w1s : w2s;
    } else {
        wrow = min(n0 + br, N - 1);
        wcb = w1c;
        wsb = w1s;
    }
    const int64_t wr64 = (int64_t)e * N + wrow;
    const int nch = K / 128, nc4 = (nch + 3) / 4;
    const uint8_t *bg, *sg;
    if constexpr (PACKED) {
        const int64_t rb = wr64 / 16;
        const int mm = (int)(wr64 % 16);
        bg = wcb + rb * nch * 1024 + mm * 16;
        sg = wsb + rb * nc4 * 256 + mm * 4;
    } else {
        bg = wcb + wr64 * (K / 2) + 16 * bh;
        sg = wsb + wr64 * (K / 32) + bh;
    }

    u32x4 ra0[AJ], ra1[AJ], rb0, rb1;
    uint8_t rsa0 = 0, rsa1 = 0, rsb0, rsb1;
    auto gload = [&](u32x4 *ra, uint8_t &rsa, u32x4 &rbv, uint8_t &rsb, int kt) {
        const int k0 = kt * M8_BK;
#pragma unroll
        for (int j = 0; j < AJ; j++) ra[j] = *(const u32x4 *)(ag[j] + k0);
        if (a_sc) rsa = asg[k0 / 32];
        if constexpr (PACKED) {
            const int c = kt >> 1, gg = 2 * (kt & 1) + bh;
            rbv = *(const u32x4 *)(bg + c * 1024 + gg * 256);
            rsb = sg[(c >> 2) * 256 + gg * 64 + (c & 3)];
        } else {
            rbv = *(const u32x4 *)(bg + k0 / 2);
            rsb = sg[k0 / 32];
        }
    };
    auto lstore = [&](int st, const u32x4 *ra, uint8_t rsa, const u32x4 &rbv, uint8_t rsb) {
#pragma unroll
        for (int j = 0; j < AJ; j++) {
            const int c = tid + 512 * j;
            *(u32x4 *)(&Aq[st][c >> 2][16 * (c & 3)]) = ra[j];
        }
        if (a_sc) Asc[st][tid >> 1][tid & 1] = rsa;
        *(u32x4 *)(&Bq[st][br][16 * bh]) = rbv;
        Bsc[st][br][bh] = rsb;
    };

    // ---- wave tiles
    const int g = lane >> 5, l32 = lane & 31;
    int bt[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if (GLU) bt[j] = (j >= 2 ? 128 : 0) + 64 * ch + 32 * (j & 1);  // W1 x2, then W2 x2
        else bt[j] = 128 * ch + 32 * j;
    }
    // row tiles of the wave: q, and q + 4 in the 256-row tile
    const int n_on = (32 * q < mrows ? 1 : 0) + (BM == 256 && 128 + 32 * q < mrows ? 1 : 0);
    const int nk = K / M8_BK;  // even: K is a multiple of 128

    auto run = [&](auto ni_c) {
        constexpr int NI = decltype(ni_c)::value;
        f32x16 acc[NI > 0 ? NI : 1][4];
#pragma unroll
        for (int i = 0; i < NI; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

        auto compute = [&](int st) {
            if constexpr (NI > 0) {
                i32x8 bv[4];
                int sb[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int row = bt[j] + l32;
                    const u32x4 w = *(const u32x4 *)(&Bq[st][row][16 * g]);
                    bv[j] = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
                    sb[j] = Bsc[st][row][g];
                }
#pragma unroll
                for (int i = 0; i < NI; i++) {
                    const int row = 32 * q + 128 * i + l32;
                    const u32x4 lo = *(const u32x4 *)(&Aq[st][row][16 * g]);
                    const u32x4 hi = *(const u32x4 *)(&Aq[st][row][32 + 16 * g]);
                    const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    const int sa = Asc[st][row][g];
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        // A format 0: E4M3; B format 4: E2M1; scale byte 0 of each
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            av, bv[j], acc[i][j], 0, 4, 0, sa, 0, sb[j]);
                }
            }
        };

        gload(ra0, rsa0, rb0, rsb0, 0);
        gload(ra1, rsa1, rb1, rsb1, 1);
        lstore(0, ra0, rsa0, rb0, rsb0);
        __syncthreads();
        for (int kt = 0; kt < nk; kt += 2) {
            // stage 0 holds step kt; registers set 1 hold step kt + 1
            gload(ra0, rsa0, rb0, rsb0, min(kt + 2, nk - 1));
            __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
            compute(0);
            lstore(1, ra1, rsa1, rb1, rsb1);
            __syncthreads();
            // stage 1 holds step kt + 1; registers set 0 hold step kt + 2
            gload(ra1, rsa1, rb1, rsb1, min(kt + 3, nk - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            lstore(0, ra0, rsa0, rb0, rsb0);  // past the end: a copy of the last step, unused
            __syncthreads();
        }

        // epilogue: lane holds C[8 (v / 4) + 4 g + v % 4][l32] of each tile
        auto emit = [&](int rl, int col, float val) {
            if constexpr (QOUT) {
                // every lane takes part in the reduction; the 32 columns of a
                // tile are all inside N or all past it (N % 32 == 0)
                // max over the half-wave: rotations by 8, 4, 2, 1 inside each
                // 16-lane row (DPP row_ror), then lane ^ 16 (ds_swizzle, bit
                // mode: and 0x1f, or 0, xor 0x10)
                float amax = fabsf(val);
                amax = fmaxf(amax, dpp_f<0x128>(amax));  // row_ror:8
                amax = fmaxf(amax, dpp_f<0x124>(amax));  // row_ror:4
                amax = fmaxf(amax, dpp_f<0x122>(amax));  // row_ror:2
                amax = fmaxf(amax, dpp_f<0x121>(amax));  // row_ror:1
                amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_ds_swizzle(
                                       __float_as_int(amax), 0x401F)));
                float inv;
                const int sc = mxfp8_scale(amax, inv);
                const uint32_t code = amax == 0.0f ? 0u : e4m3_code(val * inv);
                if (rl < mrows && col < N) {
                    const int64_t row = r0 + rl;
                    out[row * ldo + col] = (uint8_t)code;
                    if (l32 == 0) out_scales[row * (ldo / 32) + col / 32] = (uint8_t)sc;
                }
            } else {
                if (rl < mrows && col < N) {
                    // Y (the down projection) is read once, by the combine
                    if constexpr (GLU) store_out<OutT>(out + (int64_t)(r0 + rl) * ldo + col, val);
                    else store_out_once<OutT>(out + (int64_t)(r0 + rl) * ldo + col, val);
                }
            }
        };
#pragma unroll
        for (int i = 0; i < NI; i++) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int rl = 32 * q + 128 * i + 8 * (v >> 2) + 4 * g + (v & 3);
                if (!QOUT && rl >= mrows) continue;
                if constexpr (GLU) {
#pragma unroll
                    for (int jj = 0; jj < 2; jj++)
                        emit(rl, n0 + 64 * ch + 32 * jj + l32,
                             act_apply<ACT>(acc[i][jj][v], acc[i][2 + jj][v]));
                } else {
#pragma unroll
                    for (int j = 0; j < 4; j++) emit(rl, n0 + 128 * ch + 32 * j + l32, acc[i][j][v]);
                }
            }
        }
    };
    // every branch runs the same barriers (1 + nk)
    switch (__builtin_amdgcn_readfirstlane(n_on)) {
    case 2:
        if constexpr (BM == 256) run(std::integral_constant<int, 2>{});
        break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
    }
}

// ---------------------------------------------------------------------------
// The 256-row MX8 tile on 16 waves with direct global -> LDS loads (fp32 or
// bf16 output, K <= M8D_MAX_K): the bf16 path's gemm_tile256_w16_kernel
// arrangement on the block-scaled instruction.
// - MXFP8 rows (64 bytes per K step) and 4-bit codes go into a three-stage
//   LDS ring by global_load_lds_dwordx4; one barrier per K step publishes
//   step k and frees the stage that step k + 2 overwrites.
// - The tile's weight scales go to LDS once, by the same DMA, in the
//   streaming layout's order (16 groups of 16 weight rows); its rows' scales
//   (256 x K / 32 bytes, rows padded to an odd number of dwords) are copied
//   once, every load of a thread issued before its first store.
// - Wave w: row block q = w / 4 (two 32-row tiles) and slot c = w % 4 (gate
//   and up rows of output columns 32 c .. + 32, or weight rows 64 c .. + 64),
//   so every SIMD gets the same share of an expert's row tiles.
// - A rows sit in LDS at 64 bytes with 16-byte chunk c of row r at position
//   c ^ ((r / 4) % 4), so the 16 rows of a 16-lane read cover all banks;
//   code rows as in the bf16 kernel.
// ---------------------------------------------------------------------------
constexpr int M8D_STAGES = 3;
constexpr int M8D_A_BYTES = 256 * M8_BK;        // 16 KB of E4M3 rows
constexpr int M8D_W_BYTES = M8_BN * M8_BK / 2;  // 8 KB of E2M1 codes
constexpr int M8D_STAGE = M8D_A_BYTES + M8D_W_BYTES;
constexpr int M8D_THREADS = 1024;
constexpr int M8D_MAX_K = 4096;

__host__ __device__ constexpr int m8d_scale_row(int K)
{
    return (((K / 32 + 3) / 4) | 1) * 4;
}

// Weight scales of 16 weight rows in the streaming layout: K / 512 groups
// (rounded up) of 256 bytes; the tile's LDS table holds 16 of them.
__host__ __device__ constexpr int m8d_scale_chunk(int K)
{
    return 256 * ((K / 128 + 3) / 4);
}

__host__ __device__ constexpr int m8d_lds_bytes(int K)
{
    return M8D_STAGES * M8D_STAGE + 16 * m8d_scale_chunk(K) + 256 * m8d_scale_row(K);
}
// block-int16 output: a wave stages 32 rows of its 64 fp32 columns at a time,
// padded by 16 bytes, in the ring once the K loop is done
constexpr int M8D_Q16_PITCH = 64 * 4 + 16;
__host__ __device__ constexpr int m8d_lds_bytes_q16(int K)
{
    return m8d_lds_bytes(K) > 16 * 32 * M8D_Q16_PITCH ? m8d_lds_bytes(K)
                                                       : 16 * 32 * M8D_Q16_PITCH;
}

template <int ACT, typename OutT, bool PACKED>
__global__ __launch_bounds__(M8D_THREADS, 1) void gemm_mx8_w16_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, int64_t lda,
    const int32_t *__restrict__ a_rows, const uint8_t *__restrict__ w1c,
    const uint8_t *__restrict__ w1s, const uint8_t *__restrict__ w2c,
    const uint8_t *__restrict__ w2s, const int32_t *__restrict__ plan, int hdr, int N, int K,
    OutT *__restrict__ out, int64_t ldo, uint8_t *__restrict__ osc)
{
    constexpr bool GLU = ACT != ACT_NONE;
    constexpr int COLS = GLU ? M8_BN / 2 : M8_BN;
    constexpr bool Q16 = std::is_same<OutT, int16_t>::value;
    static_assert(!(GLU && Q16), "block-int16 rows come from the down projection");
    extern __shared__ __attribute__((aligned(16))) uint8_t m8d_lds[];
    const int srow = m8d_scale_row(K), chunk_b = m8d_scale_chunk(K);
    uint8_t *const Wsc = m8d_lds + M8D_STAGES * M8D_STAGE;  // [16][chunk_b] weight scales
    uint8_t *const Asc = Wsc + 16 * chunk_b;                 // [256][srow] row scales

    const int nblk = (N + COLS - 1) / COLS;
    const int total = plan[0] * nblk;
    const int per_xcd = (total + 7) / 8;
    const int local = blockIdx.x / 8;
    const int wi = (blockIdx.x % 8) * per_xcd + local;
    if (local >= per_xcd || wi >= total) return;
    const int grp = wi / nblk, nb = wi - grp * nblk;
    const int2 it = ((const int2 *)(plan + hdr))[grp];
    const int e = it.x & 0xffff, r0 = it.y, rend = r0 + (it.x >> 16);
    const int mrows = rend - r0;
    const int n0 = nb * COLS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = wave & 3, q = wave >> 2;
    const int nch = K / 128;
    const int64_t lds_ = lda / 32;

    auto wsel = [&](int br, const uint8_t *&wc, const uint8_t *&ws) -> int64_t {
        int wrow;
        if (GLU) {
            wrow = min(n0 + (br & 127), N - 1);
            wc = br < 128 ? w1c : w2c;
            ws = br < 128 ? w1s : w2s;
        } else {
            wrow = min(n0 + br, N - 1);
            wc = w1c;
            ws = w1s;
        }
        return (int64_t)e * N + wrow;
    };
    auto arow_of = [&](int row) -> int64_t {
        const int rc = min(r0 + row, rend - 1);
        return a_rows ? (int64_t)a_rows[rc] : (int64_t)rc;
    };

    // ---- DMA sources. A: wave w fills rows 16 w .. + 15; lane L lands in
    // chunk position L % 4 of row 16 w + L / 4, carrying logical chunk
    // (L % 4) ^ ((L / 16) % 4).
    const uint8_t *ag = ac + arow_of(16 * wave + (lane >> 2)) * lda +
                        16 * ((lane & 3) ^ ((lane >> 4) & 3));
    // codes: threads 0..511 -> LDS weight row tid / 2, half holding MX block bh
    const bool wload = wave < 8;
    const int br = (tid & 511) >> 1, bh = (tid & 1) ^ ((br >> 3) & 1);
    const uint8_t *bg;
    {
        const uint8_t *wc, *ws;
        const int64_t wr64 = wsel(br, wc, ws);
        if constexpr (PACKED)
            bg = wc + (wr64 / 16) * nch * 1024 + (wr64 % 16) * 16;
        else
            bg = wc + wr64 * (K / 2) + 16 * bh;
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(m8d_lds));
    auto issue = [&](int kt, int st) {
        const uint32_t sb = lds0 + st * M8D_STAGE;
        dma16(ag + kt * M8_BK, sb + wave * 1024);
        if (wload) {
            const uint8_t *src;
            if constexpr (PACKED)
                src = bg + (kt >> 1) * 1024 + (2 * (kt & 1) + bh) * 256;
            else
                src = bg + kt * (M8_BK / 2);
            dma16(src, sb + M8D_A_BYTES + wave * 1024);
        }
    };

    const int nk = K / M8_BK;  // even: K is a multiple of 128

    // ---- weight scales -> LDS. Group c of 16 LDS weight rows in the
    // streaming layout's order: the scale of k-block kb of its row r is byte
    // (kb % 16) / 4 of the word at (kb / 16) * 256 + (kb % 4) * 64 + (r % 16) * 4.
    // Streaming weights: each group is contiguous in HBM (N is a multiple of
    // 16), so DMA copies ahead of the first stages (the first barrier's wait
    // covers them); groups past N take the last group's scales (their rows
    // are clamped and their outputs dropped).
    if constexpr (PACKED) {
        for (int m = wave; m < 16 * chunk_b / 1024; m += M8D_THREADS / 64) {
            const int b = 1024 * m + 16 * lane;
            const int c = b / chunk_b, off = b - c * chunk_b;
            const int wr0 = min(GLU ? n0 + ((16 * c) & 127) : n0 + 16 * c, N - 16);
            const uint8_t *ws = (GLU && c >= 8) ? w2s : w1s;
            dma16(ws + (((int64_t)e * N + wr0) / 16) * chunk_b + off,
                  lds0 + M8D_STAGES * M8D_STAGE + 1024 * m);
        }
    } else {
        // row-major scales: a word holds k-blocks 4 r .. 4 r + 3 of a row
        const int per_row = K / 128;
        for (int idx = tid; idx < 256 * per_row; idx += M8D_THREADS) {
            const int row = idx / per_row, r = idx - row * per_row;
            const uint8_t *wc, *ws;
            const int64_t wr64 = wsel(row, wc, ws);
            const uint32_t v = *(const uint32_t *)(ws + wr64 * (K / 32) + 4 * r);
            uint8_t *dst = Wsc + (row / 16) * chunk_b + (r / 4) * 256 + (row % 16) * 4 + (r % 4);
#pragma unroll
            for (int i = 0; i < 4; i++) dst[64 * i] = (uint8_t)(v >> (8 * i));
        }
    }
    issue(0, 0);
    issue(1, 1);

    // ---- the rows' scales -> LDS: every load of a thread before its first
    // store (K <= 4096: at most 8 words per thread)
    if (lds_ % 4 == 0) {
        const int per_row = K / 128;
        constexpr int MAXW = 256 * (M8D_MAX_K / 128) / M8D_THREADS;
        uint32_t v[MAXW];
        int dsto[MAXW];
#pragma unroll
        for (int u = 0; u < MAXW; u++) {
            const int idx = tid + u * M8D_THREADS;
            dsto[u] = -1;
            if (idx < 256 * per_row) {
                const int row = idx / per_row, r = idx - row * per_row;
                v[u] = *(const uint32_t *)(as + arow_of(row) * lds_ + 4 * r);
                dsto[u] = row * srow + 4 * r;
            }
        }
#pragma unroll
        for (int u = 0; u < MAXW; u++)
            if (dsto[u] >= 0) *(uint32_t *)(Asc + dsto[u]) = v[u];
    } else {
        const int per_row = K / 32;
        for (int idx = tid; idx < 256 * per_row; idx += M8D_THREADS) {
            const int row = idx / per_row, r = idx - row * per_row;
            Asc[row * srow + r] = as[arow_of(row) * lds_ + r];
        }
    }

    // ---- wave tiles
    const int h = lane >> 5, l32 = lane & 31;
    int bt[2];
#pragma unroll
    for (int j = 0; j < 2; j++) bt[j] = GLU ? 128 * j + 32 * slot : 64 * slot + 32 * j;
    const int n_on = (64 * q < mrows ? 1 : 0) + (64 * q + 32 < mrows ? 1 : 0);
    const int arow_off = (64 * q + l32) * M8_BK;
    const int akey = (l32 >> 2) & 3;
    const int lo_off = (h ^ akey) << 4, hi_off = ((2 + h) ^ akey) << 4;
    const int bpos = 16 * (h ^ ((l32 >> 3) & 1));
    // weight scales of this lane's rows and MX block h; the step adds
    // (k / 8) * 256 + (k % 2) * 128 + (k % 8) / 2 (k-block 2 k + h)
    int wso[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int row = bt[j] + l32;
        wso[j] = (row / 16) * chunk_b + (row % 16) * 4 + 64 * h;
    }

    auto run = [&](auto ni_c) {
        constexpr int NI = decltype(ni_c)::value;
        f32x16 acc[NI > 0 ? NI : 1][2];
#pragma unroll
        for (int i = 0; i < NI; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

        auto compute = [&](int st, int kt) {
            if constexpr (NI > 0) {
                const uint8_t *A = m8d_lds + st * M8D_STAGE;
                const uint8_t *Bq = A + M8D_A_BYTES;
                i32x8 bv[2];
                int sb[2];
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int row = bt[j] + l32;
                    const u32x4 w = *(const u32x4 *)(Bq + row * 32 + bpos);
                    bv[j] = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
                    sb[j] = Wsc[wso[j] + (kt >> 3) * 256 + (kt & 1) * 128 + ((kt & 7) >> 1)];
                }
#pragma unroll
                for (int i = 0; i < NI; i++) {
                    const uint8_t *ar = A + arow_off + 32 * M8_BK * i;
                    const u32x4 lo = *(const u32x4 *)(ar + lo_off);
                    const u32x4 hi = *(const u32x4 *)(ar + hi_off);
                    const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    const int sa = Asc[(64 * q + 32 * i + l32) * srow + 2 * kt + h];
#pragma unroll
                    for (int j = 0; j < 2; j++)
                        // A format 0: E4M3; B format 4: E2M1; scale byte 0 of each
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            av, bv[j], acc[i][j], 0, 4, 0, sa, 0, sb[j]);
                }
            }
        };

        for (int kt = 0; kt < nk; kt++) {
            // this wave's loads of step kt are done (those of kt + 1 -- 2 or 1
            // instructions -- may still be in flight); the barrier publishes
            // every wave's and ends the reads of step kt - 1
            if (kt + 1 < nk) {
                if (wload)
                    asm volatile("s_waitcnt vmcnt(2)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(1)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
            const int st = kt % 3;
            if (kt + 2 < nk) issue(kt + 2, st == 0 ? 2 : st - 1);
            compute(st, kt);
        }

        // lane holds C[8 (v / 4) + 4 h + v % 4][l32] of each tile
        if constexpr (Q16) {
            // Block-int16 rows (the expert outputs inside the layer, read once
            // by the combine), as the FP6X2 down projection writes them: per 32
            // columns one code e in osc, the biased exponent of the block's
            // largest magnitude (at most 252), and each value v as the integer
            // nearest 32767 v 2^(126 - e). One 32-row tile at a time is staged
            // as fp32 in the idle ring; then 16 lanes hold a row's 64 columns,
            // 4 each, and the 8 lanes of a 32-column block take its largest
            // magnitude with three DPP moves.
            __syncthreads();  // every wave is past its last step's reads
            constexpr int LPR = 16, RPI = 64 / LPR;
            uint8_t *const stg = m8d_lds + wave * (32 * M8D_Q16_PITCH);
            const int c0 = n0 + 64 * slot;
            const bool col_on = c0 < N;  // N is a multiple of 64
#pragma unroll
            for (int i = 0; i < NI; i++) {
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    float *row = (float *)(stg + (8 * (v >> 2) + 4 * h + (v & 3)) * M8D_Q16_PITCH);
#pragma unroll
                    for (int j = 0; j < 2; j++) row[32 * j + l32] = acc[i][j][v];
                }
                const int64_t r = (int64_t)r0 + 64 * q + 32 * i + lane / LPR;
                OutT *yrow = out + r * ldo + c0 + 4 * (lane % LPR);
                uint8_t *srow = osc + r * (ldo / 32) + (c0 + 4 * (lane % LPR)) / 32;
#pragma unroll
                for (int it = 0; it < 32 / RPI; it++) {
                    const int rr = RPI * it + lane / LPR, seg = lane % LPR;
                    const u32x4 val = *(const u32x4 *)(stg + rr * M8D_Q16_PITCH + 16 * seg);
                    const int rl = 64 * q + 32 * i + rr;
                    // magnitudes compared as bit patterns (non-negative floats
                    // order as their bits)
                    uint32_t mb = 0;
#pragma unroll
                    for (int c = 0; c < 4; c++) mb = max(mb, val[c] & 0x7fffffffu);
                    mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xB1, 0xF, 0xF, false));
                    mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x4E, 0xF, 0xF, false));
                    mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x141, 0xF, 0xF, false));
                    const int code = min((int)(mb >> 23), 252);
                    const float inv = __uint_as_float((uint32_t)(253 - code) << 23);  // 2^(126 - e)
                    if (col_on && rl < mrows) {
                        float x[4];
#pragma unroll
                        for (int c = 0; c < 4; c++) x[c] = __uint_as_float(val[c]) * inv;
                        const u32x2 pk = {
                            (uint32_t)__builtin_bit_cast(int, __builtin_amdgcn_cvt_pknorm_i16(x[0], x[1])),
                            (uint32_t)__builtin_bit_cast(int, __builtin_amdgcn_cvt_pknorm_i16(x[2], x[3]))};
                        __builtin_nontemporal_store(pk, (u32x2 *)(yrow + (int64_t)it * RPI * ldo));
                        if ((seg & 7) == 0) srow[(int64_t)it * RPI * (ldo / 32)] = (uint8_t)code;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NI; i++) {
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int rl = 64 * q + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (rl >= mrows) continue;
                    OutT *orow = out + (int64_t)(r0 + rl) * ldo;
                    if constexpr (GLU) {
                        const int col = n0 + 32 * slot + l32;
                        if (col < N)
                            store_out<OutT>(orow + col, act_apply<ACT>(acc[i][0][v], acc[i][1][v]));
                    } else {
#pragma unroll
                        for (int j = 0; j < 2; j++) {
                            const int col = n0 + 64 * slot + 32 * j + l32;
                            if (col < N) store_out_once<OutT>(orow + col, acc[i][j][v]);
                        }
                    }
                }
            }
        }
    };
    // every branch runs the same barriers (nk) and the same loads
    switch (__builtin_amdgcn_readfirstlane(n_on)) {
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
    }
}

template <int ACT, typename OutT, bool PACKED, int BM>
static hipError_t launch_mx8(const uint8_t *ac, const uint8_t *as, int64_t lda,
                             const int32_t *a_rows, const uint8_t *w1c, const uint8_t *w1s,
                             const uint8_t *w2c, const uint8_t *w2s, const GemmPlanArgs &pa,
                             int N, int K, OutT *out, uint8_t *out_scales, int64_t ldo,
                             hipStream_t s)
{
    constexpr int COLS = ACT != ACT_NONE ? M8_BN / 2 : M8_BN;
    const int64_t grid = (int64_t)pa.max_groups * ((N + COLS - 1) / COLS);
    if (grid <= 0) return hipSuccess;
    // the XCD-aware order maps block b to work (b % 8) * ceil(total / 8) + b / 8;
    // a grid of 8 * ceil(bound / 8) blocks covers every work item
    const int64_t G = (grid + 7) / 8 * 8;
    // fp32 / bf16 output on the 256-row tile: 16 waves, direct-to-LDS loads
    constexpr bool Q16 = std::is_same<OutT, int16_t>::value;
    if constexpr (BM == 256 && !std::is_same<OutT, uint8_t>::value) {
        if (K <= M8D_MAX_K) {
            auto kern = gemm_mx8_w16_kernel<ACT, OutT, PACKED>;
            const int lds = Q16 ? m8d_lds_bytes_q16(K) : m8d_lds_bytes(K);
            const hipError_t err = ensure_dynamic_lds((const void *)kern, lds);
            if (err != hipSuccess) return err;
            hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(M8D_THREADS), lds, s, ac, as, lda,
                               a_rows, w1c, w1s, w2c, w2s, pa.plan, pa.hdr, N, K, out, ldo,
                               out_scales);
            return hipGetLastError();
        }
    }
    if constexpr (Q16) {
        return hipErrorInvalidValue;  // block-int16 rows: the 16-wave 256-row tile only
    } else {
        hipLaunchKernelGGL((gemm_mx8_kernel<ACT, OutT, PACKED, BM>), dim3((unsigned)G),
                           dim3(M8_THREADS), 0, s, ac, as, lda, a_rows, w1c, w1s, w2c, w2s,
                           pa.plan, pa.hdr, N, K, out, out_scales, ldo);
        return hipGetLastError();
    }
}

// ---------------------------------------------------------------------------
// Streaming schedule of the MX8 mode (few rows per expert: decode), the
// counterpart of the bf16 streaming GEMM: one workgroup per (16-row group,
// block of output columns), each wave streaming 4 weight streams of 16 rows
// (gate and up pairs for GLU) once, in 128-wide K chunks, on
// v_mfma_scale_f32_16x16x128_f8f6f4. Operands, as the instruction takes them
// (lane L, m = L % 16, g = L / 16; checked with a one-wave probe against an
// fp64 evaluation):
//   B (E2M1, 16 bytes): weight row m, MX block g of the chunk: the 16 stored
//     code bytes, exactly what a lane of the streaming layout holds;
//   A (E4M3, 32 bytes): token row m, K 16 g .. + 16 in bytes 0-15 and
//     64 + 16 g .. + 16 in bytes 16-31;
//   scales: lane L gives the E8M0 scale of its row for MX block g.
// Result: lane L holds C[4 g + i][m] (token row 4 g + i, weight row m).
// Weight loads carry the non-temporal hint (read once per row group).
// ---------------------------------------------------------------------------
template <int ACT, typename OutT, int D, bool PACKED>
__global__ __launch_bounds__(256) void gemm_mx8_stream_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, int64_t lda,
    const int32_t *__restrict__ a_rows, const uint8_t *__restrict__ w1c,
    const uint8_t *__restrict__ w1s, const uint8_t *__restrict__ w2c,
    const uint8_t *__restrict__ w2s, const int32_t *__restrict__ plan, int hdr, int N, int K,
    OutT *__restrict__ out, int64_t ldo)
{
    constexpr bool GLU = ACT != ACT_NONE;
    constexpr int NS = 4;
    constexpr int COLS_W = GLU ? 8 * NS : 16 * NS;  // output columns per wave
    constexpr int COLS_B = 4 * COLS_W;
    extern __shared__ uint32_t m8_sscale[];  // canonical layout: the rows' scales
    const int nblk = (N + COLS_B - 1) / COLS_B;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;

    const int wi = blockIdx.x;
    if (wi >= plan[0] * nblk) return;
    const int grp = wi / nblk, nb = wi - grp * nblk;
    const int nb0 = nb * COLS_B;
    const int n0 = nb0 + wave * COLS_W;
    const bool wave_on = n0 < N;  // N is a multiple of COLS_W
    const int2 it = ((const int2 *)(plan + hdr))[grp];
    const int e = it.x & 0xffff, r0 = it.y, rend = r0 + (it.x >> 16);
    const int rc = min(r0 + m, rend - 1);
    const int64_t arow = a_rows ? (int64_t)a_rows[rc] : (int64_t)rc;
    const uint8_t *ap = ac + arow * lda + 16 * g;
    const uint8_t *asp = as + arow * (lda / 32) + g;

    const int nch = K / 128;  // a multiple of D
    const int nc4 = (nch + 3) / 4;
    const int sbw = K / 128;  // canonical: scale dwords per weight row
    if constexpr (!PACKED) {
        const int rows_v = min(COLS_B, N - nb0);
        const int per_mat4 = rows_v * sbw / 4;
        for (int i = threadIdx.x; i < (GLU ? 2 : 1) * per_mat4; i += blockDim.x) {
            const int mat = i / per_mat4, r = i - mat * per_mat4;
            const uint8_t *base = (mat ? w2s : w1s) + ((int64_t)e * N + nb0) * (K / 32);
            *(u32x4 *)(&m8_sscale[mat * COLS_B * sbw + 4 * r]) = *(const u32x4 *)(base + 16 * r);
        }
    }

    const uint8_t *cp[NS];
    const uint8_t *spk[NS];
    int srow[NS];
#pragma unroll
    for (int j = 0; j < NS; j++) {
        const int wr0 = GLU ? n0 + 16 * (j / 2) : n0 + 16 * j;
        const bool second = GLU && (j & 1);
        const int wr = wave_on ? wr0 : 0;
        if constexpr (PACKED) {
            const int64_t rb = ((int64_t)e * N + wr) / 16;
            cp[j] = (second ? w2c : w1c) + rb * nch * 1024 + lane * 16;
            spk[j] = (second ? w2s : w1s) + rb * nc4 * 256 + lane * 4;
            srow[j] = 0;
        } else {
            const int64_t row = (int64_t)e * N + wr + m;
            cp[j] = (second ? w2c : w1c) + row * (K / 2) + 16 * g;
            spk[j] = nullptr;
            srow[j] = ((second ? 1 : 0) * COLS_B + (wr0 - nb0) + m) * sbw;
        }
    }

    u32x4 q[D][NS];
    uint32_t sq[D][NS];
    u32x4 alo[D], ahi[D];
    uint32_t asc[D];
    f32x4 acc[NS];
#pragma unroll
    for (int j = 0; j < NS; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int c, u32x4 *qd, uint32_t *sd, u32x4 &lo, u32x4 &hi, uint32_t &sa) {
#pragma unroll
        for (int j = 0; j < NS; j++) {
            if constexpr (PACKED) {
                qd[j] = __builtin_nontemporal_load((const u32x4 *)(cp[j] + c * 1024));
                sd[j] = __builtin_nontemporal_load((const uint32_t *)(spk[j] + (c >> 2) * 256));
            } else {
                qd[j] = __builtin_nontemporal_load((const u32x4 *)(cp[j] + c * 64));
            }
        }
        lo = *(const u32x4 *)(ap + c * 128);
        hi = *(const u32x4 *)(ap + c * 128 + 64);
        sa = asp[4 * c];
    };
    auto consume = [&](int c, const u32x4 *qd, const uint32_t *sd, const u32x4 &lo,
                       const u32x4 &hi, uint32_t sa) {
        const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
        for (int j = 0; j < NS; j++) {
            uint32_t sb;
            if constexpr (PACKED) sb = (sd[j] >> (8 * (c & 3))) & 0xffu;
            else sb = (m8_sscale[srow[j] + c] >> (8 * g)) & 0xffu;
            const i32x8 bv = {(int)qd[j][0], (int)qd[j][1], (int)qd[j][2], (int)qd[j][3],
                              0, 0, 0, 0};
            // A format 0: E4M3; B format 4: E2M1; scale byte 0 of each
            acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[j], 0, 4, 0,
                                                                      (int)sa, 0, (int)sb);
        }
    };
    if (wave_on) {
#pragma unroll
        for (int d = 0; d < D; d++) issue(d, q[d], sq[d], alo[d], ahi[d], asc[d]);
    }
    if constexpr (!PACKED) __syncthreads();  // scales in LDS
    if (!wave_on) return;
    for (int c0 = 0; c0 < nch - D; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
            consume(c0 + d, q[d], sq[d], alo[d], ahi[d], asc[d]);
            issue(c0 + d + D, q[d], sq[d], alo[d], ahi[d], asc[d]);
        }
    }
#pragma unroll
    for (int d = 0; d < D; d++) consume(nch - D + d, q[d], sq[d], alo[d], ahi[d], asc[d]);

    // lane holds C[4 g + i][m] of each stream: token row r0 + 4 g + i
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int row = r0 + 4 * g + i;
        if (row >= rend) continue;
        OutT *orow = out + (int64_t)row * ldo;
        if constexpr (GLU) {
#pragma unroll
            for (int jp = 0; jp < NS / 2; jp++)
                store_out<OutT>(orow + n0 + 16 * jp + m,
                                act_apply<ACT>(acc[2 * jp][i], acc[2 * jp + 1][i]));
        } else {
#pragma unroll
            for (int j = 0; j < NS; j++) store_out_once<OutT>(orow + n0 + 16 * j + m, acc[j][i]);
        }
    }
}

template <int ACT, typename OutT, bool PACKED>
static hipError_t launch_mx8_stream(const uint8_t *ac, const uint8_t *as, int64_t lda,
                                    const int32_t *a_rows, const uint8_t *w1c,
                                    const uint8_t *w1s, const uint8_t *w2c, const uint8_t *w2s,
                                    const GemmPlanArgs &pa, int N, int K, OutT *out, int64_t ldo,
                                    hipStream_t s)
{
    constexpr int COLS_B = 4 * (ACT != ACT_NONE ? 32 : 64);
    const int64_t grid = (int64_t)pa.max_groups * ((N + COLS_B - 1) / COLS_B);
    if (grid <= 0) return hipSuccess;
    const int nch = K / 128;
    const int D = (nch % 4 == 0) ? 4 : (nch % 2 == 0 ? 2 : 1);
    const size_t lds = PACKED ? 0 : (size_t)(ACT != ACT_NONE ? 2 : 1) * COLS_B * (K / 32);
#define M8S_LAUNCH(DD)                                                                         \
    hipLaunchKernelGGL((gemm_mx8_stream_kernel<ACT, OutT, DD, PACKED>), dim3((unsigned)grid),  \
                       dim3(256), lds, s, ac, as, lda, a_rows, w1c, w1s, w2c, w2s, pa.plan,    \
                       pa.hdr, N, K, out, ldo)
    if (D == 4)
        M8S_LAUNCH(4);
    else if (D == 2)
        M8S_LAUNCH(2);
    else
        M8S_LAUNCH(1);
#undef M8S_LAUNCH
    return hipGetLastError();
}

template <typename OutT, bool PACKED, int BM>
static hipError_t mx8_act(int act, const uint8_t *ac, const uint8_t *as, int64_t lda,
                          const int32_t *a_rows, const uint8_t *w1c, const uint8_t *w1s,
                          const uint8_t *w2c, const uint8_t *w2s, const GemmPlanArgs &pa, int N,
                          int K, OutT *out, uint8_t *out_scales, int64_t ldo, hipStream_t s)
{
#define MX8_ACT(A)                                                                           \
    case A:                                                                                  \
        return launch_mx8<A, OutT, PACKED, BM>(ac, as, lda, a_rows, w1c, w1s, w2c, w2s, pa, N, \
                                               K, out, out_scales, ldo, s);
    switch (act) {
        MX8_ACT(ACT_NONE)
        MX8_ACT(ACT_SILU_MUL)
        MX8_ACT(ACT_GELU_TANH_MUL)
    default:
        return hipErrorInvalidValue;
    }
#undef MX8_ACT
}

// MX8 schedules, measured with all 896 experts (I = 1024): streaming (16-row
// groups, fp32 or bf16 output) below a mean of 16 rows per expert (0.91 vs
// 1.49 ms at a mean of 5, 1.71 vs 1.62 ms at 18); the 128-row tile from 16 to
// 128 (1.62-2.17 ms against 1.97-2.32 ms for the 256-row tile at means of 18
// to 73); the 256-row tile from 128 up (faster at the means of 146, 360 and
// 1170 rows tried). MXFP8 output (q_out) is written by the tiled kernels only.
int mx8_resolve_mode(int mode, int num_local, int max_rows, bool q_out)
{
    const int64_t rows = max_rows, nl = num_local;
    if (!q_out && (mode == MOE_SCHED_STREAM || (mode == MOE_SCHED_AUTO && rows < 16 * nl)))
        return MOE_SCHED_STREAM;
    if (mode == MOE_SCHED_TILE128 || mode == MOE_SCHED_TILE256) return mode;
    return rows < 128 * nl ? MOE_SCHED_TILE128 : MOE_SCHED_TILE256;
}

GemmPlanArgs mx8_plan_args(int num_local, int max_rows, int mode, void *ws, bool q_out)
{
    return gemm_plan_args(num_local, max_rows, mx8_resolve_mode(mode, num_local, max_rows, q_out),
                          ws);
}

bool mx8_q16_ok(int mode, int num_local, int max_rows, int K)
{
    return mx8_resolve_mode(mode, num_local, max_rows) == MOE_SCHED_TILE256 && K <= M8D_MAX_K;
}

size_t mx8_gemm_ws_bytes(int num_local, int max_rows)
{
    // the streaming schedule's 16-row grouping has the most work items
    return grouped_gemm_ws_bytes(num_local, max_rows, 0, MOE_SCHED_STREAM);
}

hipError_t launch_gemm_mx8_run(const uint8_t *ac, const uint8_t *as, int64_t lda,
                               const int32_t *a_rows, const uint8_t *w1c, const uint8_t *w1s,
                               const uint8_t *w2c, const uint8_t *w2s, int num_local,
                               int max_rows, int N, int K, int act, void *out, int out_kind,
                               uint8_t *out_scales, int64_t ldo, int mode, void *plan_ws,
                               int packed, hipStream_t s)
{
    const bool q_out = out_kind == MX8_OUT_MXFP8;
    const GemmPlanArgs pa = mx8_plan_args(num_local, max_rows, mode, plan_ws, q_out);
    const int md = mx8_resolve_mode(mode, num_local, max_rows, q_out);
    if (md == MOE_SCHED_STREAM) {
#define MX8_STREAM(OT, PK)                                                                      \
    switch (act) {                                                                              \
    case ACT_NONE:                                                                              \
        return launch_mx8_stream<ACT_NONE, OT, PK>(ac, as, lda, a_rows, w1c, w1s, w2c, w2s, pa, \
                                                   N, K, (OT *)out, ldo, s);                    \
    case ACT_SILU_MUL:                                                                          \
        return launch_mx8_stream<ACT_SILU_MUL, OT, PK>(ac, as, lda, a_rows, w1c, w1s, w2c, w2s, \
                                                       pa, N, K, (OT *)out, ldo, s);            \
    case ACT_GELU_TANH_MUL:                                                                     \
        return launch_mx8_stream<ACT_GELU_TANH_MUL, OT, PK>(ac, as, lda, a_rows, w1c, w1s, w2c, \
                                                            w2s, pa, N, K, (OT *)out, ldo, s);  \
    default:                                                                                    \
        return hipErrorInvalidValue;                                                            \
    }
        if (out_kind == MX8_OUT_F32) {
            if (packed) MX8_STREAM(float, true)
            MX8_STREAM(float, false)
        }
        if (packed) MX8_STREAM(bf16, true)
        MX8_STREAM(bf16, false)
#undef MX8_STREAM
    }
    const bool t256 = md == MOE_SCHED_TILE256;
    if (out_kind == MX8_OUT_Q16) {
        if (!mx8_q16_ok(mode, num_local, max_rows, K) || act != ACT_NONE || !out_scales ||
            ldo % 32 != 0)
            return hipErrorInvalidValue;
        if (packed)
            return launch_mx8<ACT_NONE, int16_t, true, 256>(ac, as, lda, a_rows, w1c, w1s, w2c, w2s,
                                                            pa, N, K, (int16_t *)out, out_scales,
                                                            ldo, s);
        return launch_mx8<ACT_NONE, int16_t, false, 256>(ac, as, lda, a_rows, w1c, w1s, w2c, w2s,
                                                         pa, N, K, (int16_t *)out, out_scales, ldo,
                                                         s);
    }
#define MX8_RUN(OT, PK)                                                                        \
    return t256 ? mx8_act<OT, PK, 256>(act, ac, as, lda, a_rows, w1c, w1s, w2c, w2s, pa, N, K, \
                                       (OT *)out, out_scales, ldo, s)                          \
                : mx8_act<OT, PK, 128>(act, ac, as, lda, a_rows, w1c, w1s, w2c, w2s, pa, N, K, \
                                       (OT *)out, out_scales, ldo, s)
    if (out_kind == MX8_OUT_F32) {
        if (packed) MX8_RUN(float, true);
        MX8_RUN(float, false);
    }
    if (out_kind == MX8_OUT_MXFP8) {
        if (packed) MX8_RUN(uint8_t, true);
        MX8_RUN(uint8_t, false);
    }
    if (packed) MX8_RUN(bf16, true);
    MX8_RUN(bf16, false);
#undef MX8_RUN
}

hipError_t launch_grouped_gemm_mx8(const uint8_t *ac, const uint8_t *as, int64_t lda,
                                   const int32_t *a_rows, const uint8_t *w1c, const uint8_t *w1s,
                                   const uint8_t *w2c, const uint8_t *w2s, const int32_t *off,
                                   int num_local, int max_rows, int N, int K, int act, void *out,
                                   int out_kind, uint8_t *out_scales, int64_t ldo, int mode,
                                   void *ws, int packed, hipStream_t s)
{
    hipError_t e = launch_gemm_plan_into(
        off, num_local, mx8_plan_args(num_local, max_rows, mode, ws, out_kind == MX8_OUT_MXFP8), s);
    if (e != hipSuccess) return e;
    return launch_gemm_mx8_run(ac, as, lda, a_rows, w1c, w1s, w2c, w2s, num_local, max_rows, N,
                               K, act, out, out_kind, out_scales, ldo, mode, ws, packed, s);
}

}  // namespace moe
