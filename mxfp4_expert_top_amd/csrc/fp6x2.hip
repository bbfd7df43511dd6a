// The FP6X2 carriage of activations: bf16 (or fp32) rows as two MXFP6 planes
// (OCP MX v1.0 E2M3 elements, one E8M0 scale per 32), the second plane
// holding the fp32 residual of the first, against MXFP4 weights on the
// gfx950 block-scaled instruction v_mfma_scale_f32_32x32x64_f8f6f4 with
// 6-bit A and 4-bit B operands. With both operands at most 6 bits wide the
// instruction issues a 32 x 32 x 64 product in about the time of one bf16
// 32 x 32 x 16 one, so the two planes take half the matrix-core time of the
// bf16 path and no decode instructions.
//
// The pages' layer keeps activations at higher precision than the 4-bit
// weights (P1 section 二, 第一层); the two planes carry each value to within
// 2^(E-7), E = floor(log2 amax) of its 32-block (about 3.4e-4 rms on
// N(0, 1) tokens, a third of bf16's own rounding), and layers that use them
// are held to the default accuracy contract.
//
//   fp6x2_split_kernel       rows -> two planes; one thread per 32-element
//                            block
//   gemm_fp6x2_w16_kernel    grouped projection on 256 x 256 tiles, the two
//                            planes x MXFP4 weights, fp32 accumulation
//
// Storage of a split row of K elements: 2 K bytes (the size of the bf16 row),
// one 128-byte record per 64 elements (blocks 2 s and 2 s + 1):
//   bytes   0..23  block 2 s, plane-1 codes   bytes  64..87   block 2 s + 1, plane 1
//   bytes  24..47  block 2 s, plane-2 codes   bytes  88..111  block 2 s + 1, plane 2
//   bytes  48..51  E8M0 scales: (2 s, plane 1), (2 s, plane 2), (2 s + 1,
//                  plane 1), (2 s + 1, plane 2)
//   bytes  52..63  the same four scales three more times
//   bytes 112..127 zero
// with code i of a plane at bits 6 i .. 6 i + 5 of its 24 little-endian bytes
// (the instruction's operand order). Each K step of the projection then
// reads one aligned 128-byte line per row, scales included; the two blocks
// sit in the two 64-byte halves, which keeps the lanes reading block 0 and
// those reading block 1 on different LDS banks, and the four copies of the
// scales let the 32 rows of a tile read theirs from distinct banks (one copy:
// 4-way conflicts, 80% of the kernel's LDS-active cycles).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// fp32 -> MXFP6 (E2M3). Per block: s = clamp(floor(log2 amax) - 2 + 127, 0,
// 254) (2 = emax of E2M3), q = v * 2^(127 - s) (exact), E2M3 code of q
// rounded to nearest-even with magnitudes from 7.5 up clamped to 7.5 (code
// 31); an all-zero block gets scale 0 and codes 0; the sign bit comes from
// q, so -0 and negatives rounding to zero give 0x20.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m3_code(float q)
{
    const uint32_t sign = (__float_as_uint(q) >> 26) & 0x20u;
    const float a = fabsf(q);
    uint32_t mag;
    if (a >= 7.5f) {
        mag = 31u;
    } else if (a < 1.0f) {
        // below 1 the grid is k / 8, k = 0..8 (k = 8 is the smallest normal,
        // whose code is also 8); the scaling is exact
        mag = (uint32_t)__builtin_rintf(a * 8.0f);
    } else {
        // round the 23-bit fp32 mantissa to 3 bits, nearest-even; a carry
        // moves into the exponent field (biased 127 for [1, 2) -> E2M3 field 1)
        uint32_t b = __float_as_uint(a);
        b += 0x7FFFFu + ((b >> 20) & 1u);
        mag = ((((b >> 23) & 0xFFu) - 126u) << 3) | ((b >> 20) & 7u);
    }
    return sign | mag;
}

// The E2M3 value of a code: m / 8 for exponent field 0, else
// (8 + m) * 2^(e - 4).
__device__ __forceinline__ float e2m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 3u, m = c & 7u;
    const float mag = (float)(e ? 8u + m : m) * __uint_as_float((e ? 123u + e : 124u) << 23);
    return (c & 0x20u) ? -mag : mag;
}

// The E8M0 scale code of a block with this amax, and 2^(127 - s): s =
// clamp(floor(log2 amax) - 2 + 127, 0, 254); an fp32-subnormal amax clamps to
// 0. s <= 252 for finite input, so the exponent field of 2^(127 - s) is >= 2.
__device__ __forceinline__ int mxfp6_scale(float amax, float &inv)
{
    const int ex = (int)((__float_as_uint(amax) >> 23) & 0xffu);
    const int s = (amax == 0.0f || ex == 0) ? 0 : min(254, max(0, ex - 2));
    inv = __uint_as_float((uint32_t)(254 - s) << 23);
    return s;
}

typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef int i32x6 __attribute__((ext_vector_type(6)));

// The two scaled conversions, with their results in registers apart from
// their operands (early clobber). The compiler's builtins may give the
// 6-register result of v_cvt_scalef32_2xpk16_fp6_f32 registers that overlap
// the tail of an operand; the instruction writes its first result dwords
// before it reads the last operand registers, which then turned the last
// elements' codes wrong (elements 29 and 31 when the result overlapped the
// second operand's registers 14-15).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ i32x6 cvt_fp6_of(f32x16 ev, f32x16 od, float X)
{
    i32x6 r;
    asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(ev), "v"(od), "v"(X));
    return r;
}
__device__ __forceinline__ f32x32 cvt_f32_of(i32x6 c, float X)
{
    f32x32 d;
    asm("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2" : "=&v"(d) : "v"(c), "v"(X));
    return d;
}
#pragma clang diagnostic pop

// One plane of one block: the codes of v (32 values), packed 6 bits each into
// w[0..5], and v replaced by its residual v - decode (exact in fp32).
//
// Blocks with a normal scale (s > 0) use the gfx950 scaled conversions
// (above): v_cvt_scalef32_2xpk16_fp6_f32 rounds x / X to nearest-even E2M3 with
// magnitudes beyond 7.5 saturating to 7.5 and the sign kept on zeros (output
// element 2 i from its first operand's element i, 2 i + 1 from the second's),
// and v_cvt_scalef32_pk32_f32_fp6 decodes code * X; a one-wave probe matched
// both to the rounding above on grid values, ties, near-ties, the clamp
// region and signed zeros. Blocks whose scale is the fp32 subnormal 2^-127
// (amax below 2^-125) and all-zero blocks take the element-wise path.
__device__ __forceinline__ uint32_t mxfp6_plane(float v[32], uint32_t w[6])
{
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
    float inv;
    const int s = mxfp6_scale(amax, inv);
    if (s > 0 && amax != 0.0f) {
        const float X = __uint_as_float((uint32_t)s << 23);
        f32x16 ev, od;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            ev[i] = v[2 * i];
            od[i] = v[2 * i + 1];
        }
        const i32x6 c = cvt_fp6_of(ev, od, X);
        const f32x32 d = cvt_f32_of(c, X);
#pragma unroll
        for (int j = 0; j < 6; j++) w[j] = (uint32_t)c[j];
#pragma unroll
        for (int j = 0; j < 32; j++) v[j] -= d[j];
        return (uint32_t)s;
    }
    // 2^(s - 127), an fp32 subnormal for s = 0
    const float X = s ? __uint_as_float((uint32_t)s << 23) : __uint_as_float(0x00400000u);
#pragma unroll
    for (int j = 0; j < 6; j++) w[j] = 0u;
#pragma unroll
    for (int j = 0; j < 32; j++) {
        const uint32_t c = amax == 0.0f ? 0u : e2m3_code(v[j] * inv);
        v[j] -= e2m3_value(c) * X;
        const int bit = 6 * j, wd = bit >> 5, off = bit & 31;
        w[wd] |= c << off;
        if (off > 26) w[wd + 1] |= c >> (32 - off);
    }
    return (uint32_t)s;
}

// One 128-byte record written by a lane pair: the lanes 2 m and 2 m + 1 of a
// wave hold blocks 2 s and 2 s + 1 of the record, with their 48 code bytes
// each and their two scale bytes each. The scale pairs meet in
// both lanes (a DPP swap of neighbours); the even lane stores the 16-byte
// scale chunk (four copies), the odd one the 16 zero bytes: four 16-byte
// stores per lane, none of 2 bytes. Both lanes of a pair must be active.
__device__ __forceinline__ void f6_store_pair(uint8_t *rec, int half, const uint32_t w[12],
                                              uint32_t s1, uint32_t s2)
{
    u32x4 *dst = (u32x4 *)(rec + 64 * half);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    dst[2] = u32x4{w[8], w[9], w[10], w[11]};
    const uint32_t sc = s1 | (s2 << 8);
    const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0xB1, 0xF, 0xF, false);
    const uint32_t sw = half ? 0u : (sc | (other << 16));
    dst[3] = u32x4{sw, sw, sw, sw};
}

template <typename InT>
__device__ __forceinline__ void f6_load32(const InT *p, float v[32]);
template <>
__device__ __forceinline__ void f6_load32<float>(const float *p, float v[32])
{
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const float4 t = ((const float4 *)p)[j];
        v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
    }
}
template <>
__device__ __forceinline__ void f6_load32<bf16>(const bf16 *p, float v[32])
{
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const bf16x8 t = ((const bf16x8 *)p)[j];
#pragma unroll
        for (int i = 0; i < 8; i++) v[8 * j + i] = (float)t[i];
    }
}

// Rows n < min(N, *n_dev) (all N rows when n_dev is null); one thread per
// 32-element block, grid-stride. Row n of the output at out + n * ldo bytes.
// K % 64 == 0, so the two blocks of a record sit in lanes 2 m and 2 m + 1 and
// enter and leave the loop together (f6_store_pair).
template <typename InT>
__global__ __launch_bounds__(256) void fp6x2_split_kernel(const InT *__restrict__ v, int64_t ldv,
                                                          int64_t N, int K,
                                                          const int32_t *__restrict__ n_dev,
                                                          uint8_t *__restrict__ out, int64_t ldo)
{
    const int nb = K / 32;
    const int64_t rows = n_dev ? min(N, (int64_t)max(*n_dev, 0)) : N;
    const int64_t total = rows * nb;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = i / nb;
        const int b = (int)(i - n * nb);
        float x[32];
        f6_load32<InT>(v + n * ldv + 32 * b, x);
        uint32_t w[12];
        const uint32_t s1 = mxfp6_plane(x, w);
        const uint32_t s2 = mxfp6_plane(x, w + 6);
        f6_store_pair(out + n * ldo + (b >> 1) * 128, b & 1, w, s1, s2);
    }
}

hipError_t launch_fp6x2_split(const void *v, int v_f32, int64_t ldv, int64_t N, int K,
                              uint8_t *out, int64_t ldo, hipStream_t s, const int32_t *n_dev)
{
    const int64_t nb = N * (K / 32);
    if (K % 64 != 0) return hipErrorInvalidValue;  // records pair the blocks of 64
    if (nb <= 0) return hipSuccess;
    const dim3 grid((unsigned)std::min<int64_t>((nb + 255) / 256, 16384)), block(256);
    if (v_f32)
        hipLaunchKernelGGL(fp6x2_split_kernel<float>, grid, block, 0, s, (const float *)v, ldv, N,
                           K, n_dev, out, ldo);
    else
        hipLaunchKernelGGL(fp6x2_split_kernel<bf16>, grid, block, 0, s, (const bf16 *)v, ldv, N,
                           K, n_dev, out, ldo);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped projection on the block-scaled matrix cores, 256-row tiles.
//
// Workgroup tile: up to 256 or 128 permuted rows of one expert (a work item
// of the 256- or 128-row plan) x 256 weight rows, K step 64 (two MX blocks,
// one 128-byte record of a split row). NW waves: 16 on 256-row tiles (one
// workgroup per CU); 8 on 128-row tiles, whose 80 KB of LDS and at most 128
// VGPRs let two workgroups share a CU, so that one's prologue, epilogue and
// launch overlap the other's K loop; or 8 wide waves on 256-row tiles (WIDE).
// Wave w: row block q = w / 4 (row tiles 2 q, 2 q + 1 of 32) and slot
// c = w % 4 (gate and up rows of output columns 32 c .. + 32, or weight rows
// 64 c .. + 64); a wide wave: row block w / 2 and slots 2 (w % 2) and
// 2 (w % 2) + 1. Per K step and (row tile, weight tile) two 32 x 32 x 64
// MFMAs, one per plane, into the same fp32 accumulator.
//
// Operands, as the instruction takes them (lane L, l = L % 32, g = L / 32;
// checked with a one-wave probe against an fp64 evaluation):
//   A (E2M3, 24 bytes): row l, MX block g of the step, the 24 stored bytes;
//   B (E2M1, 16 bytes): weight row l, MX block g, the 16 stored code bytes;
//   scales: lane L gives its row's (A) or weight row's (B) E8M0 code for
//     MX block g.
//
// LDS: a three-stage ring filled by global_load_lds_dwordx4 (each stage:
// 16 NW rows x 128 bytes of records, 256 weight rows x 32 code bytes), one
// barrier per K step publishing step k and freeing the stage that step k + 2
// overwrites (128-row tiles whose weight scales leave no room for a third
// stage in 80 KB, K > 1024: two stages, loads one step ahead, the barrier
// publishing step k and freeing the stage step k + 1 overwrites); the tile's
// weight scales (256 x K / 32 bytes) loaded once, in
// the streaming layout's order (16 groups of 16 weight rows, each group as
// the layout stores it), by the same DMA ahead of the first two stages. Chunk c (16 bytes) of a row's record
// sits at position c ^ ((r / 2) % 8), so the 16 rows of a 16-lane read
// cover all banks (the bf16 kernel's A arrangement); lanes 32-63 read the
// other half of each record (block 1), whose positions differ from block 0's
// by 4 (measured: 85% of LDS-active cycles in bank conflicts when the blocks
// sat at bytes 0 and 48).
// ---------------------------------------------------------------------------
constexpr int F6_BN = 256, F6_BK = 64, F6_ROW = 128;
constexpr int F6_W_BYTES = F6_BN * F6_BK / 2;    // 8 KB of E2M1 codes
// NW: 16 (256-row tiles, 32 KB of records per stage) or 8 (128-row tiles); the
// wide-wave 256-row tile sizes its LDS as the 16-wave one (f6_a_bytes(16) ...)
__host__ __device__ constexpr int f6_a_bytes(int NW) { return 16 * NW * F6_ROW; }
__host__ __device__ constexpr int f6_stage(int NW) { return f6_a_bytes(NW) + F6_W_BYTES; }
constexpr int F6_MAX_K = 4096;

// Weight scales of 16 weight rows in the streaming layout: K / 512 groups
// (rounded up) of 256 bytes; the LDS copy of a tile holds 16 of them.
__host__ __device__ constexpr int f6_scale_chunk(int K)
{
    return 256 * ((K / 128 + 3) / 4);
}

// the epilogue's staging: per wave 64 rows of up to 256 bytes, padded by 16
constexpr int F6_EPI_PITCH = 144;
// LDS per workgroup that lets two 128-row workgroups share a CU's 160 KB
constexpr int F6_LDS_HALF = 80 * 1024;

__host__ __device__ constexpr int f6_lds_bytes(int K, int NW, int STG)
{
    return STG * f6_stage(NW) + 16 * f6_scale_chunk(K) > NW * 64 * F6_EPI_PITCH
               ? STG * f6_stage(NW) + 16 * f6_scale_chunk(K)
               : NW * 64 * F6_EPI_PITCH;
}
static_assert(f6_lds_bytes(F6_MAX_K, 16, 3) <= 160 * 1024, "LDS of the FP6X2 tile");
static_assert(f6_lds_bytes(1024, 8, 3) <= F6_LDS_HALF, "three stages of 128 rows at K <= 1024");
static_assert(f6_lds_bytes(F6_MAX_K, 8, 2) <= F6_LDS_HALF, "two stages of 128 rows at any K");

// Output kinds of the projection: OutT = float or bf16 rows, uint8_t for
// split records (the next projection's input, written as moe_fp6x2_split
// would write the fp32 results), or int16_t for block-int16 rows (the expert
// outputs inside the layer, read once by the combine): per 32 columns one
// code e in osc, the biased exponent of the block's largest magnitude m
// (at most 252), and each value v as the integer q nearest 32767 v 2^(126 - e)
// (|v| 2^(126 - e) < 1), standing for q 2^(e - 126) / 32767: within
// 2^(e - 126) / 65534 <= 2^-15 m of v.
template <typename OutT>
constexpr bool f6_records = std::is_same<OutT, uint8_t>::value;
template <typename OutT>
constexpr bool f6_q16 = std::is_same<OutT, int16_t>::value;

template <int ACT, typename OutT, bool PACKED, int NW, int F6_STAGES, bool WIDE>
__global__ __launch_bounds__(NW * 64, WIDE ? 1 : 16 / NW) void gemm_fp6x2_w16_kernel(
    const uint8_t *__restrict__ ad, int64_t lda, const int32_t *__restrict__ a_rows,
    const uint8_t *__restrict__ w1c, const uint8_t *__restrict__ w1s,
    const uint8_t *__restrict__ w2c, const uint8_t *__restrict__ w2s,
    const int32_t *__restrict__ plan, int hdr, int N, int K, OutT *__restrict__ out,
    int64_t ldo, uint8_t *__restrict__ osc)
{
    constexpr bool GLU = ACT != ACT_NONE;
    constexpr int COLS = GLU ? F6_BN / 2 : F6_BN;
    static_assert(!(GLU && f6_q16<OutT>), "block-int16 rows come from the down projection");
    extern __shared__ __attribute__((aligned(16))) uint8_t f6_lds[];
    const int chunk_b = f6_scale_chunk(K);
    // WIDE: 8 waves on a 256-row tile, each wave holding two column slots
    // (64 rows x 2 COLS_W columns): per MFMA a third less LDS read than a
    // wave per slot, as a wave's A fragments serve four weight fragments
    constexpr int SPW = WIDE ? 2 : 1, NJ = 2 * SPW;
    static_assert(!WIDE || NW == 8, "wide waves tile 256 rows with 8 waves");
    constexpr int F6_THREADS = NW * 64, F6_A_BYTES = f6_a_bytes(NW * SPW),
                  F6_STAGE = f6_stage(NW * SPW);
    uint8_t *const Wsc = f6_lds + F6_STAGES * F6_STAGE;  // [16][chunk_b] weight scales

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
    // column slot (the first of the wave's SPW) and 64-row block
    const int slot0 = WIDE ? 2 * (wave & 1) : (wave & 3), q = WIDE ? wave >> 1 : wave >> 2;
    const int nch = K / 128;
    const int64_t row_b = 2 * lda;  // bytes per split row

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

    // ---- DMA sources. Records: instruction j of wave w fills rows
    // 16 SPW w + 8 j .. + 7 (lane L: chunk position L % 8 of row
    // 16 SPW w + 8 j + L / 8).
    const uint8_t *ag[2 * SPW];
#pragma unroll
    for (int j = 0; j < 2 * SPW; j++) {
        const int rt = 16 * SPW * wave + 8 * j + (lane >> 3);
        const int rc = min(r0 + rt, rend - 1);
        const int64_t arow = a_rows ? (int64_t)a_rows[rc] : (int64_t)rc;
        ag[j] = ad + arow * row_b + 16 * ((lane & 7) ^ ((rt >> 1) & 7));
    }
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
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(f6_lds));
    auto issue = [&](int kt, int st) {
        const uint32_t sb = lds0 + st * F6_STAGE;
#pragma unroll
        for (int j = 0; j < 2 * SPW; j++)
            dma16(ag[j] + kt * F6_ROW, sb + (2 * SPW * wave + j) * 1024);
        if (wload) {
            const uint8_t *src;
            if constexpr (PACKED)
                src = bg + (kt >> 1) * 1024 + (2 * (kt & 1) + bh) * 256;
            else
                src = bg + kt * (F6_BK / 2);
            dma16(src, sb + F6_A_BYTES + wave * 1024);
        }
    };

    const int nk = K / F6_BK;  // even: K is a multiple of 128

    // ---- weight scales -> LDS. Group c of 16 LDS weight rows (16 c .. +15)
    // in the streaming layout's order: the scale of k-block kb of its row r
    // is byte (kb % 16) / 4 of the word at (kb / 16) * 256 + (kb % 4) * 64 +
    // (r % 16) * 4. Streaming weights: each group is contiguous in HBM (N is
    // a multiple of 16), so 16 DMA copies, issued before the first stages so
    // that the first barrier's wait covers them; groups past N take the last
    // group's scales (their rows are clamped and their outputs dropped).
    if constexpr (PACKED) {
        for (int m = wave; m < 16 * chunk_b / 1024; m += F6_THREADS / 64) {
            const int b = 1024 * m + 16 * lane;
            const int c = b / chunk_b, off = b - c * chunk_b;
            const int wr0 = min(GLU ? n0 + ((16 * c) & 127) : n0 + 16 * c, N - 16);
            const uint8_t *ws = (GLU && c >= 8) ? w2s : w1s;
            dma16(ws + (((int64_t)e * N + wr0) / 16) * chunk_b + off,
                  lds0 + F6_STAGES * F6_STAGE + 1024 * m);
        }
    } else {
        // row-major scales: a word holds k-blocks 4 r .. 4 r + 3 of a row
        const int per_row = K / 128;
        for (int idx = tid; idx < 256 * per_row; idx += F6_THREADS) {
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
    if constexpr (F6_STAGES == 3) issue(1, 1);

    // ---- wave tiles
    const int h = lane >> 5, l32 = lane & 31;
    // weight fragment jj: slot slot0 + jj / 2, half jj % 2 (GLU: gate, up)
    int bt[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; jj++) {
        const int sl = slot0 + jj / 2, j = jj & 1;
        bt[jj] = GLU ? 128 * j + 32 * sl : 64 * sl + 32 * j;
    }
    const int n_on = (64 * q < mrows ? 1 : 0) + (64 * q + 32 < mrows ? 1 : 0);
    const int bpos = 16 * (h ^ ((l32 >> 3) & 1));
    // rows 64 q + 32 i + l32 share (row / 2) % 8 = (l32 / 2) % 8; block h is
    // logical chunks 4 h .. 4 h + 2, the scales chunk 3 (the copy that rows
    // with the same key and parity read apart)
    const int key = (l32 >> 1) & 7;
    // weight scales: this lane's rows and MX block h; the step adds
    // (k / 8) * 256 + (k % 2) * 128 + (k % 8) / 2 (k-block 2 k + h)
    int wso[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        const int row = bt[j] + l32;
        wso[j] = (row / 16) * chunk_b + (row % 16) * 4 + 64 * h;
    }
    const int apos0 = ((4 * h) ^ key) << 4, apos1 = ((4 * h + 1) ^ key) << 4,
              apos2 = ((4 * h + 2) ^ key) << 4,
              spos = ((3 ^ key) << 4) + 4 * (2 * ((l32 >> 4) & 1) + (l32 & 1)) + 2 * h;

    auto run = [&](auto ni_c) {
        constexpr int NI = decltype(ni_c)::value;
        f32x16 acc[NI > 0 ? NI : 1][NJ];
#pragma unroll
        for (int i = 0; i < NI; i++)
#pragma unroll
            for (int j = 0; j < NJ; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

        auto compute = [&](int st, int kt) {
            if constexpr (NI > 0) {
                const uint8_t *Ap = f6_lds + st * F6_STAGE;
                const uint8_t *Bq = Ap + F6_A_BYTES;
                i32x8 bv[NJ];
                int sb[NJ];
#pragma unroll
                for (int j = 0; j < NJ; j++) {
                    const int row = bt[j] + l32;
                    const u32x4 w = *(const u32x4 *)(Bq + row * 32 + bpos);
                    bv[j] = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
                    sb[j] = Wsc[wso[j] + (kt >> 3) * 256 + (kt & 1) * 128 + ((kt & 7) >> 1)];
                }
                i32x8 a1[NI > 0 ? NI : 1], a2[NI > 0 ? NI : 1];
                int sa[NI > 0 ? NI : 1];
#pragma unroll
                for (int i = 0; i < NI; i++) {
                    const uint8_t *ar = Ap + (64 * q + 32 * i + l32) * F6_ROW;
                    // plane 1 is dwords 0-5 of the lane's 48 bytes, plane 2
                    // dwords 6-11 (the instruction reads 6 registers of a
                    // 6-bit operand; lanes 6-7 are ignored)
                    const u32x4 c0 = *(const u32x4 *)(ar + apos0);
                    const u32x4 c1 = *(const u32x4 *)(ar + apos1);
                    const u32x4 c2 = *(const u32x4 *)(ar + apos2);
                    a1[i] = i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                                  (int)c1[0], (int)c1[1], 0, 0};
                    a2[i] = i32x8{(int)c1[2], (int)c1[3], (int)c2[0], (int)c2[1],
                                  (int)c2[2], (int)c2[3], 0, 0};
                    // both planes' scales: bytes 0 and 1, selected by the
                    // instruction's scale byte select
                    sa[i] = (int)*(const uint16_t *)(ar + spos);
                }
                // A format 2: E2M3; B format 4: E2M1; the A scale is byte 0
                // (plane 1) or byte 1 (plane 2) of sa, the B scale byte 0
#pragma unroll
                for (int i = 0; i < NI; i++)
#pragma unroll
                    for (int j = 0; j < NJ; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            a1[i], bv[j], acc[i][j], 2, 4, 0, sa[i], 0, sb[j]);
#pragma unroll
                for (int i = 0; i < NI; i++)
#pragma unroll
                    for (int j = 0; j < NJ; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            a2[i], bv[j], acc[i][j], 2, 4, 1, sa[i], 0, sb[j]);
            }
        };

        for (int kt = 0; kt < nk; kt++) {
            // this wave's loads of step kt are done: at most two of its loads
            // are left in flight, all of step kt + 1 (a wave that also loads
            // codes issues three per step and so waits for one of kt + 1's
            // too: one wait for every wave, no branch); the barrier publishes
            // every wave's and ends the reads of step kt - 1
            // (two stages: only step kt's loads are in flight, all waited for;
            // with 8 waves every wave issues three loads per step)
            // (wide waves: four record loads and one code load per step)
            if (F6_STAGES == 3 && kt + 1 < nk) {
                if constexpr (WIDE)
                    asm volatile("s_waitcnt vmcnt(5)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                else if constexpr (NW == 8)
                    asm volatile("s_waitcnt vmcnt(3)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(2)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
            if constexpr (F6_STAGES == 3) {
                const int st = kt % 3;
                if (kt + 2 < nk) issue(kt + 2, st == 0 ? 2 : st - 1);
                compute(st, kt);
            } else {
                const int st = kt & 1;
                if (kt + 1 < nk) issue(kt + 1, st ^ 1);
                compute(st, kt);
            }
        }

        // Epilogue through LDS (the ring is idle once every wave is past its
        // last step). Lane holds C[8 (v / 4) + 4 h + v % 4][l32] of each
        // 32 x 32 accumulator tile; a wave's output is rows 64 q .. + 63 of
        // columns c0 .. c0 + COLS_W - 1.
        __syncthreads();
        constexpr int COLS_W = GLU ? 32 : 64;
        // the staging area of row block q, slot sl: 64 rows of F6_EPI_PITCH
        auto area = [&](int sl) { return f6_lds + (4 * q + sl) * (64 * F6_EPI_PITCH); };
        if constexpr (f6_records<OutT>) {
            // (GLU only: a wave's 32 output columns are one MX block.) The
            // fp32 results of the wave's 64 rows staged, 128 bytes per row.
            // Then thread t takes row t / 4 of the tile and block t % 4 (the
            // columns of slot t % 4), from the staging of the wave that holds
            // them, converts it as the split does, and lanes 4 r, 4 r + 1 and
            // 4 r + 2, 4 r + 3 write the row's two records as pairs (a pair
            // is active together: it shares the row, and N % 64 == 0)
            static_assert(GLU, "records are written by the GLU projection");
#pragma unroll
            for (int s2 = 0; s2 < SPW; s2++) {
                uint8_t *const stg = area(slot0 + s2);
#pragma unroll
                for (int i = 0; i < NI; i++)
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int r = 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                        ((float *)(stg + r * F6_EPI_PITCH))[l32] =
                            act_apply<ACT>(acc[i][2 * s2][v], acc[i][2 * s2 + 1][v]);
                    }
            }
            __syncthreads();
#pragma unroll
            for (int pass = 0; pass < SPW; pass++) {
                const int R = (tid >> 2) + pass * (F6_THREADS / 4), bb = tid & 3;
                const int cb = n0 + 32 * bb;
                if (R < mrows && cb < N) {
                    const uint8_t *src = f6_lds + (4 * (R >> 6) + bb) * (64 * F6_EPI_PITCH) +
                                         (R & 63) * F6_EPI_PITCH;
                    float x[32];
#pragma unroll
                    for (int j = 0; j < 8; j++) {
                        const f32x4 t = *(const f32x4 *)(src + 16 * j);
                        x[4 * j] = t[0]; x[4 * j + 1] = t[1]; x[4 * j + 2] = t[2]; x[4 * j + 3] = t[3];
                    }
                    uint32_t w[12];
                    const uint32_t s1 = mxfp6_plane(x, w);
                    const uint32_t s2 = mxfp6_plane(x, w + 6);
                    const int b = cb >> 5;
                    f6_store_pair((uint8_t *)out + (int64_t)(r0 + R) * 2 * ldo + (b >> 1) * 128, b & 1, w,
                                  s1, s2);
                }
            }
        } else {
            // one 32-row tile at a time, staged (fp32 for block-int16 rows)
            // and stored as whole row segments
            using StT = typename std::conditional<f6_q16<OutT>, float, OutT>::type;
            constexpr int ROW_B = COLS_W * (int)sizeof(StT);  // 64, 128 or 256 bytes
            constexpr int PITCH = ROW_B + 16;
            constexpr int LPR = ROW_B / 16, RPI = 64 / LPR;    // lanes per row, rows per store
            static_assert(32 * PITCH <= 64 * F6_EPI_PITCH, "staging fits the wave's area");
#pragma unroll
            for (int s2 = 0; s2 < SPW; s2++) {
                const int c0 = n0 + COLS_W * (slot0 + s2);
                const bool col_on = c0 < N;  // N is a multiple of 64
                uint8_t *const stg = area(slot0 + s2);
#pragma unroll
                for (int i = 0; i < NI; i++) {
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int r = 8 * (v >> 2) + 4 * h + (v & 3);
                        StT *row = (StT *)(stg + r * PITCH);
                        if constexpr (GLU) {
                            store_out<StT>(row + l32,
                                           act_apply<ACT>(acc[i][2 * s2][v], acc[i][2 * s2 + 1][v]));
                        } else {
#pragma unroll
                            for (int j = 0; j < 2; j++)
                                store_out<StT>(row + 32 * j + l32, acc[i][2 * s2 + j][v]);
                        }
                    }
                    // block-int16 rows: this lane's row of iteration 0
                    OutT *yrow = nullptr;
                    uint8_t *srow = nullptr;
                    if constexpr (f6_q16<OutT>) {
                        const int64_t r = (int64_t)r0 + 64 * q + 32 * i + lane / LPR;
                        yrow = out + r * ldo + c0 + 4 * (lane % LPR);
                        srow = osc + r * (ldo / 32) + (c0 + 4 * (lane % LPR)) / 32;
                    }
#pragma unroll
                    for (int it = 0; it < 32 / RPI; it++) {
                        const int r = RPI * it + lane / LPR, seg = lane % LPR;
                        const u32x4 val = *(const u32x4 *)(stg + r * PITCH + 16 * seg);
                        const int rl = 64 * q + 32 * i + r;
                        if constexpr (f6_q16<OutT>) {
                            // columns c0 + 4 seg .. + 3; the 8 lanes with equal
                            // lane / 8 hold one 32-column block. Magnitudes are
                            // compared as bit patterns (non-negative floats
                            // order as their bits)
                            uint32_t mb = 0;
#pragma unroll
                            for (int c = 0; c < 4; c++) mb = max(mb, val[c] & 0x7fffffffu);
                            // max over the 8 lanes: swap neighbours, then pairs
                            // (quad_perm 1,0,3,2 and 2,3,0,1), then mirror the
                            // 8-lane half row (lane i and 7 - i): DPP moves on
                            // the vector unit, no LDS round trip
                            mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xB1, 0xF, 0xF, false));
                            mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x4E, 0xF, 0xF, false));
                            mb = max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x141, 0xF, 0xF, false));
                            // e: the block's largest biased exponent (at most
                            // 252: larger blocks saturate); x 2^(126 - e) lies
                            // in (-1, 1), and v_cvt_pknorm_i16_f32 rounds its
                            // 32767 multiple to an integer, two values a step
                            const int code = min((int)(mb >> 23), 252);
                            const float inv = __uint_as_float((uint32_t)(253 - code) << 23);
                            if (col_on && rl < mrows) {
                                float x[4];
#pragma unroll
                                for (int c = 0; c < 4; c++) x[c] = __uint_as_float(val[c]) * inv;
                                const u32x2 pk = {
                                    (uint32_t)__builtin_bit_cast(int, __builtin_amdgcn_cvt_pknorm_i16(x[0], x[1])),
                                    (uint32_t)__builtin_bit_cast(int, __builtin_amdgcn_cvt_pknorm_i16(x[2], x[3]))};
                                __builtin_nontemporal_store(pk, (u32x2 *)(yrow + (int64_t)it * RPI * ldo));
                                if ((seg & 7) == 0)
                                    srow[(int64_t)it * RPI * (ldo / 32)] = (uint8_t)code;
                            }
                        } else if (col_on && rl < mrows) {
                            u32x4 *dst = (u32x4 *)((uint8_t *)(out + (int64_t)(r0 + rl) * ldo + c0) +
                                                   16 * seg);
                            if constexpr (!GLU && sizeof(OutT) == 4) __builtin_nontemporal_store(val, dst);
                            else *dst = val;
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

template <int ACT, typename OutT, bool PACKED, int NW, bool WIDE = false>
static hipError_t launch_f6_nw(const uint8_t *ad, int64_t lda, const int32_t *a_rows,
                            const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                            const uint8_t *w2s, const int32_t *plan,
                            int max_groups, int hdr, int N, int K, OutT *out, int64_t ldo,
                            uint8_t *osc, hipStream_t s)
{
    constexpr int COLS = ACT != ACT_NONE ? F6_BN / 2 : F6_BN;
    const int64_t grid = (int64_t)max_groups * ((N + COLS - 1) / COLS);
    if (grid <= 0) return hipSuccess;
    // the XCD-aware order maps block b to work (b % 8) * ceil(total / 8) + b / 8;
    // a grid of 8 * ceil(bound / 8) blocks covers every work item
    const int64_t G = (grid + 7) / 8 * 8;
    // 128-row tiles: three stages where two workgroups still fit a CU, else
    // two (S2 keeps the 16-wave kernel on three stages only)
    // (wide waves: the 256-row tile's LDS, three stages)
    constexpr int S2 = NW == 8 && !WIDE ? 2 : 3, NR = WIDE ? 16 : NW;
    const bool three = NR == 16 || f6_lds_bytes(K, NW, 3) <= F6_LDS_HALF;
    auto kern = three ? gemm_fp6x2_w16_kernel<ACT, OutT, PACKED, NW, 3, WIDE>
                      : gemm_fp6x2_w16_kernel<ACT, OutT, PACKED, NW, S2, WIDE>;
    const int lds = f6_lds_bytes(K, NR, three ? 3 : 2);
    const hipError_t err = ensure_dynamic_lds((const void *)kern, lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(NW * 64), lds, s, ad, lda,
                       a_rows, w1c, w1s, w2c, w2s, plan, hdr, N, K, out, ldo, osc);
    return hipGetLastError();
}

hipError_t launch_gemm_fp6x2_run(const uint8_t *ad, int64_t lda, const int32_t *a_rows,
                                 const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                                 const uint8_t *w2s, int num_local, int max_rows, int N, int K,
                                 int act, void *out, int out_kind, int64_t ldo,
                                 const void *plan_ws, int packed, hipStream_t s,
                                 uint8_t *out_scales, int rows128)
{
    if (K % 128 != 0 || K > F6_MAX_K) return hipErrorInvalidValue;
    if (out_kind == F6_OUT_RECORDS && act == ACT_NONE) return hipErrorInvalidValue;
    if (out_kind == F6_OUT_Q16 && (act != ACT_NONE || out_scales == nullptr || ldo % 32 != 0))
        return hipErrorInvalidValue;
    const GemmPlanArgs pa =
        gemm_plan_args(num_local, max_rows, rows128 ? MOE_SCHED_TILE128 : MOE_SCHED_TILE256, nullptr);
    if (rows128 && out_kind != F6_OUT_Q16 && out_kind != F6_OUT_RECORDS) return hipErrorInvalidValue;
    const int32_t *plan = (const int32_t *)plan_ws;
#define F6_LAUNCH(A, OT, PK)                                                                   \
    return launch_f6_nw<A, OT, PK, 16>(ad, lda, a_rows, w1c, w1s, w2c, w2s, plan, pa.max_groups,  \
                                    pa.hdr, N, K, (OT *)out, ldo, out_scales, s)
#define F6_LAUNCHW(A, OT, PK)                                                                  \
    return launch_f6_nw<A, OT, PK, 8, true>(ad, lda, a_rows, w1c, w1s, w2c, w2s, plan,         \
                                         pa.max_groups, pa.hdr, N, K, (OT *)out, ldo,          \
                                         out_scales, s)
#define F6_LAUNCH8(A, OT, PK)                                                                  \
    return launch_f6_nw<A, OT, PK, 8>(ad, lda, a_rows, w1c, w1s, w2c, w2s, plan, pa.max_groups,   \
                                   pa.hdr, N, K, (OT *)out, ldo, out_scales, s)
#define F6_GLU(OT, PK)                                                                         \
    switch (act) {                                                                             \
    case ACT_SILU_MUL: F6_LAUNCH(ACT_SILU_MUL, OT, PK);                                       \
    case ACT_GELU_TANH_MUL: F6_LAUNCH(ACT_GELU_TANH_MUL, OT, PK);                             \
    default: return hipErrorInvalidValue;                                                      \
    }
#define F6_ANY(OT, PK)                                                                         \
    {                                                                                          \
        if (act == ACT_NONE) F6_LAUNCH(ACT_NONE, OT, PK);                                      \
        F6_GLU(OT, PK)                                                                         \
    }
    if (out_kind == F6_OUT_RECORDS && rows128) {
        switch (act) {
        case ACT_SILU_MUL:
            if (packed) F6_LAUNCH8(ACT_SILU_MUL, uint8_t, true);
            F6_LAUNCH8(ACT_SILU_MUL, uint8_t, false);
        case ACT_GELU_TANH_MUL:
            if (packed) F6_LAUNCH8(ACT_GELU_TANH_MUL, uint8_t, true);
            F6_LAUNCH8(ACT_GELU_TANH_MUL, uint8_t, false);
        default: return hipErrorInvalidValue;
        }
    }
    // 256-row gate/up tiles over at least 512 rows per expert on average
    // (the row bound's): wide waves, which read a third less LDS per MFMA;
    // over fewer rows the tiles are mostly part-filled, and 16 waves, each
    // SIMD holding a quarter of every row block's columns, keep the matrix
    // cores evenly loaded where two 64-row waves per SIMD would not
    if (out_kind == F6_OUT_RECORDS && (int64_t)max_rows >= 512 * (int64_t)num_local) {
        switch (act) {
        case ACT_SILU_MUL:
            if (packed) F6_LAUNCHW(ACT_SILU_MUL, uint8_t, true);
            F6_LAUNCHW(ACT_SILU_MUL, uint8_t, false);
        case ACT_GELU_TANH_MUL:
            if (packed) F6_LAUNCHW(ACT_GELU_TANH_MUL, uint8_t, true);
            F6_LAUNCHW(ACT_GELU_TANH_MUL, uint8_t, false);
        default: return hipErrorInvalidValue;
        }
    }
    if (out_kind == F6_OUT_RECORDS) {
        if (packed) F6_GLU(uint8_t, true)
        F6_GLU(uint8_t, false)
    }
    if (out_kind == F6_OUT_F32) {
        if (packed) F6_ANY(float, true)
        F6_ANY(float, false)
    }
    if (out_kind == F6_OUT_Q16 && rows128) {
        if (packed) F6_LAUNCH8(ACT_NONE, int16_t, true);
        F6_LAUNCH8(ACT_NONE, int16_t, false);
    }
    if (out_kind == F6_OUT_Q16) {
        if (packed) F6_LAUNCH(ACT_NONE, int16_t, true);
        F6_LAUNCH(ACT_NONE, int16_t, false);
    }
    if (packed) F6_ANY(bf16, true)
    F6_ANY(bf16, false)
#undef F6_ANY
#undef F6_GLU
#undef F6_LAUNCH
#undef F6_LAUNCH8
#undef F6_LAUNCHW
}

hipError_t launch_grouped_gemm_fp6x2(const uint8_t *ad, int64_t lda, const int32_t *a_rows,
                                     const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                                     const uint8_t *w2s, const int32_t *off, int num_local,
                                     int max_rows, int N, int K, int act, void *out,
                                     int out_kind, int64_t ldo, void *ws, int packed,
                                     hipStream_t s)
{
    hipError_t e = launch_gemm_plan_into(
        off, num_local, gemm_plan_args(num_local, max_rows, MOE_SCHED_TILE256, ws), s);
    if (e != hipSuccess) return e;
    return launch_gemm_fp6x2_run(ad, lda, a_rows, w1c, w1s, w2c, w2s, num_local, max_rows, N,
                                 K, act, out, out_kind, ldo, ws, packed, s, nullptr, 0);
}

}  // namespace moe
