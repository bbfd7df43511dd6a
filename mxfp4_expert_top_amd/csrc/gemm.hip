// Grouped expert projections with MXFP4 weights on the gfx950 bf16 matrix
// cores (P2 "SGLang 0.5.17：Kimi K3 原生 MXFP4 推理架构解析", section "MXFP4
// 原生支持": dequantisation fused into the GEMM; P1 "从Kimi K3到MiniMax-H3",
// section 二/第一层: 4-bit weights combined with higher-precision activations,
// dequantise + multiply + accumulate in the kernel).
//
// MXFP4 codes go from HBM into registers (the streaming schedule) or, still
// 4-bit, into LDS (the tiled schedules), are decoded in registers with the
// scaled FP4->bf16 convert (exact: an E2M1 value times a power of two), and
// feed the bf16 matrix instructions (16x16x32 when streaming, 32x32x16 when
// tiled) with fp32 accumulation. No dequantised copy of a weight ever
// reaches memory.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int PLAN_HDR = 64;  // int32 slots before the work items
constexpr int ST_ROWS = 16;   // streaming schedule: permuted rows per group

// ---------------------------------------------------------------------------
// Work plan: each expert's rows in ceil(count / R) groups (plan_item),
// expert-major. plan[0] = number of groups; items from plan[PLAN_HDR].
// The group counts are scanned into each expert's first group index (LDS);
// then every thread writes items p = tid, tid + 1024, ..., finding p's expert
// by binary search. One thread per expert writing its own items serialised a
// hot expert's groups (115 us on a Zipf-routed 64 K-token batch).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void gemm_plan_kernel(const int32_t *__restrict__ off, int nl,
                                                         int R, int max_groups, int balanced,
                                                         int32_t *__restrict__ plan)
{
    __shared__ int32_t part[16];
    __shared__ int32_t gstart[MOE_MAX_EXPERTS_DEV + 1];
    const int tid = threadIdx.x;
    const int per = (nl + 1023) / 1024;
    const int lo = tid * per, hi = min(lo + per, nl);
    int s = 0;
    for (int i = lo; i < hi; i++) s += (off[i + 1] - off[i] + R - 1) / R;
    int ngroups;
    int pos = block_exclusive_scan(s, part, ngroups);
    for (int i = lo; i < hi; i++) {
        gstart[i] = pos;
        pos += (off[i + 1] - off[i] + R - 1) / R;
    }
    if (tid == 0) gstart[nl] = ngroups;
    __syncthreads();
    int2 *items = (int2 *)(plan + PLAN_HDR);
    const int n = min(ngroups, max_groups);
    for (int p = tid; p < n; p += blockDim.x) {
        // the last expert e with gstart[e] <= p; it owns group p (p < gstart[e + 1])
        int a = 0, b = nl - 1;
        while (a < b) {
            const int m = (a + b + 1) >> 1;
            if (gstart[m] <= p) a = m;
            else b = m - 1;
        }
        items[p] = plan_item(a, off[a], off[a + 1] - off[a], gstart[a + 1] - gstart[a],
                             p - gstart[a], R, balanced);
    }
    if (tid == 0) plan[0] = n;
}

// ---------------------------------------------------------------------------
// Weight-streaming schedule (few rows per expert: decode batches).
//
// Work item = (row group of <= 16 rows of expert e, a block of output
// columns); one workgroup per item. Each wave streams ST_NS weight streams of
// 16 rows over all of K; every weight byte is read once per row group. For a
// GLU stage the streams pair up as (W1 rows, W2 rows) of the same output
// columns, so act(gate, up) is applied in registers; for a plain stage each
// stream is 16 more output columns.
//
// Lane L: token row m = L % 16 of the group (A operand), weight row L % 16 of
// each stream (B operand), lane group g = L / 16. Per 128-wide K chunk at kc,
// lane group g holds K elements kc + 32 g .. +32 -- exactly one MX block:
// one 16-byte code load and one scale byte per stream. MFMA step s (0..3)
// takes elements kc + 32 g + 8 s .. +8 of both operands.
//
// Latency: loads of chunk c + ST_D are issued right after chunk c is
// consumed, into a ring of ST_D register slots holding codes, scales and the
// A fragments. Vector loads complete in issue order, so the A loads ride in
// the same ring rather than behind the code prefetch.
//
// Rows past the group's end load a valid row of the group instead (no branch,
// and the repeated address coalesces); their outputs are never stored.
// ---------------------------------------------------------------------------
#ifndef ST_NS
#define ST_NS 4
#endif
#ifndef ST_DMAX
#define ST_DMAX 4
#endif
// Weight codes and scales are read once per row group, so they are loaded
// with the non-temporal hint: a plain read stream of this shape (each wave a
// contiguous run of 1 KB loads) reaches about 6.3 TB/s, with the hint about
// 7.1 TB/s, and the decode gate/up projection went from 0.401 to 0.357 ms.
template <typename T>
__device__ __forceinline__ T stream_load(const T *p)
{
    return __builtin_nontemporal_load(p);
}

template <int ACT>
__host__ __device__ constexpr int stream_cols_per_wave()
{
    return ACT != ACT_NONE ? 8 * ST_NS : 16 * ST_NS;
}

// LoRA increment of the streaming schedule (rank a multiple of 8, at most
// 64): each stream's 16 x 16 accumulator tile gains sum_k t[row][k] B[col][k]
// (t = the scaled rank factors, stored per row as bf16 hi [0, rank) and lo
// [rank, 2 rank) parts whose sum is the fp32 factor to 16 significant bits;
// B = the expert's adapter rows, bf16 [N][rank]) as two more 16x16x32 MFMAs
// (hi, then lo, on the same B fragment) per 32-wide slice of the rank. Lane
// group g supplies elements 8 g .. + 8 of the slice for its token row (A
// operand) and its weight row (B operand); groups past the rank supply zeros.
template <int ACT, typename OutT, int D, bool PACKED, bool LORA>
__global__ __launch_bounds__(256) void gemm_stream_kernel(
    const bf16 *__restrict__ a, int64_t lda, const int32_t *__restrict__ a_rows,
    const uint8_t *__restrict__ w1c, const uint8_t *__restrict__ w1s,
    const uint8_t *__restrict__ w2c, const uint8_t *__restrict__ w2s,
    const int32_t *__restrict__ plan, int N, int K,
    OutT *__restrict__ out, int64_t ldo, LoraEpi lora)
{
    constexpr bool GLU = ACT != ACT_NONE;
    constexpr int NS = ST_NS;
    constexpr int COLS_W = stream_cols_per_wave<ACT>();
    constexpr int COLS_B = 4 * COLS_W;
    // canonical layout: the scales of the workgroup's weight rows, staged in LDS
    extern __shared__ uint32_t sscale[];
    const int nblk = (N + COLS_B - 1) / COLS_B;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;

    const int wi = blockIdx.x;
    if (wi >= plan[0] * nblk) return;
    const int grp = wi / nblk, nb = wi - grp * nblk;
    const int nb0 = nb * COLS_B;                 // first output column of the workgroup
    const int n0 = nb0 + wave * COLS_W;          // first output column of the wave
    const bool wave_on = n0 < N;                 // N is a multiple of COLS_W
    const int2 it = ((const int2 *)(plan + PLAN_HDR))[grp];
    const int e = it.x & 0xffff, r0 = it.y, rend = r0 + (it.x >> 16);
    const int rc = min(r0 + m, rend - 1);
    const int64_t arow = a_rows ? (int64_t)a_rows[rc] : (int64_t)rc;
    const bf16 *ap = a + arow * lda + 32 * g;

    const int nch = K / 128;  // a multiple of D (the launcher picks D)
    const int nc4 = (nch + 3) / 4;
    const int sbw = K / 128;  // canonical: scale dwords per row
    if constexpr (!PACKED) {
        // Canonical scales: one E8M0 byte per 32 weights. Read piecemeal inside
        // the K loop they would be fetched many times over (a 128-byte line
        // holds about one row's worth and the code stream evicts it between
        // reads), so the workgroup first copies the scales of all its weight
        // rows -- one contiguous block per weight matrix -- into LDS.
        const int rows_v = min(COLS_B, N - nb0);
        const int per_mat4 = rows_v * sbw / 4;  // uint4 per matrix (rows_v % 64 == 0)
        for (int i = threadIdx.x; i < (GLU ? 2 : 1) * per_mat4; i += blockDim.x) {
            const int mat = i / per_mat4, r = i - mat * per_mat4;
            const uint8_t *base = (mat ? w2s : w1s) + ((int64_t)e * N + nb0) * (K / 32);
            *(u32x4 *)(&sscale[mat * COLS_B * sbw + 4 * r]) = *(const u32x4 *)(base + 16 * r);
        }
    }

    // Per stream: code pointer (chunk stride 64 canonical, 1024 packed) and the
    // scale source (LDS dword row canonical; global dword packed).
    const uint8_t *cp[NS];
    const uint8_t *spk[NS];
    int srow[NS];
#pragma unroll
    for (int j = 0; j < NS; j++) {
        const int wr0 = GLU ? n0 + 16 * (j / 2) : n0 + 16 * j;  // first row of the 16
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
    uint32_t sq[D][NS];  // packed: the scale dword of each slot's chunk group
    bf16x8 af[D][4];
    f32x4 acc[NS];
#pragma unroll
    for (int j = 0; j < NS; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](int c, u32x4 *qd, uint32_t *sd, bf16x8 *ad) {
#pragma unroll
        for (int j = 0; j < NS; j++) {
            if constexpr (PACKED) {
                qd[j] = stream_load((const u32x4 *)(cp[j] + c * 1024));
                sd[j] = stream_load((const uint32_t *)(spk[j] + (c >> 2) * 256));
            } else {
                qd[j] = stream_load((const u32x4 *)(cp[j] + c * 64));
            }
        }
#pragma unroll
        for (int s = 0; s < 4; s++) ad[s] = *(const bf16x8 *)(ap + c * 128 + 8 * s);
    };
    auto consume = [&](int c, const u32x4 *qd, const uint32_t *sd, const bf16x8 *ad) {
#pragma unroll
        for (int j = 0; j < NS; j++) {
            uint32_t sb;
            if constexpr (PACKED) sb = (sd[j] >> (8 * (c & 3))) & 0xffu;
            else sb = (sscale[srow[j] + c] >> (8 * g)) & 0xffu;
            const float f = e8m0_to_f32(sb);
#pragma unroll
            for (int s = 0; s < 4; s++) acc[j] = mfma16x16x32(ad[s], mx_decode8(qd[j][s], f), acc[j]);
        }
    };
    // prologue: chunks 0 .. D-1 in flight (behind the scale copy's loads)
    if (wave_on) {
#pragma unroll
        for (int d = 0; d < D; d++) issue(d, q[d], sq[d], af[d]);
    }
    if constexpr (!PACKED) __syncthreads();  // scales in LDS
    if (!wave_on) return;
    // LoRA operands, in flight behind the first chunks
    // rank factors as hi and lo bf16 parts (row: hi [0, rank), lo [rank, 2 rank))
    bf16x8 lt[2][2][2], lbf[2][NS];
    if constexpr (LORA) {
        const bf16x8 z = {};
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int k0 = 32 * c + 8 * g;
            const bool on = k0 < lora.rank;
            const int kk = on ? k0 : 0;  // a valid address either way
#pragma unroll
            for (int t = 0; t < (GLU ? 2 : 1); t++) {
                const bf16 *tr = (t ? lora.t2 : lora.t1) + (int64_t)rc * 2 * lora.rank + kk;
                const bf16x8 vh = *(const bf16x8 *)tr;
                const bf16x8 vl = *(const bf16x8 *)(tr + lora.rank);
                lt[c][t][0] = on ? vh : z;
                lt[c][t][1] = on ? vl : z;
            }
#pragma unroll
            for (int j = 0; j < NS; j++) {
                const bool second = GLU && (j & 1);
                const int wr0 = GLU ? n0 + 16 * (j / 2) : n0 + 16 * j;
                const bf16x8 v = *(const bf16x8 *)((second ? lora.b2 : lora.b1) +
                                                   ((int64_t)e * N + wr0 + m) * lora.rank + kk);
                lbf[c][j] = on ? v : z;
            }
        }
    }
    // steady state: consume chunk c, refill its slot with chunk c + D
    for (int c0 = 0; c0 < nch - D; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
            consume(c0 + d, q[d], sq[d], af[d]);
            issue(c0 + d + D, q[d], sq[d], af[d]);
        }
    }
    // drain the last D chunks
#pragma unroll
    for (int d = 0; d < D; d++) consume(nch - D + d, q[d], sq[d], af[d]);

    if constexpr (LORA) {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            if (32 * c >= lora.rank) break;
#pragma unroll
            for (int j = 0; j < NS; j++) {
                acc[j] = mfma16x16x32(lt[c][GLU && (j & 1)][0], lbf[c][j], acc[j]);
                acc[j] = mfma16x16x32(lt[c][GLU && (j & 1)][1], lbf[c][j], acc[j]);
            }
        }
    }

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

// ---------------------------------------------------------------------------
// Tiled schedule (many rows per expert: prefill).
//
// Workgroup tile: TL_BM = 128 permuted rows of one expert x TL_BN = 256 weight
// rows, K step TL_BK = 64 (two MX blocks), 8 waves as 2 (rows) x 4 (weight
// rows), each wave 64 x 64 on v_mfma_f32_32x32x16_bf16 (2 x 2 tiles). A GLU
// tile holds 128 W1 rows and the same 128 W2 rows (128 output columns); each
// wave takes 32 of each, so act(gate, up) is applied in registers. A plain
// tile is 256 output columns.
//
// LDS per stage: the A rows as bf16 and the weight rows still as 4-bit codes
// plus scales; each wave decodes the codes it needs into registers. Two
// stages; the next step's global loads are in flight during the MFMAs and
// land in the other stage, so one barrier per K step.
//
// MFMA operands (32x32x16): lane L supplies row L % 32 of A and column
// L % 32 of B, 8 contraction elements of lane group h = L / 32. Inside a K
// step, lane group h takes MX block h (elements 32 h .. 32 h + 31) and
// sub-step s (0..3) its elements 32 h + 8 s .. +8 -- one 16-byte code read
// and one scale byte per lane per weight tile. Result: lane L holds
// C[8 (v / 4) + 4 h + v % 4][L % 32], v = 0..15.
//
// Rows past the expert's end repeat the last row (never stored); 32-row
// sub-tiles wholly past the end skip their MFMAs.
// ---------------------------------------------------------------------------
constexpr int TL_BM = 128, TL_BN = 256, TL_BK = 64;
constexpr int TL_THREADS = 512;
constexpr int TL_APAD = 8;                   // bf16 pad per A row in LDS
constexpr int TL_ALD = TL_BK + TL_APAD;      // 72 bf16 = 144 bytes per row

// acc += T[trow][0..rank) . B[bcol][0..rank) over a 32 x 32 tile: the MFMA
// operand of lane L is row (A) or column (B) L % 32 with contraction elements
// 8 (L / 32) .. + 8 of each 16-wide step, which is how both factors are
// stored (rank contiguous per row / per weight row). A row of T holds the
// rank factors as two bf16 parts, hi [0, rank) and lo [rank, 2 rank) with
// hi + lo the fp32 factor to 16 significant bits; both meet the same B
// fragment, so the increment carries the factor's fp32 precision rather than
// one bf16 rounding of it.
__device__ __forceinline__ f32x16 lora_add(f32x16 acc, const bf16 *t, int64_t trow,
                                           const bf16 *b, int64_t bcol, int rank, int h)
{
    const bf16 *tr = t + trow * 2 * rank + 8 * h;
    for (int k0 = 0; k0 < rank; k0 += 16) {
        const bf16x8 ahi = *(const bf16x8 *)(tr + k0);
        const bf16x8 alo = *(const bf16x8 *)(tr + rank + k0);
        const bf16x8 bv = *(const bf16x8 *)(b + bcol * rank + k0 + 8 * h);
        acc = mfma32x32x16(ahi, bv, acc);
        acc = mfma32x32x16(alo, bv, acc);
    }
    return acc;
}

template <int ACT>
__host__ __device__ constexpr int tile_cols()
{
    return ACT != ACT_NONE ? TL_BN / 2 : TL_BN;
}

template <int ACT, typename OutT, bool PACKED, bool LORA>
__global__ __launch_bounds__(TL_THREADS, 2) void gemm_tile_kernel(
    const bf16 *__restrict__ a, int64_t lda, const int32_t *__restrict__ a_rows,
    const uint8_t *__restrict__ w1c, const uint8_t *__restrict__ w1s,
    const uint8_t *__restrict__ w2c, const uint8_t *__restrict__ w2s,
    const int32_t *__restrict__ plan, int N, int K,
    OutT *__restrict__ out, int64_t ldo, LoraEpi lora)
{
    constexpr bool GLU = ACT != ACT_NONE;
    constexpr int COLS = tile_cols<ACT>();
    __shared__ __attribute__((aligned(16))) bf16 As[2][TL_BM][TL_ALD];
    __shared__ __attribute__((aligned(16))) uint8_t Bq[2][TL_BN][TL_BK / 2];
    __shared__ uint8_t Bs[2][TL_BN][TL_BK / 32];

    const int nblk = (N + COLS - 1) / COLS;
    const int total = plan[0] * nblk;
    // XCD-aware order: workgroup b runs on XCD b % 8; each XCD takes a
    // contiguous eighth of the actual work (the device-side count, not the
    // launch bound), so a row group's column blocks share one L2.
    const int per_xcd = (total + 7) / 8;
    const int local = blockIdx.x / 8;
    const int wi = (blockIdx.x % 8) * per_xcd + local;
    if (local >= per_xcd || wi >= total) return;
    const int grp = wi / nblk, nb = wi - grp * nblk;
    const int2 it = ((const int2 *)(plan + PLAN_HDR))[grp];
    const int e = it.x & 0xffff, r0 = it.y, rend = r0 + (it.x >> 16);
    const int mrows = rend - r0;
    const int n0 = nb * COLS;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t code_row = K / 2, scale_row = K / 32;

    // ---- global -> LDS assignment
    // A: thread -> row tid / 4, 32 bytes at column 16 * (tid % 4)
    const int ar = tid >> 2, ac = (tid & 3) * 16;
    const int arc = min(r0 + ar, rend - 1);
    const int64_t arow = a_rows ? (int64_t)a_rows[arc] : (int64_t)arc;
    const bf16 *ag = a + arow * lda + ac;
    // B: thread -> weight row tid / 2 of the tile, 16 code bytes (one MX block)
    const int br = tid >> 1, bh = tid & 1;
    int wrow;
    const uint8_t *wcb, *wsb;
    if (GLU) {
        const int n = min(n0 + (br & 127), N - 1);
        wrow = n;
        wcb = br < 128 ? w1c : w2c;
        wsb = br < 128 ? w1s : w2s;
    } else {
        wrow = min(n0 + br, N - 1);
        wcb = w1c;
        wsb = w1s;
    }
    const int64_t wr64 = (int64_t)e * N + wrow;
    // canonical: row-major codes/scales; packed: 16-row blocks x 128-wide
    // chunks (a K step of 64 is half a chunk: MX blocks g = 2 (kt % 2) + bh)
    const int nch = K / 128, nc4 = (nch + 3) / 4;
    const uint8_t *bg, *sg;
    if constexpr (PACKED) {
        const int64_t rb = wr64 / 16;
        const int mm = (int)(wr64 % 16);
        bg = wcb + rb * nch * 1024 + mm * 16;
        sg = wsb + rb * nc4 * 256 + mm * 4;
    } else {
        bg = wcb + wr64 * code_row + 16 * bh;
        sg = wsb + wr64 * scale_row + bh;
    }

    u32x4 ra0, ra1, rb;
    uint8_t rs;
    auto gload = [&](int k0) {
        ra0 = *(const u32x4 *)(ag + k0);
        ra1 = *(const u32x4 *)(ag + k0 + 8);
        if constexpr (PACKED) {
            const int kt = k0 / TL_BK, c = kt >> 1, gg = 2 * (kt & 1) + bh;
            rb = *(const u32x4 *)(bg + c * 1024 + gg * 256);
            rs = sg[(c >> 2) * 256 + gg * 64 + (c & 3)];
        } else {
            rb = *(const u32x4 *)(bg + k0 / 2);
            rs = sg[k0 / 32];
        }
    };
    auto lstore = [&](int st) {
        *(u32x4 *)(&As[st][ar][ac]) = ra0;
        *(u32x4 *)(&As[st][ar][ac + 8]) = ra1;
        *(u32x4 *)(&Bq[st][br][16 * bh]) = rb;
        Bs[st][br][bh] = rs;
    };

    // ---- wave tiles
    const int h = lane >> 5, l32 = lane & 31;
    // weight-row tiles of this wave inside the LDS tile
    int bt[2];
    if (GLU) {
        bt[0] = 32 * wn;        // W1 rows -> output columns n0 + 32 wn + l32
        bt[1] = 128 + 32 * wn;  // the same columns of W2
    } else {
        bt[0] = 64 * wn;
        bt[1] = 64 * wn + 32;
    }
    const bool mt_on[2] = {wm * 64 < mrows, wm * 64 + 32 < mrows};

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    const int nk = K / TL_BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int st = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * TL_BK);
        if (mt_on[0]) {
            u32x4 q[2];
            float f[2];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int row = bt[j] + l32;
                q[j] = *(const u32x4 *)(&Bq[st][row][16 * h]);
                f[j] = e8m0_to_f32(Bs[st][row][h]);
            }
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const bf16x8 b0 = mx_decode8(q[0][s], f[0]), b1 = mx_decode8(q[1][s], f[1]);
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    if (!mt_on[i]) continue;
                    const bf16x8 af =
                        *(const bf16x8 *)(&As[st][wm * 64 + 32 * i + l32][32 * h + 8 * s]);
                    acc[i][0] = mfma32x32x16(af, b0, acc[i][0]);
                    acc[i][1] = mfma32x32x16(af, b1, acc[i][1]);
                }
            }
        }
        if (kt + 1 < nk) lstore(st ^ 1);
        __syncthreads();
    }

    if constexpr (LORA) {
        // the low-rank increment: rank / 16 more MFMA steps per tile
#pragma unroll
        for (int i = 0; i < 2; i++) {
            if (!mt_on[i]) continue;
            const int64_t trow = min(r0 + wm * 64 + 32 * i + l32, rend - 1);
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const bool w2 = GLU && j == 1;
                const int col = GLU ? n0 + 32 * wn + l32 : n0 + 64 * wn + 32 * j + l32;
                acc[i][j] = lora_add(acc[i][j], w2 ? lora.t2 : lora.t1, trow,
                                     (w2 ? lora.b2 : lora.b1) + (int64_t)e * N * lora.rank,
                                     min(col, N - 1), lora.rank, h);
            }
        }
    }

    // ---- epilogue: lane holds C[8 (v / 4) + 4 h + v % 4][l32] of each tile
#pragma unroll
    for (int i = 0; i < 2; i++) {
        if (!mt_on[i]) continue;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int rl = wm * 64 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
            if (rl >= mrows) continue;
            OutT *orow = out + (int64_t)(r0 + rl) * ldo;
            if constexpr (GLU) {
                const int col = n0 + 32 * wn + l32;
                if (col < N) store_out<OutT>(orow + col, act_apply<ACT>(acc[i][0][v], acc[i][1][v]));
            } else {
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int col = n0 + 64 * wn + 32 * j + l32;
                    if (col < N) store_out_once<OutT>(orow + col, acc[i][j][v]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled schedule with 256-row tiles (many rows per expert: prefill).
//
// Workgroup tile: TB_BM = 256 permuted rows of one expert x TB_BN = 256
// weight rows, K step 64. 8 waves as 4 row quarters x 2 weight halves; a wave
// owns 2 row tiles of 32 x 4 weight tiles of 32 on v_mfma_f32_32x32x16_bf16.
// Per MFMA sub-step a wave reads 2 A fragments and 4 decoded weight
// fragments (the weights stay 4-bit in LDS), so LDS traffic per MFMA is about
// 3/8 of a bf16 x bf16 tile of the same shape. A GLU tile holds 128 W1 rows
// and the same 128 W2 rows (128 output columns): weight half ch takes W1 and
// W2 rows 64 ch .. 64 ch + 63, and act(gate, up) is applied in registers.
//
// An expert with up to 256 rows is one tile row, so each weight byte is read
// once per expert. Row quarter q owns row tiles q and q + 4 (rows 32 q .. and
// 128 + 32 q ..); tiles wholly past the expert's end are skipped (the K loop
// is specialised on the wave's count of active tiles, so its MFMA stream has
// no branches). Wave w = 2 q + ch runs on SIMD w % 4, which spreads a short
// tile's active row tiles over the four SIMDs.
//
// Pipeline: two LDS stages and two register stages; global loads run two K
// steps ahead of the MFMAs (the last steps repeat step nk - 1, so the count
// of loads in flight is fixed); one barrier per K step.
//
// MFMA operands: lane L supplies row L % 32 and 8 contraction elements of
// lane group h = L / 32; in a K step lane group h takes MX block h, sub-step
// s its elements 32 h + 8 s .. +8.
// ---------------------------------------------------------------------------
constexpr int TB_BM = 256, TB_BN = 256, TB_BK = 64, TB_THREADS = 512;
constexpr int TB_ALD = TB_BK + 8;  // 72 bf16 = 144 bytes per A row in LDS
constexpr size_t TB_LDS = (size_t)2 * TB_BM * TB_ALD * 2 + (size_t)2 * TB_BN * (TB_BK / 2) +
                          (size_t)2 * TB_BN * (TB_BK / 32);

template <int ACT, typename OutT, bool PACKED, bool LORA>
__global__ __launch_bounds__(TB_THREADS, 1) void gemm_tile256_kernel(
    const bf16 *__restrict__ a, int64_t lda, const int32_t *__restrict__ a_rows,
    const uint8_t *__restrict__ w1c, const uint8_t *__restrict__ w1s,
    const uint8_t *__restrict__ w2c, const uint8_t *__restrict__ w2s,
    const int32_t *__restrict__ plan, int N, int K,
    OutT *__restrict__ out, int64_t ldo, LoraEpi lora)
{
    constexpr bool GLU = ACT != ACT_NONE;
    constexpr int COLS = GLU ? TB_BN / 2 : TB_BN;
    extern __shared__ __attribute__((aligned(16))) uint8_t tb_lds[];
    bf16 (*As)[TB_BM][TB_ALD] = (bf16 (*)[TB_BM][TB_ALD])tb_lds;
    uint8_t (*Bq)[TB_BN][TB_BK / 2] =
        (uint8_t (*)[TB_BN][TB_BK / 2])(tb_lds + (size_t)2 * TB_BM * TB_ALD * 2);
    uint8_t (*Bs)[TB_BN][TB_BK / 32] = (uint8_t (*)[TB_BN][TB_BK / 32])(
        tb_lds + (size_t)2 * TB_BM * TB_ALD * 2 + (size_t)2 * TB_BN * (TB_BK / 2));

    const int nblk = (N + COLS - 1) / COLS;
    const int total = plan[0] * nblk;
    // XCD-aware order (as in the 128-row tiled schedule)
    const int per_xcd = (total + 7) / 8;
    const int local = blockIdx.x / 8;
    const int wi = (blockIdx.x % 8) * per_xcd + local;
    if (local >= per_xcd || wi >= total) return;
    const int grp = wi / nblk, nb = wi - grp * nblk;
    const int2 it = ((const int2 *)(plan + PLAN_HDR))[grp];
    const int e = it.x & 0xffff, r0 = it.y, rend = r0 + (it.x >> 16);
    const int mrows = rend - r0;
    const int n0 = nb * COLS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ch = wave & 1, q = wave >> 1;

    // ---- global -> LDS assignment
    // A: 4 loads per thread, each wave instruction covers 8 whole rows of the
    // K step: row 32 wave + 8 j + lane / 8, 16 bytes at column 8 (lane % 8)
    const int acol = 8 * (lane & 7);
    const bf16 *ag[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int rc = min(r0 + 32 * wave + 8 * j + (lane >> 3), rend - 1);
        const int64_t arow = a_rows ? (int64_t)a_rows[rc] : (int64_t)rc;
        ag[j] = a + arow * lda + acol;
    }
    // B: thread -> weight row tid / 2 of the tile, 16 code bytes (one MX block)
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

    u32x4 ra0[4], ra1[4], rb0, rb1;
    uint8_t rs0, rs1;
    auto gload = [&](u32x4 *ra, u32x4 &rbv, uint8_t &rsv, int kt) {
        const int k0 = kt * TB_BK;
#pragma unroll
        for (int j = 0; j < 4; j++) ra[j] = *(const u32x4 *)(ag[j] + k0);
        if constexpr (PACKED) {
            const int c = kt >> 1, gg = 2 * (kt & 1) + bh;
            rbv = *(const u32x4 *)(bg + c * 1024 + gg * 256);
            rsv = sg[(c >> 2) * 256 + gg * 64 + (c & 3)];
        } else {
            rbv = *(const u32x4 *)(bg + k0 / 2);
            rsv = sg[k0 / 32];
        }
    };
    auto lstore = [&](int st, const u32x4 *ra, const u32x4 &rbv, uint8_t rsv) {
#pragma unroll
        for (int j = 0; j < 4; j++)
            *(u32x4 *)(&As[st][32 * wave + 8 * j + (lane >> 3)][acol]) = ra[j];
        *(u32x4 *)(&Bq[st][br][16 * bh]) = rbv;
        Bs[st][br][bh] = rsv;
    };

    // ---- wave tiles
    const int h = lane >> 5, l32 = lane & 31;
    // weight tiles j = 0..3 of this wave inside the LDS tile
    int bt[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if (GLU) bt[j] = (j >= 2 ? 128 : 0) + 64 * ch + 32 * (j & 1);  // W1 x2, then W2 x2
        else bt[j] = 128 * ch + 32 * j;
    }
    // active row tiles: q (rows 32 q ..) and q + 4 (rows 128 + 32 q ..)
    const int n_on = (32 * q < mrows ? 1 : 0) + (128 + 32 * q < mrows ? 1 : 0);
    const int nk = K / TB_BK;  // even: K is a multiple of 128

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
                u32x4 qd[4];
                float f[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int row = bt[j] + l32;
                    qd[j] = *(const u32x4 *)(&Bq[st][row][16 * h]);
                    f[j] = e8m0_to_f32(Bs[st][row][h]);
                }
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    bf16x8 af[NI];
#pragma unroll
                    for (int i = 0; i < NI; i++)
                        af[i] = *(const bf16x8 *)(&As[st][32 * q + 128 * i + l32][32 * h + 8 * s]);
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const bf16x8 bv = mx_decode8(qd[j][s], f[j]);
#pragma unroll
                        for (int i = 0; i < NI; i++) acc[i][j] = mfma32x32x16(af[i], bv, acc[i][j]);
                    }
                }
            }
        };

        gload(ra0, rb0, rs0, 0);
        gload(ra1, rb1, rs1, 1);
        lstore(0, ra0, rb0, rs0);
        __syncthreads();
        for (int kt = 0; kt < nk; kt += 2) {
            // stage 0 holds step kt; registers set 1 hold step kt + 1
            gload(ra0, rb0, rs0, min(kt + 2, nk - 1));
            __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
            compute(0);
            lstore(1, ra1, rb1, rs1);
            __syncthreads();
            // stage 1 holds step kt + 1; registers set 0 hold step kt + 2
            gload(ra1, rb1, rs1, min(kt + 3, nk - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            lstore(0, ra0, rb0, rs0);  // past the end: a copy of the last step, unused
            __syncthreads();
        }

        if constexpr (LORA) {
            // the low-rank increment: rank / 16 more MFMA steps per tile
#pragma unroll
            for (int i = 0; i < NI; i++) {
                const int64_t trow = min(r0 + 32 * q + 128 * i + l32, rend - 1);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const bool w2 = GLU && j >= 2;
                    const int col = GLU ? n0 + 64 * ch + 32 * (j & 1) + l32
                                        : n0 + 128 * ch + 32 * j + l32;
                    acc[i][j] = lora_add(acc[i][j], w2 ? lora.t2 : lora.t1, trow,
                                         (w2 ? lora.b2 : lora.b1) + (int64_t)e * N * lora.rank,
                                         min(col, N - 1), lora.rank, h);
                }
            }
        }

        // epilogue: lane holds C[8 (v / 4) + 4 h + v % 4][l32] of each tile
#pragma unroll
        for (int i = 0; i < NI; i++) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int rl = 32 * q + 128 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                if (rl >= mrows) continue;
                OutT *orow = out + (int64_t)(r0 + rl) * ldo;
                if constexpr (GLU) {
#pragma unroll
                    for (int jj = 0; jj < 2; jj++) {
                        const int col = n0 + 64 * ch + 32 * jj + l32;
                        if (col < N)
                            store_out<OutT>(orow + col,
                                            act_apply<ACT>(acc[i][jj][v], acc[i][2 + jj][v]));
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int col = n0 + 128 * ch + 32 * j + l32;
                        if (col < N) store_out_once<OutT>(orow + col, acc[i][j][v]);
                    }
                }
            }
        }
    };
    // every branch runs the same barriers (1 + nk)
    switch (__builtin_amdgcn_readfirstlane(n_on)) {
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
    }
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles with direct global -> LDS loads (K <= TD_MAX_K).
//
// Same tile, plan and epilogue as gemm_tile256_kernel, but the A rows and the
// 4-bit codes travel from memory straight into a three-stage LDS ring
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS base
// + 16 * lane), so no register staging and no LDS stores sit in the K loop,
// and the loads of step k + 2 are in flight during the MFMAs of steps k and
// k + 1. One barrier per K step: it publishes step k and frees the stage that
// step k + 2 overwrites (read during step k - 1). The scales of the whole
// tile (256 weight rows x K / 32) go to LDS once, before the loop, in the
// streaming layout's order (16 groups of 16 weight rows).
//
// A rows in LDS: 128 bytes per row, 16-byte chunk c of row r stored at
// chunk position c ^ ((r >> TD_ASWZ) % 8). With TD_ASWZ = 1 the 16 rows that
// one 16-lane group of a 16-byte read touches (two rows per 256 bytes) cover
// all 64 banks. Code rows (32 bytes): the two 16-byte halves of rows 8..15
// of every 16 swap places (TD_BSWZ), for the same reason.
// ---------------------------------------------------------------------------
constexpr int TD_STAGES = 3;
constexpr int TD_A_BYTES = TB_BM * TB_BK * 2;           // 32 KB
constexpr int TD_W_BYTES = TB_BN * TB_BK / 2;           // 8 KB
constexpr int TD_STAGE_BYTES = TD_A_BYTES + TD_W_BYTES;  // 40 KB
constexpr int TD_MAX_K = 4096;
constexpr int TD_ASWZ = 1, TD_BSWZ = 1;

// Scales of 16 weight rows in the streaming layout: K / 512 groups (rounded
// up) of 256 bytes; the tile's LDS table holds 16 of them.
__host__ __device__ constexpr int td_scale_chunk(int K)
{
    return 256 * ((K / 128 + 3) / 4);
}

// the epilogue stages up to 32 rows x (256 + 16) bytes per wave in the same LDS
constexpr int TD_EPI_BYTES = 16 * 32 * (256 + 16);

__host__ __device__ constexpr int td_lds_bytes(int K)
{
    return TD_STAGES * TD_STAGE_BYTES + 16 * td_scale_chunk(K) > TD_EPI_BYTES
               ? TD_STAGES * TD_STAGE_BYTES + 16 * td_scale_chunk(K)
               : TD_EPI_BYTES;
}

// 16 waves (4 per SIMD) share the tile. Wave w takes row block q = w / 4
// (64 rows: two 32-row tiles) and weight slot c = w % 4: for a GLU tile the
// gate and up rows of output columns 32 c .. + 32, otherwise weight rows
// 64 c .. + 64. The four waves that share a SIMD (w % 4 equal) then hold all
// four row blocks of one slot, so every SIMD gets the same share of the
// active row tiles whatever the expert's row count, and four waves per SIMD
// hide each other's LDS and barrier waits. A rows: two DMA instructions per
// wave (rows 16 w .. + 16); codes: one per wave of the first eight.
constexpr int TW_THREADS = 1024;

template <int ACT, typename OutT, bool PACKED, bool LORA>
__global__ __launch_bounds__(TW_THREADS, 1) void gemm_tile256_w16_kernel(
    const bf16 *__restrict__ a, int64_t lda, const int32_t *__restrict__ a_rows,
    const uint8_t *__restrict__ w1c, const uint8_t *__restrict__ w1s,
    const uint8_t *__restrict__ w2c, const uint8_t *__restrict__ w2s,
    const int32_t *__restrict__ plan, int N, int K,
    OutT *__restrict__ out, int64_t ldo, LoraEpi lora)
{
    constexpr bool GLU = ACT != ACT_NONE;
    constexpr int COLS = GLU ? TB_BN / 2 : TB_BN;
    extern __shared__ __attribute__((aligned(16))) uint8_t td_lds[];
    uint8_t *const Ssc = td_lds + TD_STAGES * TD_STAGE_BYTES;  // [16][chunk_b] scales
    const int chunk_b = td_scale_chunk(K);

    const int nblk = (N + COLS - 1) / COLS;
    const int total = plan[0] * nblk;
    const int per_xcd = (total + 7) / 8;
    const int local = blockIdx.x / 8;
    const int wi = (blockIdx.x % 8) * per_xcd + local;
    if (local >= per_xcd || wi >= total) return;
    const int grp = wi / nblk, nb = wi - grp * nblk;
    const int2 it = ((const int2 *)(plan + PLAN_HDR))[grp];
    const int e = it.x & 0xffff, r0 = it.y, rend = r0 + (it.x >> 16);
    const int mrows = rend - r0;
    const int n0 = nb * COLS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = wave & 3, q = wave >> 2;
    const int nch = K / 128;

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

    // ---- DMA sources. A: instruction j of wave w fills rows 16 w + 8 j .. + 7
    // (lane L: chunk position L % 8 of row 16 w + 8 j + L / 8).
    const bf16 *ag[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int rc = min(r0 + 16 * wave + 8 * j + (lane >> 3), rend - 1);
        const int64_t arow = a_rows ? (int64_t)a_rows[rc] : (int64_t)rc;
        ag[j] = a + arow * lda + 8 * ((lane & 7) ^ (((8 * j + (lane >> 3)) >> TD_ASWZ) & 7));
    }
    // codes: threads 0..511 -> LDS weight row tid / 2, half holding MX block bh
    const bool wload = wave < 8;
    const int br = (tid & 511) >> 1, bh = (tid & 1) ^ (TD_BSWZ & (br >> 3));
    const uint8_t *bg;
    {
        const uint8_t *wc, *ws;
        const int64_t wr64 = wsel(br, wc, ws);
        if constexpr (PACKED)
            bg = wc + (wr64 / 16) * nch * 1024 + (wr64 % 16) * 16;
        else
            bg = wc + wr64 * (K / 2) + 16 * bh;
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_address(td_lds));
    auto issue = [&](int kt, int st) {
        const uint32_t sb = lds0 + st * TD_STAGE_BYTES;
#pragma unroll
        for (int j = 0; j < 2; j++) dma16(ag[j] + kt * TB_BK, sb + (2 * wave + j) * 1024);
        if (wload) {
            const uint8_t *src;
            if constexpr (PACKED)
                src = bg + (kt >> 1) * 1024 + (2 * (kt & 1) + bh) * 256;
            else
                src = bg + kt * (TB_BK / 2);
            dma16(src, sb + TD_A_BYTES + wave * 1024);
        }
    };

    const int nk = K / TB_BK;  // even: K is a multiple of 128

    // ---- the tile's scales -> LDS. Group c of 16 LDS weight rows in the
    // streaming layout's order: the scale of k-block kb of its row r is byte
    // (kb % 16) / 4 of the word at (kb / 16) * 256 + (kb % 4) * 64 + (r % 16) * 4.
    // Streaming weights: each group is contiguous in HBM (N is a multiple of
    // 16), so DMA copies, issued before the first stages so that the first
    // barrier's wait covers them; groups past N take the last group's scales
    // (their rows are clamped and their outputs dropped).
    if constexpr (PACKED) {
        for (int m = wave; m < 16 * chunk_b / 1024; m += TW_THREADS / 64) {
            const int b = 1024 * m + 16 * lane;
            const int c = b / chunk_b, off = b - c * chunk_b;
            const int wr0 = min(GLU ? n0 + ((16 * c) & 127) : n0 + 16 * c, N - 16);
            const uint8_t *ws = (GLU && c >= 8) ? w2s : w1s;
            dma16(ws + (((int64_t)e * N + wr0) / 16) * chunk_b + off,
                  lds0 + TD_STAGES * TD_STAGE_BYTES + 1024 * m);
        }
    } else {
        // row-major scales: a word holds k-blocks 4 r .. 4 r + 3 of a row
        const int per_row = K / 128;
        for (int idx = tid; idx < TB_BN * per_row; idx += TW_THREADS) {
            const int row = idx / per_row, r = idx - row * per_row;
            const uint8_t *wc, *ws;
            const int64_t wr64 = wsel(row, wc, ws);
            const uint32_t v = *(const uint32_t *)(ws + wr64 * (K / 32) + 4 * r);
            uint8_t *dst = Ssc + (row / 16) * chunk_b + (r / 4) * 256 + (row % 16) * 4 + (r % 4);
#pragma unroll
            for (int i = 0; i < 4; i++) dst[64 * i] = (uint8_t)(v >> (8 * i));
        }
    }
    issue(0, 0);
    issue(1, 1);

    // ---- wave tiles: weight tiles j = 0, 1 of the slot
    const int h = lane >> 5, l32 = lane & 31;
    int bt[2];
#pragma unroll
    for (int j = 0; j < 2; j++) bt[j] = GLU ? 128 * j + 32 * slot : 64 * slot + 32 * j;
    const int n_on = (64 * q < mrows ? 1 : 0) + (64 * q + 32 < mrows ? 1 : 0);
    const int arow_off = (64 * q + l32) * 128;
    const int akey = (4 * h) ^ ((l32 >> TD_ASWZ) & 7);
    const int bpos = 16 * (h ^ (TD_BSWZ & (l32 >> 3)));
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
                const uint8_t *As = td_lds + st * TD_STAGE_BYTES;
                const uint8_t *Bq = As + TD_A_BYTES;
                u32x4 qd[2];
                float f[2];
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int row = bt[j] + l32;
                    qd[j] = *(const u32x4 *)(Bq + row * 32 + bpos);
                    f[j] = e8m0_to_f32(Ssc[wso[j] + (kt >> 3) * 256 + (kt & 1) * 128 + ((kt & 7) >> 1)]);
                }
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    bf16x8 af[NI];
#pragma unroll
                    for (int i = 0; i < NI; i++)
                        af[i] = *(const bf16x8 *)(As + arow_off + 32 * 128 * i + ((akey ^ s) << 4));
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const bf16x8 bv = mx_decode8(qd[j][s], f[j]);
#pragma unroll
                        for (int i = 0; i < NI; i++) acc[i][j] = mfma32x32x16(af[i], bv, acc[i][j]);
                    }
                }
            }
        };

        for (int kt = 0; kt < nk; kt++) {
            // this wave's loads of step kt are done (those of kt + 1 -- 3 or 2
            // instructions -- may still be in flight); the barrier publishes
            // every wave's and ends the reads of step kt - 1
            if (kt + 1 < nk) {
                if (wload)
                    asm volatile("s_waitcnt vmcnt(3)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(2)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
            const int st = kt % 3;
            if (kt + 2 < nk) issue(kt + 2, st == 0 ? 2 : st - 1);
            compute(st, kt);
        }

        if constexpr (LORA) {
#pragma unroll
            for (int i = 0; i < NI; i++) {
                const int64_t trow = min(r0 + 64 * q + 32 * i + l32, rend - 1);
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const bool w2 = GLU && j == 1;
                    const int col = GLU ? n0 + 32 * slot + l32 : n0 + 64 * slot + 32 * j + l32;
                    acc[i][j] = lora_add(acc[i][j], w2 ? lora.t2 : lora.t1, trow,
                                         (w2 ? lora.b2 : lora.b1) + (int64_t)e * N * lora.rank,
                                         min(col, N - 1), lora.rank, h);
                }
            }
        }

        // epilogue through LDS: the ring is idle once every wave is past its
        // last step, so each wave stages one 32-row tile of its output at a
        // time in a private area (rows of its COLS_W columns, padded by 16
        // bytes) and stores whole 16-byte row segments from there: 2 to 8
        // stores per row tile instead of one narrow store per row pair and
        // accumulator tile. Lane holds C[8 (v / 4) + 4 h + v % 4][l32] of each
        // 32 x 32 accumulator tile.
        __syncthreads();
        constexpr int COLS_W = GLU ? 32 : 64;                 // output columns of the wave
        constexpr int ROW_B = COLS_W * (int)sizeof(OutT);     // 64, 128 or 256 bytes
        constexpr int PITCH = ROW_B + 16;
        constexpr int LPR = ROW_B / 16, RPI = 64 / LPR;       // lanes per row, rows per store
        static_assert(16 * 32 * PITCH <= TD_EPI_BYTES, "staging fits the LDS allocation");
        uint8_t *const stg = td_lds + wave * (32 * PITCH);
        const int c0 = n0 + COLS_W * slot;                    // first output column of the wave
        const bool col_on = c0 < N;                           // N is a multiple of COLS_W
#pragma unroll
        for (int i = 0; i < NI; i++) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int r = 8 * (v >> 2) + 4 * h + (v & 3);
                OutT *row = (OutT *)(stg + r * PITCH);
                if constexpr (GLU) {
                    store_out<OutT>(row + l32, act_apply<ACT>(acc[i][0][v], acc[i][1][v]));
                } else {
#pragma unroll
                    for (int j = 0; j < 2; j++) store_out<OutT>(row + 32 * j + l32, acc[i][j][v]);
                }
            }
#pragma unroll
            for (int it = 0; it < 32 / RPI; it++) {
                const int r = RPI * it + lane / LPR, seg = lane % LPR;
                const u32x4 val = *(const u32x4 *)(stg + r * PITCH + 16 * seg);
                const int rl = 64 * q + 32 * i + r;
                if (col_on && rl < mrows) {
                    u32x4 *dst = (u32x4 *)((uint8_t *)(out + (int64_t)(r0 + rl) * ldo + c0) + 16 * seg);
                    if constexpr (!GLU && sizeof(OutT) == 4) __builtin_nontemporal_store(val, dst);
                    else *dst = val;
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

// Schedule choice from host-known sizes only: the mean rows per local expert
// (max_rows / num_local) and the bound on rows itself. Measured with all 896
// experts (I = 1024) at mean rows 2 to 585:
// - below a mean of 16 the weight-streaming schedule wins (it reads an
//   expert's weights once per 16-row group, so from two groups on the tiled
//   schedules, which read them once per 128 or 256 rows, pull ahead: 1.32 vs
//   1.47 ms at a mean of 14, 1.77 vs 1.48 ms at 18);
// - from 128 to 256 rows a typical expert is one well-filled 256-row tile,
//   and the 256-row schedule is 4-7% faster than the 128-row one (146, 183,
//   219 rows), level at 128 and 256;
// - elsewhere the 128-row schedule (more, smaller tiles) is 2-7% faster,
//   unless the bound is so large (TILE256_MIN_BOUND rows: tens of thousands
//   of tiles) that the last partial wave of workgroups no longer matters and
//   the 256-row tile's weight reuse wins again (long skewed prefill).
constexpr int TILE_MIN_ROWS = 16, TILE256_MIN_MEAN = 128, TILE256_MAX_MEAN = 256;
constexpr int64_t TILE256_MIN_BOUND = (int64_t)1 << 19;

int resolve_mode(int mode, int num_local, int max_rows)
{
    if (mode == MOE_SCHED_STREAM || mode == MOE_SCHED_TILE128 || mode == MOE_SCHED_TILE256)
        return mode;
    const int64_t rows = max_rows, nl = num_local;
    if (mode == 0 && rows < TILE_MIN_ROWS * nl) return MOE_SCHED_STREAM;
    const bool window = rows >= TILE256_MIN_MEAN * nl && rows <= TILE256_MAX_MEAN * nl;
    return window || rows >= TILE256_MIN_BOUND ? MOE_SCHED_TILE256 : MOE_SCHED_TILE128;
}

static int rows_per_group(int md)
{
    return md == MOE_SCHED_TILE256 ? TB_BM : md == MOE_SCHED_TILE128 ? TL_BM : ST_ROWS;
}

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

template <int ACT, typename OutT, bool PACKED>
static hipError_t launch_stream(const bf16 *a, int64_t lda, const int32_t *a_rows,
                                const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                                const uint8_t *w2s, const int32_t *plan,
                                int max_groups, int N, int K, OutT *out, int64_t ldo,
                                const LoraEpi *lora, hipStream_t s)
{
    // one workgroup per (row group, column block); groups past the device-side
    // count exit at once
    constexpr int COLS_B = 4 * stream_cols_per_wave<ACT>();
    const int64_t grid = (int64_t)max_groups * ((N + COLS_B - 1) / COLS_B);
    if (grid <= 0) return hipSuccess;
    // prefetch depth: the largest of ST_DMAX, 2, 1 that divides the chunk count
    const int nch = K / 128;
    const int D = (nch % ST_DMAX == 0) ? ST_DMAX : (nch % 2 == 0 ? 2 : 1);
    const size_t lds = PACKED ? 0 : (size_t)(ACT != ACT_NONE ? 2 : 1) * COLS_B * (K / 32);
    const LoraEpi le = lora ? *lora : LoraEpi{nullptr, nullptr, nullptr, nullptr, 0};
#define ST_LAUNCH(DD, LR)                                                                     \
    hipLaunchKernelGGL((gemm_stream_kernel<ACT, OutT, DD, PACKED, LR>), dim3((unsigned)grid), \
                       dim3(256), lds, s, a, lda, a_rows, w1c, w1s, w2c, w2s, plan, N, K,     \
                       out, ldo, le)
#define ST_LAUNCH_D(LR)          \
    if (D == ST_DMAX)            \
        ST_LAUNCH(ST_DMAX, LR);  \
    else if (D == 2)             \
        ST_LAUNCH(2, LR);        \
    else                         \
        ST_LAUNCH(1, LR)
    if (lora) {
        ST_LAUNCH_D(true);
    } else {
        ST_LAUNCH_D(false);
    }
#undef ST_LAUNCH_D
#undef ST_LAUNCH
    return hipGetLastError();
}

template <int ACT, typename OutT, bool PACKED>
static hipError_t launch_tile(const bf16 *a, int64_t lda, const int32_t *a_rows,
                              const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                              const uint8_t *w2s, const int32_t *plan,
                              int max_groups, int N, int K, OutT *out, int64_t ldo,
                              const LoraEpi *lora, hipStream_t s)
{
    constexpr int COLS = tile_cols<ACT>();
    const int64_t grid = (int64_t)max_groups * ((N + COLS - 1) / COLS);
    if (grid <= 0) return hipSuccess;
    // the XCD-aware order maps block b to work (b % 8) * ceil(total / 8) + b / 8;
    // a grid of 8 * ceil(bound / 8) blocks covers every work item
    const int64_t G = (grid + 7) / 8 * 8;
    const LoraEpi le = lora ? *lora : LoraEpi{nullptr, nullptr, nullptr, nullptr, 0};
    if (lora)
        hipLaunchKernelGGL((gemm_tile_kernel<ACT, OutT, PACKED, true>), dim3((unsigned)G),
                           dim3(TL_THREADS), 0, s, a, lda, a_rows, w1c, w1s, w2c, w2s, plan, N, K,
                           out, ldo, le);
    else
        hipLaunchKernelGGL((gemm_tile_kernel<ACT, OutT, PACKED, false>), dim3((unsigned)G),
                           dim3(TL_THREADS), 0, s, a, lda, a_rows, w1c, w1s, w2c, w2s, plan, N, K,
                           out, ldo, le);
    return hipGetLastError();
}

template <int ACT, typename OutT, bool PACKED>
static hipError_t launch_tile256(const bf16 *a, int64_t lda, const int32_t *a_rows,
                                 const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                                 const uint8_t *w2s, const int32_t *plan,
                                 int max_groups, int N, int K, OutT *out, int64_t ldo,
                                 const LoraEpi *lora, hipStream_t s)
{
    constexpr int COLS = ACT != ACT_NONE ? TB_BN / 2 : TB_BN;
    const int64_t grid = (int64_t)max_groups * ((N + COLS - 1) / COLS);
    if (grid <= 0) return hipSuccess;
    // direct-to-LDS loads while the tile's scales fit beside the three
    // stages; register staging (8 waves) for longer contractions
    using Kern = void (*)(const bf16 *, int64_t, const int32_t *, const uint8_t *,
                          const uint8_t *, const uint8_t *, const uint8_t *, const int32_t *,
                          int, int, OutT *, int64_t, LoraEpi);
    Kern kern = lora ? gemm_tile256_kernel<ACT, OutT, PACKED, true>
                     : gemm_tile256_kernel<ACT, OutT, PACKED, false>;
    size_t lds = TB_LDS;
    unsigned threads = TB_THREADS;
    if (K <= TD_MAX_K) {
        kern = lora ? gemm_tile256_w16_kernel<ACT, OutT, PACKED, true>
                    : gemm_tile256_w16_kernel<ACT, OutT, PACKED, false>;
        threads = TW_THREADS;
        lds = (size_t)td_lds_bytes(K);
    }
    hipError_t err = ensure_dynamic_lds((const void *)kern, (int)lds);
    if (err != hipSuccess) return err;
    const int64_t G = (grid + 7) / 8 * 8;
    const LoraEpi le = lora ? *lora : LoraEpi{nullptr, nullptr, nullptr, nullptr, 0};
    hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(threads), lds, s, a, lda, a_rows, w1c, w1s,
                       w2c, w2s, plan, N, K, out, ldo, le);
    return hipGetLastError();
}

template <typename OutT, bool PACKED>
static hipError_t dispatch_act(int act, int md, const bf16 *a, int64_t lda, const int32_t *a_rows,
                               const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                               const uint8_t *w2s, const int32_t *plan,
                               int max_groups, int N, int K, OutT *out, int64_t ldo,
                               const LoraEpi *lora, hipStream_t s)
{
    // the LoRA increment inside the GEMMs takes ranks that are multiples of 16
    if (lora && (lora->rank % 16 || lora->rank < 16 || lora->rank > 64)) return hipErrorInvalidValue;
#define MOE_GEMM_ARGS a, lda, a_rows, w1c, w1s, w2c, w2s, plan, max_groups, N, K, out, ldo
#define MOE_GEMM_CASE(A)                                                                   \
    case A:                                                                                \
        return md == MOE_SCHED_TILE256   ? launch_tile256<A, OutT, PACKED>(MOE_GEMM_ARGS, lora, s) \
               : md == MOE_SCHED_TILE128 ? launch_tile<A, OutT, PACKED>(MOE_GEMM_ARGS, lora, s)    \
                                         : launch_stream<A, OutT, PACKED>(MOE_GEMM_ARGS, lora, s);
    switch (act) {
        MOE_GEMM_CASE(ACT_NONE)
        MOE_GEMM_CASE(ACT_SILU_MUL)
        MOE_GEMM_CASE(ACT_GELU_TANH_MUL)
    default:
        return hipErrorInvalidValue;
    }
#undef MOE_GEMM_CASE
#undef MOE_GEMM_ARGS
}

GemmPlanArgs gemm_plan_args(int num_local, int max_rows, int mode, void *ws)
{
    const int md = resolve_mode(mode, num_local, max_rows);
    const int R = rows_per_group(md);
    return GemmPlanArgs{(int32_t *)ws, R, max_groups_for(num_local, max_rows, R), PLAN_HDR,
                        md == MOE_SCHED_TILE256};
}

hipError_t launch_gemm_plan_into(const int32_t *off, int num_local, const GemmPlanArgs &a,
                                 hipStream_t s)
{
    hipLaunchKernelGGL(gemm_plan_kernel, dim3(1), dim3(1024), 0, s, off, num_local,
                       a.rows_per_group, a.max_groups, a.balanced, a.plan);
    return hipGetLastError();
}

hipError_t launch_gemm_plan(const int32_t *off, int num_local, int max_rows, int mode, void *ws,
                            hipStream_t s)
{
    return launch_gemm_plan_into(off, num_local, gemm_plan_args(num_local, max_rows, mode, ws), s);
}

hipError_t launch_gemm_run(const bf16 *a, int64_t lda, const int32_t *a_rows, const uint8_t *w1c,
                           const uint8_t *w1s, const uint8_t *w2c, const uint8_t *w2s,
                           int num_local, int max_rows, int N, int K, int act,
                           void *out, int out_f32, int64_t ldo, int mode, const void *plan_ws,
                           int packed, hipStream_t s, const LoraEpi *lora)
{
    const int md = resolve_mode(mode, num_local, max_rows);
    const int max_groups = max_groups_for(num_local, max_rows, rows_per_group(md));
    const int32_t *plan = (const int32_t *)plan_ws;
#define MOE_RUN(OT, PK)                                                                    \
    return dispatch_act<OT, PK>(act, md, a, lda, a_rows, w1c, w1s, w2c, w2s, plan,         \
                                max_groups, N, K, (OT *)out, ldo, lora, s)
    if (out_f32) {
        if (packed) MOE_RUN(float, true);
        MOE_RUN(float, false);
    }
    if (packed) MOE_RUN(bf16, true);
    MOE_RUN(bf16, false);
#undef MOE_RUN
}

hipError_t launch_grouped_gemm(const bf16 *a, int64_t lda, const int32_t *a_rows,
                               const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                               const uint8_t *w2s, const int32_t *off, int num_local,
                               int max_rows, int N, int K, int act, void *out, int out_f32,
                               int64_t ldo, int mode, void *ws, int packed, hipStream_t s)
{
    hipError_t e = launch_gemm_plan(off, num_local, max_rows, mode, ws, s);
    if (e != hipSuccess) return e;
    return launch_gemm_run(a, lda, a_rows, w1c, w1s, w2c, w2s, num_local, max_rows, N, K,
                           act, out, out_f32, ldo, mode, ws, packed, s);
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
