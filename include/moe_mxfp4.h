/*
 * moe_mxfp4.h -- C ABI of a single-GPU LatentMoE layer with MXFP4 expert
 * weights for AMD Instinct MI355X (gfx950).
 *
 * The layer, as the sources describe it:
 *   P1  "从Kimi K3到MiniMax-H3：国产大模型竞争进入“推理系统战”", section 一: tokens
 *       are routed and computed in a 3584-wide latent space, 896 experts with
 *       16 active per token, with a K3-specific activation path; section
 *       二/第一层: weights ship as MXFP4 (4-bit elements sharing a scale per
 *       block) and meet higher-precision activations in the kernels.
 *   P2  "SGLang 0.5.17：Kimi K3 原生 MXFP4 推理架构解析", section "MoE 稀疏激活":
 *       a router scores every token against every expert, the top 16 are
 *       kept, and their outputs are summed with weights; section "MXFP4 原生
 *       支持": per-block scales and dequantisation fused into the GEMM.
 *   P3  "Kimi K3 Day-0 适配剖析:KDA/Gated MLA 混合注意力、MXFP4 在线量化与 896
 *       专家 MoE", section 四: dispatch -> expert compute -> combine, with
 *       dispatch's index computation and buffer planning re-done for 896
 *       experts / top-16.
 *   OCP-MX  OCP Microscaling Formats (MX) v1.0: E2M1 elements, one E8M0 scale
 *       per 32 consecutive elements.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers named as device arrays point to device memory (HBM) owned by
 *    the caller; the library never keeps them after the call returns and never
 *    allocates or frees device memory. Scratch memory comes in through `ws`
 *    (device, 256-byte aligned, at least the queried size).
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream) and return; nothing synchronises the host.
 *  - Argument checks run on the host before any HIP call and return
 *    MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE without
 *    touching the device. A failed launch returns MOE_ERR_HIP and the HIP
 *    message is kept per thread (moe_last_error()). T == 0 is a no-op.
 *  - bf16 arrays are passed as void* (16-bit payloads). Row starts of bf16
 *    activation rows must be 16-byte aligned (row strides multiple of 8).
 *  - Determinism: no floating-point atomics; two calls on the same inputs give
 *    bitwise-equal outputs.
 *
 * MXFP4 weight layout (one matrix [N, K], K the contraction dim): codes
 * [N][K/2] bytes, element 2i in bits 0-3 and element 2i+1 in bits 4-7 of
 * byte i; scales [N][K/32] bytes (E8M0: value 2^(s-127) for 0 <= s <= 254;
 * s = 255 is NaN and is a precondition violation). Element value =
 * E2M1(code) * 2^(s-127), decoded exactly for every finite scale code: s <= 1
 * gives bf16 subnormals, which decode and multiply exactly; s = 253 and 254
 * overflow to +-inf for the codes whose value exceeds the bf16 range, as the
 * same value does in fp32 (the quantiser never emits s > 252). Experts are stacked: [num_local][N][...]; code and
 * scale arrays start 16-byte aligned.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *moe_stream_t; /* hipStream_t */

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* a size out of range or a required pointer NULL */
    MOE_ERR_UNSUPPORTED = 2, /* a valid request the library does not handle    */
    MOE_ERR_WORKSPACE = 3,   /* ws smaller than the queried size, or misaligned */
    MOE_ERR_HIP = 4          /* a HIP runtime call or launch failed              */
};

enum moe_dtype {
    MOE_DT_BF16 = 0,
    MOE_DT_F32 = 1,
    MOE_DT_MXFP8 = 2, /* moe_grouped_gemm_mx8 output only */
    MOE_DT_FP6X2 = 3  /* moe_grouped_gemm_fp6x2 output only: split records */
};

/* Elementwise stage between the two expert projections. P1 (section 一)
 * names a K3-specific activation path without defining it, so the stage is
 * selectable: SILU_MUL = silu(gate) * up (default), GELU_TANH_MUL =
 * gelu_tanh(gate) * up, NONE = plain GEMM output (no second weight). */
enum moe_act { MOE_ACT_NONE = 0, MOE_ACT_SILU_MUL = 1, MOE_ACT_GELU_TANH_MUL = 2 };

/* Storage layout of MXFP4 expert weights. OCP: the canonical row-major
 * layout described above. PACKED: the streaming layout moe_mxfp4_prepack
 * produces (same codes and scales, permuted for the kernels). */
enum moe_weight_layout { MOE_LAYOUT_OCP = 0, MOE_LAYOUT_PACKED = 1 };
enum moe_precision { MOE_PREC_BF16 = 0, MOE_PREC_MX8 = 1, MOE_PREC_FP6X2 = 2 };

/* Schedules of the grouped expert GEMMs (the `mode` argument). All give the
 * same results up to fp32 summation order; they differ in how work is cut:
 *   STREAM:   groups of 16 rows, each weight streamed once per group
 *             (few rows per expert: decode)
 *   TILE128:  128-row x 256-weight-row tiles, two workgroups per CU
 *   TILE256:  256-row x 256-weight-row tiles, an expert's rows cut into
 *             nearly equal groups (an expert of up to 256 rows reads its
 *             weights once)
 *   TILED:    TILE256 when 128 <= max_rows / num_local <= 256 or
 *             max_rows >= 2^19, else TILE128
 *   AUTO:     STREAM when max_rows / num_local < 16, else TILED */
enum moe_sched {
    MOE_SCHED_AUTO = 0,
    MOE_SCHED_STREAM = 1,
    MOE_SCHED_TILED = 2,
    MOE_SCHED_TILE128 = 3,
    MOE_SCHED_TILE256 = 4
};

/* Limits of the library. */
#define MOE_MX_BLOCK 32
#define MOE_MAX_TOPK 32
#define MOE_MAX_EXPERTS 2048
#define MOE_MAX_K 8192 /* contraction length of one expert projection (d and I) */

/* ------------------------------------------------------------------------
 * moe_route -- router scores, top-k select, softmax over the selected scores,
 * expert histogram (P2 "MoE 稀疏激活": score every expert, keep the best 16,
 * weight their outputs).
 *
 *   x        [T][d] bf16          latent tokens
 *   w_router [E][d] fp32          router weights
 *   bias     [E] fp32 or NULL     added to every token's scores
 *   logits   [T][E] fp32          if logits_given: read (replayed scores);
 *                                 else written: logits[t][e] =
 *                                 sum_i x[t][i]*w_router[e][i] + bias[e]
 *                                 (fp32 accumulation; each product exact)
 *   topk_idx [T][k] int32 (out)   best expert first; a larger score wins, an
 *                                 equal score goes to the lower index, -0 == +0
 *   topk_w   [T][k] fp32 (out)    w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 *   expert_counts [E] int32 (out) assignments per expert over all T*k
 * Preconditions: finite scores. Errors: k < 1, k > E, NULL required pointer
 * -> INVALID_ARG; k > 32, E > 2048 or (scores computed) d % 128 != 0 ->
 * UNSUPPORTED. With T == 0 only expert_counts is written (zeros).
 * ------------------------------------------------------------------------ */
int moe_route(const void *x, const float *w_router, const float *bias, float *logits,
              int logits_given, int T, int d, int E, int k, int32_t *topk_idx, float *topk_w,
              int32_t *expert_counts, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_permute -- dispatch planning (P3 section 四: index computation and
 * buffer planning): offsets of each local expert's rows and a stable counting
 * sort of the row-major (t, j) assignment list by expert.
 *
 *   topk_idx [T][k] int32, expert_counts [E] int32  (from moe_route; or
 *            NULL: each local expert's rows are then counted from topk_idx,
 *            with no atomics, which suits heavily skewed routing; above 256
 *            tokens they are counted from topk_idx either way, which gives
 *            the same offsets for a histogram of topk_idx)
 *   local experts are ids [expert_begin, expert_begin + num_local)
 *   expert_offsets [num_local + 1] int32 (out): off[0] = 0,
 *                  off[i+1] = off[i] + expert_counts[expert_begin + i]
 *   perm_token [T*k] int32 (out): rows off[i]..off[i+1]-1 hold the tokens
 *                  routed to local expert i in increasing token order; entries
 *                  at and after off[num_local] are left untouched
 *   inv [T][k] int32 (out): the row of assignment (t, j), or -1 if its
 *                  expert is not local (dropped)
 *   ws / ws_bytes: scratch of moe_permute_workspace_size(T, num_local) bytes
 * ------------------------------------------------------------------------ */
size_t moe_permute_workspace_size(int T, int num_local);
int moe_permute(const int32_t *topk_idx, const int32_t *expert_counts, int T, int k, int E,
                int expert_begin, int num_local, int32_t *expert_offsets, int32_t *perm_token,
                int32_t *inv, void *ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_mxfp4_quantize -- fp32 -> MXFP4 on the device, for weights converted
 * online at load time (P3 section 三: MXFP4 online quantisation at load;
 * OCP-MX: E2M1 elements, one E8M0 scale per 32 elements).
 *   w [N][K] fp32 (device, 16-byte aligned) -> codes [N][K/2], scales
 *   [N][K/32] in the canonical layout (codes 16-byte aligned).
 * Per 32-element block: amax = max|v|; all zero -> scale code 0, codes 0;
 * else s = clamp(floor(log2 amax) - 2 + 127, 0, 254) and each element is
 * v / 2^(s-127) rounded to the nearest E2M1 value (ties to the even code,
 * magnitudes above 6 saturate to 6), sign bit from v (-0 keeps it).
 * Preconditions: finite w. Errors: K % 32 != 0 -> UNSUPPORTED; NULL or
 * misaligned pointers -> INVALID_ARG. N == 0 or K == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int moe_mxfp4_quantize(const float *w, int64_t N, int K, uint8_t *codes, uint8_t *scales,
                       moe_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_mxfp4_dequant -- decode an MXFP4 matrix to bf16 (OCP-MX element value
 * E2M1(code) * 2^(s-127), exact in bf16 for every scale code 0..254:
 * subnormal results for codes 0 and 1 included, +-inf where the value
 * overflows for codes 253 and 254).
 *   codes [N][K/2], scales [N][K/32] -> out [N][K] bf16
 * ------------------------------------------------------------------------ */
int moe_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t N, int K, void *out,
                      moe_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_mxfp4_prepack -- load-time conversion of MXFP4 weights into the
 * streaming layout (P3 section 三: the MXFP4 checkpoint is converted layer by
 * layer at load into a form the hardware runs efficiently, no offline copy).
 * A byte permutation: values are unchanged. For n_mats stacked [N][K]
 * matrices (N % 16 == 0, K % 128 == 0), with nch = K/128, nc4 = ceil(nch/4),
 * per matrix:
 *   packed codes  [N/16][nch][4][16][16 bytes]: row block, 128-wide chunk,
 *       MX block g of the chunk, row m of the block, the 16 code bytes of
 *       row 16 rb + m, block 4 c + g  (N*K/2 bytes, as the input)
 *   packed scales [N/16][nc4][4][16][4]: the scale of row 16 rb + m, block
 *       4 (4 c4 + cc) + g at byte cc; 0 past the last chunk
 *       (moe_mxfp4_packed_scale_bytes(N, K) bytes; = N*K/32 when K % 512 == 0)
 * Inputs and outputs are device arrays that must not overlap.
 * ------------------------------------------------------------------------ */
size_t moe_mxfp4_packed_scale_bytes(int N, int K);
int moe_mxfp4_prepack(const uint8_t *codes, const uint8_t *scales, int n_mats, int N, int K,
                      uint8_t *packed_codes, uint8_t *packed_scales, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_grouped_gemm_mxfp4 -- one grouped expert projection with MXFP4 weights
 * dequantised in registers and fed to bf16 matrix cores with fp32
 * accumulation (P2 "MXFP4 原生支持": dequantisation fused into the GEMM).
 *
 * For local expert e and each row r in [off[e], off[e+1]):
 *   a_row  = a + (a_rows ? a_rows[r] : r) * lda          (bf16, K elements)
 *   acc1[n] = sum_k a_row[k] * W1[e][n][k],  n < N
 *   act == MOE_ACT_NONE:  out[r][n] = acc1[n]                     (w2 NULL)
 *   otherwise:            out[r][n] = act(acc1[n], acc2[n]), acc2 from W2
 *   out + r * ldo, dtype out_dtype (bf16 rounding is to nearest even)
 *
 *   w1_codes/w1_scales, w2_codes/w2_scales: [num_local][N][K/2], [..][K/32]
 *         in layout w_layout (MOE_LAYOUT_PACKED: each expert's arrays as
 *         moe_mxfp4_prepack lays them out, experts stacked)
 *   expert_offsets [num_local + 1] int32 on the device
 *   max_rows: a host-side upper bound on off[num_local] (e.g. T*k); it sizes
 *             the launch, rows beyond off[num_local] are never touched
 *   mode: enum moe_sched (0 = choose from max_rows / num_local)
 *   ws / ws_bytes: scratch of moe_grouped_gemm_workspace_size(...) bytes (the
 *         device-built work list)
 * Requirements: lda >= K and ldo >= N, both multiples of 8; a_rows entries
 * index valid rows of `a`; a, out, code and scale arrays 16-byte aligned.
 * Errors: block_size != 32, K % 128 != 0, N % 64 != 0 or K > MOE_MAX_K ->
 * UNSUPPORTED;
 * a GLU act without w2, or w2 with MOE_ACT_NONE -> INVALID_ARG.
 * ------------------------------------------------------------------------ */
size_t moe_grouped_gemm_workspace_size(int num_local, int max_rows, int N, int mode);
/* The schedule `mode` resolves to for these sizes (MOE_SCHED_STREAM,
 * MOE_SCHED_TILE128 or MOE_SCHED_TILE256), or -1 for invalid arguments. */
int moe_grouped_gemm_schedule(int num_local, int max_rows, int mode);
int moe_grouped_gemm_mxfp4(const void *a, int64_t lda, const int32_t *a_rows,
                           const uint8_t *w1_codes, const uint8_t *w1_scales,
                           const uint8_t *w2_codes, const uint8_t *w2_scales,
                           const int32_t *expert_offsets, int num_local, int max_rows, int N,
                           int K, int block_size, int w_layout, int act, void *out,
                           int out_dtype, int64_t ldo, int mode, void *ws, size_t ws_bytes,
                           moe_stream_t stream);

/* ------------------------------------------------------------------------
 * The block-scaled precision mode (MX8). The pages' layer pairs 4-bit weights
 * with higher-precision activations (P1 section 二, 第一层); this mode instead
 * rounds the activations to MXFP8 so that both operands and their scales go
 * to the gfx950 block-scaled matrix instruction as stored (8-bit rate, no
 * decode). It is a separate accuracy contract, defined with OCP-MX v1.0
 * formats: E4M3 elements (bias 7, largest magnitude 448), one E8M0 scale per
 * 32 elements along the contraction.
 * ------------------------------------------------------------------------ */

/* moe_mxfp8_quantize -- rows of v (bf16 or fp32, row stride ldv elements) to
 * MXFP8: codes [N][K] (one E4M3 byte per element), scales [N][K/32].
 * Per 32-element block: amax = max|v|; all zero -> scale code 0, codes 0;
 * else s = clamp(floor(log2 amax) - 8 + 127, 0, 254), and each element is
 * v / 2^(s-127) rounded to the nearest E4M3 value (ties to the even code),
 * magnitudes from 448 up clamped to 448, sign bit from v (-0 keeps it).
 * Preconditions: finite v. Errors: K % 32 != 0 -> UNSUPPORTED; v_dtype not
 * a moe_dtype, ldv < K, ldv % 8 != 0, NULL or misaligned (16-byte) pointers
 * -> INVALID_ARG. N == 0 is a no-op. */
int moe_mxfp8_quantize(const void *v, int v_dtype, int64_t ldv, int64_t N, int K,
                       uint8_t *codes, uint8_t *scales, moe_stream_t stream);

/* moe_grouped_gemm_mx8 -- moe_grouped_gemm_mxfp4 with MXFP8 rows:
 *   a_row  = (a_rows ? a_rows[r] : r)
 *   acc1[n] = sum_k A(a_row, k) * W1[e][n][k], A(r, k) = E4M3(a_codes[r *
 *             lda + k]) * 2^(a_scales[r * (lda/32) + k/32] - 127)
 * on the block-scaled matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4
 * on the tiled schedules, v_mfma_scale_f32_16x16x128_f8f6f4 on the streaming
 * one; exact products; each 64- or 128-long partial sum is formed inside the
 * instruction, then accumulated in fp32); out as in moe_grouped_gemm_mxfp4,
 * or with out_dtype MOE_DT_MXFP8 the fp32 results converted as
 * moe_mxfp8_quantize does (blocks of 32 along N): codes to out [rows][ldo]
 * (bytes), scales to out_scales [rows][ldo/32] (NULL for the other dtypes).
 * mode: MOE_SCHED_STREAM streams the weights once per 16 rows (fp32 or bf16
 * output; with MOE_DT_MXFP8 -> UNSUPPORTED); MOE_SCHED_TILE128 and
 * MOE_SCHED_TILE256 give 128- and 256-row tiles; MOE_SCHED_TILED takes
 * 128-row tiles below a mean of 128 rows per local expert, else 256-row
 * tiles; MOE_SCHED_AUTO streams below a mean of 16 (except for MXFP8
 * output), else as TILED. ws holds
 * moe_grouped_gemm_mx8_workspace_size(...) bytes.
 * Requirements: lda >= K, lda % 32 == 0, ldo >= N, ldo % 8 == 0 (% 32 for
 * MXFP8 output); 16-byte aligned code and scale arrays. Errors as
 * moe_grouped_gemm_mxfp4. */
size_t moe_grouped_gemm_mx8_workspace_size(int num_local, int max_rows);
int moe_grouped_gemm_mx8(const uint8_t *a_codes, const uint8_t *a_scales, int64_t lda,
                         const int32_t *a_rows, const uint8_t *w1_codes,
                         const uint8_t *w1_scales, const uint8_t *w2_codes,
                         const uint8_t *w2_scales, const int32_t *expert_offsets, int num_local,
                         int max_rows, int N, int K, int block_size, int w_layout, int act,
                         void *out, int out_dtype, uint8_t *out_scales, int64_t ldo, int mode,
                         void *ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * The FP6X2 carriage of activations. The pages' layer pairs 4-bit weights
 * with higher-precision activations (P1 section 二, 第一层). gfx950's
 * block-scaled matrix instruction takes 6-bit x 4-bit operands at twice its
 * 8-bit rate, so activations go to it as two MXFP6 planes (OCP-MX v1.0 E2M3
 * elements: bias 1, largest magnitude 7.5; one E8M0 scale per 32 elements
 * along the contraction): plane 1 is the MXFP6 conversion of the value,
 * plane 2 that of the fp32 residual. The planes carry each value to within
 * 2^(E-7), E = floor(log2 amax) of its block; layers that use them keep the
 * default accuracy contract.
 * ------------------------------------------------------------------------ */

/* moe_fp6x2_split -- rows of v (bf16 or fp32, row stride ldv elements) as two
 * MXFP6 planes. Per 32-element block b of row n and plane p (plane 1 from v,
 * plane 2 from r = v - decode(plane 1) in fp32): amax = max|.|; all zero ->
 * scale code 0, codes 0; else s = clamp(floor(log2 amax) - 2 + 127, 0, 254),
 * and each element is ./2^(s-127) rounded to the nearest E2M3 value (ties to
 * the even code), magnitudes from 7.5 up clamped to 7.5, sign bit from the
 * element (-0 keeps it, code 0x20).
 * Output row n at out + 2 n ldo bytes (ldo in elements: a split row of K
 * elements takes the 2 K bytes of a bf16 row), one 128-byte record per 64
 * elements (blocks 2s and 2s+1):
 *   bytes   0..47  block 2s: plane-1 codes (24 bytes), plane-2 codes (24)
 *   bytes  48..51  scale codes (2s, plane 1), (2s, plane 2), (2s+1, plane 1),
 *                  (2s+1, plane 2); bytes 52..63 three more copies of them
 *   bytes  64..111 block 2s+1: plane-1 codes, plane-2 codes
 *   bytes 112..127 zero
 * with code i of a plane at bits 6i..6i+5 of its 24 little-endian bytes.
 * Preconditions: finite v. Errors: K % 64 != 0 -> UNSUPPORTED; v_dtype not
 * bf16 or fp32, ldv < K, ldv % 8 != 0, ldo < K, ldo % 64 != 0, NULL or
 * misaligned (16-byte v, 128-byte out) pointers -> INVALID_ARG. N == 0 is a
 * no-op. */
int moe_fp6x2_split(const void *v, int v_dtype, int64_t ldv, int64_t N, int K, uint8_t *out,
                    int64_t ldo, moe_stream_t stream);

/* moe_grouped_gemm_fp6x2 -- moe_grouped_gemm_mxfp4 with rows carried as two
 * MXFP6 planes:
 *   a_row  = (a_rows ? a_rows[r] : r)
 *   acc1[n] = sum_k A(a_row, k) * W1[e][n][k], A(r, k) = the plane-1 value
 *             plus the plane-2 value of element k of split row r
 * with split rows as moe_fp6x2_split writes them (row r at a + 2 r lda
 * bytes; lda in elements), on v_mfma_scale_f32_32x32x64_f8f6f4 (exact
 * products; each 64-long partial sum formed inside the instruction, one per
 * plane, then accumulated in fp32); out as in moe_grouped_gemm_mxfp4, or with
 * out_dtype MOE_DT_FP6X2 (act != NONE) the fp32 results written as
 * moe_fp6x2_split writes a row of N elements (row r at out + 2 r ldo bytes;
 * ldo % 64 == 0, 128-byte aligned out): the next projection's input.
 * Schedule: 256-row tiles (no mode argument). ws holds
 * moe_grouped_gemm_fp6x2_workspace_size(...) bytes. Requirements: lda >= K,
 * lda % 64 == 0, 128-byte aligned a, ldo >= N, ldo % 8 == 0, 16-byte aligned
 * weight and output arrays. Errors as moe_grouped_gemm_mxfp4, and K > 4096 ->
 * UNSUPPORTED. */
size_t moe_grouped_gemm_fp6x2_workspace_size(int num_local, int max_rows);
int moe_grouped_gemm_fp6x2(const uint8_t *a, int64_t lda, const int32_t *a_rows,
                           const uint8_t *w1_codes, const uint8_t *w1_scales,
                           const uint8_t *w2_codes, const uint8_t *w2_scales,
                           const int32_t *expert_offsets, int num_local, int max_rows, int N,
                           int K, int block_size, int w_layout, int act, void *out,
                           int out_dtype, int64_t ldo, void *ws, size_t ws_bytes,
                           moe_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_combine -- weighted unpermute (P3 section 四, combine: results come back
 * weighted; P2 "MoE 稀疏激活": weighted sum of the selected experts):
 *   out[t][m] = sum_{j=0..k-1, inv[t][j] >= 0} topk_w[t][j] * y[inv[t][j]][m]
 * summed in j order in fp32; a token with no local assignment gets zeros.
 *   y [rows][d] (y_dtype, row stride ldy), out [T][d] (out_dtype, stride ldo)
 * ------------------------------------------------------------------------ */
int moe_combine(const void *y, int y_dtype, int64_t ldy, const int32_t *inv,
                const float *topk_w, int T, int d, int k, void *out, int out_dtype, int64_t ldo,
                moe_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_layer -- the whole layer in one call: route -> permute -> gate/up
 * projection with activation -> down projection -> combine, enqueued as
 * kernels on `stream` with no host synchronisation. Router scores are
 * moe_route's, except that batches of 512 tokens or more multiply the tokens
 * by the router weights rounded to 16 significant bits (two bf16 parts, each
 * weight within 2^-17 of itself), within 1e-4 max(1, |score|) of the exact
 * scores on the workloads.
 * ------------------------------------------------------------------------ */
typedef struct {
    int T;            /* tokens                                   */
    int d;            /* latent width (3584 for the K3 layer)     */
    int E;            /* routed experts (896)                     */
    int k;            /* experts per token (16)                   */
    int I;            /* expert intermediate width                */
    int block_size;   /* MX block size, must be 32                */
    int expert_begin; /* first local expert id                    */
    int num_local;    /* local experts computed; others dropped   */
    int act;          /* enum moe_act, MOE_ACT_SILU_MUL default   */
    int out_dtype;    /* enum moe_dtype of `out`                  */
    int mode;         /* GEMM schedule, as moe_grouped_gemm_mxfp4 */
    int weight_layout; /* enum moe_weight_layout of all six weight arrays */
    int precision;    /* enum moe_precision: MOE_PREC_BF16 (the pages' bf16
                         activations), MOE_PREC_MX8 (tokens and h rounded to
                         MXFP8 before each projection; `mode` as in
                         moe_grouped_gemm_mx8) or MOE_PREC_FP6X2 (with mode
                         TILE256 or TILE128, or AUTO / TILED at a mean of at
                         least 128 rows per local expert over T k, and d, I
                         <= 4096, both projections take their activations --
                         the tokens, and h from its fp32 value -- as two MXFP6
                         planes, moe_grouped_gemm_fp6x2, on 256- or 128-row
                         tiles: TILE256 / TILE128 fix the tile, AUTO / TILED
                         choose it per projection, and the output does not
                         depend on it; otherwise the bf16 path) */
} moe_layer_params;

/* Scratch bytes moe_layer needs for these parameters (0 if invalid). */
size_t moe_layer_workspace_size(const moe_layer_params *p);

/*   gate/up codes [num_local][I][d/2], scales [num_local][I][d/32]
 *   down codes    [num_local][d][I/2], scales [num_local][d][I/32]
 *   out [T][d] (p->out_dtype)
 *   logits_out [T][E] f32, topk_idx_out / topk_w_out [T][k]: optional copies
 *   of the routing (NULL to skip)
 *   stage_events: NULL, or 6 hipEvent_t recorded on `stream` before the
 *   route, permute, gate/up, down and combine stages and after the last one
 *   (for per-stage timing). */
int moe_layer(const moe_layer_params *p, const void *x, const float *w_router, const float *bias,
              const uint8_t *gate_codes, const uint8_t *gate_scales, const uint8_t *up_codes,
              const uint8_t *up_scales, const uint8_t *down_codes, const uint8_t *down_scales,
              void *out, float *logits_out, int32_t *topk_idx_out, float *topk_w_out, void *ws,
              size_t ws_bytes, void **stage_events, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * moe_layer_noalloc -- moe_layer for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. It takes no workspace: its scratch is a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends (its address is looked up once per device,
 * on the first call with that device current). It calls no hipMalloc,
 * hipFree or allocating routine; the caller still owns x, the weights, out
 * and the optional routing copies, as for moe_layer.
 *
 * Arguments, layouts and results are moe_layer's (no workspace, no stage
 * events); the kernels and their results are the same. The scratch used is
 * the current device's (hipGetDevice): `stream` must belong to that device.
 * Every call on one GPU shares its scratch, so calls that overlap on one GPU
 * (two streams, two threads) race: serialise them. Nothing is carried from
 * one call to the next: each call writes every scratch word it reads.
 *
 * Errors: as moe_layer; parameters whose moe_layer_workspace_size exceeds
 * MOE_NOALLOC_SCRATCH_BYTES -> MOE_ERR_WORKSPACE before any HIP call, with
 * the sizes in moe_last_error() (64 MiB holds, for example, the 64-token
 * decode batch at d = 3584, 896 experts, top-16, I = 1024: 18 MB).
 * ------------------------------------------------------------------------ */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_noalloc(const moe_layer_params *p, const void *x, const float *w_router,
                      const float *bias, const uint8_t *gate_codes, const uint8_t *gate_scales,
                      const uint8_t *up_codes, const uint8_t *up_scales,
                      const uint8_t *down_codes, const uint8_t *down_scales, void *out,
                      float *logits_out, int32_t *topk_idx_out, float *topk_w_out,
                      moe_stream_t stream);

/* ------------------------------------------------------------------------
 * LoRA on the MXFP4 base (P1 section 二, 第五层: the large quantised base
 * stays frozen and a low-rank increment is trained on top of it).
 * ------------------------------------------------------------------------ */
#define MOE_MAX_LORA_RANK 64

/* moe_grouped_lora -- the increment of one grouped projection, added to its
 * fp32 output. For local expert e and each row r in [off[e], off[e+1]):
 *   t[j]    = scale * sum_k x_row(r)[k] * A_e[j][k]     (j < rank)
 *   y[r][n] += sum_j t[j] * B_e[n][j]                    (n < N)
 * x_row(r) = x + (x_rows ? x_rows[r] : r) * ldx (bf16, K elements);
 * lora_a [num_local][rank][K], lora_b [num_local][N][rank] bf16; y fp32
 * [rows][ldy]; fp32 accumulation. ws holds
 * moe_grouped_lora_workspace_size(max_rows, rank) bytes (the rank factors).
 * Errors: rank outside 1..MOE_MAX_LORA_RANK, K % 8 != 0 or N % 4 != 0 ->
 * UNSUPPORTED; ldx < K or not a multiple of 8, ldy < N or not a multiple of
 * 4, NULL or misaligned (16-byte x, lora_a, y) pointers -> INVALID_ARG. */
size_t moe_grouped_lora_workspace_size(int max_rows, int rank);
int moe_grouped_lora(const void *x, int64_t ldx, const int32_t *x_rows, const void *lora_a,
                     const void *lora_b, int rank, float scale, const int32_t *expert_offsets,
                     int num_local, int max_rows, int N, int K, float *y, int64_t ldy, void *ws,
                     size_t ws_bytes, moe_stream_t stream);

/* Adapters of every local expert's three projections (bf16, device):
 *   gate_a, up_a [num_local][rank][d]   gate_b, up_b [num_local][I][rank]
 *   down_a [num_local][rank][I]         down_b [num_local][d][rank]
 * Each projection becomes W v + scale * B (A v). */
typedef struct {
    int rank;
    float scale;
    const void *gate_a, *gate_b, *up_a, *up_b, *down_a, *down_b;
} moe_lora_adapters;

/* moe_layer_lora -- moe_layer with the adapters applied (bf16 precision
 * only). The increment must land before the activation. With a rank that
 * is a multiple of 16 it is added inside the grouped GEMMs (every schedule),
 * from fp32 rank factors carried as an exact hi + lo pair of bf16 parts;
 * otherwise the gate and up projections run unfused (fp32 outputs, the
 * increments, then the activation). Workspace:
 * moe_layer_lora_workspace_size(p, rank) bytes (0 if
 * invalid). Errors as moe_layer, plus a NULL lora or adapter, or an adapter
 * not 16-byte aligned -> INVALID_ARG, rank outside 1..MOE_MAX_LORA_RANK or
 * the MX8 precision -> UNSUPPORTED. */
size_t moe_layer_lora_workspace_size(const moe_layer_params *p, int rank);
int moe_layer_lora(const moe_layer_params *p, const moe_lora_adapters *lora, const void *x,
                   const float *w_router, const float *bias, const uint8_t *gate_codes,
                   const uint8_t *gate_scales, const uint8_t *up_codes, const uint8_t *up_scales,
                   const uint8_t *down_codes, const uint8_t *down_scales, void *out,
                   float *logits_out, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                   size_t ws_bytes, void **stage_events, moe_stream_t stream);

/* Static text for a status code. */
const char *moe_status_string(int status);
/* The calling thread's last error message: the last HIP error, or the size
 * message of moe_layer_noalloc ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MXFP4_H */
