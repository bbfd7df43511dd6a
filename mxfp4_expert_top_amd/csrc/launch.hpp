// Internal launchers of the gfx950 kernels (host side). Every launcher
// enqueues on `s` and returns the launch status; arguments are assumed
// validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_mxfp4.h"

#define MOE_MAX_EXPERTS_DEV 2048
#define MOE_MAX_TOPK_DEV 32

typedef __bf16 bf16;

namespace moe {

// Raise a kernel's dynamic LDS limit to `bytes` on the current device, once
// per (kernel, device); thread-safe (api.hip).
hipError_t ensure_dynamic_lds(const void *kernel, int bytes);

// route.hip
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);
// Router scores into `splits` planes of [T][E] partial sums (splits == 1:
// the final scores, bias included); splits must divide d / 128.
// zero_counts: an [E] histogram zeroed by the launch (NULL: none).
hipError_t launch_router_logits(const bf16 *x, const float *w, const float *bias, float *logits,
                                int T, int d, int E, int splits, int32_t *zero_counts,
                                hipStream_t s);
// Small batches (T <= ROUTER_SKINNY_MAX_T): weight-streaming router into
// `splits` planes (splits == 1: final scores, bias included); splits must
// divide d / 128.
constexpr int ROUTER_SKINNY_MAX_T = 64;
int router_skinny_splits(int T, int d, int E, int target_blocks);
hipError_t launch_router_skinny(const bf16 *x, const float *w, const float *bias, float *out,
                                int T, int d, int E, int splits, int32_t *zero_counts,
                                hipStream_t s);
// Larger batches: fp32 router weights -> two bf16 planes [2][E][d] (hi and
// mid, 16 significant bits), then a tiled bf16 GEMM over K' = 2 d into
// `splits` planes of [T][E].
hipError_t launch_split_router(const float *w, int E, int d, bf16 *wp, hipStream_t s);
int router_tile_splits(int T, int d, int E, int target_blocks);
hipError_t launch_router_tile(const bf16 *x, const bf16 *wp, const float *bias, float *logits,
                              int T, int d, int E, int splits, int32_t *zero_counts,
                              hipStream_t s);
// Batches at or above this many tokens use the tiled router.
constexpr int ROUTER_TILE_MIN_T = 512;
// K splits that give the router about `target_blocks` workgroups.
int router_splits(int T, int d, int E, int target_blocks);
// Top-k, softmax weights and (counts != NULL) histogram by integer atomics.
// src holds n_planes planes [T][E];
// with n_planes > 1 the scores are plane 0 + plane 1 + ... (in that order)
// + bias, and are written to `logits`; with one plane src is the final scores
// (bias and logits unused).
hipError_t launch_topk_softmax(const float *src, int n_planes, const float *bias, float *logits,
                               int T, int E, int k, int32_t *idx, float *w, int32_t *counts,
                               hipStream_t s);

// permute.hip
// Tokens per permutation block (one bitmap of local experts x tokens in LDS).
constexpr int PERM_TB = 256;
inline int perm_blocks(int T) { return (T + PERM_TB - 1) / PERM_TB; }
size_t permute_ws_bytes(int T, int num_local);
// Where a grouped-GEMM work plan goes and how it is cut (see gemm.hip).
struct GemmPlanArgs {
    int32_t *plan;
    int rows_per_group;
    int max_groups;
    int hdr;
    int balanced;  // nearly equal groups instead of rows_per_group-row groups
};
// Offsets, permutation and inverse; with `plan` also the GEMM work plan
// (built inside the same kernel for small T). counts: the expert histogram,
// or NULL to count from the dispatch bitmaps (no atomics anywhere).
hipError_t launch_permute(const int32_t *idx, const int32_t *counts, int T, int k, int e0,
                          int num_local, int32_t *off, int32_t *perm, int32_t *inv, void *ws,
                          hipStream_t s, const GemmPlanArgs *plan = nullptr);

// LoRA increment of a tiled projection, added to its accumulators before the
// epilogue: t1 / t2 are the bf16 rank factors [rows][rank] (scale applied) of
// the W1 / W2 projection, b1 / b2 the B factors [experts][N][rank]; rank is a
// multiple of 16 (rank / 16 extra 32 x 32 x 16 MFMA steps per tile).
struct LoraEpi {
    const bf16 *t1, *t2, *b1, *b2;
    int rank;
};

// gemm.hip
// Work items of the grouped GEMMs: (expert, first row) groups of `rows`
// consecutive permuted rows, built on the device from the expert offsets.
size_t gemm_plan_ws_bytes(int num_local, int max_rows, int rows_per_group);
hipError_t launch_grouped_gemm(const bf16 *a, int64_t lda, const int32_t *a_rows,
                               const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                               const uint8_t *w2s, const int32_t *off, int num_local,
                               int max_rows, int N, int K, int act, void *out, int out_f32,
                               int64_t ldo, int mode, void *ws, int packed, hipStream_t s);
size_t grouped_gemm_ws_bytes(int num_local, int max_rows, int N, int mode);
GemmPlanArgs gemm_plan_args(int num_local, int max_rows, int mode, void *ws);
hipError_t launch_gemm_plan_into(const int32_t *off, int num_local, const GemmPlanArgs &a,
                                 hipStream_t s);
// The two halves of launch_grouped_gemm: build the work plan into `ws`, then
// run the GEMM from a plan built for the same (offsets, max_rows, mode).
hipError_t launch_gemm_plan(const int32_t *off, int num_local, int max_rows, int mode, void *ws,
                            hipStream_t s);
// lora: the low-rank increment added before the epilogue (tiled schedules
// only: hipErrorInvalidValue for the streaming one)
hipError_t launch_gemm_run(const bf16 *a, int64_t lda, const int32_t *a_rows, const uint8_t *w1c,
                           const uint8_t *w1s, const uint8_t *w2c, const uint8_t *w2s,
                           int num_local, int max_rows, int N, int K, int act,
                           void *out, int out_f32, int64_t ldo, int mode, const void *plan_ws,
                           int packed, hipStream_t s, const LoraEpi *lora = nullptr);
int resolve_mode(int mode, int num_local, int max_rows);

hipError_t launch_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t N, int K,
                                bf16 *out, hipStream_t s);

// mx8.hip: the block-scaled precision mode (MXFP8 activations x MXFP4
// weights on v_mfma_scale_f32_32x32x64_f8f6f4)
hipError_t launch_mxfp8_quantize(const void *v, int v_f32, int64_t ldv, int64_t N, int K,
                                 uint8_t *codes, uint8_t *scales, hipStream_t s,
                                 const int32_t *n_dev = nullptr);
size_t mx8_gemm_ws_bytes(int num_local, int max_rows);
// MOE_SCHED_TILE128 or MOE_SCHED_TILE256 for a requested mode (AUTO / TILED
// choose as the bf16 tiled schedules do)
int mx8_resolve_mode(int mode, int num_local, int max_rows, bool q_out = false);
GemmPlanArgs mx8_plan_args(int num_local, int max_rows, int mode, void *ws, bool q_out = false);
// A: codes [rows][lda] bytes, scales [rows][lda / 32]. Output kinds: bf16,
// fp32, or MXFP8 (codes in out [rows][ldo], scales in out_scales [rows][ldo/32]).
// MX8_OUT_Q16: block-int16 rows as launch_gemm_fp6x2_run's F6_OUT_Q16 writes
// them (int16 [rows][ldo], one exponent code per 32 columns in out_scales),
// no activation, where mx8_q16_ok (the 16-wave 256-row tile) holds.
enum { MX8_OUT_BF16 = 0, MX8_OUT_F32 = 1, MX8_OUT_MXFP8 = 2, MX8_OUT_Q16 = 3 };
bool mx8_q16_ok(int mode, int num_local, int max_rows, int K);
hipError_t launch_gemm_mx8_run(const uint8_t *ac, const uint8_t *as, int64_t lda,
                               const int32_t *a_rows, const uint8_t *w1c, const uint8_t *w1s,
                               const uint8_t *w2c, const uint8_t *w2s, int num_local,
                               int max_rows, int N, int K, int act, void *out, int out_kind,
                               uint8_t *out_scales, int64_t ldo, int mode, void *plan_ws,
                               int packed, hipStream_t s);
hipError_t launch_grouped_gemm_mx8(const uint8_t *ac, const uint8_t *as, int64_t lda,
                                   const int32_t *a_rows, const uint8_t *w1c, const uint8_t *w1s,
                                   const uint8_t *w2c, const uint8_t *w2s, const int32_t *off,
                                   int num_local, int max_rows, int N, int K, int act, void *out,
                                   int out_kind, uint8_t *out_scales, int64_t ldo, int mode,
                                   void *ws, int packed, hipStream_t s);

// fp6x2.hip: activations as two MXFP6 (E2M3) planes against MXFP4 weights on
// v_mfma_scale_f32_32x32x64_f8f6f4 (6-bit x 4-bit rate). A split row of K
// elements is 2 K bytes: one 128-byte record (both blocks' planes and scales)
// per 64 elements; lda = the row stride in elements (2 lda bytes).
hipError_t launch_fp6x2_split(const void *v, int v_f32, int64_t ldv, int64_t N, int K,
                              uint8_t *out, int64_t ldo, hipStream_t s,
                              const int32_t *n_dev = nullptr);
// The 256-row tile from a 256-row work plan (MOE_SCHED_TILE256) already built
// in plan_ws, or with rows128 the 128-row tile (two workgroups per CU) from a
// 128-row plan (MOE_SCHED_TILE128; records and block-int16 outputs only);
// K % 128 == 0, K <= 4096 (hipErrorInvalidValue otherwise). Each output
// element is the same either way.
// Output kinds: bf16 or fp32 rows [rows][ldo]; (GLU only) split records of
// the fp32 results, row r at out + 2 r ldo bytes, as launch_fp6x2_split
// writes them; (no activation only) block-int16 rows: int16 [rows][ldo] and
// one exponent code per 32 columns in out_scales [rows][ldo / 32], the value
// of q under code e being q 2^(e - 126) / 32767 (ldo % 32 == 0). Non-finite
// results are not carried: an infinity saturates, a NaN comes out finite.
enum { F6_OUT_BF16 = 0, F6_OUT_F32 = 1, F6_OUT_RECORDS = 2, F6_OUT_Q16 = 3 };
hipError_t launch_gemm_fp6x2_run(const uint8_t *ad, int64_t lda, const int32_t *a_rows,
                                 const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                                 const uint8_t *w2s, int num_local, int max_rows, int N, int K,
                                 int act, void *out, int out_kind, int64_t ldo,
                                 const void *plan_ws, int packed, hipStream_t s,
                                 uint8_t *out_scales = nullptr, int rows128 = 0);
hipError_t launch_grouped_gemm_fp6x2(const uint8_t *ad, int64_t lda, const int32_t *a_rows,
                                     const uint8_t *w1c, const uint8_t *w1s, const uint8_t *w2c,
                                     const uint8_t *w2s, const int32_t *off, int num_local,
                                     int max_rows, int N, int K, int act, void *out,
                                     int out_kind, int64_t ldo, void *ws, int packed,
                                     hipStream_t s);

// lora.hip: the low-rank increment on a frozen projection (y += t B_e^T with
// t = scale x A_e^T, rows grouped by expert); t is [max_rows][rank] fp32
size_t lora_ws_bytes(int max_rows, int rank);
// the rank factors alone: t [max_rows][rank], fp32 or (t_bf16) bf16
hipError_t launch_lora_t(const bf16 *x, int64_t ldx, const int32_t *x_rows, const bf16 *la,
                         int rank, float scale, const int32_t *off, int nl, int max_rows, int K,
                         void *t, int t_bf16, hipStream_t s);
// the rank factors (bf16) on the matrix cores, along the tiled GEMM work plan
// `plan` (already built): t1 = scale x A1_e^T and, if a2, t2 = scale x A2_e^T;
// rank % 16 == 0, K % 64 == 0, plan rows per group a multiple of 32, <= 256
hipError_t launch_lora_t_plan(const bf16 *x, int64_t ldx, const int32_t *x_rows, const bf16 *a1,
                              const bf16 *a2, int rank, int K, float scale,
                              const GemmPlanArgs &plan, bf16 *t1, bf16 *t2, hipStream_t s);
hipError_t launch_lora(const bf16 *x, int64_t ldx, const int32_t *x_rows, const bf16 *la,
                       const bf16 *lb, int rank, float scale, const int32_t *off, int nl,
                       int max_rows, int N, int K, float *y, int64_t ldy, float *t,
                       hipStream_t s);
// h = act(g, u) over the first off[nl] rows of [*, I] fp32 arrays, bf16 out
hipError_t launch_glu(const float *g, const float *u, const int32_t *off, int nl, int max_rows,
                      int I, int act, bf16 *h, hipStream_t s);

// prepack.hip: the streaming weight layout (see prepack.hip) and the fp32 ->
// MXFP4 quantiser (canonical layout out)
hipError_t launch_mxfp4_quantize(const float *w, int64_t N, int K, uint8_t *codes,
                                 uint8_t *scales, hipStream_t s);
size_t packed_scale_bytes(int64_t N, int K);
hipError_t launch_prepack(const uint8_t *codes, const uint8_t *scales, int64_t n_rows, int K,
                          uint8_t *pcodes, uint8_t *pscales, hipStream_t s);

// combine.hip
// The combine over block-int16 expert outputs (F6_OUT_Q16: yq [rows][ldy],
// ys [rows][ldy / 32]); same sum, order and output as launch_combine.
hipError_t launch_combine_q16(const int16_t *yq, const uint8_t *ys, int64_t ldy,
                              const int32_t *inv, const float *w, int T, int d, int k,
                              void *out, int out_f32, int64_t ldo, hipStream_t s);
hipError_t launch_combine(const void *y, int y_f32, int64_t ldy, const int32_t *inv,
                          const float *w, int T, int d, int k, void *out, int out_f32,
                          int64_t ldo, hipStream_t s);

}  // namespace moe
