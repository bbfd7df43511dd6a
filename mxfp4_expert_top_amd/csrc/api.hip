// C ABI of the MXFP4 LatentMoE layer: argument checks (on the host, before
// any HIP call), workspace carving and the launch sequence. Declarations and
// the contract of every entry point are in include/moe_mxfp4.h.
#include <string>

#include "moe_mxfp4.h"
#include "launch.hpp"

#include <cmath>
#include <mutex>
#include <set>
#include <utility>

using namespace moe;

// Scratch of moe_layer_noalloc, for callers that cannot allocate: a device
// array of MOE_NOALLOC_SCRATCH_BYTES, one copy per GPU the library runs on,
// held until the process ends. Calls on one GPU share it.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int hip_fail(hipError_t e)
{
    g_last_error = hipGetErrorString(e);
    return MOE_ERR_HIP;
}

#define HIP_TRY(expr)                                   \
    do {                                                \
        hipError_t e_ = (expr);                         \
        if (e_ != hipSuccess) return hip_fail(e_);      \
    } while (0)

#define CHECK(cond, code)          \
    do {                           \
        if (!(cond)) return (code); \
    } while (0)

inline hipStream_t as_stream(moe_stream_t s) { return (hipStream_t)s; }

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t round_up(size_t n) { return (n + 255) & ~(size_t)255; }

int check_route(const void *x, const float *w_router, const float *logits, int logits_given,
                int T, int d, int E, int k, const int32_t *idx, const float *w,
                const int32_t *counts)
{
    CHECK(T >= 0 && E >= 1 && k >= 1 && k <= E, MOE_ERR_INVALID_ARG);
    CHECK(counts, MOE_ERR_INVALID_ARG);
    CHECK(k <= MOE_MAX_TOPK && E <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED);
    if (T == 0) return MOE_OK;
    CHECK(logits && idx && w, MOE_ERR_INVALID_ARG);
    if (!logits_given) {
        CHECK(x && w_router && d >= 1, MOE_ERR_INVALID_ARG);
        CHECK(d % 128 == 0, MOE_ERR_UNSUPPORTED);
        CHECK(aligned(x, 16) && aligned(w_router, 16), MOE_ERR_INVALID_ARG);
    }
    return MOE_OK;
}

int check_permute(const int32_t *idx, const int32_t *counts, int T, int k, int E, int e0, int nl,
                  const int32_t *off, const int32_t *perm, const int32_t *inv)
{
    CHECK(T >= 0 && k >= 1 && k <= E && E >= 1, MOE_ERR_INVALID_ARG);
    CHECK(e0 >= 0 && nl >= 1 && e0 + nl <= E, MOE_ERR_INVALID_ARG);
    CHECK(k <= MOE_MAX_TOPK && E <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED);
    CHECK(off, MOE_ERR_INVALID_ARG);  // counts may be NULL: taken from idx
    if (T > 0) CHECK(idx && perm && inv, MOE_ERR_INVALID_ARG);
    return MOE_OK;
}

int check_gemm(const void *a, int64_t lda, const uint8_t *w1c, const uint8_t *w1s,
               const uint8_t *w2c, const uint8_t *w2s, const int32_t *off, int nl, int max_rows,
               int N, int K, int block_size, int w_layout, int act, const void *out,
               int out_dtype, int64_t ldo)
{
    CHECK(w_layout == MOE_LAYOUT_OCP || w_layout == MOE_LAYOUT_PACKED, MOE_ERR_INVALID_ARG);
    CHECK(nl >= 1 && max_rows >= 0 && N >= 1 && K >= 1, MOE_ERR_INVALID_ARG);
    CHECK(act == MOE_ACT_NONE || act == MOE_ACT_SILU_MUL || act == MOE_ACT_GELU_TANH_MUL,
          MOE_ERR_INVALID_ARG);
    CHECK(out_dtype == MOE_DT_BF16 || out_dtype == MOE_DT_F32, MOE_ERR_INVALID_ARG);
    CHECK(block_size == MOE_MX_BLOCK, MOE_ERR_UNSUPPORTED);
    CHECK(K % 128 == 0 && N % 64 == 0 && K <= MOE_MAX_K, MOE_ERR_UNSUPPORTED);
    if (act == MOE_ACT_NONE)
        CHECK(!w2c && !w2s, MOE_ERR_INVALID_ARG);
    else
        CHECK(w2c && w2s, MOE_ERR_INVALID_ARG);
    if (max_rows == 0) return MOE_OK;
    CHECK(a && w1c && w1s && off && out, MOE_ERR_INVALID_ARG);
    CHECK(lda >= K && lda % 8 == 0 && ldo >= N && ldo % 8 == 0, MOE_ERR_INVALID_ARG);
    CHECK(aligned(a, 16) && aligned(w1c, 16) && aligned(w1s, 16) && aligned(out, 16),
          MOE_ERR_INVALID_ARG);
    if (w2c) CHECK(aligned(w2c, 16) && aligned(w2s, 16), MOE_ERR_INVALID_ARG);
    return MOE_OK;
}

int check_ws(const void *ws, size_t ws_bytes, size_t need)
{
    if (need == 0) return MOE_OK;
    CHECK(ws && ws_bytes >= need && aligned(ws, 256), MOE_ERR_WORKSPACE);
    return MOE_OK;
}

// Workspace layout of moe_layer; every region 256-byte aligned.
struct LayerWs {
    size_t logits, planes, wsplit, idx, w, off, perm, inv, pws, gws, h, y, total;
    size_t xq, xs, hq, hs;  // MX8 mode: MXFP8 tokens and h (codes, scales)
    size_t xf, hf;          // FP6X2: the tokens' and h's two MXFP6 planes
    bool f6;                // the FP6X2 gate/up projection runs
    bool gu128, dn128;      // FP6X2 projections on 128-row tiles (gate/up, down)
    size_t gws2;            // the down projection's own work plan (tiles differ)
    int splits;
    int router;  // ROUTER_SKINNY, ROUTER_SMALL or ROUTER_TILED
};
enum { ROUTER_SKINNY = 0, ROUTER_SMALL = 1, ROUTER_TILED = 2 };

static int router_kind(int T, int d)
{
    if (T <= ROUTER_SKINNY_MAX_T) return ROUTER_SKINNY;
    return T >= ROUTER_TILE_MIN_T && d % 64 == 0 ? ROUTER_TILED : ROUTER_SMALL;
}

// The FP6X2 precision runs on 256- or 128-row tiles. It takes them when asked
// to (MOE_SCHED_TILE256 or TILE128: both projections on those tiles) or, with
// the schedule left to the library (AUTO or TILED), from a mean of 128 rows
// per local expert over the row bound T k: EP share (16384 x 16 rows over 112
// experts, 24175 local) 1.03 ms against 1.09 ms on the bf16 path's 128-row
// tiles. Below that, and for the streaming schedule, the layer runs the bf16
// path.
static bool fp6x2_layer(const moe_layer_params *p)
{
    if (p->precision != MOE_PREC_FP6X2 || p->d > 4096 || p->I > 4096) return false;
    if (p->mode == MOE_SCHED_TILE256 || p->mode == MOE_SCHED_TILE128) return true;
    if (p->mode != MOE_SCHED_AUTO && p->mode != MOE_SCHED_TILED) return false;
    return (int64_t)p->T * p->k >= 128 * (int64_t)p->num_local;
}

// FP6X2 tiles per projection under AUTO / TILED. The 128-row tile lets two
// workgroups share a CU, so one's prologue, epilogue and launch overlap the
// other's K loop; it costs a second read of an expert's weights for each extra
// row tile. Measured (ms, 256-row -> 128-row tiles):
//   down, I = 1024: prefill 0.944 -> 0.895, EP share 0.180 -> 0.150. Taken
//     whenever I <= 1024 (three stages still fit two workgroups per CU);
//   gate/up: EP share 0.291 -> 0.257, but prefill 1.405 -> 1.598 (146-row
//     experts become a 128-row and an 18-row tile, each streaming the
//     weights) and long skewed 18.70 -> 18.71-18.83. Taken when the 256-row
//     grid, estimated from the expected local rows T k num_local / E under
//     uniform routing, gives fewer than 16 workgroups per CU (256 CUs): there
//     the finer grid also shortens the tail.
static void fp6x2_tiles(const moe_layer_params *p, bool *gu128, bool *dn128)
{
    if (p->mode == MOE_SCHED_TILE256 || p->mode == MOE_SCHED_TILE128) {
        *gu128 = *dn128 = p->mode == MOE_SCHED_TILE128;
        return;
    }
    // expected rows per local expert under uniform routing: T k / E
    const double per_expert = (double)p->T * p->k / p->E;
    const double wg = (double)p->num_local * std::ceil(per_expert / 256.0) * ((p->I + 127) / 128);
    *gu128 = wg < 16.0 * 256.0;
    *dn128 = p->I <= 1024;
}

LayerWs layer_ws(const moe_layer_params *p)
{
    LayerWs L{};
    const size_t T = (size_t)p->T, E = (size_t)p->E, k = (size_t)p->k;
    const size_t A = T * k;
    size_t o = 0;
    L.router = router_kind(p->T, p->d);
    L.splits = L.router == ROUTER_TILED   ? router_tile_splits(p->T, p->d, p->E, 256)
               : L.router == ROUTER_SMALL ? router_splits(p->T, p->d, p->E, 512)
                                          : router_skinny_splits(p->T, p->d, p->E, 256);
    L.logits = o; o += round_up(T * E * 4);
    L.planes = o; o += L.splits > 1 ? round_up((size_t)L.splits * T * E * 4) : 0;
    L.wsplit = o; o += L.router == ROUTER_TILED ? round_up(2 * E * (size_t)p->d * 2) : 0;
    L.idx = o;    o += round_up(A * 4);
    L.w = o;      o += round_up(A * 4);
    L.off = o;    o += round_up(((size_t)p->num_local + 1) * 4);
    L.perm = o;   o += round_up(A * 4);
    L.inv = o;    o += round_up(A * 4);
    L.pws = o;    o += round_up(permute_ws_bytes(p->T, p->num_local));
    L.gws = o;
    const bool mx8 = p->precision == MOE_PREC_MX8;
    L.f6 = fp6x2_layer(p);
    if (L.f6) fp6x2_tiles(p, &L.gu128, &L.dn128);
    o += round_up(mx8  ? mx8_gemm_ws_bytes(p->num_local, (int)A)
                  : L.f6 ? grouped_gemm_ws_bytes(p->num_local, (int)A, p->I,
                                                 L.gu128 ? MOE_SCHED_TILE128 : MOE_SCHED_TILE256)
                         : grouped_gemm_ws_bytes(p->num_local, (int)A, p->I, p->mode));
    L.gws2 = o;
    if (L.f6 && L.gu128 != L.dn128)
        o += round_up(grouped_gemm_ws_bytes(p->num_local, (int)A, p->d,
                                            L.dn128 ? MOE_SCHED_TILE128 : MOE_SCHED_TILE256));
    // h: bf16 for the bf16 down projection; in the MX8 mode fp32, quantised
    // from there to MXFP8 (hq, hs)
    L.h = o;      o += round_up(A * (size_t)p->I * (mx8 ? 4 : 2));
    if (L.f6) {
        L.xf = o;  o += round_up(T * (size_t)p->d * 2);
        L.hf = o;  o += round_up(A * (size_t)p->I * 2);
    }
    if (mx8) {
        L.xq = o; o += round_up(T * (size_t)p->d);
        L.xs = o; o += round_up(T * (size_t)(p->d / 32));
        L.hq = o; o += round_up(A * (size_t)p->I);
        L.hs = o; o += round_up(A * (size_t)(p->I / 32));
    }
    // fp32 expert outputs: bf16 here would spend most of the max-abs error
    // budget of the layer (measured 3.05e-2 rms against the 3e-2 bound). The
    // FP6X2 layer, and the MX8 mode on the 256-row tile, keep them as
    // block-int16 rows in the same space (A d int16, then A d / 32 scale codes)
    L.y = o;      o += round_up(A * (size_t)p->d * 4);
    L.total = o;
    return L;
}

// Router scores, top-k and softmax of the layer. With split-K planes the
// top-k kernel adds them in a fixed order, then the bias. No expert histogram:
// the permute kernels count each expert's rows from their dispatch bitmaps (a
// histogram of skewed routing would serialise atomics on the hot experts).
hipError_t layer_route(const moe_layer_params *p, const LayerWs &L, char *base, const void *x,
                       const float *w_router, const float *bias, float *logits, int32_t *idx,
                       float *w, hipStream_t s)
{
    float *planes = L.splits > 1 ? (float *)(base + L.planes) : logits;
    const float *b_in_gemm = L.splits > 1 ? nullptr : bias;
    hipError_t e;
    if (L.router == ROUTER_TILED) {
        bf16 *wp = (bf16 *)(base + L.wsplit);
        e = launch_split_router(w_router, p->E, p->d, wp, s);
        if (e != hipSuccess) return e;
        e = launch_router_tile((const bf16 *)x, wp, b_in_gemm, planes, p->T, p->d, p->E,
                               L.splits, nullptr, s);
    } else if (L.router == ROUTER_SMALL) {
        e = launch_router_logits((const bf16 *)x, w_router, b_in_gemm, planes, p->T, p->d, p->E,
                                 L.splits, nullptr, s);
    } else {
        e = launch_router_skinny((const bf16 *)x, w_router, b_in_gemm, planes, p->T, p->d, p->E,
                                 L.splits, nullptr, s);
    }
    if (e != hipSuccess) return e;
    return launch_topk_softmax(planes, L.splits, bias, logits, p->T, p->E, p->k, idx, w, nullptr,
                               s);
}

int check_layer_params(const moe_layer_params *p)
{
    CHECK(p, MOE_ERR_INVALID_ARG);
    CHECK(p->T >= 0 && p->d >= 1 && p->E >= 1 && p->k >= 1 && p->k <= p->E && p->I >= 1,
          MOE_ERR_INVALID_ARG);
    CHECK(p->expert_begin >= 0 && p->num_local >= 1 && p->expert_begin + p->num_local <= p->E,
          MOE_ERR_INVALID_ARG);
    CHECK(p->act == MOE_ACT_SILU_MUL || p->act == MOE_ACT_GELU_TANH_MUL, MOE_ERR_INVALID_ARG);
    CHECK(p->out_dtype == MOE_DT_BF16 || p->out_dtype == MOE_DT_F32, MOE_ERR_INVALID_ARG);
    CHECK(p->mode >= MOE_SCHED_AUTO && p->mode <= MOE_SCHED_TILE256, MOE_ERR_INVALID_ARG);
    CHECK(p->weight_layout == MOE_LAYOUT_OCP || p->weight_layout == MOE_LAYOUT_PACKED,
          MOE_ERR_INVALID_ARG);
    CHECK(p->precision == MOE_PREC_BF16 || p->precision == MOE_PREC_MX8 ||
              p->precision == MOE_PREC_FP6X2,
          MOE_ERR_INVALID_ARG);
    // the MX8 mode has the two tiled schedules only
    CHECK(p->block_size == MOE_MX_BLOCK, MOE_ERR_UNSUPPORTED);
    CHECK(p->k <= MOE_MAX_TOPK && p->E <= MOE_MAX_EXPERTS, MOE_ERR_UNSUPPORTED);
    CHECK(p->d % 128 == 0 && p->I % 128 == 0, MOE_ERR_UNSUPPORTED);
    CHECK(p->d <= MOE_MAX_K && p->I <= MOE_MAX_K, MOE_ERR_UNSUPPORTED);
    CHECK((int64_t)p->T * p->k <= INT32_MAX / 2, MOE_ERR_UNSUPPORTED);
    return MOE_OK;
}

}  // namespace

namespace moe {

hipError_t ensure_dynamic_lds(const void *kernel, int bytes)
{
    static std::mutex mu;
    static std::set<std::pair<const void *, int>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({kernel, dev})) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.insert({kernel, dev});
    return e;
}

}  // namespace moe

extern "C" {

const char *moe_status_string(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported by the library";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

int moe_route(const void *x, const float *w_router, const float *bias, float *logits,
              int logits_given, int T, int d, int E, int k, int32_t *topk_idx, float *topk_w,
              int32_t *expert_counts, moe_stream_t stream)
{
    int rc = check_route(x, w_router, logits, logits_given, T, d, E, k, topk_idx, topk_w,
                         expert_counts);
    if (rc) return rc;
    hipStream_t s = as_stream(stream);
    if (T == 0 || logits_given) HIP_TRY(launch_fill_i32(expert_counts, E, 0, s));
    if (T == 0) return MOE_OK;
    if (!logits_given) {
        if (router_kind(T, d) == ROUTER_SKINNY)
            HIP_TRY(launch_router_skinny((const bf16 *)x, w_router, bias, logits, T, d, E, 1,
                                         expert_counts, s));
        else
            HIP_TRY(launch_router_logits((const bf16 *)x, w_router, bias, logits, T, d, E, 1,
                                         expert_counts, s));
    }
    HIP_TRY(launch_topk_softmax(logits, 1, nullptr, logits, T, E, k, topk_idx, topk_w,
                                expert_counts, s));
    return MOE_OK;
}

size_t moe_permute_workspace_size(int T, int num_local)
{
    if (T < 0 || num_local < 1) return 0;
    return permute_ws_bytes(T, num_local);
}

int moe_permute(const int32_t *topk_idx, const int32_t *expert_counts, int T, int k, int E,
                int expert_begin, int num_local, int32_t *expert_offsets, int32_t *perm_token,
                int32_t *inv, void *ws, size_t ws_bytes, moe_stream_t stream)
{
    int rc = check_permute(topk_idx, expert_counts, T, k, E, expert_begin, num_local,
                           expert_offsets, perm_token, inv);
    if (rc) return rc;
    rc = check_ws(ws, ws_bytes, permute_ws_bytes(T, num_local));
    if (rc) return rc;
    HIP_TRY(launch_permute(topk_idx, expert_counts, T, k, expert_begin, num_local, expert_offsets,
                           perm_token, inv, ws, as_stream(stream)));
    return MOE_OK;
}

int moe_mxfp4_quantize(const float *w, int64_t N, int K, uint8_t *codes, uint8_t *scales,
                       moe_stream_t stream)
{
    CHECK(N >= 0 && K >= 0, MOE_ERR_INVALID_ARG);
    CHECK(K % 32 == 0, MOE_ERR_UNSUPPORTED);
    if (N == 0 || K == 0) return MOE_OK;
    CHECK(w && codes && scales, MOE_ERR_INVALID_ARG);
    CHECK(aligned(w, 16) && aligned(codes, 16), MOE_ERR_INVALID_ARG);
    HIP_TRY(launch_mxfp4_quantize(w, N, K, codes, scales, as_stream(stream)));
    return MOE_OK;
}

int moe_mxfp8_quantize(const void *v, int v_dtype, int64_t ldv, int64_t N, int K,
                       uint8_t *codes, uint8_t *scales, moe_stream_t stream)
{
    CHECK(N >= 0 && K >= 0, MOE_ERR_INVALID_ARG);
    CHECK(v_dtype == MOE_DT_BF16 || v_dtype == MOE_DT_F32, MOE_ERR_INVALID_ARG);
    CHECK(K % 32 == 0, MOE_ERR_UNSUPPORTED);
    if (N == 0 || K == 0) return MOE_OK;
    CHECK(v && codes && scales, MOE_ERR_INVALID_ARG);
    CHECK(ldv >= K && ldv % 8 == 0, MOE_ERR_INVALID_ARG);
    CHECK(aligned(v, 16) && aligned(codes, 16), MOE_ERR_INVALID_ARG);
    HIP_TRY(launch_mxfp8_quantize(v, v_dtype == MOE_DT_F32, ldv, N, K, codes, scales,
                                  as_stream(stream)));
    return MOE_OK;
}

int moe_fp6x2_split(const void *v, int v_dtype, int64_t ldv, int64_t N, int K, uint8_t *out,
                    int64_t ldo, moe_stream_t stream)
{
    CHECK(N >= 0 && K >= 0, MOE_ERR_INVALID_ARG);
    CHECK(v_dtype == MOE_DT_BF16 || v_dtype == MOE_DT_F32, MOE_ERR_INVALID_ARG);
    CHECK(K % 64 == 0, MOE_ERR_UNSUPPORTED);
    if (N == 0 || K == 0) return MOE_OK;
    CHECK(v && out, MOE_ERR_INVALID_ARG);
    CHECK(ldv >= K && ldv % 8 == 0 && ldo >= K && ldo % 64 == 0, MOE_ERR_INVALID_ARG);
    CHECK(aligned(v, 16) && aligned(out, 128), MOE_ERR_INVALID_ARG);
    HIP_TRY(launch_fp6x2_split(v, v_dtype == MOE_DT_F32, ldv, N, K, out, 2 * ldo,
                               as_stream(stream)));
    return MOE_OK;
}

size_t moe_grouped_gemm_fp6x2_workspace_size(int num_local, int max_rows)
{
    if (num_local < 1 || max_rows < 0) return 0;
    return grouped_gemm_ws_bytes(num_local, max_rows, 0, MOE_SCHED_TILE256);
}

int moe_grouped_gemm_fp6x2(const uint8_t *a, int64_t lda, const int32_t *a_rows,
                           const uint8_t *w1_codes, const uint8_t *w1_scales,
                           const uint8_t *w2_codes, const uint8_t *w2_scales,
                           const int32_t *expert_offsets, int num_local, int max_rows, int N,
                           int K, int block_size, int w_layout, int act, void *out,
                           int out_dtype, int64_t ldo, void *ws, size_t ws_bytes,
                           moe_stream_t stream)
{
    const bool rec = out_dtype == MOE_DT_FP6X2;
    int rc = check_gemm(a, lda, w1_codes, w1_scales, w2_codes, w2_scales, expert_offsets,
                        num_local, max_rows, N, K, block_size, w_layout, act, out,
                        rec ? MOE_DT_BF16 : out_dtype, ldo);
    if (rc) return rc;
    CHECK(K <= 4096, MOE_ERR_UNSUPPORTED);
    CHECK(!(rec && act == MOE_ACT_NONE), MOE_ERR_UNSUPPORTED);
    if (max_rows == 0) return MOE_OK;
    CHECK(lda % 64 == 0 && aligned(a, 128), MOE_ERR_INVALID_ARG);
    if (rec) CHECK(ldo % 64 == 0 && aligned(out, 128), MOE_ERR_INVALID_ARG);
    rc = check_ws(ws, ws_bytes, grouped_gemm_ws_bytes(num_local, max_rows, 0, MOE_SCHED_TILE256));
    if (rc) return rc;
    const int kind = rec ? F6_OUT_RECORDS : out_dtype == MOE_DT_F32 ? F6_OUT_F32 : F6_OUT_BF16;
    HIP_TRY(launch_grouped_gemm_fp6x2(a, lda, a_rows, w1_codes, w1_scales, w2_codes, w2_scales,
                                      expert_offsets, num_local, max_rows, N, K, act, out, kind,
                                      ldo, ws, w_layout == MOE_LAYOUT_PACKED, as_stream(stream)));
    return MOE_OK;
}

size_t moe_grouped_gemm_mx8_workspace_size(int num_local, int max_rows)
{
    if (num_local < 1 || max_rows < 0) return 0;
    return mx8_gemm_ws_bytes(num_local, max_rows);
}

int moe_grouped_gemm_mx8(const uint8_t *a_codes, const uint8_t *a_scales, int64_t lda,
                         const int32_t *a_rows, const uint8_t *w1_codes,
                         const uint8_t *w1_scales, const uint8_t *w2_codes,
                         const uint8_t *w2_scales, const int32_t *expert_offsets, int num_local,
                         int max_rows, int N, int K, int block_size, int w_layout, int act,
                         void *out, int out_dtype, uint8_t *out_scales, int64_t ldo, int mode,
                         void *ws, size_t ws_bytes, moe_stream_t stream)
{
    const bool q_out = out_dtype == MOE_DT_MXFP8;
    CHECK(mode == MOE_SCHED_AUTO || mode == MOE_SCHED_STREAM || mode == MOE_SCHED_TILED ||
              mode == MOE_SCHED_TILE128 || mode == MOE_SCHED_TILE256,
          MOE_ERR_INVALID_ARG);
    // MXFP8 output is written by the tiled schedules only
    CHECK(!(q_out && mode == MOE_SCHED_STREAM), MOE_ERR_UNSUPPORTED);
    int rc = check_gemm(a_codes, lda, w1_codes, w1_scales, w2_codes, w2_scales, expert_offsets,
                        num_local, max_rows, N, K, block_size, w_layout, act, out,
                        q_out ? MOE_DT_BF16 : out_dtype, ldo);
    if (rc) return rc;
    CHECK(q_out == (out_scales != nullptr), MOE_ERR_INVALID_ARG);
    if (max_rows == 0) return MOE_OK;
    CHECK(a_scales && lda % 32 == 0, MOE_ERR_INVALID_ARG);
    if (q_out) CHECK(ldo % 32 == 0 && aligned(out, 16), MOE_ERR_INVALID_ARG);
    rc = check_ws(ws, ws_bytes, mx8_gemm_ws_bytes(num_local, max_rows));
    if (rc) return rc;
    HIP_TRY(launch_grouped_gemm_mx8(a_codes, a_scales, lda, a_rows, w1_codes, w1_scales,
                                    w2_codes, w2_scales, expert_offsets, num_local, max_rows, N,
                                    K, act, out,
                                    q_out ? MX8_OUT_MXFP8
                                          : out_dtype == MOE_DT_F32 ? MX8_OUT_F32 : MX8_OUT_BF16,
                                    out_scales, ldo, mode, ws, w_layout == MOE_LAYOUT_PACKED,
                                    as_stream(stream)));
    return MOE_OK;
}

int moe_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int64_t N, int K, void *out,
                      moe_stream_t stream)
{
    CHECK(N >= 0 && K >= 0, MOE_ERR_INVALID_ARG);
    CHECK(K % 32 == 0, MOE_ERR_UNSUPPORTED);
    if (N == 0 || K == 0) return MOE_OK;
    CHECK(codes && scales && out, MOE_ERR_INVALID_ARG);
    CHECK(aligned(codes, 4) && aligned(out, 16), MOE_ERR_INVALID_ARG);
    HIP_TRY(launch_mxfp4_dequant(codes, scales, N, K, (bf16 *)out, as_stream(stream)));
    return MOE_OK;
}

size_t moe_mxfp4_packed_scale_bytes(int N, int K)
{
    if (N < 0 || K < 0 || N % 16 || K % 128) return 0;
    return packed_scale_bytes(N, K);
}

int moe_mxfp4_prepack(const uint8_t *codes, const uint8_t *scales, int n_mats, int N, int K,
                      uint8_t *packed_codes, uint8_t *packed_scales, moe_stream_t stream)
{
    CHECK(n_mats >= 0 && N >= 0 && K >= 0, MOE_ERR_INVALID_ARG);
    CHECK(N % 16 == 0 && K % 128 == 0, MOE_ERR_UNSUPPORTED);
    if (n_mats == 0 || N == 0 || K == 0) return MOE_OK;
    CHECK(codes && scales && packed_codes && packed_scales, MOE_ERR_INVALID_ARG);
    CHECK(aligned(codes, 16) && aligned(packed_codes, 16), MOE_ERR_INVALID_ARG);
    HIP_TRY(launch_prepack(codes, scales, (int64_t)n_mats * N, K, packed_codes, packed_scales,
                           as_stream(stream)));
    return MOE_OK;
}

int moe_grouped_gemm_schedule(int num_local, int max_rows, int mode)
{
    if (num_local < 1 || max_rows < 0 || mode < MOE_SCHED_AUTO || mode > MOE_SCHED_TILE256)
        return -1;
    return resolve_mode(mode, num_local, max_rows);
}

size_t moe_grouped_gemm_workspace_size(int num_local, int max_rows, int N, int mode)
{
    if (num_local < 1 || max_rows < 0 || mode < MOE_SCHED_AUTO || mode > MOE_SCHED_TILE256)
        return 0;
    return grouped_gemm_ws_bytes(num_local, max_rows, N, mode);
}

int moe_grouped_gemm_mxfp4(const void *a, int64_t lda, const int32_t *a_rows,
                           const uint8_t *w1_codes, const uint8_t *w1_scales,
                           const uint8_t *w2_codes, const uint8_t *w2_scales,
                           const int32_t *expert_offsets, int num_local, int max_rows, int N,
                           int K, int block_size, int w_layout, int act, void *out,
                           int out_dtype, int64_t ldo, int mode, void *ws, size_t ws_bytes,
                           moe_stream_t stream)
{
    CHECK(mode >= MOE_SCHED_AUTO && mode <= MOE_SCHED_TILE256, MOE_ERR_INVALID_ARG);
    int rc = check_gemm(a, lda, w1_codes, w1_scales, w2_codes, w2_scales, expert_offsets,
                        num_local, max_rows, N, K, block_size, w_layout, act, out, out_dtype,
                        ldo);
    if (rc) return rc;
    if (max_rows == 0) return MOE_OK;
    rc = check_ws(ws, ws_bytes, grouped_gemm_ws_bytes(num_local, max_rows, N, mode));
    if (rc) return rc;
    HIP_TRY(launch_grouped_gemm((const bf16 *)a, lda, a_rows, w1_codes, w1_scales, w2_codes,
                                w2_scales, expert_offsets, num_local, max_rows, N, K, act, out,
                                out_dtype == MOE_DT_F32, ldo, mode, ws,
                                w_layout == MOE_LAYOUT_PACKED, as_stream(stream)));
    return MOE_OK;
}

int moe_combine(const void *y, int y_dtype, int64_t ldy, const int32_t *inv,
                const float *topk_w, int T, int d, int k, void *out, int out_dtype, int64_t ldo,
                moe_stream_t stream)
{
    CHECK(T >= 0 && d >= 1 && k >= 1, MOE_ERR_INVALID_ARG);
    CHECK(y_dtype == MOE_DT_BF16 || y_dtype == MOE_DT_F32, MOE_ERR_INVALID_ARG);
    CHECK(out_dtype == MOE_DT_BF16 || out_dtype == MOE_DT_F32, MOE_ERR_INVALID_ARG);
    CHECK(k <= MOE_MAX_TOPK, MOE_ERR_UNSUPPORTED);
    CHECK(d % 8 == 0, MOE_ERR_UNSUPPORTED);
    if (T == 0) return MOE_OK;
    CHECK(y && inv && topk_w && out, MOE_ERR_INVALID_ARG);
    CHECK(ldy >= d && ldy % 8 == 0 && ldo >= d && ldo % 8 == 0, MOE_ERR_INVALID_ARG);
    CHECK(aligned(y, 16) && aligned(out, 16), MOE_ERR_INVALID_ARG);
    HIP_TRY(launch_combine(y, y_dtype == MOE_DT_F32, ldy, inv, topk_w, T, d, k, out,
                           out_dtype == MOE_DT_F32, ldo, as_stream(stream)));
    return MOE_OK;
}

size_t moe_layer_workspace_size(const moe_layer_params *p)
{
    if (check_layer_params(p) != MOE_OK) return 0;
    return layer_ws(p).total;
}

namespace {
// Pointer checks shared by moe_layer and moe_layer_noalloc (the parameters
// already checked).
int check_layer_ptrs(const void *x, const float *w_router, const uint8_t *gate_codes,
                     const uint8_t *gate_scales, const uint8_t *up_codes,
                     const uint8_t *up_scales, const uint8_t *down_codes,
                     const uint8_t *down_scales, const void *out)
{
    CHECK(x && w_router && out && gate_codes && gate_scales && up_codes && up_scales &&
              down_codes && down_scales,
          MOE_ERR_INVALID_ARG);
    CHECK(aligned(x, 16) && aligned(out, 16) && aligned(w_router, 16), MOE_ERR_INVALID_ARG);
    CHECK(aligned(gate_codes, 16) && aligned(up_codes, 16) && aligned(down_codes, 16) &&
              aligned(gate_scales, 16) && aligned(up_scales, 16) && aligned(down_scales, 16),
          MOE_ERR_INVALID_ARG);
    return MOE_OK;
}

// The layer's launch sequence over the scratch at `base` (L.total bytes,
// 256-byte aligned). Every scratch word a kernel reads was written earlier in
// the same call, so the scratch need not start cleared.
int layer_run(const moe_layer_params *p, const LayerWs &L, char *base, const void *x,
              const float *w_router, const float *bias, const uint8_t *gate_codes,
              const uint8_t *gate_scales, const uint8_t *up_codes, const uint8_t *up_scales,
              const uint8_t *down_codes, const uint8_t *down_scales, void *out,
              float *logits_out, int32_t *topk_idx_out, float *topk_w_out, void **stage_events,
              moe_stream_t stream)
{
    float *logits = logits_out ? logits_out : (float *)(base + L.logits);
    int32_t *idx = topk_idx_out ? topk_idx_out : (int32_t *)(base + L.idx);
    float *w = topk_w_out ? topk_w_out : (float *)(base + L.w);
    int32_t *off = (int32_t *)(base + L.off);
    int32_t *perm = (int32_t *)(base + L.perm);
    int32_t *inv = (int32_t *)(base + L.inv);
    bf16 *h = (bf16 *)(base + L.h);
    float *y = (float *)(base + L.y);
    const int A = p->T * p->k;
    const int packed = p->weight_layout == MOE_LAYOUT_PACKED;
    hipStream_t s = as_stream(stream);
    hipEvent_t *ev = (hipEvent_t *)stage_events;

    if (ev) HIP_TRY(hipEventRecord(ev[0], s));
    HIP_TRY(layer_route(p, L, base, x, w_router, bias, logits, idx, w, s));
    if (ev) HIP_TRY(hipEventRecord(ev[1], s));
    int32_t *counts = nullptr;
    // one work plan serves both projections (same offsets, bound and schedule;
    // the FP6X2 gate/up takes 256- or 128-row groups, and a down projection on
    // the other tile gets a plan of its own)
    const GemmPlanArgs plan =
        gemm_plan_args(p->num_local, A,
                       L.f6 ? (L.gu128 ? MOE_SCHED_TILE128 : MOE_SCHED_TILE256) : p->mode,
                       base + L.gws);
    if (p->precision == MOE_PREC_MX8) {
        const GemmPlanArgs pm = mx8_plan_args(p->num_local, A, p->mode, base + L.gws);
        HIP_TRY(launch_permute(idx, counts, p->T, p->k, p->expert_begin, p->num_local, off, perm,
                               inv, base + L.pws, s, &pm));
        uint8_t *xq = (uint8_t *)(base + L.xq), *xs = (uint8_t *)(base + L.xs);
        uint8_t *hq = (uint8_t *)(base + L.hq), *hs = (uint8_t *)(base + L.hs);
        float *h32 = (float *)(base + L.h);
        if (ev) HIP_TRY(hipEventRecord(ev[2], s));
        // gate/up stage: the tokens to MXFP8, then the projection with act
        // (h in fp32). A separate pass converts h: quantising in the GEMM
        // epilogue (MX8_OUT_MXFP8) measured slower, as its per-element
        // reduction and rounding work sits on the MFMA-bound kernel.
        HIP_TRY(launch_mxfp8_quantize(x, 0, p->d, p->T, p->d, xq, xs, s));
        HIP_TRY(launch_gemm_mx8_run(xq, xs, p->d, perm, gate_codes, gate_scales, up_codes,
                                    up_scales, p->num_local, A, p->I, p->d, p->act, h32,
                                    MX8_OUT_F32, nullptr, p->I, p->mode, base + L.gws, packed,
                                    s));
        if (ev) HIP_TRY(hipEventRecord(ev[3], s));
        // down stage: h to MXFP8 (only the off[num_local] rows it holds: A is
        // the host bound, T k, eight times the local rows on an EP share), then
        // the projection; on the 256-row tile Y leaves as block-int16 rows
        // (half fp32's bytes, within 2^-15 of each 32-column block's largest
        // magnitude) for the matching combine
        HIP_TRY(launch_mxfp8_quantize(h32, 1, p->I, A, p->I, hq, hs, s, off + p->num_local));
        const bool q16 = mx8_q16_ok(p->mode, p->num_local, A, p->I);
        int16_t *yq = (int16_t *)y;
        uint8_t *ys = (uint8_t *)(base + L.y) + (size_t)A * p->d * 2;
        HIP_TRY(launch_gemm_mx8_run(hq, hs, p->I, nullptr, down_codes, down_scales, nullptr,
                                    nullptr, p->num_local, A, p->d, p->I, MOE_ACT_NONE,
                                    q16 ? (void *)yq : (void *)y,
                                    q16 ? MX8_OUT_Q16 : MX8_OUT_F32, q16 ? ys : nullptr, p->d,
                                    p->mode, base + L.gws, packed, s));
        if (ev) HIP_TRY(hipEventRecord(ev[4], s));
        if (q16)
            HIP_TRY(launch_combine_q16(yq, ys, p->d, inv, w, p->T, p->d, p->k, out,
                                       p->out_dtype == MOE_DT_F32, p->d, s));
        else
            HIP_TRY(launch_combine(y, 1, p->d, inv, w, p->T, p->d, p->k, out,
                                   p->out_dtype == MOE_DT_F32, p->d, s));
        if (ev) HIP_TRY(hipEventRecord(ev[5], s));
        return MOE_OK;
    }
    HIP_TRY(launch_permute(idx, counts, p->T, p->k, p->expert_begin, p->num_local, off, perm, inv,
                           base + L.pws, s, &plan));
    // FP6X2: the tokens as two MXFP6 planes, with the dispatch (the gate/up
    // stage is then the projection alone)
    if (L.f6)
        HIP_TRY(launch_fp6x2_split(x, 0, p->d, p->T, p->d, (uint8_t *)(base + L.xf),
                                   2 * (int64_t)p->d, s));
    if (ev) HIP_TRY(hipEventRecord(ev[2], s));
    if (L.f6) {
        const uint8_t *xf = (const uint8_t *)(base + L.xf);
        // h leaves the epilogue as split records (from fp32, no bf16 h)
        HIP_TRY(launch_gemm_fp6x2_run(xf, p->d, perm, gate_codes, gate_scales, up_codes,
                                      up_scales, p->num_local, A, p->I, p->d, p->act,
                                      base + L.hf, F6_OUT_RECORDS, p->I, base + L.gws, packed,
                                      s, nullptr, L.gu128));
    } else {
        HIP_TRY(launch_gemm_run((const bf16 *)x, p->d, perm, gate_codes, gate_scales, up_codes,
                                up_scales, p->num_local, A, p->I, p->d, p->act, h, 0, p->I,
                                p->mode, base + L.gws, packed, s));
    }
    if (ev) HIP_TRY(hipEventRecord(ev[3], s));
    // FP6X2: the expert outputs as block-int16 rows (each value within 2^-15
    // of its 32-column block's largest magnitude), half the bytes of fp32
    // for the down projection to write and the combine to read
    int16_t *yq = (int16_t *)y;
    uint8_t *ys = (uint8_t *)(base + L.y) + (size_t)A * p->d * 2;
    if (L.f6) {
        const bool own_plan = L.gu128 != L.dn128;
        if (own_plan)
            HIP_TRY(launch_gemm_plan_into(
                off, p->num_local,
                gemm_plan_args(p->num_local, A, L.dn128 ? MOE_SCHED_TILE128 : MOE_SCHED_TILE256,
                               base + L.gws2), s));
        HIP_TRY(launch_gemm_fp6x2_run((const uint8_t *)(base + L.hf), p->I, nullptr,
                                      down_codes, down_scales, nullptr, nullptr, p->num_local, A,
                                      p->d, p->I, MOE_ACT_NONE, yq, F6_OUT_Q16, p->d,
                                      base + (own_plan ? L.gws2 : L.gws), packed, s, ys,
                                      L.dn128));
    } else {
        HIP_TRY(launch_gemm_run(h, p->I, nullptr, down_codes, down_scales, nullptr, nullptr,
                                p->num_local, A, p->d, p->I, MOE_ACT_NONE, y, 1, p->d, p->mode,
                                base + L.gws, packed, s));
    }
    if (ev) HIP_TRY(hipEventRecord(ev[4], s));
    if (L.f6)
        HIP_TRY(launch_combine_q16(yq, ys, p->d, inv, w, p->T, p->d, p->k, out,
                                   p->out_dtype == MOE_DT_F32, p->d, s));
    else
        HIP_TRY(launch_combine(y, 1, p->d, inv, w, p->T, p->d, p->k, out,
                               p->out_dtype == MOE_DT_F32, p->d, s));
    if (ev) HIP_TRY(hipEventRecord(ev[5], s));
    return MOE_OK;
}

// The scratch of moe_layer_noalloc is `scratch` (file scope, above). In host
// code that name is a host-side stand-in, never the device memory: kernels
// get the address hipGetSymbolAddress returns for the current device, looked
// up once per device on its first call and kept in g_scratch_ptr.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

int noalloc_scratch(char **base)
{
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) {
        g_last_error = "moe_layer_noalloc: device ordinal outside the scratch table";
        return MOE_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr || !aligned(ptr, 256)) {
            g_last_error = "moe_layer_noalloc: scratch symbol address missing or misaligned";
            return MOE_ERR_HIP;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *base = (char *)g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

int moe_layer(const moe_layer_params *p, const void *x, const float *w_router, const float *bias,
              const uint8_t *gate_codes, const uint8_t *gate_scales, const uint8_t *up_codes,
              const uint8_t *up_scales, const uint8_t *down_codes, const uint8_t *down_scales,
              void *out, float *logits_out, int32_t *topk_idx_out, float *topk_w_out, void *ws,
              size_t ws_bytes, void **stage_events, moe_stream_t stream)
{
    int rc = check_layer_params(p);
    if (rc) return rc;
    if (p->T == 0) return MOE_OK;
    rc = check_layer_ptrs(x, w_router, gate_codes, gate_scales, up_codes, up_scales, down_codes,
                          down_scales, out);
    if (rc) return rc;
    const LayerWs L = layer_ws(p);
    rc = check_ws(ws, ws_bytes, L.total);
    if (rc) return rc;
    return layer_run(p, L, (char *)ws, x, w_router, bias, gate_codes, gate_scales, up_codes,
                     up_scales, down_codes, down_scales, out, logits_out, topk_idx_out,
                     topk_w_out, stage_events, stream);
}

int moe_layer_noalloc(const moe_layer_params *p, const void *x, const float *w_router,
                      const float *bias, const uint8_t *gate_codes, const uint8_t *gate_scales,
                      const uint8_t *up_codes, const uint8_t *up_scales,
                      const uint8_t *down_codes, const uint8_t *down_scales, void *out,
                      float *logits_out, int32_t *topk_idx_out, float *topk_w_out,
                      moe_stream_t stream)
{
    int rc = check_layer_params(p);
    if (rc) return rc;
    if (p->T == 0) return MOE_OK;
    rc = check_layer_ptrs(x, w_router, gate_codes, gate_scales, up_codes, up_scales, down_codes,
                          down_scales, out);
    if (rc) return rc;
    const LayerWs L = layer_ws(p);
    if (L.total > MOE_NOALLOC_SCRATCH_BYTES) {
        g_last_error = "moe_layer_noalloc: these parameters need " + std::to_string(L.total) +
                       " bytes of scratch, more than the " +
                       std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES) +
                       "-byte static scratch; use moe_layer with a workspace";
        return MOE_ERR_WORKSPACE;
    }
    char *base = nullptr;
    rc = noalloc_scratch(&base);
    if (rc) return rc;
    return layer_run(p, L, base, x, w_router, bias, gate_codes, gate_scales, up_codes,
                     up_scales, down_codes, down_scales, out, logits_out, topk_idx_out,
                     topk_w_out, nullptr, stream);
}

size_t moe_grouped_lora_workspace_size(int max_rows, int rank)
{
    if (max_rows < 0 || rank < 1 || rank > MOE_MAX_LORA_RANK) return 0;
    return lora_ws_bytes(max_rows, rank);
}

int moe_grouped_lora(const void *x, int64_t ldx, const int32_t *x_rows, const void *lora_a,
                     const void *lora_b, int rank, float scale, const int32_t *expert_offsets,
                     int num_local, int max_rows, int N, int K, float *y, int64_t ldy, void *ws,
                     size_t ws_bytes, moe_stream_t stream)
{
    CHECK(num_local >= 1 && max_rows >= 0 && N >= 1 && K >= 1, MOE_ERR_INVALID_ARG);
    CHECK(rank >= 1 && rank <= MOE_MAX_LORA_RANK, MOE_ERR_UNSUPPORTED);
    CHECK(K % 8 == 0 && N % 4 == 0, MOE_ERR_UNSUPPORTED);
    if (max_rows == 0) return MOE_OK;
    CHECK(x && lora_a && lora_b && expert_offsets && y, MOE_ERR_INVALID_ARG);
    CHECK(ldx >= K && ldx % 8 == 0 && ldy >= N && ldy % 4 == 0, MOE_ERR_INVALID_ARG);
    CHECK(aligned(x, 16) && aligned(lora_a, 16) && aligned(y, 16), MOE_ERR_INVALID_ARG);
    int rc = check_ws(ws, ws_bytes, lora_ws_bytes(max_rows, rank));
    if (rc) return rc;
    HIP_TRY(launch_lora((const bf16 *)x, ldx, x_rows, (const bf16 *)lora_a,
                        (const bf16 *)lora_b, rank, scale, expert_offsets, num_local, max_rows, N,
                        K, y, ldy, (float *)ws, as_stream(stream)));
    return MOE_OK;
}

namespace {
// moe_layer's workspace plus fp32 gate and up projections and the rank factor
struct LoraWs {
    LayerWs L;
    size_t g, u, t, total;
};

// The increment rides in the GEMMs (rank factors as hi + lo bf16 parts, two
// more MFMAs per output tile and 16 or 32 ranks) when the rank is a multiple
// of 16; otherwise the gate and up projections run unfused.
bool lora_fused(const moe_layer_params *p, int rank)
{
    (void)p;
    return rank % 16 == 0;
}

LoraWs lora_layer_ws(const moe_layer_params *p, int rank)
{
    LoraWs W;
    W.L = layer_ws(p);
    const size_t A = (size_t)p->T * p->k;
    size_t o = W.L.total;
    if (lora_fused(p, rank)) {
        // three rank-factor arrays (gate, up, down), hi and lo bf16 parts
        W.g = W.u = 0;
        W.t = o; o += 3 * round_up(A * (size_t)rank * 4);
    } else {
        W.g = o; o += round_up(A * (size_t)p->I * 4);
        W.u = o; o += round_up(A * (size_t)p->I * 4);
        W.t = o; o += lora_ws_bytes((int)A, rank);
    }
    W.total = o;
    return W;
}

int check_lora(const moe_layer_params *p, const moe_lora_adapters *lora)
{
    CHECK(lora, MOE_ERR_INVALID_ARG);
    CHECK(lora->rank >= 1 && lora->rank <= MOE_MAX_LORA_RANK, MOE_ERR_UNSUPPORTED);
    CHECK(p->precision == MOE_PREC_BF16, MOE_ERR_UNSUPPORTED);
    return MOE_OK;
}
}  // namespace

size_t moe_layer_lora_workspace_size(const moe_layer_params *p, int rank)
{
    if (check_layer_params(p) != MOE_OK || p->precision != MOE_PREC_BF16 || rank < 1 ||
        rank > MOE_MAX_LORA_RANK)
        return 0;
    return lora_layer_ws(p, rank).total;
}

int moe_layer_lora(const moe_layer_params *p, const moe_lora_adapters *lora, const void *x,
                   const float *w_router, const float *bias, const uint8_t *gate_codes,
                   const uint8_t *gate_scales, const uint8_t *up_codes, const uint8_t *up_scales,
                   const uint8_t *down_codes, const uint8_t *down_scales, void *out,
                   float *logits_out, int32_t *topk_idx_out, float *topk_w_out, void *ws,
                   size_t ws_bytes, void **stage_events, moe_stream_t stream)
{
    int rc = check_layer_params(p);
    if (rc) return rc;
    rc = check_lora(p, lora);
    if (rc) return rc;
    if (p->T == 0) return MOE_OK;
    CHECK(x && w_router && out && gate_codes && gate_scales && up_codes && up_scales &&
              down_codes && down_scales,
          MOE_ERR_INVALID_ARG);
    CHECK(lora->gate_a && lora->gate_b && lora->up_a && lora->up_b && lora->down_a &&
              lora->down_b,
          MOE_ERR_INVALID_ARG);
    CHECK(aligned(x, 16) && aligned(out, 16) && aligned(w_router, 16), MOE_ERR_INVALID_ARG);
    CHECK(aligned(gate_codes, 16) && aligned(up_codes, 16) && aligned(down_codes, 16) &&
              aligned(gate_scales, 16) && aligned(up_scales, 16) && aligned(down_scales, 16),
          MOE_ERR_INVALID_ARG);
    CHECK(aligned(lora->gate_a, 16) && aligned(lora->up_a, 16) && aligned(lora->down_a, 16) &&
              aligned(lora->gate_b, 16) && aligned(lora->up_b, 16) && aligned(lora->down_b, 16),
          MOE_ERR_INVALID_ARG);
    const LoraWs W = lora_layer_ws(p, lora->rank);
    const LayerWs &L = W.L;
    rc = check_ws(ws, ws_bytes, W.total);
    if (rc) return rc;

    char *base = (char *)ws;
    float *logits = logits_out ? logits_out : (float *)(base + L.logits);
    int32_t *idx = topk_idx_out ? topk_idx_out : (int32_t *)(base + L.idx);
    float *w = topk_w_out ? topk_w_out : (float *)(base + L.w);
    int32_t *off = (int32_t *)(base + L.off);
    int32_t *perm = (int32_t *)(base + L.perm);
    int32_t *inv = (int32_t *)(base + L.inv);
    bf16 *h = (bf16 *)(base + L.h);
    float *y = (float *)(base + L.y);
    float *g32 = (float *)(base + W.g), *u32 = (float *)(base + W.u), *t = (float *)(base + W.t);
    const int A = p->T * p->k, nl = p->num_local, r = lora->rank;
    const float sc = lora->scale;
    const int packed = p->weight_layout == MOE_LAYOUT_PACKED;
    hipStream_t s = as_stream(stream);
    hipEvent_t *ev = (hipEvent_t *)stage_events;

    if (ev) HIP_TRY(hipEventRecord(ev[0], s));
    HIP_TRY(layer_route(p, L, base, x, w_router, bias, logits, idx, w, s));
    if (ev) HIP_TRY(hipEventRecord(ev[1], s));
    const GemmPlanArgs plan = gemm_plan_args(nl, A, p->mode, base + L.gws);
    HIP_TRY(launch_permute(idx, nullptr, p->T, p->k, p->expert_begin, nl, off, perm, inv,
                           base + L.pws, s, &plan));
    if (ev) HIP_TRY(hipEventRecord(ev[2], s));
    const bf16 *xb = (const bf16 *)x;
    if (lora_fused(p, r)) {
        // rank factors first (hi + lo bf16), then the projections with the
        // increment added to their accumulators before the activation / output
        const size_t tb = round_up((size_t)A * r * 4);
        bf16 *tg = (bf16 *)(base + W.t), *tu = (bf16 *)(base + W.t + tb),
             *td = (bf16 *)(base + W.t + 2 * tb);
        HIP_TRY(launch_lora_t_plan(xb, p->d, perm, (const bf16 *)lora->gate_a,
                                   (const bf16 *)lora->up_a, r, p->d, sc, plan, tg, tu, s));
        const LoraEpi lg{tg, tu, (const bf16 *)lora->gate_b, (const bf16 *)lora->up_b, r};
        HIP_TRY(launch_gemm_run(xb, p->d, perm, gate_codes, gate_scales, up_codes, up_scales, nl,
                                A, p->I, p->d, p->act, h, 0, p->I, p->mode, base + L.gws, packed,
                                s, &lg));
        if (ev) HIP_TRY(hipEventRecord(ev[3], s));
        HIP_TRY(launch_lora_t_plan(h, p->I, nullptr, (const bf16 *)lora->down_a, nullptr, r, p->I,
                                   sc, plan, td, nullptr, s));
        const LoraEpi ld{td, nullptr, (const bf16 *)lora->down_b, nullptr, r};
        HIP_TRY(launch_gemm_run(h, p->I, nullptr, down_codes, down_scales, nullptr, nullptr, nl,
                                A, p->d, p->I, MOE_ACT_NONE, y, 1, p->d, p->mode, base + L.gws,
                                packed, s, &ld));
        if (ev) HIP_TRY(hipEventRecord(ev[4], s));
        HIP_TRY(launch_combine(y, 1, p->d, inv, w, p->T, p->d, p->k, out,
                               p->out_dtype == MOE_DT_F32, p->d, s));
        if (ev) HIP_TRY(hipEventRecord(ev[5], s));
        return MOE_OK;
    }
    // gate and up unfused: the frozen projections, each plus its low-rank
    // increment, then the activation (the increment must land before it)
    HIP_TRY(launch_gemm_run(xb, p->d, perm, gate_codes, gate_scales, nullptr, nullptr, nl, A,
                            p->I, p->d, MOE_ACT_NONE, g32, 1, p->I, p->mode, base + L.gws, packed,
                            s));
    HIP_TRY(launch_gemm_run(xb, p->d, perm, up_codes, up_scales, nullptr, nullptr, nl, A, p->I,
                            p->d, MOE_ACT_NONE, u32, 1, p->I, p->mode, base + L.gws, packed, s));
    HIP_TRY(launch_lora(xb, p->d, perm, (const bf16 *)lora->gate_a, (const bf16 *)lora->gate_b,
                        r, sc, off, nl, A, p->I, p->d, g32, p->I, t, s));
    HIP_TRY(launch_lora(xb, p->d, perm, (const bf16 *)lora->up_a, (const bf16 *)lora->up_b, r,
                        sc, off, nl, A, p->I, p->d, u32, p->I, t, s));
    HIP_TRY(launch_glu(g32, u32, off, nl, A, p->I, p->act, h, s));
    if (ev) HIP_TRY(hipEventRecord(ev[3], s));
    HIP_TRY(launch_gemm_run(h, p->I, nullptr, down_codes, down_scales, nullptr, nullptr, nl, A,
                            p->d, p->I, MOE_ACT_NONE, y, 1, p->d, p->mode, base + L.gws, packed,
                            s));
    HIP_TRY(launch_lora(h, p->I, nullptr, (const bf16 *)lora->down_a, (const bf16 *)lora->down_b,
                        r, sc, off, nl, A, p->d, p->I, y, p->d, t, s));
    if (ev) HIP_TRY(hipEventRecord(ev[4], s));
    HIP_TRY(launch_combine(y, 1, p->d, inv, w, p->T, p->d, p->k, out,
                           p->out_dtype == MOE_DT_F32, p->d, s));
    if (ev) HIP_TRY(hipEventRecord(ev[5], s));
    return MOE_OK;
}

}  // extern "C"
