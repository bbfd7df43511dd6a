/*
 * moe_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A plain, slow, single-threaded CPU statement of what one Kimi-K3-style
 * LatentMoE layer with MXFP4 expert weights computes, from routing to combine.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. It shares no code, header, table or constant with the
 * GPU library, and never includes anything from it.
 *
 * Arithmetic is IEEE fp32 (build with -O2 -fno-fast-math -ffp-contract=off so
 * every product is rounded before it is added), with sums taken in increasing
 * index order. bf16 inputs are widened to fp32 exactly.
 *
 * Sources (cited below by key and section):
 *   P1  "从Kimi K3到MiniMax-H3：国产大模型竞争进入“推理系统战”" (gyznsw.cn)
 *   P2  "SGLang 0.5.17：Kimi K3 原生 MXFP4 推理架构解析" (mindlynx.top)
 *   P3  "Kimi K3 Day-0 适配剖析:KDA/Gated MLA 混合注意力、MXFP4 在线量化与
 *        896 专家 MoE" (7yue.com MUSA learning center, m8-l14)
 *   OCP-MX  OCP Microscaling Formats (MX) Specification v1.0: the E2M1 and
 *        E4M3 element types, the E8M0 shared scale with 32-element blocks, and
 *        the conversion to MX (shared exponent floor(log2 amax) minus the
 *        element type's emax, elements rounded to nearest-even and clamped).
 *
 * Two precision modes. The default one keeps the latent tokens and h in
 * bf16/fp32 against MXFP4 weights, as the pages describe (4-bit weights
 * combined with higher-precision activations, P1 §二 第一层). The MX8 mode
 * (functions ending in _mx8) quantises the tokens and h to MXFP8 (E4M3) before
 * each projection, the input contract of block-scaled 8-bit x 4-bit matrix
 * instructions; it is a separate accuracy contract, not an approximation of
 * the default mode. The FP6X2 functions state the two-plane MXFP6 (E2M3)
 * carriage of activations that the block-scaled 6-bit x 4-bit instructions
 * take; layers that use it are held to the default mode's contract.
 *
 * Pins (tests/test_oracle_*.py): the E2M1 table against its bit-field
 * definition; every E8M0 scale; every (code, scale) decode; hand-built
 * round-to-nearest-even blocks; byte equality with the independently written
 * generator quantiser; top-k against sorting; softmax sums and the k=1 and
 * all-equal closed forms; permutation invariants and permute-then-unpermute
 * identity; the layer against a dense, mask-weighted fp64 evaluation of every
 * expert that bypasses the permutation; E=1,k=1 against a textbook MLP; and
 * the all-ones closed form out = I*S*silu(S). MX8 mode: every E4M3 code
 * against torch's float8_e4m3fn and the spec's landmark values; the MXFP8
 * quantiser against frexp plus torch's round-to-nearest-even fp8 conversion
 * on tie, clamp, zero and extreme-exponent blocks; the layer against a dense
 * fp64 evaluation with its own quantisation; closed forms of all-ones
 * weights whose h lands on the E4M3 grid, on a tie and on the 448 clamp.
 * LoRA: zero B factors give the base layer bit for bit; the layer against a
 * dense fp64 evaluation with W + scale * B A as each expert's weights.
 * FP6X2: every E2M3 code against its bit fields and the spec's landmark
 * values; the MXFP6 quantiser against an arithmetic round-half-even on each
 * binade's step with a bit-field encoder, on tie, clamp, zero and
 * extreme-exponent blocks; a split worked by hand; the per-element bound
 * 2^(E-7) that two planes imply.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 and the MXFP4 element / scale types                            */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an fp32 bit pattern: widening is exact. */
static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP-MX E2M1: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0;
 * exponent 0 is subnormal (0 or 0.5). The values, listed by code. MXFP4 is
 * the 4-bit element with one shared scale per small block (P1 §二 第一层;
 * P2 §MXFP4原生支持). */
static const float E2M1_VALUE[16] = {
    0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
    -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f,
};

float oracle_e2m1_value(int code) { return E2M1_VALUE[code & 15]; }

/* OCP-MX E8M0: the scale is 2^(s-127); s = 255 is NaN and outside the
 * input contract. 2^-127 is an fp32 subnormal and still exact. */
float oracle_e8m0_value(int s) { return ldexpf(1.0f, s - 127); }

/* One stored element: E2M1 value times its block's scale (exact in fp32). */
static float mx_value(const uint8_t *codes, const uint8_t *scales, int64_t K,
                      int64_t n, int64_t i)
{
    uint8_t byte = codes[n * (K / 2) + i / 2];
    int code = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
    int s = scales[n * (K / 32) + i / 32];
    return ldexpf(E2M1_VALUE[code], s - 127);
}

/* Decode a whole [N, K] matrix: codes [N, K/2] (element 2i in the low nibble
 * of byte i), scales [N, K/32]. */
void oracle_mxfp4_decode(const uint8_t *codes, const uint8_t *scales,
                         int64_t N, int64_t K, float *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t i = 0; i < K; i++)
            out[n * K + i] = mx_value(codes, scales, K, n, i);
}

/* Round a magnitude in [0, 8) to the nearest E2M1 magnitude; on a tie take
 * the even code. Written as an argmin over the eight grid points. */
static int e2m1_round_magnitude(float a)
{
    int best = 0;
    float best_dist = fabsf(a - E2M1_VALUE[0]);
    for (int c = 1; c < 8; c++) {
        float dist = fabsf(a - E2M1_VALUE[c]);
        if (dist < best_dist || (dist == best_dist && (c % 2) == 0 && (best % 2) != 0)) {
            best = c;
            best_dist = dist;
        }
    }
    return best;
}

/* OCP-MX conversion of one 32-element block: shared exponent
 * floor(log2 amax) - emax(E2M1)=2, taken exactly from frexp; elements divided
 * by the scale (a power of two, so exactly) and rounded to nearest-even, with
 * magnitudes beyond 6 clamped to 6. All-zero block: scale 0, codes 0. */
void oracle_mxfp4_quantize(const float *w, int64_t N, int64_t K,
                           uint8_t *codes, uint8_t *scales)
{
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < K / 32; b++) {
            const float *v = w + n * K + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; i++)
                if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            int s = 0;
            if (amax != 0.0f) {
                int e2;
                frexpf(amax, &e2); /* amax = m * 2^e2, m in [0.5, 1) */
                s = (e2 - 1) - 2 + 127;
                if (s < 0) s = 0;
                if (s > 254) s = 254;
            }
            scales[n * (K / 32) + b] = (uint8_t)s;
            for (int i = 0; i < 32; i += 2) {
                int c[2] = {0, 0};
                for (int h = 0; h < 2; h++) {
                    if (amax == 0.0f) continue;
                    float q = v[i + h] / ldexpf(1.0f, s - 127);
                    float a = fabsf(q);
                    int mag = (a >= 6.0f) ? 7 : e2m1_round_magnitude(a);
                    c[h] = mag | (signbit(q) ? 8 : 0);
                }
                codes[n * (K / 2) + (b * 32 + i) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* MXFP8 activations (the block-scaled precision mode)                 */
/* ------------------------------------------------------------------ */

/* OCP-MX E4M3 (FP8): sign bit 7, exponent bits 6-3 (bias 7), mantissa bits
 * 2-0; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN, so the
 * largest finite magnitude is S.1111.110 = 448. No infinities. */
float oracle_e4m3_value(int code)
{
    code &= 0xff;
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    float v = (e == 0) ? ldexpf((float)m / 8.0f, -6) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -v : v;
}

/* Round a magnitude in [0, 448] to the nearest finite E4M3 magnitude
 * (codes 0x00..0x7E); on a tie take the even code. An argmin over the grid. */
static int e4m3_round_magnitude(float a)
{
    int best = 0;
    float best_dist = fabsf(a - oracle_e4m3_value(0));
    for (int c = 1; c <= 0x7E; c++) {
        float dist = fabsf(a - oracle_e4m3_value(c));
        if (dist < best_dist || (dist == best_dist && (c % 2) == 0 && (best % 2) != 0)) {
            best = c;
            best_dist = dist;
        }
    }
    return best;
}

/* OCP-MX conversion of [N, K] fp32 to MXFP8 (E4M3 elements, E8M0 scale per
 * 32-element block along K): shared exponent floor(log2 amax) - emax(E4M3)=8,
 * taken exactly from frexp and clamped to the E8M0 range; elements divided by
 * the scale (a power of two, so exactly) and rounded to nearest-even, with
 * magnitudes beyond 448 clamped to 448. All-zero block: scale 0, codes 0.
 * A negative element that rounds to zero keeps its sign (code 0x80).
 * codes [N, K] (one byte per element), scales [N, K/32]. */
void oracle_mxfp8_quantize(const float *v, int64_t N, int64_t K,
                           uint8_t *codes, uint8_t *scales)
{
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < K / 32; b++) {
            const float *blk = v + n * K + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; i++)
                if (fabsf(blk[i]) > amax) amax = fabsf(blk[i]);
            int s = 0;
            if (amax != 0.0f) {
                int e2;
                frexpf(amax, &e2); /* amax = m * 2^e2, m in [0.5, 1) */
                s = (e2 - 1) - 8 + 127;
                if (s < 0) s = 0;
                if (s > 254) s = 254;
            }
            scales[n * (K / 32) + b] = (uint8_t)s;
            for (int i = 0; i < 32; i++) {
                int c = 0;
                if (amax != 0.0f) {
                    float q = blk[i] / ldexpf(1.0f, s - 127);
                    float a = fabsf(q);
                    int mag = (a >= 448.0f) ? 0x7E : e4m3_round_magnitude(a);
                    c = mag | (signbit(q) ? 0x80 : 0);
                }
                codes[n * K + b * 32 + i] = (uint8_t)c;
            }
        }
    }
}

/* Decode [N, K] MXFP8: element value times its block's scale (exact). */
void oracle_mxfp8_decode(const uint8_t *codes, const uint8_t *scales,
                         int64_t N, int64_t K, float *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t i = 0; i < K; i++)
            out[n * K + i] = ldexpf(oracle_e4m3_value(codes[n * K + i]),
                                    (int)scales[n * (K / 32) + i / 32] - 127);
}

/* ------------------------------------------------------------------ */
/* Two-plane MXFP6 carriage of the activations (the FP6X2 mode)        */
/* ------------------------------------------------------------------ */

/* OCP-MX E2M3 (FP6): sign bit 5, exponent bits 4-3 (bias 1), mantissa bits
 * 2-0; exponent 0 is subnormal (m/8); the largest magnitude is 0.11.111 =
 * 7.5. No infinities or NaN. */
float oracle_e2m3_value(int code)
{
    code &= 0x3f;
    int sign = code >> 5, e = (code >> 3) & 3, m = code & 7;
    float v = (e == 0) ? (float)m / 8.0f : ldexpf(1.0f + (float)m / 8.0f, e - 1);
    return sign ? -v : v;
}

/* Round a magnitude in [0, 7.5] to the nearest E2M3 magnitude (codes
 * 0..31); on a tie take the even code. An argmin over the grid. */
static int e2m3_round_magnitude(float a)
{
    int best = 0;
    float best_dist = fabsf(a - oracle_e2m3_value(0));
    for (int c = 1; c < 32; c++) {
        float dist = fabsf(a - oracle_e2m3_value(c));
        if (dist < best_dist || (dist == best_dist && (c % 2) == 0 && (best % 2) != 0)) {
            best = c;
            best_dist = dist;
        }
    }
    return best;
}

/* OCP-MX conversion of [N, K] fp32 to MXFP6 (E2M3 elements, E8M0 scale per
 * 32-element block along K): shared exponent floor(log2 amax) - emax(E2M3)=2,
 * taken exactly from frexp and clamped to the E8M0 range; elements divided by
 * the scale (a power of two, so exactly) and rounded to nearest-even, with
 * magnitudes beyond 7.5 clamped to 7.5. All-zero block: scale 0, codes 0. A
 * negative element that rounds to zero keeps its sign (code 0x20).
 * codes [N, K] (one code per byte), scales [N, K/32]. */
void oracle_mxfp6_quantize(const float *v, int64_t N, int64_t K,
                           uint8_t *codes, uint8_t *scales)
{
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < K / 32; b++) {
            const float *blk = v + n * K + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; i++)
                if (fabsf(blk[i]) > amax) amax = fabsf(blk[i]);
            const int emax_e2m3 = 2;
            int s = 0;
            if (amax != 0.0f) {
                int e2;
                frexpf(amax, &e2); /* amax = m * 2^e2, m in [0.5, 1) */
                s = (e2 - 1) - emax_e2m3 + 127;
                if (s < 0) s = 0;
                if (s > 254) s = 254;
            }
            scales[n * (K / 32) + b] = (uint8_t)s;
            for (int i = 0; i < 32; i++) {
                int c = 0;
                if (amax != 0.0f) {
                    float q = blk[i] / ldexpf(1.0f, s - 127);
                    float a = fabsf(q);
                    int mag = (a >= 7.5f) ? 31 : e2m3_round_magnitude(a);
                    c = mag | (signbit(q) ? 0x20 : 0);
                }
                codes[n * K + b * 32 + i] = (uint8_t)c;
            }
        }
    }
}

/* Decode [N, K] MXFP6: element value times its block's scale (exact). */
void oracle_mxfp6_decode(const uint8_t *codes, const uint8_t *scales,
                         int64_t N, int64_t K, float *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t i = 0; i < K; i++)
            out[n * K + i] = ldexpf(oracle_e2m3_value(codes[n * K + i]),
                                    (int)scales[n * (K / 32) + i / 32] - 127);
}

/* The FP6X2 carriage of [N, K] activations as two MXFP6 planes, for the
 * block-scaled 6-bit x 4-bit matrix instructions (the pages keep activations
 * at higher precision than the 4-bit weights, P1 §二 第一层; two 6-bit planes
 * carry each value to within 2^(E-7), E = floor(log2 amax) of its block):
 *   plane 1 = MXFP6(v),
 *   plane 2 = MXFP6(v - decode(plane 1)), the difference taken in fp32.
 * The value carried is decode(plane 1) + decode(plane 2).
 * codes [2][N][K] (one code per byte), scales [2][N][K/32]. */
int oracle_fp6x2_split(const float *v, int64_t N, int64_t K, uint8_t *codes,
                       uint8_t *scales)
{
    float *d1 = (float *)malloc(sizeof(float) * (size_t)(N * K));
    float *r = (float *)malloc(sizeof(float) * (size_t)(N * K));
    if (!d1 || !r) {
        free(d1);
        free(r);
        return -1;
    }
    oracle_mxfp6_quantize(v, N, K, codes, scales);
    oracle_mxfp6_decode(codes, scales, N, K, d1);
    for (int64_t i = 0; i < N * K; i++) r[i] = v[i] - d1[i];
    oracle_mxfp6_quantize(r, N, K, codes + N * K, scales + N * (K / 32));
    free(d1);
    free(r);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Routing                                                             */
/* ------------------------------------------------------------------ */

/* Router scores: a score of every token against every expert, as the
 * token-by-router-weight product (P2 §MoE稀疏激活, the routing sketch),
 * plus an optional per-expert bias.
 * logits[t,e] = (sum_i x[t,i] * W_r[e,i]) + bias[e], fp32, i increasing. */
void oracle_router_logits(const uint16_t *x, const float *w_router, const float *bias,
                          int64_t T, int64_t d, int64_t E, float *logits)
{
    for (int64_t t = 0; t < T; t++) {
        for (int64_t e = 0; e < E; e++) {
            float acc = 0.0f;
            for (int64_t i = 0; i < d; i++)
                acc += bf16_bits_to_float(x[t * d + i]) * w_router[e * d + i];
            if (bias) acc += bias[e];
            logits[t * E + e] = acc;
        }
    }
}

/* Expert e beats expert f when its score is larger, or equal with the lower
 * index (IEEE compare: -0 equals +0). */
static int beats(float le, int64_t e, float lf, int64_t f)
{
    return le > lf || (le == lf && e < f);
}

/* Top-k selection (P2 §MoE稀疏激活: pick the 16 best of 896 per token;
 * P1 §一: 896 experts, 16 active) and the gate weights: a softmax over the
 * k selected scores, which weight the expert outputs in the final sum.
 * idx[t, 0..k-1] lists the winners best first. */
void oracle_topk_softmax(const float *logits, int64_t T, int64_t E, int64_t k,
                         int32_t *idx, float *w)
{
    char *taken = (char *)malloc((size_t)E);
    float *z = (float *)malloc((size_t)k * sizeof(float));
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int64_t j = 0; j < k; j++) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || beats(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            idx[t * k + j] = (int32_t)best;
        }
        float m = l[idx[t * k]];
        float sum = 0.0f;
        for (int64_t j = 0; j < k; j++) {
            z[j] = expf(l[idx[t * k + j]] - m);
            sum += z[j];
        }
        for (int64_t j = 0; j < k; j++)
            w[t * k + j] = z[j] / sum;
    }
    free(z);
    free(taken);
}

/* Dispatch index computation and buffer planning (P3 §四: dispatch sends each
 * token to its experts; the index computation and buffer plan are the
 * single-GPU part of it). */

/* counts[e] = number of (t, j) with idx[t,j] == e, over all E experts. */
void oracle_histogram(const int32_t *idx, int64_t T, int64_t k, int64_t E, int32_t *counts)
{
    for (int64_t e = 0; e < E; e++) counts[e] = 0;
    for (int64_t a = 0; a < T * k; a++) counts[idx[a]] += 1;
}

/* Exclusive prefix sum over the local expert range [e0, e0 + n_local). */
void oracle_offsets(const int32_t *counts, int64_t e0, int64_t n_local, int32_t *off)
{
    off[0] = 0;
    for (int64_t i = 0; i < n_local; i++) off[i + 1] = off[i] + counts[e0 + i];
}

/* Stable counting sort of the row-major (t, j) list by expert: rows of local
 * expert e occupy [off[e-e0], off[e-e0+1]) in increasing t. Assignments to
 * experts outside the local range are dropped: inv = -1. */
void oracle_permute(const int32_t *idx, const int32_t *off, int64_t T, int64_t k,
                    int64_t e0, int64_t n_local, int32_t *perm_token, int32_t *inv)
{
    int32_t *cur = (int32_t *)calloc((size_t)n_local, sizeof(int32_t));
    for (int64_t t = 0; t < T; t++) {
        for (int64_t j = 0; j < k; j++) {
            int64_t le = (int64_t)idx[t * k + j] - e0;
            if (le < 0 || le >= n_local) {
                inv[t * k + j] = -1;
                continue;
            }
            int32_t pos = off[le] + cur[le]++;
            perm_token[pos] = (int32_t)t;
            inv[t * k + j] = pos;
        }
    }
    free(cur);
}

/* ------------------------------------------------------------------ */
/* Expert compute                                                      */
/* ------------------------------------------------------------------ */

enum { ACT_NONE = 0, ACT_SILU_MUL = 1, ACT_GELU_TANH_MUL = 2 };

/* The elementwise stage between the two expert projections. The pages name
 * a K3-specific activation path without defining it (P1 §一), so the stage is
 * pluggable; SILU_MUL, silu(g) * u with silu(g) = g / (1 + e^-g), is the
 * default. GELU_TANH_MUL uses the tanh form of GELU. */
static float act_apply(int act, float g, float u)
{
    if (act == ACT_SILU_MUL) {
        float silu = g / (1.0f + expf(-g));
        return silu * u;
    }
    if (act == ACT_GELU_TANH_MUL) {
        const float c = 0.7978845608028654f; /* sqrt(2/pi) */
        float inner = c * (g + 0.044715f * g * g * g);
        float gelu = 0.5f * g * (1.0f + tanhf(inner));
        return gelu * u;
    }
    return g;
}

/* One expert's FFN on one latent token, weights already decoded to fp32:
 * g = Wg x, u = Wu x (each [I]), h = act(g, u), y = Wd h ([d]).
 * Higher-precision activations meet dequantised 4-bit weights and the
 * products are accumulated (P1 §二 第一层); the dequantisation is fused into
 * the matmul on the GPU (P2 §MXFP4原生支持) -- here it is done up front. */
static void expert_ffn(const float *xt, const float *wg, const float *wu, const float *wd,
                       int64_t d, int64_t I, int act, float *h, float *y)
{
    for (int64_t n = 0; n < I; n++) {
        float g = 0.0f, u = 0.0f;
        for (int64_t i = 0; i < d; i++) g += xt[i] * wg[n * d + i];
        for (int64_t i = 0; i < d; i++) u += xt[i] * wu[n * d + i];
        h[n] = act_apply(act, g, u);
    }
    for (int64_t m = 0; m < d; m++) {
        float acc = 0.0f;
        for (int64_t n = 0; n < I; n++) acc += h[n] * wd[m * I + n];
        y[m] = acc;
    }
}

/* The same FFN in the block-scaled precision mode (MX8): the latent token
 * arrives quantised to MXFP8 (xq, decoded values), and h is quantised to
 * MXFP8 along I before the down projection. A product of two MX values is
 * exact, so each projection sums in fp64 and rounds to fp32 once; h is
 * act(g, u) in fp32 as above. hq receives the decoded quantised h; hc, hs are
 * scratch for its codes [I] and scales [I/32]. */
static void expert_ffn_mx8(const float *xq, const float *wg, const float *wu, const float *wd,
                           int64_t d, int64_t I, int act, float *h, uint8_t *hc, uint8_t *hs,
                           float *hq, float *y)
{
    for (int64_t n = 0; n < I; n++) {
        double g = 0.0, u = 0.0;
        for (int64_t i = 0; i < d; i++) g += (double)xq[i] * (double)wg[n * d + i];
        for (int64_t i = 0; i < d; i++) u += (double)xq[i] * (double)wu[n * d + i];
        h[n] = act_apply(act, (float)g, (float)u);
    }
    oracle_mxfp8_quantize(h, 1, I, hc, hs);
    oracle_mxfp8_decode(hc, hs, 1, I, hq);
    for (int64_t m = 0; m < d; m++) {
        double acc = 0.0;
        for (int64_t n = 0; n < I; n++) acc += (double)hq[n] * (double)wd[m * I + n];
        y[m] = (float)acc;
    }
}

/* One token's latent row as the FFN input: bf16 widened to fp32, and in the
 * MX8 mode quantised to MXFP8 along d and decoded again. xc, xs: scratch of
 * d and d/32 bytes. */
static void token_input(const uint16_t *x, int64_t t, int64_t d, int mx8, uint8_t *xc,
                        uint8_t *xs, float *xt)
{
    for (int64_t i = 0; i < d; i++) xt[i] = bf16_bits_to_float(x[t * d + i]);
    if (mx8) {
        oracle_mxfp8_quantize(xt, 1, d, xc, xs);
        oracle_mxfp8_decode(xc, xs, 1, d, xt);
    }
}

/* Scratch for one FFN evaluation. */
typedef struct {
    float *xt, *h, *hq, *y;
    uint8_t *xc, *xs, *hc, *hs;
} ffn_scratch;

static int scratch_alloc(ffn_scratch *sc, int64_t d, int64_t I)
{
    sc->xt = (float *)malloc((size_t)d * sizeof(float));
    sc->h = (float *)malloc((size_t)I * sizeof(float));
    sc->hq = (float *)malloc((size_t)I * sizeof(float));
    sc->y = (float *)malloc((size_t)d * sizeof(float));
    sc->xc = (uint8_t *)malloc((size_t)d);
    sc->xs = (uint8_t *)malloc((size_t)(d / 32 > 0 ? d / 32 : 1));
    sc->hc = (uint8_t *)malloc((size_t)I);
    sc->hs = (uint8_t *)malloc((size_t)(I / 32 > 0 ? I / 32 : 1));
    return (sc->xt && sc->h && sc->hq && sc->y && sc->xc && sc->xs && sc->hc && sc->hs) ? 0 : -1;
}

static void scratch_free(ffn_scratch *sc)
{
    free(sc->xt);
    free(sc->h);
    free(sc->hq);
    free(sc->y);
    free(sc->xc);
    free(sc->xs);
    free(sc->hc);
    free(sc->hs);
}

typedef struct {
    float *wg, *wu, *wd;
} decoded_expert;

static int decode_expert(const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                         const uint8_t *us, const uint8_t *dc, const uint8_t *ds,
                         int64_t le, int64_t d, int64_t I, decoded_expert *out)
{
    out->wg = (float *)malloc((size_t)(I * d) * sizeof(float));
    out->wu = (float *)malloc((size_t)(I * d) * sizeof(float));
    out->wd = (float *)malloc((size_t)(I * d) * sizeof(float));
    if (!out->wg || !out->wu || !out->wd) return -1;
    oracle_mxfp4_decode(gc + le * I * (d / 2), gs + le * I * (d / 32), I, d, out->wg);
    oracle_mxfp4_decode(uc + le * I * (d / 2), us + le * I * (d / 32), I, d, out->wu);
    oracle_mxfp4_decode(dc + le * d * (I / 2), ds + le * d * (I / 32), d, I, out->wd);
    return 0;
}

static void free_expert(decoded_expert *e)
{
    free(e->wg);
    free(e->wu);
    free(e->wd);
}

/* Grouped expert compute over the permuted rows: for local expert le, rows
 * [off[le], off[le+1]) hold tokens perm_token[...]; y[pos, :] is that
 * expert's output for that token (fp32 [A, d]); h is fp32 [A, I].
 * Weight arrays index local experts: gate/up codes [n_local][I][d/2],
 * scales [n_local][I][d/32]; down codes [n_local][d][I/2], scales
 * [n_local][d][I/32]. */
static int expert_compute_impl(const uint16_t *x, int64_t d, int64_t I,
                               const int32_t *off, const int32_t *perm_token, int64_t n_local,
                               const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                               const uint8_t *us, const uint8_t *dc, const uint8_t *ds,
                               int act, int mx8, float *h, float *y)
{
    ffn_scratch sc;
    if (scratch_alloc(&sc, d, I)) {
        scratch_free(&sc);
        return -1;
    }
    for (int64_t le = 0; le < n_local; le++) {
        if (off[le + 1] == off[le]) continue;
        decoded_expert we;
        if (decode_expert(gc, gs, uc, us, dc, ds, le, d, I, &we)) {
            scratch_free(&sc);
            return -1;
        }
        for (int64_t pos = off[le]; pos < off[le + 1]; pos++) {
            token_input(x, perm_token[pos], d, mx8, sc.xc, sc.xs, sc.xt);
            if (mx8) {
                expert_ffn_mx8(sc.xt, we.wg, we.wu, we.wd, d, I, act, sc.h, sc.hc, sc.hs,
                               h + pos * I, y + pos * d);
            } else {
                expert_ffn(sc.xt, we.wg, we.wu, we.wd, d, I, act, h + pos * I, y + pos * d);
            }
        }
        free_expert(&we);
    }
    scratch_free(&sc);
    return 0;
}

int oracle_expert_compute(const uint16_t *x, int64_t d, int64_t I,
                          const int32_t *off, const int32_t *perm_token, int64_t n_local,
                          const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                          const uint8_t *us, const uint8_t *dc, const uint8_t *ds,
                          int act, float *h, float *y)
{
    return expert_compute_impl(x, d, I, off, perm_token, n_local, gc, gs, uc, us, dc, ds, act,
                               0, h, y);
}

/* The MX8 mode of the grouped expert compute; h receives the decoded
 * MXFP8-quantised h that feeds the down projection. */
int oracle_expert_compute_mx8(const uint16_t *x, int64_t d, int64_t I,
                              const int32_t *off, const int32_t *perm_token, int64_t n_local,
                              const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                              const uint8_t *us, const uint8_t *dc, const uint8_t *ds,
                              int act, float *h, float *y)
{
    return expert_compute_impl(x, d, I, off, perm_token, n_local, gc, gs, uc, us, dc, ds, act,
                               1, h, y);
}

/* Combine (P3 §四: results come back weighted; P2 §MoE稀疏激活: the weighted
 * sum of the selected experts' outputs):
 * out[t, m] = sum_{j=0..k-1, inv[t,j] >= 0} w[t,j] * y[inv[t,j], m], in j order.
 * A token with no local assignment gets a zero row. */
void oracle_combine(const float *y, const int32_t *inv, const float *w,
                    int64_t T, int64_t k, int64_t d, float *out)
{
    for (int64_t t = 0; t < T; t++) {
        for (int64_t m = 0; m < d; m++) {
            float acc = 0.0f;
            for (int64_t j = 0; j < k; j++) {
                int32_t r = inv[t * k + j];
                if (r < 0) continue;
                acc += w[t * k + j] * y[(int64_t)r * d + m];
            }
            out[t * d + m] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Whole layer                                                         */
/* ------------------------------------------------------------------ */

/* Route -> dispatch -> expert compute -> combine, in the pages' order
 * (P3 §四: the three MoE steps). If logits_given, `logits` is read instead of
 * computed (so routing can be replayed from another implementation's fp32
 * scores); otherwise it is written. Outputs: out [T, d] fp32, idx/w [T, k],
 * counts [E], off [n_local+1], perm_token [T*k], inv [T, k]. Returns the
 * number of local assignments A, or -1 on allocation failure. */
static int64_t layer_impl(const uint16_t *x, const float *w_router, const float *bias,
                          float *logits, int logits_given,
                          int64_t T, int64_t d, int64_t E, int64_t k, int64_t I,
                          int64_t e0, int64_t n_local,
                          const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                          const uint8_t *us, const uint8_t *dc, const uint8_t *ds, int act,
                          int mx8, int32_t *idx, float *w, int32_t *counts, int32_t *off,
                          int32_t *perm_token, int32_t *inv, float *out)
{
    if (!logits_given) oracle_router_logits(x, w_router, bias, T, d, E, logits);
    oracle_topk_softmax(logits, T, E, k, idx, w);
    oracle_histogram(idx, T, k, E, counts);
    oracle_offsets(counts, e0, n_local, off);
    oracle_permute(idx, off, T, k, e0, n_local, perm_token, inv);
    int64_t A = off[n_local];
    float *h = (float *)malloc((size_t)(A > 0 ? A : 1) * (size_t)I * sizeof(float));
    float *y = (float *)malloc((size_t)(A > 0 ? A : 1) * (size_t)d * sizeof(float));
    if (!h || !y) {
        free(h);
        free(y);
        return -1;
    }
    int rc = expert_compute_impl(x, d, I, off, perm_token, n_local, gc, gs, uc, us, dc, ds,
                                 act, mx8, h, y);
    if (rc == 0) oracle_combine(y, inv, w, T, k, d, out);
    free(h);
    free(y);
    return rc == 0 ? A : -1;
}

/* Route -> dispatch -> expert compute -> combine, in the pages' order
 * (P3 §四: the three MoE steps). If logits_given, `logits` is read instead of
 * computed (so routing can be replayed from another implementation's fp32
 * scores); otherwise it is written. Outputs: out [T, d] fp32, idx/w [T, k],
 * counts [E], off [n_local+1], perm_token [T*k], inv [T, k]. Returns the
 * number of local assignments A, or -1 on allocation failure. */
int64_t oracle_layer(const uint16_t *x, const float *w_router, const float *bias,
                     float *logits, int logits_given,
                     int64_t T, int64_t d, int64_t E, int64_t k, int64_t I,
                     int64_t e0, int64_t n_local,
                     const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                     const uint8_t *us, const uint8_t *dc, const uint8_t *ds, int act,
                     int32_t *idx, float *w, int32_t *counts, int32_t *off,
                     int32_t *perm_token, int32_t *inv, float *out)
{
    return layer_impl(x, w_router, bias, logits, logits_given, T, d, E, k, I, e0, n_local, gc,
                      gs, uc, us, dc, ds, act, 0, idx, w, counts, off, perm_token, inv, out);
}

/* The whole layer in the MX8 mode: routing as above (the router reads the
 * bf16 tokens), expert FFNs as expert_ffn_mx8. */
int64_t oracle_layer_mx8(const uint16_t *x, const float *w_router, const float *bias,
                         float *logits, int logits_given,
                         int64_t T, int64_t d, int64_t E, int64_t k, int64_t I,
                         int64_t e0, int64_t n_local,
                         const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                         const uint8_t *us, const uint8_t *dc, const uint8_t *ds, int act,
                         int32_t *idx, float *w, int32_t *counts, int32_t *off,
                         int32_t *perm_token, int32_t *inv, float *out)
{
    return layer_impl(x, w_router, bias, logits, logits_given, T, d, E, k, I, e0, n_local, gc,
                      gs, uc, us, dc, ds, act, 1, idx, w, counts, off, perm_token, inv, out);
}

/* The same arithmetic for chosen tokens only, given their routing: for each
 * listed token t, out_rows[r, :] = sum_j w[t,j] * FFN_{idx[t,j]}(x[t]) over
 * local experts, in j order. This is what the layer computes for row t,
 * evaluated one token at a time (used where the full layer is too slow). */
static int token_rows_impl(const uint16_t *x, int64_t d, int64_t I, int64_t k,
                           const int32_t *idx, const float *w, const int64_t *tokens,
                           int64_t n_tokens, int64_t e0, int64_t n_local,
                           const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                           const uint8_t *us, const uint8_t *dc, const uint8_t *ds, int act,
                           int mx8, float *out_rows)
{
    ffn_scratch sc;
    if (scratch_alloc(&sc, d, I)) {
        scratch_free(&sc);
        return -1;
    }
    for (int64_t r = 0; r < n_tokens; r++) {
        int64_t t = tokens[r];
        float *o = out_rows + r * d;
        for (int64_t m = 0; m < d; m++) o[m] = 0.0f;
        token_input(x, t, d, mx8, sc.xc, sc.xs, sc.xt);
        for (int64_t j = 0; j < k; j++) {
            int64_t le = (int64_t)idx[t * k + j] - e0;
            if (le < 0 || le >= n_local) continue;
            decoded_expert we;
            if (decode_expert(gc, gs, uc, us, dc, ds, le, d, I, &we)) {
                scratch_free(&sc);
                return -1;
            }
            if (mx8)
                expert_ffn_mx8(sc.xt, we.wg, we.wu, we.wd, d, I, act, sc.h, sc.hc, sc.hs, sc.hq,
                               sc.y);
            else
                expert_ffn(sc.xt, we.wg, we.wu, we.wd, d, I, act, sc.h, sc.y);
            free_expert(&we);
            for (int64_t m = 0; m < d; m++) o[m] += w[t * k + j] * sc.y[m];
        }
    }
    scratch_free(&sc);
    return 0;
}

int oracle_token_rows(const uint16_t *x, int64_t d, int64_t I, int64_t k,
                      const int32_t *idx, const float *w, const int64_t *tokens,
                      int64_t n_tokens, int64_t e0, int64_t n_local,
                      const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                      const uint8_t *us, const uint8_t *dc, const uint8_t *ds, int act,
                      float *out_rows)
{
    return token_rows_impl(x, d, I, k, idx, w, tokens, n_tokens, e0, n_local, gc, gs, uc, us,
                           dc, ds, act, 0, out_rows);
}

int oracle_token_rows_mx8(const uint16_t *x, int64_t d, int64_t I, int64_t k,
                          const int32_t *idx, const float *w, const int64_t *tokens,
                          int64_t n_tokens, int64_t e0, int64_t n_local,
                          const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                          const uint8_t *us, const uint8_t *dc, const uint8_t *ds, int act,
                          float *out_rows)
{
    return token_rows_impl(x, d, I, k, idx, w, tokens, n_tokens, e0, n_local, gc, gs, uc, us,
                           dc, ds, act, 1, out_rows);
}

/* ------------------------------------------------------------------ */
/* LoRA on the MXFP4 base (the low-rank increment of P1 §二 第五层)     */
/* ------------------------------------------------------------------ */

/* A projection with a LoRA delta: the frozen MXFP4 product plus scale times
 * the low-rank increment, whose rank-r factor t = A v is taken first:
 *   out[n] = sum_i v[i] W[n][i] + scale * sum_j t[j] B[n][j],
 *   t[j] = sum_i v[i] A[j][i],
 * in fp32 with sums in increasing index order. A [r][K] and B [N][r] are
 * bf16 (widened exactly); W is decoded fp32 [N][K]. */
static void lora_projection(const float *v, const float *W, const uint16_t *A,
                            const uint16_t *B, int64_t N, int64_t K, int64_t r, float scale,
                            float *t, float *out)
{
    for (int64_t j = 0; j < r; j++) {
        float acc = 0.0f;
        for (int64_t i = 0; i < K; i++) acc += v[i] * bf16_bits_to_float(A[j * K + i]);
        t[j] = acc;
    }
    for (int64_t n = 0; n < N; n++) {
        float base = 0.0f;
        for (int64_t i = 0; i < K; i++) base += v[i] * W[n * K + i];
        float delta = 0.0f;
        for (int64_t j = 0; j < r; j++) delta += t[j] * bf16_bits_to_float(B[n * r + j]);
        out[n] = base + scale * delta;
    }
}

/* One expert's FFN with LoRA on all three projections (adapters of local
 * expert le: gate/up A [r][d], B [I][r]; down A [r][I], B [d][r]). */
static int expert_ffn_lora(const float *xt, const decoded_expert *we, const uint16_t *ga,
                           const uint16_t *gb, const uint16_t *ua, const uint16_t *ub,
                           const uint16_t *da, const uint16_t *db, int64_t le, int64_t d,
                           int64_t I, int64_t r, float scale, int act, float *y)
{
    float *g = (float *)malloc((size_t)I * sizeof(float));
    float *u = (float *)malloc((size_t)I * sizeof(float));
    float *t = (float *)malloc((size_t)(r > 0 ? r : 1) * sizeof(float));
    if (!g || !u || !t) {
        free(g);
        free(u);
        free(t);
        return -1;
    }
    lora_projection(xt, we->wg, ga + le * r * d, gb + le * I * r, I, d, r, scale, t, g);
    lora_projection(xt, we->wu, ua + le * r * d, ub + le * I * r, I, d, r, scale, t, u);
    for (int64_t n = 0; n < I; n++) g[n] = act_apply(act, g[n], u[n]);  /* g becomes h */
    lora_projection(g, we->wd, da + le * r * I, db + le * d * r, d, I, r, scale, t, y);
    free(g);
    free(u);
    free(t);
    return 0;
}

/* The whole layer with LoRA adapters on every local expert's three
 * projections (rank r, one scale), otherwise as oracle_layer. Adapters
 * index local experts: gate_a/up_a [n_local][r][d], gate_b/up_b
 * [n_local][I][r], down_a [n_local][r][I], down_b [n_local][d][r], bf16. */
int64_t oracle_layer_lora(const uint16_t *x, const float *w_router, const float *bias,
                          float *logits, int logits_given,
                          int64_t T, int64_t d, int64_t E, int64_t k, int64_t I,
                          int64_t e0, int64_t n_local,
                          const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                          const uint8_t *us, const uint8_t *dc, const uint8_t *ds, int act,
                          const uint16_t *ga, const uint16_t *gb, const uint16_t *ua,
                          const uint16_t *ub, const uint16_t *da, const uint16_t *db, int64_t r,
                          float scale, int32_t *idx, float *w, int32_t *counts, int32_t *off,
                          int32_t *perm_token, int32_t *inv, float *out)
{
    if (!logits_given) oracle_router_logits(x, w_router, bias, T, d, E, logits);
    oracle_topk_softmax(logits, T, E, k, idx, w);
    oracle_histogram(idx, T, k, E, counts);
    oracle_offsets(counts, e0, n_local, off);
    oracle_permute(idx, off, T, k, e0, n_local, perm_token, inv);
    int64_t A = off[n_local];
    float *y = (float *)malloc((size_t)(A > 0 ? A : 1) * (size_t)d * sizeof(float));
    float *xt = (float *)malloc((size_t)d * sizeof(float));
    if (!y || !xt) {
        free(y);
        free(xt);
        return -1;
    }
    int rc = 0;
    for (int64_t le = 0; le < n_local && rc == 0; le++) {
        if (off[le + 1] == off[le]) continue;
        decoded_expert we;
        if (decode_expert(gc, gs, uc, us, dc, ds, le, d, I, &we)) {
            rc = -1;
            break;
        }
        for (int64_t pos = off[le]; pos < off[le + 1] && rc == 0; pos++) {
            int64_t tk = perm_token[pos];
            for (int64_t i = 0; i < d; i++) xt[i] = bf16_bits_to_float(x[tk * d + i]);
            rc = expert_ffn_lora(xt, &we, ga, gb, ua, ub, da, db, le, d, I, r, scale, act,
                                 y + pos * d);
        }
        free_expert(&we);
    }
    if (rc == 0) oracle_combine(y, inv, w, T, k, d, out);
    free(y);
    free(xt);
    return rc == 0 ? A : -1;
}

/* The LoRA layer's output for chosen tokens only, given their routing: as
 * oracle_token_rows, with each selected local expert's FFN carrying its
 * adapters (expert_ffn_lora). Used where the whole LoRA layer is too slow. */
int oracle_token_rows_lora(const uint16_t *x, int64_t d, int64_t I, int64_t k,
                           const int32_t *idx, const float *w, const int64_t *tokens,
                           int64_t n_tokens, int64_t e0, int64_t n_local,
                           const uint8_t *gc, const uint8_t *gs, const uint8_t *uc,
                           const uint8_t *us, const uint8_t *dc, const uint8_t *ds, int act,
                           const uint16_t *ga, const uint16_t *gb, const uint16_t *ua,
                           const uint16_t *ub, const uint16_t *da, const uint16_t *db, int64_t r,
                           float scale, float *out_rows)
{
    ffn_scratch sc;
    if (scratch_alloc(&sc, d, I)) {
        scratch_free(&sc);
        return -1;
    }
    int rc = 0;
    for (int64_t q = 0; q < n_tokens && rc == 0; q++) {
        int64_t t = tokens[q];
        float *o = out_rows + q * d;
        for (int64_t m = 0; m < d; m++) o[m] = 0.0f;
        token_input(x, t, d, 0, sc.xc, sc.xs, sc.xt);
        for (int64_t j = 0; j < k && rc == 0; j++) {
            int64_t le = (int64_t)idx[t * k + j] - e0;
            if (le < 0 || le >= n_local) continue;
            decoded_expert we;
            if (decode_expert(gc, gs, uc, us, dc, ds, le, d, I, &we)) {
                rc = -1;
                break;
            }
            rc = expert_ffn_lora(sc.xt, &we, ga, gb, ua, ub, da, db, le, d, I, r, scale, act,
                                 sc.y);
            free_expert(&we);
            if (rc == 0)
                for (int64_t m = 0; m < d; m++) o[m] += w[t * k + j] * sc.y[m];
        }
    }
    scratch_free(&sc);
    return rc;
}
