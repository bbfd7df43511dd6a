// Dispatch planning on one GPU (P3 "Kimi K3 Day-0 适配剖析", section 四: the
// index computation and buffer planning of dispatch, re-done for 896 experts
// and top-16): expert offsets and a deterministic stable counting sort of the
// row-major (token, slot) list by expert.
//
// A token selects k distinct experts, so inside one expert's segment the rows
// are exactly the tokens that chose it, in increasing token order. Tokens are
// cut into blocks of PERM_TB; per block an LDS bitmap bits[expert][token] is
// built with integer ORs (order-independent). Popcounts of the bitmap give
// (a) each block's per-expert count, and (b) each assignment's rank among the
// earlier tokens of its block. A column scan over blocks turns (a) into each
// block's base row per expert. No step depends on atomic ordering, so the
// permutation is the same on every run.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int PERM_WORDS = PERM_TB / 32;  // bitmap words per expert

__device__ __forceinline__ void build_bitmap(uint32_t *bits, const int32_t *__restrict__ idx,
                                             int T, int k, int e0, int nl, int t0)
{
    for (int i = threadIdx.x; i < nl * PERM_WORDS; i += blockDim.x) bits[i] = 0u;
    __syncthreads();
    const int tl = threadIdx.x;
    const int t = t0 + tl;
    if (t < T) {
        int le[MOE_MAX_TOPK_DEV];
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK_DEV; j++)
            if (j < k) le[j] = idx[(int64_t)t * k + j] - e0;
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK_DEV; j++)
            if (j < k && le[j] >= 0 && le[j] < nl)
                atomicOr(&bits[le[j] * PERM_WORDS + tl / 32], 1u << (tl % 32));
    }
    __syncthreads();
}

__global__ __launch_bounds__(PERM_TB) void permute_count_kernel(
    const int32_t *__restrict__ idx, int T, int k, int e0, int nl, int32_t *__restrict__ blk)
{
    extern __shared__ uint32_t bits[];
    build_bitmap(bits, idx, T, k, e0, nl, blockIdx.x * PERM_TB);
    for (int le = threadIdx.x; le < nl; le += blockDim.x) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < PERM_WORDS; w++) c += __popc(bits[le * PERM_WORDS + w]);
        blk[(int64_t)blockIdx.x * nl + le] = c;
    }
}

// One workgroup: offsets over the local range, then per expert a scan of the
// block counts (in place: blk[b][e] becomes block b's first row for e).
// Expert counts come from `counts` (the histogram) or, when it is NULL, from
// the block counts themselves. Loading one block count at a time, each load
// behind the previous store, took 93 us at 256 blocks; one wave per expert
// (lanes over blocks) was slower still, 16 waves walking 896 experts.
__global__ __launch_bounds__(1024) void permute_scan_kernel(
    const int32_t *__restrict__ counts, int e0, int nl, int nblk, int32_t *__restrict__ off,
    int32_t *__restrict__ blk)
{
    __shared__ int32_t part[16];
    const int tid = threadIdx.x;
    // each thread owns a contiguous run of at most two experts (nl <= 2048)
    const int per = (nl + 1023) / 1024;
    const int lo = tid * per, hi = min(lo + per, nl);
    auto count = [&](int i) {
        if (counts) return counts[e0 + i];
        int c = 0;
        for (int b = 0; b < nblk; b++) c += blk[(int64_t)b * nl + i];
        return c;
    };
    const int c0 = lo < hi ? count(lo) : 0, c1 = lo + 1 < hi ? count(lo + 1) : 0;
    int total;
    const int run = block_exclusive_scan(c0 + c1, part, total);  // exclusive prefix of the run
    if (lo < hi) off[lo] = run;
    if (lo + 1 < hi) off[lo + 1] = run + c0;
    if (tid == 0) off[nl] = total;
    __syncthreads();
    // thread per expert (loads coalesce across experts); each chunk of block
    // counts is loaded before its stores, so 16 loads are in flight per wait
    for (int le = tid; le < nl; le += 1024) {
        int r = off[le];
        for (int b0 = 0; b0 < nblk; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; i++) c[i] = b0 + i < nblk ? blk[(int64_t)(b0 + i) * nl + le] : 0;
#pragma unroll
            for (int i = 0; i < 16; i++)
                if (b0 + i < nblk) {
                    blk[(int64_t)(b0 + i) * nl + le] = r;
                    r += c[i];
                }
        }
    }
}

__global__ __launch_bounds__(PERM_TB) void permute_scatter_kernel(
    const int32_t *__restrict__ idx, int T, int k, int e0, int nl,
    const int32_t *__restrict__ base, int32_t *__restrict__ perm, int32_t *__restrict__ inv)
{
    extern __shared__ uint32_t bits[];
    const int t0 = blockIdx.x * PERM_TB;
    build_bitmap(bits, idx, T, k, e0, nl, t0);
    const int tl = threadIdx.x, t = t0 + tl;
    if (t >= T) return;
    const int64_t cap = (int64_t)T * k;
    const int w = tl / 32;
    const uint32_t below = (1u << (tl % 32)) - 1u;
    int lej[MOE_MAX_TOPK_DEV];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK_DEV; j++)
        if (j < k) lej[j] = idx[(int64_t)t * k + j] - e0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK_DEV; j++) {
        if (j < k) {
            const int le = lej[j];
            int pos = -1;
            if (le >= 0 && le < nl) {
                const uint32_t *row = bits + le * PERM_WORDS;
                int rank = __popc(row[w] & below);
                for (int i = 0; i < w; i++) rank += __popc(row[i]);
                int64_t p = (int64_t)base[(int64_t)blockIdx.x * nl + le] + rank;
                if (p >= 0 && p < cap) {
                    pos = (int)p;
                    perm[pos] = t;
                }
            }
            inv[(int64_t)t * k + j] = pos;
        }
    }
}

// Small batches (T <= PERM_TB): the whole plan in one workgroup -- bitmap,
// offsets, ranks and, when `plan` is given, the grouped-GEMM work list
// (groups of R rows, as gemm_plan_kernel builds it). One thread per
// (token, slot) assignment, all of a thread's index loads issued together.
constexpr int PS_PER = PERM_TB * MOE_MAX_TOPK_DEV / 1024;  // assignments per thread

__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ counts, int T, int k, int e0,
    int nl, int32_t *__restrict__ off, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int R, int max_groups, int balanced, int32_t *__restrict__ plan, int plan_hdr)
{
    extern __shared__ uint32_t bits[];  // nl * PERM_WORDS
    __shared__ int32_t part[16];
    __shared__ int32_t soff[MOE_MAX_EXPERTS_DEV + 1];
    const int tid = threadIdx.x;
    const int A = T * k;
    int le[PS_PER];
    if (A > 0) {
#pragma unroll
        for (int u = 0; u < PS_PER; u++) le[u] = idx[min(tid + 1024 * u, A - 1)] - e0;
    }
#pragma unroll
    for (int u = 0; u < PS_PER; u++)
        if (A == 0 || tid + 1024 * u >= A || le[u] < 0 || le[u] >= nl) le[u] = -1;
    for (int i = tid; i < nl * PERM_WORDS; i += 1024) bits[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PS_PER; u++) {
        if (le[u] < 0) continue;
        const int t = (tid + 1024 * u) / k;
        atomicOr(&bits[le[u] * PERM_WORDS + t / 32], 1u << (t % 32));
    }
    // offsets: each thread owns two consecutive local experts (nl <= 2048);
    // counts from the histogram or, when it is NULL, from the bitmap
    const int i0 = 2 * tid;
    if (!counts) __syncthreads();  // the bitmap is complete
    auto count = [&](int i) {
        if (i >= nl) return 0;
        if (counts) return (int)counts[e0 + i];
        int c = 0;
#pragma unroll
        for (int w = 0; w < PERM_WORDS; w++) c += __popc(bits[i * PERM_WORDS + w]);
        return c;
    };
    const int c0 = count(i0), c1 = count(i0 + 1);
    int total;
    const int ex = block_exclusive_scan(c0 + c1, part, total);  // also orders the bitmap ORs
    if (i0 < nl) soff[i0] = ex;
    if (i0 + 1 < nl) soff[i0 + 1] = ex + c0;
    if (tid == 0) soff[nl] = total;
    __syncthreads();
    for (int i = tid; i <= nl; i += 1024) off[i] = soff[i];
    const int64_t cap = (int64_t)A;
#pragma unroll
    for (int u = 0; u < PS_PER; u++) {
        const int a = tid + 1024 * u;
        if (a < A) {
            const int t = a / k;
            int pos = -1;
            if (le[u] >= 0) {
                const uint32_t *row = bits + le[u] * PERM_WORDS;
                const int w = t / 32;
                int rank = __popc(row[w] & ((1u << (t % 32)) - 1u));
                for (int i = 0; i < w; i++) rank += __popc(row[i]);
                const int64_t p = (int64_t)soff[le[u]] + rank;
                if (p < cap) {
                    pos = (int)p;
                    perm[pos] = t;
                }
            }
            inv[a] = pos;
        }
    }
    if (!plan) return;
    // grouped-GEMM work list: ceil(count / R) groups per expert, expert-major
    const int g0 = i0 < nl ? (c0 + R - 1) / R : 0, g1 = i0 + 1 < nl ? (c1 + R - 1) / R : 0;
    int ngroups;
    int pos = block_exclusive_scan(g0 + g1, part, ngroups);
    int2 *items = (int2 *)(plan + plan_hdr);
    for (int h = 0; h < 2; h++) {
        const int i = i0 + h;
        if (i >= nl) break;
        const int c = h ? c1 : c0, g = (c + R - 1) / R;
        for (int j = 0; j < g; j++, pos++)
            if (pos < max_groups) items[pos] = plan_item(i, soff[i], c, g, j, R, balanced);
    }
    if (tid == 0) plan[0] = min(ngroups, max_groups);
}

size_t permute_ws_bytes(int T, int num_local)
{
    size_t n = (size_t)perm_blocks(T) * (size_t)num_local * sizeof(int32_t);
    return (n + 255) & ~(size_t)255;
}

hipError_t launch_permute(const int32_t *idx, const int32_t *counts, int T, int k, int e0,
                          int num_local, int32_t *off, int32_t *perm, int32_t *inv, void *ws,
                          hipStream_t s, const GemmPlanArgs *plan)
{
    const int nblk = perm_blocks(T);
    int32_t *blk = (int32_t *)ws;
    const size_t lds = (size_t)num_local * PERM_WORDS * sizeof(uint32_t);
    hipError_t e;
    if (nblk == 1 && num_local <= 1024) {  // bitmap <= 32 KB of LDS
        hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), lds, s, idx, counts, T, k, e0,
                           num_local, off, perm, inv, plan ? plan->rows_per_group : 0,
                           plan ? plan->max_groups : 0, plan ? plan->balanced : 0,
                           plan ? plan->plan : nullptr,
                           plan ? plan->hdr : 0);
        return hipGetLastError();
    }
    if (nblk > 0) {
        hipLaunchKernelGGL(permute_count_kernel, dim3(nblk), dim3(PERM_TB), lds, s, idx, T, k, e0,
                           num_local, blk);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, counts, e0, num_local,
                       nblk, off, blk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nblk > 0) {
        hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(PERM_TB), lds, s, idx, T, k,
                           e0, num_local, (const int32_t *)blk, perm, inv);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (plan) return launch_gemm_plan_into(off, num_local, *plan, s);
    return hipSuccess;
}

}  // namespace moe
