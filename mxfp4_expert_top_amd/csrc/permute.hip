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
// block's base row per expert (relative to the expert's first row) and the
// expert's total; every scatter block scans the totals for the experts' first
// rows. No step depends on atomic ordering, so the permutation is the same on
// every run.
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

// Column scan over the blocks, many workgroups: workgroup x takes local
// experts 64 x .. 64 x + 63 and 16 thread groups, group g summing a
// contiguous run of the blocks (loads coalesced across the 64 experts, 16 of a
// run in flight at a time); the runs' sums meet in LDS. In place, blk[b][e]
// becomes block b's first row for expert e counted from the expert's first
// row, and tot[e] the expert's rows. (One workgroup scanning every expert's
// column took 81 us at 256 blocks, its per-expert chain of loads being the
// whole kernel.)
constexpr int CS_E = 64, CS_G = 16, CS_CHUNK = 16;

__global__ __launch_bounds__(CS_E * CS_G) void permute_colscan_kernel(int nl, int nblk,
                                                                      int32_t *__restrict__ blk,
                                                                      int32_t *__restrict__ tot)
{
    __shared__ int32_t part[CS_G][CS_E];
    const int el = threadIdx.x % CS_E, g = threadIdx.x / CS_E;
    const int e = blockIdx.x * CS_E + el;
    const int per = (nblk + CS_G - 1) / CS_G;
    const int b0 = min(g * per, nblk), b1 = min(b0 + per, nblk);
    int sum = 0;
    if (e < nl)
        for (int c = b0; c < b1; c += CS_CHUNK) {
            int v[CS_CHUNK];
#pragma unroll
            for (int i = 0; i < CS_CHUNK; i++)
                v[i] = c + i < b1 ? blk[(int64_t)(c + i) * nl + e] : 0;
#pragma unroll
            for (int i = 0; i < CS_CHUNK; i++) sum += v[i];
        }
    part[g][el] = sum;
    __syncthreads();
    int run = 0, all = 0;
#pragma unroll
    for (int h = 0; h < CS_G; h++) {
        const int t = part[h][el];
        run += h < g ? t : 0;
        all += t;
    }
    if (e >= nl) return;
    if (g == 0) tot[e] = all;
    // the run's counts again (its own, unchanged so far), then its bases
    for (int c = b0; c < b1; c += CS_CHUNK) {
        int v[CS_CHUNK];
#pragma unroll
        for (int i = 0; i < CS_CHUNK; i++) v[i] = c + i < b1 ? blk[(int64_t)(c + i) * nl + e] : 0;
#pragma unroll
        for (int i = 0; i < CS_CHUNK; i++)
            if (c + i < b1) {
                blk[(int64_t)(c + i) * nl + e] = run;
                run += v[i];
            }
    }
}

__global__ __launch_bounds__(PERM_TB) void permute_scatter_kernel(
    const int32_t *__restrict__ idx, int T, int k, int e0, int nl,
    const int32_t *__restrict__ base, const int32_t *__restrict__ tot, int32_t *__restrict__ off,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv)
{
    extern __shared__ uint32_t bits[];
    __shared__ int32_t part[16];
    __shared__ int32_t soff[MOE_MAX_EXPERTS_DEV];
    const int t0 = blockIdx.x * PERM_TB;
    // the local experts' first rows: an exclusive scan of their totals, each
    // thread owning a run of at most 8 consecutive experts (nl <= 2048);
    // block 0 also writes them out
    {
        constexpr int RUN = MOE_MAX_EXPERTS_DEV / PERM_TB;
        const int per = (nl + PERM_TB - 1) / PERM_TB;
        const int lo = threadIdx.x * per;
        int c[RUN], sum = 0;
#pragma unroll
        for (int i = 0; i < RUN; i++) {
            c[i] = i < per && lo + i < nl ? tot[lo + i] : 0;
            sum += c[i];
        }
        int total;
        int run = block_exclusive_scan(sum, part, total);
#pragma unroll
        for (int i = 0; i < RUN; i++)
            if (i < per && lo + i < nl) {
                soff[lo + i] = run;
                if (blockIdx.x == 0) off[lo + i] = run;
                run += c[i];
            }
        if (blockIdx.x == 0 && threadIdx.x == 0) off[nl] = total;
    }
    build_bitmap(bits, idx, T, k, e0, nl, t0);  // its barriers publish soff
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
                int64_t p = (int64_t)soff[le] + base[(int64_t)blockIdx.x * nl + le] + rank;
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

// block counts [blocks][num_local], then the experts' totals [num_local]
size_t permute_ws_bytes(int T, int num_local)
{
    size_t n = ((size_t)perm_blocks(T) + 1) * (size_t)num_local * sizeof(int32_t);
    return (n + 255) & ~(size_t)255;
}

hipError_t launch_permute(const int32_t *idx, const int32_t *counts, int T, int k, int e0,
                          int num_local, int32_t *off, int32_t *perm, int32_t *inv, void *ws,
                          hipStream_t s, const GemmPlanArgs *plan)
{
    const int nblk = perm_blocks(T);
    int32_t *blk = (int32_t *)ws;
    int32_t *tot = blk + (size_t)nblk * num_local;
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
    // (more than one block: the rows are counted from the dispatch bitmaps,
    // which give the histogram's offsets for any consistent `counts`)
    if (nblk > 0) {
        hipLaunchKernelGGL(permute_count_kernel, dim3(nblk), dim3(PERM_TB), lds, s, idx, T, k, e0,
                           num_local, blk);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(permute_colscan_kernel, dim3((num_local + CS_E - 1) / CS_E),
                           dim3(CS_E * CS_G), 0, s, num_local, nblk, blk, tot);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(permute_scatter_kernel, dim3(nblk), dim3(PERM_TB), lds, s, idx, T, k,
                           e0, num_local, (const int32_t *)blk, (const int32_t *)tot, off, perm,
                           inv);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        e = launch_fill_i32(off, (int64_t)num_local + 1, 0, s);  // no tokens: no rows
        if (e != hipSuccess) return e;
    }
    if (plan) return launch_gemm_plan_into(off, num_local, *plan, s);
    return hipSuccess;
}

}  // namespace moe
