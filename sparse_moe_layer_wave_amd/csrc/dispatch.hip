// Dispatch order: a stable counting sort of the T*k (token, slot) pairs by
// expert.  Rows of one expert are contiguous, in ascending token order, which
// is the grouping the per-expert loop of "DeepSeek V4-Flash architecture Q&A"
// (Q8.4) performs, laid out so one grouped GEMM launch covers every expert.
//
// Tokens are cut into routing blocks of 64.  The router's top-k kernel already
// counted, per block, the pairs of every expert (popcount of a 64-bit token
// mask held in LDS).  Here:
//   k_block_scan   one workgroup per expert: exclusive scan of its per-block
//                  counts -> base of each block inside the expert; total count;
//   k_offsets      one workgroup: exclusive scan of the counts -> offsets, and
//                  of the per-expert M-tile counts of the grouped GEMMs;
//   k_scatter      one workgroup per routing block: rebuilds the token masks
//                  and gives pair (t, j) of expert e the row
//                  offsets[e] + base[e, block] + #(tokens of the block before t
//                  that chose e).
// A batch of one routing block (T <= 64) does all three in one workgroup
// (k_dispatch_one).  All of it is integer work with no atomics whose order
// matters, so the result is the same on every run.
//
// A routing the caller supplies (hy3moe_permute) is checked as it is read
// (the CHECKED instances): a pair whose expert is outside [0, E), or repeats
// an expert listed earlier for the same token, takes no row (row_of = -1) and
// is counted for no expert.  The router's own routing needs no check.  With the shared expert of the full block
// ("Tencent Hy3-Flash Q&A", Q4.7), it becomes expert E, whose rows are
// T*k + t, one per token: the GEMMs then treat it like any routed expert.

#include "internal.h"

namespace hy3 {
namespace {

// Whether pair j of a token row is dispatched: always for the router's own
// routing; for a caller's, only an expert in [0, E) not listed earlier in the
// row.
template <bool CHECKED>
__device__ __forceinline__ bool pair_ok(const int32_t* __restrict__ row, int j, int e, int E) {
    if constexpr (!CHECKED) return true;
    if (e < 0 || e >= E) return false;
    for (int i = 0; i < j; ++i)
        if (row[i] == e) return false;
    return true;
}

// Exclusive scan over one workgroup of 256 threads; returns the total.
__device__ int block_exclusive_scan(int v, int* lds /* >= 256 + 1 ints */, int& excl) {
    const int tid = threadIdx.x;
    lds[tid] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int add = tid >= off ? lds[tid - off] : 0;
        __syncthreads();
        lds[tid] += add;
        __syncthreads();
    }
    const int incl = lds[tid];
    const int total = lds[255];
    __syncthreads();
    excl = incl - v;
    return total;
}

__global__ __launch_bounds__(256) void k_block_scan(const int32_t* __restrict__ blk_counts,
                                                   int32_t* __restrict__ blk_base,
                                                   int32_t* __restrict__ counts, int nb) {
    __shared__ int lds[256];
    const int e = blockIdx.x;
    const int32_t* c = blk_counts + static_cast<size_t>(e) * nb;
    int32_t* b = blk_base + static_cast<size_t>(e) * nb;
    int running = 0;
    for (int base = 0; base < nb; base += 256 * 4) {
        int v[4];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = base + threadIdx.x * 4 + i;
            v[i] = p < nb ? c[p] : 0;
            sum += v[i];
        }
        int excl;
        const int total = block_exclusive_scan(sum, lds, excl);
        int acc = running + excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = base + threadIdx.x * 4 + i;
            if (p < nb) b[p] = acc;
            acc += v[i];
        }
        running += total;
    }
    if (threadIdx.x == 0) counts[e] = running;
}

// One workgroup of 1024 threads over n = E (+1 with a shared expert, whose
// count is `extra`) <= 1024 experts.  offsets = exclusive scan of the counts;
// tile_off = exclusive scan of ceil(count / bm), the row blocks of the grouped
// GEMMs.
__global__ __launch_bounds__(1024) void k_offsets(const int32_t* __restrict__ counts, int E,
                                                  int extra, int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ tile_off, int bm,
                                                  int32_t* __restrict__ zero, int nzero) {
    __shared__ int s_cnt[1024];
    __shared__ int s_til[1024];
    const int tid = threadIdx.x;
    for (int i = tid; i < nzero; i += 1024) zero[i] = 0;
    const int n = E + (extra > 0 ? 1 : 0);
    const int c = tid < E ? counts[tid] : (tid < n ? extra : 0);
    const int nt = (c + bm - 1) / bm;
    s_cnt[tid] = c;
    s_til[tid] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int a0 = tid >= off ? s_cnt[tid - off] : 0;
        const int a1 = tid >= off ? s_til[tid - off] : 0;
        __syncthreads();
        s_cnt[tid] += a0;
        s_til[tid] += a1;
        __syncthreads();
    }
    if (tid < n) {
        offsets[tid] = s_cnt[tid] - c;
        tile_off[tid] = s_til[tid] - nt;
    }
    if (tid == 0) {
        offsets[n] = s_cnt[1023];
        tile_off[n] = s_til[1023];
    }
}

// shared_row0 >= 0: the shared expert's rows start there, one per token in
// token order.
template <bool CHECKED>
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ idx, int T, int E,
                                                int k, int nb,
                                                const int32_t* __restrict__ blk_base,
                                                const int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ row_of,
                                                int32_t* __restrict__ tok_of, int shared_row0) {
    __shared__ unsigned long long mask[1024];
    for (int e = threadIdx.x; e < E; e += 256) mask[e] = 0ull;
    __syncthreads();
    const int b = blockIdx.x;
    const int npairs = kRouteBlock * k;
    for (int p = threadIdx.x; p < npairs; p += 256) {
        const int tl = p / k;
        const int t = b * kRouteBlock + tl;
        if (t < T) {
            const int32_t* row = idx + static_cast<size_t>(t) * k;
            const int e = row[p - tl * k];
            if (pair_ok<CHECKED>(row, p - tl * k, e, E)) atomicOr(&mask[e], 1ull << tl);
        }
    }
    __syncthreads();
    for (int p = threadIdx.x; p < npairs; p += 256) {
        const int tl = p / k;
        const int t = b * kRouteBlock + tl;
        if (t < T) {
            const size_t pair = static_cast<size_t>(t) * k + (p - tl * k);
            const int e = idx[pair];
            if (!pair_ok<CHECKED>(idx + static_cast<size_t>(t) * k, p - tl * k, e, E)) {
                row_of[pair] = -1;
                continue;
            }
            const int rank = __popcll(mask[e] & ((1ull << tl) - 1ull));
            const int row = offsets[e] + blk_base[static_cast<size_t>(e) * nb + b] + rank;
            row_of[pair] = row;
            tok_of[row] = t;
        }
    }
    if (shared_row0 >= 0) {
        for (int tl = threadIdx.x; tl < kRouteBlock; tl += 256) {
            const int t = b * kRouteBlock + tl;
            if (t < T) tok_of[shared_row0 + t] = t;
        }
    }
}

// A single routing block (T <= 64): counts, offsets, tile offsets and the
// dispatch order in one workgroup of 1024 threads, the same results as
// k_block_scan + k_offsets + k_scatter with nb = 1 (every block base is 0).
template <bool CHECKED>
__global__ __launch_bounds__(1024) void k_dispatch_one(const int32_t* __restrict__ idx, int T, int E,
                                                      int k, int extra, int bm,
                                                      int32_t* __restrict__ blk_base,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ tile_off,
                                                      int32_t* __restrict__ row_of,
                                                      int32_t* __restrict__ tok_of, int shared_row0,
                                                      int32_t* __restrict__ zero, int nzero) {
    __shared__ unsigned long long mask[1024];
    __shared__ int s_cnt[1024];
    __shared__ int s_til[1024];
    __shared__ int s_off[1024];
    const int tid = threadIdx.x;
    for (int i = tid; i < nzero; i += 1024) zero[i] = 0;
    mask[tid] = 0ull;
    __syncthreads();
    const int npairs = T * k;
    for (int p = tid; p < npairs; p += 1024) {
        const int t = p / k;
        const int e = idx[p];
        if (pair_ok<CHECKED>(idx + static_cast<size_t>(t) * k, p - t * k, e, E)) atomicOr(&mask[e], 1ull << t);
    }
    __syncthreads();
    const int n = E + (extra > 0 ? 1 : 0);
    const int c = tid < E ? __popcll(mask[tid]) : (tid < n ? extra : 0);
    const int nt = (c + bm - 1) / bm;
    s_cnt[tid] = c;
    s_til[tid] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int a0 = tid >= off ? s_cnt[tid - off] : 0;
        const int a1 = tid >= off ? s_til[tid - off] : 0;
        __syncthreads();
        s_cnt[tid] += a0;
        s_til[tid] += a1;
        __syncthreads();
    }
    s_off[tid] = s_cnt[tid] - c;
    if (tid < E) {
        counts[tid] = c;
        blk_base[tid] = 0;
    }
    if (tid < n) {
        offsets[tid] = s_cnt[tid] - c;
        tile_off[tid] = s_til[tid] - nt;
    }
    if (tid == 0) {
        offsets[n] = s_cnt[1023];
        tile_off[n] = s_til[1023];
    }
    __syncthreads();
    for (int p = tid; p < npairs; p += 1024) {
        const int t = p / k;
        const int e = idx[p];
        if (!pair_ok<CHECKED>(idx + static_cast<size_t>(t) * k, p - t * k, e, E)) {
            row_of[p] = -1;
            continue;
        }
        const int row = s_off[e] + __popcll(mask[e] & ((1ull << t) - 1ull));
        row_of[p] = row;
        tok_of[row] = t;
    }
    if (shared_row0 >= 0 && tid < T) tok_of[shared_row0 + tid] = tid;
}

// Per-block counts when the routing comes from the caller (hy3moe_permute),
// checked as k_scatter<true> checks it.
__global__ __launch_bounds__(256) void k_block_counts(const int32_t* __restrict__ idx, int T,
                                                     int E, int k, int nb,
                                                     int32_t* __restrict__ blk_counts) {
    __shared__ int cnt[1024];
    for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
    __syncthreads();
    const int b = blockIdx.x;
    for (int p = threadIdx.x; p < kRouteBlock * k; p += 256) {
        const int t = b * kRouteBlock + p / k;
        if (t < T) {
            const int32_t* row = idx + static_cast<size_t>(t) * k;
            const int e = row[p % k];
            if (pair_ok<true>(row, p % k, e, E)) atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
        blk_counts[static_cast<size_t>(e) * nb + b] = cnt[e];
}

}  // namespace

hipError_t launch_block_counts(const int32_t* idx, int T, int E, int k, int nb,
                               int32_t* blk_counts, hipStream_t s) {
    hipLaunchKernelGGL(k_block_counts, dim3(nb), dim3(256), 0, s, idx, T, E, k, nb, blk_counts);
    return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* idx, int T, int E, int k, int nb,
                           const int32_t* blk_counts, int32_t* blk_base, int32_t* counts,
                           int32_t* offsets, int32_t* tile_off, int bm, int32_t* row_of,
                           int32_t* tok_of, int shared, hipStream_t s, bool checked,
                           int32_t* zero, int nzero) {
    if (nb == 1) {
        auto kern = checked ? k_dispatch_one<true> : k_dispatch_one<false>;
        hipLaunchKernelGGL(kern, dim3(1), dim3(1024), 0, s, idx, T, E, k, shared ? T : 0, bm,
                           blk_base, counts, offsets, tile_off, row_of, tok_of, shared ? T * k : -1,
                           zero, nzero);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_block_scan, dim3(E), dim3(256), 0, s, blk_counts, blk_base, counts, nb);
    hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, s, counts, E, shared ? T : 0, offsets,
                       tile_off, bm, zero, nzero);
    auto scatter = checked ? k_scatter<true> : k_scatter<false>;
    hipLaunchKernelGGL(scatter, dim3(nb), dim3(256), 0, s, idx, T, E, k, nb, blk_base, offsets,
                       row_of, tok_of, shared ? T * k : -1);
    return hipGetLastError();
}

}  // namespace hy3
