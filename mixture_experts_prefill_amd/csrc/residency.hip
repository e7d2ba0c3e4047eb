// Residency of experts by use, on the GPU.
//
// The experts.rs page (fn prepare_expert_jobs) keeps a layer's most-used
// experts resident: the non-empty experts sorted by descending row count
// (a stable sort, so ties keep ascending expert id), the first `budget` of
// them kept, the rest streamed through the ring.  The decode.rs page
// (fn lookahead_layer) looks one block ahead: while a block runs, the next
// layer's experts are predicted so they can be fetched early.
//
// Both kernels below order the experts in one workgroup of 1024 threads:
// expert e with row count c gets the 64-bit key c * 2^10 + (1023 - e), unique
// and larger for more rows, then for a lower id, so the keys in descending
// order (a bitonic network in LDS over the next power of two >= E, padded
// with zero keys) list the experts by count descending, ties in ascending
// id: the pages' stable order.  The non-empty experts come first.
// The row counts come from the grouping's offsets (this block) or from a
// top-k (the next layer's router run on this block's input, for the
// lookahead).  Exact integer work: the result does not depend on timing.
// Up to 256 experts a direct count of the larger keys per expert is cheaper
// than the sort's barriers; beyond, ranking every expert against all others
// (E^2 compares) took 15-40 us at E = 512-1024 against about 9-15 for the
// sort.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr uint64_t kIdBits = 10;
static_assert(MOE_MAX_EXPERTS <= (1 << kIdBits), "expert ids fit the key's low bits");

__device__ __forceinline__ uint64_t expert_key(uint32_t c, int e) {
    return ((uint64_t)c << kIdBits) | (uint64_t)(MOE_MAX_EXPERTS - 1 - e);
}
__device__ __forceinline__ int key_expert(uint64_t k) { return MOE_MAX_EXPERTS - 1 - (int)(k & ((1u << kIdBits) - 1)); }
__device__ __forceinline__ uint32_t key_count(uint64_t k) { return (uint32_t)(k >> kIdBits); }

// Sorts key[0 .. N) descending, N a power of two with 64 <= N <= 1024, with
// all 1024 threads of the workgroup (every thread reaches every barrier).
// Thread i keeps element i in registers; at stage (k, j) it takes the larger
// or the smaller of its element and that of thread i ^ j (the larger when its
// block of k is descending and it is the lower of the pair, or ascending and
// the upper).  Partners closer than 64 are in the same wave and exchange by
// cross-lane shuffle; farther ones through LDS between two barriers.
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void sort_desc(uint64_t *key, int N) {
    const int tid = threadIdx.x;
    uint64_t mine = tid < N ? key[tid] : 0ull;
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            uint64_t other;
            if (j >= 64) {
                if (tid < N) key[tid] = mine;
                __syncthreads();
                other = tid < N ? key[tid ^ j] : 0ull;
                __syncthreads();
            } else {
                other = shfl_xor64(mine, j);
            }
            const bool take_max = ((tid & k) == 0) == ((tid & j) == 0);
            mine = take_max ? (mine > other ? mine : other) : (mine < other ? mine : other);
        }
    }
    if (tid < N) key[tid] = mine;
    __syncthreads();
}

__device__ __forceinline__ int pow2_at_least(int E) {
    int N = 1;
    while (N < E) N <<= 1;
    return N;
}

// rank_of[e] = position of expert e in the descending order of the keys
// key[0 .. E) (unique; zero past E up to a power of two).  Up to 256 experts
// each thread counts the larger keys directly (broadcast LDS reads, one
// 64-bit compare each: cheaper than the sort's barriers); beyond, the keys
// are sorted and each position hands its expert its rank.  key[] is
// reordered in the second case.  Ends with a barrier.
__device__ __forceinline__ void rank_keys(uint64_t *key, uint32_t *rank_of, int E) {
    const int tid = threadIdx.x;
    if (E <= 256) {
        if (tid < E) {
            const uint64_t mine = key[tid];
            uint32_t r0 = 0, r1 = 0;
            int j = 0;
            for (; j + 1 < E; j += 2) {
                r0 += key[j] > mine;
                r1 += key[j + 1] > mine;
            }
            if (j < E) r0 += key[j] > mine;
            rank_of[tid] = r0 + r1;
        }
    } else {
        sort_desc(key, pow2_at_least(E));
        if (tid < E) rank_of[key_expert(key[tid])] = (uint32_t)tid;
    }
    __syncthreads();
}

template <bool FROM_TOPK>
__global__ void __launch_bounds__(1024) k_rank_experts(const uint32_t *__restrict__ offsets,
                                                       const uint32_t *__restrict__ idx, int tk, int E,
                                                       int budget, uint32_t *__restrict__ counts,
                                                       uint32_t *__restrict__ order, uint8_t *__restrict__ keep) {
    __shared__ uint32_t cnt[MOE_MAX_EXPERTS];
    __shared__ uint32_t rank_of[MOE_MAX_EXPERTS];
    __shared__ uint64_t key[MOE_MAX_EXPERTS];
    __shared__ uint32_t used_n;
    const int tid = threadIdx.x;
    const int N = pow2_at_least(E);
    if (tid == 0) used_n = 0;
    if (FROM_TOPK) {
        if (tid < E) cnt[tid] = 0;
        __syncthreads();
        for (int i = tid; i < tk; i += 1024) {
            const uint32_t e = idx[i];
            if (e < (uint32_t)E) atomicAdd(&cnt[e], 1u);
        }
    } else {
        if (tid < E) cnt[tid] = offsets[tid + 1] - offsets[tid];
    }
    __syncthreads();
    if (tid < N) key[tid] = tid < E ? expert_key(cnt[tid], tid) : 0ull;
    if (tid < E) {
        if (counts) counts[tid] = cnt[tid];
        if (cnt[tid] > 0) atomicAdd(&used_n, 1u);
    }
    __syncthreads();
    rank_keys(key, rank_of, E);
    // the non-empty experts hold ranks 0 .. n-1 (their keys exceed every
    // empty expert's), so order[] gets each of them once and 0xFFFFFFFF at
    // the n .. E-1 slots: every slot is written by exactly one thread
    if (tid < E) {
        const uint32_t r = rank_of[tid];
        const bool used = cnt[tid] > 0;
        if (used) order[r] = (uint32_t)tid;
        if ((uint32_t)tid >= used_n) order[tid] = 0xffffffffu;
        keep[tid] = (uint8_t)(used && r < (uint32_t)budget);
    }
}

// Row statistics of the chunk, from the same ranking: the n non-empty
// experts hold ranks 0 .. n-1 (count descending), so the most rows are at
// rank 0, the fewest at n - 1, and the ((n - 1) / 2)-th smallest count at
// rank n - 1 - (n - 1) / 2 (equal counts make the order of ties irrelevant).
__global__ void __launch_bounds__(1024) k_chunk_stats(const uint32_t *__restrict__ offsets, int t, int E,
                                                      moe_chunk_stats *__restrict__ out) {
    __shared__ uint32_t cnt[MOE_MAX_EXPERTS];
    __shared__ uint32_t rank_of[MOE_MAX_EXPERTS];
    __shared__ uint64_t key[MOE_MAX_EXPERTS];
    __shared__ uint32_t touched, cmax, cmin, med;
    const int tid = threadIdx.x;
    const int N = pow2_at_least(E);
    if (tid == 0) {
        touched = 0;
        cmax = cmin = med = 0;
    }
    __syncthreads();
    if (tid < N) {
        const uint32_t c = tid < E ? offsets[tid + 1] - offsets[tid] : 0u;
        if (tid < E) cnt[tid] = c;
        key[tid] = tid < E ? expert_key(c, tid) : 0ull;
        if (c > 0) atomicAdd(&touched, 1u);
    }
    __syncthreads();
    rank_keys(key, rank_of, E);
    const uint32_t n = touched;
    if (tid < E && cnt[tid] > 0) {
        const uint32_t r = rank_of[tid], c = cnt[tid];
        if (r == 0) cmax = c;
        if (r == n - 1) cmin = c;
        if (r == n - 1 - (n - 1) / 2) med = c;
    }
    __syncthreads();
    if (tid == 0) {
        moe_chunk_stats r;
        r.tokens = (uint32_t)t;
        r.assignments = offsets[E] - offsets[0];
        r.experts_touched = n;
        r.rows_max = cmax;
        r.rows_min = cmin;
        r.rows_median = med;
        r.pad[0] = r.pad[1] = 0;
        *out = r;
    }
}

}  // namespace

hipError_t launch_chunk_stats(const uint32_t *offsets, int t, int E, moe_chunk_stats *stats, hipStream_t s) {
    hipLaunchKernelGGL(k_chunk_stats, dim3(1), dim3(1024), 0, s, offsets, t, E, stats);
    return hipGetLastError();
}

hipError_t launch_rank_experts(const uint32_t *offsets, const uint32_t *topk_idx, int tk, int E, int budget,
                               uint32_t *counts, uint32_t *order, uint8_t *keep, hipStream_t s) {
    if (topk_idx)
        hipLaunchKernelGGL(k_rank_experts<true>, dim3(1), dim3(1024), 0, s, offsets, topk_idx, tk, E, budget, counts,
                           order, keep);
    else
        hipLaunchKernelGGL(k_rank_experts<false>, dim3(1), dim3(1024), 0, s, offsets, topk_idx, tk, E, budget,
                           counts, order, keep);
    return hipGetLastError();
}

}  // namespace moe
