// Residency of experts by use, on the GPU.
//
// The experts.rs page (fn prepare_expert_jobs) keeps a layer's most-used
// experts resident: the non-empty experts sorted by descending row count
// (a stable sort, so ties keep ascending expert id), the first `budget` of
// them kept, the rest streamed through the ring.  The decode.rs page
// (fn lookahead_layer) looks one block ahead: while a block runs, the next
// layer's experts are predicted so they can be fetched early.
//
// k_rank_experts ranks the experts in one workgroup of 1024 threads: the
// row counts come from the grouping's offsets (this block) or from a top-k
// (the next layer's router run on this block's input, for the lookahead),
// and thread e's rank is the number of non-empty experts that sort before
// it, a loop over the counts in LDS that every thread reads in the same
// order (broadcast reads).  Exact integer work: the result does not depend
// on timing.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

template <bool FROM_TOPK>
__global__ void __launch_bounds__(1024) k_rank_experts(const uint32_t *__restrict__ offsets,
                                                       const uint32_t *__restrict__ idx, int tk, int E,
                                                       int budget, uint32_t *__restrict__ counts,
                                                       uint32_t *__restrict__ order, uint8_t *__restrict__ keep) {
    __shared__ uint32_t cnt[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    if (FROM_TOPK) {
        for (int e = tid; e < E; e += 1024) cnt[e] = 0;
        __syncthreads();
        for (int i = tid; i < tk; i += 1024) {
            const uint32_t e = idx[i];
            if (e < (uint32_t)E) atomicAdd(&cnt[e], 1u);
        }
    } else {
        for (int e = tid; e < E; e += 1024) cnt[e] = offsets[e + 1] - offsets[e];
    }
    __syncthreads();
    for (int e = tid; e < E; e += 1024) order[e] = 0xffffffffu;   // slots past the non-empty experts
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {
        const uint32_t c = cnt[e];
        if (counts) counts[e] = c;
        int rank = -1;
        if (c > 0) {
            rank = 0;
            for (int j = 0; j < E; ++j) {
                const uint32_t cj = cnt[j];
                rank += (cj > c) || (cj == c && j < e);
            }
            order[rank] = (uint32_t)e;
        }
        keep[e] = (uint8_t)(rank >= 0 && rank < budget);
    }
}

// Row statistics of the chunk in one workgroup of 1024 threads: expert e's
// row count from the offsets into LDS; touched / max / min by LDS atomics
// (integer, so the result does not depend on their order); the median is
// the count of the touched expert whose ascending rank (count, then expert
// id) is (n - 1) / 2, found by the same broadcast loop as the ranking above.
__global__ void __launch_bounds__(1024) k_chunk_stats(const uint32_t *__restrict__ offsets, int t, int E,
                                                      moe_chunk_stats *__restrict__ out) {
    __shared__ uint32_t cnt[MOE_MAX_EXPERTS];
    __shared__ uint32_t touched, cmax, cmin, med;
    const int tid = threadIdx.x;
    if (tid == 0) {
        touched = 0;
        cmax = 0;
        cmin = 0xffffffffu;
        med = 0;
    }
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {
        const uint32_t c = offsets[e + 1] - offsets[e];
        cnt[e] = c;
        if (c > 0) {
            atomicAdd(&touched, 1u);
            atomicMax(&cmax, c);
            atomicMin(&cmin, c);
        }
    }
    __syncthreads();
    const uint32_t n = touched;
    for (int e = tid; e < E; e += 1024) {
        const uint32_t c = cnt[e];
        if (c == 0) continue;
        uint32_t rank = 0;
        for (int j = 0; j < E; ++j) {
            const uint32_t cj = cnt[j];
            rank += (cj > 0) && (cj < c || (cj == c && j < e));
        }
        if (rank == (n - 1) / 2) med = c;
    }
    __syncthreads();
    if (tid == 0) {
        moe_chunk_stats r;
        r.tokens = (uint32_t)t;
        r.assignments = offsets[E] - offsets[0];
        r.experts_touched = n;
        r.rows_max = cmax;
        r.rows_min = n ? cmin : 0u;
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
