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

}  // namespace

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
