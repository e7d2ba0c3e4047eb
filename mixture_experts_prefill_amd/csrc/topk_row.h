// Top-k with renormalised weights of one row by one wave, shared by the
// top-k kernel (router.hip) and the one-workgroup grouping kernel (csr.hip).
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

// Orderable key of a finite float: larger float -> larger key; -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Value of an order_key (the inverse map, with -0 read back as +0).
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Maximum of a 32-bit key over the wave, with DPP moves only (no LDS
// crossbar): row_shr 1, 2, 4, 8 leave each 16-lane row's maximum in its lane
// 15, row_bcast 15 and 31 carry it up, so lane 63 holds the wave's maximum,
// read back as a scalar.  Lanes whose DPP source is missing see 0, the
// smallest key.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
    return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_step<0x111, 0xf>(v);  // row_shr:1
    v = dpp_max_step<0x112, 0xf>(v);  // row_shr:2
    v = dpp_max_step<0x114, 0xf>(v);  // row_shr:4
    v = dpp_max_step<0x118, 0xf>(v);  // row_shr:8
    v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
    v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One wave per row: k rounds of a 64-lane arg-max over (value desc, id asc).
// Lane l holds the keys of experts l, l + 64, ... (KPL of them, E <= 64 KPL).
// A round takes the wave maximum of the keys, then the lowest expert id that
// holds it from one ballot per key slot (slot i before i + 1, then the lowest
// lane), and clears that key.  Round j's winner is kept by lane j, which then
// writes slot j; the winning key gives the logit back, so the softmax needs
// no second read of the row.
template <int KPL>
__device__ __forceinline__ void topk_row(const float *__restrict__ logits, int r, int E, int k,
                                         uint32_t *__restrict__ idx, float *__restrict__ wts) {
    const int lane = threadIdx.x & 63;
    const float *l = logits + (size_t)r * E;
    uint32_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? order_key(l[e]) : 0u;
    }
    uint32_t my_e = 0, my_key = 0, top = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t best = key[0];
#pragma unroll
        for (int i = 1; i < KPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u32(best);
        int e = 0;
#pragma unroll
        for (int i = KPL - 1; i >= 0; --i) {
            const uint64_t m = __ballot(key[i] == best);
            if (m) e = 64 * i + __builtin_ctzll(m);
        }
#pragma unroll
        for (int i = 0; i < KPL; ++i)
            if (lane + 64 * i == e) key[i] = 0u;   // remove the winner
        if (j == 0) top = best;
        if (lane == j) {
            my_e = (uint32_t)e;
            my_key = best;
        }
    }
    // softmax over the selected logits (renormalised top-k), fp32
    const bool mine = lane < k;
    const float lmax = key_value(top);
    const float ex = mine ? expf(key_value(my_key) - lmax) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (mine) {
        idx[(size_t)r * k + lane] = my_e;
        wts[(size_t)r * k + lane] = ex / sum;
    }
}


}  // namespace
}  // namespace moe
