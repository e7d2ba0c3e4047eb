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

// r = lane's bit of m ? b : a, as one v_cndmask_b32.  (Written out because
// the compiler turns the plain select chain of a list shift into an index
// search several times longer.)
__device__ __forceinline__ uint32_t sel32(uint32_t a, uint32_t b, uint64_t m) {
    uint32_t r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(m));
    return r;
}

// One wave per row.  Lane l holds experts l, l + 64, ... (KPL of them,
// E <= 64 KPL) and first sorts them in registers (bitonic network) by the
// selection order: logit descending, then expert id ascending.  A round
// takes the wave maximum of the lanes' first keys; the lowest expert id
// among the lanes that hold it wins (one lane unless logits tie exactly,
// when a second wave maximum over the complemented ids decides), and that
// lane drops its first entry.  Round j's winner is kept by lane j, which
// writes slot j; the winning key gives the logit back, so the softmax needs
// no second read of the row.  The results also go to the LDS arrays
// lidx / lwts when given.
template <int KPL>
__device__ __forceinline__ void topk_row(const float *__restrict__ logits, int r, int E, int k,
                                         uint32_t *__restrict__ idx, float *__restrict__ wts,
                                         uint32_t *lidx = nullptr, float *lwts = nullptr) {
    const int lane = threadIdx.x & 63;
    const float *l = logits + (size_t)r * E;
    uint32_t key[KPL], id[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? order_key(l[e]) : 0u;
        id[i] = (uint32_t)e;
    }
#pragma unroll
    for (int size = 2; size <= KPL; size *= 2)
#pragma unroll
        for (int stride = size / 2; stride > 0; stride /= 2)
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    // "a before b": a larger key, or an equal key and a lower id
                    const bool ab = key[i] > key[j] || (key[i] == key[j] && id[i] < id[j]);
                    const bool swap = ((i & size) == 0) ? !ab : ab;
                    const uint32_t ki = key[i], kj = key[j], ii = id[i], ij = id[j];
                    key[i] = swap ? kj : ki;
                    key[j] = swap ? ki : kj;
                    id[i] = swap ? ij : ii;
                    id[j] = swap ? ii : ij;
                }
            }
    uint32_t my_e = 0, my_key = 0, top = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t best = wave_max_u32(key[0]);
        const uint64_t at = __ballot(key[0] == best);
        uint32_t wid;
        if (__popcll(at) == 1) {
            wid = (uint32_t)__builtin_amdgcn_readlane((int)id[0], (int)__builtin_ctzll(at));
        } else {
            wid = ~wave_max_u32(key[0] == best ? ~id[0] : 0u);
        }
        const uint64_t win = __ballot(key[0] == best && id[0] == wid);
#pragma unroll
        for (int i = 0; i + 1 < KPL; ++i) {
            key[i] = sel32(key[i], key[i + 1], win);
            id[i] = sel32(id[i], id[i + 1], win);
        }
        key[KPL - 1] = sel32(key[KPL - 1], 0u, win);
        if (j == 0) top = best;
        if (lane == j) {
            my_e = wid;
            my_key = best;
        }
    }
    // softmax over the selected logits (renormalised top-k), fp32
    const bool sel = lane < k;
    const float lmax = key_value(top);
    const float ex = sel ? expf(key_value(my_key) - lmax) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (sel) {
        const float w = ex / sum;
        idx[(size_t)r * k + lane] = my_e;
        wts[(size_t)r * k + lane] = w;
        if (lidx) {
            lidx[r * k + lane] = my_e;
            lwts[r * k + lane] = w;
        }
    }
}

}  // namespace
}  // namespace moe
