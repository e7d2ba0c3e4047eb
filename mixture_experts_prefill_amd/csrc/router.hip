// Router logits and top-k with renormalised weights for gfx950.
//
// Computes what the router_b call produces on the cherenkov prefill.rs page
// (fn pf_layer: topk_idx u32 [t][k] and topk_w f32 [t][k] from the block
// input), with the logits in a fixed fp32 order so that top-k selections are
// reproducible bit for bit:
//   the hidden dimension is cut into 4-element chunks; chunk c feeds partial
//   c % 64; each partial is an fma chain from +0 in ascending index; then
//   p[l] += p[l + off] for off = 32, 16, 8, 4, 2, 1; the logit is p[0].
// A wavefront's 64 lanes are the 64 partials: lane l reads 4 consecutive
// elements (8 bytes of x, 16 bytes of W) per 256-element step, so every load
// is one contiguous 512 B / 1 KB segment per row.  The final tree is a
// transposed butterfly: at each level a lane keeps half of its outputs and
// adds its partner's copy of them, so after 6 levels lane l holds output l
// (addition is commutative, so p[a] + p[b] computed on either lane is the
// same value the tree defines).
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// One wave computes an RT x ET tile of logits (RT * ET outputs, a power of two <= 64).
template <int RT, int ET>
__global__ void __launch_bounds__(256) k_router(const uint16_t *__restrict__ x,
                                                const float *__restrict__ w, int t, int h, int E,
                                                float *__restrict__ logits) {
    constexpr int N = RT * ET;
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "tile must be a power of two <= 64");
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int e_tiles = (E + ET - 1) / ET;
    const int r0 = (wave / e_tiles) * RT;
    const int e0 = (wave % e_tiles) * ET;
    if (r0 >= t) return;  // whole wave leaves together

    const uint2 *xr[RT];
    const float4 *wr[ET];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        int r = min(r0 + i, t - 1);  // clamped rows are computed but not stored
        xr[i] = reinterpret_cast<const uint2 *>(x + (size_t)r * h) + lane;
    }
#pragma unroll
    for (int j = 0; j < ET; ++j) {
        int e = min(e0 + j, E - 1);
        wr[j] = reinterpret_cast<const float4 *>(w + (size_t)e * h) + lane;
    }

    float p[N];
#pragma unroll
    for (int o = 0; o < N; ++o) p[o] = 0.0f;

    const int steps = h >> 8;  // 256 elements per step, 4 per lane
    for (int s = 0; s < steps; ++s) {
        float xv[RT][4];
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            uint2 v = xr[i][s * 64];
            xv[i][0] = bf16_lo(v.x);
            xv[i][1] = bf16_hi(v.x);
            xv[i][2] = bf16_lo(v.y);
            xv[i][3] = bf16_hi(v.y);
        }
#pragma unroll
        for (int j = 0; j < ET; ++j) {
            float4 wv = wr[j][s * 64];
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                float &acc = p[i * ET + j];
                acc = __builtin_fmaf(xv[i][0], wv.x, acc);
                acc = __builtin_fmaf(xv[i][1], wv.y, acc);
                acc = __builtin_fmaf(xv[i][2], wv.z, acc);
                acc = __builtin_fmaf(xv[i][3], wv.w, acc);
            }
        }
    }

    // Transposed butterfly over the 64 partials.  While a lane holds n > 1
    // outputs it keeps the half selected by its lane bit and receives the
    // partner's copy of that half; once n == 1 it plain-reduces.
    // Selects are done on bit patterns (mask blend) so the compiler keeps p[]
    // in registers instead of selecting an address into a stack copy.
#pragma unroll
    for (int lvl = 0; lvl < 6; ++lvl) {
        const int off = 32 >> lvl;
        const int cnt = N >> lvl;  // outputs held before this level (compile-time)
        if (cnt > 1) {
            const int half = cnt >> 1;
            const uint32_t m = (lane & off) ? 0xffffffffu : 0u;
#pragma unroll
            for (int o = 0; o < half; ++o) {
                const uint32_t lo = __float_as_uint(p[o]), hi = __float_as_uint(p[o + half]);
                const float keep = __uint_as_float((lo & ~m) | (hi & m));
                const float give = __uint_as_float((hi & ~m) | (lo & m));
                p[o] = keep + __shfl_xor(give, off, 64);
            }
        } else {
            p[0] = p[0] + __shfl_xor(p[0], off, 64);
        }
    }
    // Output index o is formed by the lane bits used for splitting (MSB first);
    // with N = 2^a splits at off = 32 .. 2^(6-a), o = lane >> (6 - a).
    constexpr int shift = (N == 64) ? 0 : (N == 32) ? 1 : (N == 16) ? 2 : (N == 8) ? 3
                        : (N == 4) ? 4 : (N == 2) ? 5 : 6;
    if ((lane & ((1 << shift) - 1)) == 0) {
        const int o = lane >> shift;
        const int i = o / ET, j = o % ET;
        const int r = r0 + i, e = e0 + j;
        if (r < t && e < E) logits[(size_t)r * E + e] = p[0];
    }
}

// Orderable key of a finite float: larger float -> larger key; -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave per row: k rounds of a 64-lane arg-max over (value desc, id asc).
// Round j's winner is kept by lane j, which then writes slot j.
__global__ void __launch_bounds__(256) k_topk(const float *__restrict__ logits, int t, int E, int k,
                                              uint32_t *__restrict__ idx, float *__restrict__ wts) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (r >= t) return;
    const float *l = logits + (size_t)r * E;
    constexpr int kMaxPerLane = MOE_MAX_EXPERTS / 64;
    uint64_t key[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? ((uint64_t)order_key(l[e]) << 32) | (uint32_t)(0xffffffffu - e) : 0;
    }
    uint32_t my_e = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = __shfl_xor(best, off, 64);
            best = o > best ? o : best;
        }
        const uint32_t e = 0xffffffffu - (uint32_t)(best & 0xffffffffu);
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if ((uint32_t)(lane + 64 * i) == e) key[i] = 0;   // remove the winner
        if (lane == j) my_e = e;
    }
    // softmax over the selected logits (renormalised top-k), fp32
    const bool mine = lane < k;
    const float my_l = mine ? l[my_e] : 0.0f;
    const float lmax = __shfl(my_l, 0, 64);
    const float ex = mine ? expf(my_l - lmax) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (mine) {
        idx[(size_t)r * k + lane] = my_e;
        wts[(size_t)r * k + lane] = ex / sum;
    }
}

template <int RT, int ET>
hipError_t launch_tile(const uint16_t *x, const float *w, int t, int h, int E, float *logits,
                       hipStream_t s) {
    const int waves = ((t + RT - 1) / RT) * ((E + ET - 1) / ET);
    const int blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((k_router<RT, ET>), dim3(blocks), dim3(256), 0, s, x, w, t, h, E, logits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits(const uint16_t *x, const float *w, int t, int h, int E,
                                float *logits, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_ROUTER, s);
    // Small t: one row block and one expert per wave keeps >= E waves busy
    // streaming W; large t: 8 x 8 tiles reuse each loaded chunk 8 times.
    if (t >= 64 && E >= 8) return launch_tile<8, 8>(x, w, t, h, E, logits, s);
    if (t >= 8) return launch_tile<8, 1>(x, w, t, h, E, logits, s);
    if (t >= 4) return launch_tile<4, 1>(x, w, t, h, E, logits, s);
    if (t >= 2) return launch_tile<2, 1>(x, w, t, h, E, logits, s);
    return launch_tile<1, 1>(x, w, t, h, E, logits, s);
}

hipError_t launch_topk(const float *logits, int t, int E, int k, uint32_t *idx, float *wts,
                       hipStream_t s) {
    ProfileScope prof(MOE_PHASE_TOPK, s);
    hipLaunchKernelGGL(k_topk, dim3((t + 3) / 4), dim3(256), 0, s, logits, t, E, k, idx, wts);
    return hipGetLastError();
}

}  // namespace moe
