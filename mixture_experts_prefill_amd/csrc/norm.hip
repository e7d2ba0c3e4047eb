// The block output injected into the residual stream and read by the next
// fused norm, on gfx950.
//
// The cherenkov pages run a block's MoE output into the next layer through
// its fused norm (decode.rs page, step_rows: the output is "pending" until
// the next fused norm injects it; prefill.rs page, pf_layer: pf_hc_read with
// the pending output produces the next block input `mixed`; prefill_chunk:
// pf_inject after the last layer).  The arithmetic of those kernels is not
// shown; the reading implemented here: a row's residual stream is n fp32
// copies of h values,
//
//   copy_i += beta_i * y                  (the injection)
//   z       = sum_i alpha_i * copy_i      (the read, copies in ascending i)
//   mixed   = bf16( z * rsqrt(mean(z^2) + eps) * gamma )
//
// k_next_norm runs it for one row per workgroup.  With FUSED the row's block
// output y is formed in the workgroup itself from the down projections
// (ye) exactly as the combine forms it (shared term first, then the k
// routed terms in ascending CSR position, fp32 fma), so the block output
// is never written to memory: the combine, the injection and the norm are
// one pass over ye, the copies and gamma.  Without FUSED, y is read from an
// fp32 [t][h] buffer (or absent).
//
// Each of the 256 threads owns 8 consecutive columns per 2048 (chunks q =
// tid + 256 j), so every load and store is 16 or 32 bytes per lane and
// coalesced; z stays in registers between the sum of squares and the
// scaling.  The row's sum of squares is reduced in a fixed order (the
// thread's chunks in order, a butterfly inside each wave, then the four wave
// sums in order), so results do not depend on timing.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kNT = 256;  // threads per row

__device__ __forceinline__ uint32_t pk_bf16_rne(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void load8(const float *p, float v[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store8(float *p, const float v[8]) {
    *reinterpret_cast<f32x4 *>(p) = (f32x4){v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = (f32x4){v[4], v[5], v[6], v[7]};
}

// y of one 8-column chunk, as k_combine forms it with accumulate = 0.
__device__ __forceinline__ void combine8(const uint16_t *__restrict__ ye, const uint32_t *ps,
                                         const float *__restrict__ csr_w, int k, int h, int r, int c,
                                         const uint16_t *__restrict__ ys, const float *__restrict__ gate,
                                         float acc[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if (ys) {
        const uint4 v = *reinterpret_cast<const uint4 *>(ys + (size_t)r * h + c);
        const float g = gate ? gate[r] : 1.0f;
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = acc[2 * i] + g * __uint_as_float(u[i] << 16);
            acc[2 * i + 1] = acc[2 * i + 1] + g * __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    for (int j0 = 0; j0 < k; j0 += 16) {
        uint4 v[16];
        float wj[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (j0 + j < k) {
                const uint32_t p = ps[j0 + j];
                const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ye + (size_t)p * h + c));
                v[j] = make_uint4(q.x, q.y, q.z, q.w);
                wj[j] = csr_w[p];
            }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (j0 + j < k) {
                const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = __builtin_fmaf(wj[j], __uint_as_float(u[i] << 16), acc[2 * i]);
                    acc[2 * i + 1] = __builtin_fmaf(wj[j], __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
                }
            }
    }
}

template <bool FUSED, int NQ>
__global__ void __launch_bounds__(kNT) k_next_norm(NextNormArgs a) {
    __shared__ uint32_t ps[MOE_MAX_K];
    __shared__ float wsum[kNT / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int h = a.h, n = a.n;
    if (FUSED && tid < 64) {
        // the row's k CSR positions in ascending order (= ascending expert id)
        const uint32_t mine = tid < a.k ? a.pos[(size_t)r * a.k + tid] : 0xffffffffu;
        int rank = 0;
        for (int i = 0; i < a.k; ++i) rank += (uint32_t)__builtin_amdgcn_readlane((int)mine, i) < mine;
        if (tid < a.k) ps[rank] = mine;
    }
    if (FUSED) __syncthreads();
    float z[NQ][8];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int c = (tid + kNT * j) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) z[j][i] = 0.0f;
        if (c >= h) continue;
        float y[8];
        bool have_y = true;
        if (FUSED) {
            combine8(a.ye, ps, a.csr_w, a.k, h, r, c, a.ys, a.gate, y);
        } else if (a.y) {
            load8(a.y + (size_t)r * h + c, y);
        } else {
            have_y = false;
        }
        for (int cp = 0; cp < n; ++cp) {
            float *hp = a.hyper + ((size_t)r * n + cp) * h + c;
            float v[8];
            load8(hp, v);
            if (have_y) {
                const float b = a.beta[cp];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(b, y[i], v[i]);
                store8(hp, v);
            }
            const float al = a.alpha[cp];
#pragma unroll
            for (int i = 0; i < 8; ++i) z[j][i] = __builtin_fmaf(al, v[i], z[j][i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(z[j][i], z[j][i], ss);
    }
    // row sum of squares in a fixed order
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((tid & 63) == 0) wsum[tid >> 6] = ss;
    __syncthreads();
    float tot = wsum[0];
#pragma unroll
    for (int w = 1; w < kNT / 64; ++w) tot += wsum[w];
    const float inv = 1.0f / __fsqrt_rn(tot / (float)h + a.eps);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int c = (tid + kNT * j) * 8;
        if (c >= h) continue;
        float g[8];
        load8(a.gamma + c, g);
        uint4 o;
        o.x = pk_bf16_rne(z[j][0] * inv * g[0], z[j][1] * inv * g[1]);
        o.y = pk_bf16_rne(z[j][2] * inv * g[2], z[j][3] * inv * g[3]);
        o.z = pk_bf16_rne(z[j][4] * inv * g[4], z[j][5] * inv * g[5]);
        o.w = pk_bf16_rne(z[j][6] * inv * g[6], z[j][7] * inv * g[7]);
        *reinterpret_cast<uint4 *>(a.mixed + (size_t)r * h + c) = o;
    }
}

template <bool FUSED>
hipError_t launch_nq(const NextNormArgs &a, hipStream_t s) {
    const int nq = (a.h / 8 + kNT - 1) / kNT;
    const dim3 grid(a.t), block(kNT);
    if (nq <= 1) hipLaunchKernelGGL((k_next_norm<FUSED, 1>), grid, block, 0, s, a);
    else if (nq <= 2) hipLaunchKernelGGL((k_next_norm<FUSED, 2>), grid, block, 0, s, a);
    else if (nq <= 4) hipLaunchKernelGGL((k_next_norm<FUSED, 4>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_next_norm<FUSED, 8>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_next_norm(const NextNormArgs &a, hipStream_t s) {
    ProfileScope ps(MOE_PHASE_NORM, s);
    return a.ye ? launch_nq<true>(a, s) : launch_nq<false>(a, s);
}

}  // namespace moe
