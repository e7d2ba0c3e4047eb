// Grouped 4-bit expert GEMMs on gfx950 matrix cores.
//
// The cherenkov experts.rs page (fn pf_experts) runs, per non-empty expert,
// gather_rows -> expert_qmm_from (gate) -> expert_qmm_from (up) -> silu_mul
// -> expert_qmm_from (down) -> scatter_add_rows.  Here all experts of a call
// run in two launches: one gate/up kernel whose epilogue applies
// SiLU(gate) * up, and one down kernel; the weighted scatter-add becomes a
// separate deterministic combine (k_combine) so that no two writers touch a
// row concurrently.
//
// Work decomposition.  The MFMA is v_mfma_f32_32x32x16_bf16 with the weight
// matrix as operand A (32 output features) and token rows as operand B (32
// tokens).  A workgroup (4 waves) owns one M-tile of BM CSR positions of one
// expert and a block of output features; each wave owns two 32-feature
// fragments (gate and up of the same features, or two adjacent down
// features) for all BM tokens, so every activation fragment read from LDS
// feeds two MFMAs.  Per 64-wide K step:
//   - the workgroup stages BM activation rows x 128 bytes into LDS (gathered
//     through csr_rows for the routed gate/up projection), double-buffered,
//     16-byte chunks XOR-swizzled by row so the B-fragment reads of 32 rows
//     at one column hit distinct banks;
//   - each wave loads its two 1 KB code tiles (one 16-byte load per lane,
//     fully coalesced thanks to the record's tile order) and their fp16
//     scale/bias pairs, and dequantises in registers: a nibble pair OR'ed
//     into the fp16 pattern 0x6400 (= 1024 + q) feeds v_fma_mix_f32 with
//     scale s and offset (bias - 1024 s) kept in fp32, then
//     v_cvt_pk_bf16_f32 packs the MFMA operand;
//   - 4 MFMA steps of K = 16.  Inside a lane's 16 bytes the K order is
//     permuted (lane half L/32 takes 32 consecutive columns), and the
//     activation fragment uses the same permutation, so the products pair up.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Mode { GU_GATHER = 0, GU_DENSE = 1, DOWN_YE = 2, DOWN_OUT = 3 };

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// 8 codes of one 32-bit word -> 8 bf16 weights (element j = code j).
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s, float c) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t h = ((w >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
        const half2_t hv = __builtin_bit_cast(half2_t, h);
        o[p] = pk_bf16(__builtin_fmaf((float)hv.x, s, c), __builtin_fmaf((float)hv.y, s, c));
    }
    uint4 u = make_uint4(o[0], o[1], o[2], o[3]);
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

template <int MODE, int BM>
__global__ void __launch_bounds__(256, 2) k_gemm(const GemmArgs a) {
    constexpr bool kGateUp = (MODE == GU_GATHER || MODE == GU_DENSE);
    constexpr int TB = BM / 32;            // token blocks of 32
    constexpr int CH = BM * 8 / 256;       // 16-byte row chunks staged per thread per K step
    static_assert(BM % 32 == 0 && CH >= 1, "BM must be a multiple of 32");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * 128];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---- M-tile
    int expert = 0, p0, n;
    if (MODE == GU_DENSE || MODE == DOWN_OUT) {
        p0 = blockIdx.y * BM;
        if (p0 >= a.t) return;
        n = min(BM, a.t - p0);
    } else {
        if (blockIdx.y >= *a.sched_n) return;
        const int4 tl = a.sched[blockIdx.y];
        expert = tl.x;
        p0 = tl.y;
        n = tl.z;
    }
    const uint8_t *rec = static_cast<const uint8_t *>(
        a.records ? reinterpret_cast<const void *>(a.records[expert]) : a.record);

    // ---- features of this wave: two fragments of 32 rows of the weight matrix
    const int n_out = kGateUp ? a.inter : a.hidden;   // rows of the weight matrix
    const int K = kGateUp ? a.hidden : a.inter;       // reduction length
    const int nk = K >> 6;
    const int obs = n_out >> 5;                       // 32-row blocks
    int ob[2];
    if (kGateUp) {
        ob[0] = ob[1] = blockIdx.x * 4 + wave;        // gate and up of the same features
    } else {
        ob[0] = blockIdx.x * 8 + wave * 2;
        ob[1] = ob[0] + 1;
    }
    const bool live0 = ob[0] < obs, live1 = ob[1] < obs;
    const uint64_t woff[2] = {a.w_off, kGateUp ? a.w2_off : a.w_off};
    const uint64_t soff[2] = {a.sb_off, kGateUp ? a.sb2_off : a.sb_off};
    const int sb_tile_bytes = (64 / a.group) * 32 * 4;
    const int sb_entry = (a.group == 64) ? (lane & 31) : lane;

    // ---- B-operand source rows for the chunks this thread stages
    const uint16_t *src[CH];
    bool valid[CH];
    int lds_off[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int ch = tid + 256 * c;
        const int i = ch >> 3, q = ch & 7;   // tile row, 16-byte chunk
        valid[c] = i < n;
        const int ii = valid[c] ? i : 0;
        size_t row;
        int ld;
        if (MODE == GU_GATHER) {
            row = a.rows[p0 + ii];
            ld = a.hidden;
        } else if (MODE == GU_DENSE) {
            row = (size_t)(p0 + ii);
            ld = a.hidden;
        } else {
            row = (size_t)(p0 + ii);
            ld = a.inter;
        }
        const uint16_t *base = kGateUp ? a.x : a.act;
        src[c] = base + row * ld + q * 8;
        lds_off[c] = (i * 8 + (q ^ (i & 7))) * 16;
    }

    auto load_b = [&](int kb, uint4 *v) {
#pragma unroll
        for (int c = 0; c < CH; ++c)
            v[c] = valid[c] ? *reinterpret_cast<const uint4 *>(src[c] + kb * 64) : make_uint4(0, 0, 0, 0);
    };
    auto load_a = [&](int kb, uint4 *codes, uint32_t *sb) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const bool live = f ? live1 : live0;
            const size_t tile = (size_t)(live ? ob[f] : 0) * nk + kb;
            codes[f] = *reinterpret_cast<const uint4 *>(rec + woff[f] + tile * 1024 + lane * 16);
            sb[f] = *reinterpret_cast<const uint32_t *>(rec + soff[f] + tile * sb_tile_bytes + sb_entry * 4);
        }
    };

    f32x16 acc[2][TB];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][b][r] = 0.0f;

    uint4 bv[CH], codes[2];
    uint32_t sb[2];
    load_b(0, bv);
    load_a(0, codes, sb);

    // B-fragment read position: row (tb*32 + lane%32), chunk 4*(lane/32) + s.
    const int brow = lane & 31, bhalf = lane >> 5;

    for (int kb = 0; kb < nk; ++kb) {
        uint8_t *buf = lds[kb & 1];
#pragma unroll
        for (int c = 0; c < CH; ++c) *reinterpret_cast<uint4 *>(buf + lds_off[c]) = bv[c];
        const uint4 cur[2] = {codes[0], codes[1]};
        const uint32_t csb[2] = {sb[0], sb[1]};
        __syncthreads();
        if (kb + 1 < nk) {
            load_b(kb + 1, bv);
            load_a(kb + 1, codes, sb);
        }
        float s[2], off[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const half2_t h = __builtin_bit_cast(half2_t, csb[f]);
            s[f] = (float)h.x;
            off[f] = __builtin_fmaf(-1024.0f, s[f], (float)h.y);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            bf16x8 af[2];
            af[0] = dequant8(st == 0 ? cur[0].x : st == 1 ? cur[0].y : st == 2 ? cur[0].z : cur[0].w, s[0], off[0]);
            af[1] = dequant8(st == 0 ? cur[1].x : st == 1 ? cur[1].y : st == 2 ? cur[1].z : cur[1].w, s[1], off[1]);
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                const int row = b * 32 + brow;
                const int q = (4 * bhalf + st) ^ (row & 7);
                const bf16x8 bf = *reinterpret_cast<const bf16x8 *>(buf + (row * 8 + q) * 16);
                acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bf, acc[0][b], 0, 0, 0);
                acc[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bf, acc[1][b], 0, 0, 0);
            }
        }
    }

    // ---- epilogue.  acc[f][b][r]: feature 8*(r/4) + 4*(lane/32) + r%4 of
    // fragment f, token b*32 + lane%32 of the tile.
#pragma unroll
    for (int b = 0; b < TB; ++b) {
        const int tok = b * 32 + brow;
        if (tok >= n) continue;
        const size_t p = (size_t)(p0 + tok);
        if (kGateUp) {
            if (!live0) continue;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int feat = ob[0] * 32 + 8 * q4 + 4 * bhalf;
                uint2 v;
                v.x = pk_bf16(silu_mul(acc[0][b][4 * q4 + 0], acc[1][b][4 * q4 + 0]),
                              silu_mul(acc[0][b][4 * q4 + 1], acc[1][b][4 * q4 + 1]));
                v.y = pk_bf16(silu_mul(acc[0][b][4 * q4 + 2], acc[1][b][4 * q4 + 2]),
                              silu_mul(acc[0][b][4 * q4 + 3], acc[1][b][4 * q4 + 3]));
                *reinterpret_cast<uint2 *>(a.hg + p * a.inter + feat) = v;
            }
        } else {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                if (!(f ? live1 : live0)) continue;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int feat = ob[f] * 32 + 8 * q4 + 4 * bhalf;
                    if (MODE == DOWN_YE) {
                        uint2 v;
                        v.x = pk_bf16(acc[f][b][4 * q4 + 0], acc[f][b][4 * q4 + 1]);
                        v.y = pk_bf16(acc[f][b][4 * q4 + 2], acc[f][b][4 * q4 + 3]);
                        *reinterpret_cast<uint2 *>(a.ye + p * a.hidden + feat) = v;
                    } else {
                        const float g = a.gate ? a.gate[p] : 1.0f;
                        float4 *o = reinterpret_cast<float4 *>(a.out + p * a.hidden + feat);
                        float4 v = make_float4(g * acc[f][b][4 * q4 + 0], g * acc[f][b][4 * q4 + 1],
                                               g * acc[f][b][4 * q4 + 2], g * acc[f][b][4 * q4 + 3]);
                        if (a.accumulate) {
                            const float4 old = *o;
                            v.x += old.x;
                            v.y += old.y;
                            v.z += old.z;
                            v.w += old.w;
                        }
                        *o = v;
                    }
                }
            }
        }
    }
}

// out[r, :] (+)= sum over the row's k CSR entries, in ascending CSR position
// (= ascending expert id), of csr_w[p] * ye[p, :].  One workgroup per row.
__global__ void __launch_bounds__(256) k_combine(const uint16_t *__restrict__ ye,
                                                 const uint32_t *__restrict__ pos,
                                                 const float *__restrict__ csr_w, int t, int k,
                                                 int h, float *__restrict__ out, int accumulate) {
    const int r = blockIdx.x;
    uint32_t ps[MOE_MAX_K];
    float ws[MOE_MAX_K];
    for (int j = 0; j < k; ++j) ps[j] = pos[(size_t)r * k + j];
    for (int j = 1; j < k; ++j)  // insertion sort, k <= 32
        for (int i = j; i > 0 && ps[i] < ps[i - 1]; --i) {
            uint32_t tmp = ps[i];
            ps[i] = ps[i - 1];
            ps[i - 1] = tmp;
        }
    for (int j = 0; j < k; ++j) ws[j] = csr_w[ps[j]];
    for (int c = threadIdx.x * 8; c < h; c += blockDim.x * 8) {
        float acc[8];
        float4 *o = reinterpret_cast<float4 *>(out + (size_t)r * h + c);
        if (accumulate) {
            const float4 o0 = o[0], o1 = o[1];
            acc[0] = o0.x; acc[1] = o0.y; acc[2] = o0.z; acc[3] = o0.w;
            acc[4] = o1.x; acc[5] = o1.y; acc[6] = o1.z; acc[7] = o1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        }
        for (int j = 0; j < k; ++j) {
            const uint4 v = *reinterpret_cast<const uint4 *>(ye + (size_t)ps[j] * h + c);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = __builtin_fmaf(ws[j], __uint_as_float(u[i] << 16), acc[2 * i]);
                acc[2 * i + 1] = __builtin_fmaf(ws[j], __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
            }
        }
        o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

// g[r] = sigmoid(x_r . gate_w), one wave per row, fp32.
__global__ void __launch_bounds__(256) k_shared_gate(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ gw, int t, int h,
                                                     float *__restrict__ g) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= t) return;
    float s = 0.0f;
    for (int i = lane; i < h; i += 64)
        s = __builtin_fmaf(__uint_as_float((uint32_t)x[(size_t)r * h + i] << 16),
                           __uint_as_float((uint32_t)gw[i] << 16), s);
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) g[r] = 1.0f / (1.0f + expf(-s));
}

template <int MODE>
hipError_t launch_mode(const GemmArgs &a, int bm, hipStream_t s) {
    const bool gu = (MODE == GU_GATHER || MODE == GU_DENSE);
    const int n_out = gu ? a.inter : a.hidden;
    const int per_wg = gu ? 128 : 256;
    const bool dense = (MODE == GU_DENSE || MODE == DOWN_OUT);
    const int tiles = dense ? (a.t + bm - 1) / bm : a.max_tiles;
    const dim3 grid((n_out + per_wg - 1) / per_wg, tiles);
    switch (bm) {
    case 32: hipLaunchKernelGGL((k_gemm<MODE, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((k_gemm<MODE, 64>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_gemm<MODE, 128>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gateup(const GemmArgs &a, int bm, hipStream_t s) {
    ProfileScope prof(a.sched ? MOE_PHASE_GATEUP : MOE_PHASE_SHARED_GU, s);
    return a.sched ? launch_mode<GU_GATHER>(a, bm, s) : launch_mode<GU_DENSE>(a, bm, s);
}

hipError_t launch_down(const GemmArgs &a, int bm, hipStream_t s) {
    ProfileScope prof(a.sched ? MOE_PHASE_DOWN : MOE_PHASE_SHARED_DOWN, s);
    return a.sched ? launch_mode<DOWN_YE>(a, bm, s) : launch_mode<DOWN_OUT>(a, bm, s);
}

hipError_t launch_shared_gate(const uint16_t *x, const uint16_t *gate_w, int t, int h, float *g,
                              hipStream_t s) {
    hipLaunchKernelGGL(k_shared_gate, dim3((t + 3) / 4), dim3(256), 0, s, x, gate_w, t, h, g);
    return hipGetLastError();
}

hipError_t launch_combine(const uint16_t *ye, const uint32_t *pos, const float *csr_w, int t,
                          int k, int h, float *out, int accumulate, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_COMBINE, s);
    hipLaunchKernelGGL(k_combine, dim3(t), dim3(256), 0, s, ye, pos, csr_w, t, k, h, out, accumulate);
    return hipGetLastError();
}

}  // namespace moe
