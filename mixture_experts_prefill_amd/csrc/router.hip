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
#include "lds_dma.h"
#include "moe_internal.h"
#include "topk_row.h"

namespace moe {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Transposed butterfly over the 64 partials of N outputs (N a power of two,
// at most 64).  While a lane holds n > 1 outputs it keeps the half selected
// by its lane bit and receives the partner's copy of that half; once n == 1
// it plain-reduces.  Selects are done on bit patterns (mask blend) so the
// compiler keeps p[] in registers instead of selecting an address into a
// stack copy.  The output index is formed by the lane bits used for
// splitting (MSB first): with N = 2^a, lanes whose low 6 - a bits are zero
// hold output lane >> (6 - a).
constexpr int tree_shift(int n) {
    return n == 64 ? 0 : n == 32 ? 1 : n == 16 ? 2 : n == 8 ? 3 : n == 4 ? 4 : n == 2 ? 5 : 6;
}
template <int N>
__device__ __forceinline__ float tree64(float (&p)[N], int lane) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "a power of two <= 64");
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
    return p[0];
}

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

    const float v = tree64(p, lane);
    constexpr int shift = tree_shift(N);
    if ((lane & ((1 << shift) - 1)) == 0) {
        const int o = lane >> shift;
        const int i = o / ET, j = o % ET;
        const int r = r0 + i, e = e0 + j;
        if (r < t && e < E) logits[(size_t)r * E + e] = v;
    }
}

// Few-row router (t <= 8, h <= 4096): a workgroup of 4 waves owns every row
// of the chunk and 4 / RS experts; the RS waves of one expert take RT rows
// each.  Each wave loads its expert's whole W row into registers (h/64
// floats per lane) while the workgroup stages the rows' x in LDS (at most
// 64 KB), so the kernel waits on memory about twice instead of once per
// 256-element step.  Lane l still owns partial l of every logit and runs the
// same fma chains and tree.  Two waves per expert for 5-8 rows halve each
// wave's chain length and spread the experts over twice the workgroups.
constexpr int kFewRows = 8, kFewSteps = 16;
template <int RT, int RS>
__global__ void __launch_bounds__(256) k_router_few(const uint16_t *__restrict__ x,
                                                    const float *__restrict__ w, int t, int h, int E,
                                                    float *__restrict__ logits) {
    constexpr int TR = RT * RS;  // rows staged
    __shared__ __attribute__((aligned(16))) uint16_t xs[TR * kFewSteps * 256];
    const int tid = threadIdx.x, lane = tid & 63, wv_id = tid >> 6;
    const int e = blockIdx.x * (4 / RS) + wv_id / RS;
    const int rbase = (wv_id % RS) * RT;
    const int steps = h >> 8;
    const float4 *wr = reinterpret_cast<const float4 *>(w + (size_t)min(e, E - 1) * h) + lane;
    // Loads are unconditional, at clamped (in-bounds) addresses, so that they
    // all go out before the first wait; clamped copies are never used.
    float4 wv[kFewSteps];
#pragma unroll
    for (int s = 0; s < kFewSteps; ++s) wv[s] = wr[min(s, steps - 1) * 64];
    // rows 0 .. t-1 are contiguous: t * h / 8 chunks of 16 bytes
    constexpr int kCh = TR * kFewSteps * 256 / 8 / 256;
    const int nch = t * (h >> 3);
    const uint4 *xg = reinterpret_cast<const uint4 *>(x);
    uint4 xv[kCh];
#pragma unroll
    for (int j = 0; j < kCh; ++j) xv[j] = xg[min(tid + 256 * j, nch - 1)];
    // (a clamped chunk is stored again where its own thread stores it, with
    // the same bytes; the stores have no branch, so the loads are not sunk
    // into one wait each)
#pragma unroll
    for (int j = 0; j < kCh; ++j) reinterpret_cast<uint4 *>(xs)[min(tid + 256 * j, nch - 1)] = xv[j];
    __syncthreads();

    float p[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) p[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < kFewSteps; ++s) {
        if (s < steps) {
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                const int r = rbase + i < t ? rbase + i : t - 1;  // rows past t repeat the last row, never stored
                const uint2 v = *reinterpret_cast<const uint2 *>(xs + r * h + s * 256 + 4 * lane);
                p[i] = __builtin_fmaf(bf16_lo(v.x), wv[s].x, p[i]);
                p[i] = __builtin_fmaf(bf16_hi(v.x), wv[s].y, p[i]);
                p[i] = __builtin_fmaf(bf16_lo(v.y), wv[s].z, p[i]);
                p[i] = __builtin_fmaf(bf16_hi(v.y), wv[s].w, p[i]);
            }
        }
    }
    const float v = tree64(p, lane);
    constexpr int shift = tree_shift(RT);
    if ((lane & ((1 << shift) - 1)) == 0) {
        const int r = rbase + (lane >> shift);
        if (r < t && e < E) logits[(size_t)r * E + e] = v;
    }
}

// Large-t router: a workgroup of 4 or 8 waves owns LR rows x LE experts;
// every 256-element step stages the rows' x chunks (widened once to fp32 on
// the way in) and the experts' W chunks in LDS, double-buffered, and each
// wave computes WR rows x WE experts from LDS (lane l still owns partial l
// of every logit).  Two shapes: 32 x 32 with 8 waves of 16 x 8 (128 KB of
// LDS, one workgroup per CU) where the chunk gives at least one workgroup
// per CU, else 16 x 16 with 4 waves of 8 x 8 (64 KB, two per CU), whose 4x
// more workgroups fill the GPU for mid-sized chunks (t = 512, E = 64:
// 20.5 -> 12.0 us; at t = 4096, E = 128 the 32 x 32 shape is faster, 47 vs 57 us).
// W (fp32, used as stored) goes from memory straight into its LDS buffer by
// DMA one step ahead; only x, which is widened, passes through registers
// (two steps ahead), so the registers the staging held are free for the
// compute loop's LDS reads.
template <int LR, int LE, int WR, int WE>
__global__ void __launch_bounds__(64 * (LR / WR) * (LE / WE), (LR * LE >= 1024) ? 1 : 2)
k_router_lds(const uint16_t *__restrict__ x, const float *__restrict__ w, int t, int h, int E,
             float *__restrict__ logits) {
    using namespace lds;
    constexpr int kWaves = (LR / WR) * (LE / WE);
    constexpr int kThreads = 64 * kWaves;
    constexpr int kXBytes = LR * 1024, kWBytes = LE * 1024; // staged bytes per step (x as fp32)
    constexpr int kWavesE = LE / WE;                        // waves along the experts
    // x: LR rows x 32 source chunks of 8 bf16 (16 bytes), kPer per thread;
    // W: LE rows of 1 KB, one DMA of 64 x 16 bytes each, kWPer per wave.
    constexpr int kPer = LR * 32 / kThreads, kWPer = LE / kWaves;
    static_assert(kPer * kThreads == LR * 32 && kWPer * kWaves == LE, "whole chunks per thread / wave");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_x[2][kXBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_w[2][kWBytes];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e_blocks = (E + LE - 1) / LE;
    const int r0 = (blockIdx.x / e_blocks) * LR, e0 = (blockIdx.x % e_blocks) * LE;
    const int wr = (wave / kWavesE) * WR, we = (wave % kWavesE) * WE;   // this wave's rows / experts

    // Rows past t read row t - 1 (computed, never stored), so every load is
    // unconditional and the compiler's wait counts stay exact.
    const uint8_t *src[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int ch = tid + kThreads * c;
        const int r = ch >> 5, q = ch & 31;
        src[c] = reinterpret_cast<const uint8_t *>(x + (size_t)min(r0 + r, t - 1) * h) + q * 16;
    }
    // Experts past E read row E - 1: computed, never stored.
    const i32x4 rw = buffer_rsrc(w);
    uint32_t wvo[kWPer];
#pragma unroll
    for (int j = 0; j < kWPer; ++j)
        wvo[j] = (uint32_t)min(e0 + wave * kWPer + j, E - 1) * (uint32_t)h * 4u + (uint32_t)lane * 16u;
    const uint32_t wl = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(&lds_w[0][0]));
    // step s covers elements [256 s, 256 s + 256): x bytes 512 s, W bytes 1024 s
    auto load_x = [&](int s, uint4 *v) {
#pragma unroll
        for (int c = 0; c < kPer; ++c)
            v[c] = *reinterpret_cast<const uint4 *>(src[c] + (size_t)s * 512);
    };
    auto load_w = [&](int s) {
#pragma unroll
        for (int j = 0; j < kWPer; ++j)
            dma16(wl + (s & 1) * kWBytes + (wave * kWPer + j) * 1024, wvo[j], rw, (uint32_t)s * 1024u);
    };

    constexpr int N = WR * WE;  // outputs of the wave
    static_assert(N == 64 || N == 128, "one or two outputs per lane");
    float p[N];
#pragma unroll
    for (int o = 0; o < N; ++o) p[o] = 0.0f;

    // Issue order: W of step s + 1, then x of step s + 2; so when step s + 1
    // starts, the compiler's wait for its x registers (everything but the
    // x loads of s + 2 complete) also covers its W, and wait_vm<kPer>
    // states it.  The loop is unrolled by two to keep each x register set in
    // fixed registers.  Past the last step the loads repeat the last step
    // into the free buffer, so every step waits for the same count.
    uint4 va[kPer], vb[kPer];
    const int steps = h >> 8;
    load_w(0);
    load_x(0, va);
    load_x(min(1, steps - 1), vb);
    auto step = [&](int s, uint4 (&v)[kPer]) {
        uint8_t *xb = lds_x[s & 1];
        const uint8_t *wb = lds_w[s & 1];
#pragma unroll
        for (int c = 0; c < kPer; ++c) {  // 8 bf16 -> 8 fp32 (exact)
            const int ch = tid + kThreads * c;
            const uint4 q = v[c];
            *reinterpret_cast<float4 *>(xb + ch * 32) = make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
            *reinterpret_cast<float4 *>(xb + ch * 32 + 16) = make_float4(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w));
        }
        wait_vm<kPer>();      // this step's W (only the x loads of s + 1 may be in flight)
        barrier_no_fence();   // x and W of step s are in LDS; buffers of s - 1 are free
        load_w(min(s + 1, steps - 1));
        load_x(min(s + 2, steps - 1), v);
        float wv[WE][4];
#pragma unroll
        for (int j = 0; j < WE; ++j) {
            const float4 q = *reinterpret_cast<const float4 *>(wb + (we + j) * 1024 + lane * 16);
            wv[j][0] = q.x;
            wv[j][1] = q.y;
            wv[j][2] = q.z;
            wv[j][3] = q.w;
        }
        // Rows in groups of four: the LDS reads of group g + 1 are issued
        // ahead of group g's FMAs, so a read's latency hides behind 4 WE x 4
        // FMAs instead of being waited for right after its issue.
        constexpr int G = WR / 4;
        float4 xq[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xq[0][i] = *reinterpret_cast<const float4 *>(xb + (wr + i) * 1024 + lane * 16);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xq[(g + 1) & 1][i] = *reinterpret_cast<const float4 *>(xb + (wr + 4 * (g + 1) + i) * 1024 + lane * 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 q = xq[g & 1][i];
#pragma unroll
                for (int j = 0; j < WE; ++j) {
                    float &acc = p[(4 * g + i) * WE + j];
                    acc = __builtin_fmaf(q.x, wv[j][0], acc);
                    acc = __builtin_fmaf(q.y, wv[j][1], acc);
                    acc = __builtin_fmaf(q.z, wv[j][2], acc);
                    acc = __builtin_fmaf(q.w, wv[j][3], acc);
                }
            }
            if (g + 1 < G) {
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);        // next group's reads first
                __builtin_amdgcn_sched_group_barrier(0x002, 16 * WE, 0);  // then this group's FMAs
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // Pairs without a condition inside, so that every entry to the loop head
    // has the same loads in flight (x of the step in va, then x of the next
    // in vb) and the compiler waits for va alone.
    int s = 0;
    for (; s + 1 < steps; s += 2) {
        step(s, va);
        step(s + 1, vb);
    }
    if (s < steps) step(s, va);
    wait_vm<0>();  // retire the trailing (repeated) loads

    // Transposed butterfly over the 64 partials: 6 splitting levels leave
    // N / 64 outputs per lane: output `lane` (N = 64), or outputs 2 lane and
    // 2 lane + 1 (N = 128); output o is row o / WE, expert o % WE.
    // Levels off = 32 and 16 use v_permlane32/16_swap: swapping the upper
    // lanes of p[o] with the lower lanes of p[o + half] hands each lane its
    // partner's copy of the output it keeps, so one add finishes the pair
    // (lane l < off: p_l + p_(l+off); lane l >= off: p_(l-off) + p_l).
#pragma unroll
    for (int o = 0; o < N / 2; ++o) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[o]), __float_as_uint(p[o + N / 2]), false, false);
        p[o] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
#pragma unroll
    for (int o = 0; o < N / 4; ++o) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[o]), __float_as_uint(p[o + N / 4]), false, false);
        p[o] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
#pragma unroll
    for (int lvl = 2; lvl < 6; ++lvl) {
        const int off = 32 >> lvl;
        const int half = N >> (lvl + 1);
        const uint32_t m = (lane & off) ? 0xffffffffu : 0u;
#pragma unroll
        for (int o = 0; o < half; ++o) {
            const uint32_t lo = __float_as_uint(p[o]), hi = __float_as_uint(p[o + half]);
            const float keep = __uint_as_float((lo & ~m) | (hi & m));
            const float give = __uint_as_float((hi & ~m) | (lo & m));
            p[o] = keep + __shfl_xor(give, off, 64);
        }
    }
    constexpr int PER = N / 64;
    const int o = PER * lane, i = o / WE, j = o % WE;
    const int r = r0 + wr + i, e = e0 + we + j;
    if (r < t) {
#pragma unroll
        for (int q = 0; q < PER; ++q)
            if (e + q < E) logits[(size_t)r * E + e + q] = p[q];
    }
}

template <int KPL>
__global__ void __launch_bounds__(256) k_topk(const float *__restrict__ logits, int t, int E, int k,
                                              uint32_t *__restrict__ idx, float *__restrict__ wts) {
    const int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (r >= t) return;
    topk_row<KPL>(logits, r, E, k, idx, wts);
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
    // t <= 8: rows staged once per workgroup, W rows held in registers;
    // small t: one row block and one expert per wave keeps >= E waves busy
    // streaming W; large t: LDS-shared 32 x 32 tiles.
    if (t >= 128 && E >= 32) {
        const int big = ((t + 31) / 32) * ((E + 31) / 32);
        if (big >= 256) {
            hipLaunchKernelGGL((k_router_lds<32, 32, 16, 8>), dim3(big), dim3(512), 0, s, x, w, t, h, E, logits);
        } else {
            const int blocks = ((t + 15) / 16) * ((E + 15) / 16);
            hipLaunchKernelGGL((k_router_lds<16, 16, 8, 8>), dim3(blocks), dim3(256), 0, s, x, w, t, h, E, logits);
        }
        return hipGetLastError();
    }
    if (t <= kFewRows && h <= kFewSteps * 256) {
        const dim3 grid((E + 3) / 4), grid2((E + 1) / 2), block(256);
        if (t == 1) hipLaunchKernelGGL((k_router_few<1, 1>), grid, block, 0, s, x, w, t, h, E, logits);
        else if (t == 2) hipLaunchKernelGGL((k_router_few<2, 1>), grid, block, 0, s, x, w, t, h, E, logits);
        else if (t <= 4) hipLaunchKernelGGL((k_router_few<4, 1>), grid, block, 0, s, x, w, t, h, E, logits);
        else hipLaunchKernelGGL((k_router_few<4, 2>), grid2, block, 0, s, x, w, t, h, E, logits);
        return hipGetLastError();
    }
    if (t >= 64 && E >= 8) return launch_tile<8, 8>(x, w, t, h, E, logits, s);
    if (t >= 8) return launch_tile<8, 1>(x, w, t, h, E, logits, s);
    if (t >= 4) return launch_tile<4, 1>(x, w, t, h, E, logits, s);
    if (t >= 2) return launch_tile<2, 1>(x, w, t, h, E, logits, s);
    return launch_tile<1, 1>(x, w, t, h, E, logits, s);
}

hipError_t launch_topk(const float *logits, int t, int E, int k, uint32_t *idx, float *wts,
                       hipStream_t s) {
    ProfileScope prof(MOE_PHASE_TOPK, s);
    const dim3 grid((t + 3) / 4), block(256);
    if (E <= 64) hipLaunchKernelGGL(k_topk<1>, grid, block, 0, s, logits, t, E, k, idx, wts);
    else if (E <= 128) hipLaunchKernelGGL(k_topk<2>, grid, block, 0, s, logits, t, E, k, idx, wts);
    else if (E <= 256) hipLaunchKernelGGL(k_topk<4>, grid, block, 0, s, logits, t, E, k, idx, wts);
    else if (E <= 512) hipLaunchKernelGGL(k_topk<8>, grid, block, 0, s, logits, t, E, k, idx, wts);
    else hipLaunchKernelGGL(k_topk<MOE_MAX_EXPERTS / 64>, grid, block, 0, s, logits, t, E, k, idx, wts);
    return hipGetLastError();
}

}  // namespace moe
