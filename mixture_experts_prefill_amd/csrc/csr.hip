// Grouping of rows by expert (CSR) on the GPU, and the M-tile schedule.
//
// The cherenkov experts.rs page (fn prepare_expert_jobs) reads topk_idx back
// to the host, appends (row, weight) to a list per expert while walking rows
// in order, and concatenates the lists in expert order.  The same lists are
// built here without leaving the device:
//   1. k_csr_count: per tile of 64 rows, a 64-bit mask per expert of the
//      tile's rows that chose it (LDS atomics), and its popcount.
//   2. k_csr_scan:  one workgroup turns the per-tile counts into the
//      segment start of every (tile, expert) and the offsets array.
//   3. k_csr_place: every (row, slot) entry goes to
//      segment base + number of earlier rows of its tile in the mask.
// A row's k experts are distinct, so "earlier entries of expert e" are the
// entries of earlier rows: the placement is the stable order of the pages.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TR = kCsrTileRows;

// Block of 256 threads per tile of 64 rows.
__global__ void __launch_bounds__(256) k_csr_count(const uint32_t *__restrict__ idx, int t, int k,
                                                   int E, uint32_t *__restrict__ hist) {
    __shared__ unsigned long long mask[MOE_MAX_EXPERTS];
    const int tile = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
    __syncthreads();
    const int r0 = tile * TR;
    const int nr = min(TR, t - r0);
    for (int i = threadIdx.x; i < nr * k; i += blockDim.x) {
        const int r = i / k;
        const uint32_t e = idx[(size_t)(r0 + r) * k + (i % k)];
        if (e < (uint32_t)E) atomicOr(&mask[e], 1ull << r);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hist[(size_t)tile * E + e] = (uint32_t)__popcll(mask[e]);
}

// One workgroup of 1024 threads (16 waves).  Row tiles number at most
// 4096 / 64 = 64, so a wave scans one expert's per-tile counts with lane =
// tile (shuffle scan), 8 experts per pass with their loads issued together.
// A block scan over the expert totals then gives the offsets, and every
// (tile, expert) entry becomes its absolute segment start.
__global__ void __launch_bounds__(1024) k_csr_scan(int tiles, int E, int total,
                                                   uint32_t *__restrict__ hist,
                                                   uint32_t *__restrict__ offsets) {
    __shared__ uint32_t tot[1024];
    __shared__ uint32_t part[1024];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kPass = 8;
    for (int e0 = wave * kPass; e0 < E; e0 += 16 * kPass) {
        uint32_t v[kPass];
#pragma unroll
        for (int j = 0; j < kPass; ++j)
            v[j] = (lane < tiles && e0 + j < E) ? hist[(size_t)lane * E + e0 + j] : 0u;
#pragma unroll
        for (int j = 0; j < kPass; ++j) {
            uint32_t incl = v[j];
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t o = __shfl_up(incl, d, 64);
                if (lane >= d) incl += o;
            }
            if (e0 + j < E) {
                if (lane < tiles) hist[(size_t)lane * E + e0 + j] = incl - v[j];
                if (lane == 63) tot[e0 + j] = incl;
            }
        }
    }
    __syncthreads();
    const uint32_t mine = tid < E ? tot[tid] : 0u;
    part[tid] = mine;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // Hillis-Steele inclusive scan
        const uint32_t o = tid >= d ? part[tid - d] : 0u;
        __syncthreads();
        part[tid] += o;
        __syncthreads();
    }
    if (tid < E) {
        tot[tid] = part[tid] - mine;  // exclusive: segment start of expert tid
        offsets[tid] = part[tid] - mine;
    }
    if (tid == 0) offsets[E] = (uint32_t)total;
    __syncthreads();
    for (int e0 = wave * kPass; e0 < E; e0 += 16 * kPass)
#pragma unroll
        for (int j = 0; j < kPass; ++j)
            if (lane < tiles && e0 + j < E) hist[(size_t)lane * E + e0 + j] += tot[e0 + j];
}

__global__ void __launch_bounds__(256) k_csr_place(const uint32_t *__restrict__ idx,
                                                   const float *__restrict__ wts, int t, int k,
                                                   int E, const uint32_t *__restrict__ base,
                                                   uint32_t *__restrict__ rows,
                                                   float *__restrict__ csr_w,
                                                   uint32_t *__restrict__ pos) {
    __shared__ unsigned long long mask[MOE_MAX_EXPERTS];
    const int tile = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
    __syncthreads();
    const int r0 = tile * TR;
    const int nr = min(TR, t - r0);
    for (int i = threadIdx.x; i < nr * k; i += blockDim.x) {
        const int r = i / k;
        const uint32_t e = idx[(size_t)(r0 + r) * k + (i % k)];
        if (e < (uint32_t)E) atomicOr(&mask[e], 1ull << r);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nr * k; i += blockDim.x) {
        const int r = i / k;
        const size_t src = (size_t)(r0 + r) * k + (i % k);
        const uint32_t e = idx[src];
        if (e >= (uint32_t)E) continue;
        const unsigned long long below = (r == 0) ? 0ull : (mask[e] & ((1ull << r) - 1ull));
        const uint32_t p = base[(size_t)tile * E + e] + (uint32_t)__popcll(below);
        rows[p] = (uint32_t)(r0 + r);
        csr_w[p] = wts[src];
        pos[src] = p;
    }
}

// One workgroup: tiles of bm rows for experts [e0, e1), in ascending expert id.
__global__ void __launch_bounds__(1024) k_schedule(const uint32_t *__restrict__ offsets, int e0,
                                                   int e1, int bm, int4 *__restrict__ sched,
                                                   uint32_t *__restrict__ sched_n) {
    __shared__ uint32_t part[1024];
    const int tid = threadIdx.x;
    const int n_e = e1 - e0;
    // each thread owns a contiguous run of experts
    const int per = (n_e + 1023) / 1024;
    const int a = e0 + tid * per, b = min(e1, a + per);
    uint32_t cnt = 0;
    for (int e = a; e < b; ++e) cnt += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
    part[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        uint32_t v = (tid >= d) ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    uint32_t w = part[tid] - cnt;
    for (int e = a; e < b; ++e) {
        const uint32_t p0 = offsets[e], n = offsets[e + 1] - p0;
        for (uint32_t m = 0; m < n; m += bm)
            sched[w++] = make_int4(e, (int)(p0 + m), (int)min((uint32_t)bm, n - m), 0);
    }
    if (tid == 1023) sched_n[0] = part[1023];
}

}  // namespace

hipError_t launch_csr(const uint32_t *idx, const float *wts, int t, int k, int E,
                      uint32_t *offsets, uint32_t *rows, float *csr_w, uint32_t *pos,
                      uint32_t *hist, hipStream_t s) {
    const int tiles = (t + TR - 1) / TR;
    ProfileScope prof(MOE_PHASE_CSR, s);
    hipLaunchKernelGGL(k_csr_count, dim3(tiles), dim3(256), 0, s, idx, t, k, E, hist);
    hipLaunchKernelGGL(k_csr_scan, dim3(1), dim3(1024), 0, s, tiles, E, t * k, hist, offsets);
    hipLaunchKernelGGL(k_csr_place, dim3(tiles), dim3(256), 0, s, idx, wts, t, k, E, hist, rows,
                       csr_w, pos);
    return hipGetLastError();
}

hipError_t launch_schedule(const uint32_t *offsets, int e0, int e1, int bm, int4 *sched,
                           uint32_t *sched_n, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_SCHEDULE, s);
    hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), 0, s, offsets, e0, e1, bm, sched, sched_n);
    return hipGetLastError();
}

}  // namespace moe
