// Grouping of rows by expert (CSR) on the GPU, and the M-tile schedule.
//
// The cherenkov experts.rs page (fn prepare_expert_jobs) reads topk_idx back
// to the host, appends (row, weight) to a list per expert while walking rows
// in order, and concatenates the lists in expert order.  The same lists are
// built here without leaving the device:
//   1. k_csr_count: per tile of 64 rows, a 64-bit mask per expert of the
//      tile's rows that chose it (LDS atomics), and its popcount.
//   2. k_csr_scan:  one workgroup turns the per-tile counts into the
//      segment start of every (expert, tile) and the offsets array.
//   3. k_csr_place: every (row, slot) entry goes to
//      segment base + number of earlier rows of its tile in the mask.
// A row's k experts are distinct, so "earlier entries of expert e" are the
// entries of earlier rows: the placement is the stable order of the pages.
#include "moe_internal.h"
#include "topk_row.h"

namespace moe {
namespace {

constexpr int TR = kCsrTileRows;

// Inclusive scan over the 64 lanes of a wave with DPP moves only (no LDS
// crossbar): row_shr 1, 2, 4, 8 scan each 16-lane row, then row_bcast 15
// adds row 0's total to row 1 and row 2's to row 3, and row_bcast 31 adds
// the total of rows 0-1 to rows 2-3.  Lanes whose DPP source is missing, and
// rows outside a step's row mask, add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_add_step(uint32_t v) {
    return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
    v = dpp_add_step<0x111, 0xf>(v);  // row_shr:1
    v = dpp_add_step<0x112, 0xf>(v);  // row_shr:2
    v = dpp_add_step<0x114, 0xf>(v);  // row_shr:4
    v = dpp_add_step<0x118, 0xf>(v);  // row_shr:8
    v = dpp_add_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
    v = dpp_add_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
    return v;
}

// Inclusive scan of one value per thread over a workgroup of 1024 threads
// (16 waves): DPP scan in each wave, then the wave totals.  `wsum` is
// 16 words of LDS.  Returns the inclusive prefix; *total gets the sum.
__device__ __forceinline__ uint32_t block_scan_1024(uint32_t v, uint32_t *wsum, uint32_t *total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    v = wave_scan_incl(v);
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const uint32_t x = wsum[w];
        before += (w < wave) ? x : 0u;
        all += x;
    }
    __syncthreads();  // wsum may be reused by the caller's next scan
    *total = all;
    return v + before;
}

// Block of 256 threads per tile of 64 rows.  A thread's entries (at most 8:
// 64 rows x k <= 32) are loaded before any is used, so the kernel waits for
// memory once.
constexpr int kCountThreads = 256, kTileEntriesPer = TR * MOE_MAX_K / kCountThreads;
__global__ void __launch_bounds__(kCountThreads) k_csr_count(const uint32_t *__restrict__ idx, int t, int k,
                                                             int E, uint32_t *__restrict__ hist) {
    __shared__ unsigned long long mask[MOE_MAX_EXPERTS];
    const int tile = blockIdx.x;
    const int r0 = tile * TR;
    const int nr = min(TR, t - r0);
    const uint32_t *tidx = idx + (size_t)r0 * k;   // the tile's nr k entries, row-major
    uint32_t ev[kTileEntriesPer];
#pragma unroll
    for (int j = 0; j < kTileEntriesPer; ++j) {
        const int i = threadIdx.x + kCountThreads * j;
        ev[j] = i < nr * k ? tidx[i] : 0xffffffffu;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTileEntriesPer; ++j) {
        const int i = threadIdx.x + kCountThreads * j;
        if (ev[j] < (uint32_t)E) atomicOr(&mask[ev[j]], 1ull << (i / k));
    }
    __syncthreads();
    const int tiles = gridDim.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hist[(size_t)e * tiles + tile] = (uint32_t)__popcll(mask[e]);
}

// One workgroup of 1024 threads (16 waves).  Row tiles number at most
// 4096 / 64 = 64, so a wave scans one expert's per-tile counts (contiguous in
// hist) with lane = tile, 8 experts per pass with their loads issued
// together.  A block scan over the expert totals then gives the offsets, and
// every (expert, tile) entry becomes its absolute segment start.  With at most
// 128 experts (one pass) the per-tile prefixes stay in registers; beyond
// that they are re-read and re-scanned.
__global__ void __launch_bounds__(1024) k_csr_scan(int tiles, int E, int total,
                                                   uint32_t *__restrict__ hist,
                                                   uint32_t *__restrict__ offsets) {
    __shared__ uint32_t tot[MOE_MAX_EXPERTS];
    __shared__ uint32_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kPass = 8;
    uint32_t ex[kPass];  // exclusive per-tile prefix of the last pass
    auto pass = [&](int e0, bool totals) {
        uint32_t v[kPass];
#pragma unroll
        for (int j = 0; j < kPass; ++j)
            v[j] = (lane < tiles && e0 + j < E) ? hist[(size_t)(e0 + j) * tiles + lane] : 0u;
#pragma unroll
        for (int j = 0; j < kPass; ++j) {
            const uint32_t incl = wave_scan_incl(v[j]);
            ex[j] = incl - v[j];
            if (totals && e0 + j < E && lane == 63) tot[e0 + j] = incl;
        }
    };
    for (int e0 = wave * kPass; e0 < E; e0 += 16 * kPass) pass(e0, true);
    __syncthreads();
    uint32_t all;
    const uint32_t mine = tid < E ? tot[tid] : 0u;
    const uint32_t incl = block_scan_1024(mine, wsum, &all);
    if (tid < E) {
        tot[tid] = incl - mine;  // exclusive: segment start of expert tid
        offsets[tid] = incl - mine;
    }
    if (tid == 0) offsets[E] = (uint32_t)total;
    __syncthreads();
    const bool one_pass = E <= 16 * kPass;
    for (int e0 = wave * kPass; e0 < E; e0 += 16 * kPass) {
        if (!one_pass) pass(e0, false);
#pragma unroll
        for (int j = 0; j < kPass; ++j)
            if (lane < tiles && e0 + j < E) hist[(size_t)(e0 + j) * tiles + lane] = tot[e0 + j] + ex[j];
    }
}

// Placement of one 64-row tile's entries: its rows' masks per expert in LDS
// (again, as in the count), then every entry to its segment base plus the
// number of earlier rows of the tile that chose the same expert.  Any
// block size; `tiles` is the number of row tiles (the stride of base).
__device__ __forceinline__ void csr_place_body(int tile, int tiles, const uint32_t *__restrict__ idx,
                                               const float *__restrict__ wts, int t, int k, int E,
                                               const uint32_t *__restrict__ base, uint32_t *__restrict__ rows,
                                               float *__restrict__ csr_w, uint32_t *__restrict__ pos) {
    __shared__ unsigned long long mask[MOE_MAX_EXPERTS];
    const int r0 = tile * TR;
    const int nr = min(TR, t - r0);
    const size_t e0 = (size_t)r0 * k;              // the tile's first entry (row-major)
    // a thread's entries (at most 8 with 256 threads), loaded together once
    constexpr int kMaxPer = TR * MOE_MAX_K / 256;
    uint32_t ev[kMaxPer];
    float wv[kMaxPer];
    const int nt = blockDim.x;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
        const int i = threadIdx.x + nt * j;
        const bool in = i < nr * k;
        ev[j] = in ? idx[e0 + i] : 0xffffffffu;
        wv[j] = in ? wts[e0 + i] : 0.0f;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
        const int i = threadIdx.x + nt * j;
        if (ev[j] < (uint32_t)E) atomicOr(&mask[ev[j]], 1ull << (i / k));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
        const int i = threadIdx.x + nt * j, r = i / k;
        const uint32_t e = ev[j];
        if (e >= (uint32_t)E) continue;               // also every i >= nr k
        const unsigned long long below = (r == 0) ? 0ull : (mask[e] & ((1ull << r) - 1ull));
        const uint32_t p = base[(size_t)e * tiles + tile] + (uint32_t)__popcll(below);
        rows[p] = (uint32_t)(r0 + r);
        csr_w[p] = wv[j];
        pos[e0 + i] = p;
    }
}

__global__ void __launch_bounds__(256) k_csr_place(const uint32_t *__restrict__ idx,
                                                   const float *__restrict__ wts, int t, int k,
                                                   int E, const uint32_t *__restrict__ base,
                                                   uint32_t *__restrict__ rows,
                                                   float *__restrict__ csr_w,
                                                   uint32_t *__restrict__ pos) {
    csr_place_body(blockIdx.x, gridDim.x, idx, wts, t, k, E, base, rows, csr_w, pos);
}

// Small chunks (t <= kCsrSmallTiles * 64 rows): the same three steps in one
// workgroup of 1024 threads, with the masks, counts and segment starts in
// LDS, so a chunk of up to 512 rows costs one launch instead of three (mid
// chunk, t = 512: 13.7 -> 10.4 us; 96 KB of LDS).  Thread e
// owns expert e (E <= 1024).
constexpr int kCsrSmallTiles = 8;
// The body, also run by k_csr_schedule; `soff` (LDS, or nullptr) receives a
// copy of the offsets for the caller's next phase.
// PRELOAD: the entries come from global memory and are loaded once, all at
// once; otherwise (the merged decode kernel: from LDS, at most 16 rows) each
// pass reads them where they are.
template <bool PRELOAD>
__device__ __forceinline__ void csr_small_body(const uint32_t *__restrict__ idx,
                                               const float *__restrict__ wts, int t, int k, int E,
                                               uint32_t *__restrict__ offsets,
                                               uint32_t *__restrict__ rows,
                                               float *__restrict__ csr_w,
                                               uint32_t *__restrict__ pos, uint32_t *soff) {
    __shared__ unsigned long long mask[kCsrSmallTiles][MOE_MAX_EXPERTS];
    __shared__ uint32_t base[kCsrSmallTiles][MOE_MAX_EXPERTS];
    __shared__ uint32_t wsum[16];
    const int tid = threadIdx.x;
    const int tiles = (t + TR - 1) / TR;
    // The thread's entries i = tid + 1024 j (at most 16: t <= 512, k <= 32);
    // with PRELOAD loaded once and all at once, so the grouping waits for
    // memory once rather than once per entry in each of its two passes
    // (mid chunk, t = 512: block 0.1129 -> 0.1098 ms).
    constexpr int kPer = kCsrSmallTiles * TR * MOE_MAX_K / 1024;
    const int n = t * k;
    uint32_t ev[PRELOAD ? kPer : 1];
    float wv[PRELOAD ? kPer : 1];
    if constexpr (PRELOAD) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid + 1024 * j;
            ev[j] = i < n ? idx[i] : 0xffffffffu;
            wv[j] = i < n ? wts[i] : 0.0f;
        }
    }
    // only the chunk's own row tiles are read below
    for (int i = tid; i < tiles * MOE_MAX_EXPERTS; i += 1024) (&mask[0][0])[i] = 0ull;
    __syncthreads();
    if constexpr (PRELOAD) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid + 1024 * j, r = i / k;
            if (ev[j] < (uint32_t)E) atomicOr(&mask[r / TR][ev[j]], 1ull << (r % TR));
        }
    } else {
        for (int i = tid; i < n; i += 1024) {
            const int r = i / k;
            const uint32_t e = idx[i];
            if (e < (uint32_t)E) atomicOr(&mask[r / TR][e], 1ull << (r % TR));
        }
    }
    __syncthreads();
    // expert tid: counts per tile, total, then its segment start
    uint32_t cnt[kCsrSmallTiles], tot = 0;
#pragma unroll
    for (int j = 0; j < kCsrSmallTiles; ++j) {
        cnt[j] = (tid < E && j < tiles) ? (uint32_t)__popcll(mask[j][tid]) : 0u;
        tot += cnt[j];
    }
    uint32_t all;
    const uint32_t start = block_scan_1024(tot, wsum, &all) - tot;
    if (tid < E) {
        offsets[tid] = start;
        if (soff) soff[tid] = start;
        uint32_t b = start;
#pragma unroll
        for (int j = 0; j < kCsrSmallTiles; ++j) {
            base[j][tid] = b;
            b += cnt[j];
        }
    }
    if (tid == 0) {
        offsets[E] = (uint32_t)(t * k);
        if (soff) soff[E] = (uint32_t)(t * k);
    }
    __syncthreads();
    auto place = [&](int i, uint32_t e, float w) {
        const int r = i / k, tile = r / TR, rr = r % TR;
        if (e >= (uint32_t)E) return;   // also every preloaded i >= t k
        const unsigned long long below = (rr == 0) ? 0ull : (mask[tile][e] & ((1ull << rr) - 1ull));
        const uint32_t p = base[tile][e] + (uint32_t)__popcll(below);
        rows[p] = (uint32_t)r;
        csr_w[p] = w;
        pos[i] = p;
    };
    if constexpr (PRELOAD) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) place(tid + 1024 * j, ev[j], wv[j]);
    } else {
        for (int i = tid; i < n; i += 1024) place(i, idx[i], wts[i]);
    }
}

__global__ void __launch_bounds__(1024) k_csr_small(const uint32_t *__restrict__ idx,
                                                    const float *__restrict__ wts, int t, int k, int E,
                                                    uint32_t *__restrict__ offsets,
                                                    uint32_t *__restrict__ rows,
                                                    float *__restrict__ csr_w,
                                                    uint32_t *__restrict__ pos) {
    csr_small_body<true>(idx, wts, t, k, E, offsets, rows, csr_w, pos, nullptr);
}

// One workgroup builds the M-tile schedule of experts [e0, e1):
//   1. tiles of up to bm rows per expert, in ascending expert id (kept in LDS);
//   2. each XCD gets a contiguous share of those tiles of about one eighth of
//      the total cost (kTileCostBase + token blocks per tile), so an expert's
//      tiles share one L2;
//   3. within its share, an XCD lists the shared expert's tiles, then every
//      tile of the experts with several tiles (in expert order, so an
//      expert's tiles run back to back and reuse its weights from L2), then
//      the one-tile experts by token blocks, descending, so the cheapest
//      tiles fill the end of the launch;
//   4. every listed tile is written as a TileEntry (rows, expert, record
//      address) to order[x * xcap + j].
// sched_n[kSchedXcnt + x] is the number of tiles of XCD x, sched_n[0] the total.
// Whether a schedule fills its tiles with all threads (see schedule_body):
// when a segment of up to `rows` rows can span more than four tiles.
__host__ __device__ __forceinline__ bool sched_parallel(int rows, int bm) { return (rows + bm - 1) / bm > 4; }

template <int MAXT>
__device__ __forceinline__ void schedule_body(const uint32_t *offsets, int e0, int e1, int bm,
                                              const uint64_t *__restrict__ records,
                                              uint32_t *__restrict__ sched_n,
                                              TileEntry *__restrict__ order, int xcap, SharedSeg sh,
                                              bool par) {
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t tp0[MAXT];   // first CSR position of each tile
    __shared__ uint16_t tex[MAXT];   // expert of each tile
    __shared__ uint8_t tbl[MAXT];    // token blocks (32 rows) of each tile
    __shared__ uint8_t trows[MAXT];  // rows of each tile - 1
    __shared__ uint8_t xof[MAXT];    // XCD of each tile
    __shared__ uint16_t tne[MAXT];   // tiles of its expert
    __shared__ uint16_t perm[MAXT];  // listing position -> tile
    __shared__ uint64_t erec[MOE_MAX_EXPERTS + 1]; // record address of each expert (+ shared)
    __shared__ uint32_t tfirst[MOE_MAX_EXPERTS + 2]; // first tile of each segment, then the total
    __shared__ uint32_t xstart[9];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // 1. tiles in expert order.  Each thread counts the tiles of a contiguous
    // run of experts and a scan gives every segment's first tile.  When a
    // segment can hold many tiles (`par`: the chunk's rows span more than four
    // tiles) the tiles are then filled by all threads at once, tile i by the
    // thread i mod 1024, which finds its segment by binary search over the
    // first tiles, so the shared expert's segment (t rows) does not fall to
    // one thread (full chunk: 13.2 -> 10.0 us with the listing below); else
    // each thread fills its own segments' few tiles.  Local index n_e (after
    // the routed experts) is the shared expert's segment when the call has
    // one.
    const int n_e = e1 - e0;
    const int n_all = n_e + (sh.rec ? 1 : 0);
    const int per = (n_all + 1023) / 1024;
    const int a = tid * per, b = min(n_all, a + per);
    auto seg = [&](int le, uint32_t &p0, uint32_t &n) {
        if (le < n_e) {
            p0 = offsets[e0 + le];
            n = offsets[e0 + le + 1] - p0;
        } else {
            p0 = (uint32_t)sh.p0;
            n = (uint32_t)sh.n;
        }
    };
    uint32_t cnt = 0;
    for (int le = a; le < b; ++le) {
        uint32_t p0, n;
        seg(le, p0, n);
        cnt += (n + bm - 1) / bm;
        erec[le] = le < n_e ? records[e0 + le] : (uint64_t)(uintptr_t)sh.rec;
    }
    uint32_t T;
    uint32_t w = block_scan_1024(cnt, wsum, &T) - cnt;
    // The tile arrays hold MAXT tiles and each XCD's list xcap: offsets that
    // would need more (never those of a chunk whose size the host checked)
    // schedule nothing rather than write past them.  T is the same in every
    // thread, so the whole workgroup leaves together.
    if (T > (uint32_t)MAXT || T > (uint32_t)xcap) {
        if (tid < 16) sched_n[tid] = 0u;
        return;
    }
    if (!par) {
        for (int le = a; le < b; ++le) {
            uint32_t p0, n;
            seg(le, p0, n);
            const uint32_t ne = (n + bm - 1) / bm;
            uint32_t m = 0;
            for (uint32_t j = 0; j < ne; ++j, m += bm, ++w) {
                const uint32_t rows = min((uint32_t)bm, n - m);
                tp0[w] = p0 + m;
                tex[w] = (uint16_t)le;
                trows[w] = (uint8_t)(rows - 1);
                tne[w] = (uint16_t)ne;
                tbl[w] = (uint8_t)((rows + 31) / 32);
            }
        }
    } else {
        for (int le = a; le < b; ++le) {
            uint32_t p0, n;
            seg(le, p0, n);
            tfirst[le] = w;
            w += (n + bm - 1) / bm;
        }
        if (tid == 0) tfirst[n_all] = T;
        __syncthreads();
        for (uint32_t i = tid; i < T; i += 1024) {
            // the last segment whose first tile is <= i holds tile i (empty
            // segments share the next one's first tile, so the last match is
            // the segment with tiles)
            int lo = 0, hi = n_all;  // tfirst[lo] <= i < tfirst[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (tfirst[mid] <= i) lo = mid;
                else hi = mid;
            }
            uint32_t p0, n;
            seg(lo, p0, n);
            const uint32_t j = i - tfirst[lo], m = j * (uint32_t)bm;
            const uint32_t rows = min((uint32_t)bm, n - m);
            tp0[i] = p0 + m;
            tex[i] = (uint16_t)lo;
            trows[i] = (uint8_t)(rows - 1);
            tne[i] = (uint16_t)(tfirst[lo + 1] - tfirst[lo]);
            tbl[i] = (uint8_t)((rows + 31) / 32);
        }
    }
    __syncthreads();
    // 2. cost prefix over tiles; tile i goes to XCD floor(8 (S_i + c_i / 2) / C)
    const uint32_t per2 = (T + 1023) / 1024;
    const uint32_t a2 = min(T, tid * per2), b2 = min(T, a2 + per2);
    uint32_t csum = 0;
    for (uint32_t i = a2; i < b2; ++i) csum += kTileCostBase + tbl[i];
    uint32_t Ctot;
    uint64_t S = block_scan_1024(csum, wsum, &Ctot) - csum;
    const uint64_t C = Ctot;
    for (uint32_t i = a2; i < b2; ++i) {
        const uint32_t c = kTileCostBase + tbl[i];
        xof[i] = (uint8_t)min<uint64_t>(7, (8 * (2 * S + c)) / (2 * C));
        S += c;
    }
    if (tid < 9) xstart[tid] = T;
    __syncthreads();
    // share starts: tile i opens every XCD in (x of tile i-1, x of tile i]
    for (uint32_t i = a2; i < b2; ++i) {
        const int lo = i ? (int)xof[i - 1] + 1 : 0;
        for (int x = lo; x <= (int)xof[i]; ++x) xstart[x] = i;
    }
    __syncthreads();
    // 3. wave x lists XCD x's tiles by class, descending, and in tile order
    // within a class (a stable partition).  The shared expert's tiles come
    // first (class 9): its rows are dense and, in small chunks, its tiles
    // stream far more weight bytes than a routed tile.  Every tile of an
    // expert with several tiles takes class 4, so the expert's tiles, its
    // last partial one included, run back to back while its weights are in
    // the XCD's L2 (full chunk, against listing partial tiles by their own
    // token blocks: gate/up fetches 440 instead of 535 MB, down 182 instead
    // of 230 MB, block 0.455 -> 0.448 ms).  The experts with one tile follow
    // by token blocks, descending, so the last workgroups an XCD starts are
    // its cheapest and the launch ends with short tiles.
    // A counting sort without branches: one pass over the XCD's tiles counts
    // each class (a ballot per class), the counts give each class's first
    // position, and a second pass places every tile at its class's position
    // plus the number of tiles of its class before it.
    static_assert(kMaxBM <= 128, "token-block classes 1-4");
    if (wave < 8) {
        const uint32_t s0 = xstart[wave], s1 = xstart[wave + 1];
        auto cls_of = [&](uint32_t i) {
            return i < s1 ? ((int)tex[i] == n_e ? 9 : tne[i] > 1 ? 4 : (int)tbl[i]) : 0;
        };
        constexpr int kClasses = 5;
        constexpr int kCls[kClasses] = {9, 4, 3, 2, 1};  // listing order
        uint32_t next[kClasses];                         // next free position of each class
        {
            uint32_t cnt_c[kClasses] = {0, 0, 0, 0, 0};
            for (uint32_t base = s0; base < s1; base += 64) {
                const int c = cls_of(base + lane);
#pragma unroll
                for (int q = 0; q < kClasses; ++q) cnt_c[q] += (uint32_t)__popcll(__ballot(c == kCls[q]));
            }
            uint32_t acc = s0;
#pragma unroll
            for (int q = 0; q < kClasses; ++q) {
                next[q] = acc;
                acc += cnt_c[q];
            }
        }
        const unsigned long long below = (1ull << lane) - 1ull;
        for (uint32_t base = s0; base < s1; base += 64) {
            const uint32_t i = base + lane;
            const int c = cls_of(i);
            uint32_t pos = 0;
#pragma unroll
            for (int q = 0; q < kClasses; ++q) {
                const unsigned long long m = __ballot(c == kCls[q]);
                pos = c == kCls[q] ? next[q] + (uint32_t)__popcll(m & below) : pos;
                next[q] += (uint32_t)__popcll(m);
            }
            if (i < s1) perm[pos] = (uint16_t)i;
        }
        if (lane == 0) sched_n[kSchedXcnt + wave] = s1 - s0;
    }
    __syncthreads();
    // 4. position q of the listing belongs to the XCD of its tile, at index
    // q - xstart of that XCD.
    for (uint32_t q = tid; q < T; q += 1024) {
        const uint32_t i = perm[q];
        const uint32_t x = xof[i];
        TileEntry te;
        te.p0 = (int)tp0[i];
        te.n = (int)trows[i] + 1;
        te.expert = e0 + (int)tex[i];
        te.tiles = (int)tne[i];
        te.rec = reinterpret_cast<const void *>(erec[tex[i]]);
        te.done = 0;
        te.pad2 = 0;
        order[(size_t)x * xcap + (q - xstart[x])] = te;
    }
    if (tid == 0) sched_n[0] = T;
}

__global__ void __launch_bounds__(1024) k_schedule(const uint32_t *__restrict__ offsets, int e0,
                                                   int e1, int bm, const uint64_t *__restrict__ records,
                                                   uint32_t *__restrict__ sched_n,
                                                   TileEntry *__restrict__ order, int xcap,
                                                   SharedSeg sh, int par) {
    schedule_body<kSchedMaxTiles>(offsets, e0, e1, bm, records, sched_n, order, xcap, sh, par != 0);
}

// Chunks of up to kCsrSmallTiles * 64 rows: grouping and schedule in one
// workgroup and one launch (the offsets pass from one phase to the next in
// LDS); the schedule's tile arrays are sized for such chunks.
constexpr int kSchedSmallTiles = 2048;
static_assert(kCsrSmallTiles * 64 * MOE_MAX_K / kMinBM + MOE_MAX_EXPERTS + kCsrSmallTiles * 64 / kMinBM + 2 <=
                  kSchedSmallTiles, "tiles of a small chunk");
__global__ void __launch_bounds__(1024) k_csr_schedule(const uint32_t *__restrict__ idx,
                                                       const float *__restrict__ wts, int t, int k, int E,
                                                       uint32_t *__restrict__ offsets,
                                                       uint32_t *__restrict__ rows,
                                                       float *__restrict__ csr_w,
                                                       uint32_t *__restrict__ pos, int bm,
                                                       const uint64_t *__restrict__ records,
                                                       uint32_t *__restrict__ sched_n,
                                                       TileEntry *__restrict__ order, int xcap,
                                                       SharedSeg sh) {
    __shared__ uint32_t soff[MOE_MAX_EXPERTS + 1];
    csr_small_body<true>(idx, wts, t, k, E, offsets, rows, csr_w, pos, soff);
    __syncthreads();
    schedule_body<kSchedSmallTiles>(soff, 0, E, bm, records, sched_n, order, xcap, sh, sched_parallel(t, bm));
}

// Larger chunks, after the scan (k_csr_scan): the placement (workgroups
// 0 .. tiles-1, one per 64-row tile) and the schedule (the last workgroup)
// in one launch.  Both need only the scan's offsets and segment bases, so
// neither waits for the other (full chunk: scan + schedule, then placement,
// 10.6 + 5.1 us, became scan, then placement with the schedule, 4.8 + 7.7
// us; block 0.4547 -> 0.4522 ms).
__global__ void __launch_bounds__(1024) k_place_schedule(const uint32_t *__restrict__ idx,
                                                         const float *__restrict__ wts, int t, int k, int E,
                                                         int tiles, const uint32_t *__restrict__ base,
                                                         uint32_t *__restrict__ rows, float *__restrict__ csr_w,
                                                         uint32_t *__restrict__ pos,
                                                         const uint32_t *__restrict__ offsets, int bm,
                                                         const uint64_t *__restrict__ records,
                                                         uint32_t *__restrict__ sched_n,
                                                         TileEntry *__restrict__ order, int xcap, SharedSeg sh) {
    if ((int)blockIdx.x == tiles) {
        __shared__ uint32_t soff[MOE_MAX_EXPERTS + 1];
        for (int e = threadIdx.x; e <= E; e += 1024) soff[e] = offsets[e];
        __syncthreads();
        schedule_body<kSchedMaxTiles>(soff, 0, E, bm, records, sched_n, order, xcap, sh,
                                      sched_parallel(tiles * TR, bm));
        return;
    }
    csr_place_body(blockIdx.x, tiles, idx, wts, t, k, E, base, rows, csr_w, pos);
}


constexpr int kTopkCsrRows = 16;   // one wave per row in a 1024-thread workgroup
// Decode-sized chunks (t <= 16): the top-k of each row (one wave per row),
// then grouping and schedule, in one workgroup and one launch.  The top-k
// results pass to the grouping in LDS, and the experts' record addresses
// are read while the top-k runs.
template <int KPL>
__global__ void __launch_bounds__(1024) k_topk_csr_schedule(const float *__restrict__ logits, int t, int E, int k,
                                                            uint32_t *__restrict__ idx, float *__restrict__ wts,
                                                            uint32_t *__restrict__ offsets,
                                                            uint32_t *__restrict__ rows,
                                                            float *__restrict__ csr_w,
                                                            uint32_t *__restrict__ pos, int bm,
                                                            const uint64_t *__restrict__ records,
                                                            uint32_t *__restrict__ sched_n,
                                                            TileEntry *__restrict__ order, int xcap,
                                                            SharedSeg sh) {
    __shared__ uint32_t soff[MOE_MAX_EXPERTS + 1];
    __shared__ uint32_t sidx[kTopkCsrRows * MOE_MAX_K];
    __shared__ float swts[kTopkCsrRows * MOE_MAX_K];
    __shared__ uint64_t srec[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x, wave = tid >> 6;
    // the record addresses load while the rows' top-k runs
    const uint64_t rec = tid < E ? records[tid] : 0ull;
    if (wave < t) topk_row<KPL>(logits, wave, E, k, idx, wts, sidx, swts);
    if (tid < E) srec[tid] = rec;
    __syncthreads();
    csr_small_body<false>(sidx, swts, t, k, E, offsets, rows, csr_w, pos, soff);
    __syncthreads();
    schedule_body<kSchedSmallTiles>(soff, 0, E, bm, srec, sched_n, order, xcap, sh, sched_parallel(t, bm));
}

}  // namespace

hipError_t launch_csr(const uint32_t *idx, const float *wts, int t, int k, int E,
                      uint32_t *offsets, uint32_t *rows, float *csr_w, uint32_t *pos,
                      uint32_t *hist, hipStream_t s) {
    const int tiles = (t + TR - 1) / TR;
    ProfileScope prof(MOE_PHASE_CSR, s);
    if (tiles <= kCsrSmallTiles) {
        hipLaunchKernelGGL(k_csr_small, dim3(1), dim3(1024), 0, s, idx, wts, t, k, E, offsets, rows, csr_w, pos);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_csr_count, dim3(tiles), dim3(256), 0, s, idx, t, k, E, hist);
    hipLaunchKernelGGL(k_csr_scan, dim3(1), dim3(1024), 0, s, tiles, E, t * k, hist, offsets);
    hipLaunchKernelGGL(k_csr_place, dim3(tiles), dim3(256), 0, s, idx, wts, t, k, E, hist, rows,
                       csr_w, pos);
    return hipGetLastError();
}

bool csr_schedule_fits(int t) { return (t + TR - 1) / TR <= kCsrSmallTiles; }

hipError_t launch_csr_with_schedule(const uint32_t *idx, const float *wts, int t, int k, int E, uint32_t *offsets,
                                    uint32_t *rows, float *csr_w, uint32_t *pos, uint32_t *hist, int bm,
                                    const uint64_t *records, uint32_t *sched_n, TileEntry *order, int xcap,
                                    SharedSeg sh, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_CSR, s);
    const int tiles = (t + TR - 1) / TR;
    hipLaunchKernelGGL(k_csr_count, dim3(tiles), dim3(256), 0, s, idx, t, k, E, hist);
    hipLaunchKernelGGL(k_csr_scan, dim3(1), dim3(1024), 0, s, tiles, E, t * k, hist, offsets);
    hipLaunchKernelGGL(k_place_schedule, dim3(tiles + 1), dim3(1024), 0, s, idx, wts, t, k, E, tiles, hist, rows,
                       csr_w, pos, offsets, bm, records, sched_n, order, xcap, sh);
    return hipGetLastError();
}
bool topk_csr_schedule_fits(int t) { return t <= kTopkCsrRows; }

hipError_t launch_topk_csr_schedule(const float *logits, int t, int E, int k, uint32_t *idx, float *wts,
                                    uint32_t *offsets, uint32_t *rows, float *csr_w, uint32_t *pos, int bm,
                                    const uint64_t *records, uint32_t *sched_n, TileEntry *order, int xcap,
                                    SharedSeg sh, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_CSR, s);
#define MOE_TCS(KPL)                                                                                            \
    hipLaunchKernelGGL(k_topk_csr_schedule<KPL>, dim3(1), dim3(1024), 0, s, logits, t, E, k, idx, wts, offsets, \
                       rows, csr_w, pos, bm, records, sched_n, order, xcap, sh)
    if (E <= 64) MOE_TCS(1);
    else if (E <= 128) MOE_TCS(2);
    else if (E <= 256) MOE_TCS(4);
    else if (E <= 512) MOE_TCS(8);
    else MOE_TCS(MOE_MAX_EXPERTS / 64);
#undef MOE_TCS
    return hipGetLastError();
}

hipError_t launch_csr_schedule(const uint32_t *idx, const float *wts, int t, int k, int E, uint32_t *offsets,
                               uint32_t *rows, float *csr_w, uint32_t *pos, int bm, const uint64_t *records,
                               uint32_t *sched_n, TileEntry *order, int xcap, SharedSeg sh, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_CSR, s);
    hipLaunchKernelGGL(k_csr_schedule, dim3(1), dim3(1024), 0, s, idx, wts, t, k, E, offsets, rows, csr_w, pos, bm,
                       records, sched_n, order, xcap, sh);
    return hipGetLastError();
}

hipError_t launch_schedule(const uint32_t *offsets, int e0, int e1, int bm, int rows_bound,
                           const uint64_t *records, uint32_t *sched_n, TileEntry *order, int xcap, hipStream_t s,
                           SharedSeg sh) {
    ProfileScope prof(MOE_PHASE_SCHEDULE, s);
    hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), 0, s, offsets, e0, e1, bm, records, sched_n, order,
                       xcap, sh, sched_parallel(rows_bound, bm) ? 1 : 0);
    return hipGetLastError();
}

}  // namespace moe
