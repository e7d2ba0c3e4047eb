// Internal declarations shared by the HIP kernels and the host API of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "../../include/moe_debug.h"
#include "profile.h"

namespace moe {

// ------------------------------------------------------------------ workspace

// Disjoint regions of the caller's workspace, 256-byte aligned.
struct Workspace {
    size_t csr_hist;   // u32 [row_tiles][E]: per-tile expert counts, then segment bases
    size_t sched_n;    // u32 [16]: number of M-tiles; [kSchedXcnt + x]: tiles of XCD x
    size_t order;      // TileEntry [8][max_tiles]: per XCD, its tiles in run order
    size_t jobs;       // u64 [E]: record address per expert for the ring path
    size_t hg;         // bf16 [t*k][I]: SiLU(gate)*up of every CSR entry
    size_t ye;         // bf16 [t*k][h]: down projection of every CSR entry
    size_t hs;         // bf16 [t][I_s]: shared expert's SiLU(gate)*up
    size_t part;       // f32 split-K partial sums of the shared expert (small t only)
    size_t gate;       // f32 [t]: shared-expert gate factors
    size_t total;
};

constexpr int kCsrTileRows = 64;  // rows per CSR tile (one 64-bit mask per expert)
constexpr int kMinBM = 32;        // smallest GEMM M-tile
constexpr int kMaxBM = 128;       // largest GEMM M-tile
constexpr int kSchedMaxTiles = 8192;  // tiles one schedule can hold (>= t*k/kMinBM + E + 1)
constexpr int kSchedXcnt = 8;     // sched_n[kSchedXcnt + x] = tiles of XCD x
// Relative cost of an M-tile with b token blocks of 32 rows: kTileCostBase + b
// (per-workgroup timestamps put a gate/up tile at about 28 + 7.3 b us: the
// weight dequantisation of the tile costs about as much as four token blocks
// of MFMAs; 4 measured 1% faster than 5 for the full chunk).
constexpr int kTileCostBase = 4;

bool workspace_plan(int t, int k, int E, const moe_layout *routed, const moe_layout *shared,
                    Workspace *out);

// ------------------------------------------------------------------ launchers
// Every launcher only enqueues; arguments were validated by the caller.

hipError_t launch_router_logits(const uint16_t *x, const float *w, int t, int h, int E,
                                float *logits, hipStream_t s);
hipError_t launch_topk(const float *logits, int t, int E, int k, uint32_t *idx, float *wts,
                       hipStream_t s);
hipError_t launch_csr(const uint32_t *idx, const float *wts, int t, int k, int E,
                      uint32_t *offsets, uint32_t *rows, float *csr_w, uint32_t *pos,
                      uint32_t *hist, hipStream_t s);

// One M-tile of the grouped GEMMs: CSR rows [p0, p0 + n) of `expert`, the
// expert's record, and the number of M-tiles of the expert's segment (1:
// this tile is the only reader of the expert's weights).  `done` counts the
// tile's finished gate/up workgroups in the merged gate/up + down launch
// (written 0 by the schedule, then only by L2 atomics).
struct TileEntry {
    int p0, n, expert, tiles;
    const void *rec;
    uint32_t done, pad2;
};
static_assert(sizeof(TileEntry) == 32, "one 32-byte load per tile");

// M-tile schedule of the grouped GEMMs: for experts [e0, e1) with rows, tiles of
// up to bm rows (sched, sched_n[0]), split over the 8 XCDs by cost and listed
// per XCD (order[x * xcap ..], sched_n[kSchedXcnt + x]) with each entry's
// record address taken from records[expert].
// Optional extra segment of dense rows (the shared expert) scheduled with the
// routed experts: n rows at CSR-like positions p0 .. p0+n-1, record rec
// (rec == nullptr: none).  Its tiles are listed first on their XCD.
struct SharedSeg {
    const void *rec;
    int p0, n;
};
// rows_bound: the most rows a segment can hold (the chunk's t); only picks
// how the tiles are filled, any value gives the same schedule.
hipError_t launch_schedule(const uint32_t *offsets, int e0, int e1, int bm, int rows_bound,
                           const uint64_t *records, uint32_t *sched_n, TileEntry *order, int xcap, hipStream_t s,
                           SharedSeg sh = SharedSeg{nullptr, 0, 0});

// Grouping and schedule in one workgroup and one launch, for chunks whose
// CSR fits the one-workgroup path (csr_schedule_fits).
bool csr_schedule_fits(int t);
// Larger chunks: count, then scan and schedule in one launch, then place.
hipError_t launch_csr_with_schedule(const uint32_t *idx, const float *wts, int t, int k, int E, uint32_t *offsets,
                                    uint32_t *rows, float *csr_w, uint32_t *pos, uint32_t *hist, int bm,
                                    const uint64_t *records, uint32_t *sched_n, TileEntry *order, int xcap,
                                    SharedSeg sh, hipStream_t s);
// ... and, for decode-sized chunks, the top-k too (its own launch otherwise).
bool topk_csr_schedule_fits(int t);
hipError_t launch_topk_csr_schedule(const float *logits, int t, int E, int k, uint32_t *idx, float *wts,
                                    uint32_t *offsets, uint32_t *rows, float *csr_w, uint32_t *pos, int bm,
                                    const uint64_t *records, uint32_t *sched_n, TileEntry *order, int xcap,
                                    SharedSeg sh, hipStream_t s);
hipError_t launch_csr_schedule(const uint32_t *idx, const float *wts, int t, int k, int E, uint32_t *offsets,
                               uint32_t *rows, float *csr_w, uint32_t *pos, int bm, const uint64_t *records,
                               uint32_t *sched_n, TileEntry *order, int xcap, SharedSeg sh, hipStream_t s);

struct GemmArgs {
    // B-operand rows (tokens): x rows gathered through `rows` (routed gate/up),
    // identity rows (shared gate/up), or consecutive rows of `act` (down).
    const uint16_t *x;       // bf16 [t][h] block input
    const uint32_t *rows;    // CSR row list (routed gate/up) or nullptr
    const uint16_t *act;     // bf16 activations for the down projection
    const uint64_t *records; // device table of record addresses, per expert
    const void *record;      // the one record (shared expert) when records == nullptr
    const uint32_t *sched_n;
    const TileEntry *order;  // per-XCD tile lists (routed) or nullptr (dense rows 0..t)
    int xcap;                // stride of order between XCDs
    int max_tiles;           // bound on M-tiles of the call
    int t;                   // rows (dense mode)
    int hidden, inter, group;
    uint64_t w_off, sb_off, w2_off, sb2_off;  // sections: gate & up (gate/up), down (down)
    // outputs
    uint16_t *hg;            // gate/up: bf16 [rows][inter]
    uint16_t *ye;            // down routed: bf16 [t*k][hidden]
    float *out;              // down shared: fp32 [t][hidden]
    const float *gate;       // shared gate factors or nullptr
    int accumulate;
    int ksplit;              // dense calls: K ranges run by separate workgroups (1 = none)
    float *part;             // split partial sums [ksplit][t][2 I or h]
    // Routed gate/up with the shared expert in the same launch: positions
    // p >= shared_p0 are the shared expert's rows, x row p - shared_p0
    // (only when shared_rows != 0).
    int shared_rows, shared_p0;
    // Merged gate/up + down launch: the gate/up workgroups per tile, whose
    // completion a down workgroup waits for, a zero the kernel adds
    // atomically to read the count, and the most polls of the count before
    // the workgroup gives up (and writes NaN in place of its outputs).
    int wait_need, wait_zero, wait_spins;
};
// Merged launch wait settings for tests (moe_debug_tile_wait): the poll
// limit (0: the default) and a number added to the count a down workgroup
// waits for (0; above 0 the wait cannot complete and every down workgroup
// takes its give-up path).
void tile_wait_debug(int *spins, int *extra);
// Staged-row bytes of the few-row path in 32-row tiles (the row ring of
// k_gemm<MODE, 32, 4>); the kernel checks that the two agree.
constexpr int kFewRowBytes = 16384;
// Whether a routed launch over K inputs (h for gate/up, I for down) of a
// call of t rows runs as a few-row launch (k_gemm<MODE, 32, 4, true>): every
// tile then has t <= 2 rows whose whole K fits the row ring, and the waves
// split the K steps, each keeping at least 16 (with 6 per wave, the down
// projection of the decode-shaped t = 1 chunk, each workgroup's start-up
// outweighed the split: 11.5 -> 22 us).
inline bool few_row_launch(int t, int K) {
    return t >= 1 && t <= 2 && ((t * K * 2 + 1023) / 1024) * 1024 <= kFewRowBytes && (K / 64) % 4 == 0 &&
           K / 64 / 4 >= 16;
}

hipError_t launch_gateup(const GemmArgs &a, int bm, hipStream_t s);
// The routed gate/up and down projections in one launch (k_gemm_gu_down),
// for routed launches that are not few-row launches (gateup_down_merged).
bool gateup_down_merged(const GemmArgs &a, int bm);
hipError_t launch_gateup_down(const GemmArgs &gu, const GemmArgs &dn, int bm, hipStream_t s);
hipError_t launch_down(const GemmArgs &a, int bm, hipStream_t s);
hipError_t launch_reduce_gu(const float *part, int S, int t, int I, uint16_t *hs, hipStream_t s);
hipError_t launch_reduce_down(const float *part, int S, int t, int h, const float *gate, float *out,
                              int accumulate, hipStream_t s);
// K splits of the shared expert's dense GEMMs: for small chunks, so that
// enough workgroups stream the weights; a divisor of the K step count.
int shared_ksplit(int t, int ksteps, int nblk);
hipError_t launch_shared_gate(const uint16_t *x, const uint16_t *gate_w, int t, int h, float *g,
                              hipStream_t s);
// ys (optional): bf16 [t][h] shared-expert rows added first, scaled by gate[r]
// when gate is given.
hipError_t launch_combine(const uint16_t *ye, const uint32_t *pos, const float *csr_w, int t,
                          int k, int h, float *out, int accumulate, hipStream_t s,
                          const uint16_t *ys = nullptr, const float *gate = nullptr);

// The block output injected into the n residual copies and read by the next
// fused norm (norm.hip).  With ye set, y is formed from the down projections
// as the combine forms it (ye, pos, csr_w, k, ys, gate as for launch_combine)
// and never written; otherwise y is the fp32 [t][h] buffer (or nullptr: no
// injection).
struct NextNormArgs {
    const uint16_t *ye;
    const uint32_t *pos;
    const float *csr_w;
    const uint16_t *ys;
    const float *gate;
    const float *y;
    int t, k, h, n;
    float *hyper;          // fp32 [t][n][h], updated in place
    float alpha[MOE_MAX_HC], beta[MOE_MAX_HC];
    const float *gamma;    // fp32 [h]
    // h <= kNormMaxHidden (8 columns per thread per 2048, at most 8 chunks)
    float eps;
    uint16_t *mixed;       // bf16 [t][h]
};
// 2-bit miss records expanded into 4-bit records (lowbit.hip): up to
// kExpandMax records per launch, src in the miss layout, dst in the routed one.
constexpr int kExpandMax = 16;
struct ExpandJob {
    const uint8_t *src;
    uint8_t *dst;
};
struct ExpandArgs {
    ExpandJob job[kExpandMax];
    int n;
    uint64_t src_w[3], src_sb[3], dst_w[3], dst_sb[3];  // gate, up, down sections
    uint32_t tiles[3];                                   // code tiles of each matrix
    uint32_t sb_bytes[3];                                // scale/bias bytes of each matrix
};
ExpandArgs expand_args(const moe_layout *L4, const moe_layout *L2);
hipError_t launch_expand2(const ExpandArgs &a, hipStream_t s);

// Experts ranked by row count (residency.hip): counts from offsets, or from
// a top-k (topk_idx non-null, tk = t*k entries); counts may be nullptr.
hipError_t launch_rank_experts(const uint32_t *offsets, const uint32_t *topk_idx, int tk, int E, int budget,
                               uint32_t *counts, uint32_t *order, uint8_t *keep, hipStream_t s);
// Row statistics of a grouped chunk (residency.hip), into device memory.
hipError_t launch_chunk_stats(const uint32_t *offsets, int t, int E, moe_chunk_stats *stats, hipStream_t s);

constexpr int kNormMaxHidden = 16384;
hipError_t launch_next_norm(const NextNormArgs &a, hipStream_t s);

}  // namespace moe
