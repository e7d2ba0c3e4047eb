/*
 * moe_debug.h -- inspection and measurement hooks of libmoe, for tests and
 * benchmarks.
 *
 * moe_ring_plan_debug: the expert ring's host schedule for one call, without
 * touching a GPU.  offsets [E+1] as produced by moe_build_csr; resident [E]
 * nonzero for experts whose record is in device memory; n_slots and group as
 * given to moe_ring_create.  Fills slot[e] (ring slot of a streamed expert,
 * -1 if resident or without rows), batch[e] (batch of expert e, -1 without
 * rows) and wait[b] (the batch whose completion gates batch b's copies, -1 if
 * none; wait must hold at least E entries).  Returns the number of batches.
 * The schedule follows the experts.rs page (fns prepare_expert_jobs and
 * pf_experts): jobs are the non-empty experts in ascending id, slot =
 * ordinal among streamed jobs mod n_slots, batches of `group` jobs, and batch
 * b's copies wait for batch b - n_slots/group.
 */
#ifndef MOE_DEBUG_H
#define MOE_DEBUG_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
int moe_ring_plan_debug(const uint32_t *offsets, const uint64_t *resident, int32_t E, int32_t n_slots,
                        int32_t group, int32_t *slot, int32_t *batch, int32_t *wait);

/*
 * Per-kernel timing.  moe_profile_begin(mask) makes later calls on this
 * process record a pair of HIP events on their own stream around every
 * kernel launch whose phase bit is set in `mask` (bit p = phase p below);
 * moe_profile_end synchronises those events, writes the summed milliseconds
 * and launch counts per phase into ms[MOE_PHASES] and launches[MOE_PHASES]
 * (either may be NULL), and stops recording.  Returns the number of timed
 * launches, or -1 on a HIP error.  Not thread safe; meant for benchmarks.
 */
enum {
    MOE_PHASE_ROUTER = 0,      /* router logits */
    MOE_PHASE_TOPK = 1,        /* top-k and weights */
    MOE_PHASE_CSR = 2,         /* CSR count, scan and place */
    MOE_PHASE_SHARED_GU = 3,   /* shared expert gate/up + SiLU*up */
    MOE_PHASE_SHARED_DOWN = 4, /* shared expert down, writes out */
    MOE_PHASE_SCHEDULE = 5,    /* M-tile schedule */
    MOE_PHASE_GATEUP = 6,      /* routed grouped gate/up + SiLU*up */
    MOE_PHASE_DOWN = 7,        /* routed grouped down */
    MOE_PHASE_COMBINE = 8,     /* weighted combine into out */
    MOE_PHASE_NORM = 9,        /* injection into the residual copies and the next norm */
    MOE_PHASE_EXPERTS = 10,    /* routed grouped gate/up + SiLU*up and down in one launch */
    MOE_PHASES = 11
};
void moe_profile_begin(uint32_t mask);
int moe_profile_end(double *ms, int64_t *launches);
/*
 * Changes which phases later launches time, keeping the events already
 * recorded since moe_profile_begin (mask 0 pauses timing), so that a
 * benchmark can time a sample of its steps' launches.
 */
void moe_profile_set_mask(uint32_t mask);

/*
 * HBM read probe, the reference point of the HBM-bound kernels: one launch
 * that reads `bytes` of device memory at `src` once (16-byte non-temporal
 * loads, four in flight per thread, `blocks` workgroups of 256 threads in a
 * grid-stride loop) and keeps nothing but a word per workgroup in `sink`
 * (u32 [blocks], written only for one unlikely checksum, so the loads cannot
 * be dropped).  Time it with events on `stream`: bytes / time is the read
 * bandwidth a plain streaming kernel reaches on this device.  src 16-byte
 * aligned, bytes a multiple of 16, 1 <= blocks <= 65536.  Returns 0, 1 for
 * bad arguments, 5 for a launch error.
 */
int moe_debug_read_probe(const void *src, size_t bytes, int32_t blocks, uint32_t *sink, void *stream);

/*
 * Which XCD (accelerator complex die) each workgroup of a launch runs on,
 * for the test of what the merged gate/up + down launch relies on: a
 * launch of `blocks` workgroups of 64 threads writes xcc[i] = the hardware
 * XCC id of workgroup i (u32 [blocks], device).  The merged launch needs
 * workgroups whose ids agree modulo 8 to share an XCD (and so an L2).
 * 1 <= blocks <= 1 << 20.  Returns 0, 1 for bad arguments, 5 for a launch
 * error.
 */
int moe_debug_xcc_map(uint32_t *xcc, int32_t blocks, void *stream);

/*
 * The wait of the merged gate/up + down launch, for tests of its give-up
 * path.  A down workgroup polls its tile's completion count (an atomic round
 * trip and a short sleep per poll) at most `spins` times (0: the default of
 * 32768, tens of milliseconds); if the count is still short it writes bf16
 * NaN over its rows and features of the down output instead of computing
 * them, so the block's output shows the failure.  extra = 1 makes every
 * down workgroup wait for one completion more than its tile can reach,
 * which forces that path (with a small `spins`, a launch still ends in
 * well under a second); 0 is normal operation.  Applies to launches enqueued
 * after the call, process-wide.  0 <= spins <= 32768, extra 0 or 1.  Returns
 * 0, or 1 for bad arguments.
 */
int moe_debug_tile_wait(int32_t spins, int32_t extra);

/*
 * The grouped GEMMs' tile schedule alone, for tests: the schedule kernel
 * that moe_prefill_experts and moe_prefill_fused enqueue before their GEMMs,
 * run on a CSR `offsets` [E+1] (device memory, non-decreasing) for experts
 * 0 .. E-1 with M-tiles of `bm` rows (32, 64 or 128; `rows_bound` >= 0, the
 * most rows a segment can hold, only picks how the kernel fills its tiles:
 * the schedule is the same for any value), each entry's record
 * address taken from `records` [E] (device memory; only copied), plus an
 * optional segment of shared_n dense rows at positions shared_p0 .. with
 * record address shared_rec (NULL: none).  Writes sched_n (u32 [16], device:
 * [0] = tiles, [8 + x] = tiles listed for XCD x) and `order` (device,
 * [8][xcap] entries of 32 bytes {int32 p0, n, expert, tiles; u64 rec; u32 done = 0, 0}:
 * XCD x's list from entry x * xcap).  The schedule refuses, on the device, a
 * call whose tiles exceed xcap or its own capacity: it then sets sched_n to
 * zero and writes no entry.  Returns 0, 1 for bad arguments, 5 for a launch
 * error.
 */
int moe_debug_schedule(const uint32_t *offsets, int32_t E, int32_t bm, int32_t rows_bound, const uint64_t *records,
                       const void *shared_rec, int32_t shared_p0, int32_t shared_n, uint32_t *sched_n,
                       void *order, int32_t xcap, void *stream);
#ifdef __cplusplus
}
#endif
#endif
