// Expert ring: records that are not resident stream from pinned host memory
// through device slots, batch by batch, on a copy stream guarded by events.
#pragma once

#include <hip/hip_runtime.h>

#include <vector>

#include "moe_internal.h"

namespace moe {

moe_status fail(moe_status st, const char *fmt, ...);
moe_status hip_fail(hipError_t e, const char *what);

// Pure host schedule of one call: which slot each streamed job uses, which
// batch it belongs to, and which earlier batch must be done before the
// batch's copies may start.  Kept free of HIP calls so it can be tested on
// the CPU.
struct RingJob {
    int expert;
    int rows;
    int streamed;   // 1 = copied into `slot`, 0 = resident
    int slot;       // ring slot, -1 if resident
};
struct RingPlan {
    std::vector<RingJob> jobs;         // non-empty experts, ascending id
    std::vector<int> batch_first;      // first job of each batch (+ sentinel = jobs.size())
    std::vector<int> wait_batch;       // batch whose "done" gates this batch's copies, -1 = none
};
// offsets [E+1], resident[e] != 0 if expert e is in device memory.
void ring_plan(const uint32_t *offsets, const uint64_t *resident, int E, int n_slots, int group,
               RingPlan *plan);

struct RingState {
    uint64_t stride = 0;
    uint8_t *slots = nullptr;
    int n_slots = 0, group = 0;
    hipStream_t copy = nullptr;
    hipEvent_t start = nullptr;
    std::vector<hipEvent_t> fetched, done;
    // pinned host staging: offsets and the record table read back, and the
    // per-expert address table sent to the device
    uint32_t *h_offsets = nullptr;
    uint64_t *h_records = nullptr;
    uint64_t *h_jobs = nullptr;
    // Streamed records in a 2-bit miss layout (moe_ring_set_miss_layout):
    // copied into staging slots, then expanded into the 4-bit ring slots.
    bool lowbit = false;
    moe_layout miss{};
    uint8_t *staging = nullptr;
    moe_ring_stats stats{};
    bool poison = false;      // fill released slots with 0xFF before reuse (test hook)
    int delay_us = 0;         // host sleep between batch enqueues (test hook)
    bool skip_copy = false;   // run on whatever the slots hold (timing hook)
};

moe_status ring_run(moe_ring *ring, const void *const *host_records, GemmArgs a, int bm,
                    const uint32_t *offsets, const uint32_t *csr_pos, const float *csr_w, int t,
                    int k, int E, const moe_layout *L, float *out, int accumulate,
                    uint64_t *jobs_dev, hipStream_t s);

}  // namespace moe

struct moe_ring {
    moe::RingState st;
};
