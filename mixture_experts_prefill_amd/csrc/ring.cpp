// Expert ring (the streaming scheme of the cherenkov prefill pages: consts
// RING = 64 and GROUP = 8 on the prefill.rs page; fn prepare_expert_jobs,
// fn pf_experts and fn read_expert_batch on the experts.rs page).
//
// Jobs are the non-empty experts in ascending id.  A job whose record is not
// resident gets slot = (its ordinal among streamed jobs) % n_slots.  Jobs are
// cut into batches of `group`.  The pages' host thread spins until the GPU
// has signalled batch bi - RING/GROUP before reading batch bi into the ring,
// then signals "fetched" for bi; the GPU waits for "fetched" before running
// the batch and signals "done" after.  Here the same protocol runs entirely
// on the GPU's queues: the copy stream waits on the compute stream's "done"
// event of batch bi - n_slots/group, copies the batch's records from pinned
// host memory, and records "fetched"; the compute stream waits on "fetched",
// runs the batch's grouped GEMMs and records "done".  The host only enqueues.
//
// Each batch holds at most `group` streamed jobs, so a slot's previous user
// is at least n_slots/group batches earlier: waiting on batch
// bi - n_slots/group covers it (the pages' comment says "at most"; the code
// waits on exactly that batch, which is the safe bound).
#include "ring.h"
#include "../../include/moe_debug.h"

#include <chrono>
#include <cstdlib>
#include <cstring>
#include <thread>

namespace moe {

void ring_plan(const uint32_t *offsets, const uint64_t *resident, int E, int n_slots, int group,
               RingPlan *plan) {
    plan->jobs.clear();
    plan->batch_first.clear();
    plan->wait_batch.clear();
    int ring_pos = 0;
    for (int e = 0; e < E; ++e) {
        const int n = (int)(offsets[e + 1] - offsets[e]);
        if (n == 0) continue;
        RingJob j{e, n, resident[e] ? 0 : 1, -1};
        if (j.streamed) j.slot = ring_pos++ % n_slots;
        plan->jobs.push_back(j);
    }
    const int nj = (int)plan->jobs.size();
    const int lag = n_slots / group;
    for (int b = 0; b * group < nj; ++b) {
        plan->batch_first.push_back(b * group);
        plan->wait_batch.push_back(b >= lag ? b - lag : -1);
    }
    plan->batch_first.push_back(nj);
}

static moe_status ensure_events(RingState &st, size_t n) {
    while (st.fetched.size() < n) {
        hipEvent_t f, d;
        hipError_t e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "ring event");
        e = hipEventCreateWithFlags(&d, hipEventDisableTiming);
        if (e != hipSuccess) {
            hipEventDestroy(f);
            return hip_fail(e, "ring event");
        }
        st.fetched.push_back(f);
        st.done.push_back(d);
    }
    return MOE_OK;
}

moe_status ring_run(moe_ring *ring, const void *const *host_records, GemmArgs a, int bm,
                    const uint32_t *offsets, const uint32_t *csr_pos, const float *csr_w, int t,
                    int k, int E, const moe_layout *L, float *out, int accumulate,
                    uint64_t *jobs_dev, hipStream_t s) {
    if (!ring) return fail(MOE_ERR_INVALID, "experts: host records given without a ring");
    RingState &st = ring->st;
    if (st.stride != L->stride) return fail(MOE_ERR_INVALID, "experts: ring slot size %llu != record stride %llu",
                                            (unsigned long long)st.stride, (unsigned long long)L->stride);
    // Read offsets and the residency table back (the pages read topk back
    // here: experts.rs page, fn prepare_expert_jobs).  The host blocks until
    // the stream has reached this point; that time is the call's host wait.
    hipError_t e = hipMemcpyAsync(st.h_offsets, offsets, sizeof(uint32_t) * (E + 1), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(st.h_records, a.records, sizeof(uint64_t) * E, hipMemcpyDeviceToHost, s);
    const auto sync0 = std::chrono::steady_clock::now();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "experts: offsets read-back");
    double wait_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - sync0).count();

    RingPlan plan;
    ring_plan(st.h_offsets, st.h_records, E, st.n_slots, st.group, &plan);
    int streamed = 0;
    for (const RingJob &j : plan.jobs)
        if (j.streamed) {
            if (!host_records || !host_records[j.expert])
                return fail(MOE_ERR_INVALID, "experts: expert %d is not resident and has no host record", j.expert);
            ++streamed;
        }
    const int nb = (int)plan.batch_first.size() - 1;
    if (moe_status rc = ensure_events(st, (size_t)nb)) return rc;

    // Record address per expert for this call: resident address or slot.
    std::memset(st.h_jobs, 0, sizeof(uint64_t) * E);
    for (const RingJob &j : plan.jobs)
        st.h_jobs[j.expert] = j.streamed ? (uint64_t)(st.slots + (size_t)j.slot * st.stride)
                                         : st.h_records[j.expert];
    e = hipMemcpyAsync(jobs_dev, st.h_jobs, sizeof(uint64_t) * E, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "experts: job table upload");
    a.records = jobs_dev;

    // Slots may still be read by the previous call on this ring: copies start
    // after everything already enqueued on the compute stream.
    e = hipEventRecord(st.start, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(st.copy, st.start, 0);
    if (e != hipSuccess) return hip_fail(e, "experts: ring start");

    // Slot reuse is ordered on the GPU (the copy stream waits on "done"), so
    // the host does not wait in this loop; only the test delay below sleeps.
    for (int b = 0; b < nb; ++b) {
        const int j0 = plan.batch_first[b], j1 = plan.batch_first[b + 1];
        if (plan.wait_batch[b] >= 0) {
            const int wb = plan.wait_batch[b];
            e = hipStreamWaitEvent(st.copy, st.done[wb], 0);
            if (e != hipSuccess) return hip_fail(e, "experts: wait for slot reuse");
            if (st.poison) {
                // The slots written by batch wb are free now; poison them so a
                // read before their next copy would show.
                for (int j = plan.batch_first[wb]; j < plan.batch_first[wb + 1]; ++j)
                    if (plan.jobs[j].streamed) {
                        e = hipMemsetAsync(st.slots + (size_t)plan.jobs[j].slot * st.stride, 0xFF, st.stride, st.copy);
                        if (e == hipSuccess && st.lowbit)
                            e = hipMemsetAsync(st.staging + (size_t)plan.jobs[j].slot * st.miss.stride, 0xFF,
                                               st.miss.stride, st.copy);
                        if (e != hipSuccess) return hip_fail(e, "experts: poison");
                    }
            }
        }
        // Streamed records: straight into their ring slot, or, in the 2-bit
        // miss layout, into the slot's staging area (expanded below).  A run
        // of streamed jobs whose host records follow one another (the next
        // job's record starts where this one ends) goes out as one copy: their
        // slots follow one another too (a batch's streamed jobs take
        // consecutive slots and never wrap), and each copy has a fixed cost
        // on the link that per-record copies pay once per record.
        const uint64_t rec_bytes = st.lowbit ? st.miss.stride : st.stride;
        if (!st.skip_copy)
            for (int j = j0; j < j1;) {
                const RingJob &jb = plan.jobs[j];
                if (!jb.streamed) {
                    ++j;
                    continue;
                }
                uint8_t *dst = st.lowbit ? st.staging + (size_t)jb.slot * st.miss.stride
                                         : st.slots + (size_t)jb.slot * st.stride;
                const uint8_t *src = static_cast<const uint8_t *>(host_records[jb.expert]);
                uint64_t bytes = rec_bytes;
                int jn = j + 1;
                while (jn < j1 && plan.jobs[jn].streamed && plan.jobs[jn].slot == plan.jobs[jn - 1].slot + 1 &&
                       static_cast<const uint8_t *>(host_records[plan.jobs[jn].expert]) == src + bytes) {
                    bytes += rec_bytes;
                    ++jn;
                }
                e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st.copy);
                if (e != hipSuccess) return hip_fail(e, "experts: ring copy");
                j = jn;
            }
        e = hipEventRecord(st.fetched[b], st.copy);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, st.fetched[b], 0);
        if (e != hipSuccess) return hip_fail(e, "experts: fetched event");
        if (st.lowbit) {
            // the batch's 2-bit records become the 4-bit records its GEMMs read
            ExpandArgs x = expand_args(L, &st.miss);
            for (int j = j0; j < j1; ++j) {
                const RingJob &jb = plan.jobs[j];
                if (!jb.streamed) continue;
                x.job[x.n++] = ExpandJob{st.staging + (size_t)jb.slot * st.miss.stride,
                                         st.slots + (size_t)jb.slot * st.stride};
                if (x.n == kExpandMax) {
                    e = launch_expand2(x, s);
                    if (e != hipSuccess) return hip_fail(e, "experts: expand low-bit records");
                    x.n = 0;
                }
            }
            if (x.n > 0) {
                e = launch_expand2(x, s);
                if (e != hipSuccess) return hip_fail(e, "experts: expand low-bit records");
            }
        }

        const int e0 = plan.jobs[j0].expert, e1 = plan.jobs[j1 - 1].expert + 1;
        e = launch_schedule(offsets, e0, e1, bm, t, a.records, const_cast<uint32_t *>(a.sched_n),
                            const_cast<TileEntry *>(a.order), a.xcap, s);
        if (e != hipSuccess) return hip_fail(e, "experts: schedule");
        int rows = 0;
        for (int j = j0; j < j1; ++j) rows += plan.jobs[j].rows;
        a.max_tiles = rows / bm + (j1 - j0) + 1;
        a.w_off = L->gate_w;
        a.sb_off = L->gate_sb;
        a.w2_off = L->up_w;
        a.sb2_off = L->up_sb;
        a.act = nullptr;
        e = launch_gateup(a, bm, s);
        if (e != hipSuccess) return hip_fail(e, "experts: gate/up");
        a.act = a.hg;
        a.w_off = L->down_w;
        a.sb_off = L->down_sb;
        e = launch_down(a, bm, s);
        if (e != hipSuccess) return hip_fail(e, "experts: down");
        e = hipEventRecord(st.done[b], s);
        if (e != hipSuccess) return hip_fail(e, "experts: done event");
        if (st.delay_us > 0) {
            const auto w0 = std::chrono::steady_clock::now();
            std::this_thread::sleep_for(std::chrono::microseconds(st.delay_us));
            wait_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - w0).count();
        }
    }
    e = launch_combine(a.ye, csr_pos, csr_w, t, k, L->hidden, out, accumulate, s);
    if (e != hipSuccess) return hip_fail(e, "experts: combine");

    st.stats.jobs = (int)plan.jobs.size();
    st.stats.streamed = streamed;
    st.stats.batches = nb;
    st.stats.fetched_bytes = st.skip_copy ? 0 : (uint64_t)streamed * (st.lowbit ? st.miss.stride : st.stride);
    st.stats.wait_ms = wait_ms;
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_ring_create(const moe_layout *L, void *slots, int32_t n_slots, int32_t group,
                           moe_ring **out) {
    if (!L || !slots || !out) return fail(MOE_ERR_INVALID, "ring: null pointer");
    moe_layout ref;
    if (moe_layout_make(L->hidden, L->inter, L->group, &ref) != MOE_OK || std::memcmp(&ref, L, sizeof ref))
        return fail(MOE_ERR_INVALID, "ring: layout not made by moe_layout_make");
    if (group < 1 || n_slots < group || n_slots % group)
        return fail(MOE_ERR_INVALID, "ring: need n_slots >= group >= 1 and n_slots %% group == 0 (got %d, %d)", n_slots, group);
    moe_ring *r = new moe_ring();
    RingState &st = r->st;
    st.stride = L->stride;
    st.slots = static_cast<uint8_t *>(slots);
    st.n_slots = n_slots;
    st.group = group;
    const char *p = std::getenv("MOE_RING_POISON");
    st.poison = p && *p && *p != '0';
    const char *d = std::getenv("MOE_RING_DELAY_US");
    st.delay_us = d ? std::atoi(d) : 0;
    const char *sk = std::getenv("MOE_RING_SKIP_COPY");
    st.skip_copy = sk && *sk && *sk != '0';
    hipError_t e = hipStreamCreateWithFlags(&st.copy, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st.start, hipEventDisableTiming);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void **>(&st.h_offsets), sizeof(uint32_t) * (MOE_MAX_EXPERTS + 1), hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void **>(&st.h_records), sizeof(uint64_t) * MOE_MAX_EXPERTS, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void **>(&st.h_jobs), sizeof(uint64_t) * MOE_MAX_EXPERTS, hipHostMallocDefault);
    if (e != hipSuccess) {
        moe_ring_destroy(r);
        return hip_fail(e, "ring create");
    }
    *out = r;
    return MOE_OK;
}

void moe_ring_destroy(moe_ring *r) {
    if (!r) return;
    RingState &st = r->st;
    if (st.copy) hipStreamSynchronize(st.copy);
    for (hipEvent_t ev : st.fetched) hipEventDestroy(ev);
    for (hipEvent_t ev : st.done) hipEventDestroy(ev);
    if (st.start) hipEventDestroy(st.start);
    if (st.copy) hipStreamDestroy(st.copy);
    if (st.h_offsets) hipHostFree(st.h_offsets);
    if (st.h_records) hipHostFree(st.h_records);
    if (st.h_jobs) hipHostFree(st.h_jobs);
    delete r;
}

moe_status moe_ring_set_miss_layout(moe_ring *ring, const moe_layout *Lmiss, void *staging) {
    if (!ring) return fail(MOE_ERR_INVALID, "ring miss layout: null ring");
    RingState &st = ring->st;
    if (!Lmiss) {
        st.lowbit = false;
        st.staging = nullptr;
        return MOE_OK;
    }
    moe_layout ref;
    if (moe_layout_make_bits(Lmiss->hidden, Lmiss->inter, Lmiss->group, Lmiss->bits, &ref) != MOE_OK ||
        std::memcmp(&ref, Lmiss, sizeof ref) || Lmiss->bits != 2)
        return fail(MOE_ERR_INVALID, "ring miss layout: a 2-bit layout made by moe_layout_make_bits is required");
    moe_layout L4;
    if (moe_layout_make(Lmiss->hidden, Lmiss->inter, Lmiss->group, &L4) != MOE_OK || L4.stride != st.stride)
        return fail(MOE_ERR_INVALID, "ring miss layout: shape (h %d, inter %d, group %d) differs from the ring's",
                    Lmiss->hidden, Lmiss->inter, Lmiss->group);
    if (!staging || (reinterpret_cast<uintptr_t>(staging) & 15))
        return fail(MOE_ERR_INVALID, "ring miss layout: staging must be a 16-byte aligned device buffer");
    st.miss = *Lmiss;
    st.staging = static_cast<uint8_t *>(staging);
    st.lowbit = true;
    return MOE_OK;
}

moe_status moe_ring_get_stats(const moe_ring *ring, moe_ring_stats *out) {
    if (!ring || !out) return fail(MOE_ERR_INVALID, "ring stats: null pointer");
    *out = ring->st.stats;
    return MOE_OK;
}

// Host-only view of the ring schedule, for tests: fills slot[e] (-1 resident
// or empty), batch[e] (-1 empty) and wait[b] for the given offsets and
// residency.  Returns the number of batches.
int moe_ring_plan_debug(const uint32_t *offsets, const uint64_t *resident, int32_t E, int32_t n_slots,
                        int32_t group, int32_t *slot, int32_t *batch, int32_t *wait) {
    RingPlan plan;
    ring_plan(offsets, resident, E, n_slots, group, &plan);
    for (int e = 0; e < E; ++e) slot[e] = batch[e] = -1;
    const int nb = (int)plan.batch_first.size() - 1;
    for (int b = 0; b < nb; ++b) {
        for (int j = plan.batch_first[b]; j < plan.batch_first[b + 1]; ++j) {
            slot[plan.jobs[j].expert] = plan.jobs[j].slot;
            batch[plan.jobs[j].expert] = b;
        }
        wait[b] = plan.wait_batch[b];
    }
    return nb;
}

}  // extern "C"
