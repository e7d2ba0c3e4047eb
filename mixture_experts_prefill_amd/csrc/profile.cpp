// Optional per-kernel timing with HIP events (declared in moe_debug.h).
#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/moe_debug.h"
#include "profile.h"

namespace moe {
namespace {
struct Mark {
    int phase;
    hipEvent_t a, b;
};
uint32_t g_mask = 0;
std::vector<Mark> g_marks;
std::vector<hipEvent_t> g_pool;

hipEvent_t take() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    // Timing only: no system-scope fence when the event completes (the host
    // synchronises the stream before it reads the times), which would
    // otherwise hold back the next kernel on the stream.
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

ProfileScope::ProfileScope(int phase, hipStream_t s, bool attached)
    : phase_(phase), s_(s), attached_(attached) {
    if (!(g_mask & (1u << phase))) return;
    a_ = take();
    b_ = take();
    if (!a_ || !b_) {
        if (a_) g_pool.push_back(a_);
        if (b_) g_pool.push_back(b_);
        a_ = b_ = nullptr;
        return;
    }
    if (!attached_) hipEventRecord(a_, s_);
}

ProfileScope::~ProfileScope() {
    if (!a_ || !b_) return;
    if (!attached_) hipEventRecord(b_, s_);
    g_marks.push_back(Mark{phase_, a_, b_});
}

}  // namespace moe

using namespace moe;

extern "C" {

void moe_profile_begin(uint32_t mask) {
    g_mask = mask;
    for (auto &m : g_marks) {
        g_pool.push_back(m.a);
        g_pool.push_back(m.b);
    }
    g_marks.clear();
}

void moe_profile_set_mask(uint32_t mask) { g_mask = mask; }

int moe_profile_end(double *ms, int64_t *launches) {
    g_mask = 0;
    if (ms)
        for (int p = 0; p < MOE_PHASES; ++p) ms[p] = 0.0;
    if (launches)
        for (int p = 0; p < MOE_PHASES; ++p) launches[p] = 0;
    int n = 0;
    bool ok = true;
    for (auto &m : g_marks) {
        if (hipEventSynchronize(m.b) != hipSuccess) ok = false;
        float t = 0.0f;
        if (ok && hipEventElapsedTime(&t, m.a, m.b) != hipSuccess) ok = false;
        if (ms) ms[m.phase] += t;
        if (launches) launches[m.phase] += 1;
        ++n;
        g_pool.push_back(m.a);
        g_pool.push_back(m.b);
    }
    g_marks.clear();
    return ok ? n : -1;
}

}  // extern "C"
