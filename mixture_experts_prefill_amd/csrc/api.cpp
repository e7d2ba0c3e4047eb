// C ABI of libmoe: argument checks, workspace plan and launch sequencing.
//
// Every entry point validates all arguments before it enqueues anything, in
// the manner of the cherenkov prefill.rs page (fn prefill_chunk: "empty
// chunk" and capacity checks up front, errors returned with a message).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.h"
#include "ring.h"

namespace moe {

static thread_local std::string g_err;

moe_status fail(moe_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

moe_status hip_fail(hipError_t e, const char *what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int shared_ksplit(int t, int ksteps, int nblk) {
    if (t > 64) return 1;
    const int mt = (t + 31) / 32;
    for (int d = 1; d <= ksteps; ++d)
        if (ksteps % d == 0 && mt * nblk * d >= 128) return d;
    return ksteps;
}

// How the shared expert runs for t rows: tile height, K splits of its two
// GEMMs (workgroup counts follow the GEMM's launch rule) and the bytes of
// split partial sums it needs.
struct SharedPlan {
    int bm, s_gu, s_dn;
    size_t part_bytes;
};
static SharedPlan shared_plan(int t, const moe_layout *Ls) {
    SharedPlan sp;
    sp.bm = t >= 512 ? 128 : t >= 64 ? 64 : 32;
    const int mt = (t + sp.bm - 1) / sp.bm;
    // feature blocks of the 4-wave GEMM workgroups: 128 (gate/up), 256 (down)
    const int nblk_gu = (Ls->inter + 127) / 128;
    const int nblk_dn = (Ls->hidden + 255) / 256;
    (void)mt;
    sp.s_gu = shared_ksplit(t, Ls->hidden / 64, nblk_gu);
    sp.s_dn = shared_ksplit(t, Ls->inter / 64, nblk_dn);
    size_t pb = 0;
    if (sp.s_gu > 1) pb = (size_t)sp.s_gu * t * 2 * Ls->inter * 4;
    if (sp.s_dn > 1) pb = std::max(pb, (size_t)sp.s_dn * t * Ls->hidden * 4);
    sp.part_bytes = pb;
    return sp;
}

static bool layout_ok(const moe_layout *L) {
    if (!L) return false;
    moe_layout ref;
    if (moe_layout_make(L->hidden, L->inter, L->group, &ref) != MOE_OK) return false;
    return std::memcmp(&ref, L, sizeof ref) == 0;
}

// The shared expert can share the routed experts' grouped launches when its
// record has the routed layout (same hidden, inter and group).
static bool fusable(const moe_layout *routed, const moe_layout *shared) {
    return shared && routed && shared->hidden == routed->hidden && shared->inter == routed->inter &&
           shared->group == routed->group;
}

bool workspace_plan(int t, int k, int E, const moe_layout *routed, const moe_layout *shared,
                    Workspace *w) {
    if (t < 1 || t > MOE_MAX_ROWS || k < 1 || k > MOE_MAX_K || E < k || E > MOE_MAX_EXPERTS)
        return false;
    if (!layout_ok(routed) || (shared && !layout_ok(shared))) return false;
    if (shared && shared->hidden != routed->hidden) return false;
    const size_t P = (size_t)t * k;
    const size_t tiles = (size_t)(t + kCsrTileRows - 1) / kCsrTileRows;
    // A shared expert of the routed shape can run inside the routed launches
    // (moe_prefill_fused): its t rows follow the t*k CSR positions in hg / ye
    // and its tiles join the schedule.
    const size_t Q = P + (fusable(routed, shared) ? (size_t)t : 0);
    const size_t max_mt = Q / kMinBM + (size_t)E + 2;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    w->csr_hist = take(tiles * E * 4);
    w->sched_n = take(64);
    w->order = take(8 * max_mt * sizeof(TileEntry));
    w->jobs = take((size_t)E * 8);
    w->hg = take(Q * routed->inter * 2);
    w->ye = take(Q * routed->hidden * 2);
    w->part = take(shared ? shared_plan(t, shared).part_bytes : 0);
    w->hs = take(shared ? (size_t)t * shared->inter * 2 : 0);
    w->gate = take((size_t)t * 4);
    w->total = off;
    return true;
}

// Largest M-tile height.  Tiles only run their non-empty 32-row blocks, so a
// taller tile costs no padding; it halves the dequantisation per MFMA each
// time it doubles, but there must stay enough workgroups (about 1.5 per CU)
// for the cost-ordered schedule to balance.  With about one token block per
// expert (small chunks) 32-row tiles with 4 waves cover fewer features each
// and so spread the weight stream over more workgroups.
int pick_bm(int t, int k, int E, int inter, int hidden) {
    const long P = (long)t * k;
    const long used = P < E ? P : E;  // at most this many non-empty experts
    const long mean = P / (used > 0 ? used : 1);
    if (mean < 48) return 32;
    (void)hidden;
    const long nblk = (inter + 127) / 128;  // gate/up workgroups cover 128 features
    for (int bm = kMaxBM; bm >= 64; bm /= 2)
        if ((P / bm + used) * nblk >= 384) return bm;
    return 64;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static moe_status check_rows(int t) {
    if (t < 1) return fail(MOE_ERR_CAPACITY, "empty chunk (t = %d)", t);
    if (t > MOE_MAX_ROWS) return fail(MOE_ERR_CAPACITY, "t = %d exceeds the %d-row chunk cap", t, MOE_MAX_ROWS);
    return MOE_OK;
}

static moe_status check_routing(int t, int k, int E) {
    if (moe_status st = check_rows(t)) return st;
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID, "E = %d outside 1..%d", E, MOE_MAX_EXPERTS);
    if (k < 1 || k > E || k > MOE_MAX_K) return fail(MOE_ERR_INVALID, "k = %d outside 1..min(E = %d, %d)", k, E, MOE_MAX_K);
    return MOE_OK;
}

// Checks shared by moe_prefill_fused and moe_block: the routed layout, the
// shared layout (optional for moe_block, required for the fused call) equal
// to it, the inputs, the 32-bit offsets and the workspace.
static moe_status check_fused(const uint16_t *x, int t, int k, int E, const moe_layout *L,
                              const uint64_t *records, const moe_layout *Ls, const void *shared_record,
                              const float *out, const void *workspace, size_t workspace_bytes,
                              bool shared_optional, const char *who) {
    if (!layout_ok(L) || (Ls && !layout_ok(Ls)) || (!Ls && !shared_optional))
        return fail(MOE_ERR_INVALID, "%s: layout not made by moe_layout_make", who);
    if (Ls && !fusable(L, Ls))
        return fail(MOE_ERR_INVALID, "%s: the shared layout (h %d, inter %d, group %d) must equal the routed one "
                    "(h %d, inter %d, group %d)", who, Ls->hidden, Ls->inter, Ls->group, L->hidden, L->inter, L->group);
    if (!x || !records || (Ls && !shared_record) || !out || !workspace)
        return fail(MOE_ERR_INVALID, "%s: null pointer", who);
    if (!aligned16(x) || !aligned16(out) || (Ls && !aligned16(shared_record)))
        return fail(MOE_ERR_INVALID, "%s: x, out and the shared record must be 16-byte aligned", who);
    const uint64_t Q = (uint64_t)t * (k + (Ls ? 1 : 0));
    if (Q * L->inter * 2 > 0xffffffffull || (uint64_t)t * L->hidden * 2 > 0xffffffffull)
        return fail(MOE_ERR_CAPACITY, "%s: t*(k+1)*inter or t*hidden too large for 32-bit offsets", who);
    Workspace w;
    workspace_plan(t, k, E, L, Ls, &w);
    if (workspace_bytes < w.total)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", who, workspace_bytes, w.total);
    return MOE_OK;
}

// GEMM arguments of the grouped launches, with the shared expert's t rows
// after the t*k CSR positions when `shared`.
static GemmArgs fused_args(const uint16_t *x, int t, int k, int E, const moe_layout *L, const uint32_t *csr_rows,
                           const uint64_t *records, uint8_t *ws, const Workspace &w, bool shared) {
    const size_t Q = (size_t)t * (k + (shared ? 1 : 0));
    GemmArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = x;
    a.rows = csr_rows;
    a.records = records;
    a.sched_n = reinterpret_cast<uint32_t *>(ws + w.sched_n);
    a.order = reinterpret_cast<TileEntry *>(ws + w.order);
    a.xcap = (int)(Q / kMinBM + (size_t)E + 2);
    a.t = t;
    a.hidden = L->hidden;
    a.inter = L->inter;
    a.group = L->group;
    a.hg = reinterpret_cast<uint16_t *>(ws + w.hg);
    a.ye = reinterpret_cast<uint16_t *>(ws + w.ye);
    a.shared_rows = shared ? 1 : 0;
    a.shared_p0 = t * k;
    return a;
}

static moe_status shared_gate(const uint16_t *x, int t, const moe_layout *L, const uint16_t *gate_w, uint8_t *g,
                              hipStream_t s) {
    if (!gate_w) return MOE_OK;
    hipError_t e = launch_shared_gate(x, gate_w, t, L->hidden, reinterpret_cast<float *>(g), s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "shared gate");
}

// Arguments of the next-norm kernel from the caller's description.
static NextNormArgs next_norm_args(const moe_next_norm *nn, int t, int h) {
    NextNormArgs n;
    std::memset(&n, 0, sizeof n);
    n.t = t;
    n.h = h;
    n.n = nn->n;
    n.hyper = nn->hyper;
    for (int i = 0; i < nn->n; ++i) {
        n.alpha[i] = nn->alpha[i];
        n.beta[i] = nn->beta[i];
    }
    n.gamma = nn->gamma;
    n.eps = nn->eps;
    n.mixed = nn->mixed;
    return n;
}

static bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

static moe_status check_next_norm(const moe_next_norm *nn, int t, int h, const float *y, const char *who) {
    if (!nn) return fail(MOE_ERR_INVALID, "%s: null next-norm description", who);
    if (nn->n < 1 || nn->n > MOE_MAX_HC)
        return fail(MOE_ERR_INVALID, "%s: n = %d residual copies outside 1..%d", who, nn->n, MOE_MAX_HC);
    if (!nn->hyper || !nn->gamma || !nn->mixed) return fail(MOE_ERR_INVALID, "%s: null pointer", who);
    if (!aligned16(nn->hyper) || !aligned16(nn->gamma) || !aligned16(nn->mixed) || (y && !aligned16(y)))
        return fail(MOE_ERR_INVALID, "%s: hyper, gamma, mixed and y must be 16-byte aligned", who);
    if (!(nn->eps >= 0.0f) || nn->eps == __builtin_inff())
        return fail(MOE_ERR_INVALID, "%s: eps must be finite and >= 0", who);
    if (h % 256 || h > kNormMaxHidden)
        return fail(MOE_ERR_INVALID, "%s: h = %d must be a multiple of 256 and at most %d", who, h, kNormMaxHidden);
    const size_t hyper_bytes = (size_t)t * nn->n * h * 4, mixed_bytes = (size_t)t * h * 2;
    if (overlaps(nn->hyper, hyper_bytes, nn->mixed, mixed_bytes) ||
        (y && (overlaps(y, (size_t)t * h * 4, nn->hyper, hyper_bytes) ||
               overlaps(y, (size_t)t * h * 4, nn->mixed, mixed_bytes))))
        return fail(MOE_ERR_INVALID, "%s: hyper, mixed and y must not overlap", who);
    return MOE_OK;
}

// Gate/up, down and combine of a scheduled call (the schedule already
// enqueued); with `nn` the combine's pass goes into the next fused norm
// instead of writing out.
static moe_status fused_gemms(GemmArgs a, int bm, const moe_layout *L, int t, int k, int E,
                              const uint32_t *csr_pos, const float *csr_w, float *out, int accumulate,
                              const float *g, bool shared, hipStream_t s, const moe_next_norm *nn = nullptr) {
    const size_t Q = (size_t)t * (k + (shared ? 1 : 0));
    // With t <= bm every non-empty expert, and the shared segment, is a single
    // tile: the tighter bound shrinks the grid to the workgroups that can
    // have work (decode-shaped chunk: 6336 -> 1152 gate/up workgroups
    // launched; block 0.1588 -> 0.1575 and 0.1562 -> 0.1559 ms on two boxes,
    // t = 1: 0.0549 -> 0.0541 ms).
    a.max_tiles = t <= bm ? std::min(E, t * k) + (shared ? 1 : 0) : (int)(Q / bm + (size_t)E + 2);
    GemmArgs gu = a;
    gu.w_off = L->gate_w;
    gu.sb_off = L->gate_sb;
    gu.w2_off = L->up_w;
    gu.sb2_off = L->up_sb;
    a.act = a.hg;
    a.w_off = L->down_w;
    a.sb_off = L->down_sb;
    hipError_t e;
    if (gateup_down_merged(gu, bm)) {
        e = launch_gateup_down(gu, a, bm, s);
        if (e != hipSuccess) return hip_fail(e, "experts gate/up and down");
    } else {
        e = launch_gateup(gu, bm, s);
        if (e != hipSuccess) return hip_fail(e, "experts gate/up");
        e = launch_down(a, bm, s);
        if (e != hipSuccess) return hip_fail(e, "experts down");
    }
    const uint16_t *ys = shared ? a.ye + (size_t)t * k * L->hidden : nullptr;
    if (nn) {
        NextNormArgs n = next_norm_args(nn, t, L->hidden);
        n.ye = a.ye;
        n.pos = csr_pos;
        n.csr_w = csr_w;
        n.k = k;
        n.ys = ys;
        n.gate = g;
        e = launch_next_norm(n, s);
        if (e != hipSuccess) return hip_fail(e, "combine into the next norm");
        return MOE_OK;
    }
    e = launch_combine(a.ye, csr_pos, csr_w, t, k, L->hidden, out, accumulate, s, ys, g);
    if (e != hipSuccess) return hip_fail(e, "combine");
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_last_error(void) { return g_err.c_str(); }

moe_status moe_layout_make(int32_t hidden, int32_t inter, int32_t group, moe_layout *out) {
    return moe_layout_make_bits(hidden, inter, group, 4, out);
}

moe_status moe_layout_make_bits(int32_t hidden, int32_t inter, int32_t group, int32_t bits, moe_layout *out) {
    if (!out) return fail(MOE_ERR_INVALID, "layout: null output");
    if (hidden <= 0 || hidden % 256) return fail(MOE_ERR_INVALID, "hidden = %d must be a positive multiple of 256", hidden);
    if (inter <= 0 || inter % 64) return fail(MOE_ERR_INVALID, "inter = %d must be a positive multiple of 64", inter);
    if (group != 32 && group != 64) return fail(MOE_ERR_INVALID, "group = %d must be 32 or 64", group);
    if (bits != 4 && bits != 2) return fail(MOE_ERR_INVALID, "bits = %d must be 4 or 2", bits);
    moe_layout L;
    std::memset(&L, 0, sizeof L);
    L.hidden = hidden;
    L.inter = inter;
    L.group = group;
    L.bits = bits;
    const uint64_t codes = (uint64_t)hidden * inter * bits / 8;
    const uint64_t sb = (uint64_t)hidden * inter / group * 4;
    uint64_t off = 0;
    uint64_t *secs[6] = {&L.gate_w, &L.gate_sb, &L.up_w, &L.up_sb, &L.down_w, &L.down_sb};
    for (int m = 0; m < 3; ++m) {
        *secs[2 * m] = off;
        off = (off + codes + 255) / 256 * 256;
        *secs[2 * m + 1] = off;
        off = (off + sb + 255) / 256 * 256;
    }
    L.stride = (off + 4095) / 4096 * 4096;
    // The GEMMs address a record with 32-bit byte offsets.
    if (L.stride > 0xffffffffull)
        return fail(MOE_ERR_INVALID, "layout: record of %llu bytes exceeds 4 GiB", (unsigned long long)L.stride);
    *out = L;
    return MOE_OK;
}

size_t moe_workspace_bytes(int32_t t, int32_t k, int32_t E, const moe_layout *routed,
                           const moe_layout *shared) {
    Workspace w;
    return workspace_plan(t, k, E, routed, shared, &w) ? w.total : 0;
}

moe_status moe_route(const uint16_t *x, const float *w_router, int32_t t, int32_t h, int32_t E,
                     int32_t k, float *logits, uint32_t *topk_idx, float *topk_w, void *stream) {
    if (moe_status st = check_routing(t, k, E)) return st;
    if (h <= 0 || h % 256) return fail(MOE_ERR_INVALID, "route: h = %d must be a positive multiple of 256", h);
    if (!x || !w_router || !logits || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID, "route: null pointer");
    if (!aligned16(x) || !aligned16(w_router)) return fail(MOE_ERR_INVALID, "route: x and w_router must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_router_logits(x, w_router, t, h, E, logits, s);
    if (e != hipSuccess) return hip_fail(e, "router logits");
    e = launch_topk(logits, t, E, k, topk_idx, topk_w, s);
    if (e != hipSuccess) return hip_fail(e, "top-k");
    return MOE_OK;
}

moe_status moe_build_csr(const uint32_t *topk_idx, const float *topk_w, int32_t t, int32_t k,
                         int32_t E, uint32_t *offsets, uint32_t *csr_rows, float *csr_w,
                         uint32_t *csr_pos, void *workspace, size_t workspace_bytes, void *stream) {
    if (moe_status st = check_routing(t, k, E)) return st;
    if (!topk_idx || !topk_w || !offsets || !csr_rows || !csr_w || !csr_pos || !workspace)
        return fail(MOE_ERR_INVALID, "build_csr: null pointer");
    const size_t need = (size_t)((t + kCsrTileRows - 1) / kCsrTileRows) * E * 4;
    if (workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "build_csr: workspace %zu bytes < %zu needed", workspace_bytes, need);
    // the CSR scratch sits at the start of the workspace in every plan
    uint32_t *hist = static_cast<uint32_t *>(workspace);
    hipError_t e = launch_csr(topk_idx, topk_w, t, k, E, offsets, csr_rows, csr_w, csr_pos, hist,
                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "build_csr");
    return MOE_OK;
}

moe_status moe_shared(const uint16_t *x, int32_t t, const moe_layout *Ls, const void *record,
                      const uint16_t *gate_w, float *out, int32_t accumulate, void *workspace,
                      size_t workspace_bytes, void *stream) {
    if (moe_status st = check_rows(t)) return st;
    if (!layout_ok(Ls)) return fail(MOE_ERR_INVALID, "shared: layout not made by moe_layout_make");
    if (!x || !record || !out || !workspace) return fail(MOE_ERR_INVALID, "shared: null pointer");
    if (!aligned16(x) || !aligned16(record) || !aligned16(out))
        return fail(MOE_ERR_INVALID, "shared: x, record and out must be 16-byte aligned");
    if ((uint64_t)t * Ls->inter * 2 > 0xffffffffull || (uint64_t)t * Ls->hidden * 2 > 0xffffffffull)
        return fail(MOE_ERR_CAPACITY, "shared: t*inter or t*hidden too large for 32-bit offsets");
    // The shared expert's scratch is the end of the workspace: [.. | part | hs | gate].
    const SharedPlan sp = shared_plan(t, Ls);
    const size_t g_bytes = align256((size_t)t * 4), hs_bytes = align256((size_t)t * Ls->inter * 2);
    const size_t p_bytes = align256(sp.part_bytes);
    const size_t end = workspace_bytes & ~size_t(255);
    if (end < g_bytes + hs_bytes + p_bytes)
        return fail(MOE_ERR_WORKSPACE, "shared: workspace %zu bytes < %zu needed", workspace_bytes,
                    g_bytes + hs_bytes + p_bytes);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint16_t *hs = reinterpret_cast<uint16_t *>(ws + end - g_bytes - hs_bytes);
    float *g = reinterpret_cast<float *>(ws + end - g_bytes);
    float *part = reinterpret_cast<float *>(ws + end - g_bytes - hs_bytes - p_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (gate_w) {
        e = launch_shared_gate(x, gate_w, t, Ls->hidden, g, s);
        if (e != hipSuccess) return hip_fail(e, "shared gate");
    }
    GemmArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = x;
    a.record = record;
    a.t = t;
    a.hidden = Ls->hidden;
    a.inter = Ls->inter;
    a.group = Ls->group;
    a.w_off = Ls->gate_w;
    a.sb_off = Ls->gate_sb;
    a.w2_off = Ls->up_w;
    a.sb2_off = Ls->up_sb;
    a.hg = hs;
    a.part = part;
    const int bm = sp.bm;
    // Small chunks split K over workgroups (partial sums reduced in a fixed
    // order by k_reduce_*); larger ones run the GEMM with its epilogue.
    a.ksplit = sp.s_gu;
    e = launch_gateup(a, bm, s);
    if (e == hipSuccess && sp.s_gu > 1) e = launch_reduce_gu(part, sp.s_gu, t, Ls->inter, hs, s);
    if (e != hipSuccess) return hip_fail(e, "shared gate/up");
    a.act = hs;
    a.w_off = Ls->down_w;
    a.sb_off = Ls->down_sb;
    a.out = out;
    a.gate = gate_w ? g : nullptr;
    a.accumulate = accumulate;
    a.ksplit = sp.s_dn;
    e = launch_down(a, bm, s);
    if (e == hipSuccess && sp.s_dn > 1)
        e = launch_reduce_down(part, sp.s_dn, t, Ls->hidden, gate_w ? g : nullptr, out, accumulate, s);
    if (e != hipSuccess) return hip_fail(e, "shared down");
    return MOE_OK;
}

moe_status moe_prefill_experts(const uint16_t *x, int32_t t, int32_t k, int32_t E,
                               const moe_layout *L, const uint32_t *offsets,
                               const uint32_t *csr_rows, const float *csr_w,
                               const uint32_t *csr_pos, const uint64_t *records,
                               const void *const *host_records, moe_ring *ring, float *out,
                               int32_t accumulate, void *workspace, size_t workspace_bytes,
                               void *stream) {
    if (moe_status st = check_routing(t, k, E)) return st;
    if (!layout_ok(L)) return fail(MOE_ERR_INVALID, "experts: layout not made by moe_layout_make");
    if (!x || !offsets || !csr_rows || !csr_w || !csr_pos || !records || !out || !workspace)
        return fail(MOE_ERR_INVALID, "experts: null pointer");
    if (!aligned16(x) || !aligned16(out)) return fail(MOE_ERR_INVALID, "experts: x and out must be 16-byte aligned");
    // The GEMMs address x and the intermediate rows with 32-bit byte offsets.
    if ((uint64_t)t * k * L->inter * 2 > 0xffffffffull || (uint64_t)t * L->hidden * 2 > 0xffffffffull)
        return fail(MOE_ERR_CAPACITY, "experts: t*k*inter or t*hidden too large for 32-bit offsets");
    Workspace w;
    workspace_plan(t, k, E, L, nullptr, &w);
    const size_t need = w.gate;  // everything before the shared scratch
    if (workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "experts: workspace %zu bytes < %zu needed", workspace_bytes, need);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);

    GemmArgs a;
    std::memset(&a, 0, sizeof a);
    a.x = x;
    a.rows = csr_rows;
    a.records = records;
    a.sched_n = reinterpret_cast<uint32_t *>(ws + w.sched_n);
    a.order = reinterpret_cast<TileEntry *>(ws + w.order);
    a.xcap = (int)((size_t)t * k / kMinBM + (size_t)E + 1);
    a.t = t;
    a.hidden = L->hidden;
    a.inter = L->inter;
    a.group = L->group;
    a.hg = reinterpret_cast<uint16_t *>(ws + w.hg);
    a.ye = reinterpret_cast<uint16_t *>(ws + w.ye);
    const int bm = pick_bm(t, k, E, L->inter, L->hidden);
    a.max_tiles = t <= bm ? std::min(E, t * k) : (int)((size_t)t * k / bm + (size_t)E + 1);

    if (ring || host_records) {
        return ring_run(ring, host_records, a, bm, offsets, csr_pos, csr_w, t, k, E, L, out,
                        accumulate, reinterpret_cast<uint64_t *>(ws + w.jobs), s);
    }

    hipError_t e = launch_schedule(offsets, 0, E, bm, t, records, const_cast<uint32_t *>(a.sched_n),
                                   const_cast<TileEntry *>(a.order), a.xcap, s);
    if (e != hipSuccess) return hip_fail(e, "schedule");
    GemmArgs gu = a;
    gu.w_off = L->gate_w;
    gu.sb_off = L->gate_sb;
    gu.w2_off = L->up_w;
    gu.sb2_off = L->up_sb;
    a.act = a.hg;
    a.w_off = L->down_w;
    a.sb_off = L->down_sb;
    if (gateup_down_merged(gu, bm)) {
        e = launch_gateup_down(gu, a, bm, s);
        if (e != hipSuccess) return hip_fail(e, "experts gate/up and down");
    } else {
        e = launch_gateup(gu, bm, s);
        if (e != hipSuccess) return hip_fail(e, "experts gate/up");
        e = launch_down(a, bm, s);
        if (e != hipSuccess) return hip_fail(e, "experts down");
    }
    e = launch_combine(a.ye, csr_pos, csr_w, t, k, L->hidden, out, accumulate, s);
    if (e != hipSuccess) return hip_fail(e, "combine");
    return MOE_OK;
}

moe_status moe_prefill_fused(const uint16_t *x, int32_t t, int32_t k, int32_t E, const moe_layout *L,
                             const uint32_t *offsets, const uint32_t *csr_rows, const float *csr_w,
                             const uint32_t *csr_pos, const uint64_t *records, const moe_layout *Ls,
                             const void *shared_record, const uint16_t *shared_gate_w, float *out,
                             int32_t accumulate, void *workspace, size_t workspace_bytes, void *stream) {
    if (moe_status st = check_routing(t, k, E)) return st;
    if (!offsets || !csr_rows || !csr_w || !csr_pos) return fail(MOE_ERR_INVALID, "fused: null pointer");
    if (moe_status st = check_fused(x, t, k, E, L, records, Ls, shared_record, out, workspace, workspace_bytes,
                                    false, "fused"))
        return st;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    Workspace w;
    workspace_plan(t, k, E, L, Ls, &w);
    GemmArgs a = fused_args(x, t, k, E, L, csr_rows, records, ws, w, true);
    const int bm = pick_bm(t, k, E, L->inter, L->hidden);
    if (moe_status st = shared_gate(x, t, L, shared_gate_w, ws + w.gate, s)) return st;
    hipError_t e = launch_schedule(offsets, 0, E, bm, t, records, const_cast<uint32_t *>(a.sched_n),
                                   const_cast<TileEntry *>(a.order), a.xcap, s,
                                   SharedSeg{shared_record, a.shared_p0, t});
    if (e != hipSuccess) return hip_fail(e, "schedule");
    return fused_gemms(a, bm, L, t, k, E, csr_pos, csr_w, out, accumulate,
                       shared_gate_w ? reinterpret_cast<float *>(ws + w.gate) : nullptr, true, s);
}

}  // extern "C"

namespace moe {

// Argument checks of moe_block and moe_block_noalloc (everything but the
// workspace size, which `ws_check` bytes stand in for).
static moe_status block_check(const uint16_t *x, const float *w_router, int t, int k, int E, const moe_layout *L,
                              const uint64_t *records, const moe_layout *Ls, const void *shared_record,
                              const float *logits, const uint32_t *topk_idx, const float *topk_w,
                              const uint32_t *offsets, const uint32_t *csr_rows, const float *csr_w,
                              const uint32_t *csr_pos, const float *out, const void *workspace, size_t ws_check,
                              const char *who) {
    if (moe_status st = check_routing(t, k, E)) return st;
    if (!w_router || !logits || !topk_idx || !topk_w || !offsets || !csr_rows || !csr_w || !csr_pos)
        return fail(MOE_ERR_INVALID, "%s: null pointer", who);
    if (!aligned16(w_router)) return fail(MOE_ERR_INVALID, "%s: w_router must be 16-byte aligned", who);
    return check_fused(x, t, k, E, L, records, Ls, shared_record, out, workspace, ws_check, true, who);
}

// The block's launches on validated arguments.
static moe_status block_run(const uint16_t *x, const float *w_router, int t, int k, int E, const moe_layout *L,
                            const uint64_t *records, const moe_layout *Ls, const void *shared_record,
                            const uint16_t *shared_gate_w, float *logits, uint32_t *topk_idx, float *topk_w,
                            uint32_t *offsets, uint32_t *csr_rows, float *csr_w, uint32_t *csr_pos, float *out,
                            int accumulate, uint8_t *ws, hipStream_t s, const moe_next_norm *nn = nullptr) {
    const bool shared = Ls != nullptr;
    Workspace w;
    workspace_plan(t, k, E, L, Ls, &w);
    const int h = L->hidden;
    hipError_t e = launch_router_logits(x, w_router, t, h, E, logits, s);
    if (e != hipSuccess) return hip_fail(e, "router logits");
    const bool merged_topk = topk_csr_schedule_fits(t);
    if (!merged_topk) {
        e = launch_topk(logits, t, E, k, topk_idx, topk_w, s);
        if (e != hipSuccess) return hip_fail(e, "top-k");
    }
    if (shared)
        if (moe_status st = shared_gate(x, t, L, shared_gate_w, ws + w.gate, s)) return st;
    GemmArgs a = fused_args(x, t, k, E, L, csr_rows, records, ws, w, shared);
    const int bm = pick_bm(t, k, E, L->inter, L->hidden);
    const SharedSeg sh{shared ? shared_record : nullptr, a.shared_p0, shared ? t : 0};
    if (merged_topk) {
        e = launch_topk_csr_schedule(logits, t, E, k, topk_idx, topk_w, offsets, csr_rows, csr_w, csr_pos, bm,
                                     records, const_cast<uint32_t *>(a.sched_n), const_cast<TileEntry *>(a.order),
                                     a.xcap, sh, s);
        if (e != hipSuccess) return hip_fail(e, "top-k, grouping and schedule");
    } else if (csr_schedule_fits(t)) {
        e = launch_csr_schedule(topk_idx, topk_w, t, k, E, offsets, csr_rows, csr_w, csr_pos, bm, records,
                                const_cast<uint32_t *>(a.sched_n), const_cast<TileEntry *>(a.order), a.xcap, sh, s);
        if (e != hipSuccess) return hip_fail(e, "grouping and schedule");
    } else {
        e = launch_csr_with_schedule(topk_idx, topk_w, t, k, E, offsets, csr_rows, csr_w, csr_pos,
                                     reinterpret_cast<uint32_t *>(ws + w.csr_hist), bm, records,
                                     const_cast<uint32_t *>(a.sched_n), const_cast<TileEntry *>(a.order), a.xcap,
                                     sh, s);
        if (e != hipSuccess) return hip_fail(e, "grouping and schedule");
    }
    return fused_gemms(a, bm, L, t, k, E, csr_pos, csr_w, out, accumulate,
                       (shared && shared_gate_w) ? reinterpret_cast<float *>(ws + w.gate) : nullptr, shared, s, nn);
}

// Scratch of moe_block_noalloc: one array per GPU, held by the loaded code
// object until the process ends.  Host code must not use `scratch` itself
// (on the host it is only a stand-in symbol); it uses the device address
// that hipGetSymbolAddress returns for the current device, kept per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device.
static moe_status scratch_ptr(uint8_t **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "block_noalloc: current device");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_INVALID, "block_noalloc: device %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "block_noalloc: scratch address");
        if (!p) return fail(MOE_ERR_HIP, "block_noalloc: scratch address is null");
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<uint8_t *>(g_scratch_ptr[dev]);
    return MOE_OK;
}

}  // namespace moe

extern "C" {

moe_status moe_block(const uint16_t *x, const float *w_router, int32_t t, int32_t k, int32_t E,
                     const moe_layout *L, const uint64_t *records, const moe_layout *Ls,
                     const void *shared_record, const uint16_t *shared_gate_w, float *logits,
                     uint32_t *topk_idx, float *topk_w, uint32_t *offsets, uint32_t *csr_rows,
                     float *csr_w, uint32_t *csr_pos, float *out, int32_t accumulate, void *workspace,
                     size_t workspace_bytes, void *stream) {
    if (moe_status st = block_check(x, w_router, t, k, E, L, records, Ls, shared_record, logits, topk_idx, topk_w,
                                    offsets, csr_rows, csr_w, csr_pos, out, workspace, workspace_bytes, "block"))
        return st;
    return block_run(x, w_router, t, k, E, L, records, Ls, shared_record, shared_gate_w, logits, topk_idx, topk_w,
                     offsets, csr_rows, csr_w, csr_pos, out, accumulate, static_cast<uint8_t *>(workspace),
                     static_cast<hipStream_t>(stream));
}

moe_status moe_block_noalloc(const uint16_t *x, const float *w_router, int32_t t, int32_t k, int32_t E,
                             const moe_layout *L, const uint64_t *records, const moe_layout *Ls,
                             const void *shared_record, const uint16_t *shared_gate_w, float *logits,
                             uint32_t *topk_idx, float *topk_w, uint32_t *offsets, uint32_t *csr_rows,
                             float *csr_w, uint32_t *csr_pos, float *out, int32_t accumulate, void *stream) {
    // Every check that needs no device first, the scratch size among them:
    // a non-null stand-in takes the workspace pointer's place.
    static const uint8_t stand_in[16] = {0};
    if (moe_status st = block_check(x, w_router, t, k, E, L, records, Ls, shared_record, logits, topk_idx, topk_w,
                                    offsets, csr_rows, csr_w, csr_pos, out, stand_in, (size_t)-1, "block_noalloc"))
        return st;
    Workspace w;
    workspace_plan(t, k, E, L, Ls, &w);
    if (w.total > MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_CAPACITY, "block_noalloc: this chunk needs %zu bytes of scratch, more than the %llu "
                    "bytes of the library's static scratch (use moe_block with a workspace)", w.total,
                    (unsigned long long)MOE_NOALLOC_SCRATCH_BYTES);
    uint8_t *ws = nullptr;
    if (moe_status st = scratch_ptr(&ws)) return st;
    return block_run(x, w_router, t, k, E, L, records, Ls, shared_record, shared_gate_w, logits, topk_idx, topk_w,
                     offsets, csr_rows, csr_w, csr_pos, out, accumulate, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_inject_norm(const float *y, int32_t t, int32_t h, const moe_next_norm *nn, void *stream) {
    if (moe_status st = check_rows(t)) return st;
    if (moe_status st = check_next_norm(nn, t, h, y, "inject_norm")) return st;
    NextNormArgs n = next_norm_args(nn, t, h);
    n.y = y;
    hipError_t e = launch_next_norm(n, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "inject_norm");
    return MOE_OK;
}

moe_status moe_block_next_norm(const uint16_t *x, const float *w_router, int32_t t, int32_t k, int32_t E,
                               const moe_layout *L, const uint64_t *records, const moe_layout *Ls,
                               const void *shared_record, const uint16_t *shared_gate_w, float *logits,
                               uint32_t *topk_idx, float *topk_w, uint32_t *offsets, uint32_t *csr_rows,
                               float *csr_w, uint32_t *csr_pos, const moe_next_norm *nn, void *workspace,
                               size_t workspace_bytes, void *stream) {
    if (!nn) return fail(MOE_ERR_INVALID, "block_next_norm: null next-norm description");
    // the copies stand in for out in the shared checks (non-null, aligned)
    if (moe_status st = block_check(x, w_router, t, k, E, L, records, Ls, shared_record, logits, topk_idx, topk_w,
                                    offsets, csr_rows, csr_w, csr_pos, nn->hyper, workspace, workspace_bytes,
                                    "block_next_norm"))
        return st;
    if (moe_status st = check_next_norm(nn, t, L->hidden, nullptr, "block_next_norm")) return st;
    return block_run(x, w_router, t, k, E, L, records, Ls, shared_record, shared_gate_w, logits, topk_idx, topk_w,
                     offsets, csr_rows, csr_w, csr_pos, nullptr, 0, static_cast<uint8_t *>(workspace),
                     static_cast<hipStream_t>(stream), nn);
}

moe_status moe_residency(const uint32_t *offsets, int32_t E, int32_t budget, uint32_t *order, uint8_t *keep,
                         void *stream) {
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID, "residency: E = %d outside 1..%d", E, MOE_MAX_EXPERTS);
    if (budget < 0) return fail(MOE_ERR_INVALID, "residency: budget = %d < 0", budget);
    if (!offsets || !order || !keep) return fail(MOE_ERR_INVALID, "residency: null pointer");
    hipError_t e = launch_rank_experts(offsets, nullptr, 0, E, budget, nullptr, order, keep,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "residency");
    return MOE_OK;
}

int moe_debug_schedule(const uint32_t *offsets, int32_t E, int32_t bm, int32_t rows_bound, const uint64_t *records,
                       const void *shared_rec, int32_t shared_p0, int32_t shared_n, uint32_t *sched_n,
                       void *order, int32_t xcap, void *stream) {
    if (!offsets || !records || !sched_n || !order || E < 1 || E > MOE_MAX_EXPERTS ||
        (bm != 32 && bm != 64 && bm != 128) || rows_bound < 0 || xcap < 1 || shared_p0 < 0 || shared_n < 0 ||
        (shared_rec && shared_n < 1))
        return 1;
    hipError_t e = launch_schedule(offsets, 0, E, bm, rows_bound, records, sched_n, static_cast<TileEntry *>(order), xcap,
                                   static_cast<hipStream_t>(stream), SharedSeg{shared_rec, shared_p0, shared_n});
    return e == hipSuccess ? 0 : 5;
}

moe_status moe_chunk_stats_fill(const uint32_t *offsets, int32_t t, int32_t E, moe_chunk_stats *stats,
                                void *stream) {
    if (E < 1 || E > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_INVALID, "chunk stats: E = %d outside 1..%d", E, MOE_MAX_EXPERTS);
    if (t < 0) return fail(MOE_ERR_INVALID, "chunk stats: t = %d < 0", t);
    if (!offsets || !stats) return fail(MOE_ERR_INVALID, "chunk stats: null pointer");
    if (reinterpret_cast<uintptr_t>(stats) & 3) return fail(MOE_ERR_INVALID, "chunk stats: stats not 4-byte aligned");
    hipError_t e = launch_chunk_stats(offsets, t, E, stats, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "chunk stats");
    return MOE_OK;
}

moe_status moe_lookahead(const uint16_t *x, const float *w_router_next, int32_t t, int32_t h, int32_t E,
                         int32_t k, int32_t budget, float *logits, uint32_t *topk_idx, float *topk_w,
                         uint32_t *counts, uint32_t *order, uint8_t *keep, void *stream) {
    if (budget < 0) return fail(MOE_ERR_INVALID, "lookahead: budget = %d < 0", budget);
    if (!counts || !order || !keep) return fail(MOE_ERR_INVALID, "lookahead: null pointer");
    if (moe_status st = moe_route(x, w_router_next, t, h, E, k, logits, topk_idx, topk_w, stream)) return st;
    hipError_t e = launch_rank_experts(nullptr, topk_idx, t * k, E, budget, counts, order, keep,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "lookahead");
    return MOE_OK;
}

moe_status moe_block_from_residual(const float *pending_y, const moe_next_norm *in_norm, const float *w_router,
                                   int32_t t, int32_t k, int32_t E, const moe_layout *L, const uint64_t *records,
                                   const moe_layout *Ls, const void *shared_record, const uint16_t *shared_gate_w,
                                   float *logits, uint32_t *topk_idx, float *topk_w, uint32_t *offsets,
                                   uint32_t *csr_rows, float *csr_w, uint32_t *csr_pos, const moe_next_norm *out_norm,
                                   float *out, int32_t accumulate, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    if (moe_status st = check_rows(t)) return st;
    if (!in_norm) return fail(MOE_ERR_INVALID, "block_from_residual: null input-norm description");
    if (!L) return fail(MOE_ERR_INVALID, "block_from_residual: null layout");
    if (moe_status st = check_next_norm(in_norm, t, L->hidden, pending_y, "block_from_residual (input)")) return st;
    // the block reads x = in_norm->mixed; out_norm stands in for out when given
    const uint16_t *x = in_norm->mixed;
    float *out_or_copies = out_norm ? out_norm->hyper : out;
    if (moe_status st = block_check(x, w_router, t, k, E, L, records, Ls, shared_record, logits, topk_idx, topk_w,
                                    offsets, csr_rows, csr_w, csr_pos, out_or_copies, workspace, workspace_bytes,
                                    "block_from_residual"))
        return st;
    if (out_norm)
        if (moe_status st = check_next_norm(out_norm, t, L->hidden, nullptr, "block_from_residual (output)")) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    NextNormArgs n = next_norm_args(in_norm, t, L->hidden);
    n.y = pending_y;
    hipError_t e = launch_next_norm(n, s);
    if (e != hipSuccess) return hip_fail(e, "block_from_residual: input norm");
    return block_run(x, w_router, t, k, E, L, records, Ls, shared_record, shared_gate_w, logits, topk_idx, topk_w,
                     offsets, csr_rows, csr_w, csr_pos, out, accumulate, static_cast<uint8_t *>(workspace), s,
                     out_norm);
}

}  // extern "C"
