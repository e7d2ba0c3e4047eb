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
//   - the workgroup stages BM activation rows x 128 bytes (gathered through
//     csr_rows for the routed gate/up projection) and each wave its two 1 KB
//     code tiles and their fp16 scale/bias pairs straight from memory into
//     an LDS ring of 3-4 K steps (buffer loads with the lds modifier); rows
//     are XOR-swizzled in 16-byte chunks so that the B-fragment reads of 32
//     rows at one column hit distinct banks;
//   - each wave dequantises its code tiles in registers: a nibble pair OR'ed
//     into the fp16 pattern 0x6400 (= 1024 + q) feeds v_fma_mix_f32 with
//     scale s and offset (bias - 1024 s) kept in fp32, then
//     v_cvt_pk_bf16_f32 packs the MFMA operand;
//   - 4 MFMA steps of K = 16.  Inside a lane's 16 bytes the K order is
//     permuted (lane half L/32 takes 32 consecutive columns), and the
//     activation fragment uses the same permutation, so the products pair up.
// The shared expert can ride in the routed launches as one more segment of
// dense rows (moe_prefill_fused), and tiles of one or two rows take a
// matrix-core-free path (see gemv below).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

using namespace lds;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Pointers into device memory, so loads compile to global_* rather than flat_*.
#define GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_g16(const void *p) {
    const u32x4 v = *reinterpret_cast<const GLOBAL u32x4 *>(reinterpret_cast<uintptr_t>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_g4(const void *p) {
    return *reinterpret_cast<const GLOBAL uint32_t *>(reinterpret_cast<uintptr_t>(p));
}

// GU_PART / DOWN_PART: dense rows, one K range (split) per workgroup, raw
// fp32 accumulators written to a.part for k_reduce_gu / k_reduce_down.
enum Mode { GU_GATHER = 0, GU_DENSE = 1, DOWN_YE = 2, DOWN_OUT = 3, GU_PART = 4, DOWN_PART = 5 };

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Per-lane dequantisation constants of one (row, group): codes at nibble
// positions 0-3 / 16-19 become fp16 1024 + q, codes at 4-7 / 20-23 become
// 1024 + 16 q, so  w = v * s + (b - 1024 s)  or  w = v * (s/16) + (b - 64 s).
// The scale stays fp16 (v_fma_mix_f32 widens it exactly); the other three
// constants are fp32, each one v_fma_mix_f32 from the fp16 pair.
struct Deq {
    _Float16 s;
    float c, s16, c16;
};
__device__ __forceinline__ Deq deq_consts(uint32_t sb) {
    const half2_t h = __builtin_bit_cast(half2_t, sb);
    return Deq{h.x, __builtin_fmaf(-1024.0f, (float)h.x, (float)h.y), __builtin_fmaf((float)h.x, 0.0625f, 0.0f),
               __builtin_fmaf(-64.0f, (float)h.x, (float)h.y)};
}

// Loop-invariant bit masks kept in VGPRs: VOP3 on gfx950 takes no literal, so
// hiding the constants lets the compiler form v_and_or_b32.
struct Masks {
    uint32_t lo, hi, magic;
};
__device__ __forceinline__ Masks make_masks() {
    Masks m;
    asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(m.lo));
    asm volatile("v_mov_b32 %0, 0xf000f0" : "=v"(m.hi));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m.magic));
    return m;
}

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) { return (x & m) | c; }

// 8 codes of one 32-bit word (code j at bit 4*(j/2) + 16*(j%2)) -> 8 bf16 weights.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, const Deq &d, const Masks &m) {
    const uint32_t w8 = w >> 8;
    const half2_t p0 = __builtin_bit_cast(half2_t, and_or(w, m.lo, m.magic));   // q0, q1
    const half2_t p1 = __builtin_bit_cast(half2_t, and_or(w, m.hi, m.magic));   // 16 q2, 16 q3
    const half2_t p2 = __builtin_bit_cast(half2_t, and_or(w8, m.lo, m.magic));  // q4, q5
    const half2_t p3 = __builtin_bit_cast(half2_t, and_or(w8, m.hi, m.magic));  // 16 q6, 16 q7
    uint4 u;
    u.x = pk_bf16(__builtin_fmaf((float)p0.x, (float)d.s, d.c), __builtin_fmaf((float)p0.y, (float)d.s, d.c));
    u.y = pk_bf16(__builtin_fmaf((float)p1.x, d.s16, d.c16), __builtin_fmaf((float)p1.y, d.s16, d.c16));
    u.z = pk_bf16(__builtin_fmaf((float)p2.x, (float)d.s, d.c), __builtin_fmaf((float)p2.y, (float)d.s, d.c));
    u.w = pk_bf16(__builtin_fmaf((float)p3.x, d.s16, d.c16), __builtin_fmaf((float)p3.y, d.s16, d.c16));
    return __builtin_bit_cast(bf16x8, u);
}

// Few-row path: the 8 codes of one word (code j at bit 4*(j/2) + 16*(j%2))
// become four bf16 pairs 128 + q (a nibble moved to bits 0-3 / 16-19 and
// OR'ed into bf16 128.0, exact) dotted with the matching x pairs, so
// P = sum_j (128 + q_j) x_j and sum_j q_j x_j = P - 128 X.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float dot8(uint32_t w, const uint4 &xp, uint32_t mask, uint32_t mag, float p) {
    p = dot2bf(and_or(w, mask, mag), xp.x, p);          // codes 0, 1
    p = dot2bf(and_or(w >> 4, mask, mag), xp.y, p);     // codes 2, 3
    p = dot2bf(and_or(w >> 8, mask, mag), xp.z, p);     // codes 4, 5
    p = dot2bf(and_or(w >> 12, mask, mag), xp.w, p);    // codes 6, 7
    return p;
}

// SiLU(g) * u with the hardware exp and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Codes and scale/bias of a wave's two fragments for one 64-wide K step.
struct Stage {
    uint4 c[2];
    uint32_t sb[2];
};

// Staged activation rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r
// sits at position c ^ xswz(r).  For the 32 rows a B-fragment read touches at
// one logical chunk this gives 32 distinct 16-byte bank groups modulo 8, 16
// and 32, i.e. no bank conflicts for 32-, 64- or 128-bank LDS.
__device__ __forceinline__ int xswz(int r) { return (r ^ (r >> 3)) & 7; }

// LDS bytes of one workgroup of k_gemm<MODE, BM, WAVES, FEW> (see gemm_wg).
template <int MODE, int BM, int WAVES, bool FEW>
constexpr int gemm_lds_bytes() {
    constexpr bool part = (MODE == GU_PART || MODE == DOWN_PART);
    constexpr int XSTAGE = BM * 128, WSTAGE = WAVES * 2 * (1024 + 256), STAGE = XSTAGE + WSTAGE;
    constexpr int NS = (WAVES == 4 && BM == 128) ? 3 : (4 * STAGE <= 160 * 1024) ? 4 : 3;
    constexpr int EB = (MODE == DOWN_OUT || part) ? 4 : 2;
    constexpr int RING = NS * STAGE, EPI = WAVES * 32 * (32 * EB + 16);
    return FEW ? NS * XSTAGE + 3 * WSTAGE : RING > EPI ? RING : EPI;
}

// Spin limit of a down workgroup that waits for its tile's gate/up
// workgroups in the merged launch (k_gemm_gu_down): each poll is an atomic
// round trip plus a sleep of about 0.3 us, so the limit (tens of ms) is
// far beyond any one gate/up workgroup's run (well under a millisecond).
// Past it the workgroup does not hold the GPU any longer: it writes NaN in
// place of its outputs, so that a wait that never completes shows in the
// block's output instead of leaving plausible values computed from rows
// that were not ready.
constexpr int kTileWaitSpins = 1 << 15;

// One workgroup `bid` of a grouped launch.  Returns the index of the tile
// entry it ran (routed launches), else -1.  With `wait_tile`, before any
// load of its activation rows it waits until the tile entry's completion
// count (TileEntry::done, an L2 atomic) reaches a.wait_need.
// FEW: a routed launch whose every tile has one or two rows (few_row_launch):
// only the few-row path, with the waves splitting K and a 3-stage weight
// ring (46 KB of LDS, three workgroups per CU, so an XCD's list of two
// decode-shaped tiles, 2 x 48 workgroups, runs in one round).
template <int MODE, int BM, int WAVES, bool FEW = false>
__device__ __forceinline__ int gemm_wg(const GemmArgs &a, int bid, uint8_t *lds_raw, bool wait_tile) {
    constexpr bool kGateUp = (MODE == GU_GATHER || MODE == GU_DENSE || MODE == GU_PART);
    constexpr bool kPart = (MODE == GU_PART || MODE == DOWN_PART);
    constexpr bool kDense = (MODE == GU_DENSE || MODE == DOWN_OUT || kPart);
    constexpr int TB = BM / 32;                         // token blocks of 32
    // Two waves per SIMD leave 256 registers per wave: 128 accumulators
    // (two fragments x 4 token blocks) is the most that fits beside the
    // pipeline's operands, so tiles stop at 128 rows.
    static_assert(TB == 1 || TB == 2 || TB == 4, "M-tiles of 32, 64 or 128 rows");
    constexpr int XBLK = BM / 8;                        // 1 KB blocks (8 rows) per staged K step
    constexpr int XPW = XBLK / WAVES;                   // direct-to-LDS loads per wave per K step
    static_assert(BM % 32 == 0 && XBLK % WAVES == 0 && XPW >= 1, "every wave stages whole row blocks");
    constexpr int XSTAGE = BM * 128;                    // staged activation rows of one K step
    constexpr int WSTAGE = WAVES * 2 * (1024 + 256);    // per wave: 2 code tiles + 2 scale/bias blocks
    constexpr int STAGE = XSTAGE + WSTAGE;
    // ring depth: 3 K steps of lookahead when four stages fit in 160 KB of LDS,
    // else 2; 128-row tiles of 4 waves keep 3 stages (78 KB) so that two
    // workgroups fit a CU
    constexpr int NS = (WAVES == 4 && BM == 128) ? 3 : (4 * STAGE <= 160 * 1024) ? 4 : 3;
    // LDS: the NS activation stages, then the NS weight stages.
    constexpr int WRING = NS * XSTAGE;
    constexpr int FEAT = kGateUp ? 32 * WAVES : 64 * WAVES;  // output features per workgroup
    constexpr int VM_PER_STEP = XPW + 4;                // vector-memory ops a wave issues per K step
    // Epilogue: per wave 32 token rows x 32 columns, row padded by 16 bytes.
    constexpr int EB = (MODE == DOWN_OUT || kPart) ? 4 : 2;
    constexpr int EROW = 32 * EB + 16;
    constexpr int RING = NS * STAGE, EPI = WAVES * 32 * EROW;
    static_assert(!FEW || (BM == 32 && WAVES == 4 && (MODE == GU_GATHER || MODE == DOWN_YE)),
                  "few-row launches: routed, 32-row tiles, 4 waves");
    constexpr int LDS_BYTES = FEW ? NS * XSTAGE + 3 * WSTAGE : RING > EPI ? RING : EPI;
    static_assert(LDS_BYTES == gemm_lds_bytes<MODE, BM, WAVES, FEW>(), "one LDS size rule");
    // LDS byte address of the ring (wave-uniform, for the DMA's M0).
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_raw));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar

    // ---- which (M-tile, feature block).  Workgroups are dispatched to the 8
    // XCDs round-robin (XCD = blockIdx % 8) and in order within an XCD.
    // Routed: XCD x runs the tiles of its list (its share of the experts,
    // costliest tiles first), each with all its feature blocks in a row.
    // Dense: each XCD runs a contiguous eighth of the (M-tile, feature block)
    // pairs.  Either way an XCD's CUs share the weights and rows in its L2.
    const int n_out = kGateUp ? a.inter : a.hidden;
    // Few-row launches: the workgroup's waves split the K steps of one
    // fragment pair, so a workgroup covers 32 gate/up features (64 down) and
    // a launch has four times the workgroups streaming weights (each wave's
    // loop over all of K is bound by its own per-step waits).
    constexpr bool ksplit = FEW;
    const int feat_wg = ksplit ? (kGateUp ? 32 : 64) : FEAT;
    const int nblk = (n_out + feat_wg - 1) / feat_wg;
    const int xcd = bid & 7, slot_in_xcd = bid >> 3;
    int nb, expert = 0, p0, n, split = 0, tix = -1;
    // Weights that no other tile reads (the expert's only M-tile) load with
    // the non-temporal hint in 32-row tiles, the decode-shaped case; with
    // taller tiles the hint measured slower.
    bool stream_w;
    const uint8_t *rec;
    if (kDense) {
        const int per_split = ((a.t + BM - 1) / BM) * nblk;
        const int total = per_split * (kPart ? a.ksplit : 1);
        const int chunk = (total + 7) >> 3;
        const int logical = xcd * chunk + slot_in_xcd;
        if (slot_in_xcd >= chunk || logical >= total) return -1;
        split = logical / per_split;
        const int rest = logical % per_split;
        nb = rest % nblk;
        p0 = (rest / nblk) * BM;
        n = min(BM, a.t - p0);
        stream_w = BM == 32 && a.t <= BM;
        rec = static_cast<const uint8_t *>(a.record);
    } else {
        // The entry is loaded together with the count (the grid never
        // exceeds xcap slots per XCD, so the read stays inside the list).
        tix = xcd * a.xcap + slot_in_xcd / nblk;
        const TileEntry te = a.order[tix];
        if (slot_in_xcd >= (int)a.sched_n[kSchedXcnt + xcd] * nblk) return -1;
        nb = slot_in_xcd % nblk;
        expert = te.expert;
        p0 = te.p0;
        n = te.n;
        stream_w = BM == 32 && te.tiles == 1;
        rec = static_cast<const uint8_t *>(te.rec);
        if (!rec) return -1;   // a used expert left without a record: no read of address 0
    }
    (void)expert;

    const int K = kGateUp ? a.hidden : a.inter;
    // K steps of this workgroup: all of them, or one split's range
    // (the host picks splits that divide the step count)
    const int nk_all = K >> 6;                            // K steps of the record's rows
    const int nk = kPart ? nk_all / a.ksplit : nk_all;
    const int kbase = split * nk;
    const int obs = n_out >> 5;
    int ob[2];
    const int fblk = ksplit ? nb : nb * WAVES + wave;   // this wave's fragment pair
    if (kGateUp) {
        ob[0] = ob[1] = fblk;                            // gate and up of the same 32 features
    } else {
        ob[0] = fblk * 2;                                // two adjacent 32-feature blocks
        ob[1] = ob[0] + 1;
    }
    const bool live0 = ob[0] < obs, live1 = ob[1] < obs;
    const i32x4 rrec = buffer_rsrc(rec);
    uint32_t wvo[2], svo[2];                              // per-lane byte offsets in the record
    const int sb_tile_bytes = (64 / a.group) * 32 * 4;
    const int sb_entry = (a.group == 64) ? (lane & 31) : lane;
    #pragma unroll
    for (int f = 0; f < 2; ++f) {
        const bool live = f ? live1 : live0;
        const uint32_t row0 = (uint32_t)(live ? ob[f] : 0) * nk_all;  // first tile of the row block
        const uint32_t wo = (uint32_t)((kGateUp && f) ? a.w2_off : a.w_off);
        const uint32_t so = (uint32_t)((kGateUp && f) ? a.sb2_off : a.sb_off);
        wvo[f] = wo + row0 * 1024 + lane * 16;
        svo[f] = so + row0 * sb_tile_bytes + sb_entry * 4;
    }

    // ---- activation rows this wave stages: block blk = wave*XPW + j covers
    // rows 8*blk .. 8*blk+7; lane s writes LDS bytes 16 s of the block, which
    // hold chunk (s%8) ^ xswz(row) of row 8*blk + s/8.  Rows past the tile
    // load row 0 of the tile (never read back for a stored output).
    const i32x4 rx = buffer_rsrc(kGateUp ? a.x : a.act);
    uint32_t xvo[XPW];                                    // per-lane byte offsets of the staged rows
    #pragma unroll
    for (int j = 0; j < XPW; ++j) {
        const int r = (wave * XPW + j) * 8 + (lane >> 3);
        const int rr = r < n ? r : 0;
        uint32_t row;
        if (MODE == GU_GATHER)
            row = (a.shared_rows && p0 >= a.shared_p0) ? (uint32_t)(p0 + rr - a.shared_p0) : a.rows[p0 + rr];
        else
            row = (uint32_t)(p0 + rr);
        xvo[j] = row * (uint32_t)(kGateUp ? a.hidden : a.inter) * 2u + (uint32_t)(((lane & 7) ^ xswz(r)) * 16);
    }
    // Everything a K step needs goes straight from memory into its ring slot
    // by DMA: the wave's share of the activation rows, its two 1 KB code tiles
    // and their scale/bias entries.  No loop load has a register destination,
    // so the only waits are the explicit vmcnt counts below.
    auto wcode = [&](int slot, int f) { return WRING + (slot % NS) * WSTAGE + (wave * 2 + f) * 1024; };
    auto wsb = [&](int slot, int f) { return WRING + (slot % NS) * WSTAGE + WAVES * 2048 + (wave * 2 + f) * 256; };
    // The wave's weights of K step ks (code tiles and scale/bias), 4 loads.
    auto issue_w = [&](int ks, int slot) {
        const int kg = kbase + ks;
        #pragma unroll
        for (int f = 0; f < 2; ++f) {
            if (stream_w) {
                dma16nt(lds_base + wcode(slot, f), wvo[f], rrec, (uint32_t)kg * 1024u);
                dma4nt(lds_base + wsb(slot, f), svo[f], rrec, (uint32_t)(kg * sb_tile_bytes));
            } else {
                dma16(lds_base + wcode(slot, f), wvo[f], rrec, (uint32_t)kg * 1024u);
                dma4(lds_base + wsb(slot, f), svo[f], rrec, (uint32_t)(kg * sb_tile_bytes));
            }
        }
    };
    auto issue = [&](int ks, int slot) {
        const uint32_t xd = lds_base + (slot % NS) * XSTAGE + wave * XPW * 1024;
        const uint32_t xs = (uint32_t)(kbase + ks) * 128u;
        #pragma unroll
        for (int j = 0; j < XPW; ++j) dma16(xd + j * 1024, xvo[j], rx, xs);
        issue_w(ks, slot);
    };
    // This wave's weights of the K step in `slot`, from LDS.
    auto read_w = [&](int slot, Stage &st) {
        #pragma unroll
        for (int f = 0; f < 2; ++f) {
            st.c[f] = *reinterpret_cast<const uint4 *>(lds_raw + wcode(slot, f) + lane * 16);
            st.sb[f] = *reinterpret_cast<const uint32_t *>(lds_raw + wsb(slot, f) + lane * 4);
        }
    };

    // The tile's token blocks that hold rows: the K loop and epilogue below
    // are compiled for each count, so MFMAs and LDS reads of empty blocks are
    // skipped (row staging stays uniform).
    auto body = [&](auto tbr_c) {
        constexpr int TBR = decltype(tbr_c)::value;
        f32x16 acc[2][TBR];
        #pragma unroll
        for (int f = 0; f < 2; ++f)
            #pragma unroll
            for (int b = 0; b < TBR; ++b)
                #pragma unroll
                for (int r = 0; r < 16; ++r) acc[f][b][r] = 0.0f;

        const Masks msk = make_masks();
        const int brow = lane & 31, bhalf = lane >> 5;
        // Lane offset of the B fragment of token block b at MFMA step st:
        // row b*32 + brow, chunk (4*bhalf + st) ^ xswz(row).  Since
        // xswz(b*32 + brow) = xswz(brow) ^ 4*(b&1), the offset is
        // b*4096 + boff[b&1][st]: eight lane offsets plus immediates.
        uint32_t boff[2][4];
        #pragma unroll
        for (int p = 0; p < 2; ++p)
            #pragma unroll
            for (int st = 0; st < 4; ++st)
                boff[p][st] = brow * 128 + (((4 * bhalf + st) ^ xswz(brow) ^ (4 * p)) & 7) * 16;

        // Prologue: one K step in flight per ring slot.  Every step issues the
        // same loads -- past the last step it reloads step nk-1 into a free slot
        // -- so the vmcnt counts below hold on every iteration.
        #pragma unroll
        for (int j = 0; j < NS; ++j) issue(min(j, nk - 1), j);

        auto frag = [&](const Stage &sg, int st, const Deq &d0, const Deq &d1, bf16x8 *out) {
            const uint32_t w0 = st == 0 ? sg.c[0].x : st == 1 ? sg.c[0].y : st == 2 ? sg.c[0].z : sg.c[0].w;
            const uint32_t w1 = st == 0 ? sg.c[1].x : st == 1 ? sg.c[1].y : st == 2 ? sg.c[1].z : sg.c[1].w;
            out[0] = dequant8(w0, d0, msk);
            out[1] = dequant8(w1, d1, msk);
        };
        // B fragments (32 token rows x 8 K values per lane) of MFMA step st of the
        // K step staged in `slot`.
        auto read_b = [&](int slot, int st, bf16x8 *out) {
            const uint32_t sx = (uint32_t)((slot % NS) * XSTAGE);
            const uint32_t o0 = sx + boff[0][st], o1 = sx + boff[1][st];
            #pragma unroll
            for (int b = 0; b < TBR; ++b)
                out[b] = *reinterpret_cast<const bf16x8 *>(lds_raw + ((b & 1) ? o1 : o0) + b * 4096);
        };
        // Step 0 has landed for every wave once each has waited for its own loads
        // and all have met at the barrier.
        wait_vm<(NS - 1) * VM_PER_STEP>();
        barrier_no_fence();
        Stage cur;
        read_w(0, cur);
        bf16x8 af[2], bcur[TBR];
        read_b(0, 0, bcur);
        // dequantisation constants of the current K step's two fragments,
        // formed once (region 3 of the step before forms the next ones)
        Deq dq0 = deq_consts(cur.sb[0]), dq1 = deq_consts(cur.sb[1]);
        frag(cur, 0, dq0, dq1, af);

        // K step kb: four MFMA steps of K = 16, each a scheduling region of its
        // own.  Region st issues the LDS reads of region st+1's operands (the next
        // B fragments; in region 3 the first B fragments and the weights of step
        // kb+1) ahead of its MFMAs and dequantises the next weight fragments
        // between them, so no MFMA waits for an LDS read issued just before it.
        // After region 2's MFMAs every wave waits for its own loads of step kb+1
        // and meets the others at a barrier: step kb+1 is then complete in LDS,
        // and slot kb, whose last reads were issued in region 2, is free for the
        // loads of step kb+NS.
        // The step's ring slot (kb mod NS) is a compile-time constant of each
        // copy of the body, so every LDS read address is a fixed lane offset
        // plus an immediate: no per-step address arithmetic on the VALU.
        auto kstep = [&](int kb, auto slot_c) {
            constexpr int SL = decltype(slot_c)::value;   // == kb % NS
            const Deq d0 = dq0, d1 = dq1;
            Stage nxt;
            #pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 a0 = af[0], a1 = af[1];
                bf16x8 bnxt[TBR];
                if (st < 3) {
                    read_b(SL, st + 1, bnxt);
                    frag(cur, st + 1, d0, d1, af);
                } else {
                    read_w(SL + 1, nxt);                       // past the end: a reloaded step, unused
                    read_b(SL + 1, 0, bnxt);
                    dq0 = deq_consts(nxt.sb[0]);
                    dq1 = deq_consts(nxt.sb[1]);
                    frag(nxt, 0, dq0, dq1, af);
                }
                #pragma unroll
                for (int b = 0; b < TBR; ++b) {
                    acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bcur[b], acc[0][b], 0, 0, 0);
                    acc[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bcur[b], acc[1][b], 0, 0, 0);
                }
                if (st < 3)
                    __builtin_amdgcn_sched_group_barrier(0x100, TBR, 0);       // the LDS reads first
                else
                    __builtin_amdgcn_sched_group_barrier(0x100, TBR + 4, 0);
                #pragma unroll
                for (int m = 0; m < 2 * TBR; ++m) {
                    // one MFMA, then a slice of VALU that issues during its
                    // 32 cycles (an MFMA pair would block the wave at the
                    // second MFMA with no VALU in between); slices of about
                    // 40 / (2 TBR) spread a region's ~37 VALU over all its
                    // MFMAs (same box: 1% faster than 48 / (2 TBR))
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 20 / TBR, 0);
                }
                if (st == 2) {
                    wait_vm<(NS - 2) * VM_PER_STEP>();
                    barrier_no_fence();
                    issue(min(kb + NS, nk - 1), SL);
                }
                __builtin_amdgcn_sched_barrier(0);
                #pragma unroll
                for (int b = 0; b < TBR; ++b) bcur[b] = bnxt[b];
            }
            cur = nxt;
        };
        for (int kb = 0; kb < nk; kb += NS) {
            kstep(kb, std::integral_constant<int, 0>{});
            if (kb + 1 < nk) kstep(kb + 1, std::integral_constant<int, 1>{});
            if (kb + 2 < nk) kstep(kb + 2, std::integral_constant<int, 2>{});
            if constexpr (NS > 3)
                if (kb + 3 < nk) kstep(kb + 3, std::integral_constant<int, 3>{});
        }
        wait_vm<0>();  // retire the trailing (unused) loads before the ring is reused

        // ---- epilogue.  acc[f][b][r] holds feature 8*(r/4) + 4*(lane/32) + r%4 of
        // fragment f for token b*32 + lane%32.  Each 32-token block of one
        // fragment goes through the wave's LDS tile so that global stores are
        // whole 16-byte pieces of contiguous 64 or 128 byte row segments.
        __syncthreads();  // every wave is done reading the ring
        if (!live0) return;
        uint8_t *ep = lds_raw + wave * 32 * EROW;
        constexpr int CPR = 32 * EB / 16;                    // 16-byte chunks per row
        constexpr int PER_LANE = 32 * CPR / 64;
        constexpr int PASSES = (kGateUp && !kPart) ? 1 : 2;
        #pragma unroll
        for (int b = 0; b < TBR; ++b) {
            #pragma unroll
            for (int f = 0; f < PASSES; ++f) {
                if (f == 1 && !live1) break;
                #pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int col = 8 * q4 + 4 * bhalf;
                    if (kGateUp && !kPart) {
                        uint2 v;
                        v.x = pk_bf16(silu_mul(acc[0][b][4 * q4 + 0], acc[1][b][4 * q4 + 0]),
                                      silu_mul(acc[0][b][4 * q4 + 1], acc[1][b][4 * q4 + 1]));
                        v.y = pk_bf16(silu_mul(acc[0][b][4 * q4 + 2], acc[1][b][4 * q4 + 2]),
                                      silu_mul(acc[0][b][4 * q4 + 3], acc[1][b][4 * q4 + 3]));
                        *reinterpret_cast<uint2 *>(ep + brow * EROW + col * 2) = v;
                    } else if (MODE == DOWN_YE) {
                        uint2 v;
                        v.x = pk_bf16(acc[f][b][4 * q4 + 0], acc[f][b][4 * q4 + 1]);
                        v.y = pk_bf16(acc[f][b][4 * q4 + 2], acc[f][b][4 * q4 + 3]);
                        *reinterpret_cast<uint2 *>(ep + brow * EROW + col * 2) = v;
                    } else {
                        *reinterpret_cast<float4 *>(ep + brow * EROW + col * 4) =
                            make_float4(acc[f][b][4 * q4 + 0], acc[f][b][4 * q4 + 1], acc[f][b][4 * q4 + 2],
                                        acc[f][b][4 * q4 + 3]);
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                const int colf = ob[f] * 32;                   // first feature of this fragment
                #pragma unroll
                for (int i = 0; i < PER_LANE; ++i) {
                    const int idx = lane + 64 * i;
                    const int row = idx / CPR, ch = idx % CPR;
                    const int tok = b * 32 + row;
                    if (tok >= n) continue;
                    const int col = ch * 16 / EB;
                    const size_t p = (size_t)(p0 + tok);
                    const uint4 v = *reinterpret_cast<const uint4 *>(ep + row * EROW + ch * 16);
                    if (kPart) {
                        // gate/up partials: gate in [0, I), up in [I, 2I) of each row
                        const size_t nf = kGateUp ? 2 * (size_t)a.inter : (size_t)a.hidden;
                        const size_t f0 = (kGateUp && f) ? (size_t)a.inter : 0;
                        *reinterpret_cast<uint4 *>(a.part + ((size_t)split * a.t + p) * nf + f0 + colf + col) = v;
                    } else if (kGateUp) {
                        *reinterpret_cast<uint4 *>(a.hg + p * a.inter + colf + col) = v;
                    } else if (MODE == DOWN_YE) {
                        *reinterpret_cast<uint4 *>(a.ye + p * a.hidden + colf + col) = v;
                    } else {
                        const float g = a.gate ? a.gate[p] : 1.0f;
                        float4 *o = reinterpret_cast<float4 *>(a.out + p * a.hidden + colf + col);
                        float4 r = make_float4(g * __uint_as_float(v.x), g * __uint_as_float(v.y),
                                               g * __uint_as_float(v.z), g * __uint_as_float(v.w));
                        if (a.accumulate) {
                            const float4 old = *o;
                            r.x += old.x;
                            r.y += old.y;
                            r.z += old.z;
                            r.w += old.w;
                        }
                        *o = r;
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            }
        }
    };
    // ---- few-row path (routed tiles of 1 or 2 rows): no MFMA; each lane
    // dots its 32 codes per K step with the rows' x values and applies the
    // group's scale and bias once per step:  w.x summed over the lane's
    // columns = s P + (b - 128 s) X, with X the sum of those x.  The weights
    // are never rounded to bf16.  Lanes L and L+32 hold the two column halves
    // of feature row 32 ob + L%32 and are added at the end.
    // The NR rows are staged whole, once, at the start of the row ring (the
    // caller checks that they fit); after that every wave streams only its
    // own weight slots, so the K loop has no barrier: a wave waits for its
    // own loads and for its own LDS reads of a slot before refilling it.
    auto gemv = [&](auto nr_c) {
        constexpr int NR = decltype(nr_c)::value;
        constexpr int VMW = 4;                            // weight loads per K step
        // weight ring: the LDS after the staged rows (as many stages as the
        // MFMA path's ring; six stages measured no faster)
        constexpr int WR0 = NS * XSTAGE;
        constexpr int NSG = (LDS_BYTES - WR0) / WSTAGE < 8 ? (LDS_BYTES - WR0) / WSTAGE : 8;
        static_assert(NSG >= 3, "a weight ring of at least three stages");
        auto gcode = [&](int slot, int f) { return WR0 + (slot % NSG) * WSTAGE + (wave * 2 + f) * 1024; };
        auto gsb = [&](int slot, int f) { return WR0 + (slot % NSG) * WSTAGE + WAVES * 2048 + (wave * 2 + f) * 256; };
        auto issue_g = [&](int ks, int slot) {
            #pragma unroll
            for (int f = 0; f < 2; ++f) {
                dma16nt(lds_base + gcode(slot, f), wvo[f], rrec, (uint32_t)ks * 1024u);
                dma4nt(lds_base + gsb(slot, f), svo[f], rrec, (uint32_t)(ks * sb_tile_bytes));
            }
        };
        auto read_g = [&](int slot, Stage &st) {
            #pragma unroll
            for (int f = 0; f < 2; ++f) {
                st.c[f] = *reinterpret_cast<const uint4 *>(lds_raw + gcode(slot, f) + lane * 16);
                st.sb[f] = *reinterpret_cast<const uint32_t *>(lds_raw + gsb(slot, f) + lane * 4);
            }
        };
        uint32_t mask, mag, one2;
        asm volatile("v_mov_b32 %0, 0xf000f" : "=v"(mask));
        asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(mag));      // bf16 128.0 pair
        asm volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(one2));     // bf16 1.0 pair
        const int half = lane >> 5;
        const int rowb = K * 2;                           // bytes of one staged row
        // K steps [k0, k0 + kw) of this wave (all of them unless the waves
        // split K; the host then picks step counts that divide by 4).  The
        // first NSG steps go out before the rows: their addresses need only
        // the tile entry, the rows' need the row ids loaded first.
        const int kw = ksplit ? nk / WAVES : nk;
        const int k0 = ksplit ? wave * kw : 0;
        #pragma unroll
        for (int j = 0; j < NSG; ++j) issue_g(k0 + min(j, kw - 1), j);
        {
            // rows r < NR at LDS byte r * rowb; 1 KB DMA chunks, lane i of
            // chunk j carries bytes 1024 j + 16 i (rows are 128-byte multiples,
            // so a 16-byte piece never straddles two rows; pieces past the end
            // reload the first piece and land inside the row ring).
            uint32_t rowbase[NR];
            #pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int q = p0 + min(r, n - 1);
                const bool sh = a.shared_rows && p0 >= a.shared_p0;   // shared expert: dense rows
                const uint32_t row = (MODE == GU_GATHER && !sh) ? __builtin_nontemporal_load(a.rows + q)
                                     : (MODE == GU_GATHER) ? (uint32_t)(q - a.shared_p0) : (uint32_t)q;
                rowbase[r] = __builtin_amdgcn_readfirstlane(row) * (uint32_t)rowb;
            }
            const int total = NR * rowb;
            const int chunks = (total + 1023) >> 10;
            for (int j = wave; j < chunks; j += WAVES) {
                const int bt = j * 1024 + lane * 16;
                const int r = (NR == 2 && bt >= rowb) ? 1 : 0;
                const uint32_t voff = bt < total ? rowbase[r] + (uint32_t)(bt - r * rowb) : rowbase[0];
                dma16(lds_base + j * 1024, voff, rx, 0);
            }
        }
        auto read_x = [&](int kb, uint4 (&xw)[NR][4]) {
            #pragma unroll
            for (int r = 0; r < NR; ++r)
                #pragma unroll
                for (int c = 0; c < 4; ++c)
                    xw[r][c] = *reinterpret_cast<const uint4 *>(lds_raw + r * rowb + kb * 128 + half * 64 + c * 16);
        };
        float acc[2][NR];
        #pragma unroll
        for (int f = 0; f < 2; ++f)
            #pragma unroll
            for (int r = 0; r < NR; ++r) acc[f][r] = 0.0f;
        // every wave's rows and this wave's first NSG steps have landed; the
        // barrier makes the rows visible to all waves
        wait_vm<0>();
        barrier_no_fence();
        Stage cur;
        uint4 xc[NR][4];
        read_g(0, cur);
        read_x(k0, xc);
        for (int j = 0; j < kw; ++j) {
            // local step j+1 of this wave has landed; its reads of slot j are done
            wait_vm<(NSG - 2) * VMW>();
            __builtin_amdgcn_s_waitcnt((15 << 0) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
            issue_g(k0 + min(j + NSG, kw - 1), j + NSG);
            Stage nxt;
            uint4 xn[NR][4];
            read_g(j + 1, nxt);                           // past the end: a reloaded step, unused
            read_x(k0 + min(j + 1, kw - 1), xn);
            #pragma unroll
            for (int r = 0; r < NR; ++r) {
                float X = 0.0f;
                #pragma unroll
                for (int c = 0; c < 4; ++c) {
                    X = dot2bf(one2, xc[r][c].x, X);
                    X = dot2bf(one2, xc[r][c].y, X);
                    X = dot2bf(one2, xc[r][c].z, X);
                    X = dot2bf(one2, xc[r][c].w, X);
                }
                #pragma unroll
                for (int f = 0; f < 2; ++f) {
                    float P = 0.0f;
                    P = dot8(cur.c[f].x, xc[r][0], mask, mag, P);
                    P = dot8(cur.c[f].y, xc[r][1], mask, mag, P);
                    P = dot8(cur.c[f].z, xc[r][2], mask, mag, P);
                    P = dot8(cur.c[f].w, xc[r][3], mask, mag, P);
                    const half2_t sb = __builtin_bit_cast(half2_t, cur.sb[f]);
                    const float cc = __builtin_fmaf(-128.0f, (float)sb.x, (float)sb.y);
                    acc[f][r] = __builtin_fmaf(cc, X, __builtin_fmaf((float)sb.x, P, acc[f][r]));
                }
            }
            cur = nxt;
            #pragma unroll
            for (int r = 0; r < NR; ++r)
                #pragma unroll
                for (int c = 0; c < 4; ++c) xc[r][c] = xn[r][c];
        }
        wait_vm<0>();  // retire the trailing (unused) loads before the workgroup's LDS goes away
        // both column halves of a feature: lane l and l +- 32
        #pragma unroll
        for (int f = 0; f < 2; ++f)
            #pragma unroll
            for (int r = 0; r < NR; ++r) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[f][r]), __float_as_uint(acc[f][r]),
                                                                 false, false);
                acc[f][r] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
        if (ksplit) {
            // the waves' K ranges, added in wave order by wave 0: every wave
            // is done with its ring (loads retired above) and the staged
            // rows, so the row area holds the partial sums
            float *red = reinterpret_cast<float *>(lds_raw);   // [WAVES][2][NR][32]
            barrier_no_fence();
            if (lane < 32) {
                #pragma unroll
                for (int f = 0; f < 2; ++f)
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) red[((wave * 2 + f) * NR + r) * 32 + lane] = acc[f][r];
            }
            barrier_no_fence();
            if (wave != 0) return;
            #pragma unroll
            for (int f = 0; f < 2; ++f)
                #pragma unroll
                for (int r = 0; r < NR; ++r) {
                    float v = red[(f * NR + r) * 32 + (lane & 31)];
                    #pragma unroll
                    for (int w = 1; w < WAVES; ++w) v += red[((w * 2 + f) * NR + r) * 32 + (lane & 31)];
                    acc[f][r] = v;
                }
        }
        if (!live0) return;
        const int feat = lane & 31;
        #pragma unroll
        for (int r = 0; r < NR; ++r) {
            if (r >= n) break;
            const size_t p = (size_t)(p0 + r);
            if (kGateUp) {
                if (half == 0) {
                    const float v = silu_mul(acc[0][r], acc[1][r]);
                    a.hg[p * a.inter + ob[0] * 32 + feat] = (uint16_t)(pk_bf16(v, 0.0f) & 0xffffu);
                }
            } else {
                // lanes 0-31 store fragment 0, lanes 32-63 fragment 1
                const int f = half;
                if (f == 0 || live1) {
                    const float v = f ? acc[1][r] : acc[0][r];
                    a.ye[p * a.hidden + ob[f] * 32 + feat] = (uint16_t)(pk_bf16(v, 0.0f) & 0xffffu);
                }
            }
        }
    };
    if (MODE == DOWN_YE && wait_tile) {
        // The tile's rows come from the gate/up workgroups of the same XCD
        // list entry, which ran on this XCD (workgroup i goes to XCD i mod 8
        // and the merged launch keeps each tile's producers and consumers on
        // one residue), so their stores sit in this XCD's L2; once the count
        // is complete only this CU's vector L1 may hold stale lines.
        // The count is read with an atomic add of a.wait_zero (0, unknown to
        // the compiler), so the read is a read-modify-write performed where
        // the gate/up workgroups' additions are, never a plain load.
        __shared__ int gave_up;
        if (tid == 0) {
            uint32_t *done = const_cast<uint32_t *>(&a.order[tix].done);
            int ready = 0;
            for (int i = 0; i < a.wait_spins; ++i) {
                if (__hip_atomic_fetch_add(done, (uint32_t)a.wait_zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                    (uint32_t)a.wait_need) {
                    ready = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(10);
            }
            gave_up = !ready;
        }
        __syncthreads();
        if (gave_up) {
            // bf16 quiet NaN over this workgroup's rows and features of ye
            const int c0 = nb * feat_wg, nc = min(feat_wg, n_out - c0);
            if constexpr (MODE == DOWN_YE)
                for (int i = tid; i < n * nc; i += 64 * WAVES)
                    a.ye[(size_t)(p0 + i / nc) * n_out + c0 + i % nc] = 0x7fc0;
            return tix;
        }
        asm volatile("buffer_inv sc0" ::: "memory");
    }
    if constexpr (!kDense) {
        static_assert(BM != 32 || NS * XSTAGE == kFewRowBytes, "few-row staging size known to the host");
        // few rows whose whole K fits in the row ring: the no-MFMA path
        // (a few-row launch has only such tiles: n <= t <= 2, rows checked
        // to fit by the host)
        if (FEW || (n <= 2 && ((n * K * 2 + 1023) >> 10) * 1024 <= NS * XSTAGE)) {
            if (n == 1) gemv(std::integral_constant<int, 1>{});
            else gemv(std::integral_constant<int, 2>{});
            return tix;
        }
    }
    if constexpr (!FEW) {   // (a discarded branch: no matrix-core path in a few-row launch)
        const int tbr = (n + 31) >> 5;
        if constexpr (TB == 4) {
            if (tbr >= 4) body(std::integral_constant<int, 4>{});
            else if (tbr == 3) body(std::integral_constant<int, 3>{});
            else if (tbr == 2) body(std::integral_constant<int, 2>{});
            else body(std::integral_constant<int, 1>{});
        } else if constexpr (TB == 2) {
            if (tbr >= 2) body(std::integral_constant<int, 2>{});
            else body(std::integral_constant<int, 1>{});
        } else {
            body(std::integral_constant<int, 1>{});
        }
    }
    return tix;
}

template <int MODE, int BM, int WAVES, bool FEW = false>
__global__ void __launch_bounds__(64 * WAVES, FEW ? 3 : (WAVES >= 8 ? 1 : 2)) k_gemm(const GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[gemm_lds_bytes<MODE, BM, WAVES, FEW>()];
    gemm_wg<MODE, BM, WAVES, FEW>(a, blockIdx.x, lds_raw, false);
}

// The routed gate/up and down projections in one launch: workgroups
// [0, g1) run the gate/up grid, the rest the down grid over the same tile
// lists.  A gate/up workgroup, once its SiLU*up rows are stored, adds one
// to its tile entry's count; a down workgroup waits for the count of its
// tile to reach the tile's number of gate/up workgroups.  Workgroups reach
// each XCD in ascending order, so every gate/up workgroup of an XCD is
// dispatched before its first down workgroup, which therefore only fills
// slots the gate/up launch would have left idle at its end; g1 is a
// multiple of 8, so a tile's down workgroups run on the XCD of its gate/up
// workgroups and read their rows from that XCD's L2.
template <int BM>
__global__ void __launch_bounds__(256, 2) k_gemm_gu_down(const GemmArgs gu, const GemmArgs dn, int g1) {
    constexpr int kLds = gemm_lds_bytes<GU_GATHER, BM, 4, false>() > gemm_lds_bytes<DOWN_YE, BM, 4, false>()
                             ? gemm_lds_bytes<GU_GATHER, BM, 4, false>()
                             : gemm_lds_bytes<DOWN_YE, BM, 4, false>();
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[kLds];
    const int bid = blockIdx.x;
    if (bid < g1) {
        const int tix = gemm_wg<GU_GATHER, BM, 4, false>(gu, bid, lds_raw, false);
        if (tix >= 0) {
            wait_vm<0>();   // this wave's stores of hg have reached the L2
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(const_cast<uint32_t *>(&gu.order[tix].done), 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        gemm_wg<DOWN_YE, BM, 4, false>(dn, bid - g1, lds_raw, true);
    }
}

// out[r, :] (+)= sum over the row's k CSR entries, in ascending CSR position
// (= ascending expert id), of csr_w[p] * ye[p, :].  One workgroup of CT
// threads per (row, 8 CT columns); each thread owns 8 columns.  The first
// wave ranks the row's k positions (distinct, k <= 32) into LDS; then every
// thread issues the loads of up to 16 entries and their weights before the
// FMAs, so it waits for memory once per 16 entries; the FMAs still run in
// ascending position.
template <int CT>
__global__ void __launch_bounds__(CT) k_combine(const uint16_t *__restrict__ ye,
                                                const uint32_t *__restrict__ pos,
                                                const float *__restrict__ csr_w, int t, int k,
                                                int h, float *__restrict__ out, int accumulate,
                                                const uint16_t *__restrict__ ys,
                                                const float *__restrict__ gate) {
    __shared__ uint32_t ps[MOE_MAX_K];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int c = (blockIdx.y * CT + tid) * 8;
    const bool live = c < h;
    float acc[8];
    float4 *o = reinterpret_cast<float4 *>(out + (size_t)r * h + (live ? c : 0));
    if (accumulate && live) {
        const float4 o0 = o[0], o1 = o[1];
        acc[0] = o0.x; acc[1] = o0.y; acc[2] = o0.z; acc[3] = o0.w;
        acc[4] = o1.x; acc[5] = o1.y; acc[6] = o1.z; acc[7] = o1.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    if (ys && live) {
        // the shared expert's row first (scaled by its gate), as the separate
        // shared call would have left it in out
        const uint4 v = *reinterpret_cast<const uint4 *>(ys + (size_t)r * h + c);
        const float g = gate ? gate[r] : 1.0f;
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = acc[2 * i] + g * __uint_as_float(u[i] << 16);
            acc[2 * i + 1] = acc[2 * i + 1] + g * __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    if (tid < 64) {
        const uint32_t mine = tid < k ? pos[(size_t)r * k + tid] : 0xffffffffu;
        int rank = 0;
        for (int i = 0; i < k; ++i) rank += (uint32_t)__builtin_amdgcn_readlane((int)mine, i) < mine;
        if (tid < k) ps[rank] = mine;
    }
    __syncthreads();
    if (!live) return;
    for (int j0 = 0; j0 < k; j0 += 16) {
        uint4 v[16];
        float wj[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (j0 + j < k) {
                const uint32_t p = ps[j0 + j];
                // ye is read once: non-temporal loads (and stores of out below)
                const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ye + (size_t)p * h + c));
                v[j] = make_uint4(q.x, q.y, q.z, q.w);
                wj[j] = csr_w[p];
            }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j0 + j < k) {
                const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = __builtin_fmaf(wj[j], __uint_as_float(u[i] << 16), acc[2 * i]);
                    acc[2 * i + 1] = __builtin_fmaf(wj[j], __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
                }
            }
        }
    }
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store((f32x4_t){acc[0], acc[1], acc[2], acc[3]}, reinterpret_cast<f32x4_t *>(o));
    __builtin_nontemporal_store((f32x4_t){acc[4], acc[5], acc[6], acc[7]}, reinterpret_cast<f32x4_t *>(o) + 1);
}

// Split-K reductions of the shared expert (small chunks): partial sums of
// the S K ranges added in ascending range order, then the epilogue of the
// unsplit kernel (SiLU(g)*u to bf16, or gate * d (+ out) in fp32).
// One thread per 4 consecutive features of one row.
__global__ void __launch_bounds__(256) k_reduce_gu(const float *__restrict__ part, int S, int t, int I,
                                                   uint16_t *__restrict__ hs) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= t * (I / 4)) return;
    const int r = i / (I / 4), c = (i % (I / 4)) * 4;
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
    // splits in ascending order; the loads of 16 splits go out together
    for (int s0 = 0; s0 < S; s0 += 16) {
        float4 a[16], b[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (s0 + j < S) {
                const float *row = part + ((size_t)(s0 + j) * t + r) * 2 * I;
                a[j] = *reinterpret_cast<const float4 *>(row + c);
                b[j] = *reinterpret_cast<const float4 *>(row + I + c);
            }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (s0 + j < S) {
                g.x += a[j].x; g.y += a[j].y; g.z += a[j].z; g.w += a[j].w;
                u.x += b[j].x; u.y += b[j].y; u.z += b[j].z; u.w += b[j].w;
            }
    }
    uint2 v;
    v.x = pk_bf16(silu_mul(g.x, u.x), silu_mul(g.y, u.y));
    v.y = pk_bf16(silu_mul(g.z, u.z), silu_mul(g.w, u.w));
    *reinterpret_cast<uint2 *>(hs + (size_t)r * I + c) = v;
}

__global__ void __launch_bounds__(256) k_reduce_down(const float *__restrict__ part, int S, int t, int h,
                                                     const float *__restrict__ gate, float *__restrict__ out,
                                                     int accumulate) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= t * (h / 4)) return;
    const int r = i / (h / 4), c = (i % (h / 4)) * 4;
    float4 d = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < S; s0 += 16) {
        float4 a[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (s0 + j < S) a[j] = *reinterpret_cast<const float4 *>(part + ((size_t)(s0 + j) * t + r) * h + c);
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (s0 + j < S) {
                d.x += a[j].x; d.y += a[j].y; d.z += a[j].z; d.w += a[j].w;
            }
    }
    const float gr = gate ? gate[r] : 1.0f;
    float4 *o = reinterpret_cast<float4 *>(out + (size_t)r * h + c);
    float4 res = make_float4(gr * d.x, gr * d.y, gr * d.z, gr * d.w);
    if (accumulate) {
        const float4 old = *o;
        res.x += old.x; res.y += old.y; res.z += old.z; res.w += old.w;
    }
    *o = res;
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

inline int routed_per_xcd(const GemmArgs &a, int bm);

// moe_debug_tile_wait's settings (host side, process-wide).
std::atomic<int> g_wait_spins{0}, g_wait_extra{0};

template <int MODE, int WAVES>
hipError_t launch_waves(const GemmArgs &a, int bm, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const bool gu = (MODE == GU_GATHER || MODE == GU_DENSE || MODE == GU_PART);
    const bool part = (MODE == GU_PART || MODE == DOWN_PART);
    const bool dense = (MODE == GU_DENSE || MODE == DOWN_OUT || part);
    const int n_out = gu ? a.inter : a.hidden;
    const bool few = (MODE == GU_GATHER || MODE == DOWN_YE) && bm == 32 && few_row_launch(a.t, gu ? a.hidden : a.inter);
    const int feat = few ? (gu ? 32 : 64) : (gu ? 32 * WAVES : 64 * WAVES);
    const int nblk = (n_out + feat - 1) / feat;
    int grid;
    if (dense) {
        // 1-D grid, rounded so every XCD slot of the remap exists
        grid = (((a.t + bm - 1) / bm * nblk * (part ? a.ksplit : 1) + 7) / 8) * 8 + 8;
    } else {
        grid = 8 * routed_per_xcd(a, bm) * nblk;
    }
    // hipExtLaunchKernel only when timing events are attached: it leaves an
    // idle gap of a few microseconds before the kernel even without events
    // (decode-shaped chunk, three untimed GEMM launches: 0.212 -> 0.203 ms).
    auto go = [&](auto kernel, int threads) {
        if (e0 || e1)
            hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, e0, e1, 0, a);
        else
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, a);
    };
    if constexpr ((MODE == GU_GATHER || MODE == DOWN_YE) && WAVES == 4) {
        if (few) {
            go(k_gemm<MODE, 32, 4, true>, 256);
            return hipGetLastError();
        }
    }
    switch (bm) {
    case 32:
        if constexpr (WAVES == 4)
            go(k_gemm<MODE, 32, 4>, 256);
        else
            return hipErrorInvalidValue;  // a 32-row tile has 4 row blocks: 4 waves only
        break;
    case 64: go(k_gemm<MODE, 64, WAVES>, 64 * WAVES); break;
    case 128: go(k_gemm<MODE, 128, WAVES>, 64 * WAVES); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Workgroups per XCD of a routed launch: an XCD's tiles cost at most an
// eighth of the total plus one tile, and each costs at least
// kTileCostBase + 1, which bounds their count.
inline int routed_per_xcd(const GemmArgs &a, int bm) {
    const long T = a.max_tiles, cmax = kTileCostBase + bm / 32, cmin = kTileCostBase + 1;
    return (int)std::min<long>(T, (T * cmax / 8 + cmax) / cmin + 1);
}

template <int MODE>
hipError_t launch_mode(const GemmArgs &a, int bm, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    // 4 waves (one per SIMD), so two workgroups share a CU and one's
    // prologue, epilogue and barriers overlap the other's MFMAs.  Against 8
    // waves (two per SIMD of one workgroup, each staged activation tile
    // serving twice the features) this measured: mid chunk routed gate/up
    // -21%, down -18%, shared expert -30%; full chunk -2% / -5%.
    return launch_waves<MODE, 4>(a, bm, s, e0, e1);
}

}  // namespace

void tile_wait_debug(int *spins, int *extra) {
    *spins = g_wait_spins.load(std::memory_order_relaxed);
    *extra = g_wait_extra.load(std::memory_order_relaxed);
}

hipError_t launch_gateup(const GemmArgs &a, int bm, hipStream_t s) {
    ProfileScope prof(a.order ? MOE_PHASE_GATEUP : MOE_PHASE_SHARED_GU, s, true);
    const hipEvent_t e0 = prof.start(), e1 = prof.stop();
    if (a.order) return launch_mode<GU_GATHER>(a, bm, s, e0, e1);
    return a.ksplit > 1 ? launch_mode<GU_PART>(a, bm, s, e0, e1) : launch_mode<GU_DENSE>(a, bm, s, e0, e1);
}

bool gateup_down_merged(const GemmArgs &a, int bm) {
    return a.order && (bm == 32 || bm == 64 || bm == 128) && !few_row_launch(a.t, a.hidden) &&
           !few_row_launch(a.t, a.inter);
}

hipError_t launch_gateup_down(const GemmArgs &gu, const GemmArgs &dn, int bm, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_EXPERTS, s, true);
    const hipEvent_t e0 = prof.start(), e1 = prof.stop();
    if (!gateup_down_merged(gu, bm)) return hipErrorInvalidValue;
    const int per_xcd = routed_per_xcd(gu, bm);
    const int nblk_gu = (gu.inter + 127) / 128, nblk_dn = (dn.hidden + 255) / 256;
    const int g1 = 8 * per_xcd * nblk_gu, grid = g1 + 8 * per_xcd * nblk_dn;
    GemmArgs d = dn;
    int spins = 0, extra = 0;
    tile_wait_debug(&spins, &extra);
    d.wait_need = nblk_gu + extra;
    d.wait_zero = 0;
    d.wait_spins = spins > 0 ? spins : kTileWaitSpins;
    auto go = [&](auto kernel) {
        if (e0 || e1)
            hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, e0, e1, 0, gu, d, g1);
        else
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, gu, d, g1);
    };
    switch (bm) {
    case 32: go(k_gemm_gu_down<32>); break;
    case 64: go(k_gemm_gu_down<64>); break;
    default: go(k_gemm_gu_down<128>); break;
    }
    return hipGetLastError();
}

hipError_t launch_down(const GemmArgs &a, int bm, hipStream_t s) {
    ProfileScope prof(a.order ? MOE_PHASE_DOWN : MOE_PHASE_SHARED_DOWN, s, true);
    const hipEvent_t e0 = prof.start(), e1 = prof.stop();
    if (a.order) return launch_mode<DOWN_YE>(a, bm, s, e0, e1);
    return a.ksplit > 1 ? launch_mode<DOWN_PART>(a, bm, s, e0, e1) : launch_mode<DOWN_OUT>(a, bm, s, e0, e1);
}

hipError_t launch_reduce_gu(const float *part, int S, int t, int I, uint16_t *hs, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_SHARED_GU, s);
    const int n = t * (I / 4);
    hipLaunchKernelGGL(k_reduce_gu, dim3((n + 255) / 256), dim3(256), 0, s, part, S, t, I, hs);
    return hipGetLastError();
}

hipError_t launch_reduce_down(const float *part, int S, int t, int h, const float *gate, float *out,
                              int accumulate, hipStream_t s) {
    ProfileScope prof(MOE_PHASE_SHARED_DOWN, s);
    const int n = t * (h / 4);
    hipLaunchKernelGGL(k_reduce_down, dim3((n + 255) / 256), dim3(256), 0, s, part, S, t, h, gate, out, accumulate);
    return hipGetLastError();
}

hipError_t launch_shared_gate(const uint16_t *x, const uint16_t *gate_w, int t, int h, float *g,
                              hipStream_t s) {
    hipLaunchKernelGGL(k_shared_gate, dim3((t + 3) / 4), dim3(256), 0, s, x, gate_w, t, h, g);
    return hipGetLastError();
}

hipError_t launch_combine(const uint16_t *ye, const uint32_t *pos, const float *csr_w, int t,
                          int k, int h, float *out, int accumulate, hipStream_t s, const uint16_t *ys,
                          const float *gate) {
    ProfileScope prof(MOE_PHASE_COMBINE, s);
    // few rows: 64-thread workgroups over 512 columns spread one row over
    // h / 512 workgroups; many rows: 256 threads cover 2048 columns.
    if (t < 256) {
        hipLaunchKernelGGL(k_combine<64>, dim3(t, (h + 511) / 512), dim3(64), 0, s, ye, pos, csr_w, t, k, h,
                           out, accumulate, ys, gate);
    } else {
        hipLaunchKernelGGL(k_combine<256>, dim3(t, (h + 2047) / 2048), dim3(256), 0, s, ye, pos, csr_w, t, k, h,
                           out, accumulate, ys, gate);
    }
    return hipGetLastError();
}

}  // namespace moe

extern "C" int moe_debug_tile_wait(int32_t spins, int32_t extra) {
    if (spins < 0 || spins > moe::kTileWaitSpins || extra < 0 || extra > 1) return 1;
    moe::g_wait_spins.store(spins, std::memory_order_relaxed);
    moe::g_wait_extra.store(extra, std::memory_order_relaxed);
    return 0;
}
