/*
 * moe.h -- C ABI of the routed-expert MoE prefill block for MI355X (gfx950).
 *
 * One block over a chunk of t <= 4096 token rows (the row cap of the
 * cherenkov prefill engine: prefill.rs page, const MAX_PREFILL_ROWS):
 *
 *   1. moe_shared(accumulate = 0)    shared expert over all rows -> out
 *   2. moe_route                     router logits, top-k, renormalised weights
 *   3. moe_build_csr                 rows grouped by expert (CSR)
 *   4. moe_prefill_experts(acc = 1)  per-expert gather, gate/up, SiLU*up, down,
 *                                    weighted add into out
 *
 * This is the order the experts.rs page runs the block in (fn pf_experts:
 * zero the output, shared expert over all rows, then the routed experts one
 * at a time, each scatter-added with its routing weight), so each row sums
 * its terms as shared first, then experts in ascending id.
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless marked [host].  Buffers are owned
 *     by the caller; the library never allocates or frees device memory in
 *     these calls.  Device buffers must stay alive until the stream has
 *     passed the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it, except moe_prefill_experts with
 *     streamed experts, which reads the expert offsets back (one small
 *     device-to-host copy and a stream synchronisation).
 *   - Arguments are validated before anything is enqueued; on any error
 *     nothing runs, outputs are untouched, the status is returned and
 *     moe_last_error() describes it.  Kernel faults are asynchronous and
 *     surface at the caller's next synchronisation.
 *   - bf16 values are passed as uint16_t bit patterns.  Every row of every
 *     matrix argument is contiguous (row-major) and 16-byte aligned.
 *   - Calls are reentrant.  A ring handle serves one call at a time.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_ROWS 4096   /* t <= 4096: prefill.rs page, const MAX_PREFILL_ROWS */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_K 32

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,   /* bad argument (shape, null pointer, alignment) */
    MOE_ERR_CAPACITY = 2,  /* t outside 1..MOE_MAX_ROWS ("empty chunk" / row cap) */
    MOE_ERR_WORKSPACE = 3, /* workspace smaller than moe_workspace_bytes() */
    MOE_ERR_HIP = 4        /* the HIP runtime returned an error */
} moe_status;

/* Message of the last failing call on this thread (empty if none). */
const char *moe_last_error(void);

/*
 * Byte layout of one expert record: six sections (codes and scale/bias of
 * the gate, up and down matrices) in one contiguous record of `stride`
 * bytes, the structure the experts.rs page addresses with per-matrix w/s/b
 * offsets inside a record of `stride` bytes (fn pf_experts, struct Q views
 * at_offset(rec); fn ring_read: record e at e * stride).  gate and up are
 * [inter x hidden], down is [hidden x inter] (rows = outputs).
 *
 * Codes: unsigned 4-bit q, weight = scale * q + bias, one fp16 (scale, bias)
 * pair per `group` consecutive inputs of a row.  Code tiles are 32 rows x 64
 * columns, tile (ob, kb) at byte (ob * (K/64) + kb) * 1024 of the code
 * section; lane L in [0, 64) of a tile owns bytes [16L, 16L+16): row
 * 32*ob + L%32, columns 64*kb + 32*(L/32) + c, c in [0, 32), code c in the
 * little-endian 32-bit word c/8 at bit 4*((c%8)/2) + 16*(c%2).  The
 * scale/bias section holds, per tile in the same order, (64/group)*32
 * entries of 4 bytes (fp16 scale, fp16 bias): entry gi*32 + row%32 for the
 * tile's group gi.  Sections are 256-byte aligned, the stride 4096-byte
 * aligned.  bits is 4 (2 for the miss records of moe_layout_make_bits).
 */
typedef struct {
    int32_t hidden, inter, group, bits;
    uint64_t gate_w, gate_sb, up_w, up_sb, down_w, down_sb; /* byte offsets */
    uint64_t stride;                                        /* record bytes */
} moe_layout;

/*
 * Fills *out [host] for hidden % 256 == 0, inter % 64 == 0, group in {32, 64}.
 * Returns MOE_ERR_INVALID otherwise.  Host only; needs no GPU.
 */
moe_status moe_layout_make(int32_t hidden, int32_t inter, int32_t group, moe_layout *out);

/*
 * The layout of a record with `bits`-wide codes: 4 (as moe_layout_make) or
 * 2, the low-bit form in which streamed experts may cross the host link
 * (experts.rs page, fn prepare_expert_jobs: transient misses take the miss
 * layout of the low-bit store; fn read_expert_batch reads 4-bit and low-bit
 * records into the ring separately).  A 2-bit record has the same sections,
 * scale/bias layout and tile order; its codes are unsigned 0..3
 * (weight = scale * q + bias), a code tile of 32 rows x 64 columns is 512
 * bytes, and lane L of a tile (row 32*ob + L%32, columns
 * 64*kb + 32*(L/32) + c, c in [0, 32)) owns two little-endian 32-bit
 * words, word j at byte 256*j + 4*L, code c in word c/16 at bit
 * 2*((c%16)/2) + 16*(c%2).  Only the ring takes 2-bit layouts
 * (moe_ring_set_miss_layout); the compute calls take 4-bit ones.
 */
moe_status moe_layout_make_bits(int32_t hidden, int32_t inter, int32_t group, int32_t bits, moe_layout *out);

/*
 * Bytes of the one workspace buffer that moe_build_csr, moe_shared and
 * moe_prefill_experts share for t rows, top-k k, E experts, routed layout
 * `routed` [host] and shared layout `shared` [host] (NULL: no shared
 * expert).  The three calls use disjoint parts of it.  Returns 0 for invalid
 * arguments.  Host only.
 */
size_t moe_workspace_bytes(int32_t t, int32_t k, int32_t E, const moe_layout *routed,
                           const moe_layout *shared);

/*
 * Router, top-k and renormalised weights (prefill.rs page, fn pf_layer: the
 * router_b call on the block input `mixed`, writing topk_idx and topk_w for
 * k = num_experts_per_tok; experts.rs page, fn prepare_expert_jobs reads
 * them back as u32 and f32).
 *
 *   x         bf16 [t][h]   block input rows
 *   w_router  fp32 [E][h]   router weight, one row per expert
 *   logits    fp32 [t][E]   output: logit[r][e] in the canonical fp32 order
 *                           (h cut into 4-element chunks, chunk c feeds
 *                           partial c % 64, each partial an fma chain from +0
 *                           in ascending index, then p[l] += p[l+off] for
 *                           off = 32, 16, 8, 4, 2, 1; the logit is p[0])
 *   topk_idx  u32  [t][k]   output: the k largest logits per row, descending,
 *                           ties to the lower expert id
 *   topk_w    fp32 [t][k]   output: exp(l_j - l_max) / sum_selected exp(l - l_max)
 *                           (softmax, top-k, renormalise)
 * Requires 1 <= t <= 4096, h % 256 == 0, 1 <= k <= min(E, 32), E <= 1024.
 */
moe_status moe_route(const uint16_t *x, const float *w_router, int32_t t, int32_t h, int32_t E,
                     int32_t k, float *logits, uint32_t *topk_idx, float *topk_w, void *stream);

/*
 * Rows grouped by expert (experts.rs page, fn prepare_expert_jobs: each
 * expert's rows listed in row order, lists concatenated in expert order;
 * this call builds the same lists on the GPU instead of on the host).
 *
 *   topk_idx, topk_w  [t][k] from moe_route
 *   offsets   u32 [E+1]  output: expert e's segment is [offsets[e], offsets[e+1]);
 *                        offsets[E] = t*k
 *   csr_rows  u32 [t*k]  output: row index of each CSR entry, ascending within a segment
 *   csr_w     fp32 [t*k] output: that entry's routing weight (a copy of topk_w)
 *   csr_pos   u32 [t*k]  output: csr_pos[r*k+j] = CSR index of (r, topk_idx[r][j])
 * Every topk_idx value must be < E, and the k experts of a row distinct
 * (as moe_route produces); other input gives unspecified (in-bounds) output.
 */
moe_status moe_build_csr(const uint32_t *topk_idx, const float *topk_w, int32_t t, int32_t k,
                         int32_t E, uint32_t *offsets, uint32_t *csr_rows, float *csr_w,
                         uint32_t *csr_pos, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Shared expert over all t rows (experts.rs page, fn pf_experts: qmm with
 * the shared gate/up/down matrices over `mixed`, silu_mul, then
 * shared_add_rows into the block output, one row per threadgroup with the
 * shared-gate tensor bound):
 *
 *   out[r] (+)= g_r * W_down (silu(W_gate x_r) * (W_up x_r))
 *
 *   x        bf16 [t][h]
 *   Ls       [host] layout of the shared record (Ls->hidden == h)
 *   record   the shared expert's record (Ls->stride bytes)
 *   gate_w   bf16 [h] or NULL: g_r = sigmoid(x_r . gate_w), or 1 without it
 *   out      fp32 [t][h]; accumulate = 0 overwrites, 1 adds
 */
moe_status moe_shared(const uint16_t *x, int32_t t, const moe_layout *Ls, const void *record,
                      const uint16_t *gate_w, float *out, int32_t accumulate, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Expert ring for records that are not resident in device memory
 * (prefill.rs page, consts RING = 64 slots and GROUP = 8 experts per fetch
 * batch; experts.rs page, fn pf_experts: batch bi's records are copied into
 * ring slots only after the GPU has finished batch bi - RING/GROUP, and the
 * experts of batch bi run only after their copy is done).
 *
 *   L        [host] routed layout (the slot size is L->stride)
 *   slots    device buffer of n_slots * L->stride bytes, owned by the caller
 *   n_slots  ring slots (64 in the pages), group = jobs per batch (8); requires
 *            n_slots >= group >= 1 and n_slots % group == 0
 *   out      [host] receives the handle
 * The handle owns HIP events, a copy stream and pinned host bookkeeping;
 * moe_ring_destroy releases them (after synchronising its copy stream).
 */
typedef struct moe_ring moe_ring;
moe_status moe_ring_create(const moe_layout *L, void *slots, int32_t n_slots, int32_t group,
                           moe_ring **out);
void moe_ring_destroy(moe_ring *ring);

/*
 * Streamed records in the 2-bit miss layout Lmiss [host] (made by
 * moe_layout_make_bits with the ring's hidden, inter and group, bits = 2):
 * from now on moe_prefill_experts copies each streamed expert's host record
 * (Lmiss->stride bytes) into staging slot `slot` and, once the copy is in,
 * expands it on the GPU into the 4-bit record in ring slot `slot` that the
 * GEMMs read.  The expansion is exact (codes 0..3 are 4-bit codes, the
 * scale/bias sections are copied), so results equal those of 4-bit records
 * holding the same codes; only the bytes over the host link shrink
 * (Lmiss->stride vs the ring's stride).  Staging slots follow the ring's
 * reuse rule.
 *   staging  device buffer of n_slots * Lmiss->stride bytes, 16-byte
 *            aligned, owned by the caller; Lmiss = NULL returns to 4-bit
 *            streamed records.
 */
moe_status moe_ring_set_miss_layout(moe_ring *ring, const moe_layout *Lmiss, void *staging);

/* Counters of the last moe_prefill_experts call that used the ring. */
typedef struct {
    int32_t jobs;           /* non-empty experts */
    int32_t streamed;       /* of which streamed through the ring */
    int32_t batches;        /* batches of `group` jobs */
    uint64_t fetched_bytes; /* bytes copied host -> device (streamed * record bytes) */
    double wait_ms;         /* host time blocked in the call: the stream sync of the
                               offsets read-back (slot reuse itself is ordered on
                               the GPU by events, so the host never waits for a slot) */
} moe_ring_stats;
moe_status moe_ring_get_stats(const moe_ring *ring, moe_ring_stats *out);

/*
 * Routed experts (experts.rs page, fn pf_experts: per non-empty expert in
 * ascending id, gather its rows, gate and up projections, silu_mul, down
 * projection, scatter_add_rows with the routing weights):
 *
 *   out[r] (+)= sum over the row's k entries, in ascending expert id, of
 *               csr_w[p] * W_down,e (silu(W_gate,e x_r) * (W_up,e x_r))
 *
 *   x          bf16 [t][h]
 *   L          [host] routed layout (L->hidden == h)
 *   offsets, csr_rows, csr_w, csr_pos   from moe_build_csr
 *   records    u64 [E] device array: device address of expert e's record,
 *              or 0 if expert e is not resident and must be streamed
 *   host_records [host] array of E pinned host pointers (hipHostMalloc or
 *              torch pin_memory) to each streamed expert's record; may be
 *              NULL when every used expert is resident
 *   ring       required when a used expert has records[e] == 0 (without
 *              one, such an expert's entries get unspecified values; its
 *              record is never dereferenced)
 *   out        fp32 [t][h]; accumulate = 0 overwrites, 1 adds
 * Experts with no rows cost nothing and are never read.  The sum over a
 * row's entries is taken in a fixed order, so results are bitwise
 * reproducible and independent of residency.
 */
moe_status moe_prefill_experts(const uint16_t *x, int32_t t, int32_t k, int32_t E,
                               const moe_layout *L, const uint32_t *offsets,
                               const uint32_t *csr_rows, const float *csr_w,
                               const uint32_t *csr_pos, const uint64_t *records,
                               const void *const *host_records, moe_ring *ring, float *out,
                               int32_t accumulate, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * The shared expert and the routed experts in the same grouped launches
 * (experts.rs page, fn pf_experts: the shared expert's qmm/silu_mul over all
 * rows, shared_add_rows, then the routed experts).  The result is that of
 * moe_shared(accumulate) followed by moe_prefill_experts(accumulate = 1) with
 * every expert resident, up to rounding: each row sums, in this order,
 *
 *   out[r] (if accumulate) + g_r * shared(x_r) + the routed terms in ascending
 *   expert id,
 *
 * where the shared expert's down output is rounded to bf16 like a routed
 * one's.  Its t rows are scheduled as one more segment beside the routed
 * experts' rows, so the shared expert streams its weights in the same
 * launches instead of four or two of its own.
 *
 *   x, t, k, E, L, offsets, csr_rows, csr_w, csr_pos, records
 *              as for moe_prefill_experts; every used expert resident
 *              (records[e] != 0 for each expert with rows)
 *   Ls         [host] shared layout; must equal *L in hidden, inter and group
 *   shared_record  the shared expert's record (Ls->stride bytes, 16-byte aligned)
 *   shared_gate_w  bf16 [h] or NULL, as gate_w of moe_shared
 *   out        fp32 [t][h]; accumulate = 0 overwrites, 1 adds
 *   workspace  at least moe_workspace_bytes(t, k, E, L, Ls) bytes
 * Returns MOE_ERR_INVALID for a shared layout other than the routed one, and
 * MOE_ERR_CAPACITY when t*(k+1)*inter*2 or t*h*2 bytes exceed 2^32.
 */
moe_status moe_prefill_fused(const uint16_t *x, int32_t t, int32_t k, int32_t E, const moe_layout *L,
                             const uint32_t *offsets, const uint32_t *csr_rows, const float *csr_w,
                             const uint32_t *csr_pos, const uint64_t *records, const moe_layout *Ls,
                             const void *shared_record, const uint16_t *shared_gate_w, float *out,
                             int32_t accumulate, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The whole block in one call: moe_route, moe_build_csr and
 * moe_prefill_fused (or moe_prefill_experts when Ls is NULL) in this order,
 * on one stream, with the same outputs and the same arithmetic.  Being one
 * call lets it merge launches that the separate calls cannot: for chunks of
 * up to 512 rows the grouping (CSR) and the experts' tile schedule run in
 * one workgroup and one launch, which up to 16 rows also runs the top-k;
 * above 512 rows the scan of the grouping's counts and the schedule share a
 * launch.  Calls on different streams may overlap: the call keeps no state
 * outside its arguments.
 *
 *   x, w_router, t, k, E, logits, topk_idx, topk_w   as for moe_route (h = L->hidden)
 *   offsets, csr_rows, csr_w, csr_pos                outputs, as for moe_build_csr
 *   L, records, Ls, shared_record, shared_gate_w,
 *   out, accumulate                                  as for moe_prefill_fused; Ls may be
 *                                                    NULL (no shared expert)
 *   workspace  at least moe_workspace_bytes(t, k, E, L, Ls) bytes
 * Every used expert must be resident.  Errors as for the separate calls.
 */
moe_status moe_block(const uint16_t *x, const float *w_router, int32_t t, int32_t k, int32_t E,
                     const moe_layout *L, const uint64_t *records, const moe_layout *Ls,
                     const void *shared_record, const uint16_t *shared_gate_w, float *logits,
                     uint32_t *topk_idx, float *topk_w, uint32_t *offsets, uint32_t *csr_rows,
                     float *csr_w, uint32_t *csr_pos, float *out, int32_t accumulate, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Residency by use, on the GPU (experts.rs page, fn prepare_expert_jobs: the
 * non-empty experts sorted by descending row count, ties kept in expert
 * order, and the first `budget` of them kept resident, the rest streamed).
 *
 *   offsets  u32 [E+1] from moe_build_csr
 *   order    u32 [E] output: order[i] = the i-th non-empty expert by use;
 *            0xFFFFFFFF past the last non-empty one
 *   keep     u8 [E] output: 1 for the first min(budget, non-empty) experts
 *            of `order`, else 0
 * Requires 1 <= E <= 1024, budget >= 0.  Enqueues one kernel; nothing is
 * read back.
 */
moe_status moe_residency(const uint32_t *offsets, int32_t E, int32_t budget, uint32_t *order, uint8_t *keep,
                         void *stream);

/*
 * One-block lookahead (decode.rs page, fn lookahead_layer: while a block
 * runs, the next layer's experts are predicted from the current rows, one
 * block ahead only): the next layer's router applied to this block's input
 * x, its top-k, the predicted rows per expert and their residency by use,
 * all on the GPU, so the next block's kept records can be fetched while
 * this one computes.
 *
 *   x, t, h, E, k       as for moe_route; w_router_next fp32 [E][h]: the next
 *                       layer's router
 *   logits, topk_idx, topk_w   outputs as for moe_route (the prediction)
 *   counts   u32 [E] output: predicted rows per expert
 *   order, keep         outputs as for moe_residency, for `budget`
 */
moe_status moe_lookahead(const uint16_t *x, const float *w_router_next, int32_t t, int32_t h, int32_t E,
                         int32_t k, int32_t budget, float *logits, uint32_t *topk_idx, float *topk_w,
                         uint32_t *counts, uint32_t *order, uint8_t *keep, void *stream);

/*
 * Row statistics of a grouped chunk, for the per-chunk report of the
 * prefill.rs page (struct ChunkStats: tokens of the chunk; the records the
 * experts' stage fetched and their bytes, which the ring's moe_ring_stats
 * gives for streamed experts).  Filled on the device from the grouping's
 * offsets, so the report costs no host synchronisation until it is read.
 *
 *   offsets  u32 [E+1] from moe_build_csr (or moe_block)
 *   t        rows of the chunk (copied to tokens)
 *   stats    device memory, 4-byte aligned: the output below
 * Requires 1 <= E <= 1024, t >= 0.  Enqueues one kernel; nothing is read
 * back.
 */
typedef struct {
    uint32_t tokens;          /* t */
    uint32_t assignments;     /* offsets[E] - offsets[0]: rows x experts per row */
    uint32_t experts_touched; /* experts with at least one row */
    uint32_t rows_max;        /* most rows of one expert (0 if none is touched) */
    uint32_t rows_min;        /* fewest rows of a touched expert (0 if none) */
    uint32_t rows_median;     /* lower median of the touched experts' row counts:
                                 the count at 0-based position (n - 1) / 2 of the n
                                 counts sorted ascending (0 if none) */
    uint32_t pad[2];
} moe_chunk_stats;
moe_status moe_chunk_stats_fill(const uint32_t *offsets, int32_t t, int32_t E, moe_chunk_stats *stats,
                                void *stream);

/*
 * The next fused norm: a block's output injected into the residual stream
 * and read back as the next block's input (decode.rs page, fn step_rows: a
 * block's MoE output is "pending" until the next fused norm injects it;
 * prefill.rs page, fn pf_layer: pf_hc_read with the pending output produces
 * the next block input `mixed`, and fn prefill_chunk: pf_inject after the
 * last layer).  The pages show these calls, not their arithmetic; the
 * reading here: a row's residual stream is n fp32 copies of h values, and
 *
 *   copy_i += beta_i * y                          (injection, i = 0..n-1)
 *   z       = sum_i alpha_i * copy_i              (read, ascending i, fp32 fma)
 *   mixed   = bf16(z * gamma / sqrt(mean(z^2) + eps))   (RMS norm, round to
 *                                                        nearest even)
 *
 * with the row's sum of squares reduced in a fixed order (the results are
 * bitwise reproducible).
 *
 *   hyper   fp32 [t][n][h], updated in place (16-byte aligned)
 *   n       1..MOE_MAX_HC residual copies
 *   alpha, beta  [host values] the read and injection weight of each copy
 *   gamma   fp32 [h] norm gain
 *   eps     >= 0
 *   mixed   bf16 [t][h] output (16-byte aligned; must not overlap hyper)
 */
#define MOE_MAX_HC 16
typedef struct {
    float *hyper;
    int32_t n;
    float alpha[MOE_MAX_HC];
    float beta[MOE_MAX_HC];
    const float *gamma;
    float eps;
    uint16_t *mixed;
} moe_next_norm;

/*
 * The next fused norm on its own: y fp32 [t][h] (or NULL: nothing injected,
 * the copies are only read) into nn->hyper, and nn->mixed written.
 * Requires 1 <= t <= 4096, h % 256 == 0, h <= 16384.
 */
moe_status moe_inject_norm(const float *y, int32_t t, int32_t h, const moe_next_norm *nn /*[host]*/,
                           void *stream);

/*
 * moe_block whose block output goes straight into the next fused norm: the
 * combine's last pass forms each row's output in the same order and
 * precision as moe_block (accumulate = 0) and injects it into nn->hyper and
 * normalises into nn->mixed in the same workgroup, so the output is never
 * written to memory and no separate launch reads it back.  The result is
 * bitwise that of moe_block followed by moe_inject_norm on its `out`.
 * Arguments as for moe_block, with `nn` [host] in place of out and
 * accumulate (h = L->hidden <= 16384).
 */
moe_status moe_block_next_norm(const uint16_t *x, const float *w_router, int32_t t, int32_t k, int32_t E,
                               const moe_layout *L, const uint64_t *records, const moe_layout *Ls,
                               const void *shared_record, const uint16_t *shared_gate_w, float *logits,
                               uint32_t *topk_idx, float *topk_w, uint32_t *offsets, uint32_t *csr_rows,
                               float *csr_w, uint32_t *csr_pos, const moe_next_norm *nn, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * A whole MoE sub-layer from the residual stream, in one call (prefill.rs
 * page, fn pf_layer: pf_hc_read(mlp_hc, ..., mix_out) injects the pending
 * attention output into the residual copies and produces the block input
 * `mixed`, which router_b and the experts then read; decode.rs page,
 * fn step_rows: the block's own output stays pending for the next fused
 * norm):
 *
 *   1. in_norm:  pending_y (fp32 [t][h], or NULL) injected into
 *                in_norm->hyper, the copies read and RMS-normalised into
 *                in_norm->mixed (bf16 [t][h]), as moe_inject_norm;
 *   2. the block (moe_block) on x = in_norm->mixed;
 *   3. out_norm: NULL -> the block output is written to out (accumulate as
 *                for moe_block); else it goes into the next fused norm as in
 *                moe_block_next_norm (out and accumulate unused).
 *
 * The result is bitwise that of the separate calls in this order.  in_norm
 * and out_norm may describe the same residual copies (their hyper pointers
 * equal): the block's injection then follows the first read.
 */
moe_status moe_block_from_residual(const float *pending_y, const moe_next_norm *in_norm, const float *w_router,
                                   int32_t t, int32_t k, int32_t E, const moe_layout *L, const uint64_t *records,
                                   const moe_layout *Ls, const void *shared_record, const uint16_t *shared_gate_w,
                                   float *logits, uint32_t *topk_idx, float *topk_w, uint32_t *offsets,
                                   uint32_t *csr_rows, float *csr_w, uint32_t *csr_pos, const moe_next_norm *out_norm,
                                   float *out, int32_t accumulate, void *workspace, size_t workspace_bytes,
                                   void *stream);

/*
 * moe_block without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and arithmetic
 * as moe_block, whose kernels it runs; the scratch they need (the grouping
 * counts, the tile schedule and the hg / ye intermediates) is instead a
 * static device array inside the library of MOE_NOALLOC_SCRATCH_BYTES
 * (64 MiB), one per GPU, held from the library's first use on that GPU until
 * the process ends.  The call allocates and frees nothing (with per-kernel
 * profiling off, its default).
 *
 *   Returns MOE_ERR_CAPACITY, before anything is enqueued, when the chunk
 *   needs more scratch than that: moe_workspace_bytes(t, k, E, L, Ls) must
 *   be <= MOE_NOALLOC_SCRATCH_BYTES (decode-shaped chunks and, at hidden
 *   2048, inter 768, k = 8 with a shared expert, up to about 1200 rows).
 *   No part of the scratch needs to start at zero: each call writes all it
 *   reads, so a call is not affected by what the previous one left there.
 *   All calls on one GPU share its array: calls that overlap on one GPU
 *   (different streams, or different host threads) race and give undefined
 *   results; order them on one stream or with events.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)
moe_status moe_block_noalloc(const uint16_t *x, const float *w_router, int32_t t, int32_t k, int32_t E,
                             const moe_layout *L, const uint64_t *records, const moe_layout *Ls,
                             const void *shared_record, const uint16_t *shared_gate_w, float *logits,
                             uint32_t *topk_idx, float *topk_w, uint32_t *offsets, uint32_t *csr_rows,
                             float *csr_w, uint32_t *csr_pos, float *out, int32_t accumulate, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
