/*
 * Plain CPU oracle for the routed-expert MoE prefill block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * links, loads or calls it, and this file includes none of the GPU
 * library's headers: the two implementations share no code.
 *
 * What is computed, and where it is described (cherenkov source pages):
 *   - router logits and top-k with renormalised weights: prefill.rs page,
 *     fn pf_layer (the router_b call producing topk_idx / topk_w), and the
 *     experts.rs page, fn prepare_expert_jobs (topk_idx read as u32,
 *     topk_w as f32);
 *   - the grouping of rows by expert: experts.rs page, fn
 *     prepare_expert_jobs (per-expert row lists filled row by row, then
 *     concatenated in expert order, empty experts skipped);
 *   - per-expert FFN (gather, gate/up, SiLU(gate)*up, down, scatter-add with
 *     the routing weight): prefill.rs page, module doc, and experts.rs page,
 *     fn pf_experts (gather_rows, expert_qmm_from, silu_mul,
 *     scatter_add_rows);
 *   - the shared expert over all rows, added into a zeroed output before the
 *     routed experts: experts.rs page, fn pf_experts (zero, qmm x3,
 *     silu_mul, shared_add_rows);
 *   - residency of the most-used experts: experts.rs page, fn
 *     prepare_expert_jobs (stable sort by descending row count, first
 *     `budget` kept).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *   - Router arithmetic (canonical fp32 order).  logit[r,e] is fp32.  The
 *     hidden dimension is cut into chunks of 4 consecutive elements; chunk c
 *     belongs to partial sum l = c mod 64.  Each of the 64 partials starts
 *     at +0 and accumulates fmaf(x_i, W[e,i], p) over its elements in
 *     ascending i.  Then for off = 32, 16, 8, 4, 2, 1: p[l] = p[l] + p[l+off]
 *     for l < off.  The logit is p[0].  Requires h % 256 == 0.
 *   - Top-k order: logits descending, ties to the lower expert id.
 *     Weights: exp(l_j - l_max) / sum over the selected of exp(l - l_max)
 *     (softmax, then top-k, then renormalise), in double, rounded to float.
 *   - int4 code: unsigned q in 0..15, W = scale * q + bias, per group of G
 *     along the input dimension; record layout as stated in orc_layout.
 *   - Low-bit records of streamed experts (experts.rs page,
 *     prepare_expert_jobs: transient misses take the miss layout of the
 *     low-bit store; read_expert_batch keeps 4-bit and other reads apart):
 *     the same affine group code with 2-bit q in 0..3, layout in
 *     orc_layout_bits and orc_dequant2.
 *   - Combine order: shared expert first, then experts in ascending id.
 *   - Shared gate: none (factor 1) or sigmoid(x_r . gate_w).
 *   - Injection into the next fused norm (orc_inject_norm): the residual
 *     stream of a row is n fp32 copies of h values; the block output y is
 *     added to copy i with weight beta_i, the copies are read back as
 *     z = sum_i alpha_i copy_i, and the next block's input is the RMS norm
 *     of z times a gain gamma, rounded to bf16.
 *
 * All floating-point accumulation here is double, except the router logits,
 * which follow the fp32 order above exactly (this file must be compiled
 * without fast-math and with -ffp-contract=off).  Every parallel loop gives
 * each output to one thread, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD 1

/* ------------------------------------------------------------------ formats */

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* IEEE binary16 -> double, written out from the format's definition. */
static double f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);               /* subnormal: man * 2^-24 */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), exp - 25); /* (1 + man/1024) * 2^(exp-15) */
    return sign ? -v : v;
}

static uint64_t align_up(uint64_t n, uint64_t a) { return (n + a - 1) / a * a; }

/*
 * Record layout: sections gate codes, gate scale/bias, up codes, up
 * scale/bias, down codes, down scale/bias, each padded to 256 bytes, stride
 * padded to 4096.  gate and up are [inter x hidden], down is [hidden x inter]
 * (rows = outputs), the shapes the experts.rs page gives its Q views in
 * pf_experts.  out = {gate_w, gate_sb, up_w, up_sb, down_w, down_sb, stride}.
 */
int orc_layout_bits(int hidden, int inter, int group, int bits, uint64_t out[7])
{
    if (!(group == 32 || group == 64) || hidden <= 0 || inter <= 0 || hidden % 64 || inter % 64)
        return ORC_BAD;
    if (bits != 4 && bits != 2)
        return ORC_BAD;
    uint64_t codes = (uint64_t)hidden * inter * bits / 8;
    uint64_t sb = (uint64_t)hidden * inter / group * 4;
    uint64_t off = 0;
    for (int m = 0; m < 3; m++) {
        out[2 * m] = off;
        off = align_up(off + codes, 256);
        out[2 * m + 1] = off;
        off = align_up(off + sb, 256);
    }
    out[6] = align_up(off, 4096);
    return ORC_OK;
}

int orc_layout(int hidden, int inter, int group, uint64_t out[7])
{
    return orc_layout_bits(hidden, inter, group, 4, out);
}

/*
 * Decode matrix [N x K] from its code section `w` and scale/bias section `sb`.
 * Code tiles are 32 rows x 64 columns, tile (ob, kb) at (ob*(K/64)+kb)*1024
 * bytes; in a tile, lane L owns 16 bytes at 16*L for row 32*ob + L%32 and
 * columns 64*kb + 32*(L/32) + c, c in [0,32); code c is in little-endian word
 * c/8 at bit 4*((c%8)/2) + 16*(c%2).  Scale/bias entries (fp16 pair, scale
 * first) are per tile, (64/G)*32 of them, entry gi*32 + row%32 for group gi
 * of the tile.  W[n,k] = scale*q + bias (exact in double).
 */
void orc_dequant(const uint8_t *w, const uint8_t *sb, int N, int K, int G, double *W)
{
    int kt = K / 64, per_tile = 64 / G;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        int ob = n / 32, r = n % 32;
        for (int k = 0; k < K; k++) {
            int kb = k / 64, half = (k % 64) / 32, c = k % 32;
            uint64_t tile = (uint64_t)ob * kt + kb;
            int lane = r + 32 * half;
            const uint8_t *wp = w + tile * 1024 + 16 * lane + 4 * (c / 8);
            uint32_t word = (uint32_t)wp[0] | ((uint32_t)wp[1] << 8) | ((uint32_t)wp[2] << 16) |
                            ((uint32_t)wp[3] << 24);
            int bit = 4 * ((c % 8) / 2) + 16 * (c % 2);
            int q = (word >> bit) & 15;
            int gi = (k % 64) / G;
            const uint8_t *ep = sb + (tile * per_tile * 32 + (uint64_t)gi * 32 + r) * 4;
            double s = f16_to_double((uint16_t)(ep[0] | (ep[1] << 8)));
            double b = f16_to_double((uint16_t)(ep[2] | (ep[3] << 8)));
            W[(uint64_t)n * K + k] = s * q + b;
        }
    }
}

/*
 * Decode a matrix [N x K] stored with 2-bit codes (the low-bit records of
 * streamed experts).  Code tiles are 32 rows x 64 columns of 512 bytes, tile
 * (ob, kb) at (ob*(K/64)+kb)*512; lane L of a tile (row 32*ob + L%32,
 * columns 64*kb + 32*(L/32) + c, c in [0,32)) owns two little-endian 32-bit
 * words, word j at byte 256*j + 4*L; code c is in word c/16 at bit
 * 2*((c%16)/2) + 16*(c%2).  Scale/bias entries exactly as for 4-bit codes.
 * W[n,k] = scale*q + bias with q in 0..3.
 */
void orc_dequant2(const uint8_t *w, const uint8_t *sb, int N, int K, int G, double *W)
{
    int kt = K / 64, per_tile = 64 / G;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        int ob = n / 32, r = n % 32;
        for (int k = 0; k < K; k++) {
            int kb = k / 64, half = (k % 64) / 32, c = k % 32;
            uint64_t tile = (uint64_t)ob * kt + kb;
            int lane = r + 32 * half;
            const uint8_t *wp = w + tile * 512 + 256 * (c / 16) + 4 * lane;
            uint32_t word = (uint32_t)wp[0] | ((uint32_t)wp[1] << 8) | ((uint32_t)wp[2] << 16) |
                            ((uint32_t)wp[3] << 24);
            int c16 = c % 16;
            int bit = 2 * (c16 / 2) + 16 * (c16 % 2);
            int q = (word >> bit) & 3;
            int gi = (k % 64) / G;
            const uint8_t *ep = sb + (tile * per_tile * 32 + (uint64_t)gi * 32 + r) * 4;
            double s = f16_to_double((uint16_t)(ep[0] | (ep[1] << 8)));
            double b = f16_to_double((uint16_t)(ep[2] | (ep[3] << 8)));
            W[(uint64_t)n * K + k] = s * q + b;
        }
    }
}

/* Decode with the code width of the record (4 or 2 bits). */
static void dequant_bits(const uint8_t *w, const uint8_t *sb, int N, int K, int G, int bits, double *W)
{
    if (bits == 2)
        orc_dequant2(w, sb, N, K, G, W);
    else
        orc_dequant(w, sb, N, K, G, W);
}

/* ------------------------------------------------------------------ router */

/* One logit in the canonical fp32 order stated in the header. */
static float canonical_dot(const uint16_t *x, const float *w, int h)
{
    float p[64];
    for (int l = 0; l < 64; l++)
        p[l] = 0.0f;
    for (int i = 0; i < h; i++) {
        int l = (i / 4) % 64;
        p[l] = fmaf(bf16_to_float(x[i]), w[i], p[l]);
    }
    for (int off = 32; off >= 1; off /= 2)
        for (int l = 0; l < off; l++)
            p[l] = p[l] + p[l + off];
    return p[0];
}

/* logits[t x E] = x[t x h] . Wr[E x h]^T in the canonical order. */
int orc_router_logits(const uint16_t *x, const float *Wr, int t, int h, int E, float *logits)
{
    if (h % 256)
        return ORC_BAD;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < t; r++)
        for (int e = 0; e < E; e++)
            logits[(uint64_t)r * E + e] = canonical_dot(x + (uint64_t)r * h, Wr + (uint64_t)e * h, h);
    return ORC_OK;
}

/* a ranks before b: larger logit first, ties to the lower id (-0 == +0). */
static int ranks_before(float la, int a, float lb, int b)
{
    if (la > lb)
        return 1;
    if (la < lb)
        return 0;
    return a < b;
}

/*
 * Per row: the k largest logits in rank order, and their softmax weights
 * renormalised over the selection (equal to softmax over all E, then top-k,
 * then dividing by the selected mass).
 */
int orc_topk(const float *logits, int t, int E, int k, uint32_t *idx, float *wts)
{
    if (k < 1 || k > E)
        return ORC_BAD;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int r = 0; r < t; r++) {
        const float *l = logits + (uint64_t)r * E;
        unsigned char *taken = calloc((size_t)E, 1);
        for (int e = 0; e < E; e++)
            if (!isfinite(l[e]))
                bad = 1;
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best))
                    best = e;
            }
            taken[best] = 1;
            idx[(uint64_t)r * k + j] = (uint32_t)best;
        }
        free(taken);
        double lmax = l[idx[(uint64_t)r * k]];
        double sum = 0.0;
        for (int j = 0; j < k; j++)
            sum += exp((double)l[idx[(uint64_t)r * k + j]] - lmax);
        for (int j = 0; j < k; j++)
            wts[(uint64_t)r * k + j] = (float)(exp((double)l[idx[(uint64_t)r * k + j]] - lmax) / sum);
    }
    return bad ? ORC_BAD : ORC_OK;
}

/* ------------------------------------------------------------------ grouping */

/*
 * Rows grouped by expert: each expert's list gets (r, w) for r ascending and
 * j ascending, and the lists are concatenated in expert order.  offsets[e] is
 * the start of expert e's segment (offsets[E] = t*k); pos[r*k+j] is the CSR
 * index of the pair (r, idx[r*k+j]).
 */
int orc_build_csr(const uint32_t *idx, const float *wts, int t, int k, int E,
                  uint32_t *offsets, uint32_t *rows, float *csr_w, uint32_t *pos)
{
    uint32_t *count = calloc((size_t)E, sizeof(uint32_t));
    uint32_t *fill = calloc((size_t)E, sizeof(uint32_t));
    int rc = ORC_OK;
    for (uint64_t i = 0; i < (uint64_t)t * k; i++) {
        if (idx[i] >= (uint32_t)E) {
            rc = ORC_BAD;
            goto done;
        }
        count[idx[i]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + count[e];
    for (int r = 0; r < t; r++)
        for (int j = 0; j < k; j++) {
            uint32_t e = idx[(uint64_t)r * k + j];
            uint32_t p = offsets[e] + fill[e]++;
            rows[p] = (uint32_t)r;
            csr_w[p] = wts[(uint64_t)r * k + j];
            pos[(uint64_t)r * k + j] = p;
        }
done:
    free(count);
    free(fill);
    return rc;
}

/*
 * Residency: non-empty experts ordered by descending row count, stable in
 * expert id; the first n_keep are marked resident (keep[e] = 1).  order
 * (may be NULL) receives that order, 0xFFFFFFFF past the last non-empty
 * expert.
 */
void orc_residency_order(const uint32_t *offsets, int E, int n_keep, uint8_t *keep, uint32_t *order_out)
{
    int *order = malloc(sizeof(int) * (size_t)E);
    int n = 0;
    for (int e = 0; e < E; e++) {
        keep[e] = 0;
        if (offsets[e + 1] > offsets[e])
            order[n++] = e;
    }
    /* insertion sort: stable */
    for (int i = 1; i < n; i++) {
        int v = order[i];
        uint32_t cv = offsets[v + 1] - offsets[v];
        int j = i - 1;
        while (j >= 0 && offsets[order[j] + 1] - offsets[order[j]] < cv) {
            order[j + 1] = order[j];
            j--;
        }
        order[j + 1] = v;
    }
    for (int i = 0; i < n && i < n_keep; i++)
        keep[order[i]] = 1;
    if (order_out)
        for (int i = 0; i < E; i++)
            order_out[i] = i < n ? (uint32_t)order[i] : 0xffffffffu;
    free(order);
}

void orc_residency(const uint32_t *offsets, int E, int n_keep, uint8_t *keep)
{
    orc_residency_order(offsets, E, n_keep, keep, NULL);
}

/* ------------------------------------------------------------------ expert FFN */

typedef struct {
    double *g, *u, *d; /* gate [I x h], up [I x h], down [h x I] */
    int h, I;
} ffn_weights;

/* Decode one record whose codes are `bits` wide (its layout from orc_layout_bits). */
static int ffn_decode_bits(const uint8_t *rec, int h, int I, int G, int bits, ffn_weights *f)
{
    uint64_t lay[7];
    if (orc_layout_bits(h, I, G, bits, lay))
        return ORC_BAD;
    f->h = h;
    f->I = I;
    f->g = malloc(sizeof(double) * (size_t)h * I);
    f->u = malloc(sizeof(double) * (size_t)h * I);
    f->d = malloc(sizeof(double) * (size_t)h * I);
    if (!f->g || !f->u || !f->d)
        return ORC_BAD;
    dequant_bits(rec + lay[0], rec + lay[1], I, h, G, bits, f->g);
    dequant_bits(rec + lay[2], rec + lay[3], I, h, G, bits, f->u);
    dequant_bits(rec + lay[4], rec + lay[5], h, I, G, bits, f->d);
    return ORC_OK;
}

static int ffn_decode(const uint8_t *rec, const uint64_t lay[7], int h, int I, int G, ffn_weights *f)
{
    (void)lay;
    return ffn_decode_bits(rec, h, I, G, 4, f);
}

static void ffn_free(ffn_weights *f)
{
    free(f->g);
    free(f->u);
    free(f->d);
}

/* y[h] = W_d (silu(W_g x) * (W_u x)) for one row x[h] (bf16), all in double. */
static void ffn_row(const ffn_weights *f, const uint16_t *x, double *y)
{
    int h = f->h, I = f->I;
    double *xd = malloc(sizeof(double) * (size_t)h);
    double *a = malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < h; i++)
        xd[i] = bf16_to_double(x[i]);
    for (int o = 0; o < I; o++) {
        double g = 0.0, u = 0.0;
        const double *wg = f->g + (uint64_t)o * h, *wu = f->u + (uint64_t)o * h;
        for (int i = 0; i < h; i++) {
            g += wg[i] * xd[i];
            u += wu[i] * xd[i];
        }
        a[o] = g / (1.0 + exp(-g)) * u;
    }
    for (int n = 0; n < h; n++) {
        double s = 0.0;
        const double *wd = f->d + (uint64_t)n * I;
        for (int o = 0; o < I; o++)
            s += wd[o] * a[o];
        y[n] = s;
    }
    free(xd);
    free(a);
}

/* Gate factor of the shared expert: 1 without a gate, else sigmoid(x . gate_w). */
static double shared_gate(const uint16_t *x, const uint16_t *gate_w, int h)
{
    if (!gate_w)
        return 1.0;
    double z = 0.0;
    for (int i = 0; i < h; i++)
        z += bf16_to_double(x[i]) * bf16_to_double(gate_w[i]);
    return 1.0 / (1.0 + exp(-z));
}

/*
 * FFN of one expert over a list of rows: y[n x h] for x rows rows[0..n).
 * Exposed so tests can check the expert maths on its own.
 */
int orc_expert_rows(const uint8_t *rec, int h, int I, int G, const uint16_t *x,
                    const uint32_t *rows, int n, double *y)
{
    uint64_t lay[7];
    ffn_weights f;
    if (orc_layout(h, I, G, lay) || ffn_decode(rec, lay, h, I, G, &f))
        return ORC_BAD;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; i++)
        ffn_row(&f, x + (uint64_t)rows[i] * h, y + (uint64_t)i * h);
    ffn_free(&f);
    return ORC_OK;
}

/* Shared expert over all t rows with its gate factor: ys[t x h] in double. */
int orc_shared(const uint8_t *rec, int h, int Is, int G, const uint16_t *x, int t,
               const uint16_t *gate_w, double *ys)
{
    uint64_t lay[7];
    ffn_weights f;
    if (orc_layout(h, Is, G, lay) || ffn_decode(rec, lay, h, Is, G, &f))
        return ORC_BAD;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < t; r++) {
        double *y = ys + (uint64_t)r * h;
        ffn_row(&f, x + (uint64_t)r * h, y);
        double g = shared_gate(x + (uint64_t)r * h, gate_w, h);
        for (int n = 0; n < h; n++)
            y[n] *= g;
    }
    ffn_free(&f);
    return ORC_OK;
}

/* ------------------------------------------------------------------ the block */

/*
 * The whole block through the grouped (CSR) path, as the pages run it: the
 * shared expert into the zeroed output, then each non-empty expert in
 * ascending id, its rows gathered, run through the FFN and added back with
 * their routing weights.  records[e] points at expert e's record.  out is
 * [t x h] float (the double sum rounded once); the routing outputs are
 * returned too.  shared_rec may be NULL (no shared expert).
 */
int orc_block(const uint16_t *x, const float *Wr, int t, int h, int I, int Is, int E, int k, int G,
              const uint8_t *const *records, const uint8_t *rec_bits, const uint8_t *shared_rec,
              const uint16_t *gate_w, float *out, uint32_t *idx, float *wts, uint32_t *offsets,
              uint32_t *rows, float *csr_w, uint32_t *pos)
{
    uint64_t lay[7];
    if (t < 1 || orc_layout(h, I, G, lay))
        return ORC_BAD;
    float *logits = malloc(sizeof(float) * (size_t)t * E);
    double *acc = calloc((size_t)t * h, sizeof(double));
    int rc = orc_router_logits(x, Wr, t, h, E, logits);
    if (!rc)
        rc = orc_topk(logits, t, E, k, idx, wts);
    if (!rc)
        rc = orc_build_csr(idx, wts, t, k, E, offsets, rows, csr_w, pos);
    if (!rc && shared_rec)
        rc = orc_shared(shared_rec, h, Is, G, x, t, gate_w, acc);
    for (int e = 0; e < E && !rc; e++) {
        int n = (int)(offsets[e + 1] - offsets[e]);
        if (n == 0)
            continue;
        ffn_weights f;
        if (ffn_decode_bits(records[e], h, I, G, rec_bits ? rec_bits[e] : 4, &f)) {
            rc = ORC_BAD;
            break;
        }
        /* rows inside one expert's segment are distinct: no two threads touch one row */
#pragma omp parallel for schedule(dynamic, 1)
        for (int i = 0; i < n; i++) {
            uint32_t p = offsets[e] + (uint32_t)i;
            double *y = malloc(sizeof(double) * (size_t)h);
            ffn_row(&f, x + (uint64_t)rows[p] * h, y);
            double *o = acc + (uint64_t)rows[p] * h;
            for (int c = 0; c < h; c++)
                o[c] += (double)csr_w[p] * y[c];
            free(y);
        }
        ffn_free(&f);
    }
    if (!rc)
        for (uint64_t i = 0; i < (uint64_t)t * h; i++)
            out[i] = (float)acc[i];
    free(logits);
    free(acc);
    return rc;
}

/*
 * Brute force per token, without any grouping: for each sample row, its own
 * logits, top-k and weights, then out = g*shared(x) + sum_j w_j * FFN_{e_j}(x)
 * in double.  order = 0 sums the k terms in ascending expert id (the order
 * the grouped path adds them), order = 1 in top-k slot order.  Each needed
 * expert is decoded once.  out_rows is [ns x h] double.
 */
int orc_tokens_bruteforce(const uint16_t *x, const float *Wr, int t, int h, int I, int Is, int E, int k,
                          int G, const uint8_t *const *records, const uint8_t *rec_bits,
                          const uint8_t *shared_rec, const uint16_t *gate_w, const int *sample, int ns,
                          int order, double *out_rows)
{
    uint64_t lay[7];
    if (orc_layout(h, I, G, lay) || k < 1 || k > E)
        return ORC_BAD;
    uint32_t *sidx = malloc(sizeof(uint32_t) * (size_t)ns * k);
    float *sw = malloc(sizeof(float) * (size_t)ns * k);
    float *lg = malloc(sizeof(float) * (size_t)E);
    double *terms = calloc((size_t)ns * k * h, sizeof(double));
    int rc = ORC_OK;
    for (int s = 0; s < ns && !rc; s++) {
        if (sample[s] < 0 || sample[s] >= t) {
            rc = ORC_BAD;
            break;
        }
        rc = orc_router_logits(x + (uint64_t)sample[s] * h, Wr, 1, h, E, lg);
        if (!rc)
            rc = orc_topk(lg, 1, E, k, sidx + (uint64_t)s * k, sw + (uint64_t)s * k);
    }
    for (int e = 0; e < E && !rc; e++) {
        int used = 0;
        for (int i = 0; i < ns * k; i++)
            used |= sidx[i] == (uint32_t)e;
        if (!used)
            continue;
        ffn_weights f;
        if (ffn_decode_bits(records[e], h, I, G, rec_bits ? rec_bits[e] : 4, &f)) {
            rc = ORC_BAD;
            break;
        }
#pragma omp parallel for schedule(dynamic, 1)
        for (int i = 0; i < ns * k; i++)
            if (sidx[i] == (uint32_t)e)
                ffn_row(&f, x + (uint64_t)sample[i / k] * h, terms + (uint64_t)i * h);
        ffn_free(&f);
    }
    if (!rc) {
        double *ys = NULL;
        if (shared_rec) {
            ffn_weights f;
            uint64_t ls[7];
            if (orc_layout(h, Is, G, ls) || ffn_decode(shared_rec, ls, h, Is, G, &f))
                rc = ORC_BAD;
            else {
                ys = calloc((size_t)ns * h, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
                for (int s = 0; s < ns; s++)
                    ffn_row(&f, x + (uint64_t)sample[s] * h, ys + (uint64_t)s * h);
                ffn_free(&f);
            }
        }
        for (int s = 0; s < ns && !rc; s++) {
            double *o = out_rows + (uint64_t)s * h;
            double g = shared_gate(x + (uint64_t)sample[s] * h, gate_w, h);
            for (int c = 0; c < h; c++)
                o[c] = ys ? g * ys[(uint64_t)s * h + c] : 0.0;
            int *slot = malloc(sizeof(int) * (size_t)k);
            for (int j = 0; j < k; j++)
                slot[j] = j;
            if (order == 0) /* ascending expert id */
                for (int a = 1; a < k; a++)
                    for (int b = a; b > 0 && sidx[(uint64_t)s * k + slot[b]] < sidx[(uint64_t)s * k + slot[b - 1]]; b--) {
                        int tmp = slot[b];
                        slot[b] = slot[b - 1];
                        slot[b - 1] = tmp;
                    }
            for (int jj = 0; jj < k; jj++) {
                int j = slot[jj];
                const double *y = terms + ((uint64_t)s * k + j) * h;
                for (int c = 0; c < h; c++)
                    o[c] += (double)sw[(uint64_t)s * k + j] * y[c];
            }
            free(slot);
        }
        free(ys);
    }
    free(sidx);
    free(sw);
    free(lg);
    free(terms);
    return rc;
}

/* ------------------------------------------------------------------ next norm */

/*
 * Round a double to the nearest bfloat16 (ties to even), returned as its bit
 * pattern: 8 significant bits for normal values, a fixed quantum of 2^-133
 * below 2^-126 (the format's subnormals), infinity past the largest finite
 * value.  Done in one step from the double, so no intermediate float
 * rounding can move a value across a tie.
 */
uint16_t orc_round_bf16(double v)
{
    if (isnan(v))
        return 0x7fc0;
    int sign = signbit(v) ? 1 : 0;
    double a = fabs(v), r;
    if (a == 0.0)
        return (uint16_t)(sign << 15);
    if (a < ldexp(1.0, -126)) {
        r = ldexp(nearbyint(ldexp(a, 133)), -133); /* default mode: ties to even */
    } else {
        int e;
        double m = frexp(a, &e);                       /* a = m 2^e, m in [0.5, 1) */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);      /* 8 significant bits */
    }
    float f = (float)r;                                /* exact: r has <= 8 bits */
    if (r >= ldexp(1.0, 128))
        f = INFINITY;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u >> 16) | (uint32_t)(sign << 15));
}

/*
 * The block output y [t x h] injected into the residual stream and read by
 * the next fused norm (decode.rs page, step_rows: a block's MoE output is
 * injected by the next fused norm, `pending`; prefill.rs page, pf_layer and
 * prefill_chunk: pf_hc_read with the pending output, pf_inject).  The pages
 * show the calls, not their arithmetic; the reading taken here:
 *
 *   hyper[r][i][c] += beta[i] * y[r][c]                 for the n copies i
 *   z[r][c]         = sum_i alpha[i] * hyper[r][i][c]   (after the update)
 *   mixed[r][c]     = bf16( z[r][c] * gamma[c] / sqrt(mean_c z[r][c]^2 + eps) )
 *
 * hyper is fp32 [t][n][h]; hyper_out receives the updated copies (rounded to
 * float once from double); mixed is bf16 [t][h].  y may be NULL (nothing
 * injected: the plain read).  All arithmetic in double.
 */
int orc_inject_norm(const float *hyper, const float *y, int t, int n, int h, const float *alpha,
                    const float *beta, const float *gamma, double eps, float *hyper_out, uint16_t *mixed)
{
    if (t < 1 || n < 1 || h < 1 || eps < 0.0)
        return ORC_BAD;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < t; r++) {
        double *z = calloc((size_t)h, sizeof(double));
        for (int i = 0; i < n; i++) {
            const float *hp = hyper + ((uint64_t)r * n + i) * h;
            float *op = hyper_out + ((uint64_t)r * n + i) * h;
            for (int c = 0; c < h; c++) {
                double v = (double)hp[c];
                if (y)
                    v += (double)beta[i] * (double)y[(uint64_t)r * h + c];
                op[c] = (float)v;
                z[c] += (double)alpha[i] * v;
            }
        }
        double ss = 0.0;
        for (int c = 0; c < h; c++)
            ss += z[c] * z[c];
        double inv = 1.0 / sqrt(ss / h + eps);
        for (int c = 0; c < h; c++)
            mixed[(uint64_t)r * h + c] = orc_round_bf16(z[c] * inv * (double)gamma[c]);
        free(z);
    }
    return ORC_OK;
}

/* Threads the parallel loops use from now on (the results do not depend on it). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
