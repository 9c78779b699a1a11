/*
 * oracle.c -- plain, slow FP64 CPU oracle for block-sparse paged prefill
 * attention with per-split partial outputs and an LSE combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or constant with the GPU library: every format decoder and
 * every step below is written out here from the definitions.
 *
 * What it computes, and where the pages define it:
 *   - MiniMax-AI/MSA PR 21, section "K1": each query row attends the pages it
 *     selected; only its own page needs the causal mask.
 *   - Same page, section "Combine": the forward writes one partial output and
 *     one partial log-sum-exp per selected page for every (query, head) row;
 *     the combine merges them per row.
 *   - Same page, section "Build the prefill for SM107": an NVFP4 element is an
 *     E2M1 code times an E4M3 block scale, rounded once to E4M3.
 *   - 1Cat-vLLM PR 387, section "Purpose": 4-token microblock selections keep
 *     an exact 4-bit mask per query row; a group of rows that sees nothing
 *     gives bitwise zero (section "Test Result").
 *
 * Readings where the pages are silent (also listed with the design notes):
 *   - sel_idx holds LOGICAL unit ids of the row's request; they are mapped to
 *     physical pages through the page table.
 *   - a key at absolute position t is visible to a query at position p iff
 *     t <= p and t < seq_len of the request (and, for units smaller than a
 *     page, bit (t mod unit) of the slot's mask is set).
 *   - logits use the natural exponential; lse = m + ln(sum exp(s - m)).
 *   - partial outputs are normalised by their own row sum and carry v_scale.
 *   - an empty split has lse = -inf and output 0; a row whose splits are all
 *     empty gives output +0 and lse = -inf.
 *   - a slot repeating an earlier valid unit of the same (row, KV head) is
 *     ignored (first occurrence wins) and flagged.
 *   - E4M3 is the OCP "FN" variant (bias 7, max 448, no infinities); the
 *     rounding to it is round-to-nearest-even with saturation at +-448.
 *
 * parity pins: see the not-gpu tests (codecs exhaustive, dense equivalence,
 * split/combine identity, invariances, closed forms, brute force).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FMT_F64 0
#define ORC_FMT_E4M3 1
#define ORC_FMT_NVFP4 2

#define ORC_ERR_SEL_RANGE 1u   /* selected unit outside the page table row */
#define ORC_ERR_PHYS_RANGE 2u  /* page table entry outside the physical cache */
#define ORC_ERR_QSEQ_RANGE 4u  /* query row names a request that does not exist */
#define ORC_ERR_DUPLICATE 8u   /* a row selected the same unit twice */

/* ---------------------------------------------------------------- formats */

/* OCP E4M3 (FN): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa.  Exponent field 0 is subnormal (m * 2^-9).  0x7F/0xFF are NaN. */
double orc_e4m3_decode(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Nearest finite E4M3 value to x, ties to the code with an even mantissa,
 * keeping the sign of x (so tiny negatives give -0).  Choosing among the
 * finite values only is the same as round-to-nearest-even followed by
 * saturation to +-448.  Brute force over the 127 non-negative finite codes,
 * which increase monotonically with the code. */
uint8_t orc_e4m3_encode(double x)
{
    if (isnan(x))
        return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(orc_e4m3_decode((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent 0 is subnormal: m * 0.5. */
double orc_e2m1_decode(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* NVFP4 element: E2M1 code times its E4M3 block scale, rounded once to
 * E4M3.  The product of the two decoded values is computed exactly in
 * double (small integers times powers of two). */
uint8_t orc_nvfp4_dequant(uint8_t code, uint8_t scale)
{
    return orc_e4m3_encode(orc_e2m1_decode(code) * orc_e4m3_decode(scale));
}

/* ---------------------------------------------------------------- combine */

/* Merge S partial (output, lse) pairs of one row of width dv:
 *   M = max lse;  M = -inf  -> out = 0, lse = -inf;
 *   else w_s = exp(lse_s - M), out = sum w_s o_s / sum w_s,
 *        lse = M + ln(sum w_s).
 * po[s*po_stride + c], pl[s*pl_stride]. */
static void combine_row(int S, int dv, const double *po, int64_t po_stride,
                        const double *pl, int64_t pl_stride, double *out, double *lse)
{
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
        if (pl[s * pl_stride] > M)
            M = pl[s * pl_stride];
    if (M == -INFINITY) {
        for (int c = 0; c < dv; ++c)
            out[c] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double W = 0.0;
    for (int c = 0; c < dv; ++c)
        out[c] = 0.0;
    for (int s = 0; s < S; ++s) {
        double l = pl[s * pl_stride];
        if (l == -INFINITY)
            continue;
        double w = exp(l - M);
        W += w;
        for (int c = 0; c < dv; ++c)
            out[c] += w * po[s * po_stride + c];
    }
    for (int c = 0; c < dv; ++c)
        out[c] /= W;
    *lse = M + log(W);
}

/* Standalone combine over a flat row list:
 * po [S][rows][dv], pl [S][rows] -> out [rows][dv], lse [rows]. */
void orc_combine(int S, int64_t rows, int dv, const double *po, const double *pl,
                 double *out, double *lse)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        combine_row(S, dv, po + r * dv, rows * dv, pl + r, rows, out + r * dv, lse + r);
}

/* ------------------------------------------------------------- attention */

typedef struct {
    /* problem */
    int num_seqs, total_q, Hq, Hkv, d_qk, d_v;
    int page_size, unit_tokens, num_slots, slots_per_split;
    int max_pages, pt_stride, num_phys_pages;
    double sm_scale, q_scale, k_scale, v_scale;
    /* query rows */
    const int32_t *q_seq, *q_pos, *seq_lens, *page_table;
    /* Q: F64 values or E4M3 bytes, [total_q][Hq][d_qk] */
    int q_fmt;
    const void *q;
    /* KV: F64 or E4M3 bytes [P][page][Hkv][d]; NVFP4 codes [P][page][Hkv][d/2]
     * (element 2i in the low nibble) with E4M3 scales [P][page][Hkv][d/16] */
    int kv_fmt;
    const void *k, *v;
    const uint8_t *k_sf, *v_sf;
    /* selections [total_q][Hkv][num_slots] */
    const int32_t *sel_idx;
    const uint8_t *sel_mask;
} orc_problem;

/* 16 x 256 table of NVFP4 element values, built once per call. */
static void build_dequant_table(double tab[16][256])
{
    for (int c = 0; c < 16; ++c)
        for (int s = 0; s < 256; ++s)
            tab[c][s] = orc_e4m3_decode(orc_nvfp4_dequant((uint8_t)c, (uint8_t)s));
}

static double q_value(const orc_problem *p, int tok, int h, int d)
{
    int64_t i = ((int64_t)tok * p->Hq + h) * p->d_qk + d;
    if (p->q_fmt == ORC_FMT_E4M3)
        return orc_e4m3_decode(((const uint8_t *)p->q)[i]);
    return ((const double *)p->q)[i];
}

static double kv_value(const orc_problem *p, const double tab[16][256], int is_v,
                       int phys, int off, int g, int d)
{
    int dim = is_v ? p->d_v : p->d_qk;
    int64_t base = ((int64_t)phys * p->page_size + off) * p->Hkv + g;
    if (p->kv_fmt == ORC_FMT_NVFP4) {
        const uint8_t *codes = (const uint8_t *)(is_v ? p->v : p->k);
        const uint8_t *sf = is_v ? p->v_sf : p->k_sf;
        uint8_t byte = codes[base * (dim / 2) + d / 2];
        uint8_t code = (d & 1) ? (byte >> 4) : (byte & 15);
        uint8_t scale = sf[base * (dim / 16) + d / 16];
        return tab[code][scale];
    }
    if (p->kv_fmt == ORC_FMT_E4M3)      /* per-tensor scaled FP8 cache */
        return orc_e4m3_decode(((const uint8_t *)(is_v ? p->v : p->k))[base * dim + d]);
    return ((const double *)(is_v ? p->v : p->k))[base * dim + d];
}

/* The decoded K or V cache, [P][page][Hkv][dim] doubles: kv_value of every
 * element, computed once per call so that the attention loops read plain
 * values (the same values, so the arithmetic is unchanged).  F64 caches are
 * used in place (*owned = 0). */
static const double *decode_cache(const orc_problem *p, const double tab[16][256], int is_v,
                                  int *owned)
{
    if (p->kv_fmt == ORC_FMT_F64) {
        *owned = 0;
        return (const double *)(is_v ? p->v : p->k);
    }
    int dim = is_v ? p->d_v : p->d_qk;
    int64_t rows = (int64_t)p->num_phys_pages * p->page_size * p->Hkv;
    double *out = (double *)malloc(sizeof(double) * (size_t)(rows * dim));
    if (!out)
        abort();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int g = (int)(r % p->Hkv);
        int off = (int)((r / p->Hkv) % p->page_size);
        int phys = (int)(r / ((int64_t)p->Hkv * p->page_size));
        for (int d = 0; d < dim; ++d)
            out[r * dim + d] = kv_value(p, tab, is_v, phys, off, g, d);
    }
    *owned = 1;
    return out;
}

/* A visible key of one (row, KV head): absolute token position, the slot
 * that selected it, its physical page and offset. */
typedef struct {
    int t, slot, phys, off;
} vis_key;

/* Collect the visible keys of (token r, KV head g), in slot order.  Returns
 * the count; err collects ORC_ERR_* bits. */
static int gather_visible(const orc_problem *p, int r, int g, vis_key *keys, uint32_t *err)
{
    int b = p->q_seq[r], pos = p->q_pos[r];
    if (pos < 0)
        return 0;                       /* padding row: nothing is visible */
    if (b < 0 || b >= p->num_seqs) {
        *err |= ORC_ERR_QSEQ_RANGE;
        return 0;
    }
    int seq_len = p->seq_lens[b];
    int ut = p->unit_tokens;
    int n = 0;
    const int32_t *idx = p->sel_idx + ((int64_t)r * p->Hkv + g) * p->num_slots;
    const uint8_t *msk = p->sel_mask + ((int64_t)r * p->Hkv + g) * p->num_slots;
    for (int j = 0; j < p->num_slots; ++j) {
        if (msk[j] == 0)
            continue;
        int u = idx[j];
        if (u < 0 || (int64_t)(u + 1) * ut > (int64_t)p->max_pages * p->page_size) {
            *err |= ORC_ERR_SEL_RANGE;
            continue;
        }
        int dup = 0;
        for (int jj = 0; jj < j; ++jj)
            if (msk[jj] != 0 && idx[jj] == u)
                dup = 1;
        if (dup) {
            *err |= ORC_ERR_DUPLICATE;
            continue;
        }
        for (int i = 0; i < ut; ++i) {
            int t = u * ut + i;
            int vis = (t <= pos) && (t < seq_len);
            if (ut != p->page_size)
                vis = vis && ((msk[j] >> i) & 1);
            if (!vis)
                continue;
            int phys = p->page_table[(int64_t)b * p->pt_stride + t / p->page_size];
            if (phys < 0 || phys >= p->num_phys_pages) {
                *err |= ORC_ERR_PHYS_RANGE;
                continue;
            }
            keys[n].t = t;
            keys[n].slot = j;
            keys[n].phys = phys;
            keys[n].off = t % p->page_size;
            ++n;
        }
    }
    return n;
}

/* Softmax of the selected keys of `keys` for query (r, h) whose decoded
 * vector is q[d_qk]: writes o[d_v] (normalised, times v_scale) and returns
 * lse, or -inf with o = 0 when the set is empty.  kd / vd are the decoded
 * caches; `s` is scratch for the logits. */
static double softmax_pv(const orc_problem *p, const double *kd, const double *vd, const double *q,
                         int g, const vis_key *keys, const int *sel, int nsel, double *s, double *o)
{
    for (int c = 0; c < p->d_v; ++c)
        o[c] = 0.0;
    if (nsel == 0)
        return -INFINITY;
    double scale = p->sm_scale * p->q_scale * p->k_scale;
    double m = -INFINITY;
    for (int i = 0; i < nsel; ++i) {
        const vis_key *kk = &keys[sel[i]];
        const double *k = kd + (((int64_t)kk->phys * p->page_size + kk->off) * p->Hkv + g) * p->d_qk;
        double dot = 0.0;
        for (int d = 0; d < p->d_qk; ++d)
            dot += q[d] * k[d];
        s[i] = scale * dot;
        if (s[i] > m)
            m = s[i];
    }
    double l = 0.0;
    for (int i = 0; i < nsel; ++i) {
        const vis_key *kk = &keys[sel[i]];
        const double *v = vd + (((int64_t)kk->phys * p->page_size + kk->off) * p->Hkv + g) * p->d_v;
        double e = exp(s[i] - m);
        l += e;
        for (int c = 0; c < p->d_v; ++c)
            o[c] += e * p->v_scale * v[c];
    }
    for (int c = 0; c < p->d_v; ++c)
        o[c] /= l;
    return m + log(l);
}

/*
 * Compute the rows of the requested tokens.
 * Outputs, per requested token index i (0..n_req-1) and query head h:
 *   part_o  [n_req][Hq][S][d_v]   partial outputs of each split
 *   part_lse[n_req][Hq][S]        partial lse (-inf = empty split)
 *   out     [n_req][Hq][d_v], lse [n_req][Hq]   combine of the partials
 *   out1    [n_req][Hq][d_v], lse1[n_req][Hq]   single-pass softmax over the
 *                                               union of all visible keys
 * Any output pointer may be NULL.  Returns the OR of ORC_ERR_* bits seen.
 */
uint32_t orc_prefill_rows(const orc_problem *p, int n_req, const int32_t *row_tokens,
                          double *part_o, double *part_lse, double *out, double *lse,
                          double *out1, double *lse1)
{
    static double tab[16][256];
    if (p->kv_fmt == ORC_FMT_NVFP4)
        build_dequant_table(tab);
    int k_owned, v_owned;
    const double *kd = decode_cache(p, tab, 0, &k_owned);
    const double *vd = decode_cache(p, tab, 1, &v_owned);
    const int S = p->num_slots / p->slots_per_split;
    const int G = p->Hq / p->Hkv;
    const int max_keys = p->num_slots * p->unit_tokens;
    uint32_t err_all = 0;

#pragma omp parallel reduction(| : err_all)
    {
        vis_key *keys = (vis_key *)malloc(sizeof(vis_key) * (size_t)(max_keys + 1));
        int *sel = (int *)malloc(sizeof(int) * (size_t)(max_keys + 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(max_keys + 1));
        double *po = (double *)malloc(sizeof(double) * (size_t)S * p->d_v);
        double *pl = (double *)malloc(sizeof(double) * (size_t)S);
        double *tmp_o = (double *)malloc(sizeof(double) * (size_t)p->d_v);
        double *qrow = (double *)malloc(sizeof(double) * (size_t)p->d_qk);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n_req; ++i) {
            int r = row_tokens[i];
            for (int g = 0; g < p->Hkv; ++g) {
                uint32_t err = 0;
                int n = gather_visible(p, r, g, keys, &err);
                err_all |= err;
                for (int hl = 0; hl < G; ++hl) {
                    int h = g * G + hl;
                    int64_t row = (int64_t)i * p->Hq + h;
                    for (int d = 0; d < p->d_qk; ++d)
                        qrow[d] = q_value(p, r, h, d);
                    /* per split: keys whose slot falls in the split */
                    for (int sp = 0; sp < S; ++sp) {
                        int nsel = 0;
                        for (int k = 0; k < n; ++k)
                            if (keys[k].slot / p->slots_per_split == sp)
                                sel[nsel++] = k;
                        pl[sp] = softmax_pv(p, kd, vd, qrow, g, keys, sel, nsel, s,
                                            po + (int64_t)sp * p->d_v);
                    }
                    if (part_o)
                        memcpy(part_o + row * S * p->d_v, po, sizeof(double) * S * p->d_v);
                    if (part_lse)
                        memcpy(part_lse + row * S, pl, sizeof(double) * S);
                    if (out || lse) {
                        double l0;
                        combine_row(S, p->d_v, po, p->d_v, pl, 1, tmp_o, &l0);
                        if (out)
                            memcpy(out + row * p->d_v, tmp_o, sizeof(double) * p->d_v);
                        if (lse)
                            lse[row] = l0;
                    }
                    if (out1 || lse1) {
                        for (int k = 0; k < n; ++k)
                            sel[k] = k;
                        double l1 = softmax_pv(p, kd, vd, qrow, g, keys, sel, n, s, tmp_o);
                        if (out1)
                            memcpy(out1 + row * p->d_v, tmp_o, sizeof(double) * p->d_v);
                        if (lse1)
                            lse1[row] = l1;
                    }
                }
            }
        }
        free(keys);
        free(sel);
        free(s);
        free(po);
        free(pl);
        free(tmp_o);
        free(qrow);
    }
    if (k_owned)
        free((void *)kd);
    if (v_owned)
        free((void *)vd);
    return err_all;
}

/* Per (token, KV head, slot): 1 if the slot contributes at least one visible
 * key, else 0 (empty).  Used to check which partial slabs must hold -inf. */
void orc_slot_nonempty(const orc_problem *p, uint8_t *nonempty /* [total_q][Hkv][K] */)
{
    const int max_keys = p->num_slots * p->unit_tokens;
#pragma omp parallel
    {
        vis_key *keys = (vis_key *)malloc(sizeof(vis_key) * (size_t)(max_keys + 1));
#pragma omp for schedule(static)
        for (int r = 0; r < p->total_q; ++r)
            for (int g = 0; g < p->Hkv; ++g) {
                uint32_t err = 0;
                int n = gather_visible(p, r, g, keys, &err);
                uint8_t *ne = nonempty + ((int64_t)r * p->Hkv + g) * p->num_slots;
                memset(ne, 0, (size_t)p->num_slots);
                for (int k = 0; k < n; ++k)
                    ne[keys[k].slot] = 1;
            }
        free(keys);
    }
}

/* ------------------------------------------------------- prefill indexer */

/* Page scores of the paged prefill indexer (vllm-project/MSA PR 36, sections
 * "Overview" and "Changes": an FP8-query / FP8-cache scorer whose per-page
 * score is a max taken over the page, written to a per-(query, head) row of
 * pages, followed by a top-k over that row).
 *
 * Readings (the page gives no formula):
 *   - score(r, h, j) = q_scale * k_scale * max over the keys t of logical
 *     page j of request q_seq[r] that are visible to the row (t <= q_pos[r],
 *     t < seq_len) of sum_d q[r,h,d] * k[t,h,d], with q and k the decoded
 *     E4M3 values; -inf when no key of the page is visible, for padding
 *     rows and for pages past the request's table row;
 *   - query head h scores against cache head h (one indexer head per KV
 *     head). */
typedef struct {
    int num_seqs, total_q, H, d, page_size, max_pages, pt_stride, num_phys_pages;
    double q_scale, k_scale;
    const int32_t *q_seq, *q_pos, *seq_lens, *page_table;
    const uint8_t *q;   /* E4M3 [total_q][H][d] */
    const uint8_t *k;   /* E4M3 [phys page][page_size][H][d] */
} orc_index_problem;

/* scores: [total_q][H][max_pages].  Returns ORC_ERR_* bits (QSEQ_RANGE for a
 * row naming a missing request, PHYS_RANGE for a page with visible keys whose
 * table entry is outside the cache; both give -inf). */
uint32_t orc_index_scores(const orc_index_problem *p, double *scores)
{
    uint32_t err_all = 0;
#pragma omp parallel for reduction(| : err_all) schedule(dynamic, 4)
    for (int r = 0; r < p->total_q; ++r) {
        int b = p->q_seq[r], pos = p->q_pos[r];
        int valid = pos >= 0;
        if (valid && (b < 0 || b >= p->num_seqs)) {
            err_all |= ORC_ERR_QSEQ_RANGE;
            valid = 0;
        }
        for (int h = 0; h < p->H; ++h) {
            double *row = scores + ((int64_t)r * p->H + h) * p->max_pages;
            for (int j = 0; j < p->max_pages; ++j) {
                row[j] = -INFINITY;
                if (!valid)
                    continue;
                int seq_len = p->seq_lens[b];
                int t0 = j * p->page_size;
                int t1 = t0 + p->page_size - 1;     /* last key of the page */
                if (t1 > pos) t1 = pos;
                if (t1 > seq_len - 1) t1 = seq_len - 1;
                if (t1 < t0)
                    continue;                       /* nothing visible */
                int phys = p->page_table[(int64_t)b * p->pt_stride + j];
                if (phys < 0 || phys >= p->num_phys_pages) {
                    err_all |= ORC_ERR_PHYS_RANGE;
                    continue;
                }
                double best = -INFINITY;
                for (int t = t0; t <= t1; ++t) {
                    const uint8_t *kk = p->k + (((int64_t)phys * p->page_size + (t - t0)) * p->H + h) * p->d;
                    const uint8_t *qq = p->q + ((int64_t)r * p->H + h) * p->d;
                    double dot = 0.0;
                    for (int d = 0; d < p->d; ++d)
                        dot += orc_e4m3_decode(qq[d]) * orc_e4m3_decode(kk[d]);
                    if (dot > best)
                        best = dot;
                }
                row[j] = p->q_scale * p->k_scale * best;
            }
        }
    }
    return err_all;
}

/* Top-k of each of `rows` rows of n scores (reading: the K largest finite
 * scores in descending order, equal scores by ascending page index; slots
 * beyond the finite count get index -1 and mask 0). */
void orc_topk_rows(int64_t rows, int n, const double *scores, int K, int32_t *idx, uint8_t *mask)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *row = scores + r * n;
        int32_t *oi = idx + r * K;
        uint8_t *om = mask + r * K;
        for (int s = 0; s < K; ++s) {
            int best = -1;
            for (int j = 0; j < n; ++j) {
                if (!(row[j] > -INFINITY))
                    continue;
                int taken = 0;
                for (int q = 0; q < s; ++q)
                    taken |= (oi[q] == j);
                if (taken)
                    continue;
                if (best < 0 || row[j] > row[best])
                    best = j;                       /* strict: the lower index keeps a tie */
            }
            oi[s] = best;
            om[s] = best >= 0;
        }
    }
}

int orc_abi_version(void) { return 1; }

/* Array forms of the format routines, for the tests. */
void orc_e4m3_decode_n(const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_decode(in[i]);
}

void orc_e4m3_encode_n(const double *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(in[i]);
}

void orc_e2m1_decode_n(const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e2m1_decode(in[i]);
}

void orc_nvfp4_dequant_n(const uint8_t *codes, const uint8_t *scales, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_nvfp4_dequant(codes[i], scales[i]);
}
