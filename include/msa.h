/*
 * msa.h -- C ABI of libmsa: block-sparse paged prefill attention with
 * per-split partial outputs, and the streaming LSE combine, for AMD MI355X
 * (gfx950).
 *
 * The operation (MiniMax-AI/MSA PR 21, sections "K1" and "Combine"; 1Cat-vLLM
 * PR 387, section "Purpose"):
 *   every query row (token r, query head h) attends only the KV units it
 *   selected -- whole pages, or 4-token microblocks with an exact per-row
 *   bit mask -- gathered through a page table, with the causal rule applied
 *   (a key at position t is visible iff t <= q_pos[r] and t < seq_len).
 *   For each split of its selections it writes one partial output
 *   (normalised by its own softmax sum) and one partial log-sum-exp; the
 *   combine merges a row's partials by their LSEs.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing and never synchronises the host.  Work is
 *     enqueued on `stream` (a hipStream_t; NULL = the legacy default stream).
 *   - Host-checkable errors (null pointers, sizes, strides, alignment,
 *     dtype combinations, workspace size) are detected before anything is
 *     enqueued and returned synchronously; msa_last_error() then describes
 *     the failure for the calling thread.
 *   - Errors that depend on device-resident data (a selected unit outside
 *     the request's page-table row, a page-table entry outside the physical
 *     cache, a query row naming a missing request, a duplicated selection)
 *     never cause an out-of-bounds access: the offending unit contributes
 *     nothing and a bit is set in *err_flags (MSA_ERRF_*).
 *   - Strides are in ELEMENTS unless the name ends in _bytes.
 *   - An empty batch (total_q = 0) is valid: nothing is read or launched
 *     beyond clearing *err_flags, and its buffers may be NULL.
 *   - Calls on different streams with different workspaces may run
 *     concurrently; a workspace must not be shared by calls in flight.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 1

typedef enum {
    MSA_OK = 0,
    MSA_ERR_INVALID_ARG = 1,          /* bad pointer, size, stride or layout */
    MSA_ERR_UNSUPPORTED = 2,          /* valid request this build has no kernel for */
    MSA_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below msa_prefill_workspace_bytes() */
    MSA_ERR_HIP = 4                   /* a HIP runtime call or kernel launch failed */
} msa_status;

typedef enum {
    MSA_F32 = 0,
    MSA_BF16 = 1,
    MSA_F16 = 2,
    MSA_E4M3 = 3,   /* OCP FP8 E4M3 (FN): bias 7, max 448, no infinities */
    MSA_NVFP4 = 4   /* E2M1 codes, two per byte (element 2i in the low nibble),
                       one E4M3 scale per 16 contiguous elements along d */
} msa_dtype;

/* Bits of *err_flags (data errors found on the device). */
#define MSA_ERRF_SEL_RANGE 1u   /* selected unit < 0 or beyond max_pages * page_size */
#define MSA_ERRF_PHYS_RANGE 2u  /* page-table entry outside [0, num_phys_pages) */
#define MSA_ERRF_QSEQ_RANGE 4u  /* q_seq outside [0, num_seqs) */
#define MSA_ERRF_DUPLICATE 8u   /* a (row, KV head) selected a unit twice; the
                                   later slot is ignored */

/*
 * Description of one prefill layer.  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads).  The flat output row of (token r, query
 * head h) is r * num_q_heads + h.
 */
typedef struct msa_prefill_desc {
    uint32_t struct_size;      /* = sizeof(msa_prefill_desc) */

    /* problem */
    int32_t num_seqs;          /* B requests */
    int32_t total_q;           /* query tokens of all requests, concatenated */
    int32_t num_q_heads;       /* Hq */
    int32_t num_kv_heads;      /* Hkv, divides Hq */
    int32_t head_dim_qk;
    int32_t head_dim_v;
    int32_t page_size;         /* tokens per physical page */
    int32_t unit_tokens;       /* tokens per selectable unit: page_size (page
                                  selections) or 4 (microblocks, each with a
                                  4-bit mask) */
    int32_t num_slots;         /* K selections per (token, KV head) */
    int32_t slots_per_split;   /* slots merged into one partial; the number of
                                  partial splits is num_slots / slots_per_split,
                                  split s holding slots [s*spp, (s+1)*spp).
                                  Page selections: 1 (one partial per page).
                                  Microblocks: any divisor of num_slots; below
                                  num_slots this is the split-k form for small
                                  chunks (1Cat-vLLM PR 387, section "Purpose":
                                  the single-row route kept as a
                                  many-partition fallback), every (8-token
                                  group, KV head, split) then being its own
                                  work item.  A unit selected again by a row
                                  in a later slot is ignored there, whichever
                                  split that slot is in. */
    float sm_scale;            /* softmax scale; 0 selects 1/sqrt(head_dim_qk) */
    float q_scale;             /* per-tensor dequant scales (1 for float data): */
    float k_scale;             /*   logit = sm_scale*q_scale*k_scale * (q . k) */
    float v_scale;             /*   value = v_scale * v */

    /* queries: [total_q][Hq][head_dim_qk], d contiguous */
    const void *q;
    int32_t q_dtype;           /* msa_dtype: F32, BF16, F16 or E4M3 */
    int64_t q_stride_tok;
    int64_t q_stride_head;

    /* query rows */
    const int32_t *q_seq;      /* [total_q] request of each token */
    const int32_t *q_pos;      /* [total_q] absolute position; < 0 = padding row
                                  (no visible key, output zero) */
    const int32_t *seq_lens;   /* [num_seqs] KV tokens present, incl. the chunk */

    /* paged KV cache: element (page p, offset o, KV head g, dim d) lives at
     * base + p*kv_stride_page_bytes + o*kv_stride_tok_bytes
     *      + g*kv_stride_head_bytes + bytes(d).  K and V share the strides;
     * separate bases let K/V-interleaved layouts work. */
    const void *k_cache;
    const void *v_cache;
    int32_t kv_dtype;          /* F32 (with Q F32), BF16 (with Q BF16),
                                  F16 (with Q F16), NVFP4 or E4M3 (with Q
                                  E4M3; E4M3 = per-tensor scaled FP8 cache) */
    int64_t kv_stride_page_bytes;
    int64_t kv_stride_tok_bytes;
    int64_t kv_stride_head_bytes;
    /* NVFP4 only: E4M3 scales, [page][tok][head][d/16] by these strides */
    const uint8_t *k_sf;
    const uint8_t *v_sf;
    int64_t sf_stride_page_bytes;
    int64_t sf_stride_tok_bytes;
    int64_t sf_stride_head_bytes;

    /* page table: logical page j of request b is physical page
     * page_table[b * page_table_stride + j], j < max_pages */
    const int32_t *page_table;
    int64_t page_table_stride;
    int32_t max_pages;
    int32_t num_phys_pages;

    /* selections: unit u of slot j of (token r, KV head g) is
     * sel_idx[r*sel_stride_tok + g*sel_stride_head + j], a LOGICAL unit id of
     * the row's request (tokens u*unit_tokens .. +unit_tokens-1).  sel_mask
     * has the same layout: 0 = slot unused; for page units nonzero = used;
     * for microblocks bit i keeps token u*unit_tokens + i.  sel_stride_head
     * may be 0 to share one selection across KV heads. */
    const int32_t *sel_idx;
    const uint8_t *sel_mask;
    int64_t sel_stride_tok;
    int64_t sel_stride_head;

    /* outputs: partial_o[s*po_split_stride + row*po_row_stride + c] (of
     * partial_dtype, c < head_dim_v) and partial_lse[s*pl_split_stride + row]
     * (FP32).  An empty split gets lse = -inf and an unspecified partial_o
     * row.  partial_o must be 16-byte aligned, its strides multiples of 4. */
    void *partial_o;
    int64_t po_split_stride;
    int64_t po_row_stride;
    float *partial_lse;
    int64_t pl_split_stride;
    uint32_t *err_flags;       /* nullable; set (not OR-ed) by the plan step */

    /* Scheduling hint of the page route: work units are ordered by slices of
     * about this many query tokens, so that the queries a slice re-reads (once
     * per selected page) stay in one XCD's L2 while its units run.  0 picks a
     * value from the problem's shape.  Results are bitwise independent of it:
     * every (row, split) partial is computed on its own. */
    int32_t order_slice_tokens;

    /* dtype of partial_o: F32 (0, the default), or BF16 / F16 (rounded to
     * nearest even) to halve the partial bytes; not for F32 queries.  FP16
     * partials need |v_scale * v| < 65504. */
    int32_t partial_dtype;
} msa_prefill_desc;

/* Workspace needed by msa_prefill_plan/_attend for this problem (bytes),
 * so that a caller sizes it up front (MiniMax-AI/MSA PR 21, section "Place
 * the partials by memory locality domain": the workspace object is sized
 * once with a required-bytes query and may serve several layers run in order
 * on one stream).  Depends only on host-side fields; nothing is launched.
 * Returns the descriptor's validation status; *bytes is written on MSA_OK. */
msa_status msa_prefill_workspace_bytes(const msa_prefill_desc *d, size_t *bytes);

/* The same query in the one-value form: the workspace bytes, or 0 when the
 * descriptor is rejected (msa_last_error() then says why). */
size_t msa_sparse_prefill_workspace_bytes(const msa_prefill_desc *d);

/* Step 1: build the work plan in `workspace` from the selections: the
 * inverted index of queries per (request, logical page, KV head) for page
 * selections (MiniMax-AI/MSA PR 21, section "K1": one workgroup per (page,
 * head, query split)), or the per-group unit union, ordered by split, for
 * microblock selections (1Cat-vLLM PR 387, section "Purpose":
 * deterministic planner).
 * Writes lse = -inf for every empty split and sets *err_flags. */
msa_status msa_prefill_plan(const msa_prefill_desc *d, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Step 2: the attention kernel; consumes the plan built by step 1 with the
 * same descriptor and workspace, writes partial_o / partial_lse. */
msa_status msa_prefill_attend(const msa_prefill_desc *d, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Steps 1 + 2. */
msa_status msa_sparse_prefill(const msa_prefill_desc *d, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * msa_sparse_prefill without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The plan lives in a fixed scratch
 * array of msa_noalloc_scratch_bytes() bytes (32 MiB) inside the library:
 * every GPU holds its own copy from the first call on that device until the
 * process ends, and its address is resolved once per device on that first
 * call.  Nothing is allocated per call and the results are the same as
 * msa_sparse_prefill's.
 *   - A problem whose workspace (msa_prefill_workspace_bytes) exceeds the
 *     scratch returns MSA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued
 *     (every page-selection workload up to ~4x a 16K-token, 32-head layer
 *     fits; microblock chunks up to 2048 tokens at 512 slots).
 *   - The scratch keeps the last call's contents; the plan step clears what
 *     it needs (counters, error word) with kernels of its own.
 *   - All calls on one GPU share its scratch: calls that overlap in time on
 *     one GPU (different streams, or threads) race and give wrong results.
 *     Serialise them, or use msa_sparse_prefill with separate workspaces.
 */
msa_status msa_sparse_prefill_noalloc(const msa_prefill_desc *d, void *stream);

/* Size of the fixed scratch of msa_sparse_prefill_noalloc, in bytes. */
size_t msa_noalloc_scratch_bytes(void);

/*
 * LSE combine over a flat list of rows (MiniMax-AI/MSA PR 21, section
 * "Combine"): for each row, M = max_s lse_s; if M = -inf the output row is
 * +0 and lse = -inf; else w_s = exp(lse_s - M),
 * out = sum_s w_s o_s / sum_s w_s, lse = M + ln(sum_s w_s).  FP32 arithmetic.
 *   partial_o   [s*po_split_stride + row*po_row_stride + c]  FP32
 *   partial_lse [s*pl_split_stride + row]                    FP32
 *   out         [row*out_row_stride + c]  out_dtype F32, BF16 or F16 (RNE)
 *   lse         [row]                     FP32, nullable
 * partial_o must be 16-byte aligned with strides that are multiples of 4,
 * out aligned to 4 elements with a row stride that is a multiple of 4, and
 * head_dim_v a multiple of 4 (<= 1024).
 */
msa_status msa_combine(const float *partial_o, int64_t po_split_stride, int64_t po_row_stride,
                       const float *partial_lse, int64_t pl_split_stride,
                       int32_t num_splits, int64_t num_rows, int32_t head_dim_v,
                       void *out, int32_t out_dtype, int64_t out_row_stride,
                       float *lse, void *stream);

/* msa_combine for partial buffers of dtype partial_dtype (F32, BF16 or F16;
 * the pages' K1 keeps BF16/FP16 partials -- MiniMax-AI/MSA PR 21, section
 * "Combine").  Elements are widened to FP32 exactly; same layout rules. */
msa_status msa_combine_ex(const void *partial_o, int32_t partial_dtype, int64_t po_split_stride,
                          int64_t po_row_stride, const float *partial_lse, int64_t pl_split_stride,
                          int32_t num_splits, int64_t num_rows, int32_t head_dim_v,
                          void *out, int32_t out_dtype, int64_t out_row_stride,
                          float *lse, void *stream);

/*
 * Paged prefill indexer (vllm-project/MSA PR 36, sections "Overview",
 * "Changes" and "Wrapper API"): FP8 queries score every page of their
 * request against an FP8 paged cache, one score per (query token, head,
 * logical page), then keep the top_k pages per (token, head) as a selection
 * the attention entry points take (sel_idx / sel_mask layout of
 * msa_prefill_desc, one indexer head per KV head).
 *   score(r, h, j) = q_scale * k_scale * max over the keys t of page j that
 *                    row r sees (t <= q_pos[r], t < seq_len) of q[r,h] . k[t,h]
 *                    (FP32 accumulation of exact E4M3 products); -inf if the
 *                    page has no visible key, for padding rows (q_pos < 0) and
 *                    for pages past the request's table row.
 *   top-k:          the top_k largest finite scores of the row in descending
 *                   order, equal scores by ascending page; slots beyond the
 *                   finite count get sel_idx -1 and sel_mask 0.
 * Data errors (q_seq outside [0, num_seqs), a page-table entry outside the
 * cache for a page with visible keys) give -inf and set *err_flags
 * (MSA_ERRF_QSEQ_RANGE / MSA_ERRF_PHYS_RANGE), cleared by msa_index_scores.
 */
typedef struct msa_index_desc {
    uint32_t struct_size;      /* = sizeof(msa_index_desc) */
    int32_t num_seqs;
    int32_t total_q;
    int32_t num_heads;         /* indexer heads H (query head h reads cache head h) */
    int32_t head_dim;          /* 64 or 128 */
    int32_t page_size;         /* 128 */
    float q_scale;             /* per-tensor E4M3 scales (> 0) */
    float k_scale;
    const void *q;             /* E4M3 [total_q][H][head_dim], d contiguous */
    int64_t q_stride_tok;      /* elements (bytes) */
    int64_t q_stride_head;
    const int32_t *q_seq;      /* [total_q] */
    const int32_t *q_pos;      /* [total_q]; < 0 = padding row */
    const int32_t *seq_lens;   /* [num_seqs] */
    const void *k_cache;       /* E4M3, element (page, offset, head, d) at
                                  p*stride_page + o*stride_tok + h*stride_head + d */
    int64_t kv_stride_page_bytes;
    int64_t kv_stride_tok_bytes;
    int64_t kv_stride_head_bytes;
    const int32_t *page_table; /* [num_seqs][page_table_stride] logical -> physical */
    int64_t page_table_stride;
    int32_t max_pages;         /* <= 2048 */
    int32_t num_phys_pages;
    float *scores;             /* [total_q * H][score_stride], row = token * H + h,
                                  pages 0 .. max_pages-1 written */
    int64_t score_stride;      /* >= max_pages */
    int32_t top_k;             /* 1 .. 255 */
    int32_t *sel_idx;          /* selection out: [r*sel_stride_tok + h*sel_stride_head + s] */
    uint8_t *sel_mask;         /* same layout */
    int64_t sel_stride_tok;
    int64_t sel_stride_head;
    uint32_t *err_flags;       /* nullable */
} msa_index_desc;

/* Page scores only (no top-k). */
msa_status msa_index_scores(const msa_index_desc *d, void *stream);
/* Top-k of the scores already in d->scores. */
msa_status msa_index_topk(const msa_index_desc *d, void *stream);
/* msa_index_scores then msa_index_topk. */
msa_status msa_prefill_index(const msa_index_desc *d, void *stream);

/* Exact NVFP4 dequantisation used by the attention kernel, as a standalone
 * device routine (MiniMax-AI/MSA PR 21, section "Build the prefill for
 * SM107": the product of an E2M1 code and an E4M3 scale, rounded once to
 * E4M3; rounding is to nearest-even with saturation at +-448).
 * out[i] = E4M3 byte of (code codes[i] & 15) x (scale scales[i]), n bytes. */
msa_status msa_nvfp4_dequant_e4m3(const uint8_t *codes, const uint8_t *scales, uint8_t *out,
                                  int64_t n, void *stream);

/* The V-side form of the same dequantisation: the attention's PV product
 * takes the dequantised value as FP16, converted straight from the code and
 * the scale through FP16 tables (section "Build the prefill for SM107": the
 * product is exact in FP16, so the FP16 value equals the E4M3 rounding, and
 * the same bits must come out).
 * out[i] = FP16 bits of E4M3(code codes[i] & 15 x scale scales[i]); n
 * elements, out 2-byte aligned.  Only the low nibble of codes[i] is read.
 * Element i is looked up at position i % 4 of a 4-code word, as the kernel
 * does for the four codes of a 16-bit group. */
msa_status msa_nvfp4_dequant_f16(const uint8_t *codes, const uint8_t *scales, uint16_t *out,
                                 int64_t n, void *stream);

/* Per-device capability query (1Cat-vLLM PR 1236, section "Purpose": the
 * build reports, per device and cached, whether it has a kernel image for
 * the device and enough shared memory for its kernels).  1 iff `device` is a
 * gfx950 GPU whose LDS per workgroup is at least msa_required_lds_bytes(),
 * else 0 (also for a device index that does not exist).  The result is
 * cached per device. */
int msa_device_supported(int device);

/* LDS per workgroup (bytes, static + dynamic) that the largest kernel of
 * this build needs: the FP32 page-route attention at head_dim 128. */
size_t msa_required_lds_bytes(void);

const char *msa_status_str(msa_status s);

/* Detail message of the last failing call on this thread ("" if none). */
const char *msa_last_error(void);

int msa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
