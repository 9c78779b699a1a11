// Internal launch interface between the C ABI layer (api.cpp) and the
// kernels.  Everything here is resolved and validated on the host first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace msa {

constexpr int kMaxChunk = 256;  // entries per work unit (upper bound)

enum Route : int { kRouteF32 = 0, kRouteBF16 = 1, kRouteF16 = 2, kRouteQ8KV4 = 3, kRouteQ8KV8 = 4 };

// Resolved arguments of the page-selection route.
struct PageArgs {
  int32_t num_seqs, total_q, Hq, Hkv, G, D, page_size, num_slots, max_pages, num_phys_pages;
  int32_t chunk;              // entries per work unit
  uint64_t chunk_magic;       // ceil(2^32 / chunk): x / chunk = (x * chunk_magic) >> 32 for x < 2^24
  int32_t slice_rows;         // (token, KV head) rows per ordering slice, multiple of 256
  int32_t lists_per_slice;    // Hkv * num_seqs * max_pages (KV head outermost)
  int32_t route;
  float scale_log2;           // sm_scale * q_scale * k_scale * log2(e)
  float v_scale;
  const void *q;
  int64_t q_stride_tok, q_stride_head;
  const int32_t *q_seq, *q_pos, *seq_lens;
  const uint8_t *k_cache, *v_cache;
  int64_t kv_stride_page, kv_stride_tok, kv_stride_head;   // bytes
  const uint8_t *k_sf, *v_sf;
  int64_t sf_stride_page, sf_stride_tok, sf_stride_head;   // bytes
  const int32_t *page_table;
  int64_t pt_stride;
  const int32_t *sel_idx;
  const uint8_t *sel_mask;
  int64_t sel_stride_tok, sel_stride_head;
  void *partial_o;             // po_dtype elements
  int32_t po_dtype;            // MSA_F32, MSA_BF16 or MSA_F16
  int64_t po_split_stride, po_row_stride;
  float *partial_lse;
  int64_t pl_split_stride;
  uint32_t *err_flags;        // never null here (points into the workspace if the caller passed none)
  // workspace
  uint8_t *ws;
  PageLayout lay;
  int64_t max_units;          // grid bound of the attention kernel
};

hipError_t launch_page_plan(const PageArgs &a, hipStream_t s);
hipError_t launch_page_attend(const PageArgs &a, hipStream_t s);

// Output placement of a combine: row i of the flat row list goes to
// out[i * out_row] and lse[i] (rows_per_split 0), or, with rows_per_split
// R > 0, to out[(i / R) * split + (i % R) * out_row] and
// lse[(i / R) * lse_split + i % R] -- the split slabs of a partial buffer.
struct OutMap {
  int64_t rows_per_split, split, lse_split;
};
hipError_t launch_combine(const void *po, int32_t po_dtype, int64_t po_split, int64_t po_row,
                          const float *pl, int64_t pl_split, int32_t S, int64_t rows, int32_t dv,
                          void *out, int32_t out_dtype, int64_t out_row, float *lse, hipStream_t s,
                          const OutMap &om = OutMap{0, 0, 0});

// Largest LDS (static + dynamic) one workgroup of each kernel family needs.
size_t page_plan_lds_bytes();
size_t page_attend_lds_bytes();
size_t grouped_plan_lds_bytes();
size_t grouped_attend_lds_bytes();
size_t index_lds_bytes();

hipError_t launch_nvfp4_dequant(const uint8_t *codes, const uint8_t *scales, uint8_t *out,
                                int64_t n, hipStream_t s);
hipError_t launch_nvfp4_dequant_f16(const uint8_t *codes, const uint8_t *scales, uint16_t *out,
                                    int64_t n, hipStream_t s);

}  // namespace msa
