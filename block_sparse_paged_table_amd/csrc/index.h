// Resolved arguments of the paged prefill indexer (scores + top-k).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace msa {

constexpr int kIndexMaxPages = 2048;  // pages one top-k row holds in registers

struct IndexArgs {
  int32_t num_seqs, total_q, H, D, page_size, max_pages, num_phys_pages, top_k;
  float scale;                      // q_scale * k_scale (> 0)
  const uint8_t *q;                 // E4M3
  int64_t q_stride_tok, q_stride_head;
  const int32_t *q_seq, *q_pos, *seq_lens;
  const uint8_t *k_cache;           // E4M3
  int64_t kv_stride_page, kv_stride_tok, kv_stride_head;  // bytes
  const int32_t *page_table;
  int64_t pt_stride;
  float *scores;
  int64_t score_stride;
  int32_t *sel_idx;
  uint8_t *sel_mask;
  int64_t sel_stride_tok, sel_stride_head;
  uint32_t *err_flags;              // may be null
};

hipError_t launch_index_scores(const IndexArgs &a, hipStream_t s);
hipError_t launch_index_topk(const IndexArgs &a, hipStream_t s);

}  // namespace msa
