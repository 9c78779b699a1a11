// Internal interface of the grouped microblock route (planner + attention).
#pragma once

#include "common.h"

namespace msa {

constexpr int kGroupTokens = 8;        // adjacent query tokens per group
constexpr int kGPlanThreads = 256;       // planner workgroup, many groups
constexpr int kGPlanThreadsFew = 1024;  // planner workgroup when groups are few

// Workspace of the grouped route.  Per (KV head, group): a list of up to
// list_cap 8-byte entries {physical page << 5 | unit index in the page,
// mask32 (4 visible-token bits per token of the group)}, ordered by split
// and, within a split, by unit; and the num_splits + 1 offsets of the
// splits' runs in it (split s owns entries [split_off[s], split_off[s + 1])).
// `stage` is the planner's own scratch (16 bytes per candidate unit).
// With H > 1 sub-splits, `sub_po` / `sub_pl` hold the FP32 partials and LSEs
// of the runs of each split ([split][row][run][d] and [run][split][row]),
// which a combine then merges into the split's partials.
struct GroupLayout {
  size_t meta, split_off, stage, lists, sub_po, sub_pl, total;
};

__host__ inline GroupLayout group_layout(int64_t num_lists, int64_t list_cap, int64_t num_splits,
                                         int64_t sub_rows = 0, int64_t sub_dv = 0) {
  GroupLayout L;
  size_t off = 0;
  L.meta = off;   off = align_up(off + 64 * 4, 256);
  L.split_off = off; off = align_up(off + (size_t)num_lists * (num_splits + 1) * 4, 256);
  L.stage = off;  off = align_up(off + (size_t)num_lists * list_cap * 16, 256);
  // (16 bytes of slack: the attention kernel loads entries in 16-byte pairs,
  // so the last entry of a list may bring its successor along)
  L.lists = off;  off = align_up(off + (size_t)num_lists * list_cap * 8 + 16, 256);
  // sub_rows = splits x H x rows partial rows of sub_dv FP32 values each
  L.sub_po = off; off = align_up(off + (size_t)sub_rows * sub_dv * 4, 256);
  L.sub_pl = off; off = align_up(off + (size_t)sub_rows * 4, 256);
  L.total = off;
  return L;
}

struct GroupArgs {
  int32_t num_seqs, total_q, Hq, Hkv, G, D, page_size, unit_tokens, num_slots, max_pages,
      num_phys_pages;
  int32_t num_groups;  // ceil(total_q / kGroupTokens)
  int32_t plan_threads;  // kGPlanThreads, or kGPlanThreadsFew when at most one planner
                         // workgroup per CU is launched (latency over throughput)
  int32_t sort_n;      // power of two >= kGroupTokens * num_slots and >= plan_threads
  int32_t list_cap;    // kGroupTokens * num_slots
  int32_t num_splits, slots_per_split;  // split s merges slots [s * spp, (s + 1) * spp)
  int32_t sub_splits;  // H: runs each split's list is cut into (1: none)
  float scale_log2, v_scale;
  const void *q;
  int64_t q_stride_tok, q_stride_head;
  const int32_t *q_seq, *q_pos, *seq_lens;
  const uint8_t *k_cache, *v_cache;
  int64_t kv_stride_page, kv_stride_tok, kv_stride_head;  // bytes
  const int32_t *page_table;
  int64_t pt_stride;
  const int32_t *sel_idx;
  const uint8_t *sel_mask;
  int64_t sel_stride_tok, sel_stride_head;
  void *partial_o;             // po_dtype elements
  int32_t po_dtype;            // MSA_F32, MSA_BF16 or MSA_F16
  int64_t po_split_stride, po_row_stride;  // elements
  float *partial_lse;
  int64_t pl_split_stride;
  int64_t po_sub_stride, pl_sub_stride;  // run hh of a split: + hh times these (H > 1)
  uint32_t *err_flags;
  uint8_t *ws;
  GroupLayout lay;
};

hipError_t launch_grouped_plan(const GroupArgs &a, hipStream_t s);
hipError_t launch_grouped_attend(const GroupArgs &a, hipStream_t s);

}  // namespace msa
