// C ABI of libmsa: host-side validation, workspace sizing and kernel
// launches.  Nothing here allocates device memory or waits on the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "grouped.h"
#include "launch.h"
#include "index.h"

using namespace msa;

namespace {

thread_local char g_err[512] = "";

msa_status fail(msa_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

msa_status ok() {
  g_err[0] = '\0';
  return MSA_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int esize(int dt) {
  switch (dt) {
    case MSA_F32: return 4;
    case MSA_BF16: return 2;
    case MSA_F16: return 2;
    case MSA_E4M3: return 1;
    default: return 0;
  }
}

constexpr int kPageRouteRowsPerUnit = 1024;  // (token, head) rows per work unit (at most)
constexpr int kPageRouteMinRows = 64;         // rows per unit never cut below one 16-row tile per wave
constexpr int64_t kPageRouteMinUnits = 512;   // two units per compute unit before units shrink
constexpr int kMaxDevices = 64;               // devices the per-device caches cover

// Route of a descriptor (page selections), or -1.
int page_route(const msa_prefill_desc *d) {
  if (d->q_dtype == MSA_F32 && d->kv_dtype == MSA_F32) return kRouteF32;
  if (d->q_dtype == MSA_BF16 && d->kv_dtype == MSA_BF16) return kRouteBF16;
  if (d->q_dtype == MSA_F16 && d->kv_dtype == MSA_F16) return kRouteF16;
  if (d->q_dtype == MSA_E4M3 && d->kv_dtype == MSA_NVFP4) return kRouteQ8KV4;
  if (d->q_dtype == MSA_E4M3 && d->kv_dtype == MSA_E4M3) return kRouteQ8KV8;
  return -1;
}

constexpr int kMaxSubSplits = 16;            // runs per split of the grouped route (at most)
constexpr int64_t kSubSplitMaxItems = 512;   // workgroups the runs may fill (two per CU)
constexpr int kMinRunSlots = 8;              // slots of a split per run (at least)

// Workspace layout of a resolved grouped problem, and the strides of its
// runs' partials when sub_splits > 1 ([split][row][run][d], [run][split][row]).
void set_grouped_layout(GroupArgs *a) {
  const int H = a->sub_splits;
  const int64_t rows_all = (int64_t)a->total_q * a->Hq;
  const int64_t sub_rows = H > 1 ? (int64_t)a->num_splits * H * rows_all : 0;
  a->lay = group_layout((int64_t)a->num_groups * a->Hkv, a->list_cap, a->num_splits, sub_rows, a->D);
  a->po_sub_stride = H > 1 ? a->D : 0;
  a->pl_sub_stride = H > 1 ? (int64_t)a->num_splits * rows_all : 0;
}

// Grouped microblock route (4-token units with per-row bit masks).  With
// slots_per_split < num_slots it is the split-k form: every (group, KV head,
// split) is a work item of its own and writes that split's partials.
msa_status resolve_grouped(const msa_prefill_desc *d, GroupArgs *a) {
  if (d->unit_tokens != 4 || d->page_size % 4)
    return fail(MSA_ERR_UNSUPPORTED, "microblock route needs unit_tokens 4 and page_size %% 4 == 0");
  if (d->num_slots > 512) return fail(MSA_ERR_UNSUPPORTED, "microblock route: at most 512 slots");
  if (d->q_dtype != MSA_F16 || d->kv_dtype != MSA_F16)
    return fail(MSA_ERR_UNSUPPORTED, "microblock route is built for FP16 Q and KV");
  if (d->head_dim_qk != d->head_dim_v || (d->head_dim_qk != 128 && d->head_dim_qk != 256))
    return fail(MSA_ERR_UNSUPPORTED, "microblock route needs head_dim 128 or 256 (qk == v)");
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G > 8) return fail(MSA_ERR_UNSUPPORTED, "microblock route: at most 8 query heads per KV head");
  if (d->num_seqs >= (1 << 16) || (int64_t)d->max_pages * d->page_size / 4 >= (1ll << 24))
    return fail(MSA_ERR_UNSUPPORTED, "microblock route: too many requests or units");
  if (d->page_size > 128 || d->num_phys_pages >= (1 << 27))
    return fail(MSA_ERR_UNSUPPORTED, "microblock route: page_size <= 128 and fewer than 2^27 pages");
  if (!aligned(d->q, 16) || (d->q_stride_tok * 2) % 16 || (d->q_stride_head * 2) % 16 ||
      d->q_stride_head < 0 || d->q_stride_tok < 0)
    return fail(MSA_ERR_INVALID_ARG, "q must be 16-byte aligned with 16-byte aligned strides");
  if (!aligned(d->k_cache, 16) || !aligned(d->v_cache, 16) || d->kv_stride_page_bytes % 16 ||
      d->kv_stride_tok_bytes % 16 || d->kv_stride_head_bytes % 16)
    return fail(MSA_ERR_INVALID_ARG, "k/v cache and strides must be 16-byte aligned");
  if (!aligned(d->partial_o, 16) || d->po_row_stride % 4 || d->po_split_stride % 4 ||
      d->po_row_stride < d->head_dim_v)
    return fail(MSA_ERR_INVALID_ARG, "partial_o must be 16-byte aligned, row stride >= head_dim_v");
  if (!aligned(d->partial_lse, 4)) return fail(MSA_ERR_INVALID_ARG, "partial_lse misaligned");
  GroupArgs &r = *a;
  memset(&r, 0, sizeof(r));
  r.num_seqs = d->num_seqs;
  r.total_q = d->total_q;
  r.Hq = d->num_q_heads;
  r.Hkv = d->num_kv_heads;
  r.G = G;
  r.D = d->head_dim_qk;
  r.page_size = d->page_size;
  r.unit_tokens = d->unit_tokens;
  r.num_slots = d->num_slots;
  r.max_pages = d->max_pages;
  r.num_phys_pages = d->num_phys_pages;
  r.num_groups = (d->total_q + kGroupTokens - 1) / kGroupTokens;
  r.list_cap = kGroupTokens * d->num_slots;
  r.slots_per_split = d->slots_per_split;
  r.num_splits = d->num_slots / d->slots_per_split;
  // few groups: one wide planner workgroup per CU finishes sooner; many:
  // narrow workgroups keep every CU busy
  r.plan_threads = (int64_t)r.num_groups * r.Hkv <= 256 ? kGPlanThreadsFew : kGPlanThreads;
  r.sort_n = r.plan_threads;
  while (r.sort_n < r.list_cap) r.sort_n <<= 1;
  const float sm = d->sm_scale > 0.0f ? d->sm_scale : 1.0f / std::sqrt((float)d->head_dim_qk);
  r.scale_log2 = (float)((double)sm * d->q_scale * d->k_scale * 1.4426950408889634);
  r.v_scale = d->v_scale;
  r.q = d->q;
  r.q_stride_tok = d->q_stride_tok;
  r.q_stride_head = d->q_stride_head;
  r.q_seq = d->q_seq;
  r.q_pos = d->q_pos;
  r.seq_lens = d->seq_lens;
  r.k_cache = (const uint8_t *)d->k_cache;
  r.v_cache = (const uint8_t *)d->v_cache;
  r.kv_stride_page = d->kv_stride_page_bytes;
  r.kv_stride_tok = d->kv_stride_tok_bytes;
  r.kv_stride_head = d->kv_stride_head_bytes;
  r.page_table = d->page_table;
  r.pt_stride = d->page_table_stride;
  r.sel_idx = d->sel_idx;
  r.sel_mask = d->sel_mask;
  r.sel_stride_tok = d->sel_stride_tok;
  r.sel_stride_head = d->sel_stride_head;
  r.partial_o = d->partial_o;
  r.po_dtype = d->partial_dtype;
  r.po_split_stride = d->po_split_stride;
  r.po_row_stride = d->po_row_stride;
  r.partial_lse = d->partial_lse;
  r.pl_split_stride = d->pl_split_stride;
  // Runs: a grid of few (group, KV head, split) work items leaves most CUs
  // idle (two attention workgroups fit one).  Each split's list is then cut
  // into H runs, each its own workgroup writing FP32 partials of its run into
  // the workspace, and a combine merges a split's runs into the split's
  // partials.  H doubles while the grid stays within 512 workgroups and a run
  // keeps at least 8 slots' worth of the split; the runs' partials stay below
  // 24 MiB.  (Split-k small chunk, 16 splits of 32 slots: attention plus
  // merge 42 -> 32 us with 2 runs, 28 us with 4, 36 us with 8; with 32
  // splits of 16 slots 2 runs cost 3 us more than they gained.)
  const int64_t items = (int64_t)(r.num_groups + 7) / 8 * 8 * r.Hkv * r.num_splits;
  const int64_t rows_all = (int64_t)r.total_q * r.Hq;
  r.sub_splits = 1;
  if (items * 4 <= kSubSplitMaxItems) {
    while (r.sub_splits < kMaxSubSplits && items * r.sub_splits * 2 <= kSubSplitMaxItems &&
           r.slots_per_split / (r.sub_splits * 2) >= kMinRunSlots &&
           (int64_t)r.num_splits * r.sub_splits * 2 * rows_all * (r.D + 1) * 4 <= (24ll << 20))
      r.sub_splits *= 2;
  }
  set_grouped_layout(&r);
  return MSA_OK;
}

// Host checks shared by every prefill entry point.  On success fills the
// resolved arguments of the route (without workspace pointers).
msa_status check_desc(const msa_prefill_desc *d, PageArgs *a, GroupArgs *ga, bool *grouped) {
  if (!d) return fail(MSA_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->struct_size != sizeof(msa_prefill_desc))
    return fail(MSA_ERR_INVALID_ARG, "struct_size %u != %zu (ABI mismatch)", d->struct_size,
                sizeof(msa_prefill_desc));
  if (d->num_seqs < 1 || d->total_q < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(MSA_ERR_INVALID_ARG, "bad sizes: num_seqs %d total_q %d Hq %d Hkv %d", d->num_seqs,
                d->total_q, d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads)
    return fail(MSA_ERR_INVALID_ARG, "num_q_heads %d not a multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_slots < 1 || d->slots_per_split < 1 || d->num_slots % d->slots_per_split)
    return fail(MSA_ERR_INVALID_ARG, "num_slots %d must be a positive multiple of slots_per_split %d",
                d->num_slots, d->slots_per_split);
  if (d->page_size < 1 || d->unit_tokens < 1 || d->max_pages < 1 || d->num_phys_pages < 1)
    return fail(MSA_ERR_INVALID_ARG, "bad page geometry");
  if (d->page_table_stride < d->max_pages)
    return fail(MSA_ERR_INVALID_ARG, "page_table_stride %lld < max_pages %d",
                (long long)d->page_table_stride, d->max_pages);
  if (!(d->sm_scale >= 0.0f) || !std::isfinite(d->sm_scale) || !(d->q_scale > 0.0f) ||
      !std::isfinite(d->q_scale) || !(d->k_scale > 0.0f) || !std::isfinite(d->k_scale) ||
      !std::isfinite(d->v_scale))
    return fail(MSA_ERR_INVALID_ARG, "scales must be finite, sm_scale >= 0, q_scale and k_scale > 0");
  if (d->head_dim_qk < 1 || d->head_dim_v < 1)
    return fail(MSA_ERR_INVALID_ARG, "bad head dims");
  if (d->partial_dtype != MSA_F32 && d->partial_dtype != MSA_BF16 && d->partial_dtype != MSA_F16)
    return fail(MSA_ERR_INVALID_ARG, "partial_dtype must be F32, BF16 or F16");
  const void *need[] = {d->q, d->q_seq, d->q_pos, d->seq_lens, d->k_cache, d->v_cache,
                        d->page_table, d->sel_idx, d->sel_mask, d->partial_o, d->partial_lse};
  const char *names[] = {"q", "q_seq", "q_pos", "seq_lens", "k_cache", "v_cache",
                         "page_table", "sel_idx", "sel_mask", "partial_o", "partial_lse"};
  for (int i = 0; i < 11 && d->total_q > 0; ++i)  // an empty batch reads nothing
    if (!need[i]) return fail(MSA_ERR_INVALID_ARG, "%s is NULL", names[i]);
  if (d->sel_stride_tok < d->num_slots || d->sel_stride_head < 0)
    return fail(MSA_ERR_INVALID_ARG, "selection strides too small");
  if ((int64_t)d->total_q * d->num_kv_heads * d->num_slots >= (1ll << 31) ||
      (int64_t)d->total_q * d->num_q_heads >= (1ll << 31) || d->total_q >= (1 << 23))
    return fail(MSA_ERR_UNSUPPORTED, "problem too large for 32-bit plan indices");

  // ---- microblock selections take the grouped route
  if (d->unit_tokens != d->page_size) {
    *grouped = true;
    return resolve_grouped(d, ga);
  }
  *grouped = false;
  const int route = page_route(d);
  if (route < 0)
    return fail(MSA_ERR_UNSUPPORTED, "dtype pair q %d / kv %d unsupported", d->q_dtype, d->kv_dtype);
  if (d->page_size != 128)
    return fail(MSA_ERR_UNSUPPORTED, "page route is built for page_size 128 (got %d)", d->page_size);
  if (d->head_dim_qk != d->head_dim_v)
    return fail(MSA_ERR_UNSUPPORTED, "page route needs head_dim_qk == head_dim_v");
  const int D = d->head_dim_qk;
  if (!((D == 64 || D == 128) && (route != kRouteQ8KV4 || D == 128)))
    return fail(MSA_ERR_UNSUPPORTED, "head_dim %d unsupported for this dtype", D);
  if (d->slots_per_split != 1)
    return fail(MSA_ERR_UNSUPPORTED, "page route writes one partial per slot (slots_per_split 1)");
  if (route == kRouteF32 && d->partial_dtype != MSA_F32)
    return fail(MSA_ERR_UNSUPPORTED, "FP32 queries take FP32 partials");
  if (d->num_slots > 255)
    return fail(MSA_ERR_UNSUPPORTED, "at most 255 slots");

  // ---- alignment of vector accesses
  const int qb = esize(d->q_dtype);
  if (!aligned(d->q, 16) || (d->q_stride_tok * qb) % 16 || (d->q_stride_head * qb) % 16 ||
      d->q_stride_head < 0 || d->q_stride_tok < 0)
    return fail(MSA_ERR_INVALID_ARG, "q must be 16-byte aligned with 16-byte aligned strides");
  if (!aligned(d->k_cache, 16) || !aligned(d->v_cache, 16) || d->kv_stride_page_bytes % 16 ||
      d->kv_stride_tok_bytes % 16 || d->kv_stride_head_bytes % 16)
    return fail(MSA_ERR_INVALID_ARG, "k/v cache and strides must be 16-byte aligned");
  if (route == kRouteQ8KV4) {
    if (!d->k_sf || !d->v_sf) return fail(MSA_ERR_INVALID_ARG, "NVFP4 scales are NULL");
    if (!aligned(d->k_sf, 8) || !aligned(d->v_sf, 8) || d->sf_stride_page_bytes % 8 ||
        d->sf_stride_tok_bytes % 8 || d->sf_stride_head_bytes % 8)
      return fail(MSA_ERR_INVALID_ARG, "NVFP4 scale arrays and strides must be 8-byte aligned");
  }
  if (!aligned(d->partial_o, 16) || d->po_row_stride % 4 || d->po_split_stride % 4 ||
      d->po_row_stride < d->head_dim_v)
    return fail(MSA_ERR_INVALID_ARG, "partial_o must be 16-byte aligned, row stride >= head_dim_v");
  if (!aligned(d->partial_lse, 4)) return fail(MSA_ERR_INVALID_ARG, "partial_lse misaligned");

  PageArgs &r = *a;
  memset(&r, 0, sizeof(r));
  r.num_seqs = d->num_seqs;
  r.total_q = d->total_q;
  r.Hq = d->num_q_heads;
  r.Hkv = d->num_kv_heads;
  r.G = d->num_q_heads / d->num_kv_heads;
  r.D = D;
  r.page_size = d->page_size;
  r.num_slots = d->num_slots;
  r.max_pages = d->max_pages;
  r.num_phys_pages = d->num_phys_pages;
  r.chunk = std::min(kMaxChunk, (kPageRouteRowsPerUnit + r.G - 1) / r.G);
  r.route = route;
  const float sm = d->sm_scale > 0.0f ? d->sm_scale : 1.0f / std::sqrt((float)d->head_dim_qk);
  r.scale_log2 = (float)((double)sm * d->q_scale * d->k_scale * 1.4426950408889634);
  r.v_scale = d->v_scale;
  r.q = d->q;
  r.q_stride_tok = d->q_stride_tok;
  r.q_stride_head = d->q_stride_head;
  r.q_seq = d->q_seq;
  r.q_pos = d->q_pos;
  r.seq_lens = d->seq_lens;
  r.k_cache = (const uint8_t *)d->k_cache;
  r.v_cache = (const uint8_t *)d->v_cache;
  r.kv_stride_page = d->kv_stride_page_bytes;
  r.kv_stride_tok = d->kv_stride_tok_bytes;
  r.kv_stride_head = d->kv_stride_head_bytes;
  r.k_sf = d->k_sf;
  r.v_sf = d->v_sf;
  r.sf_stride_page = d->sf_stride_page_bytes;
  r.sf_stride_tok = d->sf_stride_tok_bytes;
  r.sf_stride_head = d->sf_stride_head_bytes;
  r.page_table = d->page_table;
  r.pt_stride = d->page_table_stride;
  r.sel_idx = d->sel_idx;
  r.sel_mask = d->sel_mask;
  r.sel_stride_tok = d->sel_stride_tok;
  r.sel_stride_head = d->sel_stride_head;
  r.partial_o = d->partial_o;
  r.po_dtype = d->partial_dtype;
  r.po_split_stride = d->po_split_stride;
  r.po_row_stride = d->po_row_stride;
  r.partial_lse = d->partial_lse;
  r.pl_split_stride = d->pl_split_stride;
  const int64_t L = (int64_t)d->num_seqs * d->max_pages * d->num_kv_heads;
  const int64_t NS = (int64_t)d->total_q * d->num_kv_heads * d->num_slots;
  if (L >= (1ll << 24)) return fail(MSA_ERR_UNSUPPORTED, "too many page lists");
  // Small problems: with 1024-row units a few thousand selections make a
  // handful of workgroups, each walking its rows one tile per wave at a time.
  // Shrink the units toward two per compute unit (each still reads its page
  // once); large problems keep the 1024-row units, which amortise the page
  // load best.
  if (NS < kPageRouteMinUnits * r.chunk) {
    const int floor_e = std::min<int>(r.chunk, (kPageRouteMinRows + r.G - 1) / r.G);
    r.chunk = (int32_t)std::max<int64_t>(floor_e, (NS + kPageRouteMinUnits - 1) / kPageRouteMinUnits);
  }
  r.chunk_magic = ((1ull << 32) + (uint64_t)r.chunk - 1) / (uint64_t)r.chunk;
  if (d->order_slice_tokens < 0) return fail(MSA_ERR_INVALID_ARG, "order_slice_tokens < 0");

  // Ordering slices: the plan keeps one list per (slice, KV head, request,
  // logical page), so units come out slice by slice (one KV head after the
  // other) and the workgroups in flight at one time read the queries of one
  // slice and head group only.  Automatic
  // size: none while all queries fit in 16 MiB (their re-reads then hit the
  // caches anyway); else ~512 KiB of queries per slice, but enough tokens
  // that an average page list of a slice still fills one unit.
  const int64_t rows = (int64_t)d->total_q * d->num_kv_heads;  // (token, KV head) rows
  int64_t st = d->order_slice_tokens;
  if (st == 0) {
    const int64_t q_tok_bytes = (int64_t)d->num_q_heads * D * qb;
    if ((int64_t)d->total_q * q_tok_bytes <= (16ll << 20))
      st = (int64_t)d->total_q + 1;
    else
      st = std::max<int64_t>((512 << 10) / q_tok_bytes, (int64_t)r.chunk * d->max_pages / d->num_slots);
  }
  const int64_t rows_cap = std::max<int64_t>(256, (rows + 255) / 256 * 256);
  int64_t slice_rows = std::min(rows_cap, (std::max<int64_t>(1, st * d->num_kv_heads) + 255) / 256 * 256);
  int64_t n_slices = std::max<int64_t>(1, (rows + slice_rows - 1) / slice_rows);
  while (n_slices * L > (1ll << 24) && n_slices > 1) {  // bound the plan's list arrays
    slice_rows *= 2;
    n_slices = std::max<int64_t>(1, (rows + slice_rows - 1) / slice_rows);
  }
  r.slice_rows = (int32_t)slice_rows;
  r.lists_per_slice = (int32_t)L;
  // every unit holds >= 1 entry: units <= entries/chunk + non-empty lists
  r.max_units = NS / r.chunk + std::min(n_slices * L, NS);
  r.lay = page_layout(n_slices * L, NS, r.max_units);
  return MSA_OK;
}

// Validated arguments of one call, for whichever route the descriptor takes.
struct Resolved {
  bool grouped;
  PageArgs pa;
  GroupArgs ga;
  size_t ws_bytes() const { return grouped ? ga.lay.total : pa.lay.total; }
};

msa_status resolve(const msa_prefill_desc *d, Resolved *r) {
  return check_desc(d, &r->pa, &r->ga, &r->grouped);
}

msa_status bind_workspace(Resolved *r, const msa_prefill_desc *d, void *ws, size_t bytes) {
  const size_t need = r->ws_bytes();
  if (bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", bytes, need);
  if (!ws) return fail(MSA_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  uint8_t *w = (uint8_t *)ws;
  if (r->grouped) {
    r->ga.ws = w;
    r->ga.err_flags = d->err_flags ? d->err_flags : (uint32_t *)(w + r->ga.lay.meta) + 1;
  } else {
    r->pa.ws = w;
    r->pa.err_flags = d->err_flags ? d->err_flags : (uint32_t *)(w + r->pa.lay.meta) + 1;
  }
  return MSA_OK;
}

msa_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Validated arguments of the indexer.  need_topk: the selection outputs are
// used (msa_index_topk / msa_prefill_index).
msa_status resolve_index(const msa_index_desc *d, bool need_topk, IndexArgs *r) {
  if (!d) return fail(MSA_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->struct_size != sizeof(msa_index_desc))
    return fail(MSA_ERR_INVALID_ARG, "struct_size %u != %zu (ABI mismatch)", d->struct_size,
                sizeof(msa_index_desc));
  if (d->num_seqs < 1 || d->total_q < 0 || d->num_heads < 1 || d->max_pages < 1 ||
      d->num_phys_pages < 1)
    return fail(MSA_ERR_INVALID_ARG, "bad sizes");
  if ((int64_t)d->total_q * d->num_heads >= (1ll << 31))
    return fail(MSA_ERR_UNSUPPORTED, "too many (token, head) rows");
  if (d->page_size != 128) return fail(MSA_ERR_UNSUPPORTED, "indexer is built for page_size 128");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "indexer head_dim must be 64 or 128");
  if (d->max_pages > kIndexMaxPages)
    return fail(MSA_ERR_UNSUPPORTED, "max_pages %d > %d", d->max_pages, kIndexMaxPages);
  if (d->page_table_stride < d->max_pages) return fail(MSA_ERR_INVALID_ARG, "page_table_stride < max_pages");
  if (!(d->q_scale > 0.0f) || !std::isfinite(d->q_scale) || !(d->k_scale > 0.0f) || !std::isfinite(d->k_scale))
    return fail(MSA_ERR_INVALID_ARG, "q_scale and k_scale must be finite and > 0");
  const bool rows = d->total_q > 0;  // an empty batch reads and writes nothing: NULL buffers pass
  if ((rows && !d->scores) || d->score_stride < d->max_pages || !aligned(d->scores, 4))
    return fail(MSA_ERR_INVALID_ARG, "scores must be a 4-byte aligned buffer with score_stride >= max_pages");
  if (rows) {  // inputs (checked for every call: one descriptor serves all three)
    const void *need[] = {d->q, d->q_seq, d->q_pos, d->seq_lens, d->k_cache, d->page_table};
    for (const void *p : need)
      if (!p) return fail(MSA_ERR_INVALID_ARG, "NULL input pointer");
    if (!aligned(d->q, 16) || d->q_stride_tok % 16 || d->q_stride_head % 16 || d->q_stride_tok < 0 ||
        d->q_stride_head < 0)
      return fail(MSA_ERR_INVALID_ARG, "q must be 16-byte aligned with 16-byte aligned strides");
    if (!aligned(d->k_cache, 16) || d->kv_stride_page_bytes % 16 || d->kv_stride_tok_bytes % 16 ||
        d->kv_stride_head_bytes % 16)
      return fail(MSA_ERR_INVALID_ARG, "k_cache and its strides must be 16-byte aligned");
  }
  if (need_topk) {
    if (d->top_k < 1 || d->top_k > 255) return fail(MSA_ERR_INVALID_ARG, "top_k must be in [1, 255]");
    if (rows && (!d->sel_idx || !d->sel_mask)) return fail(MSA_ERR_INVALID_ARG, "selection outputs are NULL");
    if (!aligned(d->sel_idx, 4) || d->sel_stride_tok < 0 || d->sel_stride_head < 0 ||
        (d->num_heads > 1 && d->sel_stride_head < d->top_k) ||
        d->sel_stride_tok < (int64_t)d->top_k + (int64_t)(d->num_heads - 1) * d->sel_stride_head)
      return fail(MSA_ERR_INVALID_ARG, "selection strides overlap");
  }
  IndexArgs &a = *r;
  memset(&a, 0, sizeof(a));
  a.num_seqs = d->num_seqs;
  a.total_q = d->total_q;
  a.H = d->num_heads;
  a.D = d->head_dim;
  a.page_size = d->page_size;
  a.max_pages = d->max_pages;
  a.num_phys_pages = d->num_phys_pages;
  a.top_k = d->top_k;
  a.scale = (float)((double)d->q_scale * d->k_scale);
  a.q = (const uint8_t *)d->q;
  a.q_stride_tok = d->q_stride_tok;
  a.q_stride_head = d->q_stride_head;
  a.q_seq = d->q_seq;
  a.q_pos = d->q_pos;
  a.seq_lens = d->seq_lens;
  a.k_cache = (const uint8_t *)d->k_cache;
  a.kv_stride_page = d->kv_stride_page_bytes;
  a.kv_stride_tok = d->kv_stride_tok_bytes;
  a.kv_stride_head = d->kv_stride_head_bytes;
  a.page_table = d->page_table;
  a.pt_stride = d->page_table_stride;
  a.scores = d->scores;
  a.score_stride = d->score_stride;
  a.sel_idx = d->sel_idx;
  a.sel_mask = d->sel_mask;
  a.sel_stride_tok = d->sel_stride_tok;
  a.sel_stride_head = d->sel_stride_head;
  a.err_flags = d->err_flags;
  return MSA_OK;
}

// ---- fixed device scratch of msa_sparse_prefill_noalloc
//
// The no-allocation entry point's workspace: one file-scope device array,
// of which every GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is used.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device

msa_status scratch_of_current_device(void **addr);

}  // namespace

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

msa_status scratch_of_current_device(void **addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MSA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_prefill_workspace_bytes(const msa_prefill_desc *d, size_t *bytes) {
  if (!bytes) return fail(MSA_ERR_INVALID_ARG, "bytes is NULL");
  Resolved r;
  msa_status s = resolve(d, &r);
  if (s != MSA_OK) return s;
  *bytes = r.ws_bytes();
  return ok();
}

size_t msa_sparse_prefill_workspace_bytes(const msa_prefill_desc *d) {
  size_t bytes = 0;
  return msa_prefill_workspace_bytes(d, &bytes) == MSA_OK ? bytes : 0;
}

msa_status msa_prefill_plan(const msa_prefill_desc *d, void *ws, size_t ws_bytes, void *stream) {
  Resolved r;
  msa_status s = resolve(d, &r);
  if (s != MSA_OK) return s;
  if ((s = bind_workspace(&r, d, ws, ws_bytes)) != MSA_OK) return s;
  if (r.grouped) return hip_status(launch_grouped_plan(r.ga, (hipStream_t)stream), "plan launch");
  return hip_status(launch_page_plan(r.pa, (hipStream_t)stream), "plan launch");
}

msa_status msa_prefill_attend(const msa_prefill_desc *d, void *ws, size_t ws_bytes, void *stream) {
  Resolved r;
  msa_status s = resolve(d, &r);
  if (s != MSA_OK) return s;
  if ((s = bind_workspace(&r, d, ws, ws_bytes)) != MSA_OK) return s;
  if (r.grouped) return hip_status(launch_grouped_attend(r.ga, (hipStream_t)stream), "attention launch");
  return hip_status(launch_page_attend(r.pa, (hipStream_t)stream), "attention launch");
}

msa_status msa_sparse_prefill(const msa_prefill_desc *d, void *ws, size_t ws_bytes, void *stream) {
  msa_status s = msa_prefill_plan(d, ws, ws_bytes, stream);
  if (s != MSA_OK) return s;
  return msa_prefill_attend(d, ws, ws_bytes, stream);
}

msa_status msa_sparse_prefill_noalloc(const msa_prefill_desc *d, void *stream) {
  Resolved r;
  msa_status s = resolve(d, &r);
  if (s != MSA_OK) return s;
  if (r.grouped && r.ga.sub_splits > 1 && r.ws_bytes() > kNoAllocScratchBytes) {
    r.ga.sub_splits = 1;  // the fixed scratch holds the problem without runs' partials
    set_grouped_layout(&r.ga);
  }
  const size_t need = r.ws_bytes();
  if (need > kNoAllocScratchBytes)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "problem needs %zu bytes of workspace, above the fixed %zu-byte scratch of the "
                "no-allocation entry point (use msa_sparse_prefill with a caller workspace)",
                need, kNoAllocScratchBytes);
  void *ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != MSA_OK) return s;
  if ((s = bind_workspace(&r, d, ws, kNoAllocScratchBytes)) != MSA_OK) return s;
  const hipStream_t st = (hipStream_t)stream;
  if (r.grouped) {
    hipError_t e = launch_grouped_plan(r.ga, st);
    if (e == hipSuccess) e = launch_grouped_attend(r.ga, st);
    return hip_status(e, "prefill launch");
  }
  hipError_t e = launch_page_plan(r.pa, st);
  if (e == hipSuccess) e = launch_page_attend(r.pa, st);
  return hip_status(e, "prefill launch");
}

size_t msa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

msa_status msa_combine_ex(const void *po, int32_t po_dtype, int64_t po_split, int64_t po_row,
                          const float *pl, int64_t pl_split, int32_t num_splits, int64_t num_rows,
                          int32_t dv, void *out, int32_t out_dtype, int64_t out_row, float *lse,
                          void *stream) {
  if (num_rows < 0 || num_splits < 1 || dv < 4 || dv > 1024 || dv % 4)
    return fail(MSA_ERR_INVALID_ARG, "bad sizes: splits %d rows %lld head_dim_v %d", num_splits,
                (long long)num_rows, dv);
  if (po_dtype != MSA_F32 && po_dtype != MSA_BF16 && po_dtype != MSA_F16)
    return fail(MSA_ERR_INVALID_ARG, "partial dtype must be F32, BF16 or F16");
  if (num_rows == 0) return ok();
  if (!po || !pl || !out) return fail(MSA_ERR_INVALID_ARG, "NULL buffer");
  if (out_dtype != MSA_F32 && out_dtype != MSA_BF16 && out_dtype != MSA_F16)
    return fail(MSA_ERR_INVALID_ARG, "out_dtype must be F32, BF16 or F16");
  const int ob = esize(out_dtype);
  if (!aligned(po, 16) || po_row % 4 || po_split % 4 || po_row < dv)
    return fail(MSA_ERR_INVALID_ARG, "partial_o must be 16-byte aligned with row stride >= head_dim_v");
  if (!aligned(out, 4 * ob) || (out_row * ob) % (4 * ob) || out_row < dv)
    return fail(MSA_ERR_INVALID_ARG, "out must be aligned to 4 elements with row stride >= head_dim_v");
  if (!aligned(pl, 4) || (lse && !aligned(lse, 4)) || pl_split < 0)
    return fail(MSA_ERR_INVALID_ARG, "lse buffers misaligned");
  return hip_status(launch_combine(po, po_dtype, po_split, po_row, pl, pl_split, num_splits, num_rows,
                                   dv, out, out_dtype, out_row, lse, (hipStream_t)stream),
                    "combine launch");
}

msa_status msa_combine(const float *po, int64_t po_split, int64_t po_row, const float *pl,
                       int64_t pl_split, int32_t num_splits, int64_t num_rows, int32_t dv, void *out,
                       int32_t out_dtype, int64_t out_row, float *lse, void *stream) {
  return msa_combine_ex(po, MSA_F32, po_split, po_row, pl, pl_split, num_splits, num_rows, dv, out,
                        out_dtype, out_row, lse, stream);
}

msa_status msa_index_scores(const msa_index_desc *d, void *stream) {
  IndexArgs a;
  msa_status s = resolve_index(d, false, &a);
  if (s != MSA_OK) return s;
  return hip_status(launch_index_scores(a, (hipStream_t)stream), "index scores launch");
}

msa_status msa_index_topk(const msa_index_desc *d, void *stream) {
  IndexArgs a;
  msa_status s = resolve_index(d, true, &a);
  if (s != MSA_OK) return s;
  return hip_status(launch_index_topk(a, (hipStream_t)stream), "index top-k launch");
}

msa_status msa_prefill_index(const msa_index_desc *d, void *stream) {
  IndexArgs a;
  msa_status s = resolve_index(d, true, &a);
  if (s != MSA_OK) return s;
  hipError_t e = launch_index_scores(a, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_index_topk(a, (hipStream_t)stream);
  return hip_status(e, "indexer launch");
}

msa_status msa_nvfp4_dequant_e4m3(const uint8_t *codes, const uint8_t *scales, uint8_t *out,
                                  int64_t n, void *stream) {
  if (n < 0) return fail(MSA_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return ok();
  if (!codes || !scales || !out) return fail(MSA_ERR_INVALID_ARG, "NULL buffer");
  return hip_status(launch_nvfp4_dequant(codes, scales, out, n, (hipStream_t)stream), "dequant launch");
}

msa_status msa_nvfp4_dequant_f16(const uint8_t *codes, const uint8_t *scales, uint16_t *out,
                                 int64_t n, void *stream) {
  if (n < 0) return fail(MSA_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return ok();
  if (!codes || !scales || !out) return fail(MSA_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned(out, 2)) return fail(MSA_ERR_INVALID_ARG, "out must be 2-byte aligned");
  return hip_status(launch_nvfp4_dequant_f16(codes, scales, out, n, (hipStream_t)stream),
                    "dequant launch");
}

size_t msa_required_lds_bytes(void) {
  const size_t sizes[] = {page_plan_lds_bytes(), page_attend_lds_bytes(), grouped_plan_lds_bytes(),
                          grouped_attend_lds_bytes(), index_lds_bytes()};
  size_t m = 0;
  for (size_t x : sizes) m = std::max(m, x);
  return m;
}

int msa_device_supported(int device) {
  static std::atomic<int> cache[kMaxDevices];  // 0 unknown, 1 yes, 2 no
  if (device < 0 || device >= kMaxDevices) return 0;
  int c = cache[device].load();
  if (c) return c == 1;
  hipDeviceProp_t prop;
  int yes = 0;
  if (hipGetDeviceProperties(&prop, device) == hipSuccess)
    yes = strncmp(prop.gcnArchName, "gfx950", 6) == 0 && prop.sharedMemPerBlock >= msa_required_lds_bytes();
  cache[device].store(yes ? 1 : 2);
  return yes;
}

const char *msa_status_str(msa_status s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char *msa_last_error(void) { return g_err; }

int msa_abi_version(void) { return MSA_ABI_VERSION; }

}  // extern "C"
