// Plan step of the page-selection route: builds the inverted index that lets
// the attention kernel keep one physical page resident and stream the
// queries that selected it (MiniMax-AI/MSA PR 21, section "K1": one
// workgroup per (page, head, query split)).
//
//   plan_zero  : clear the per-list counters and the error word
//   plan_count : per (token, KV head) -- validate every slot, write
//                lse = -inf for each empty slot, and give every used slot its
//                position inside its (request, logical page, KV head) list.
//                A workgroup first counts into an LDS histogram, then claims
//                its block of each list with one global atomic per list, so
//                the global counters see one atomic per (workgroup, list)
//                instead of one per selection.
//   plan_scan  : one workgroup -- exclusive scans of list sizes and of work
//                units (lists cut into chunks of `chunk` entries)
//   plan_fill  : scatter (token, slot, visible limit) entries to their
//                positions (no atomics)
//
// Entry order inside a list depends on atomics, but every (token, slot)
// partial is computed on its own, so the results do not depend on it.
#include "launch.h"

namespace msa {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kMaxLdsLists = 16384;  // lists an LDS histogram may hold (64 KiB)

__global__ void plan_zero(int32_t *counts, int64_t n, uint32_t *err) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counts[i] = 0;
  if (i == 0) *err = 0u;
}

struct RowCtx {
  bool valid;
  int b, last;  // request, last visible key position (-1: none)
};

__device__ __forceinline__ RowCtx row_ctx(const PageArgs &a, int r, uint32_t &err) {
  RowCtx c;
  const int pos = a.q_pos[r];
  const int b = a.q_seq[r];
  c.valid = pos >= 0;
  c.b = b;
  c.last = -1;
  if (c.valid && (b < 0 || b >= a.num_seqs)) {
    err |= MSA_ERRF_QSEQ_RANGE;
    c.valid = false;
  }
  if (c.valid) c.last = min(pos, a.seq_lens[b] - 1);
  return c;
}

template <bool LDS_HIST>
__global__ void __launch_bounds__(kPlanThreads) plan_count(const PageArgs a) {
  extern __shared__ int32_t hist[];
  const int64_t L = a.lay.num_lists;
  const int tid = threadIdx.x;
  int32_t *counts = (int32_t *)(a.ws + a.lay.counts);
  if constexpr (LDS_HIST) {
    for (int64_t i = tid; i < L; i += kPlanThreads) hist[i] = 0;
    __syncthreads();
  }
  const int64_t idx = (int64_t)blockIdx.x * kPlanThreads + tid;
  const bool live = idx < (int64_t)a.total_q * a.Hkv;
  const int K = a.num_slots;
  int32_t *slot_list = (int32_t *)(a.ws + a.lay.slot_list) + idx * K;
  int32_t *slot_pos = (int32_t *)(a.ws + a.lay.slot_pos) + idx * K;
  if (live) {
    const int r = (int)(idx / a.Hkv), g = (int)(idx - (int64_t)r * a.Hkv);
    const int32_t *sidx = a.sel_idx + r * a.sel_stride_tok + g * a.sel_stride_head;
    const uint8_t *smask = a.sel_mask + r * a.sel_stride_tok + g * a.sel_stride_head;
    uint32_t err = 0;
    const RowCtx c = row_ctx(a, r, err);
    for (int j = 0; j < K; ++j) {
      int list = -1;
      const uint32_t mk = smask[j];
      if (c.valid && mk) {
        const int u = sidx[j];
        if (u < 0 || u >= a.max_pages) {
          err |= MSA_ERRF_SEL_RANGE;
        } else {
          bool dup = false;
          for (int jj = 0; jj < j; ++jj) dup |= (smask[jj] != 0) && (sidx[jj] == u);
          if (dup) {
            err |= MSA_ERRF_DUPLICATE;
          } else if ((int64_t)u * a.page_size <= c.last) {
            const int pp = a.page_table[c.b * a.pt_stride + u];
            if (pp < 0 || pp >= a.num_phys_pages)
              err |= MSA_ERRF_PHYS_RANGE;
            else
              list = (c.b * a.max_pages + u) * a.Hkv + g;
          }
        }
      }
      slot_list[j] = list;
      if (list >= 0) {
        slot_pos[j] = LDS_HIST ? atomicAdd(&hist[list], 1) : atomicAdd(&counts[list], 1);
      } else {
        float *pl = a.partial_lse + j * a.pl_split_stride + (int64_t)r * a.Hq + g * a.G;
        for (int h = 0; h < a.G; ++h) pl[h] = -INFINITY;
      }
    }
    if (err) atomicOr(a.err_flags, err);
  }
  if constexpr (LDS_HIST) {
    __syncthreads();
    for (int64_t i = tid; i < L; i += kPlanThreads) {
      const int32_t n = hist[i];
      if (n) hist[i] = atomicAdd(&counts[i], n);  // this workgroup's block of list i
    }
    __syncthreads();
    if (live)
      for (int j = 0; j < K; ++j) {
        const int list = slot_list[j];
        if (list >= 0) slot_pos[j] += hist[list];
      }
  }
}

constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kScanThreads) plan_scan(const PageArgs a) {
  __shared__ int32_t s_e[kScanThreads];
  __shared__ int32_t s_u[kScanThreads];
  const int t = threadIdx.x;
  const int64_t L = a.lay.num_lists;
  const int32_t *counts = (const int32_t *)(a.ws + a.lay.counts);
  int32_t *list_off = (int32_t *)(a.ws + a.lay.list_off);
  int32_t *unit_off = (int32_t *)(a.ws + a.lay.unit_off);
  int32_t *meta = (int32_t *)(a.ws + a.lay.meta);
  const int64_t per = (L + kScanThreads - 1) / kScanThreads;
  const int64_t i0 = min(L, (int64_t)t * per), i1 = min(L, i0 + per);
  int32_t se = 0, su = 0;
  for (int64_t i = i0; i < i1; ++i) {
    const int32_t c = counts[i];
    se += c;
    su += (c + a.chunk - 1) / a.chunk;
  }
  s_e[t] = se;
  s_u[t] = su;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t ve = t >= off ? s_e[t - off] : 0;
    const int32_t vu = t >= off ? s_u[t - off] : 0;
    __syncthreads();
    s_e[t] += ve;
    s_u[t] += vu;
    __syncthreads();
  }
  int32_t be = s_e[t] - se, bu = s_u[t] - su;
  for (int64_t i = i0; i < i1; ++i) {
    const int32_t c = counts[i];
    list_off[i] = be;
    unit_off[i] = bu;
    be += c;
    bu += (c + a.chunk - 1) / a.chunk;
  }
  if (t == kScanThreads - 1) {
    list_off[L] = s_e[t];
    unit_off[L] = s_u[t];
    meta[0] = s_u[t];  // number of work units
    meta[2] = s_e[t];  // number of entries
  }
}

__global__ void __launch_bounds__(kPlanThreads) plan_fill(const PageArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
  if (idx >= (int64_t)a.total_q * a.Hkv) return;
  const int r = (int)(idx / a.Hkv), g = (int)(idx - (int64_t)r * a.Hkv);
  const int K = a.num_slots;
  const int32_t *sidx = a.sel_idx + r * a.sel_stride_tok + g * a.sel_stride_head;
  const int32_t *slot_list = (const int32_t *)(a.ws + a.lay.slot_list) + idx * K;
  const int32_t *slot_pos = (const int32_t *)(a.ws + a.lay.slot_pos) + idx * K;
  const int32_t *list_off = (const int32_t *)(a.ws + a.lay.list_off);
  PlanEntry *entries = (PlanEntry *)(a.ws + a.lay.entries);
  uint32_t err = 0;
  const RowCtx c = row_ctx(a, r, err);
  for (int j = 0; j < K; ++j) {
    const int list = slot_list[j];
    if (list < 0) continue;
    PlanEntry e;
    e.tok_slot = (r << 8) | j;
    e.limit = min(c.last - sidx[j] * a.page_size, a.page_size - 1);
    entries[list_off[list] + slot_pos[j]] = e;
  }
}

}  // namespace

hipError_t launch_page_plan(const PageArgs &a, hipStream_t s) {
  int32_t *counts = (int32_t *)(a.ws + a.lay.counts);
  const int64_t L = a.lay.num_lists;
  const int64_t zero_blocks = (L + 255) / 256 > 0 ? (L + 255) / 256 : 1;
  plan_zero<<<(unsigned)zero_blocks, 256, 0, s>>>(counts, L, a.err_flags);
  const int64_t rows = (int64_t)a.total_q * a.Hkv;
  const unsigned blocks = (unsigned)((rows + kPlanThreads - 1) / kPlanThreads);
  if (blocks) {
    if (L <= kMaxLdsLists)
      plan_count<true><<<blocks, kPlanThreads, (size_t)L * 4, s>>>(a);
    else
      plan_count<false><<<blocks, kPlanThreads, 0, s>>>(a);
  }
  plan_scan<<<1, kScanThreads, 0, s>>>(a);
  if (blocks) plan_fill<<<blocks, kPlanThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace msa
