// Plan step of the page-selection route: builds the inverted index that lets
// the attention kernel keep one physical page resident and stream the
// queries that selected it (MiniMax-AI/MSA PR 21, section "K1": one
// workgroup per (page, head, query split)).
//
//   plan_zero  : clear the per-list counters and the error word
//   plan_count : per (token, KV head) -- validate every slot, write
//                lse = -inf for each empty slot, and give every used slot its
//                position inside its (slice, KV head, request, logical page)
//                list.  Slices are runs of slice_rows (token, KV head) rows;
//                listing them outermost makes the work units come out slice
//                by slice, so the units running together re-read the
//                queries of one slice only (they stay in the L2s).
//                A workgroup first counts into an LDS histogram, then claims
//                its block of each list with one global atomic per list, so
//                the global counters see one atomic per (workgroup, list)
//                instead of one per selection.
//   plan_scan  : exclusive scans of list sizes and of work units (lists cut
//                evenly into units of at most `chunk` entries, numbered by
//                size class, largest first), tile by tile
//   plan_fill  : scatter (token, slot, visible limit) entries to their
//                positions (no atomics), and write one record per work unit
//                (its entries, physical page and KV head)
//
// Entry order inside a list depends on atomics, but every (token, slot)
// partial is computed on its own, so the results do not depend on it.
#include "launch.h"

namespace msa {
namespace {

constexpr int kPlanThreads = 64;  // plan_fill: one (token, KV head) row per thread, many workgroups
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

// Rows per plan_count workgroup (slice_rows is a multiple of both): 64 keeps
// many workgroups in flight; 256 when a slice has many lists, since every
// workgroup clears and claims all of its slice's lists.
constexpr int kCountThreads = 64;
constexpr int kCountThreadsWide = 256;
constexpr int kCountWideLists = 2048;  // lists per slice from which the wide form is used
constexpr int kRegSlots = 16;      // rows with at most this many slots keep them in registers

template <bool LDS_HIST, int NT>
__global__ void __launch_bounds__(NT) plan_count(const PageArgs a) {
  extern __shared__ int32_t hist[];
  const int64_t L = a.lists_per_slice;
  const int tid = threadIdx.x;
  // slice_rows is a multiple of the block size: one slice per workgroup
  const int64_t lbase = ((int64_t)blockIdx.x * NT) / a.slice_rows * L;
  int32_t *counts = (int32_t *)(a.ws + a.lay.counts);
  if constexpr (LDS_HIST) {
    for (int64_t i = tid; i < L; i += NT) hist[i] = 0;
    __syncthreads();
  }
  const int64_t idx = (int64_t)blockIdx.x * NT + tid;
  const bool live = idx < (int64_t)a.total_q * a.Hkv;
  const int K = a.num_slots;
  int32_t *slot_list = (int32_t *)(a.ws + a.lay.slot_list) + idx * K;
  int32_t *slot_pos = (int32_t *)(a.ws + a.lay.slot_pos) + idx * K;
  // rows of at most kRegSlots slots keep each slot's list (local index, -1:
  // none) and its position in the workgroup's block in registers until the
  // block offsets are known, and store the final position once
  int lr[kRegSlots], pr[kRegSlots];
#pragma unroll
  for (int j = 0; j < kRegSlots; ++j) lr[j] = -1, pr[j] = 0;
  if (live) {
    const int r = (int)(idx / a.Hkv), g = (int)(idx - (int64_t)r * a.Hkv);
    const int32_t *sidx = a.sel_idx + r * a.sel_stride_tok + g * a.sel_stride_head;
    const uint8_t *smask = a.sel_mask + r * a.sel_stride_tok + g * a.sel_stride_head;
    uint32_t err = 0;
    const RowCtx c = row_ctx(a, r, err);
    const int bb = c.valid ? c.b : 0;  // an in-bounds table row for the loads below
    // slot j: validate, find its list, claim a position (or mark the split
    // empty); returns the list (-1: none) and, in `pos`, the position claimed
    auto visit = [&](int j, uint32_t mk, int u, bool dup, int pp, int &pos, bool store_pos) -> int {
      int list = -1;
      if (c.valid && mk) {
        if (u < 0 || u >= a.max_pages) {
          err |= MSA_ERRF_SEL_RANGE;
        } else if (dup) {
          err |= MSA_ERRF_DUPLICATE;
        } else if ((int64_t)u * a.page_size <= c.last) {
          if (pp < 0 || pp >= a.num_phys_pages)
            err |= MSA_ERRF_PHYS_RANGE;
          else
            list = (g * a.num_seqs + c.b) * a.max_pages + u;  // KV head outermost
        }
      }
      slot_list[j] = list >= 0 ? (int32_t)(lbase + list) : -1;
      if (list >= 0) {
        pos = LDS_HIST ? atomicAdd(&hist[list], 1) : atomicAdd(&counts[lbase + list], 1);
        if (store_pos) slot_pos[j] = pos;
      } else {
        float *pl = a.partial_lse + j * a.pl_split_stride + (int64_t)r * a.Hq + g * a.G;
        for (int h = 0; h < a.G; ++h) pl[h] = -INFINITY;
      }
      return list;
    };
    if (K <= kRegSlots) {
      // every load of the row is issued before any is used; the duplicate
      // test runs on registers
      uint32_t mk[kRegSlots];
      int uu[kRegSlots], pp[kRegSlots];
#pragma unroll
      for (int j = 0; j < kRegSlots; ++j) {
        const int jc = j < K ? j : 0;
        mk[j] = j < K ? (uint32_t)smask[jc] : 0u;
        uu[j] = sidx[jc];
      }
#pragma unroll
      for (int j = 0; j < kRegSlots; ++j) {
        const int uc = (uu[j] >= 0 && uu[j] < a.max_pages) ? uu[j] : 0;
        pp[j] = a.page_table[bb * a.pt_stride + uc];
      }
#pragma unroll
      for (int j = 0; j < kRegSlots; ++j) {
        if (j < K) {
          bool dup = false;
#pragma unroll
          for (int jj = 0; jj < j; ++jj) dup |= (mk[jj] != 0u) && (uu[jj] == uu[j]);
          lr[j] = visit(j, mk[j], uu[j], dup, pp[j], pr[j], !LDS_HIST);
        }
      }
    } else {
      for (int j = 0; j < K; ++j) {
        const uint32_t mk = smask[j];
        const int u = sidx[j];
        bool dup = false;
        for (int jj = 0; jj < j; ++jj) dup |= (smask[jj] != 0) && (sidx[jj] == u);
        const int uc = (u >= 0 && u < a.max_pages) ? u : 0;
        int pos = 0;
        visit(j, mk, u, dup, a.page_table[bb * a.pt_stride + uc], pos, true);
      }
    }
    if (err) atomicOr(a.err_flags, err);
  }
  if constexpr (LDS_HIST) {
    __syncthreads();
    for (int64_t i = tid; i < L; i += NT) {
      const int32_t n = hist[i];
      if (n) hist[i] = atomicAdd(&counts[lbase + i], n);  // this workgroup's block of list i
    }
    __syncthreads();
    if (live) {
      if (K <= kRegSlots) {
#pragma unroll
        for (int j = 0; j < kRegSlots; ++j)
          if (lr[j] >= 0) slot_pos[j] = pr[j] + hist[lr[j]];
      } else {
        for (int j = 0; j < K; ++j) {
          const int list = slot_list[j];
          if (list >= 0) slot_pos[j] += hist[list - lbase];
        }
      }
    }
  }
}

constexpr int kScanThreads = 1024;
constexpr int kScanPer = kScanTile / kScanThreads;  // lists per thread
constexpr int kScanOneBlockMax = kScanThreads * 8;  // lists one workgroup scans alone

// With a single ordering slice (all queries fit in the caches, so there is
// no query locality to keep), work units are numbered by size class, largest
// first, and by list within a class: the workgroups dispatched last then run
// the shortest units instead of, say, the own pages of the last request,
// which would otherwise end the kernel long after the rest.  With several
// slices the units stay in list (slice) order.  A list of n entries makes
// ceil(n / chunk) units of n / units entries each; its class is 0 for units
// of at least chunk/2 entries, 1 for chunk/4, 2 for chunk/8, else 3.
constexpr int kSizeClasses = 4;
__device__ __forceinline__ int units_of(int32_t n, int chunk) { return (n + chunk - 1) / chunk; }
__device__ __forceinline__ int size_class(const PageArgs &a, int32_t n) {
  if (a.lay.num_lists != a.lists_per_slice) return 0;
  const int32_t s = n / max(1, units_of(n, a.chunk));  // entries per unit (rounded down)
  return 2 * s >= a.chunk ? 0 : (4 * s >= a.chunk ? 1 : (8 * s >= a.chunk ? 2 : 3));
}

// Per-class unit counts of one thread's lists, and its running offsets.
struct ClassCounts {
  int32_t v[kSizeClasses];
};

// Up to kScanOneBlockMax lists: one workgroup scans them all, PER lists per
// thread -- inclusive scans within each wave by shuffles, the wave totals
// through LDS behind a single barrier -- and writes the final offsets:
// list_off (entries) in list order, unit_off (the list's first unit) in
// (size class, list) order.
template <int PER>
__global__ void __launch_bounds__(kScanThreads) plan_scan_one(const PageArgs a) {
  constexpr int NW = kScanThreads / 64;
  constexpr int NC = kSizeClasses;
  __shared__ int32_t w_e[NW], w_u[NC][NW];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t L = a.lay.num_lists;
  const int32_t *counts = (const int32_t *)(a.ws + a.lay.counts);
  int32_t *list_off = (int32_t *)(a.ws + a.lay.list_off);
  int32_t *unit_off = (int32_t *)(a.ws + a.lay.unit_off);
  const int64_t i0 = (int64_t)t * PER;
  int32_t c[PER];
  int32_t se = 0;
  ClassCounts su = {};
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    // unconditional loads (clamped index; L >= 1), so that all of them are
    // in flight at once instead of one branch and wait per list
    const int32_t v = counts[min(i0 + k, L - 1)];
    c[k] = i0 + k < L ? v : 0;
    se += c[k];
    const int cl = size_class(a, c[k]), u = units_of(c[k], a.chunk);
#pragma unroll
    for (int q = 0; q < NC; ++q) su.v[q] += q == cl ? u : 0;
  }
  int32_t ie = se;  // inclusive scans over the wave's lanes
  ClassCounts iu = su;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t ve = __shfl_up(ie, off);
    ClassCounts vu;
#pragma unroll
    for (int q = 0; q < NC; ++q) vu.v[q] = __shfl_up(iu.v[q], off);
    if (lane >= off) {
      ie += ve;
#pragma unroll
      for (int q = 0; q < NC; ++q) iu.v[q] += vu.v[q];
    }
  }
  if (lane == 63) {
    w_e[w] = ie;
#pragma unroll
    for (int q = 0; q < NC; ++q) w_u[q][w] = iu.v[q];
  }
  __syncthreads();
  int32_t oe = 0;  // totals of the earlier waves
  ClassCounts ou = {}, tot = {};
  for (int k = 0; k < NW; ++k) {
    if (k < w) oe += w_e[k];
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      ou.v[q] += k < w ? w_u[q][k] : 0;
      tot.v[q] += w_u[q][k];
    }
  }
  int32_t be = oe + ie - se;
  ClassCounts bu;
  int32_t base = 0;
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    bu.v[q] = base + ou.v[q] + iu.v[q] - su.v[q];
    base += tot.v[q];
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int cl = size_class(a, c[k]), u = units_of(c[k], a.chunk);
    int32_t uo = bu.v[0];
#pragma unroll
    for (int q = 1; q < NC; ++q) uo = q == cl ? bu.v[q] : uo;
    if (i0 + k < L) {
      list_off[i0 + k] = be;
      unit_off[i0 + k] = uo;
    }
    be += c[k];
#pragma unroll
    for (int q = 0; q < NC; ++q) bu.v[q] += q == cl ? u : 0;
  }
  if (t == kScanThreads - 1) {
    int32_t *meta = (int32_t *)(a.ws + a.lay.meta);
    list_off[L] = be;
    meta[0] = base;  // number of work units
    meta[2] = be;    // number of entries
  }
}

// More lists: the same offsets in three steps -- per tile of kScanTile lists
// (offsets within the tile, per class), over the tile totals (tile offsets
// per class, class bases), then the tile offsets added back.  Per tile, the
// tiles array holds 1 + kSizeClasses words: entries, then units per class.
constexpr int kTileWords = 1 + kSizeClasses;

__global__ void __launch_bounds__(kScanThreads) plan_scan_tiles(const PageArgs a) {
  constexpr int PER = kScanPer;
  constexpr int NC = kSizeClasses;
  __shared__ int32_t s_e[kScanThreads];
  __shared__ int32_t s_u[NC][kScanThreads];
  const int t = threadIdx.x;
  const int64_t L = a.lay.num_lists;
  const int32_t *counts = (const int32_t *)(a.ws + a.lay.counts);
  int32_t *list_off = (int32_t *)(a.ws + a.lay.list_off);
  int32_t *unit_off = (int32_t *)(a.ws + a.lay.unit_off);
  const int64_t i0 = (int64_t)blockIdx.x * (kScanThreads * PER) + (int64_t)t * PER;
  int32_t c[PER];
  int32_t se = 0;
  ClassCounts su = {};
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t v = counts[min(i0 + k, L - 1)];
    c[k] = i0 + k < L ? v : 0;
    se += c[k];
    const int cl = size_class(a, c[k]), u = units_of(c[k], a.chunk);
#pragma unroll
    for (int q = 0; q < NC; ++q) su.v[q] += q == cl ? u : 0;
  }
  s_e[t] = se;
#pragma unroll
  for (int q = 0; q < NC; ++q) s_u[q][t] = su.v[q];
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t ve = t >= off ? s_e[t - off] : 0;
    ClassCounts vu;
#pragma unroll
    for (int q = 0; q < NC; ++q) vu.v[q] = t >= off ? s_u[q][t - off] : 0;
    __syncthreads();
    s_e[t] += ve;
#pragma unroll
    for (int q = 0; q < NC; ++q) s_u[q][t] += vu.v[q];
    __syncthreads();
  }
  int32_t be = s_e[t] - se;
  ClassCounts bu;
#pragma unroll
  for (int q = 0; q < NC; ++q) bu.v[q] = s_u[q][t] - su.v[q];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int cl = size_class(a, c[k]), u = units_of(c[k], a.chunk);
    int32_t uo = bu.v[0];
#pragma unroll
    for (int q = 1; q < NC; ++q) uo = q == cl ? bu.v[q] : uo;
    if (i0 + k < L) {
      list_off[i0 + k] = be;
      unit_off[i0 + k] = uo;
    }
    be += c[k];
#pragma unroll
    for (int q = 0; q < NC; ++q) bu.v[q] += q == cl ? u : 0;
  }
  if (t == kScanThreads - 1) {  // this tile's totals, for plan_scan_top
    int32_t *tiles = (int32_t *)(a.ws + a.lay.tiles) + (int64_t)blockIdx.x * kTileWords;
    tiles[0] = s_e[t];
#pragma unroll
    for (int q = 0; q < NC; ++q) tiles[1 + q] = s_u[q][t];
  }
}

__global__ void __launch_bounds__(kScanThreads) plan_scan_top(const PageArgs a, int nt) {
  constexpr int NC = kSizeClasses;
  __shared__ int32_t s_e[kScanThreads];
  __shared__ int32_t s_u[NC][kScanThreads];
  const int t = threadIdx.x;
  int32_t *tiles = (int32_t *)(a.ws + a.lay.tiles);
  const int per = (nt + kScanThreads - 1) / kScanThreads;
  const int j0 = min(nt, t * per), j1 = min(nt, j0 + per);
  int32_t se = 0;
  ClassCounts su = {};
  for (int j = j0; j < j1; ++j) {
    se += tiles[j * kTileWords];
#pragma unroll
    for (int q = 0; q < NC; ++q) su.v[q] += tiles[j * kTileWords + 1 + q];
  }
  s_e[t] = se;
#pragma unroll
  for (int q = 0; q < NC; ++q) s_u[q][t] = su.v[q];
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t ve = t >= off ? s_e[t - off] : 0;
    ClassCounts vu;
#pragma unroll
    for (int q = 0; q < NC; ++q) vu.v[q] = t >= off ? s_u[q][t - off] : 0;
    __syncthreads();
    s_e[t] += ve;
#pragma unroll
    for (int q = 0; q < NC; ++q) s_u[q][t] += vu.v[q];
    __syncthreads();
  }
  // class q's units start after all units of the classes before it
  ClassCounts base;
  int32_t total = 0;
#pragma unroll
  for (int q = 0; q < NC; ++q) {
    base.v[q] = total;
    total += s_u[q][kScanThreads - 1];
  }
  int32_t be = s_e[t] - se;
  ClassCounts bu;
#pragma unroll
  for (int q = 0; q < NC; ++q) bu.v[q] = base.v[q] + s_u[q][t] - su.v[q];
  for (int j = j0; j < j1; ++j) {  // totals -> exclusive offsets, in place
    int32_t *tj = tiles + j * kTileWords;
    const int32_t e = tj[0];
    tj[0] = be;
    be += e;
#pragma unroll
    for (int q = 0; q < NC; ++q) {
      const int32_t u = tj[1 + q];
      tj[1 + q] = bu.v[q];
      bu.v[q] += u;
    }
  }
  if (t == kScanThreads - 1) {
    const int64_t L = a.lay.num_lists;
    int32_t *meta = (int32_t *)(a.ws + a.lay.meta);
    ((int32_t *)(a.ws + a.lay.list_off))[L] = s_e[t];
    meta[0] = total;
    meta[2] = s_e[t];
  }
}

__global__ void __launch_bounds__(kScanThreads) plan_scan_add(const PageArgs a) {
  const int tile = blockIdx.x;
  const int32_t *tiles = (const int32_t *)(a.ws + a.lay.tiles) + (int64_t)tile * kTileWords;
  const int32_t oe = tiles[0];
  ClassCounts ou;
#pragma unroll
  for (int q = 0; q < kSizeClasses; ++q) ou.v[q] = tiles[1 + q];
  const int32_t *counts = (const int32_t *)(a.ws + a.lay.counts);
  int32_t *list_off = (int32_t *)(a.ws + a.lay.list_off);
  int32_t *unit_off = (int32_t *)(a.ws + a.lay.unit_off);
  const int64_t L = a.lay.num_lists;
  const int64_t i0 = (int64_t)tile * kScanTile;
  for (int k = threadIdx.x; k < kScanTile; k += kScanThreads)
    if (i0 + k < L) {
      const int cl = size_class(a, counts[i0 + k]);
      int32_t o = ou.v[0];
#pragma unroll
      for (int q = 1; q < kSizeClasses; ++q) o = q == cl ? ou.v[q] : o;
      list_off[i0 + k] += oe;
      unit_off[i0 + k] += o;
    }
}

// The work units of list l: its entries split evenly into units of at most
// a.chunk entries (from unit_off[l] on), each with the list's physical page
// (in range: a list exists only for a valid page) and KV head, so that the
// attention kernel reads one record per unit.
__device__ __forceinline__ void write_units(const PageArgs &a, int64_t l) {
  if (l >= a.lay.num_lists) return;
  const int32_t *list_off = (const int32_t *)(a.ws + a.lay.list_off);
  const int32_t *unit_off = (const int32_t *)(a.ws + a.lay.unit_off);
  const int32_t lo = list_off[l], n = list_off[l + 1] - lo;
  if (n == 0) return;
  const int32_t u0 = unit_off[l];
  const int pl = (int)(l % a.lists_per_slice);
  const int u = pl % a.max_pages;
  const int b = (pl / a.max_pages) % a.num_seqs;
  PageUnit w;
  w.g = pl / (a.max_pages * a.num_seqs);
  w.phys = a.page_table[b * a.pt_stride + u];
  PageUnit *units = (PageUnit *)(a.ws + a.lay.units) + u0;
  const int32_t nu = (n + a.chunk - 1) / a.chunk;  // the list's entries split evenly
  for (int32_t c = 0; c < nu; ++c) {
    const int32_t b0 = (int32_t)((int64_t)c * n / nu), b1 = (int32_t)((int64_t)(c + 1) * n / nu);
    w.e_begin = lo + b0;
    w.e_count = b1 - b0;
    units[c] = w;
  }
}

// Blocks [0, fill_blocks): one (token, KV head) row per thread, its entries
// into the lists; the blocks after them: one list per thread, its units.
__global__ void __launch_bounds__(kPlanThreads) plan_fill(const PageArgs a, int fill_blocks) {
  if ((int)blockIdx.x >= fill_blocks) {
    write_units(a, (int64_t)(blockIdx.x - fill_blocks) * kPlanThreads + threadIdx.x);
    return;
  }
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

size_t page_plan_lds_bytes() { return (size_t)kMaxLdsLists * 4; }  // plan_count's histogram

hipError_t launch_page_plan(const PageArgs &a, hipStream_t s) {
  int32_t *counts = (int32_t *)(a.ws + a.lay.counts);
  const int64_t L = a.lay.num_lists;  // all slices
  const int64_t zero_blocks = (L + 255) / 256 > 0 ? (L + 255) / 256 : 1;
  plan_zero<<<(unsigned)zero_blocks, 256, 0, s>>>(counts, L, a.err_flags);
  const int64_t rows = (int64_t)a.total_q * a.Hkv;
  const unsigned blocks = (unsigned)((rows + kPlanThreads - 1) / kPlanThreads);
  if (rows > 0) {
    const size_t hist_bytes = (size_t)a.lists_per_slice * 4;
    if (a.lists_per_slice > kMaxLdsLists) {
      plan_count<false, kCountThreads><<<(unsigned)((rows + kCountThreads - 1) / kCountThreads),
                                         kCountThreads, 0, s>>>(a);
    } else if (a.lists_per_slice > kCountWideLists) {
      plan_count<true, kCountThreadsWide><<<(unsigned)((rows + kCountThreadsWide - 1) / kCountThreadsWide),
                                            kCountThreadsWide, hist_bytes, s>>>(a);
    } else {
      plan_count<true, kCountThreads><<<(unsigned)((rows + kCountThreads - 1) / kCountThreads),
                                        kCountThreads, hist_bytes, s>>>(a);
    }
  }
  if (L <= kScanTile) {
    plan_scan_one<kScanPer><<<1, kScanThreads, 0, s>>>(a);
  } else if (L <= kScanOneBlockMax) {
    plan_scan_one<kScanOneBlockMax / kScanThreads><<<1, kScanThreads, 0, s>>>(a);
  } else {
    const int nt = (int)((L + kScanTile - 1) / kScanTile);
    plan_scan_tiles<<<nt, kScanThreads, 0, s>>>(a);
    plan_scan_top<<<1, kScanThreads, 0, s>>>(a, nt);
    plan_scan_add<<<nt, kScanThreads, 0, s>>>(a);
  }
  const int64_t list_blocks = (L + kPlanThreads - 1) / kPlanThreads;
  plan_fill<<<(unsigned)(blocks + list_blocks), kPlanThreads, 0, s>>>(a, (int)blocks);
  return hipGetLastError();
}

}  // namespace msa
