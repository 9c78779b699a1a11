// Plan step of the page-selection route: builds the inverted index that lets
// the attention kernel keep one physical page resident and stream the
// queries that selected it (MiniMax-AI/MSA PR 21, section "K1": one
// workgroup per (page, head, query split)).
//
//   plan_zero  : clear the per-list counters and the error word
//   plan_count : per (token, KV head, slot), one lane each -- validate, write
//                lse = -inf for an empty slot, and give a used slot its
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

constexpr int kPlanThreads = 256;  // plan_fill workgroups

// Marks v as produced here.  After a batch of loads, pinning each result
// makes all of them complete before any is used (one wait for the batch):
// without it the compiler turns a select on a uniform condition, such as
// `j < K ? x[j] : 0`, into a branch and moves the load inside, which leaves
// one load and one full wait per slot -- sixteen round trips where one does.
template <class T>
__device__ __forceinline__ void pin(T &v) {
  __asm__ volatile("" : "+v"(v));
}
constexpr int kMaxLdsLists = 15360;  // lists an LDS histogram may hold (60 KiB, + 4 KiB of slot order)

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

// plan_count puts the K slots of a (token, KV head) row on K adjacent lanes
// (K <= 64; rpw = the largest power of two <= 64 / K rows per wave, at most
// 16), so that every load and store of the slot arrays is one contiguous run
// per wave and each lane validates one slot; with K > 64 a row takes a whole
// wave and each lane walks slots lane, lane + 64, ...  (One row per thread
// walking its K slots had each wave serialise K rounds of branches and
// scattered stores; a loop over several row groups per workgroup was slower
// than more workgroups.)  A workgroup's 16 rpw rows, a power of two <= 256,
// lie within one ordering slice (slice_rows is a multiple of 256).  The
// workgroup takes its list positions in (slot, row) order.  The order in
// which a list's entries reach the partial-output slabs matters to the
// attention kernel's write stream: blocks of 64 rows in that order (1024
// threads at K = 16) gave 4-5 % faster attention on the 4 x 4096 BF16
// workload than blocks of 16 rows (256 threads).
constexpr int kCountThreads = 1024;
constexpr int kClaimBatch = 8;           // list claims (returning atomics) in flight per thread

// log2 of the rows per wave for K slots: the most rows of K lanes that fit
// in 64, at most 16.
__host__ __device__ inline int count_rpw_log2(int K) {
  int l = 0;
  while (l < 4 && K <= 32 >> l) ++l;
  return l;
}

template <bool LDS_HIST, int NT>
__global__ void __launch_bounds__(NT) plan_count(const PageArgs a) {
  extern __shared__ int32_t hist[];
  const int64_t L = a.lists_per_slice;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.num_slots;
  const int lpr = min(K, 64);  // lanes per row
  const int rpw = 1 << count_rpw_log2(K);
  const int64_t row0 = (int64_t)blockIdx.x * (NT / 64) * rpw;
  const int64_t lbase = row0 / a.slice_rows * L;
  const int64_t rows = (int64_t)a.total_q * a.Hkv;
  int32_t *counts = (int32_t *)(a.ws + a.lay.counts);
  int32_t *slot_list_all = (int32_t *)(a.ws + a.lay.slot_list);
  int32_t *slot_pos_all = (int32_t *)(a.ws + a.lay.slot_pos);
  // empty splits get lse = -inf for the G heads of the row, 16 bytes at a
  // time where the layout allows
  const bool lse4 = ((uintptr_t)a.partial_lse & 15) == 0 && (a.pl_split_stride & 3) == 0 &&
                    (a.Hq & 3) == 0 && (a.G & 3) == 0;
  if constexpr (LDS_HIST) {
    for (int64_t i = tid; i < L; i += NT) hist[i] = 0;
    __syncthreads();
  }
  const int rr = lane / lpr, j0 = lane - rr * lpr;  // row in the wave, first slot
  const int RW = (NT / 64) * rpw;                    // rows of the workgroup
  __shared__ int32_t s_q[NT];  // K <= 64: (slot, row) -> list, then -> position (K RW <= NT)
  int lr = -1, pr = 0;         // K <= 64: this lane's list (local, -1: none) and position
  {
    const int64_t idx = row0 + (int64_t)wave * rpw + rr;
    const bool live = rr < rpw && idx < rows;
    const int64_t ridx = live ? idx : 0;  // dead lanes read row 0 (rows >= 1 when launched)
    const int r = (int)(ridx / a.Hkv), g = (int)(ridx - (int64_t)r * a.Hkv);
    const int32_t *sidx = a.sel_idx + r * a.sel_stride_tok + g * a.sel_stride_head;
    const uint8_t *smask = a.sel_mask + r * a.sel_stride_tok + g * a.sel_stride_head;
    int32_t *slot_list = slot_list_all + ridx * K;
    int32_t *slot_pos = slot_pos_all + ridx * K;
    uint32_t err = 0;
    const RowCtx c = row_ctx(a, r, err);
    const int bb = c.valid ? c.b : 0;  // an in-bounds table row for the loads below
    // slot j: validate, find its list (local index, -1: none) and record it
    // -- or mark the split empty
    auto visit = [&](int j, uint32_t mk, int u, bool dup, int pp) -> int {
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
      if (list < 0) {
        float *pl = a.partial_lse + j * a.pl_split_stride + (int64_t)r * a.Hq + g * a.G;
        if (lse4) {
          for (int h = 0; h < a.G; h += 4) *(float4 *)(pl + h) = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        } else {
          for (int h = 0; h < a.G; ++h) pl[h] = -INFINITY;
        }
      }
      return list;
    };
    if (K <= 64) {
      uint32_t mk = smask[j0];
      int u = sidx[j0];
      pin(mk);
      pin(u);
      const int uc = (u >= 0 && u < a.max_pages) ? u : 0;
      const int pp = a.page_table[bb * a.pt_stride + uc];
      // duplicate: an earlier slot of the row with a mask and the same page
      // (all lanes shuffle; a row's lanes live or die together)
      const int key = mk ? u : INT_MIN;
      const int rb = rr * lpr;
      bool dup = false;
      for (int jj = 0; jj + 1 < lpr; ++jj) {
        const int kj = __shfl(key, (rb + jj) & 63);
        dup |= jj < j0 && kj == u;
      }
      if (live) lr = visit(j0, mk, u, dup, pp);
      if (!LDS_HIST && lr >= 0) slot_pos[j0] = atomicAdd(&counts[lbase + lr], 1);
      if (LDS_HIST && rr < rpw) s_q[j0 * RW + wave * rpw + rr] = lr;
    } else if (live) {
      // one row per wave (rr = 0); lane j0 takes slots j0, j0 + 64, ...
      for (int j = j0; j < K; j += 64) {
        const uint32_t mk = smask[j];
        const int u = sidx[j];
        bool dup = false;
        for (int jj = 0; jj < j; ++jj) dup |= (smask[jj] != 0) && (sidx[jj] == u);
        const int uc = (u >= 0 && u < a.max_pages) ? u : 0;
        const int list = visit(j, mk, u, dup, a.page_table[bb * a.pt_stride + uc]);
        if (list >= 0) slot_pos[j] = LDS_HIST ? atomicAdd(&hist[list], 1) : atomicAdd(&counts[lbase + list], 1);
      }
    }
    if (live && err) atomicOr(a.err_flags, err);
  }
  if constexpr (LDS_HIST) {
    if (K <= 64) {
      // positions in the workgroup's blocks, taken by one wave walking the
      // slots in (slot, row) order: a list's entries then come slot by slot,
      // rows ascending
      __syncthreads();
      if (wave == 0) {
        for (int q = lane; q < K * RW; q += 64) {
          const int l = s_q[q];
          if (l >= 0) s_q[q] = atomicAdd(&hist[l], 1);
        }
      }
      __syncthreads();
      if (lr >= 0) pr = s_q[j0 * RW + wave * rpw + rr];
    }
    __syncthreads();
    // this workgroup's block of each list it touches: the returning atomics
    // go out kClaimBatch at a time, so their round trips overlap
    for (int64_t i0 = tid; i0 < L; i0 += (int64_t)NT * kClaimBatch) {
      int32_t n[kClaimBatch], o[kClaimBatch];
#pragma unroll
      for (int b = 0; b < kClaimBatch; ++b) {
        const int64_t i = i0 + (int64_t)b * NT;
        n[b] = i < L ? hist[i] : 0;
      }
#pragma unroll
      for (int b = 0; b < kClaimBatch; ++b)
        o[b] = n[b] ? atomicAdd(&counts[lbase + i0 + (int64_t)b * NT], n[b]) : 0;
#pragma unroll
      for (int b = 0; b < kClaimBatch; ++b)
        if (n[b]) hist[i0 + (int64_t)b * NT] = o[b];
    }
    __syncthreads();
    // positions within the workgroup's blocks -> within the lists
    const int64_t idx = row0 + (int64_t)wave * rpw + rr;
    if (K <= 64) {
      if (lr >= 0) slot_pos_all[idx * K + j0] = pr + hist[lr];
    } else if (rr < rpw && idx < rows) {
      for (int j = j0; j < K; j += 64) {  // (the slot records this thread wrote, read back)
        const int list = slot_list_all[idx * K + j];
        if (list >= 0) slot_pos_all[idx * K + j] += hist[list - lbase];
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
// ceil(n / chunk) by a multiply: a list holds at most total_q < 2^23 entries,
// so x = n + chunk - 1 < 2^24, and x * ceil(2^32 / chunk) / 2^32 exceeds
// x / chunk by less than x / 2^32 < 1 / chunk -- too little to reach the
// next integer.
__device__ __forceinline__ int units_of(const PageArgs &a, int32_t n) {
  return (int)(((uint64_t)(uint32_t)(n + a.chunk - 1) * a.chunk_magic) >> 32);
}
__device__ __forceinline__ bool classed(const PageArgs &a) { return a.lay.num_lists == a.lists_per_slice; }
// Class of a list of n entries in u units: s = floor(n / max(1, u)) entries
// per unit against chunk/2, chunk/4, chunk/8.  For integer s and k,
// k s >= chunk exactly when s >= ceil(chunk / k), i.e. n >= u ceil(chunk / k).
__device__ __forceinline__ int size_class(const PageArgs &a, int32_t n, int32_t u) {
  if (!classed(a)) return 0;
  const int32_t v = max(1, u);
  return n >= v * ((a.chunk + 1) >> 1) ? 0 : (n >= v * ((a.chunk + 3) >> 2) ? 1 : (n >= v * ((a.chunk + 7) >> 3) ? 2 : 3));
}

// Per-class unit counts of one thread's lists, and its running offsets.
struct ClassCounts {
  int32_t v[kSizeClasses];
};

// Up to kScanOneBlockMax lists: one workgroup scans them all, PER lists per
// thread -- inclusive scans within each wave by shuffles, the wave totals
// through LDS behind a single barrier -- and writes the final offsets:
// list_off (entries) in list order, unit_off (the list's first unit) in
// (size class, list) order.  Thread t scans lists [PER t, PER t + PER), but
// global memory is read and written through an LDS transpose (element
// k * threads + t by thread t): per-thread runs of PER words gave every load
// and store instruction 64 scattered words, and the one workgroup's CU spent
// most of the kernel issuing them.
// NC = kSizeClasses with one ordering slice, else 1 (every unit in class 0:
// the class sums then cost nothing).
template <int PER, int NC>
__global__ void __launch_bounds__(kScanThreads) plan_scan_one(const PageArgs a) {
  constexpr int NW = kScanThreads / 64;
  __shared__ int32_t w_e[NW], w_u[NC][NW];
  __shared__ int32_t s_x[kScanThreads * PER];  // the transpose buffer
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t L = a.lay.num_lists;
  const int32_t *counts = (const int32_t *)(a.ws + a.lay.counts);
  int32_t *list_off = (int32_t *)(a.ws + a.lay.list_off);
  int32_t *unit_off = (int32_t *)(a.ws + a.lay.unit_off);
  int32_t c[PER], cls[PER], nun[PER];
  // unconditional loads (clamped index; L >= 1), all in flight at once;
  // lists past L count 0
#pragma unroll
  for (int k = 0; k < PER; ++k) c[k] = counts[min((int64_t)k * kScanThreads + t, L - 1)];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    pin(c[k]);
    s_x[k * kScanThreads + t] = (int64_t)k * kScanThreads + t < L ? c[k] : 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; ++k) c[k] = s_x[t * PER + k];
  int32_t se = 0;
  ClassCounts su = {};
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    se += c[k];
    nun[k] = units_of(a, c[k]);
    cls[k] = NC == 1 ? 0 : size_class(a, c[k], nun[k]);
#pragma unroll
    for (int q = 0; q < NC; ++q) su.v[q] += q == cls[k] ? nun[k] : 0;
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
  // unit offsets through the buffer (each thread rewrites only its own run,
  // which only it has read), then the entry offsets
  int32_t eo[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    int32_t uo = bu.v[0];
#pragma unroll
    for (int q = 1; q < NC; ++q) uo = q == cls[k] ? bu.v[q] : uo;
    s_x[t * PER + k] = uo;
    eo[k] = be;
    be += c[k];
#pragma unroll
    for (int q = 0; q < NC; ++q) bu.v[q] += q == cls[k] ? nun[k] : 0;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if ((int64_t)k * kScanThreads + t < L) unit_off[k * kScanThreads + t] = s_x[k * kScanThreads + t];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; ++k) s_x[t * PER + k] = eo[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if ((int64_t)k * kScanThreads + t < L) list_off[k * kScanThreads + t] = s_x[k * kScanThreads + t];
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
  int32_t c[PER], cls[PER], nun[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) c[k] = counts[min(i0 + k, L - 1)];
  int32_t se = 0;
  ClassCounts su = {};
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    pin(c[k]);
    c[k] = i0 + k < L ? c[k] : 0;
    se += c[k];
    nun[k] = units_of(a, c[k]);
    cls[k] = NC == 1 ? 0 : size_class(a, c[k], nun[k]);
#pragma unroll
    for (int q = 0; q < NC; ++q) su.v[q] += q == cls[k] ? nun[k] : 0;
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
    int32_t uo = bu.v[0];
#pragma unroll
    for (int q = 1; q < NC; ++q) uo = q == cls[k] ? bu.v[q] : uo;
    if (i0 + k < L) {
      list_off[i0 + k] = be;
      unit_off[i0 + k] = uo;
    }
    be += c[k];
#pragma unroll
    for (int q = 0; q < NC; ++q) bu.v[q] += q == cls[k] ? nun[k] : 0;
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
      const int32_t n = counts[i0 + k];
      const int cl = size_class(a, n, units_of(a, n));
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
  // the list's entries split evenly: the first n % nu units take one more
  const int32_t nu = units_of(a, n), q = n / nu, rem = n - q * nu;
  int32_t b0 = lo;
  for (int32_t c = 0; c < nu; ++c) {
    w.e_begin = b0;
    w.e_count = q + (c < rem ? 1 : 0);
    b0 += w.e_count;
    units[c] = w;
  }
}

// Blocks [0, fill_blocks): the rows' slots, one per lane as in plan_count
// (K <= 64: K adjacent lanes per row; else a wave per row, each lane taking
// every 64th slot); the blocks after them: one list per thread, its units.
__global__ void __launch_bounds__(kPlanThreads) plan_fill(const PageArgs a, int fill_blocks) {
  if ((int)blockIdx.x >= fill_blocks) {
    write_units(a, (int64_t)(blockIdx.x - fill_blocks) * kPlanThreads + threadIdx.x);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.num_slots, lpr = min(K, 64);
  const int rpw = 1 << count_rpw_log2(K);
  const int rr = lane / lpr, j0 = lane - rr * lpr;
  const int64_t idx = ((int64_t)blockIdx.x * (kPlanThreads / 64) + wave) * rpw + rr;
  if (rr >= rpw || idx >= (int64_t)a.total_q * a.Hkv) return;
  const int r = (int)(idx / a.Hkv), g = (int)(idx - (int64_t)r * a.Hkv);
  const int32_t *sidx = a.sel_idx + r * a.sel_stride_tok + g * a.sel_stride_head;
  const int32_t *slot_list = (const int32_t *)(a.ws + a.lay.slot_list) + idx * K;
  const int32_t *slot_pos = (const int32_t *)(a.ws + a.lay.slot_pos) + idx * K;
  const int32_t *list_off = (const int32_t *)(a.ws + a.lay.list_off);
  PlanEntry *entries = (PlanEntry *)(a.ws + a.lay.entries);
  uint32_t err = 0;
  const RowCtx c = row_ctx(a, r, err);
  for (int j = j0; j < K; j += 64) {
    const int list = slot_list[j];
    if (list < 0) continue;
    PlanEntry e;
    e.tok_slot = (r << 8) | j;
    e.limit = min(c.last - sidx[j] * a.page_size, a.page_size - 1);
    entries[list_off[list] + slot_pos[j]] = e;
  }
}

}  // namespace

size_t page_plan_lds_bytes() { return (size_t)kMaxLdsLists * 4 + kCountThreads * 4; }  // plan_count

hipError_t launch_page_plan(const PageArgs &a, hipStream_t s) {
  int32_t *counts = (int32_t *)(a.ws + a.lay.counts);
  const int64_t L = a.lay.num_lists;  // all slices
  const int64_t zero_blocks = (L + 255) / 256 > 0 ? (L + 255) / 256 : 1;
  plan_zero<<<(unsigned)zero_blocks, 256, 0, s>>>(counts, L, a.err_flags);
  const int64_t rows = (int64_t)a.total_q * a.Hkv;
  auto row_blocks = [&](int64_t per) { return (unsigned)((rows + per - 1) / per); };
  const unsigned blocks = row_blocks((int64_t)(kPlanThreads / 64) << count_rpw_log2(a.num_slots));
  if (rows > 0) {
    const size_t hist_bytes = (size_t)a.lists_per_slice * 4;
    const unsigned cblocks = row_blocks((kCountThreads / 64) << count_rpw_log2(a.num_slots));
    if (a.lists_per_slice > kMaxLdsLists)
      plan_count<false, kCountThreads><<<cblocks, kCountThreads, 0, s>>>(a);
    else
      plan_count<true, kCountThreads><<<cblocks, kCountThreads, hist_bytes, s>>>(a);
  }
  const bool cl = L == a.lists_per_slice;  // one ordering slice: units by size class
  if (L <= kScanTile) {
    if (cl) plan_scan_one<kScanPer, kSizeClasses><<<1, kScanThreads, 0, s>>>(a);
    else plan_scan_one<kScanPer, 1><<<1, kScanThreads, 0, s>>>(a);
  } else if (L <= kScanOneBlockMax) {
    if (cl) plan_scan_one<kScanOneBlockMax / kScanThreads, kSizeClasses><<<1, kScanThreads, 0, s>>>(a);
    else plan_scan_one<kScanOneBlockMax / kScanThreads, 1><<<1, kScanThreads, 0, s>>>(a);
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
