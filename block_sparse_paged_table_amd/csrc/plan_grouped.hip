// Planner of the grouped microblock route (1Cat-vLLM PR 387, section
// "Purpose"; 1Cat-vLLM PR 1236, section "Purpose").  It turns each group's
// logical selections into the list of physical 4-token units the attention
// kernel loads once for all rows of the group.  On the GPU and
// deterministically, it drops any selection it cannot honour (a padding
// row, a request id outside the batch, a unit past the request's table row
// or its tail, a table entry outside the cache) and flags it.  Each unit
// carries the row tiles that use it, so a tile with nothing in a batch of
// units skips it.  The union of a group is bounded by its 8 rows times their
// slots, and the order of the list is a function of the splits and the
// logical units alone, never of scheduling.
//
// One workgroup per (group of kGroupTokens consecutive query tokens, KV head):
//   1. every (token, slot) selection becomes a 64-bit key
//        request:16 | unit:24 | token-in-group:3 | slot:10 | visible bits:4
//      (bits 41.. | 17.. | 14.. | 4.. | 0..)
//      (invalid selections sort to the end);
//   2. bitonic sort of the keys in LDS (or, for one request, steps 2-4
//      through bitmaps of the request's units and of the (split, unit)
//      entries: see union_one_split_by_bitmap and union_by_bitmap);
//   3. duplicates of a (request, unit, token) beyond the first slot are
//      dropped and flagged; the first slot of each (request, unit, token)
//      names its split (slot / slots_per_split); each distinct (split,
//      request, unit) gets a 32-bit mask, 4 visible-token bits per token of
//      the group; units no row sees are dropped; the physical page is looked
//      up and checked;
//   4. the union is ordered by (split, request, unit): each split's units
//      are contiguous, and within a split the units ascend, so the groups an
//      XCD runs together walk the cache in step and share its L2;
//   5. the group's list is written, 8 bytes per unit: its physical page and
//      its index inside the page (page << 5 | unit), and its mask32; then
//      the offsets of the splits' runs in the list.
#include "grouped.h"

namespace msa {
namespace {

constexpr uint64_t kInvalidKey = ~0ull;
constexpr int kBitmapUnits = 65535;          // largest unit count the bitmap pass takes
constexpr int64_t kBitmapPassWords = 15360;   // and its LDS budget (60 KiB) with many planner
                                               // workgroups (256 threads)
constexpr int64_t kBitmapPassWordsFew = 28672; // with at most 256 of them (1024 threads, a
                                               // latency-bound grid): 112 KiB, room for
                                               // 64 splits of 64 slots
template <int NT> constexpr int64_t bitmap_budget() {
  return NT == kGPlanThreadsFew ? kBitmapPassWordsFew : kBitmapPassWords;
}

// Ascending bitonic sort of n = E * blockDim.x keys held in LDS.  Thread t
// keeps the keys of sorted positions tE .. tE+E-1 in registers: compare-
// exchange steps whose partner lies within the thread (stride < E) run in
// registers, those whose partner thread is in the same wave (stride < 64 E)
// through cross-lane shuffles, the others through LDS; every thread computes
// its own new key.  During the sort the LDS copy is laid out position p -> slot
// (p % E) * nt + p / E, so a wave's accesses hit consecutive slots; the
// input is taken in that layout too (any input order sorts the same).  The
// result is written back in sorted order with one padding slot after each
// thread's E keys (position p at p + p / E, see sorted_at): a thread that
// then walks its own E consecutive positions has its lanes 8 * (E + 1)
// bytes apart, at most two to an LDS bank, instead of E / 2.
template <int E, typename T>
__device__ __forceinline__ void bitonic_core(T *k, int n, T (&r)[E]) {
  const int t = threadIdx.x, nt = blockDim.x;
  const int base = t * E;
  // sizes up to E: within the thread's registers; base is a multiple of E,
  // so the direction of position base + i is fixed by i (compile time) below
  // size E and by base at size E
#pragma unroll
  for (int size = 2; size <= E; size <<= 1) {
#pragma unroll
    for (int st = size >> 1; st >= 1; st >>= 1) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if (i & st) continue;
        const int j = i | st;
        const bool up = size < E ? (i & size) == 0 : (base & size) == 0;
        const T x = r[i], y = r[j];
        const bool sw = (x > y) == up;
        r[i] = sw ? y : x;
        r[j] = sw ? x : y;
      }
    }
  }
  for (int size = 2 * E; size <= n; size <<= 1) {
    // every position of the thread has the direction of its block, (base &
    // size) == 0, as size > E > i
    const bool up = (base & size) == 0;
    for (int stride = size >> 1; stride >= E; stride >>= 1) {
      const int m = stride / E;  // the partner thread is t ^ m (same register i)
      // Position p = base + i, partner p ^ stride: as stride >= E > i, whether
      // p is the lower of the pair (bit `stride` clear) depends on base only,
      // so every register of the thread keeps the minimum, or every one the
      // maximum.  It keeps its own key exactly when (own < partner) ==
      // keep_min (equal keys are interchangeable: valid keys are distinct,
      // invalid ones all-ones).
      const bool keep_min = ((base & stride) == 0) == up;
      if (m < kWave) {
        // partner in this wave: a cross-lane shuffle, no LDS round trip and
        // no barrier (the wave's lanes run in lockstep)
#pragma unroll
        for (int i = 0; i < E; ++i) {
          T o;
          if constexpr (sizeof(T) == 8) {
            const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)r[i], m);
            const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)((uint64_t)r[i] >> 32), m);
            o = (T)(((uint64_t)hi << 32) | lo);
          } else {
            o = (T)__shfl_xor((int)r[i], m);
          }
          r[i] = ((r[i] < o) == keep_min) ? r[i] : o;
        }
        continue;
      }
      __syncthreads();  // everyone is done reading the previous round
#pragma unroll
      for (int i = 0; i < E; ++i) k[i * nt + t] = r[i];
      __syncthreads();
      const int tq = t ^ m;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const T o = k[i * nt + tq];
        r[i] = ((r[i] < o) == keep_min) ? r[i] : o;
      }
    }
    // strides below E: partners in this thread's registers (compile-time
    // indices, so the keys stay in registers)
#pragma unroll
    for (int st = E >> 1; st >= 1; st >>= 1) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if (i & st) continue;
        const int j = i | st;
        const T x = r[i], y = r[j];
        const bool sw = (x > y) == up;
        r[i] = sw ? y : x;
        r[j] = sw ? x : y;
      }
    }
  }
}


// 64-bit keys: loaded from, exchanged through and written back to k.
template <int E>
__device__ __forceinline__ void bitonic_sort_e(uint64_t *k, int n) {
  uint64_t r[E];
  const int t = threadIdx.x, nt = blockDim.x;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) r[i] = k[i * nt + t];
  bitonic_core<E, uint64_t>(k, n, r);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) k[t * E + t + i] = r[i];
  __syncthreads();
}

// The same sort of 64-bit keys that map one-to-one, order-preserving, onto
// 32-bit keys (narrow; invalid keys onto all-ones, which no valid key takes):
// run on the 32-bit keys (half the compares, selects and exchanges), then
// written back widened (wide).
template <int E, typename Narrow, typename Wide>
__device__ __forceinline__ void bitonic_sort_e32(uint64_t *k, int n, Narrow narrow, Wide wide) {
  uint32_t r[E];
  const int t = threadIdx.x, nt = blockDim.x;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) r[i] = narrow(k[i * nt + t]);
  bitonic_core<E, uint32_t>((uint32_t *)k, n, r);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) k[t * E + t + i] = r[i] == ~0u ? kInvalidKey : wide(r[i]);
  __syncthreads();
}

// Sorted position p of a bitonic_sort whose threads held 2^sh keys each.
__device__ __forceinline__ uint64_t sorted_at(const uint64_t *k, int sh, int p) {
  return k[p + (p >> sh)];
}

// n: a power of two in [blockDim.x, 16 * blockDim.x]; k holds n + blockDim.x
// keys (the sorted output is padded)
__device__ __forceinline__ void bitonic_sort(uint64_t *k, int n) {
  switch (n / (int)blockDim.x) {
    case 1: bitonic_sort_e<1>(k, n); break;
    case 2: bitonic_sort_e<2>(k, n); break;
    case 4: bitonic_sort_e<4>(k, n); break;
    case 8: bitonic_sort_e<8>(k, n); break;
    default: bitonic_sort_e<16>(k, n); break;
  }
}
template <typename Narrow, typename Wide>
__device__ __forceinline__ void bitonic_sort32(uint64_t *k, int n, Narrow narrow, Wide wide) {
  switch (n / (int)blockDim.x) {
    case 1: bitonic_sort_e32<1>(k, n, narrow, wide); break;
    case 2: bitonic_sort_e32<2>(k, n, narrow, wide); break;
    case 4: bitonic_sort_e32<4>(k, n, narrow, wide); break;
    case 8: bitonic_sort_e32<8>(k, n, narrow, wide); break;
    default: bitonic_sort_e32<16>(k, n, narrow, wide); break;
  }
}

// Exclusive prefix of v over the workgroup's threads, and the total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int &total) {
  __shared__ int wsum[NT / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  __syncthreads();  // wsum free (an earlier scan may still read it)
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    before += k < w ? wsum[k] : 0;
    total += wsum[k];
  }
  return before + x - v;
}

// LDS words the bitmap pass needs (sizing on the host and checks here).
__host__ __device__ inline int64_t bitmap_pass_words(int64_t nunits, int64_t cap, int64_t splits) {
  const int64_t nw = (nunits + 31) / 32, pw = (cap + 31) / 32;
  if (splits == 1) return 2 * nw + 2 * cap + kGroupTokens * pw;  // union_one_split_by_bitmap
  return 2 * nw + 2 * ((cap + 1) / 2) + 2 * splits * pw + cap + kGroupTokens * pw;
}

// The union of a group whose valid rows belong to one request, with units
// below 2^16 (contexts up to 256K tokens), without sorting.  Two levels of
// bitmaps: one over the request's units gives each selected unit its rank in
// ascending unit order; one over (split, rank) pairs, split-major, gives each
// list entry its place in (split, unit) order -- the order the sort gives.
// Each (token, unit) ORs its visible bits into its entry's mask word.  A
// per-token presence bitmap over the ranks catches a token that selected a
// unit twice (in any splits): then the kernel falls back to the sort, which
// applies the first-slot rule (returns false).  Entries no row sees (mask
// 0) are dropped, as by the sort path; the list and split offsets it writes
// are the same.  LDS (the keys array, reused): bitmap_pass_words words.
template <int NT, int JI>
__device__ __forceinline__ bool union_by_bitmap(const GroupArgs &a, const uint64_t (&kr)[kGroupTokens][JI],
                                                int b0, int nunits, uint2 *out, int *soff, uint32_t &err) {
  extern __shared__ uint64_t keys[];
  const int t = threadIdx.x;
  const int S = a.num_splits;
  const int nw = (nunits + 31) >> 5;   // <= 2048
  const int cap = a.list_cap;          // bound on the union and on the entries
  const int pw = (cap + 31) >> 5;      // words of a rank bitmap
  const int sw = S * pw;               // words of the (split, rank) bitmap
  uint32_t *ubm = (uint32_t *)keys;    // units
  uint32_t *upre = ubm + nw;           // ranks before each unit word
  uint16_t *uor = (uint16_t *)(upre + nw);  // unit of each rank
  uint32_t *ebm = upre + nw + (cap + 1) / 2;  // (split, rank) entries
  uint32_t *epre = ebm + sw;           // entries before each entry word
  uint32_t *msk = epre + sw;           // mask of each entry
  uint32_t *pres = msk + cap;          // (token, rank) presence
  uint16_t *erank = (uint16_t *)(pres + kGroupTokens * pw);  // rank of each entry
  const uint32_t split_mul = ((1u << 20) + (uint32_t)a.slots_per_split - 1u) / (uint32_t)a.slots_per_split;
  auto split_of = [&](uint64_t k) { return (int)((((uint32_t)(k >> 4) & 0x3ffu) * split_mul) >> 20); };
  auto below = [](uint32_t w, uint32_t bit) { return (uint32_t)__popc(w & ((1u << bit) - 1u)); };
  for (int e = t; e < nw; e += NT) ubm[e] = 0u;
  for (int e = t; e < sw; e += NT) ebm[e] = 0u;
  for (int e = t; e < cap; e += NT) msk[e] = 0u;
  for (int e = t; e < kGroupTokens * pw; e += NT) pres[e] = 0u;
  __syncthreads();
  // the selected units
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau)
#pragma unroll
    for (int i = 0; i < JI; ++i) {
      const uint64_t k = kr[tau][i];
      if (k == kInvalidKey) continue;
      const uint32_t u = (uint32_t)(k >> 17) & 0xffffu;
      atomicOr(&ubm[u >> 5], 1u << (u & 31u));
    }
  __syncthreads();
  // unit ranks: thread t takes words [t * wpt, t * wpt + wpt)
  {
    const int wpt = (nw + NT - 1) / NT;
    const int w0 = min(t * wpt, nw), w1 = min(w0 + wpt, nw);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(ubm[w]);
    int nunion;
    int run = block_exclusive_scan<NT>(cnt, nunion);
    for (int w = w0; w < w1; ++w) {
      upre[w] = (uint32_t)run;
      for (uint32_t bits = ubm[w]; bits; bits &= bits - 1u) uor[run++] = (uint16_t)(w * 32 + __builtin_ctz(bits));
    }
  }
  __syncthreads();
  // presence of (token, rank): a token meeting a unit twice is a duplicate;
  // the (split, rank) entries
  bool dup = false;
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau)
#pragma unroll
    for (int i = 0; i < JI; ++i) {
      const uint64_t k = kr[tau][i];
      if (k == kInvalidKey) continue;
      const uint32_t u = (uint32_t)(k >> 17) & 0xffffu;
      const uint32_t r = upre[u >> 5] + below(ubm[u >> 5], u & 31u);
      const uint32_t bit = 1u << (r & 31u);
      if (atomicOr(&pres[tau * pw + (r >> 5)], bit) & bit) dup = true;
      atomicOr(&ebm[split_of(k) * pw + (r >> 5)], bit);
    }
  if (__syncthreads_or(dup)) return false;
  // entry positions
  const int wpt = (sw + NT - 1) / NT;
  const int w0 = min(t * wpt, sw), w1 = min(w0 + wpt, sw);
  {
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(ebm[w]);
    int nent;
    int run = block_exclusive_scan<NT>(cnt, nent);
    for (int w = w0; w < w1; ++w) {
      epre[w] = (uint32_t)run;
      for (uint32_t bits = ebm[w]; bits; bits &= bits - 1u)
        erank[run++] = (uint16_t)((w % pw) * 32 + __builtin_ctz(bits));
    }
  }
  __syncthreads();
  // visible bits of each (token, unit) into its entry's mask
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau)
#pragma unroll
    for (int i = 0; i < JI; ++i) {
      const uint64_t k = kr[tau][i];
      const uint32_t vis = (uint32_t)k & 0xfu;
      if (k == kInvalidKey || vis == 0u) continue;
      const uint32_t u = (uint32_t)(k >> 17) & 0xffffu;
      const uint32_t r = upre[u >> 5] + below(ubm[u >> 5], u & 31u);
      const int ew = split_of(k) * pw + (int)(r >> 5);
      atomicOr(&msk[epre[ew] + below(ebm[ew], r & 31u)], vis << (4 * tau));
    }
  __syncthreads();
  // entries with a visible key, in entry order; split s starts at entry word
  // s * pw, and the thread holding that word records its output offset
  int nz = 0;
  for (int w = w0; w < w1; ++w) {
    const int p0 = (int)epre[w], n = __popc(ebm[w]);
    for (int q = p0; q < p0 + n; ++q) nz += msk[q] != 0u;
  }
  int total;
  int o = block_exclusive_scan<NT>(nz, total);
  const int upp = a.page_size / a.unit_tokens;  // units per page
  const int32_t *ptrow = a.page_table + (int64_t)max(b0, 0) * a.pt_stride;
  if (total == (int)epre[sw - 1] + __popc(ebm[sw - 1])) {
    // (the usual case) no entry drops out: output e is entry e, written by
    // thread e mod NT -- four page-table loads in flight per thread, and
    // each wave's stores one contiguous run
    for (int e0 = t; e0 < total; e0 += 4 * NT) {
      int uu[4], phys[4];
      uint32_t mm[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int ec = min(e0 + x * NT, total - 1);
        uu[x] = uor[erank[ec]];
        mm[x] = msk[ec];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) phys[x] = ptrow[uu[x] / upp];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if (e0 + x * NT >= total) continue;
        uint2 e;
        if (phys[x] < 0 || phys[x] >= a.num_phys_pages) {
          err |= MSA_ERRF_PHYS_RANGE;
          e = make_uint2(0u, 0u);  // mask 0: contributes nothing
        } else {
          e = make_uint2(((uint32_t)phys[x] << 5) | (uint32_t)(uu[x] % upp), mm[x]);
        }
        out[e0 + x * NT] = e;
      }
    }
    for (int sp = t; sp < S; sp += NT) soff[sp] = (int)epre[sp * pw];
    if (t == 0) soff[S] = total;
    return true;
  }
  for (int w = w0; w < w1; ++w) {
    if (w % pw == 0) soff[w / pw] = o;
    uint32_t bits = ebm[w];
    int q = (int)epre[w];
    const int rbase = (w % pw) * 32;
    while (bits) {
      // up to 8 entries at a time: their page-table loads first, then the writes
      int uu[8], phys[8];
      uint32_t mm[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        uu[x] = -1;
        mm[x] = 0u;
        if (bits) {
          const int r = rbase + __builtin_ctz(bits);
          bits &= bits - 1u;
          uu[x] = uor[r];
          mm[x] = msk[q++];
        }
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) phys[x] = (uu[x] >= 0 && mm[x] != 0u) ? ptrow[uu[x] / upp] : 0;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        if (uu[x] < 0 || mm[x] == 0u) continue;
        uint2 e;
        if (phys[x] < 0 || phys[x] >= a.num_phys_pages) {
          err |= MSA_ERRF_PHYS_RANGE;
          e = make_uint2(0u, 0u);  // mask 0: contributes nothing
        } else {
          e = make_uint2(((uint32_t)phys[x] << 5) | (uint32_t)(uu[x] % upp), mm[x]);
        }
        out[o++] = e;
      }
    }
  }
  if (t == 0) soff[S] = total;
  return true;
}

// One split: the same in one level.  The union of a group whose valid rows
// belong to one request, with units below 2^16, without sorting: a bitmap of the request's
// units marks the selected ones, so the union comes out in ascending unit
// order (the order the sort gives) with a unit's rank = the set bits below
// it; each (token, unit) ORs its visible bits into the unit's mask word.  A
// per-token presence bitmap over the ranks catches a token that selected a
// unit twice: then the kernel falls back to the sort, which applies the
// first-slot rule (returns false).  Units no row sees (mask 0) are dropped,
// as by the sort path; the list and split offsets it writes are the same.
// LDS (the keys array, reused): bitmap and rank bases of ceil(nunits / 32)
// words each, a mask word and a unit id per union entry and 8 presence bits
// per entry.
template <int NT, int JI>
__device__ __forceinline__ bool union_one_split_by_bitmap(const GroupArgs &a, const uint64_t (&kr)[kGroupTokens][JI],
                                                int b0, int nunits, uint2 *out, int *soff, uint32_t &err) {
  extern __shared__ uint64_t keys[];
  const int t = threadIdx.x;
  const int nw = (nunits + 31) >> 5;   // <= 2048
  const int cap = a.list_cap;          // bound on the union
  const int pw = (cap + 31) >> 5;      // presence words per token
  uint32_t *bm = (uint32_t *)keys;
  uint32_t *pre = bm + nw;
  uint32_t *msk = pre + nw;
  uint32_t *pres = msk + cap;
  uint32_t *uor = pres + kGroupTokens * pw;  // unit of each rank
  for (int e = t; e < nw; e += NT) bm[e] = 0u;
  for (int e = t; e < cap; e += NT) msk[e] = 0u;
  for (int e = t; e < kGroupTokens * pw; e += NT) pres[e] = 0u;
  __syncthreads();
  // the selected units
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau)
#pragma unroll
    for (int i = 0; i < JI; ++i) {
      const uint64_t k = kr[tau][i];
      if (k == kInvalidKey) continue;
      const uint32_t u = (uint32_t)(k >> 17) & 0xffffffu;
      atomicOr(&bm[u >> 5], 1u << (u & 31u));
    }
  __syncthreads();
  // rank bases: thread t takes words [t * wpt, t * wpt + wpt)
  const int wpt = (nw + NT - 1) / NT;
  const int w0 = min(t * wpt, nw), w1 = min(w0 + wpt, nw);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  int nunion;
  const int base = block_exclusive_scan<NT>(cnt, nunion);
  {
    int run = base;
    for (int w = w0; w < w1; ++w) {
      pre[w] = (uint32_t)run;
      for (uint32_t bits = bm[w]; bits; bits &= bits - 1u) uor[run++] = (uint32_t)(w * 32 + __builtin_ctz(bits));
    }
  }
  __syncthreads();
  // visible bits per (unit, token); a token meeting a unit twice is a duplicate
  bool dup = false;
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau)
#pragma unroll
    for (int i = 0; i < JI; ++i) {
      const uint64_t k = kr[tau][i];
      if (k == kInvalidKey) continue;
      const uint32_t u = (uint32_t)(k >> 17) & 0xffffffu;
      const uint32_t rank = pre[u >> 5] + (uint32_t)__popc(bm[u >> 5] & ((1u << (u & 31u)) - 1u));
      const uint32_t bit = 1u << (rank & 31u);
      if (atomicOr(&pres[tau * pw + (rank >> 5)], bit) & bit) dup = true;
      const uint32_t vis = (uint32_t)k & 0xfu;
      if (vis) atomicOr(&msk[rank], vis << (4 * tau));
    }
  if (__syncthreads_or(dup)) return false;
  // entries with a visible key, in rank order: thread t's ranks are those of
  // its words
  int nz = 0;
  for (int w = w0; w < w1; ++w) {
    const int r0 = (int)pre[w], n = __popc(bm[w]);
    for (int r = r0; r < r0 + n; ++r) nz += msk[r] != 0u;
  }
  int total;
  int o = block_exclusive_scan<NT>(nz, total);
  const int upp = a.page_size / a.unit_tokens;  // units per page
  const int32_t *ptrow = a.page_table + (int64_t)max(b0, 0) * a.pt_stride;
  if (total == nunion) {
    // (the usual case) every unit of the union is seen by some row: entry r
    // is rank r, written by thread r mod NT -- four page-table loads in
    // flight per thread, and each wave's stores one contiguous run
    for (int r0 = t; r0 < total; r0 += 4 * NT) {
      int uu[4], phys[4];
      uint32_t mm[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rc = min(r0 + q * NT, total - 1);
        uu[q] = (int)uor[rc];
        mm[q] = msk[rc];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) phys[q] = ptrow[uu[q] / upp];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (r0 + q * NT >= total) continue;
        uint2 e;
        if (phys[q] < 0 || phys[q] >= a.num_phys_pages) {
          err |= MSA_ERRF_PHYS_RANGE;
          e = make_uint2(0u, 0u);  // mask 0: contributes nothing
        } else {
          e = make_uint2(((uint32_t)phys[q] << 5) | (uint32_t)(uu[q] % upp), mm[q]);
        }
        out[r0 + q * NT] = e;
      }
    }
    if (t == 0) {
      soff[0] = 0;
      soff[1] = total;
    }
    return true;
  }
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bm[w];
    int r = (int)pre[w];
    while (bits) {
      // up to 8 set units at a time: their page-table loads first, then the writes
      int uu[8], phys[8];
      uint32_t mm[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uu[q] = -1;
        if (bits) {
          const int j = __builtin_ctz(bits);
          bits &= bits - 1u;
          uu[q] = w * 32 + j;
          mm[q] = msk[r++];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) phys[q] = (uu[q] >= 0 && mm[q] != 0u) ? ptrow[uu[q] / upp] : 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (uu[q] < 0 || mm[q] == 0u) continue;
        uint2 e;
        if (phys[q] < 0 || phys[q] >= a.num_phys_pages) {
          err |= MSA_ERRF_PHYS_RANGE;
          e = make_uint2(0u, 0u);  // mask 0: contributes nothing
        } else {
          e = make_uint2(((uint32_t)phys[q] << 5) | (uint32_t)(uu[q] % upp), mm[q]);
        }
        out[o++] = e;
      }
    }
  }
  if (t == 0) {
    soff[0] = 0;
    soff[1] = total;
  }
  return true;
}

template <int NT>
__global__ void __launch_bounds__(NT) gplan_kernel(const GroupArgs a) {
  extern __shared__ uint64_t keys[];  // npow2 + NT entries
  const int grp = blockIdx.x, g = blockIdx.y;
  const int K = a.num_slots;
  const int npow2 = a.sort_n;
  const int tok0 = grp * kGroupTokens;
  uint32_t err = 0;

  // ---- 1. keys.  Every thread issues all of its loads (the group's 8 token
  // rows, then 8 tokens x up to 2 slots of selections) before using any.
  constexpr int JI = (512 + NT - 1) / NT;  // slot iterations per token (K <= 512)
  int pos_t[kGroupTokens], b_t[kGroupTokens], last_t[kGroupTokens];
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau) {
    const int tok = min(tok0 + tau, a.total_q - 1);
    pos_t[tau] = a.q_pos[tok];
    b_t[tau] = a.q_seq[tok];
    if (tok0 + tau >= a.total_q) pos_t[tau] = -1;  // past the batch: no row
  }
  uint32_t mk[kGroupTokens][JI];
  int ui[kGroupTokens][JI];
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau)
#pragma unroll
    for (int i = 0; i < JI; ++i) {
      const int tok = min(tok0 + tau, a.total_q - 1);
      const int j = min((int)threadIdx.x + i * NT, K - 1);
      const int64_t so = (int64_t)tok * a.sel_stride_tok + (int64_t)g * a.sel_stride_head + j;
      mk[tau][i] = a.sel_mask[so];
      ui[tau][i] = a.sel_idx[so];
    }
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau) {
    const int bc = min(max(b_t[tau], 0), a.num_seqs - 1);
    last_t[tau] = min(pos_t[tau], a.seq_lens[bc] - 1);
  }
  uint64_t kr[kGroupTokens][JI];  // this thread's keys (invalid past slot K)
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau)
#pragma unroll
    for (int i = 0; i < JI; ++i) {
      const int j = threadIdx.x + i * NT;
      uint64_t key = kInvalidKey;
      if (j >= K) {
        kr[tau][i] = key;
        continue;
      }
      if (pos_t[tau] >= 0 && mk[tau][i] != 0) {
        const int b = b_t[tau], u = ui[tau][i];
        if (b < 0 || b >= a.num_seqs) {
          err |= MSA_ERRF_QSEQ_RANGE;
        } else if (u < 0 || (int64_t)(u + 1) * a.unit_tokens > (int64_t)a.max_pages * a.page_size) {
          err |= MSA_ERRF_SEL_RANGE;
        } else {
          // visible bits: t = u*4 + i with t <= pos, t < seq_len, bit i set
          const int nvis = min(max(last_t[tau] - u * a.unit_tokens + 1, 0), a.unit_tokens);
          const uint32_t vis = mk[tau][i] & ((1u << nvis) - 1u) & 0xfu;
          key = ((uint64_t)b << 41) | ((uint64_t)u << 17) | ((uint64_t)tau << 14) |
                ((uint64_t)j << 4) | vis;
        }
      }
      kr[tau][i] = key;
    }
  // One request among the group's valid rows (every thread holds their
  // request ids) and units below 2^15 - 1 (valid units are below max_pages *
  // page_size / unit_tokens: contexts under ~128K tokens): the low 32 bits of
  // the keys order them (the request bits are common, and no valid key has an
  // all-ones low word), so the sort runs on 32-bit keys.
  int b0 = -1;
  bool one_req = true;
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau) {
    const int b = b_t[tau];
    if (pos_t[tau] < 0 || b < 0 || b >= a.num_seqs) continue;
    if (b0 < 0) b0 = b;
    else if (b != b0) one_req = false;
  }
  const int64_t nunits = (int64_t)a.max_pages * a.page_size / a.unit_tokens;
  const int64_t li = (int64_t)g * a.num_groups + grp;
  const int64_t list_base = li * a.list_cap;
  uint2 *out = (uint2 *)(a.ws + a.lay.lists) + list_base;
  int *soff = (int *)(a.ws + a.lay.split_off) + li * (a.num_splits + 1);
  if (one_req && nunits <= kBitmapUnits &&
      bitmap_pass_words(nunits, a.list_cap, a.num_splits) <= bitmap_budget<NT>()) {
    // one request, units below 2^16: the union straight from bitmaps (done,
    // unless some token selected a unit twice)
    if (a.num_splits == 1 ? union_one_split_by_bitmap<NT>(a, kr, b0, (int)nunits, out, soff, err)
                          : union_by_bitmap<NT>(a, kr, b0, (int)nunits, out, soff, err)) {
      if (err) atomicOr(a.err_flags, err);
      return;
    }
  }
  // ---- 2. the keys to LDS, sorted
  __syncthreads();  // the bitmap pass may have used the same LDS
  for (int e = kGroupTokens * K + threadIdx.x; e < npow2; e += NT) keys[e] = kInvalidKey;
#pragma unroll
  for (int tau = 0; tau < kGroupTokens; ++tau)
#pragma unroll
    for (int i = 0; i < JI; ++i) {
      const int j = threadIdx.x + i * NT;
      if (j < K) keys[tau * K + j] = kr[tau][i];
    }
  if (one_req && nunits <= 32767) {
    const uint64_t hi = b0 < 0 ? 0ull : (uint64_t)b0 << 41;
    bitonic_sort32(keys, npow2, [](uint64_t x) { return (uint32_t)x; },
                   [hi](uint32_t x) { return hi | x; });
  } else {
    bitonic_sort(keys, npow2);
  }

  // ---- 3. distinct (split, unit) pairs, their masks.  In sorted order,
  // position p is the first entry of its token in its (request, unit) run
  // when the previous key has another (request, unit, token): it holds the
  // token's lowest slot, whose split is the token's split for that unit.
  // Such an entry leads its (split, unit) pair when no earlier first entry
  // of the run has the same split; the leader emits the pair with the
  // visible bits of every first entry of the run in that split.  Positions
  // are taken strided (p = i * NT + thread), and leaders are
  // numbered in sorted order by wave ballots.
  const int per = npow2 / NT;  // npow2 >= NT, per <= 16 (8 * 512 keys)
  const int sh1 = __builtin_ctz((unsigned)per);
  const bool one_split = a.num_splits == 1;
  // slot / slots_per_split as (slot * ceil(2^20 / spp)) >> 20: exact for
  // slot < 1024 and spp <= 512 (the rounding excess stays below 1 / 1024)
  const uint32_t split_mul = ((1u << 20) + (uint32_t)a.slots_per_split - 1u) / (uint32_t)a.slots_per_split;
  auto at = [&](int p) { return sorted_at(keys, sh1, p); };
  auto split_of = [&](uint64_t k) {
    return one_split ? 0 : (int)((((uint32_t)(k >> 4) & 0x3ffu) * split_mul) >> 20);
  };
  auto tok_bits = [](uint64_t k) { return (uint32_t)(k & 0xfu) << (4 * ((k >> 14) & 7u)); };
  struct Lead {
    bool on;
    int split;
    uint32_t m32;
    uint64_t unit;
  };
  auto analyze = [&](int p) {
    Lead L{false, 0, 0u, 0ull};
    const uint64_t k = at(p);
    if (k == kInvalidKey) return L;
    const uint64_t unit = k >> 17;
    const uint64_t kp = p > 0 ? at(p - 1) : kInvalidKey;
    if ((kp >> 14) == (k >> 14)) {  // a later slot of the same (request, unit, token)
      err |= MSA_ERRF_DUPLICATE;
      return L;
    }
    const int sg = split_of(k);
    if (one_split) {
      if ((kp >> 17) == unit) return L;  // the run start leads
    } else {
      uint64_t kq = kp;
      for (int q = p - 1; q >= 0 && (kq >> 17) == unit; --q) {
        const uint64_t kb = q > 0 ? at(q - 1) : kInvalidKey;
        if ((kb >> 14) != (kq >> 14) && split_of(kq) == sg) return L;  // an earlier first entry
        kq = kb;
      }
    }
    uint32_t m32 = tok_bits(k);
    uint64_t last = k;
    for (int q = p + 1; q < npow2; ++q) {
      const uint64_t kq = at(q);
      if ((kq >> 17) != unit) break;
      if ((kq >> 14) != (last >> 14) && split_of(kq) == sg) m32 |= tok_bits(kq);
      last = kq;
    }
    L.on = m32 != 0u;
    L.split = sg;
    L.m32 = m32;
    L.unit = unit;
    return L;
  };
  constexpr int NW = NT / 64;
  __shared__ int wave_count[16][NW];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // stage the distinct (split, unit)s: (unit id lo, hi, mask32, split), in
  // sorted order: round i's leaders follow every leader of the rounds before
  // it and, within the round, those of lower waves and lanes
  uint4 *stage = (uint4 *)(a.ws + a.lay.stage) + list_base;
  int total = 0;
  for (int i = 0; i < per; ++i) {
    const Lead L = analyze(i * NT + threadIdx.x);
    const uint64_t bal = __ballot(L.on);
    if (lane == 0) wave_count[i][wv] = __popcll(bal);
    __syncthreads();
    int before = total;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wv) before += wave_count[i][w];
      total += wave_count[i][w];
    }
    if (L.on) {
      const int off = before + __popcll(bal & ((1ull << lane) - 1ull));
      stage[off] = make_uint4((uint32_t)L.unit, (uint32_t)(L.unit >> 32), L.m32, (uint32_t)L.split);
    }
  }
  __syncthreads();

  // ---- 4. list order: (split, request, unit).  The staged order is already
  // (request, unit) with each unit's split; units are kept in that order
  // inside each split, so the groups running together on one XCD sweep the
  // cache in the same direction and share its L2 (their unions overlap).
  int n2 = NT;  // the union is usually far smaller than npow2
  while (n2 < total) n2 <<= 1;
  if (!one_split) {
    // (split:10 | staged index:16) sorts on 32 bits (index < 8 * 512)
    for (int e = threadIdx.x; e < n2; e += NT)
      keys[e] = e < total ? ((uint64_t)stage[e].w << 48) | (uint64_t)e : kInvalidKey;
    bitonic_sort32(keys, n2,
                   [](uint64_t x) {
                     return x == kInvalidKey ? ~0u : (uint32_t)((x >> 48) << 16 | (x & 0xffffu));
                   },
                   [](uint32_t x) { return (uint64_t)(x >> 16) << 48 | (x & 0xffffu); });
  }
  const int sh2 = __builtin_ctz((unsigned)(n2 / NT));
  if (one_split) {  // already in order: written in the sorted (padded) layout
    __syncthreads();
    for (int e = threadIdx.x; e < n2; e += NT) keys[e + (e >> sh2)] = e < total ? (uint64_t)e : kInvalidKey;
    __syncthreads();
  }

  // ---- 5. final list: byte offset of the unit's first K/V row, mask, tiles
  // (four entries per thread in flight: their page-table loads overlap)
  for (int e0 = threadIdx.x; e0 < total; e0 += 4 * NT) {
    uint64_t ck[4];
    uint4 st[4];
    int phys[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ck[i] = sorted_at(keys, sh2, min(e0 + i * NT, total - 1));
      st[i] = stage[(int)(ck[i] & 0xffffffffu)];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t unit_id = (uint64_t)st[i].x | ((uint64_t)st[i].y << 32);
      const int b = (int)(unit_id >> 24), u = (int)(unit_id & 0xffffffu);
      phys[i] = a.page_table[(int64_t)b * a.pt_stride + u * a.unit_tokens / a.page_size];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + i * NT;
      if (e >= total) continue;
      const uint64_t unit_id = (uint64_t)st[i].x | ((uint64_t)st[i].y << 32);
      const int upp = a.page_size / a.unit_tokens;  // units per page
      uint2 r;
      if (phys[i] < 0 || phys[i] >= a.num_phys_pages) {
        err |= MSA_ERRF_PHYS_RANGE;
        r = make_uint2(0u, 0u);  // mask 0: contributes nothing
      } else {
        r = make_uint2(((uint32_t)phys[i] << 5) | (uint32_t)((int)(unit_id & 0xffffffu) % upp), st[i].z);
      }
      out[e] = r;
    }
  }
  // split s owns sorted entries [first with split >= s, first with split >= s + 1)
  for (int sp = threadIdx.x; sp <= a.num_splits; sp += NT) {
    int lo = 0, hi = total;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)(sorted_at(keys, sh2, mid) >> 48) < sp) lo = mid + 1; else hi = mid;
    }
    soff[sp] = lo;
  }
  if (err) atomicOr(a.err_flags, err);
}

__global__ void gplan_zero(uint32_t *err) { *err = 0u; }

}  // namespace

// Dynamic LDS (the sort's keys, or the bitmap pass's words, at most
// kBitmapPassWordsFew) plus the static wave counters and scan sums.
size_t grouped_plan_lds_bytes() {
  size_t n = 1;
  while (n < (size_t)kGroupTokens * 512 || n < (size_t)kGPlanThreadsFew) n <<= 1;
  const size_t sort = (n + kGPlanThreadsFew) * 8;
  const size_t bitmap = (size_t)kBitmapPassWordsFew * 4;
  return (sort > bitmap ? sort : bitmap) + 16 * (kGPlanThreadsFew / 64) * 4 + (kGPlanThreadsFew / 64) * 4;
}

hipError_t launch_grouped_plan(const GroupArgs &a, hipStream_t s) {
  gplan_zero<<<1, 1, 0, s>>>(a.err_flags);
  if (a.num_groups == 0) return hipGetLastError();
  dim3 grid((unsigned)a.num_groups, (unsigned)a.Hkv);
  // the sort's keys, or the bitmap pass's words if that is larger
  size_t lds = ((size_t)a.sort_n + a.plan_threads) * 8;
  const int64_t nunits = (int64_t)a.max_pages * a.page_size / a.unit_tokens;
  const bool few = a.plan_threads == kGPlanThreadsFew;
  if (nunits <= kBitmapUnits) {
    const int64_t words = bitmap_pass_words(nunits, a.list_cap, a.num_splits);
    const size_t bm = (size_t)words * 4;
    if (words <= (few ? kBitmapPassWordsFew : kBitmapPassWords) && bm > lds) lds = bm;
  }
  if (few) {
    if (lds > 64 * 1024) {
      // allow the whole budget once (the function attribute, not a stream operation)
      static const hipError_t attr =
          hipFuncSetAttribute((const void *)gplan_kernel<kGPlanThreadsFew>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(kBitmapPassWordsFew * 4));
      if (attr != hipSuccess) return attr;
    }
    gplan_kernel<kGPlanThreadsFew><<<grid, kGPlanThreadsFew, lds, s>>>(a);
  } else {
    gplan_kernel<kGPlanThreads><<<grid, kGPlanThreads, lds, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace msa
