// Planner of the grouped microblock route (1Cat-vLLM PR 387, section
// "Purpose": a deterministic GPU planner maps the logical selections through
// the paged cache, groups blocks by active-row category and validates
// request, visibility, logical-page, tail and physical-page bounds; PR 1236,
// section "Purpose": a group of eight rows holds at most 8 x 513
// microblocks and the plan order depends only on category and logical
// owner).
//
// One workgroup per (group of kGroupTokens consecutive query tokens, KV head):
//   1. every (token, slot) selection becomes a 64-bit key
//        request:16 | unit:24 | token-in-group:3 | slot:10 | visible bits:4
//      (bits 41.. | 17.. | 14.. | 4.. | 0..)
//      (invalid selections sort to the end);
//   2. bitonic sort of the keys in LDS;
//   3. duplicates of a (request, unit, token) beyond the first slot are
//      dropped and flagged; each distinct (request, unit) gets a 32-bit mask,
//      4 visible-token bits per token of the group; units no row sees are
//      dropped; the physical page is looked up and checked;
//   4. the union is sorted again by (active row tiles, active tokens,
//      request, unit) so consecutive units share their category and whole
//      row tiles can skip a batch;
//   5. the group's list is written: {K/V row offset of the unit's first
//      token in bytes (low, high), mask32, active tiles} per unit.
#include "grouped.h"

namespace msa {
namespace {

constexpr uint64_t kInvalidKey = ~0ull;

// Ascending bitonic sort of n = E * blockDim.x keys held in LDS.  Thread t
// keeps the keys of sorted positions tE .. tE+E-1 in registers: compare-
// exchange steps whose partner lies within the thread (stride < E) run in
// registers; the others exchange through LDS, every thread computing its own
// new key.  During the sort the LDS copy is laid out position p -> slot
// (p % E) * nt + p / E, so a wave's accesses hit consecutive slots; the
// input is taken in that layout too (any input order sorts the same), and
// the result is written back in plain sorted order.
template <int E>
__device__ __forceinline__ void bitonic_sort_e(uint64_t *k, int n) {
  uint64_t r[E];
  const int t = threadIdx.x, nt = blockDim.x;
  const int base = t * E;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) r[i] = k[i * nt + t];
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride >= E; stride >>= 1) {
      __syncthreads();  // everyone is done reading the previous round
#pragma unroll
      for (int i = 0; i < E; ++i) k[i * nt + t] = r[i];
      __syncthreads();
      const int tq = t ^ (stride / E);  // the partner thread (same register i)
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int p = base + i, q = p ^ stride;
        const uint64_t o = k[i * nt + tq];
        const bool up = (p & size) == 0;
        const bool keep_min = (p < q) == up;
        r[i] = keep_min ? (r[i] < o ? r[i] : o) : (r[i] > o ? r[i] : o);
      }
    }
    // strides below E: partners in this thread's registers (compile-time
    // indices, so the keys stay in registers)
#pragma unroll
    for (int st = E >> 1; st >= 1; st >>= 1) {
      if (st < size) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if (i & st) continue;
          const int j = i | st;
          const bool up = ((base + i) & size) == 0;
          const uint64_t x = r[i], y = r[j];
          const bool sw = (x > y) == up;
          r[i] = sw ? y : x;
          r[j] = sw ? x : y;
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < E; ++i) k[base + i] = r[i];
  __syncthreads();
}

// n: a power of two in [blockDim.x, 16 * blockDim.x]
__device__ __forceinline__ void bitonic_sort(uint64_t *k, int n) {
  switch (n / (int)blockDim.x) {
    case 1: bitonic_sort_e<1>(k, n); break;
    case 2: bitonic_sort_e<2>(k, n); break;
    case 4: bitonic_sort_e<4>(k, n); break;
    case 8: bitonic_sort_e<8>(k, n); break;
    default: bitonic_sort_e<16>(k, n); break;
  }
}

// Exclusive block-wide scan of one int per thread (blockDim.x <= 1024).
__device__ __forceinline__ int block_exclusive_scan(int v, int *tmp, int &total) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const int x = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += x;
    __syncthreads();
  }
  total = tmp[blockDim.x - 1];
  const int r = tmp[t] - v;
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kGPlanThreads) gplan_kernel(const GroupArgs a) {
  extern __shared__ uint64_t keys[];  // npow2 entries
  __shared__ int scan_tmp[kGPlanThreads];
  const int grp = blockIdx.x, g = blockIdx.y;
  const int K = a.num_slots;
  const int npow2 = a.sort_n;
  const int tok0 = grp * kGroupTokens;
  uint32_t err = 0;

  // ---- 1. keys
  for (int e = threadIdx.x; e < npow2; e += kGPlanThreads) {
    uint64_t key = kInvalidKey;
    if (e < kGroupTokens * K) {
      const int tau = e / K, j = e - tau * K;
      const int tok = tok0 + tau;
      if (tok < a.total_q) {
        const int pos = a.q_pos[tok];
        const int b = a.q_seq[tok];
        const int64_t so = (int64_t)tok * a.sel_stride_tok + (int64_t)g * a.sel_stride_head + j;
        const uint32_t mk = a.sel_mask[so];
        if (pos >= 0 && mk != 0) {
          if (b < 0 || b >= a.num_seqs) {
            err |= MSA_ERRF_QSEQ_RANGE;
          } else {
            const int u = a.sel_idx[so];
            if (u < 0 || (int64_t)(u + 1) * a.unit_tokens > (int64_t)a.max_pages * a.page_size) {
              err |= MSA_ERRF_SEL_RANGE;
            } else {
              // visible bits: t = u*4 + i with t <= pos, t < seq_len, bit i set
              const int last = min(pos, a.seq_lens[b] - 1);
              const int nvis = min(max(last - u * a.unit_tokens + 1, 0), a.unit_tokens);
              const uint32_t vis = mk & ((1u << nvis) - 1u) & 0xfu;
              key = ((uint64_t)b << 41) | ((uint64_t)u << 17) | ((uint64_t)tau << 14) |
                    ((uint64_t)j << 4) | vis;
            }
          }
        }
      }
    }
    keys[e] = key;
  }
  bitonic_sort(keys, npow2);

  // ---- 3. distinct units, their masks, physical pages.  Each thread owns a
  // contiguous run of sorted positions, so scans preserve the sorted order.
  const int per = npow2 / kGPlanThreads;  // npow2 >= kGPlanThreads
  const int p0 = threadIdx.x * per;
  int emit_n = 0;
  for (int p = p0; p < p0 + per; ++p) {
    const uint64_t k = keys[p];
    if (k == kInvalidKey) break;
    const uint64_t unit_id = k >> 17;
    if (p > 0 && (keys[p - 1] >> 17) == unit_id) {
      if ((keys[p - 1] >> 14) == (k >> 14)) err |= MSA_ERRF_DUPLICATE;
      continue;  // not the unit's first entry
    }
    uint32_t m32 = 0;
    for (int q = p; q < npow2 && (keys[q] >> 17) == unit_id; ++q) {
      const bool first_of_tok = (q == p) || ((keys[q - 1] >> 14) != (keys[q] >> 14));
      if (first_of_tok) m32 |= (uint32_t)(keys[q] & 0xfu) << (4 * ((keys[q] >> 14) & 7u));
    }
    if (m32 != 0) ++emit_n;
  }
  int total;
  int wpos = block_exclusive_scan(emit_n, scan_tmp, total);
  // stage the distinct units' (unit id, mask32) in the workspace staging area
  const int64_t list_base = ((int64_t)g * a.num_groups + grp) * a.list_cap;
  uint4 *stage = (uint4 *)(a.ws + a.lay.stage) + list_base;
  uint4 *out = (uint4 *)(a.ws + a.lay.lists) + list_base;
  for (int p = p0; p < p0 + per; ++p) {
    const uint64_t k = keys[p];
    if (k == kInvalidKey) break;
    const uint64_t unit_id = k >> 17;
    if (p > 0 && (keys[p - 1] >> 17) == unit_id) continue;
    uint32_t m32 = 0;
    for (int q = p; q < npow2 && (keys[q] >> 17) == unit_id; ++q) {
      const bool first_of_tok = (q == p) || ((keys[q - 1] >> 14) != (keys[q] >> 14));
      if (first_of_tok) m32 |= (uint32_t)(keys[q] & 0xfu) << (4 * ((keys[q] >> 14) & 7u));
    }
    if (m32 == 0) continue;
    stage[wpos++] = make_uint4((uint32_t)unit_id, (uint32_t)(unit_id >> 32), m32, 0u);
  }
  __syncthreads();

  // ---- 4. category keys: (tiles, tokens, index in the (request, unit) order)
  const int G = a.G;
  int n2 = kGPlanThreads;  // the union is usually far smaller than npow2
  while (n2 < total) n2 <<= 1;
  for (int e = threadIdx.x; e < n2; e += kGPlanThreads) {
    uint64_t key = kInvalidKey;
    if (e < total) {
      const uint32_t m32 = stage[e].z;
      uint32_t toks = 0, tiles = 0;
#pragma unroll
      for (int tau = 0; tau < kGroupTokens; ++tau)
        if ((m32 >> (4 * tau)) & 0xfu) {
          toks |= 1u << tau;
          const int r0 = tau * G, r1 = tau * G + G - 1;  // rows of this token
          tiles |= (1u << (r0 >> 4)) | (1u << (r1 >> 4));
        }
      key = ((uint64_t)tiles << 40) | ((uint64_t)toks << 32) | (uint64_t)e;
    }
    keys[e] = key;
  }
  bitonic_sort(keys, n2);

  // ---- 5. final list: byte offset of the unit's first K/V row, mask, tiles
  for (int e = threadIdx.x; e < total; e += kGPlanThreads) {
    const uint64_t ck = keys[e];
    const uint4 st = stage[(int)(ck & 0xffffffffu)];
    const uint64_t unit_id = (uint64_t)st.x | ((uint64_t)st.y << 32);
    const int b = (int)(unit_id >> 24), u = (int)(unit_id & 0xffffffu);
    const int t0 = u * a.unit_tokens;
    const int phys = a.page_table[(int64_t)b * a.pt_stride + t0 / a.page_size];
    uint4 r;
    if (phys < 0 || phys >= a.num_phys_pages) {
      err |= MSA_ERRF_PHYS_RANGE;
      r = make_uint4(0u, 0u, 0u, 0u);  // mask 0: contributes nothing
    } else {
      const int64_t off = (int64_t)phys * a.kv_stride_page + (int64_t)(t0 % a.page_size) * a.kv_stride_tok +
                          (int64_t)g * a.kv_stride_head;
      r = make_uint4((uint32_t)off, (uint32_t)((uint64_t)off >> 32), st.z, (uint32_t)(ck >> 40));
    }
    out[e] = r;
  }
  if (threadIdx.x == 0) ((int *)(a.ws + a.lay.counts))[(int64_t)g * a.num_groups + grp] = total;
  if (err) atomicOr(a.err_flags, err);
}

__global__ void gplan_zero(uint32_t *err) { *err = 0u; }

}  // namespace

hipError_t launch_grouped_plan(const GroupArgs &a, hipStream_t s) {
  gplan_zero<<<1, 1, 0, s>>>(a.err_flags);
  if (a.num_groups == 0) return hipGetLastError();
  dim3 grid((unsigned)a.num_groups, (unsigned)a.Hkv);
  gplan_kernel<<<grid, kGPlanThreads, (size_t)a.sort_n * 8, s>>>(a);
  return hipGetLastError();
}

}  // namespace msa
