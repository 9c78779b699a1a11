// Attention step of the grouped microblock route (1Cat-vLLM PR 387, section
// "Purpose": eight adjacent query rows share one load of their overlapping
// sparse K/V blocks while each row keeps its exact 4-bit mask; inactive row
// tiles are skipped), written for gfx950.
//
// One workgroup per (group of 8 query tokens, KV head, split).  The group's
// G query heads per token make 8*G (token, head) rows, cut into 16-row
// tiles; wave w owns tile w.  The union of the group's microblocks (built by
// the planner, ordered by category) streams through LDS in batches of 8
// units = 32 keys, double-buffered: the next batch's K/V is in flight in
// registers while the current one is computed, and the unit offsets of the
// batch after it are read meanwhile, so each batch costs one round trip to
// memory.  Per batch and active tile:
//
//   S^T = K . Q^T     f16 MFMA 16x16x32, FP32 accumulate (Q held in registers)
//   mask              key i of unit b is visible to the row of token tau iff
//                     bit 4*tau + i of the unit's mask word is set (the planner
//                     already folded the causal and tail rules into it)
//   online softmax    running max / sums per row, rescaling O when the max
//                     grows
//   O^T += V^T . P^T  f16 MFMA, P in FP16, V^T built in LDS at load time
//
// A tile none of whose rows selected any unit of the batch skips it (the
// wave-uniform test uses the units' active-tile bits).  Each split (the
// units whose first slot for a row lies in that split's slot range) is an
// independent softmax: partial_o = O / l * v_scale and lse = m + ln l (or
// -inf with zeros for a row that sees nothing in the split).
#include "grouped.h"

namespace msa {
namespace {

constexpr int GT = 256;  // threads per workgroup
constexpr int BK = 32;   // keys per batch

template <int D> struct GGeom {
  static constexpr int RB = D * 2;            // K row bytes (FP16)
  static constexpr int CPR = RB / 16;         // 16-byte chunks per K row
  static constexpr int LANE_CH = CPR / 4;     // chunks of a Q/K row one lane holds
  static constexpr int K_BYTES = BK * RB;
  static constexpr int V_BYTES = D * BK * 2;  // V^T: [D][32 keys] FP16
  static constexpr int STAGE = K_BYTES + V_BYTES + 2 * kGUnitsPerBatch * 4;
  static constexpr int KLD = BK * CPR / GT;   // K chunks per thread per batch
  static constexpr int VDB = D / 16;          // dims per thread in the V load
  static constexpr int VLD = VDB * 2 / 16;    // 16-byte chunks per key per thread
  static_assert(KLD >= 1 && VLD >= 1, "head_dim 128 or 256");
};

// Key (0..31 in the batch) carried by A-operand row m of key tile t (0, 1):
// the two tiles interleave so a lane's 8 S^T registers are 8 consecutive keys.
__device__ __forceinline__ int gkey_of(int t, int m) { return (m >> 2) * 8 + t * 4 + (m & 3); }
__device__ __forceinline__ int grow_of_key(int k) { return (k & 3) | (((k >> 3) & 3) << 2); }
template <int D> __device__ __forceinline__ int gk_off(int key, int c) {
  return key * GGeom<D>::RB + ((c ^ grow_of_key(key)) << 4);
}
// V^T row dv: the batch's 32 keys, 4 chunks of 8 keys, XOR-swizzled.
__device__ __forceinline__ int gvt_off(int dv, int c) { return dv * 64 + ((c ^ ((dv >> 2) & 3)) << 4); }

template <typename T> __device__ __forceinline__ T gld(const void *p) { return *(const T *)p; }

template <int D> struct BatchRegs {
  u32x4 k[GGeom<D>::KLD];
  u32x4 v[2][GGeom<D>::VLD];
  uint32_t mask, tiles;
};

// Byte offset (within the K / V caches) of unit u of the group's list, or -1
// past the end of the list.
__device__ __forceinline__ int64_t unit_off(const uint4 *list, int count, int u) {
  if (u >= count) return -1;
  const uint2 e = *(const uint2 *)&list[u];
  return (int64_t)((uint64_t)e.x | ((uint64_t)e.y << 32));
}

// Unit offsets (and the batch's mask / active-tile words) of this thread's
// chunks of batch beta.  They are fetched one batch ahead of the K / V loads
// that use them: a wait between an offset and its data load would also wait
// for every data load issued before it, one round trip each.
template <int D> struct BatchOffs {
  int64_t k[GGeom<D>::KLD];
  int64_t v;
  uint32_t mask, tiles;
};
template <int D>
__device__ __forceinline__ void fetch_offs(const uint4 *list, int count, int beta, BatchOffs<D> &o) {
  using Gm = GGeom<D>;
  const int tid = threadIdx.x;
  const int u0 = beta * kGUnitsPerBatch;
#pragma unroll
  for (int it = 0; it < Gm::KLD; ++it) {
    const int key = (it * GT + tid) / Gm::CPR;
    o.k[it] = unit_off(list, count, u0 + (key >> 2));
  }
  o.v = unit_off(list, count, u0 + ((tid & 15) >> 1));
  o.mask = o.tiles = 0u;
  if (tid < kGUnitsPerBatch && u0 + tid < count) {
    const uint2 e = *(const uint2 *)((const uint32_t *)&list[u0 + tid] + 2);
    o.mask = e.x;
    o.tiles = e.y;
  }
}

// The K and V chunks of this thread for the batch whose offsets are `o`.
template <int D>
__device__ __forceinline__ void load_batch(const GroupArgs &a, const BatchOffs<D> &o, BatchRegs<D> &r) {
  using Gm = GGeom<D>;
  const int tid = threadIdx.x;
  const int kp = tid & 15, db = tid >> 4;  // V: key pair, block of D/16 dims
#pragma unroll
  for (int it = 0; it < Gm::KLD; ++it) {
    const int q = it * GT + tid, key = q / Gm::CPR, c = q % Gm::CPR;
    r.k[it] = o.k[it] >= 0 ? gld<u32x4>(a.k_cache + o.k[it] + (key & 3) * a.kv_stride_tok + c * 16)
                           : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int c = 0; c < Gm::VLD; ++c)
      r.v[kk][c] = o.v >= 0 ? gld<u32x4>(a.v_cache + o.v + ((2 * kp + kk) & 3) * a.kv_stride_tok +
                                         db * Gm::VDB * 2 + c * 16)
                            : u32x4{0u, 0u, 0u, 0u};
  r.mask = o.mask;
  r.tiles = o.tiles;
}

template <int D>
__device__ __forceinline__ void store_batch(uint8_t *st, const BatchRegs<D> &r) {
  using Gm = GGeom<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < Gm::KLD; ++it) {
    const int q = it * GT + tid, key = q / Gm::CPR, c = q % Gm::CPR;
    *(u32x4 *)(st + gk_off<D>(key, c)) = r.k[it];
  }
  uint8_t *sv = st + Gm::K_BYTES;
  const int kp = tid & 15, db = tid >> 4;
#pragma unroll
  for (int c = 0; c < Gm::VLD; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int dv = db * Gm::VDB + c * 8 + w * 2 + hh;
        const uint32_t b0 = hh ? (r.v[0][c][w] >> 16) : (r.v[0][c][w] & 0xffffu);
        const uint32_t b1 = hh ? (r.v[1][c][w] >> 16) : (r.v[1][c][w] & 0xffffu);
        *(uint32_t *)(sv + gvt_off(dv, kp >> 2) + ((kp & 3) << 2)) = b0 | (b1 << 16);
      }
  uint32_t *meta = (uint32_t *)(st + Gm::K_BYTES + Gm::V_BYTES);
  if (tid < kGUnitsPerBatch) {
    meta[tid] = r.mask;
    meta[kGUnitsPerBatch + tid] = r.tiles;
  }
}

// PO: dtype of partial_o (MSA_F32, MSA_BF16 or MSA_F16).
template <int D, int PO>
__global__ void __launch_bounds__(GT, 2) k_grouped_attend(const GroupArgs a) {
  using Gm = GGeom<D>;
  constexpr int MT = D / 16;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * Gm::STAGE];
  const int grp = blockIdx.x, g = blockIdx.y, split = blockIdx.z;
  const int64_t li = (int64_t)g * a.num_groups + grp;
  const int *soff = (const int *)(a.ws + a.lay.split_off) + li * (a.num_splits + 1) + split;
  const int count = soff[1] - soff[0];
  const uint4 *list = (const uint4 *)(a.ws + a.lay.lists) + li * a.list_cap + soff[0];
  const int nb = (count + kGUnitsPerBatch - 1) / kGUnitsPerBatch;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, gl = lane >> 4;
  const int G = a.G;
  const int rows = kGroupTokens * G;
  const bool has_tile = wave * 16 < rows;  // wave-uniform

  // this lane's row: (token tau of the group, query head h)
  const int rho = wave * 16 + n;
  const int tau = rho / G;
  const int tok = grp * kGroupTokens + tau;
  const bool active = rho < rows && tok < a.total_q;
  const int h = g * G + (active ? rho - tau * G : 0);
  const int tok_c = active ? tok : 0;

  u32x4 qreg[Gm::LANE_CH];
  {
    const uint8_t *qp = (const uint8_t *)a.q +
                        ((int64_t)tok_c * a.q_stride_tok + (int64_t)h * a.q_stride_head) * 2 + gl * (Gm::RB / 4);
#pragma unroll
    for (int c = 0; c < Gm::LANE_CH; ++c) qreg[c] = gld<u32x4>(qp + c * 16);
  }
  f32x4 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f, lp = 0.0f;
  const float sc = a.scale_log2;

  BatchRegs<D> br;
  BatchOffs<D> bo;  // offsets of the next batch to load
  if (nb > 0) {
    fetch_offs<D>(list, count, 0, bo);
    load_batch<D>(a, bo, br);
    fetch_offs<D>(list, count, 1, bo);
    store_batch<D>(smem, br);
  }
  __syncthreads();

  for (int beta = 0; beta < nb; ++beta) {
    if (beta + 1 < nb) {
      load_batch<D>(a, bo, br);                     // batch beta + 1
      fetch_offs<D>(list, count, beta + 2, bo);     // offsets of batch beta + 2
    }
    const uint8_t *st = smem + (beta & 1) * Gm::STAGE;
    const uint32_t *meta = (const uint32_t *)(st + Gm::K_BYTES + Gm::V_BYTES);
    uint32_t tiles = 0;
#pragma unroll
    for (int b = 0; b < kGUnitsPerBatch; ++b) tiles |= meta[kGUnitsPerBatch + b];
    if (has_tile && ((tiles >> wave) & 1u)) {
#pragma clang fp contract(off)
      // ---- S^T = K Q^T for the batch's 32 keys
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int c = 0; c < Gm::LANE_CH; ++c)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 kr = *(const u32x4 *)(st + gk_off<D>(gkey_of(t, n), gl * Gm::LANE_CH + c));
          acc[t] = mfma_f16(kr, qreg[c], acc[t]);
        }
      // ---- exact masks: lane holds keys 8*gl + 4*t + i = unit 2*gl + t, bit i
      const uint32_t mu[2] = {meta[2 * gl], meta[2 * gl + 1]};
      float mb = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = active && ((mu[t] >> (4 * tau + i)) & 1u);
          const float x = vis ? acc[t][i] * sc : -INFINITY;
          acc[t][i] = x;
          mb = fmaxf(mb, x);
        }
      mb = quarter_reduce<true>(mb);
      const float mn = fmaxf(m, mb);
      // ---- rescale when some row's running max grew
      if (__any(mn > m)) {
        const float alpha = (mn > m) ? ((m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn)) : 1.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
        l *= alpha;
        lp *= alpha;
        m = mn;
      }
      // ---- P (0 for masked keys), sums, FP16 pairs
      uint32_t pk[4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = (acc[t][i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(acc[t][i] - m);
          l += p[i];
        }
        pk[2 * t] = pack_f16x2(p[0], p[1]);
        pk[2 * t + 1] = pack_f16x2(p[2], p[3]);
        lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[2 * t]), f16x2{(_Float16)1.0f, (_Float16)1.0f}, lp, false);
        lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[2 * t + 1]), f16x2{(_Float16)1.0f, (_Float16)1.0f}, lp, false);
      }
      // ---- O^T += V^T P^T (one 32-key step)
      const u32x4 pf = {pk[0], pk[1], pk[2], pk[3]};
      const uint8_t *sv = st + Gm::K_BYTES;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4 vf = *(const u32x4 *)(sv + gvt_off(mt * 16 + n, gl));
        o[mt] = mfma_f16(vf, pf, o[mt]);
      }
    }
    if (beta + 1 < nb) store_batch<D>(smem + ((beta + 1) & 1) * Gm::STAGE, br);
    __syncthreads();
  }

  // ---- epilogue: row n of the tile, columns 16*mt + 4*gl + [0,4)
  if (!has_tile || !active) return;
  l = quarter_reduce<false>(l);
  lp = quarter_reduce<false>(lp);
  const int64_t row = (int64_t)tok * a.Hq + h;
  const int64_t off = (int64_t)split * a.po_split_stride + row * a.po_row_stride + gl * 4;
  float *lse_dst = a.partial_lse + (int64_t)split * a.pl_split_stride + row;
  if (l > 0.0f) {
    const float inv = a.v_scale / lp;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) store_partial4<PO>(a.partial_o, off + mt * 16, o[mt] * inv);
    if (gl == 0) *lse_dst = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) store_partial4<PO>(a.partial_o, off + mt * 16, f32x4{0.f, 0.f, 0.f, 0.f});
    if (gl == 0) *lse_dst = -INFINITY;
  }
}

}  // namespace

size_t grouped_attend_lds_bytes() {
  return (size_t)(2 * (GGeom<256>::STAGE > GGeom<128>::STAGE ? GGeom<256>::STAGE : GGeom<128>::STAGE));
}

hipError_t launch_grouped_attend(const GroupArgs &a, hipStream_t s) {
  if (a.num_groups == 0) return hipSuccess;
  dim3 grid((unsigned)a.num_groups, (unsigned)a.Hkv, (unsigned)a.num_splits);
  switch ((a.D == 256 ? 8 : 0) + a.po_dtype) {
    case 8 + MSA_F32: k_grouped_attend<256, MSA_F32><<<grid, GT, 0, s>>>(a); break;
    case 8 + MSA_BF16: k_grouped_attend<256, MSA_BF16><<<grid, GT, 0, s>>>(a); break;
    case 8 + MSA_F16: k_grouped_attend<256, MSA_F16><<<grid, GT, 0, s>>>(a); break;
    case MSA_BF16: k_grouped_attend<128, MSA_BF16><<<grid, GT, 0, s>>>(a); break;
    case MSA_F16: k_grouped_attend<128, MSA_F16><<<grid, GT, 0, s>>>(a); break;
    default: k_grouped_attend<128, MSA_F32><<<grid, GT, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace msa
