// LSE combine (MiniMax-AI/MSA PR 21, section "Combine"), written for gfx950.
//
// All (token, head) rows of the batch form one flat list; the kernel is a
// pure stream over the partial buffer, so its job is to keep enough loads in
// flight.  Partials are FP32, or BF16 / FP16 widened exactly on load.  A thread owns four consecutive columns of one row; a
// workgroup owns a run of consecutive rows, i.e. one contiguous block of
// every split slab.  Per row:
//   M = max_s lse_s                       (-inf for a row with no key at all)
//   w_s = exp(lse_s - M), W = sum_s w_s
//   out = sum_s w_s o_s / W,  lse = M + ln W
// A row whose splits are all empty writes +0 and lse = -inf without reading
// partial_o (empty splits' partial rows are never read).  All split loads of
// a row are issued before the accumulation (up to 16 splits at once; more
// splits are streamed in batches of 16 once M is known).  Every thread of a
// row reads the row's LSEs itself; those loads hit the same addresses across
// the row's lanes and are served from the cache.  Four columns per thread:
// each load instruction then covers one contiguous 1 KiB (two rows), which
// measured faster than wider per-thread strips.
#include "launch.h"

namespace msa {
namespace {

// Four consecutive partial elements of dtype IN at element offset `off`, as
// FP32 (exact for every input dtype); streamed, so loaded non-temporally.
template <int IN>
__device__ __forceinline__ f32x4 load_partial4(const void *base, int64_t off) {
  if constexpr (IN == MSA_F32) {
    return __builtin_nontemporal_load((const f32x4 *)((const float *)base + off));
  } else {
    if constexpr (IN == MSA_F16) {
      const f16x4 h = __builtin_nontemporal_load((const f16x4 *)((const uint16_t *)base + off));
      return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    } else {
      const u32x2 w = __builtin_nontemporal_load((const u32x2 *)((const uint16_t *)base + off));
      return f32x4{bf16_bits_to_f32(w[0] & 0xffffu), bf16_bits_to_f32(w[0] >> 16),
                   bf16_bits_to_f32(w[1] & 0xffffu), bf16_bits_to_f32(w[1] >> 16)};
    }
  }
}

// Eight consecutive 16-bit partial elements (one 16-byte word) as FP32.  The
// words stay 16-bit in registers while in flight (4 VGPRs per split, so all
// of a row's 16 splits fit) and are widened (exactly) where they are used.
template <int IN>
__device__ __forceinline__ void widen8(const u32x4 w, f32x4 &lo, f32x4 &hi) {
  if constexpr (IN == MSA_F16) {
    const f16x8 h = __builtin_bit_cast(f16x8, w);
    lo = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    hi = f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
  } else {
    lo = f32x4{bf16_bits_to_f32(w[0] & 0xffffu), bf16_bits_to_f32(w[0] >> 16),
               bf16_bits_to_f32(w[1] & 0xffffu), bf16_bits_to_f32(w[1] >> 16)};
    hi = f32x4{bf16_bits_to_f32(w[2] & 0xffffu), bf16_bits_to_f32(w[2] >> 16),
               bf16_bits_to_f32(w[3] & 0xffffu), bf16_bits_to_f32(w[3] >> 16)};
  }
}

template <int CPT, int B, int OUT, int IN>
__global__ void __launch_bounds__(512) combine_kernel(const void *__restrict__ po, int64_t po_split,
                                                      int64_t po_row, const float *__restrict__ pl,
                                                      int64_t pl_split, int S, int64_t rows, int dv,
                                                      void *__restrict__ out, int64_t out_row,
                                                      float *__restrict__ lse_out, const OutMap om) {
  constexpr int NV = CPT / 4;                   // 16-byte vectors per split and thread
  const int tpr = dv / CPT;                     // threads per row
  const int rows_per_block = blockDim.x / tpr;  // host guarantees tpr <= 256 (blocks of 512)
  const int tid = threadIdx.x;
  const int r_local = tid / tpr;
  const int cc = tid - r_local * tpr;
  const int64_t row = (int64_t)blockIdx.x * rows_per_block + r_local;
  const bool live = r_local < rows_per_block && row < rows;
  const int64_t rr = live ? row : 0;
  const float *plr = pl + rr;

  float l[B];
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < B; ++i) {
    l[i] = (i < S) ? plr[(int64_t)i * pl_split] : -INFINITY;
    M = fmaxf(M, l[i]);
  }
#pragma unroll 1
  for (int s = B; s < S; ++s) M = fmaxf(M, plr[(int64_t)s * pl_split]);
  f32x4 acc[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float W = 0.0f;
  if (M != -INFINITY) {
    const int64_t base = rr * po_row + cc * CPT;
#pragma unroll 1
    for (int s0 = 0; s0 < S; s0 += B) {
      if (s0 > 0) {
#pragma unroll
        for (int i = 0; i < B; ++i)
          l[i] = (s0 + i < S) ? plr[(int64_t)(s0 + i) * pl_split] : -INFINITY;
      }
      if constexpr (IN != MSA_F32 && NV % 2 == 0) {  // 16 bytes per 16-bit load
        u32x4 raw[B][NV / 2];
#pragma unroll
        for (int i = 0; i < B; ++i)
          if (l[i] != -INFINITY) {
#pragma unroll
            for (int k = 0; k < NV / 2; ++k)
              raw[i][k] = __builtin_nontemporal_load(
                  (const u32x4 *)((const uint16_t *)po + base + (int64_t)(s0 + i) * po_split + 8 * k));
          }
#pragma unroll
        for (int i = 0; i < B; ++i)
          if (l[i] != -INFINITY) {
            const float w = __builtin_amdgcn_exp2f((l[i] - M) * 1.4426950408889634f);
            W += w;
#pragma unroll
            for (int k = 0; k < NV / 2; ++k) {
              f32x4 lo, hi;
              widen8<IN>(raw[i][k], lo, hi);
              acc[2 * k] += w * lo;
              acc[2 * k + 1] += w * hi;
            }
          }
      } else {
        f32x4 v[B][NV];
#pragma unroll
        for (int i = 0; i < B; ++i)
          if (l[i] != -INFINITY) {
#pragma unroll
            for (int k = 0; k < NV; ++k)
              v[i][k] = load_partial4<IN>(po, base + (int64_t)(s0 + i) * po_split + 4 * k);
          }
#pragma unroll
        for (int i = 0; i < B; ++i)
          if (l[i] != -INFINITY) {
            const float w = __builtin_amdgcn_exp2f((l[i] - M) * 1.4426950408889634f);
            W += w;
#pragma unroll
            for (int k = 0; k < NV; ++k) acc[k] += w * v[i][k];
          }
      }
    }
    const float inv = 1.0f / W;
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k] = acc[k] * inv;
  }
  if (!live) return;
  int64_t orow = row * out_row, lrow = row;
  if (om.rows_per_split > 0) {  // placed into split slabs
    const int64_t sp = row / om.rows_per_split, rs = row - sp * om.rows_per_split;
    orow = sp * om.split + rs * out_row;
    lrow = sp * om.lse_split + rs;
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const f32x4 a = acc[k];
    const int64_t o = orow + cc * CPT + 4 * k;
    if constexpr (OUT == MSA_F32) {
      *(f32x4 *)((float *)out + o) = a;
    } else if constexpr (OUT == MSA_BF16) {
      const uint32_t lo = pack_bf16x2(a[0], a[1]);
      const uint32_t hi = pack_bf16x2(a[2], a[3]);
      *(u32x2 *)((uint16_t *)out + o) = u32x2{lo, hi};
    } else {
      *(u32x2 *)((uint16_t *)out + o) = u32x2{pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3])};
    }
  }
  if (lse_out && cc == 0)
    lse_out[lrow] = (M == -INFINITY) ? -INFINITY : M + __builtin_amdgcn_logf(W) * 0.69314718055994530942f;
}

template <int CPT, int B, int IN>
hipError_t launch_cb(const void *po, int64_t po_split, int64_t po_row, const float *pl,
                     int64_t pl_split, int32_t S, int64_t rows, int32_t dv, void *out,
                     int32_t out_dtype, int64_t out_row, float *lse, hipStream_t s, const OutMap &om) {
  const int tpr = dv / CPT;  // <= 256 (head_dim_v <= 1024)
  const int rpb = 512 / tpr;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks == 0) return hipSuccess;
  switch (out_dtype) {
    case MSA_F32:
      combine_kernel<CPT, B, MSA_F32, IN><<<(unsigned)blocks, 512, 0, s>>>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_row, lse, om);
      break;
    case MSA_BF16:
      combine_kernel<CPT, B, MSA_BF16, IN><<<(unsigned)blocks, 512, 0, s>>>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_row, lse, om);
      break;
    default:
      combine_kernel<CPT, B, MSA_F16, IN><<<(unsigned)blocks, 512, 0, s>>>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_row, lse, om);
      break;
  }
  return hipGetLastError();
}

template <int IN>
hipError_t launch_in(const void *po, int64_t po_split, int64_t po_row, const float *pl,
                     int64_t pl_split, int32_t S, int64_t rows, int32_t dv, void *out,
                     int32_t out_dtype, int64_t out_row, float *lse, hipStream_t s, const OutMap &om) {
  if constexpr (IN != MSA_F32) {  // 8 columns per thread: one 16-byte load per split
    // (only where every row of every split starts 16-byte aligned; rows
    // padded to a multiple of 4 elements only take the 8-byte path below)
    if (dv % 8 == 0 && (po_row | po_split) % 8 == 0) {
      if (S <= 4) return launch_cb<8, 4, IN>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
      if (S <= 8) return launch_cb<8, 8, IN>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
      return launch_cb<8, 16, IN>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
    }
  }
  if (S <= 4) return launch_cb<4, 4, IN>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
  if (S <= 8) return launch_cb<4, 8, IN>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
  return launch_cb<4, 16, IN>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
}

}  // namespace

hipError_t launch_combine(const void *po, int32_t po_dtype, int64_t po_split, int64_t po_row,
                          const float *pl, int64_t pl_split, int32_t S, int64_t rows, int32_t dv,
                          void *out, int32_t out_dtype, int64_t out_row, float *lse, hipStream_t s,
                          const OutMap &om) {
  switch (po_dtype) {
    case MSA_BF16: return launch_in<MSA_BF16>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
    case MSA_F16: return launch_in<MSA_F16>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
    default: return launch_in<MSA_F32>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s, om);
  }
}

}  // namespace msa
