// LSE combine (MiniMax-AI/MSA PR 21, section "Combine"), written for gfx950.
//
// All (token, head) rows of the batch form one flat list; the kernel is a
// pure stream over the partial buffer, so its job is to keep enough 16-byte
// loads in flight.  A thread owns four consecutive columns of one row; a
// workgroup owns a run of consecutive rows, i.e. one contiguous block of
// every split slab.  Per row:
//   M = max_s lse_s                       (-inf for a row with no key at all)
//   w_s = exp(lse_s - M), W = sum_s w_s
//   out = sum_s w_s o_s / W,  lse = M + ln W
// A row whose splits are all empty writes +0 and lse = -inf without reading
// partial_o (empty splits' partial rows are never read).  All split loads of
// a row are issued before the accumulation (up to 16 splits at once; more
// splits are streamed in batches of 16).  Every thread of a row reads the
// row's LSEs itself; those loads hit the same addresses across the row's
// lanes and are served from the cache.
#include "launch.h"

namespace msa {
namespace {

template <int SMAX, int OUT>
__global__ void __launch_bounds__(256) combine_kernel(const float *__restrict__ po, int64_t po_split,
                                                      int64_t po_row, const float *__restrict__ pl,
                                                      int64_t pl_split, int S, int64_t rows, int dv,
                                                      void *__restrict__ out, int64_t out_row,
                                                      float *__restrict__ lse_out) {
  const int tpr = dv >> 2;                      // threads per row
  const int rows_per_block = blockDim.x / tpr;  // host guarantees tpr | 256
  const int tid = threadIdx.x;
  const int r_local = tid / tpr;
  const int c4 = tid - r_local * tpr;
  const int64_t row = (int64_t)blockIdx.x * rows_per_block + r_local;
  const bool live = r_local < rows_per_block && row < rows;
  const int64_t rr = live ? row : 0;
  constexpr int BATCH = SMAX > 0 ? SMAX : 16;

  float l[BATCH];
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < BATCH; ++s) {
    l[s] = (s < S) ? pl[(int64_t)s * pl_split + rr] : -INFINITY;
    M = fmaxf(M, l[s]);
  }
  if constexpr (SMAX == 0)
    for (int s = BATCH; s < S; ++s) M = fmaxf(M, pl[(int64_t)s * pl_split + rr]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.0f;
  if (M != -INFINITY) {
    const float *base = po + rr * po_row + c4 * 4;
    for (int s0 = 0; s0 < S; s0 += BATCH) {
      if (s0 > 0) {
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
          l[i] = (s0 + i < S) ? pl[(int64_t)(s0 + i) * pl_split + rr] : -INFINITY;
      }
      f32x4 v[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        if (l[i] != -INFINITY)
          v[i] = __builtin_nontemporal_load((const f32x4 *)(base + (int64_t)(s0 + i) * po_split));
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        if (l[i] != -INFINITY) {
          const float w = __builtin_amdgcn_exp2f((l[i] - M) * 1.4426950408889634f);
          W += w;
          acc += w * v[i];
        }
      if constexpr (SMAX > 0) break;
    }
    acc = acc * (1.0f / W);
  }
  if (!live) return;
  if constexpr (OUT == MSA_F32) {
    *(f32x4 *)((float *)out + row * out_row + c4 * 4) = acc;
  } else if constexpr (OUT == MSA_BF16) {
    uint32_t lo = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
    uint32_t hi = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    *(u32x2 *)((uint16_t *)out + row * out_row + c4 * 4) = u32x2{lo, hi};
  } else {
    *(u32x2 *)((uint16_t *)out + row * out_row + c4 * 4) =
        u32x2{pack_f16x2(acc[0], acc[1]), pack_f16x2(acc[2], acc[3])};
  }
  if (lse_out && c4 == 0)
    lse_out[row] = (M == -INFINITY) ? -INFINITY : M + __builtin_amdgcn_logf(W) * 0.69314718055994530942f;
}

template <int SMAX>
hipError_t launch_s(const float *po, int64_t po_split, int64_t po_row, const float *pl,
                    int64_t pl_split, int32_t S, int64_t rows, int32_t dv, void *out,
                    int32_t out_dtype, int64_t out_row, float *lse, hipStream_t s) {
  const int tpr = dv / 4;  // <= 256 (head_dim_v <= 1024)
  const int rpb = 256 / tpr;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks == 0) return hipSuccess;
  switch (out_dtype) {
    case MSA_F32:
      combine_kernel<SMAX, MSA_F32><<<(unsigned)blocks, 256, 0, s>>>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_row, lse);
      break;
    case MSA_BF16:
      combine_kernel<SMAX, MSA_BF16><<<(unsigned)blocks, 256, 0, s>>>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_row, lse);
      break;
    default:
      combine_kernel<SMAX, MSA_F16><<<(unsigned)blocks, 256, 0, s>>>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_row, lse);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float *po, int64_t po_split, int64_t po_row, const float *pl,
                          int64_t pl_split, int32_t S, int64_t rows, int32_t dv, void *out,
                          int32_t out_dtype, int64_t out_row, float *lse, hipStream_t s) {
  if (S <= 4) return launch_s<4>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s);
  if (S <= 8) return launch_s<8>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s);
  if (S <= 16) return launch_s<16>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s);
  return launch_s<0>(po, po_split, po_row, pl, pl_split, S, rows, dv, out, out_dtype, out_row, lse, s);
}

}  // namespace msa
