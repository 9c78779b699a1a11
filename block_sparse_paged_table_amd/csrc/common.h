// Internal helpers shared by the gfx950 kernels of libmsa: vector types,
// MFMA wrappers, exact number-format conversions and the plan layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/msa.h"

namespace msa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- MFMA
// All 16x16 variants share one accumulator layout: lane l, register i holds
// D[4*(l/16) + i][l % 16].  Operand A lane l carries row l % 16, operand B
// lane l carries column l % 16; both take their k elements from the same
// (l / 16, element) slots, so any permutation of the contraction index that
// is applied to both operands gives the same product.

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_fp8(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a),
                                                    __builtin_bit_cast(long, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- formats

// OCP E4M3 byte -> float (exact).  NaN codes are not special-cased.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (b & 0x80u) ? -v : v;
}

// E2M1 code (low 4 bits) -> float (exact): magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float v = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : (m ? 0.5f : 0.0f);
  return (c & 8u) ? -v : v;
}

// float -> OCP E4M3 byte, round to nearest even, saturating to +-448; the
// sign of zero is kept.  NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7fffffffu;
  uint32_t code;
  if (a > 0x7f800000u) return 0x7fu;
  if (a >= 0x43e80000u) {            // |x| >= 464: beyond the last rounding midpoint
    code = 0x7eu;
  } else if (a < 0x3c800000u) {      // |x| < 2^-6: subnormal grid of step 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t e = (a >> 23) - 120u;   // biased E4M3 exponent, 1..15
    const uint32_t mant = a & 0x7fffffu;
    const uint32_t keep = mant >> 20, rem = mant & 0xfffffu;
    const uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (keep & 1u));
    code = ((e << 3) | keep) + up;
  }
  return sign | code;
}

// NVFP4 element: E2M1 code x E4M3 scale, rounded once to E4M3.  The float
// product is exact (at most 6 significant bits), so the single rounding is
// the conversion.
__device__ __forceinline__ uint32_t nvfp4_to_e4m3(uint32_t code, uint32_t scale) {
  return f32_to_e4m3(e2m1_to_f32(code) * e4m3_to_f32(scale));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__host__ __device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u;
#if defined(__HIP_DEVICE_COMPILE__)
  u = __float_as_uint(f);
#else
  __builtin_memcpy(&u, &f, 4);
#endif
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- plan layout

// One entry of the page route's inverted index: a (token, slot) that selected
// the list's page, and the last visible in-page key offset for that token.
struct PlanEntry {
  int32_t tok_slot;   // token << 8 | slot
  int32_t limit;      // min(q_pos, seq_len - 1) - page_start, in [0, page)
};

struct PageLayout {
  int64_t num_lists;     // num_seqs * max_pages * Hkv
  int64_t num_sel;       // total_q * Hkv * num_slots
  size_t counts, list_off, unit_off, slot_list, slot_pos, entries, meta, total;
};

__host__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ inline PageLayout page_layout(int64_t num_lists, int64_t num_sel) {
  PageLayout L;
  L.num_lists = num_lists;
  L.num_sel = num_sel;
  size_t off = 0;
  L.meta = off;      off = align_up(off + 64 * 4, 256);
  L.counts = off;    off = align_up(off + (size_t)num_lists * 4, 256);
  L.list_off = off;  off = align_up(off + (size_t)(num_lists + 1) * 4, 256);
  L.unit_off = off;  off = align_up(off + (size_t)(num_lists + 1) * 4, 256);
  L.slot_list = off; off = align_up(off + (size_t)num_sel * 4, 256);
  L.slot_pos = off;  off = align_up(off + (size_t)num_sel * 4, 256);
  L.entries = off;   off = align_up(off + (size_t)num_sel * sizeof(PlanEntry), 256);
  L.total = off;
  return L;
}

}  // namespace msa
