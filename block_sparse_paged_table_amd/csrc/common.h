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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

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

// FP8 x FP8 over K = 128 (gfx950 v_mfma_f32_16x16x128_f8f6f4; E4M3 both
// sides, no block scales): each lane brings 32 bytes of its A row and 32
// bytes of its B column.  The contraction pairs byte j of lane (m, group)
// with byte j of lane (n, group), so any placement of the K elements that A
// and B share gives the full dot product.
__device__ __forceinline__ f32x4 mfma_fp8_k128(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x4 c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- formats

// NVFP4 dequantisation (MiniMax-AI/MSA PR 21, section "Build the prefill for
// SM107"): an element is its E2M1 code times its block's E4M3 scale, rounded
// once to E4M3 (the float product is exact: at most 6 significant bits).
// Rounding is symmetric, so a block needs only the 8 magnitudes
// |e2m1(c)| * |scale|, c = 0..7; an element's byte is its magnitude with the
// sign bit XOR-ed from the code and the scale (an IEEE product's sign, which
// also gives the sign of zero).
//
// nvfp4_mag_table: the 8 magnitude bytes, byte c of the 8-byte pair.  The
// products are exact in FP32; clamping them to 448 and converting with the
// hardware's round-to-nearest-even FP8 conversion gives the saturating RNE
// rounding (every product above 448 rounds to 448).
__device__ __forceinline__ u32x2 nvfp4_mag_table(uint32_t scale) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)(scale & 0x7fu), 0);
  const float top = 448.0f;
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(0.0f, 0.5f * s, 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(s, fminf(1.5f * s, top), w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(2.0f * s, top), fminf(3.0f * s, top), 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(4.0f * s, top), fminf(6.0f * s, top), w1, true);
  return u32x2{(uint32_t)w0, (uint32_t)w1};
}

// The same 8 magnitudes as FP16 (exact: E4M3 values are FP16 values), split
// into a table of their low bytes and one of their high bytes (byte c of
// each pair), for byte-permute lookups.
__device__ __forceinline__ void nvfp4_f16_tables(u32x2 tab, uint32_t lo[2], uint32_t hi[2]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)tab[w], false);
    const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)tab[w], true);
    const uint32_t h01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f01[0], f01[1]));
    const uint32_t h23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f23[0], f23[1]));
    lo[w] = __builtin_amdgcn_perm(h23, h01, 0x06040200u);
    hi[w] = __builtin_amdgcn_perm(h23, h01, 0x07050301u);
  }
}

// Spread 4 nibbles (bits 4i..4i+3) to the low nibbles of 4 bytes.
__device__ __forceinline__ uint32_t spread_nibbles(uint32_t x) {
  return (x & 0xfu) | ((x & 0xf0u) << 4) | ((x & 0xf00u) << 8) | ((x & 0xf000u) << 12);
}

// Four E4M3 bytes (byte i) of the four codes in the low 16 bits of `codes`
// (element i in bits 4i..4i+3), all sharing one block scale.
// `sign_flip` = 0x80808080 if the scale is negative, else 0.
__device__ __forceinline__ uint32_t nvfp4_lookup4(uint32_t codes, u32x2 tab, uint32_t sign_flip) {
  const uint32_t sp = spread_nibbles(codes & 0xffffu);
  const uint32_t mags = __builtin_amdgcn_perm(tab[1], tab[0], sp & 0x07070707u);
  return (mags | ((sp & 0x08080808u) << 4)) ^ sign_flip;
}

// Single element at position pos (0..3) of a 4-code word (standalone
// dequantisation entry point; same tables and lookup as the attention).
__device__ __forceinline__ uint32_t nvfp4_to_e4m3(uint32_t code, uint32_t scale, int pos) {
  const uint32_t b4 = nvfp4_lookup4((code & 15u) << (4 * pos), nvfp4_mag_table(scale),
                                    (scale & 0x80u) ? 0x80808080u : 0u);
  return (b4 >> (8 * pos)) & 0xffu;
}

// The V side of the same dequantisation, straight to the FP16 operand of the
// PV product (every E4M3 value is an FP16 value, so this is exact): a block's
// eight FP16 magnitudes as byte-permute tables of their low and high bytes,
// and the sign flip of a negative scale.
struct Nvfp4F16Tab {
  uint32_t lo[2], hi[2], flip;
};

__device__ __forceinline__ Nvfp4F16Tab nvfp4_f16_tab(uint32_t scale) {
  Nvfp4F16Tab t;
  nvfp4_f16_tables(nvfp4_mag_table(scale), t.lo, t.hi);
  t.flip = (scale & 0x80u) ? 0x80008000u : 0u;
  return t;
}

// Four elements sharing one block scale (codes in the low 16 bits of
// `codes`, element i in bits 4i..4i+3) as FP16: word 0 holds elements 0 (low
// half) and 1, word 1 elements 2 and 3.  A code's sign bit becomes the FP16
// sign (XOR the scale's), which also signs the zeros.
__device__ __forceinline__ u32x2 nvfp4_lookup4_f16(uint32_t codes, const Nvfp4F16Tab &t) {
  const uint32_t sp = spread_nibbles(codes & 0xffffu);
  const uint32_t sel = sp & 0x07070707u, sg = sp & 0x08080808u;
  const uint32_t L = __builtin_amdgcn_perm(t.lo[1], t.lo[0], sel);
  const uint32_t H = __builtin_amdgcn_perm(t.hi[1], t.hi[0], sel);
  const uint32_t p01 = __builtin_amdgcn_perm(H, L, 0x05010400u) | ((sg & 0x8u) << 12) | ((sg & 0x800u) << 20);
  const uint32_t p23 = __builtin_amdgcn_perm(H, L, 0x07030602u) | ((sg & 0x80000u) >> 4) | ((sg & 0x8000000u) << 4);
  return u32x2{p01 ^ t.flip, p23 ^ t.flip};
}

// Single element at position pos (0..3) as FP16 bits (standalone entry point).
__device__ __forceinline__ uint32_t nvfp4_to_f16(uint32_t code, uint32_t scale, int pos) {
  const u32x2 w = nvfp4_lookup4_f16((code & 15u) << (4 * pos), nvfp4_f16_tab(scale));
  return (w[pos >> 1] >> (16 * (pos & 1))) & 0xffffu;
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

// Two floats as BF16 (round to nearest even; finite values), low half first:
// one packed hardware conversion on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Four consecutive partial-output elements at element offset `off` of a
// buffer of dtype PO (MSA_F32, or MSA_BF16 / MSA_F16 rounded to nearest even).
template <int PO>
__device__ __forceinline__ void store_partial4(void *base, int64_t off, f32x4 v) {
  if constexpr (PO == MSA_F32) {
    *(f32x4 *)((float *)base + off) = v;
  } else if constexpr (PO == MSA_F16) {
    *(u32x2 *)((uint16_t *)base + off) = u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
  } else {
    *(u32x2 *)((uint16_t *)base + off) =
        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// ---------------------------------------------------------------- plan layout

// One entry of the page route's inverted index: a (token, slot) that selected
// the list's page, and the last visible in-page key offset for that token.
struct PlanEntry {
  int32_t tok_slot;   // token << 8 | slot
  int32_t limit;      // min(q_pos, seq_len - 1) - page_start, in [0, page)
};

// One work unit of the page route, as the plan writes it: a chunk of one
// list's entries and the list's physical page and KV head.
struct PageUnit {
  int32_t e_begin, e_count, phys, g;
};

struct PageLayout {
  int64_t num_lists;     // slices * num_seqs * max_pages * Hkv
  int64_t num_sel;       // total_q * Hkv * num_slots
  int64_t max_units;     // bound on the work units
  size_t counts, list_off, unit_off, slot_list, slot_pos, entries, units, meta, dump, tiles, total;
};

constexpr int kScanTile = 4096;  // lists per block of the plan's scan

__host__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ inline PageLayout page_layout(int64_t num_lists, int64_t num_sel, int64_t max_units) {
  PageLayout L;
  L.num_lists = num_lists;
  L.num_sel = num_sel;
  L.max_units = max_units;
  size_t off = 0;
  L.meta = off;      off = align_up(off + 64 * 4, 256);
  L.dump = off;      off = align_up(off + 1024 * 4, 256);  // scratch for masked-off stores
  L.counts = off;    off = align_up(off + (size_t)num_lists * 4, 256);
  L.list_off = off;  off = align_up(off + (size_t)(num_lists + 1) * 4, 256);
  L.unit_off = off;  off = align_up(off + (size_t)(num_lists + 1) * 4, 256);
  L.slot_list = off; off = align_up(off + (size_t)num_sel * 4, 256);
  L.slot_pos = off;  off = align_up(off + (size_t)num_sel * 4, 256);
  L.entries = off;   off = align_up(off + (size_t)num_sel * sizeof(PlanEntry), 256);
  L.units = off;     off = align_up(off + (size_t)max_units * sizeof(PageUnit), 256);
  L.tiles = off;     off = align_up(off + (size_t)((num_lists + kScanTile - 1) / kScanTile + 1) * 4 * 8, 256);
  L.total = off;
  return L;
}

// Max (MAX) or sum of x over the four lanes l, l^16, l^32, l^48 -- the
// quarters of one row -- on every lane, through the gfx950 row swaps
// (v_permlane16_swap: rows 0<->1 and 2<->3; v_permlane32_swap: rows 0,1 <->
// 2,3), VALU operations instead of LDS-routed permutes.  Both lanes of a
// pair add the same two values, so every lane holds the same bits.
template <bool MAX>
__device__ __forceinline__ float quarter_reduce(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y0 = __uint_as_float(a[0]), y1 = __uint_as_float(a[1]);
  const float y = MAX ? fmaxf(y0, y1) : y0 + y1;
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  const float z0 = __uint_as_float(b[0]), z1 = __uint_as_float(b[1]);
  return MAX ? fmaxf(z0, z1) : z0 + z1;
}

#define LDS_AS __attribute__((address_space(3)))

// s_waitcnt with vmcnt(n) and lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8).
template <int N> __device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// One 16-byte load per lane straight into LDS (global_load_lds_dwordx4):
// lane i reads base + voff (base a wave-uniform 64-bit address, voff this
// lane's 32-bit offset) and writes LDS bytes [lds + 16 i, lds + 16 i + 16);
// M0 holds the LDS address, with the one wait state its write needs before
// the load.  It is issued from asm so that the compiler, which cannot tell
// which LDS bytes such a load writes, adds no wait for it before every later
// LDS read: the kernel counts these loads itself (vmcnt, which a
// __syncthreads also drains) and publishes them with a barrier.  No register
// is written: the data goes to LDS.
__device__ __forceinline__ void lds_dma16(const uint8_t *base, uint32_t voff, uint32_t lds) {
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(lds), "v"(voff), "s"(base)
                   : "memory");
}

// Workgroup barrier that waits for nothing by itself (the waits are explicit)
// and that the compiler may not move memory accesses across.
__device__ __forceinline__ void stage_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

}  // namespace msa
