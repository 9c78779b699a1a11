// Attention step of the page-selection route (MiniMax-AI/MSA PR 21, section
// "K1"), written for gfx950.
//
// One workgroup owns one work unit: a chunk of the queries that selected one
// (request, logical page, KV head).  It loads that physical page once --
// K as the QK operand type, V transposed to [d][key] as FP16 (or FP32) --
// into LDS, then its four waves stream 16-row tiles of (query token, query
// head) rows through:
//
//   S^T = K . Q^T        MFMA, FP32 accumulate (K rows = A operand from LDS,
//                        Q rows = B operand straight from HBM/L2)
//   mask                 only where a row can see part of the page: the key
//                        offset must not pass the row's visible limit; a
//                        wave-uniform ballot skips the select when every row
//                        of the tile sees the whole page (section "K1",
//                        "Softmax" bullet)
//   softmax              row max / sum over 128 keys in registers
//   O^T = V^T . P^T      MFMA; P in FP16 (BF16 P would miss 1e-3), FP32 acc
//   epilogue             partial_o = O / l * v_scale (FP32), lse = m + ln l
//
// Computing S^T rather than S leaves each lane holding one query row's
// scores in exactly the register layout the B operand of O^T = V^T P^T
// needs (the key order inside a 32-key block is chosen to make that true),
// and leaves each lane holding one output row for the epilogue, so no
// cross-lane shuffles are needed except the 4-lane row reductions (and, for
// FP32 partials, one swap between half rows that turns the stores into
// whole 128-byte lines).
//
// Routes (Q / KV storage -> MFMA types):
//   F32   : f32 / f32    -> QK 16x16x4 f32, PV 16x16x4 f32
//   BF16  : bf16 / bf16  -> QK 16x16x32 bf16, PV 16x16x32 f16 with V scaled by
//           a power of two per page so every BF16 value is exact in FP16
//   F16   : f16 / f16    -> QK and PV 16x16x32 f16
//   Q8KV4 : e4m3 / nvfp4 -> NVFP4 dequantised once per page to E4M3 (exact
//           product, one rounding; section "Build the prefill for SM107"),
//           QK 16x16x32 fp8, V E4M3 -> FP16 (exact), PV 16x16x32 f16
//   Q8KV8 : e4m3 / e4m3  -> per-tensor scaled FP8 cache: K copied as is, QK
//           16x16x32 fp8, V E4M3 -> FP16 (exact), PV 16x16x32 f16
#include <type_traits>
#include <utility>

#include "launch.h"

namespace msa {
namespace {

constexpr int PAGE = 128;
constexpr int NT = PAGE / 16;  // key tiles of 16 keys
constexpr int THREADS = 256;
constexpr bool kPipelineLds = true;  // batch a chunk's LDS operand reads ahead of its MFMAs
constexpr int NWAVES = THREADS / kWave;

template <int ROUTE> struct RouteInfo;
template <> struct RouteInfo<kRouteF32> { static constexpr int QB = 4; static constexpr bool F16PV = false; };
template <> struct RouteInfo<kRouteBF16> { static constexpr int QB = 2; static constexpr bool F16PV = true; };
template <> struct RouteInfo<kRouteF16> { static constexpr int QB = 2; static constexpr bool F16PV = true; };
template <> struct RouteInfo<kRouteQ8KV4> { static constexpr int QB = 1; static constexpr bool F16PV = true; };
template <> struct RouteInfo<kRouteQ8KV8> { static constexpr int QB = 1; static constexpr bool F16PV = true; };

// Key (in-page offset) carried by A-operand row m of key tile t.  For FP16
// PV the keys of tiles 2b and 2b+1 interleave so that the four S^T registers
// of a lane in both tiles are 8 consecutive keys of 32-key block b.
template <int ROUTE> __device__ __forceinline__ int key_of(int t, int m) {
  if constexpr (ROUTE == kRouteF32) return t * 16 + m;
  else return (t >> 1) * 32 + (m >> 2) * 8 + (t & 1) * 4 + (m & 3);
}
template <int ROUTE> __device__ __forceinline__ int row_of_key(int k) {
  if constexpr (ROUTE == kRouteF32) return k & 15;
  else return (k & 3) | (((k >> 3) & 3) << 2);
}

template <int ROUTE, int D> struct Geom {
  static constexpr int QB = RouteInfo<ROUTE>::QB;
  static constexpr int RB = D * QB;          // bytes of one K row in LDS
  static constexpr int CPR = RB / 16;        // 16-byte chunks per K row
  static constexpr int LANE_CH = CPR / 4;    // chunks of the row one lane holds
  static constexpr int SWZ_SHIFT = CPR >= 16 ? 0 : (CPR == 8 ? 1 : 2);
  static constexpr int K_BYTES = PAGE * RB;
  static constexpr int VROW_F32 = D * 4 + 16;  // padded V row (FP32 route)
  static constexpr int V_BYTES = RouteInfo<ROUTE>::F16PV ? D * PAGE * 2 : PAGE * VROW_F32;
  static constexpr int QPF = ROUTE == kRouteF32 ? 1 : (LANE_CH <= 2 ? 3 : 2);  // Q prefetch depth (tiles)
  static constexpr int ENT_BYTES = kMaxChunk * (int)sizeof(PlanEntry);  // the unit's entries
  static constexpr int LDS = K_BYTES + V_BYTES + 64 + ENT_BYTES;
};

// XOR swizzle of the 16-byte chunks of K row `key`, a function of the
// A-operand row r = row_of_key(key) the key feeds.  One ds_read_b128 has
// each quarter wave read one chunk of rows r = 0..15; which swizzles keep
// those reads apart on the LDS banks of gfx950 was measured (LDS probe,
// bytes per clock and CU; the plain row index conflicts two-way, ~115-120):
//   128-byte rows (FP8, d 128), keys of key_of:     (r ^ r >> 3) & 7   223
//   256-byte rows (16-bit, d 128), keys of key_of:  (r & 3) << 2 | r >> 2   223
//   256-byte rows (FP32, d 64), consecutive keys:   r bit-reversed   223
// Other row widths keep r shifted down to the row's chunk count.
template <int ROUTE, int D> __device__ __forceinline__ int k_swz(int key) {
  using Gm = Geom<ROUTE, D>;
  const int r = row_of_key<ROUTE>(key);
  if constexpr (Gm::RB == 128 && ROUTE != kRouteF32) return (r ^ (r >> 3)) & 7;
  else if constexpr (Gm::RB == 256 && ROUTE != kRouteF32) return ((r & 3) << 2) | (r >> 2);
  else if constexpr (Gm::RB == 256) return (int)(__builtin_bitreverse32((uint32_t)r) >> 28);
  else return r >> Gm::SWZ_SHIFT;
}
// Byte offset of 16-byte chunk c of K row `key`.
template <int ROUTE, int D> __device__ __forceinline__ int k_off(int key, int c) {
  using Gm = Geom<ROUTE, D>;
  return key * Gm::RB + ((c ^ k_swz<ROUTE, D>(key)) << 4);
}
// Byte offset of the 16-byte chunk holding keys [8c, 8c+8) of V^T row dv.
__device__ __forceinline__ int vt_off(int dv, int c) { return dv * (PAGE * 2) + ((c ^ (dv & 15)) << 4); }

template <typename T> __device__ __forceinline__ T ld(const void *p) { return *(const T *)p; }

// x of lane (l ^ 8) within each 16-lane row (DPP row_ror:8).
__device__ __forceinline__ uint32_t swap_half_row(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, true);
}
// On the lanes of the 4-lane banks in BANKS (0x3: lanes 0-7 of each 16-lane
// row, 0xc: lanes 8-15) x of lane (l ^ 8); elsewhere `keep` (one DPP move).
template <int BANKS>
__device__ __forceinline__ uint32_t from_half_row(uint32_t keep, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)keep, (int)x, 0x128, 0xf, BANKS, false);
}

// f(integral_constant<J>) for J = 0 .. N-1, unrolled at compile time.
template <typename F, int... Js>
__device__ __forceinline__ void for_each_index(F &&f, std::integer_sequence<int, Js...>) {
  (f(std::integral_constant<int, Js>{}), ...);
}

// Four partial-output values as 16-bit words (RNE), two per dword.
template <int PO> __device__ __forceinline__ u32x2 pack4_partial(f32x4 v) {
  if constexpr (PO == MSA_F16) {
    return u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
  } else {
    return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// ------------------------------------------------------------ page loading

// F32 / BF16 / F16: K rows copied as-is (swizzled); V transposed to FP16
// (or kept [key][d] in FP32).  Returns the factor folded into v_scale.
template <int ROUTE, int D>
__device__ __forceinline__ float load_page_float(const PageArgs &a, int phys, int g, uint8_t *sK,
                                                 uint8_t *sV, float *sRed) {
  using Gm = Geom<ROUTE, D>;
  const int tid = threadIdx.x;
  const uint8_t *kb = a.k_cache + (int64_t)phys * a.kv_stride_page + (int64_t)g * a.kv_stride_head;
  const uint8_t *vb = a.v_cache + (int64_t)phys * a.kv_stride_page + (int64_t)g * a.kv_stride_head;
  // K
  constexpr int KCH = PAGE * Gm::CPR / THREADS;
  u32x4 kreg[KCH];
#pragma unroll
  for (int it = 0; it < KCH; ++it) {
    const int q = it * THREADS + tid, key = q / Gm::CPR, c = q % Gm::CPR;
    kreg[it] = ld<u32x4>(kb + key * a.kv_stride_tok + c * 16);
  }
#pragma unroll
  for (int it = 0; it < KCH; ++it) {
    const int q = it * THREADS + tid, key = q / Gm::CPR, c = q % Gm::CPR;
    *(u32x4 *)(sK + k_off<ROUTE, D>(key, c)) = kreg[it];
  }
  if constexpr (ROUTE == kRouteF32) {
    constexpr int VCH = PAGE * D / 4 / THREADS;  // 16-byte chunks per thread
#pragma unroll
    for (int it = 0; it < VCH; ++it) {
      const int q = it * THREADS + tid, key = q / (D / 4), c = q % (D / 4);
      *(u32x4 *)(sV + key * Gm::VROW_F32 + c * 16) = ld<u32x4>(vb + key * a.kv_stride_tok + c * 16);
    }
    return 1.0f;
  } else {
    // thread -> key pair kp, d block db of D/4 elements
    const int kp = tid & 63, db = tid >> 6;
    constexpr int DB = D / 4;
    constexpr int NCH = DB * 2 / 16;  // 16-byte chunks per key
    u32x4 v0[NCH], v1[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      v0[c] = ld<u32x4>(vb + (2 * kp) * a.kv_stride_tok + db * DB * 2 + c * 16);
      v1[c] = ld<u32x4>(vb + (2 * kp + 1) * a.kv_stride_tok + db * DB * 2 + c * 16);
    }
    float scale = 1.0f, vfac = 1.0f;
    if constexpr (ROUTE == kRouteBF16) {
      // power-of-two scale so that max|v| * scale lies in [2^14, 2^15):
      // every BF16 value (8-bit significand) is then exact in FP16 unless it
      // is below 2^-14 of the page maximum.
      uint32_t mx = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = v0[c][w] & 0x7fff7fffu, a1 = v1[c][w] & 0x7fff7fffu;
          mx = max(mx, max(max(a0 & 0xffffu, a0 >> 16), max(a1 & 0xffffu, a1 >> 16)));
        }
      // wave max then block max (bf16 bit patterns of |v| order like values)
      for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
      if ((tid & 63) == 0) ((uint32_t *)sRed)[tid >> 6] = mx;
      __syncthreads();
      mx = ((uint32_t *)sRed)[0];
#pragma unroll
      for (int w = 1; w < NWAVES; ++w) mx = max(mx, ((uint32_t *)sRed)[w]);
      const float vmax = bf16_bits_to_f32(mx);
      int e = 0;
      if (vmax > 0.0f && vmax < INFINITY) {
        int x;
        (void)frexpf(vmax, &x);
        e = min(100, max(-100, 15 - x));
      }
      scale = __uint_as_float((uint32_t)(127 + e) << 23);
      vfac = __uint_as_float((uint32_t)(127 - e) << 23);
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int dv = db * DB + c * 8 + w * 2 + hh;
          const uint32_t b0 = hh ? (v0[c][w] >> 16) : (v0[c][w] & 0xffffu);
          const uint32_t b1 = hh ? (v1[c][w] >> 16) : (v1[c][w] & 0xffffu);
          uint32_t word;
          if constexpr (ROUTE == kRouteBF16) {
            word = pack_f16x2(bf16_bits_to_f32(b0) * scale, bf16_bits_to_f32(b1) * scale);
          } else {
            word = b0 | (b1 << 16);
          }
          *(uint32_t *)(sV + vt_off(dv, kp >> 2) + ((kp & 3) << 2)) = word;
        }
    return vfac;
  }
}

// Q8KV8: K rows copied as E4M3 (swizzled); V converted E4M3 -> FP16 (exact)
// and stored transposed for PV, key pairs packed as FP16x2 words.
template <int D>
__device__ __forceinline__ void load_page_fp8(const PageArgs &a, int phys, int g, uint8_t *sK,
                                              uint8_t *sV) {
  using Gm = Geom<kRouteQ8KV8, D>;
  const int tid = threadIdx.x;
  const uint8_t *kb = a.k_cache + (int64_t)phys * a.kv_stride_page + (int64_t)g * a.kv_stride_head;
  const uint8_t *vb = a.v_cache + (int64_t)phys * a.kv_stride_page + (int64_t)g * a.kv_stride_head;
  // thread -> key pair kp, block db of D/4 dims (V)
  const int kp = tid & 63, db = tid >> 6;
  constexpr int DB = D / 4;
  constexpr int NCH = DB / 16;  // 16-byte chunks per key and block
  u32x4 v0[NCH], v1[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    v0[c] = ld<u32x4>(vb + (2 * kp) * a.kv_stride_tok + db * DB + c * 16);
    v1[c] = ld<u32x4>(vb + (2 * kp + 1) * a.kv_stride_tok + db * DB + c * 16);
  }
  constexpr int KCH = PAGE * Gm::CPR / THREADS;
  u32x4 kreg[KCH];
#pragma unroll
  for (int it = 0; it < KCH; ++it) {
    const int q = it * THREADS + tid, key = q / Gm::CPR, c = q % Gm::CPR;
    kreg[it] = ld<u32x4>(kb + key * a.kv_stride_tok + c * 16);
  }
#pragma unroll
  for (int it = 0; it < KCH; ++it) {
    const int q = it * THREADS + tid, key = q / Gm::CPR, c = q % Gm::CPR;
    *(u32x4 *)(sK + k_off<kRouteQ8KV8, D>(key, c)) = kreg[it];
  }
  const int col = (kp & 3) << 2;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const auto a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)v0[c][w], false);
      const auto a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)v1[c][w], false);
      const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)v0[c][w], true);
      const auto b1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)v1[c][w], true);
      const int dv = db * DB + c * 16 + w * 4;
      const float f[4][2] = {{a0[0], a1[0]}, {a0[1], a1[1]}, {b0[0], b1[0]}, {b0[1], b1[1]}};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(uint32_t *)(sV + vt_off(dv + e, kp >> 2) + col) =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[e][0], f[e][1]));
    }
}

// Q8KV4: NVFP4 K/V dequantised to E4M3 once per page, through per-block
// magnitude tables (see nvfp4_mag_table): K stays E4M3 for the FP8 QK
// product, V becomes FP16 (exact) and is stored transposed for PV.
template <int D>
__device__ __forceinline__ void load_page_nvfp4(const PageArgs &a, int phys, int g, uint8_t *sK,
                                                uint8_t *sV) {
  static_assert(D == 128, "Q8KV4 route is built for head_dim 128");
  const int tid = threadIdx.x;
  const int64_t kvo = (int64_t)phys * a.kv_stride_page + (int64_t)g * a.kv_stride_head;
  const int64_t sfo = (int64_t)phys * a.sf_stride_page + (int64_t)g * a.sf_stride_head;
  // V first: its loads are issued before K's conversion work.
  const int kp = tid & 63, db = tid >> 6;  // key pair, block of 32 dims
  u32x4 vcw[2];
  uint32_t vsf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int key = 2 * kp + kk;
    vcw[kk] = ld<u32x4>(a.v_cache + kvo + key * a.kv_stride_tok + db * 16);
    vsf[kk] = ld<uint16_t>(a.v_sf + sfo + key * a.sf_stride_tok + db * 2);
  }
  {  // K: thread -> key tid/2, half tid%2 of the row (64 elements = 4 blocks)
    const int key = tid >> 1, half = tid & 1;
    const uint8_t *cp = a.k_cache + kvo + key * a.kv_stride_tok + half * (D / 4);
    const uint32_t sf = ld<uint32_t>(a.k_sf + sfo + key * a.sf_stride_tok + half * (D / 32));
    const u32x4 c0 = ld<u32x4>(cp), c1 = ld<u32x4>(cp + 16);
    const uint32_t words[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {  // one block: 16 codes -> 16 output bytes
      const uint32_t scale = (sf >> (8 * ch)) & 0xffu;
      const u32x2 tab = nvfp4_mag_table(scale);
      const uint32_t flip = (scale & 0x80u) ? 0x80808080u : 0u;
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        out[w] = nvfp4_lookup4(words[ch * 2 + (w >> 1)] >> (16 * (w & 1)), tab, flip);
      *(u32x4 *)(sK + k_off<kRouteQ8KV4, D>(key, half * 4 + ch)) = out;
    }
  }
  // V: per key, FP16 pairs (dims 2i, 2i+1) of the 32 dims of block db
  uint32_t hw[2][16];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const Nvfp4F16Tab tab = nvfp4_f16_tab((vsf[kk] >> (8 * b)) & 0xffu);
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // 4 codes -> two FP16 pairs
        const u32x2 w = nvfp4_lookup4_f16(vcw[kk][b * 2 + (q >> 1)] >> (16 * (q & 1)), tab);
        hw[kk][b * 8 + q * 2] = w[0];
        hw[kk][b * 8 + q * 2 + 1] = w[1];
      }
    }
  // V^T rows dv, dv+1 get the (key 2kp, key 2kp+1) pairs
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int dv = db * 32 + 2 * i;
    const int col = ((kp & 3) << 2);
    *(uint32_t *)(sV + vt_off(dv, kp >> 2) + col) = __builtin_amdgcn_perm(hw[1][i], hw[0][i], 0x05040100u);
    *(uint32_t *)(sV + vt_off(dv + 1, kp >> 2) + col) = __builtin_amdgcn_perm(hw[1][i], hw[0][i], 0x07060302u);
  }
}

// ------------------------------------------------------------ the kernel

// PO: dtype of partial_o (MSA_F32, or MSA_BF16 / MSA_F16 to halve the
// partial bytes; the LSE stays FP32).
template <int ROUTE, int D, int PO>
__global__ void __launch_bounds__(THREADS, (Geom<ROUTE, D>::LDS <= 53 * 1024 ? 3 : (Geom<ROUTE, D>::LDS <= 80 * 1024 ? 2 : 1)))
    k1_page_attend(const PageArgs a) {
  using Gm = Geom<ROUTE, D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Gm::LDS];
  uint8_t *sK = smem;
  uint8_t *sV = smem + Gm::K_BYTES;
  float *sRed = (float *)(smem + Gm::K_BYTES + Gm::V_BYTES);
  PlanEntry *sEnt = (PlanEntry *)(smem + Gm::K_BYTES + Gm::V_BYTES + 64);

  // ---- work unit.  Units go to the XCDs round robin (workgroup i runs on
  // XCD i mod 8): their sizes vary with the request (a long chunk's pages
  // carry many more queries), and contiguous unit ranges per XCD left some
  // XCDs with several times the work of others.  The slice ordering of the
  // units still keeps the queries all XCDs read at one time to one slice.
  // The unit's record is read before the unit count (both loads in flight at
  // once): the grid never exceeds the record array, whose tail past the
  // count is simply not used.
  const int unit = blockIdx.x;
  const PageUnit wu = ((const PageUnit *)(a.ws + a.lay.units))[unit];
  const int num_units = ((const int32_t *)(a.ws + a.lay.meta))[0];
  if (unit >= num_units) return;
  const int e_begin = wu.e_begin, e_count = wu.e_count, g = wu.g, phys = wu.phys;

  // ---- the unit's entries -> LDS (so the tile loop issues no dependent
  // global loads behind its own stores: vmcnt counts loads and stores alike)
  {
    const PlanEntry *ge = (const PlanEntry *)(a.ws + a.lay.entries) + e_begin;
    for (int i = threadIdx.x; i < e_count; i += THREADS) sEnt[i] = ge[i];
  }

  // ---- page -> LDS
  float vfac = 1.0f;
  if constexpr (ROUTE == kRouteQ8KV4) load_page_nvfp4<D>(a, phys, g, sK, sV);
  else if constexpr (ROUTE == kRouteQ8KV8) load_page_fp8<D>(a, phys, g, sK, sV);
  else vfac = load_page_float<ROUTE, D>(a, phys, g, sK, sV, sRed);
  __syncthreads();
  const float out_scale = a.v_scale * vfac;

  const PlanEntry *entries = sEnt;
  float *dump = (float *)(a.ws + a.lay.dump);  // scratch row for masked-off stores
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
  const int n = lane & 15, grp = lane >> 4;
  const int G = a.G;
  const int rows_total = e_count * G;
  const int n_tiles = (rows_total + 15) >> 4;
  const uint8_t *qbase = (const uint8_t *)a.q;

  // Row of this lane in a tile.  Rows past the end (ragged last tile, or the
  // prefetch beyond the last tile) read entry 0 / head 0 -- always in bounds --
  // and never store.
  struct RowInfo {
    int tok, slot, limit, h;
    bool active;
  };
  auto row_of = [&](int tile) {
    RowInfo ri;
    const int rho = tile * 16 + n;
    ri.active = rho < rows_total;
    const int e = ri.active ? rho / G : 0;
    const int hl = ri.active ? rho - e * G : 0;
    const PlanEntry ent = entries[e];
    ri.tok = ent.tok_slot >> 8;
    ri.slot = ent.tok_slot & 255;
    ri.limit = ri.active ? ent.limit : -1;
    ri.h = g * G + hl;
    return ri;
  };
  // Q operand: this lane's contiguous quarter of its row
  auto load_q = [&](const RowInfo &ri, u32x4 *q) {
    const uint8_t *qp = qbase + ((int64_t)ri.tok * a.q_stride_tok + (int64_t)ri.h * a.q_stride_head) * Gm::QB +
                        grp * (Gm::RB / 4);
#pragma unroll
    for (int c = 0; c < Gm::LANE_CH; ++c) q[c] = ld<u32x4>(qp + c * 16);
  };

  // ---- software pipeline: the Q fragments of the next QPF tiles are in
  // flight while a tile is computed.  Each prefetch in the prologue is
  // followed by one tile's worth of (scratch) stores so that the memory-op
  // pattern at loop entry matches the back-edge: the compiler's wait before
  // a tile's MFMAs then covers its own Q loads only, never the partial-output
  // stores still in flight.
  constexpr int PF = Gm::QPF;
  constexpr int MT = D / 16;
  RowInfo ri[PF];
  u32x4 qb[PF][Gm::LANE_CH];
#pragma unroll
  for (int f = 0; f < PF; ++f) {
    ri[f] = row_of(wave + f * NWAVES);
    load_q(ri[f], qb[f]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *(f32x4 *)(dump + grp * 4 + mt * 16) = f32x4{0.f, 0.f, 0.f, 0.f};
    dump[D + lane] = 0.0f;
  }
  const float sc = a.scale_log2;  // > 0 (validated on the host)

  // One tile; J (compile-time) names the prefetch buffer holding its Q.
  // The loop below is unrolled PF times so each buffer is consumed by its
  // QK and refilled in place -- rotating buffers through register moves
  // would wait on loads still in flight.
  auto step = [&](auto J_, const int tile) {
#pragma clang fp contract(off)
    constexpr int J = decltype(J_)::value;
    // The page in LDS is loop-invariant; without this compiler-only fence the
    // K/V fragment reads are hoisted out of the loop into (spilled) registers.
    __asm__ volatile("" ::: "memory");
    const int tok = ri[J].tok, slot = ri[J].slot, limit = ri[J].limit, h = ri[J].h;
    const bool active = ri[J].active;
    // ---- S^T = K Q^T  (chunk-outer so each K fragment is used once, at once)
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (Gm::QB == 1 && Gm::LANE_CH == 2) {
      // FP8 rows of 128: a lane's 32 bytes of each K row against its 32 bytes
      // of the Q row, one K = 128 MFMA per key tile; the fragments of four
      // key tiles are read before their MFMAs
#pragma unroll
      for (int t0 = 0; t0 < NT; t0 += 4) {
        u32x4 kf[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            kf[t][c] = *(const u32x4 *)(sK + k_off<ROUTE, D>(key_of<ROUTE>(t0 + t, n), grp * 2 + c));
        if constexpr (kPipelineLds) __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t0 + t] = mfma_fp8_k128(kf[t][0], kf[t][1], qb[J][0], qb[J][1], acc[t0 + t]);
      }
    } else
#pragma unroll
    for (int c = 0; c < Gm::LANE_CH; ++c) {
      // all of this chunk's K fragments are read before its MFMAs (the empty
      // asm keeps the compiler from sinking the reads next to their uses),
      // so the LDS latency is paid once per chunk, not once per MFMA pair
      u32x4 kf[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        kf[t] = *(const u32x4 *)(sK + k_off<ROUTE, D>(key_of<ROUTE>(t, n), grp * Gm::LANE_CH + c));
      if constexpr (kPipelineLds) __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 kr = kf[t];
        const u32x4 qr = qb[J][c];
        if constexpr (ROUTE == kRouteF32) {
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[t] = mfma_f32(__uint_as_float(kr[w]), __uint_as_float(qr[w]), acc[t]);
        } else if constexpr (ROUTE == kRouteBF16) {
          acc[t] = mfma_bf16(kr, qr, acc[t]);
        } else if constexpr (ROUTE == kRouteF16) {
          acc[t] = mfma_f16(kr, qr, acc[t]);
        } else {
          acc[t] = mfma_fp8(u32x2{kr[0], kr[1]}, u32x2{qr[0], qr[1]}, acc[t]);
          acc[t] = mfma_fp8(u32x2{kr[2], kr[3]}, u32x2{qr[2], qr[3]}, acc[t]);
        }
      }
    }

    // ---- softmax phase at raised wave priority (back to 0 before PV): the
    // VALU-bound stretch of one wave gets issue slots first while the other
    // waves of the SIMD keep the matrix cores busy (measured ~1-4 %)
    __builtin_amdgcn_s_setprio(1);

    // ---- prefetch tile + PF * NWAVES (inactive, in-bounds rows past the end)
    ri[J] = row_of(tile + PF * NWAVES);
    load_q(ri[J], qb[J]);

    // ---- causal mask, only for tiles where some row sees part of the page
    // (a wave-uniform branch; history pages and most own-page tiles skip it)
    if (!__all(limit >= PAGE - 1)) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key_of<ROUTE>(t, 4 * grp + i) > limit) acc[t][i] = -INFINITY;
    }
    // ---- scores in log2 units and their row max.  Scaling before the max
    // keeps the largest key's weight exactly 1 (a single visible key then
    // reproduces its value row bit for bit) -- provided the product is
    // rounded before the subtraction, hence no FMA contraction in this step.
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] *= sc;
      m = fmaxf(m, fmaxf(fmaxf(acc[t][0], acc[t][1]), fmaxf(acc[t][2], acc[t][3])));
    }
    m = quarter_reduce<true>(m);
    const float msc = (m == -INFINITY) ? 0.0f : m;  // inactive row: stay finite

    // ---- P = exp2(S - m).  l (exact FP32 sum) gives the LSE; lp, the sum of
    // the P values PV actually uses, normalises the output so that its
    // weights sum to one.
    float l = 0.0f, lp = 0.0f;
    uint32_t pk[NT * 2];  // FP16 pairs of P (16-bit PV routes)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(acc[t][i] - msc);
        acc[t][i] = p;
        l += p;
      }
      if constexpr (RouteInfo<ROUTE>::F16PV) {
        pk[2 * t] = pack_f16x2(acc[t][0], acc[t][1]);
        pk[2 * t + 1] = pack_f16x2(acc[t][2], acc[t][3]);
        lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[2 * t]), f16x2{(_Float16)1.0f, (_Float16)1.0f}, lp, false);
        lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk[2 * t + 1]), f16x2{(_Float16)1.0f, (_Float16)1.0f}, lp, false);
      }
    }
    l = quarter_reduce<false>(l);
    if constexpr (RouteInfo<ROUTE>::F16PV) {
      lp = quarter_reduce<false>(lp);
    } else {
      lp = l;
    }

    __builtin_amdgcn_s_setprio(0);

    // ---- O^T = V^T P^T
    f32x4 o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (RouteInfo<ROUTE>::F16PV) {
#pragma unroll
      for (int kb = 0; kb < PAGE / 32; ++kb) {
        const u32x4 pf = {pk[4 * kb], pk[4 * kb + 1], pk[4 * kb + 2], pk[4 * kb + 3]};
        u32x4 vf[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) vf[mt] = *(const u32x4 *)(sV + vt_off(mt * 16 + n, kb * 4 + grp));
        if constexpr (kPipelineLds) __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt] = mfma_f16(vf[mt], pf, o[mt]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = t * 16 + 4 * grp + i;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const float vv = *(const float *)(sV + key * Gm::VROW_F32 + (mt * 16 + n) * 4);
            o[mt] = mfma_f32(vv, acc[t][i], o[mt]);
          }
        }
    }

    // ---- epilogue: this lane holds row n, columns 16*mt + 4*grp + [0,4).
    // The stores are unconditional -- rows without a destination (ragged
    // last tile; the LSE of lanes other than the row's first) write to a
    // scratch row of the workspace -- so the compiler can count the stores
    // in flight across the loop back-edge.
    const float inv = out_scale / lp;  // IEEE division (v_rcp_f32 is not exact even at 1.0)
    const int64_t row = (int64_t)tok * a.Hq + h;
    void *dst = active ? a.partial_o : (void *)dump;
    const int64_t po_off = active ? (int64_t)slot * a.po_split_stride + row * a.po_row_stride + grp * 4 : grp * 4;
    if constexpr (PO == MSA_F32) {
      // Whole 128-byte lines, streamed past the caches: lanes n and n + 8 of a
      // quarter swap one of each pair of column tiles (a DPP move within the
      // 16-lane row), so each store instruction covers 128 contiguous bytes
      // of 8 rows -- tiles 2k, 2k+1 of rows 0-7, then of rows 8-15 -- instead
      // of 64 bytes of 16 rows.  Non-temporal stores of whole lines go to
      // memory without a read for ownership or a merge in L2; the combine
      // reads the partials from HBM in any case.
      // Byte offsets from partial_o (the scratch row as well), so that the
      // exchanged address still derives from a global pointer and the stores
      // stay global stores (a flat store would also count as an LDS access).
      uint8_t *const base = (uint8_t *)a.partial_o;
      const int64_t own_off = ((uint8_t *)dst - base) + po_off * 4;
      const int64_t partner_off = (int64_t)(((uint64_t)swap_half_row((uint32_t)((uint64_t)own_off >> 32)) << 32) |
                                            swap_half_row((uint32_t)own_off));
      const bool lo_half = n < 8;
      // rows 0-7 of each tile pair: lanes 0-7 write their own row, lanes 8-15
      // the partner's second tile; rows 8-15 the other way round
      uint8_t *const pa = base + (lo_half ? own_off : partner_off + 64);
      uint8_t *const pb = base + (lo_half ? partner_off : own_off + 64);
#pragma unroll
      for (int k = 0; k < MT / 2; ++k) {
        const f32x4 e0 = o[2 * k] * inv, e1 = o[2 * k + 1] * inv;
        f32x4 va, vb;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // va: e0 on lanes 0-7, the partner's e1 on lanes 8-15;
          // vb: the partner's e0 on lanes 0-7, e1 on lanes 8-15
          va[w] = __uint_as_float(from_half_row<0xc>(__float_as_uint(e0[w]), __float_as_uint(e1[w])));
          vb[w] = __uint_as_float(from_half_row<0x3>(__float_as_uint(e1[w]), __float_as_uint(e0[w])));
        }
        __builtin_nontemporal_store(va, (f32x4 *)(pa + 128 * k));
        __builtin_nontemporal_store(vb, (f32x4 *)(pb + 128 * k));
      }
    } else if ((a.po_row_stride | a.po_split_stride) % 8 != 0) {
      // 16-bit partials whose rows are only 8-byte aligned: 8 bytes per lane
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store_partial4<PO>(dst, po_off + mt * 16, o[mt] * inv);
    } else {
      // 16-bit partials: 16 bytes per lane per store.  The lane groups of a
      // row (grp 0-3, 4 columns each per tile) pair up, 0 with 1 and 2 with 3,
      // through one row swap per word: the even group keeps tile 2k's words
      // and takes its partner's, the odd group tile 2k+1's, so each lane holds
      // 8 consecutive columns and a store covers 64 contiguous bytes of each
      // of the 16 rows (4 stores per tile instead of 8).
      // Then, as for FP32 partials, lanes n and n + 8 of each 16-lane row swap
      // one of each pair of 64-byte blocks, so a store writes whole 128-byte
      // lines of 8 rows (blocks 2j, 2j+1 of rows 0-7, then of rows 8-15),
      // non-temporally; addresses are byte offsets from partial_o (the
      // scratch row's too).
      const int64_t rbase = po_off - grp * 4;  // the row's first element
      const int colo = ((grp & 1) << 4) | ((grp >> 1) << 3);
      const bool even = (grp & 1) == 0;
      u32x4 v[MT / 2];
#pragma unroll
      for (int k = 0; k < MT / 2; ++k) {
        const u32x2 w0 = pack4_partial<PO>(o[2 * k] * inv), w1 = pack4_partial<PO>(o[2 * k + 1] * inv);
        const auto sx = __builtin_amdgcn_permlane16_swap(w0[0], w1[0], false, false);
        const auto sy = __builtin_amdgcn_permlane16_swap(w0[1], w1[1], false, false);
        v[k] = even ? u32x4{w0[0], w0[1], sx[1], sy[1]} : u32x4{sx[0], sy[0], w1[0], w1[1]};
      }
      uint8_t *const base = (uint8_t *)a.partial_o;
      const int64_t own_off = ((uint8_t *)dst - base) + (rbase + colo) * 2;
      const int64_t partner_off = (int64_t)(((uint64_t)swap_half_row((uint32_t)((uint64_t)own_off >> 32)) << 32) |
                                            swap_half_row((uint32_t)own_off));
      const bool lo_half = n < 8;
      uint8_t *const pa = base + (lo_half ? own_off : partner_off + 64);
      uint8_t *const pb = base + (lo_half ? partner_off : own_off + 64);
#pragma unroll
      for (int j = 0; j < MT / 4; ++j) {
        u32x4 va, vb;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          va[w] = from_half_row<0xc>(v[2 * j][w], v[2 * j + 1][w]);
          vb[w] = from_half_row<0x3>(v[2 * j + 1][w], v[2 * j][w]);
        }
        __builtin_nontemporal_store(va, (u32x4 *)(pa + 128 * j));
        __builtin_nontemporal_store(vb, (u32x4 *)(pb + 128 * j));
      }
    }
    float *ldst = (active && grp == 0) ? a.partial_lse + (int64_t)slot * a.pl_split_stride + row
                                       : dump + D + lane;
    *ldst = (msc + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
  };

  if (wave < n_tiles) {
    for (int tile = wave;;) {
      bool done = false;  // wave-uniform
      for_each_index([&](auto J) {
        if (!done) {
          step(J, tile);
          done = (tile += NWAVES) >= n_tiles;
        }
      }, std::make_integer_sequence<int, PF>{});
      if (done) break;
    }
  }
}

template <int ROUTE, int D>
hipError_t launch_route(const PageArgs &a, hipStream_t s) {
  const int64_t grid = a.max_units;
  if (grid == 0) return hipSuccess;
  if constexpr (ROUTE == kRouteF32) {  // FP32 partials only (checked on the host)
    k1_page_attend<ROUTE, D, MSA_F32><<<(unsigned)grid, THREADS, 0, s>>>(a);
  } else {
    switch (a.po_dtype) {
      case MSA_BF16: k1_page_attend<ROUTE, D, MSA_BF16><<<(unsigned)grid, THREADS, 0, s>>>(a); break;
      case MSA_F16: k1_page_attend<ROUTE, D, MSA_F16><<<(unsigned)grid, THREADS, 0, s>>>(a); break;
      default: k1_page_attend<ROUTE, D, MSA_F32><<<(unsigned)grid, THREADS, 0, s>>>(a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

size_t page_attend_lds_bytes() {
  constexpr int sizes[] = {Geom<kRouteF32, 64>::LDS,   Geom<kRouteF32, 128>::LDS,
                           Geom<kRouteBF16, 64>::LDS,  Geom<kRouteBF16, 128>::LDS,
                           Geom<kRouteF16, 64>::LDS,   Geom<kRouteF16, 128>::LDS,
                           Geom<kRouteQ8KV4, 128>::LDS, Geom<kRouteQ8KV8, 64>::LDS,
                           Geom<kRouteQ8KV8, 128>::LDS};
  int m = 0;
  for (int x : sizes) m = x > m ? x : m;
  return (size_t)m;
}

hipError_t launch_page_attend(const PageArgs &a, hipStream_t s) {
  switch (a.route) {
    case kRouteF32:
      return a.D == 64 ? launch_route<kRouteF32, 64>(a, s) : launch_route<kRouteF32, 128>(a, s);
    case kRouteBF16:
      return a.D == 64 ? launch_route<kRouteBF16, 64>(a, s) : launch_route<kRouteBF16, 128>(a, s);
    case kRouteF16:
      return a.D == 64 ? launch_route<kRouteF16, 64>(a, s) : launch_route<kRouteF16, 128>(a, s);
    case kRouteQ8KV4:
      return launch_route<kRouteQ8KV4, 128>(a, s);
    case kRouteQ8KV8:
      return a.D == 64 ? launch_route<kRouteQ8KV8, 64>(a, s) : launch_route<kRouteQ8KV8, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

// Standalone device dequantisation (the routines the attention uses for K
// and for V).  Element i sits at position i % 4 of its 4-code word, so
// every position of the lookups is exercised.
namespace {
__global__ void nvfp4_dequant_kernel(const uint8_t *codes, const uint8_t *scales, uint8_t *out,
                                     int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)nvfp4_to_e4m3(codes[i] & 15u, scales[i], (int)(i & 3));
}
__global__ void nvfp4_dequant_f16_kernel(const uint8_t *codes, const uint8_t *scales, uint16_t *out,
                                         int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint16_t)nvfp4_to_f16(codes[i] & 15u, scales[i], (int)(i & 3));
}
}  // namespace

hipError_t launch_nvfp4_dequant(const uint8_t *codes, const uint8_t *scales, uint8_t *out,
                                int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  nvfp4_dequant_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(codes, scales, out, n);
  return hipGetLastError();
}

hipError_t launch_nvfp4_dequant_f16(const uint8_t *codes, const uint8_t *scales, uint16_t *out,
                                    int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  nvfp4_dequant_f16_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(codes, scales, out, n);
  return hipGetLastError();
}

}  // namespace msa
