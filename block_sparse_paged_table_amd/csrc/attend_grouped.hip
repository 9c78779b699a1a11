// Attention step of the grouped microblock route (1Cat-vLLM PR 387, section
// "Purpose": eight adjacent query rows share one load of their overlapping
// sparse K/V blocks while each row keeps its exact 4-bit mask), written for
// gfx950.
//
// One workgroup per (group of 8 query tokens, KV head, split).  The group's
// G query heads per token make 8*G (token, head) rows, cut into 16-row
// tiles; wave w owns tile w.  Consecutive groups run on one XCD, and the
// planner lists each split's units in ascending order, so the groups an XCD
// runs together walk the K/V cache in step and mostly hit its L2.
//
// The split's unit list (8 bytes per unit: page, unit in the page, mask)
// streams into an LDS ring of two chunks of 256 entries (32 stages each), a
// chunk loaded 32 stages before its first use.  The units stream through an
// LDS ring of NST stages of 32 keys (8 units) each -- two 16-key tiles, A
// and B -- loaded straight from the cache into LDS (global_load_lds: no
// register staging, no LDS stores): wave w loads unit w of tile A and unit
// w of tile B, each its K rows then its V rows.  Loads run NST - 1 stages
// ahead of the stage being computed, and one barrier per stage both
// publishes a landed stage and frees the slot the next loads reuse.  Inside
// the loop the only memory accesses are these counted loads and LDS
// traffic: a scalar or vector load there would make every later wait also
// wait for the loads in flight.  At head_dim 256 two 32 KiB stages and the
// 4 KiB list ring make 68 KiB of LDS (two workgroups per CU); against
// 16-key stages with the same 32 keys in flight, a stage costs half the
// barriers and softmax steps per key.  K rows are stored as they are in the
// cache with a per-row XOR swizzle of their 16-byte chunks (so that the 16
// rows of one MFMA read spread over the LDS banks); V rows likewise, read
// back transposed.  Per stage and active row tile:
//
//   S^T = K . Q^T      f16 MFMA 16x16x32 per 16-key tile, FP32 accumulate
//                      (K rows from LDS, Q rows held in registers)
//   mask               key i of unit b is visible to the row of token tau iff
//                      bit 4*tau + i of the unit's mask word is set (the
//                      planner folded the causal and tail rules into it)
//   online softmax     running max / sums per row over the 32 keys,
//                      rescaling O when the max grows
//   O^T += V^T . P^T   f16 MFMA 16x16x32 over both tiles: the V^T operand
//                      comes from the untransposed V rows through the gfx950
//                      transposing LDS read (ds_read_b64_tr_b16), and the S^T
//                      accumulators of a lane already hold its P^T operand
//                      (keys 4q..4q+3 of each tile, of its row)
//
// A tile none of whose rows selected any unit of a stage skips it.  Each
// split is an independent softmax: partial_o = O / l * v_scale and lse =
// m + ln l (or -inf with zeros for a row that sees nothing in the split).
//
// Runs: when the (group, KV head, split) grid is small, the host cuts each
// split's list into sub_splits runs of whole stages; one workgroup per run
// writes the run's FP32 partials and LSE into the workspace, and a combine
// (LSE merge over the runs) writes the split's partials.  A small grid
// otherwise leaves most CUs idle while each workgroup walks a long list.
#include <type_traits>

#include "grouped.h"
#include "launch.h"

namespace msa {
namespace {

constexpr int GT = 256;             // threads per workgroup
constexpr int SK = 32;              // keys per stage: two 16-key tiles A and B
constexpr int UPS = SK / 4;         // units per stage: wave w loads units w (tile A) and w + 4 (tile B)
static_assert(UPS == 2 * (GT / kWave), "two units per wave and stage");

typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kListChunk = 256;                // list entries per ring chunk
constexpr int kChunkStages = kListChunk / UPS;  // stages one chunk covers
constexpr int kListRing = 2 * kListChunk;       // entries the LDS ring holds

template <int D> struct GGeom {
  static constexpr int RB = D * 2;                  // K / V row bytes (FP16)
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int LANE_CH = CPR / 4;           // chunks of a Q/K row one lane holds
  static constexpr int K_BYTES = SK * RB;           // one stage's K rows
  static constexpr int TILE_B = 16 * RB;            // tile B's rows follow tile A's (K and V)
  static constexpr int STAGE = 2 * K_BYTES;         // K rows, then V rows
  static constexpr int NST = D == 256 ? 2 : 3;      // ring stages
  static constexpr int RING = NST * STAGE;
  static constexpr int LDS = RING + kListRing * 8;  // K/V ring + list ring
  static constexpr int WGS = LDS <= 53 * 1024 ? 3 : 2;  // workgroups per CU
  static constexpr int ROWS_PER_LOAD = 1024 / RB;   // rows one 1 KiB wave load covers
  static constexpr int LPP = 4 / ROWS_PER_LOAD;     // wave loads per unit and part (K or V)
  static constexpr int ULOADS = 2 * LPP;            // wave loads per unit (K and V rows)
  static constexpr int MT = D / 16;
  static_assert(ROWS_PER_LOAD * RB == 1024 && LPP >= 1, "head_dim 128 or 256");
  static_assert(WGS * LDS <= 160 * 1024, "workgroups per CU");
};

// XOR swizzle of the 16-byte chunks of K row r.  The 16 lanes of a quarter
// wave read one chunk of each of rows 0..15; at head_dim 256 (512-byte rows)
// the row index bit-reversed spreads those reads over the LDS banks of gfx950
// (measured with ds_read_b128: about 200 B per clock and CU against about 115
// for the row index itself, which conflicts); at head_dim 128 the row index.
template <int D> __device__ __forceinline__ int gk_swz(int r) {
  return D == 256 ? (int)(__builtin_bitreverse32((uint32_t)(r & 15)) >> 28) : (r & 15);
}
// XOR swizzle of the chunks of V row r: an even value, so the two chunks of
// one 16-dim block stay adjacent for the transposed reads.
__device__ __forceinline__ int gv_swz(int r) { return (r & 7) << 1; }
// Byte offset of 16-byte chunk c of K row r (r < 32) in a stage.
template <int D> __device__ __forceinline__ int gk_off(int r, int c) {
  return r * GGeom<D>::RB + ((c ^ gk_swz<D>(r)) << 4);
}

// Per-lane constants of the stage loop, computed once.
template <int D> struct LaneOffsets {
  uint32_t k[GGeom<D>::LANE_CH];  // K fragment c of row n of tile A (QK operand), from the slot
  uint32_t v[8];                  // tile A's V^T fragment of dims tile mt (mt & 7; +256 B for mt >= 8)
  uint32_t dk[GGeom<D>::LPP];     // DMA source offsets in the unit, K rows
  uint32_t dv[GGeom<D>::LPP];     //   and V rows
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(const GroupArgs &a, int w) {
  using Gm = GGeom<D>;
  LaneOffsets<D> L;
  const int lane = threadIdx.x & 63, n = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int c = 0; c < Gm::LANE_CH; ++c) L.k[c] = gk_off<D>(n, gq * Gm::LANE_CH + c);
  // transposed V read: lane (gq, r, c) addresses row 4 gq + r at dims
  // 16 mt + 4c .. +3, i.e. chunk 2 mt + c / 2, half c % 2, swizzled
  const int vr = gq * 4 + ((lane >> 2) & 3), vc = lane & 3;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    L.v[j] = Gm::K_BYTES + vr * Gm::RB + (((2 * j + (vc >> 1)) ^ gv_swz(vr)) << 4) + (vc & 1) * 8;
#pragma unroll
  for (int h = 0; h < Gm::LPP; ++h) {
    const int r = w * 4 + h * Gm::ROWS_PER_LOAD + lane / Gm::CPR, pos = lane % Gm::CPR;
    L.dk[h] = (uint32_t)((r & 3) * a.kv_stride_tok) + ((pos ^ gk_swz<D>(r)) << 4);
    L.dv[h] = (uint32_t)((r & 3) * a.kv_stride_tok) + ((pos ^ gv_swz(r)) << 4);
  }
  return L;
}

// Issue this wave's part of one stage: unit `ua` into tile A's rows 4w ..
// 4w+3 and unit `ub` into tile B's (K rows, then V rows), straight into the
// stage's LDS slot from their byte offsets in the caches.  A unit past the
// end of the run is zero-filled instead (its mask is 0, so it adds nothing;
// zeros keep the masked products finite) and issues no load.
template <int D>
__device__ __forceinline__ void issue_unit(const GroupArgs &a, uint8_t *slot, int row0, int64_t uoff, bool real,
                                           const LaneOffsets<D> &L) {
  using Gm = GGeom<D>;
  const int lane = threadIdx.x & 63;
  if (!real) {
#pragma unroll
    for (int h = 0; h < Gm::LPP; ++h) {
      const int r0 = row0 + h * Gm::ROWS_PER_LOAD;
      *(u32x4 *)(slot + r0 * Gm::RB + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      *(u32x4 *)(slot + Gm::K_BYTES + r0 * Gm::RB + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  const uint8_t *kb = a.k_cache + uoff;
  const uint8_t *vb = a.v_cache + uoff;
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS uint8_t *)slot);
#pragma unroll
  for (int h = 0; h < Gm::LPP; ++h)
    lds_dma16(kb, L.dk[h], lds + (row0 + h * Gm::ROWS_PER_LOAD) * Gm::RB);
#pragma unroll
  for (int h = 0; h < Gm::LPP; ++h)
    lds_dma16(vb, L.dv[h], lds + Gm::K_BYTES + (row0 + h * Gm::ROWS_PER_LOAD) * Gm::RB);
}

// Chunk c of a list into LDS ring slot c % 2: entries 256 c .. 256 c + 255
// from `list` (16-byte aligned), of which the first n are wanted.  Wave w
// loads entries 64 w .. 64 w + 63 of the chunk, two per lane on lanes 0..31
// (16 bytes each; lanes whose first entry is not wanted load nothing).
// Counted with the stage loads of the wave (vmcnt).
__device__ __forceinline__ void issue_list_chunk(const uint2 *list, int n, int c, int w, uint2 *sList) {
  const int lane = threadIdx.x & 63;
  const int e = c * kListChunk + w * 64 + 2 * lane;
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(LDS_AS uint8_t *)(sList + (c & 1) * kListChunk + w * 64));
  if (lane < 32 && e < n) lds_dma16((const uint8_t *)list, (uint32_t)e * 8u, lds);
}

// A row's running max may lag its true max by up to 2^kLag (log2 units)
// before O is rescaled: P = 2^(s - m) then stays below 2^kLag, well inside
// FP16, and the rescale of the 64 accumulators runs only when a logit
// exceeds the running max by more than that.
constexpr float kLag = 8.0f;

// PO: dtype of partial_o (MSA_F32, MSA_BF16 or MSA_F16).
template <int D, int PO>
__global__ void __launch_bounds__(GT, GGeom<D>::WGS)
    k_grouped_attend(const GroupArgs a, const uint2 *__restrict__ lists, const int *__restrict__ split_offs) {
  using Gm = GGeom<D>;
  constexpr int MT = Gm::MT, NST = Gm::NST;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Gm::RING];
  // ring of the split's units: {page << 5 | unit in page, mask32}; unit u at u % kListRing
  __shared__ __attribute__((aligned(16))) uint2 sList[kListRing];

  // ---- work item; consecutive groups on one XCD (workgroups are dealt to
  // the 8 XCDs round-robin, and the grid's x size is a multiple of 8)
  const int per_xcd = (a.num_groups + 7) >> 3;
  const int grp = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (grp >= a.num_groups) return;  // the whole workgroup, before any barrier
  const int g = blockIdx.y;
  const int split = blockIdx.z / a.sub_splits, run = blockIdx.z - split * a.sub_splits;
  const int64_t li = (int64_t)g * a.num_groups + grp;
  const int *soff = split_offs + li * (a.num_splits + 1) + split;
  // run `run` of the split's list: whole stages of UPS units, evenly
  int first, count;
  {
    const int f0 = soff[0], n0 = soff[1] - f0;
    const int per = ((n0 + a.sub_splits - 1) / a.sub_splits + UPS - 1) / UPS * UPS;
    const int lo = min(run * per, n0);
    first = f0 + lo;
    count = min(lo + per, n0) - lo;
  }
  // the list from the even entry at or before `first` (16-byte pairs): unit
  // u of the split is entry u + par of that run and sits at ring index
  // (u + par) % kListRing
  const int par = first & 1;
  const uint2 *list = lists + li * a.list_cap + (first - par);
  const int nlist = count + par;
  const int nst = (count + UPS - 1) / UPS;  // stages

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, gq = lane >> 4;
  const int G = a.G;
  const int rows = kGroupTokens * G;
  // row tile of this wave, rotated by group so that the waves left without
  // a tile (fewer than 64 rows) are not always on the same SIMD
  const int tile = (wave + (blockIdx.x >> 3)) & 3;
  const bool has_tile = tile * 16 < rows;  // wave-uniform

  // this lane's row: (token tau of the group, query head h)
  const int rho = tile * 16 + n;
  const int tau = rho / G;
  const int tok = grp * kGroupTokens + tau;
  const bool active = rho < rows && tok < a.total_q;
  const int h = g * G + (active ? rho - tau * G : 0);
  const int tok_c = active ? tok : 0;
  const int mshift = 4 * tau;
  // mask bits of the tokens whose rows meet this wave's tile
  uint32_t tilemask = 0u;
  if (has_tile) {
    const int t0 = (tile * 16) / G, t1 = min((tile * 16 + 15) / G, kGroupTokens - 1);
    for (int t = t0; t <= t1; ++t) tilemask |= 0xfu << (4 * t);
  }

  const LaneOffsets<D> L = lane_offsets<D>(a, wave);
  // byte offset in the K / V caches of unit u of the run (an LDS read of its
  // list entry, wave-uniform)
  const int64_t head_off = (int64_t)g * a.kv_stride_head;
  auto entry_off = [&](uint32_t e) {
    return (int64_t)(e >> 5) * a.kv_stride_page + (int64_t)((e & 31u) * 4) * a.kv_stride_tok + head_off;
  };
  auto unit_off = [&](int u) { return entry_off(__builtin_amdgcn_readfirstlane(sList[(u + par) % kListRing].x)); };
  // List entries are read from LDS one stage before they are used, so that
  // their latency hides behind a stage of compute instead of delaying the
  // loads and the K reads after each barrier: `pe` holds the cache entries
  // of the units the next stage issues (lane 0: tile A's, lane 1: tile B's),
  // `pma` / `pmb` the masks of this lane group's units of the next stage.
  // Entries past the run are read but not used.
  auto fetch_issue = [&](int s) { return sList[(UPS * s + wave + (lane & 1) * 4 + par) & (kListRing - 1)].x; };
  auto fetch_mask = [&](int u) { return sList[(u + par) & (kListRing - 1)].y; };

  // ---- prologue: the list's first two chunks into LDS, Q into registers,
  // then the first NST - 1 stages in flight.  The loop below issues no memory
  // access but the counted K/V and list loads, LDS traffic and its output
  // stores.
  issue_list_chunk(list, nlist, 0, wave, sList);
  issue_list_chunk(list, nlist, 1, wave, sList);
  u32x4 qreg[Gm::LANE_CH];
  {
    const uint8_t *qp = (const uint8_t *)a.q +
                        ((int64_t)tok_c * a.q_stride_tok + (int64_t)h * a.q_stride_head) * 2 + gq * (Gm::RB / 4);
#pragma unroll
    for (int c = 0; c < Gm::LANE_CH; ++c) qreg[c] = *(const u32x4 *)(qp + c * 16);
  }
  f32x4 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f, lp = 0.0f;
  const float sc = a.scale_log2;
  wait_vm_lgkm0<0>();  // Q and the list's first chunks landed
  stage_barrier();
  // this wave's part of stage s: units UPS s + wave (tile A) and + 4 (tile B)
  auto issue_stage = [&](uint8_t *slot, int s) {
    const int ua = UPS * s + wave, ub = ua + 4;
    issue_unit<D>(a, slot, wave * 4, ua < count ? unit_off(ua) : 0, ua < count, L);
    issue_unit<D>(a, slot, 16 + wave * 4, ub < count ? unit_off(ub) : 0, ub < count, L);
  };
  // loads this wave issues for stage s (units past the run issue none)
  auto loads_of = [&](int s) {
    const int ua = UPS * s + wave;
    return s < nst ? ((ua < count ? Gm::ULOADS : 0) + (ua + 4 < count ? Gm::ULOADS : 0)) : 0;
  };
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nst) issue_stage(smem + s * Gm::STAGE, s);
  uint32_t pe = fetch_issue(NST - 1), pma = fetch_mask(gq), pmb = fetch_mask(gq + 4);

  // One stage: J (compile time) is its ring slot.
  auto stage = [&](auto J_, const int beta) {
#pragma clang fp contract(off)
    constexpr int J = decltype(J_)::value;
    // loads this wave issued after stage beta's: those of stages beta+1 ..
    // beta+NST-2 (loads retire in order)
    int newer = 0;
#pragma unroll
    for (int s = 1; s <= NST - 2; ++s) newer += loads_of(beta + s);
    if constexpr (NST == 2) {
      wait_vm_lgkm0<0>();
    } else {
      static_assert(NST == 3, "waits written for two and three stages");
      if (newer == 0) wait_vm_lgkm0<0>();
      else if (newer == Gm::ULOADS) wait_vm_lgkm0<Gm::ULOADS>();
      else wait_vm_lgkm0<2 * Gm::ULOADS>();
    }
    stage_barrier();  // stage beta landed for every wave; slot of beta - 1 free
    if (beta + NST - 1 < nst) {
      uint8_t *slot = smem + ((J + NST - 1) % NST) * Gm::STAGE;
      const int ua = UPS * (beta + NST - 1) + wave, ub = ua + 4;
      const uint32_t ea = __builtin_amdgcn_readlane(pe, 0), eb = __builtin_amdgcn_readlane(pe, 1);
      issue_unit<D>(a, slot, wave * 4, ua < count ? entry_off(ea) : 0, ua < count, L);
      issue_unit<D>(a, slot, 16 + wave * 4, ub < count ? entry_off(eb) : 0, ub < count, L);
    }
    // List chunk c >= 2 (list positions 256 c ..) goes into the slot chunk
    // c - 2 held.  This is stage 32 c - 31; chunk c - 2 serves stages up to
    // 32 c - 33, whose entries were read by stage 32 c - 34, before this
    // stage's barrier.  Chunk c serves stages from 32 c - 1 on, whose entries
    // are first read at stage 32 c - 1 - NST, 30 - NST stages from now: the
    // stage waits cover it within NST stages (loads retire in order, and it
    // is older than the stage loads issued from the next stage on), and a
    // barrier then publishes it.  These loads are not in `newer`: a wait that
    // leaves one of them out only waits for one load more than it needs.
    if (beta >= kChunkStages + 1 && (beta - 1) % kChunkStages == 0) {
      const int c = (beta - 1) / kChunkStages + 1;
      if (c * kListChunk < nlist) issue_list_chunk(list, nlist, c, wave, sList);
    }
    const uint8_t *st = smem + J * Gm::STAGE;
    // this lane group's units of the stage (gq of tile A, 4 + gq of tile B),
    // and whether any unit of the stage has a token of this wave's tile
    const int ua = UPS * beta + gq, ub = ua + 4;
    const uint32_t mask_a = ua < count ? pma : 0u;
    const uint32_t mask_b = ub < count ? pmb : 0u;
    pe = fetch_issue(beta + NST);
    pma = fetch_mask(ua + UPS);
    pmb = fetch_mask(ub + UPS);
    if (!has_tile || !__any(((mask_a | mask_b) & tilemask) != 0u)) return;
    // ---- S^T for the stage's 32 keys, tile A then tile B (lane: keys
    // 4gq..4gq+3 of each tile, row n), each contraction over four
    // accumulators; a tile's K fragments are all requested before its MFMAs
    auto qk_tile = [&](const uint8_t *tb) {
      u32x4 kf[Gm::LANE_CH];
#pragma unroll
      for (int c = 0; c < Gm::LANE_CH; ++c) kf[c] = *(const u32x4 *)(tb + L.k[c]);
      __asm__ volatile("" ::: "memory");
      f32x4 ac[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) ac[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < Gm::LANE_CH; ++c) ac[c & 3] = mfma_f16(kf[c], qreg[c], ac[c & 3]);
      return (ac[0] + ac[1]) + (ac[2] + ac[3]);
    };
    const f32x4 acc_a = qk_tile(st);
    const f32x4 acc_b = qk_tile(st + Gm::TILE_B);
    // ---- masks and softmax at raised wave priority (back to 0 before PV):
    // this VALU stretch of one wave gets the issue slots first while the
    // other wave of the SIMD keeps the matrix cores busy
    __builtin_amdgcn_s_setprio(1);
    // ---- exact masks: key i of this lane group's unit in each tile
    const uint32_t bits_a = active ? (mask_a >> mshift) & 0xfu : 0u;
    const uint32_t bits_b = active ? (mask_b >> mshift) & 0xfu : 0u;
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = ((bits_a >> i) & 1u) ? acc_a[i] * sc : -INFINITY;
      x[4 + i] = ((bits_b >> i) & 1u) ? acc_b[i] * sc : -INFINITY;
    }
    float mb = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mb = quarter_reduce<true>(mb);
    // ---- raise the running max only when a logit passes it by kLag
    const bool up = mb > m + kLag;  // also when m is still -inf and mb is not
    if (__any(up)) {
      const float alpha = up ? ((m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mb)) : 1.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
      l *= alpha;
      lp *= alpha;
      m = up ? mb : m;
    }
    // ---- P = 2^(s - m) < 2^kLag (0 for masked keys and for rows with no
    // key yet), sums, FP16 operand: keys 4gq..4gq+3 of tile A, then of tile B
    const float ms = (m == -INFINITY) ? 0.0f : m;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = __builtin_amdgcn_exp2f(x[i] - ms);
      l += pv[i];
    }
    // (each pair is cast from a scalar: a bit cast of a vector element,
    // pf[j], was compiled as a cast of element 0)
    u32x4 pf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t pair = pack_f16x2(pv[2 * j], pv[2 * j + 1]);
      pf[j] = pair;
      lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), f16x2{(_Float16)1.0f, (_Float16)1.0f}, lp, false);
    }
    __builtin_amdgcn_s_setprio(0);
    // ---- O^T += V^T P^T over the 32 keys (16x16x32: element j of the V^T
    // operand and of the P^T operand name the same key): lane n receives V
    // rows 4gq .. 4gq+3 of each tile at dim 16 mt + n
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t vo = L.v[mt & 7] + (mt & 8) * 32;
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(st + vo));
      const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(st + Gm::TILE_B + vo));
      const u32x2 wa = __builtin_bit_cast(u32x2, va), wb = __builtin_bit_cast(u32x2, vb);
      o[mt] = mfma_f16(u32x4{wa[0], wa[1], wb[0], wb[1]}, pf, o[mt]);
    }
  };

  for (int beta0 = 0; beta0 < nst; beta0 += NST) {
    stage(std::integral_constant<int, 0>{}, beta0);
    if (beta0 + 1 < nst) stage(std::integral_constant<int, 1>{}, beta0 + 1);
    if constexpr (NST > 2) {
      if (beta0 + 2 < nst) stage(std::integral_constant<int, 2 % NST>{}, beta0 + 2);
    }
  }

  // ---- epilogue: row n of the tile, columns 16*mt + 4*gq + [0,4).  The
  // output is (O / lp) * v_scale with a true division: when one key carries
  // all the weight, O = p v exactly and lp = p, so the row is v * v_scale
  // bit for bit whatever P's scale.
  if (!has_tile || !active) return;
  l = quarter_reduce<false>(l);
  lp = quarter_reduce<false>(lp);
  const int64_t row = (int64_t)tok * a.Hq + h;
  const int64_t off = (int64_t)split * a.po_split_stride + row * a.po_row_stride + run * a.po_sub_stride + gq * 4;
  float *lse_dst = a.partial_lse + (int64_t)split * a.pl_split_stride + run * a.pl_sub_stride + row;
  if (l > 0.0f) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (o[mt][i] / lp) * a.v_scale;
      store_partial4<PO>(a.partial_o, off + mt * 16, r);
    }
    if (gq == 0) *lse_dst = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) store_partial4<PO>(a.partial_o, off + mt * 16, f32x4{0.f, 0.f, 0.f, 0.f});
    if (gq == 0) *lse_dst = -INFINITY;
  }
}

}  // namespace

size_t grouped_attend_lds_bytes() {
  return (size_t)(GGeom<256>::LDS > GGeom<128>::LDS ? GGeom<256>::LDS : GGeom<128>::LDS);
}
static_assert(kChunkStages - 2 - GGeom<256>::NST >= GGeom<256>::NST &&
                  kChunkStages - 2 - GGeom<128>::NST >= GGeom<128>::NST,
              "a list chunk has landed and is published before its entries are first read");

hipError_t launch_grouped_attend(const GroupArgs &ga, hipStream_t s) {
  if (ga.num_groups == 0) return hipSuccess;
  const int H = ga.sub_splits;
  // With runs (H > 1) the kernel writes FP32 partials of each run into the
  // workspace, [split][row][run][d] and [run][split][row]; a combine then
  // merges each split's runs into the caller's partials.
  GroupArgs a = ga;
  const int64_t rows_all = (int64_t)ga.total_q * ga.Hq;
  if (H > 1) {
    a.partial_o = ga.ws + ga.lay.sub_po;
    a.po_dtype = MSA_F32;
    a.po_split_stride = rows_all * H * ga.D;
    a.po_row_stride = (int64_t)H * ga.D;
    a.partial_lse = (float *)(ga.ws + ga.lay.sub_pl);
    a.pl_split_stride = rows_all;
  }
  dim3 grid((unsigned)((a.num_groups + 7) / 8 * 8), (unsigned)a.Hkv, (unsigned)(a.num_splits * H));
  const uint2 *lists = (const uint2 *)(a.ws + a.lay.lists);
  const int *soffs = (const int *)(a.ws + a.lay.split_off);
  switch ((a.D == 256 ? 8 : 0) + a.po_dtype) {
    case 8 + MSA_F32: k_grouped_attend<256, MSA_F32><<<grid, GT, 0, s>>>(a, lists, soffs); break;
    case 8 + MSA_BF16: k_grouped_attend<256, MSA_BF16><<<grid, GT, 0, s>>>(a, lists, soffs); break;
    case 8 + MSA_F16: k_grouped_attend<256, MSA_F16><<<grid, GT, 0, s>>>(a, lists, soffs); break;
    case MSA_BF16: k_grouped_attend<128, MSA_BF16><<<grid, GT, 0, s>>>(a, lists, soffs); break;
    case MSA_F16: k_grouped_attend<128, MSA_F16><<<grid, GT, 0, s>>>(a, lists, soffs); break;
    default: k_grouped_attend<128, MSA_F32><<<grid, GT, 0, s>>>(a, lists, soffs); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || H == 1) return e;
  // merge: the flat list of (split, row) rows, H runs each, into the split slabs
  return launch_combine(a.partial_o, MSA_F32, ga.D, (int64_t)H * ga.D, a.partial_lse, a.pl_split_stride * ga.num_splits,
                        H, (int64_t)ga.num_splits * rows_all, ga.D, ga.partial_o, ga.po_dtype, ga.po_row_stride,
                        ga.partial_lse, s, OutMap{rows_all, ga.po_split_stride, ga.pl_split_stride});
}

}  // namespace msa
