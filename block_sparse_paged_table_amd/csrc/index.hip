// Paged prefill indexer (vllm-project/MSA PR 36, sections "Overview" and
// "Changes": an FP8-query, FP8-cache scorer that keeps one score per page --
// the page's max -- for every (query, head) row, then a top-k over the row),
// written for gfx950.
//
// k_index_scores: one workgroup per (64 query tokens, head, chunk of 16
// logical pages, or 8 or 4 when that grid would not fill the GPU).  The 64 Q rows live in registers (16 per wave); each page
// of the chunk that some row of the tile can see is copied into LDS
// (double-buffered, the next page's loads in flight while the current one is
// scored), and every wave computes S^T = K Q^T for its 16 rows with FP8 MFMA
// (exact E4M3 products, FP32 accumulation), masks keys the row cannot see
// (t > q_pos, t >= seq_len), and reduces each row's max over the page's 128
// keys.  Scores collect in LDS and leave as contiguous row segments.  A tile
// whose tokens belong to several requests scores each request's pages in
// turn.
//
// k_index_topk: one wave per (token, head) row; the row's page scores sit in
// registers and top_k rounds of a wave-wide arg-max (ties: lower page) pick
// the selection.
#include "index.h"

namespace msa {
namespace {

// 4 waves per workgroup (64 query tokens): against 8, each page load is
// shared by half the rows, but twice as many workgroups share the GPU and
// four fit on a CU (0.133 vs 0.145 ms on the 16K-token, 2-head workload;
// 16-page chunks, as 32, beat 8 and 4)
constexpr int ITQ_WAVES = 4;  // waves per workgroup (16 query rows each)
// Logical pages per workgroup (PC): 16 where the grid is large; halved, down
// to 4, while the grid has fewer than kIndexMinWorkgroups workgroups, so
// that a few short chunks over long contexts still fill the GPU
// (vllm-project/MSA PR 36, "Changes": the page chunk adapts to the batch).
// Measured: 16 pages beat 8 and 4 on the 16K-token request (0.133 vs 0.158 /
// 0.215 ms) and on 8 chunks of 64..512 tokens (0.128 vs 0.144 / 0.184 ms);
// on two chunks of 64 and 40 tokens over 90K..120K contexts 4 pages win
// (0.0285 vs 0.0328 ms).
constexpr int kIndexPageChunks[] = {16, 8, 4};
constexpr int64_t kIndexMinWorkgroups = 2048;  // two per resident slot (4 per CU, 256 CUs)
constexpr int IPAGE = 128;  // tokens per page

template <int D> struct IGeom {
  // waves per workgroup: each thread copies at least one 16-byte chunk of a page
  static constexpr int WAVES = ITQ_WAVES * 64 > IPAGE * D / 16 ? IPAGE * D / 16 / 64 : ITQ_WAVES;
  static constexpr int IT = 64 * WAVES;    // threads per workgroup
  static constexpr int RB = D;              // bytes per K row (E4M3)
  static constexpr int CPR = RB / 16;       // 16-byte chunks per row
  static constexpr int LANE_CH = CPR / 4;   // chunks of a row one lane holds
  static constexpr int KCH = IPAGE * CPR / IT;  // chunks per thread per page
  static constexpr int PAGE_BYTES = IPAGE * RB;
  static_assert(KCH >= 1 && KCH * IT == IPAGE * CPR, "page copy must cover the page exactly");
};

// Byte offset of chunk c of K row `key` in LDS, XOR-swizzled so that the 16
// rows an MFMA operand reads (keys 16 t .. 16 t + 15) spread over the LDS
// banks.  For 128-byte rows (d 128) the swizzle (key & 7) ^ 5 (key >> 3 & 1)
// was measured on gfx950 at 221 B per clock and CU against 112 for key & 7,
// which conflicts two-way; other row widths keep the key's low bits.
template <int D> __device__ __forceinline__ int ik_swz(int key) {
  using Gm = IGeom<D>;
  return Gm::CPR == 8 ? (key & 7) ^ (((key >> 3) & 1) * 5) : (key & (Gm::CPR - 1));
}
template <int D> __device__ __forceinline__ int ik_off(int key, int c) {
  return key * IGeom<D>::RB + ((c ^ ik_swz<D>(key)) << 4);
}

// A K page goes straight from the cache into LDS (global_load_lds): load it
// of wave w fills LDS chunks [q0, q0 + 64), q0 = it * IT + 64 w, each lane
// one 16-byte chunk q0 + lane = row * CPR + physical chunk; this lane's
// source offset in the page (the logical chunk is the physical one XOR the
// row's swizzle) is dma_off(it).
template <int D> __device__ __forceinline__ uint32_t kpage_src_off(const IndexArgs &a, int it) {
  using Gm = IGeom<D>;
  const int q = it * Gm::IT + (int)threadIdx.x, key = q / Gm::CPR, pc = q % Gm::CPR;
  return (uint32_t)(key * a.kv_stride_tok) + (uint32_t)((pc ^ ik_swz<D>(key)) << 4);
}

// RPW: 16-row tiles per wave.  With 2 every K fragment read from LDS feeds
// two MFMAs (half the LDS reads per row) and a page load serves twice the
// rows: 0.091 -> 0.083 ms on the 16K-token request; on short chunks the
// 128-token tiles straddle requests and idle rows, so those keep 1 (there 2
// took 0.103 -> 0.174 ms, and 0.024 -> 0.056 ms on two chunks of 64 and 40).
template <int D, int RPW> constexpr int index_tile_tokens() { return 16 * IGeom<D>::WAVES * RPW; }

template <int D, int IPC, int RPW>
__global__ void __launch_bounds__(IGeom<D>::IT, RPW == 2 ? 3 : 4) k_index_scores(const IndexArgs a) {
  using Gm = IGeom<D>;
  constexpr int IT = Gm::IT, ITQ = index_tile_tokens<D, RPW>();
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][Gm::PAGE_BYTES];
  __shared__ float sScore[ITQ][IPC + 1];
  __shared__ int sRowB[ITQ], sRowLast[ITQ];
  __shared__ int sReq[ITQ], sReqLast[ITQ];
  __shared__ int sNreq, sMinB, sMaxB, sMaxLast;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int tok0 = blockIdx.x * ITQ, h = blockIdx.y, j0 = blockIdx.z * IPC;
  const int npg = min(IPC, a.max_pages - j0);

  // ---- rows of the tile: request and last visible position (-1: none)
  if (tid < ITQ) {
    const int tok = tok0 + tid;
    int b = -1, last = -1;
    if (tok < a.total_q) {
      const int pos = a.q_pos[tok], bb = a.q_seq[tok];
      if (pos >= 0) {
        if (bb < 0 || bb >= a.num_seqs) {
          if (a.err_flags && h == 0 && blockIdx.z == 0) atomicOr(a.err_flags, MSA_ERRF_QSEQ_RANGE);
        } else {
          b = bb;
          last = min(pos, a.seq_lens[bb] - 1);
          if (last < 0) b = -1;
        }
      }
    }
    sRowB[tid] = b;
    sRowLast[tid] = last;
  }
  if (tid == 0) {
    sMinB = INT32_MAX;
    sMaxB = -1;
    sMaxLast = -1;
  }
  for (int i = tid; i < ITQ * (IPC + 1); i += IT) (&sScore[0][0])[i] = -INFINITY;
  __syncthreads();
  if (tid < ITQ && sRowB[tid] >= 0) {
    atomicMin(&sMinB, sRowB[tid]);
    atomicMax(&sMaxB, sRowB[tid]);
    atomicMax(&sMaxLast, sRowLast[tid]);
  }
  __syncthreads();
  if (tid == 0 && sMinB == sMaxB) {  // one request (or none): the usual tile
    sReq[0] = sMinB;
    sReqLast[0] = sMaxLast;
    sNreq = sMaxB >= 0 ? 1 : 0;
  } else if (tid == 0) {  // the distinct requests of the tile, in order of appearance
    int nr = 0;
    for (int r = 0; r < ITQ; ++r) {
      const int b = sRowB[r];
      if (b < 0) continue;
      int k = 0;
      while (k < nr && sReq[k] != b) ++k;
      if (k == nr) {
        sReq[nr] = b;
        sReqLast[nr] = sRowLast[r];
        ++nr;
      } else {
        sReqLast[k] = max(sReqLast[k], sRowLast[r]);
      }
    }
    sNreq = nr;
  }
  __syncthreads();

  // ---- this lane's Q rows (row wave*16*RPW + 16p + n of the tile), its quarter of d
  int rho[RPW], my_b[RPW], my_last[RPW];
  u32x4 qr[RPW][Gm::LANE_CH];
#pragma unroll
  for (int p = 0; p < RPW; ++p) {
    rho[p] = wave * 16 * RPW + 16 * p + n;
    my_b[p] = sRowB[rho[p]];
    my_last[p] = sRowLast[rho[p]];
    const int tok = my_b[p] >= 0 ? tok0 + rho[p] : 0;  // rows that see nothing read token 0
    const uint8_t *qp = a.q + (int64_t)tok * a.q_stride_tok + (int64_t)h * a.q_stride_head + grp * (Gm::RB / 4);
#pragma unroll
    for (int c = 0; c < Gm::LANE_CH; ++c) qr[p][c] = *(const u32x4 *)(qp + c * 16);
  }

  uint32_t dma_off[Gm::KCH];
#pragma unroll
  for (int it = 0; it < Gm::KCH; ++it) dma_off[it] = kpage_src_off<D>(a, it);

  const int nreq = sNreq;
  for (int ri = 0; ri < nreq; ++ri) {
    const int cb = sReq[ri];
    const int lastmax = sReqLast[ri];
    // pages of this chunk that some row of request cb can see
    const int jn = min(npg, lastmax / IPAGE - j0 + 1);
    if (jn <= 0) continue;
    // the chunk's physical pages in one load (lane j: page j; -1 out of range)
    const int32_t *ptrow = a.page_table + (int64_t)cb * a.pt_stride + j0;
    int pt = -1;
    if (lane < jn) {
      const int p = ptrow[lane];
      pt = (p >= 0 && p < a.num_phys_pages) ? p : -1;
    }
    auto phys_of = [&](int jj) { return __builtin_amdgcn_readlane(pt, jj); };
    // this wave's part of a page into buffer sk: KCH loads of 64 chunks
    auto issue_page = [&](int phys, uint8_t *sk) {
      const uint8_t *kb = a.k_cache + (int64_t)phys * a.kv_stride_page + (int64_t)h * a.kv_stride_head;
      const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS uint8_t *)sk);
#pragma unroll
      for (int it = 0; it < Gm::KCH; ++it) lds_dma16(kb, dma_off[it], lds + (it * IT + wave * 64) * 16);
    };
    int phys_next = phys_of(0);
    if (phys_next >= 0) issue_page(phys_next, sK[0]);
    for (int jj = 0; jj < jn; ++jj) {
      const int phys = phys_next;
      const uint8_t *sk = sK[jj & 1];
      // page jj landed (each wave waits for its own loads; the barrier
      // publishes them), and every wave is done with page jj - 1's buffer
      wait_vm_lgkm0<0>();
      stage_barrier();
      if (jj + 1 < jn) {
        phys_next = phys_of(jj + 1);
        if (phys_next >= 0) issue_page(phys_next, sK[(jj + 1) & 1]);
      }
      if (phys < 0) {
        if (a.err_flags && tid == 0) atomicOr(a.err_flags, MSA_ERRF_PHYS_RANGE);
        continue;  // scores stay -inf
      }
      // ---- S^T = K Q^T: lane holds keys 16t + 4grp + i of row n (of each tile)
      f32x4 acc[RPW][IPAGE / 16];
#pragma unroll
      for (int p = 0; p < RPW; ++p)
#pragma unroll
        for (int t = 0; t < IPAGE / 16; ++t) acc[p][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (Gm::LANE_CH == 2) {
        // d = 128: the lane's 32 bytes of a K row against its 32 bytes of the
        // Q row, one K = 128 MFMA per key tile and row tile
#pragma unroll
        for (int t = 0; t < IPAGE / 16; ++t) {
          const u32x4 k0 = *(const u32x4 *)(sk + ik_off<D>(t * 16 + n, grp * 2));
          const u32x4 k1 = *(const u32x4 *)(sk + ik_off<D>(t * 16 + n, grp * 2 + 1));
#pragma unroll
          for (int p = 0; p < RPW; ++p) acc[p][t] = mfma_fp8_k128(k0, k1, qr[p][0], qr[p][1], acc[p][t]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < Gm::LANE_CH; ++c)
#pragma unroll
          for (int t = 0; t < IPAGE / 16; ++t) {
            const u32x4 k4 = *(const u32x4 *)(sk + ik_off<D>(t * 16 + n, grp * Gm::LANE_CH + c));
#pragma unroll
            for (int p = 0; p < RPW; ++p) {
              acc[p][t] = mfma_fp8(u32x2{k4[0], k4[1]}, u32x2{qr[p][c][0], qr[p][c][1]}, acc[p][t]);
              acc[p][t] = mfma_fp8(u32x2{k4[2], k4[3]}, u32x2{qr[p][c][2], qr[p][c][3]}, acc[p][t]);
            }
          }
      }
      // ---- max over the keys each row sees
      const int jabs = j0 + jj;
#pragma unroll
      for (int p = 0; p < RPW; ++p) {
        const int vis_to = (my_b[p] == cb) ? my_last[p] - jabs * IPAGE : -1;  // last visible in-page key
        float m = -INFINITY;
        if (__all(vis_to >= IPAGE - 1)) {
          // every row of the tile sees the whole page (all pages but a row's
          // own): a plain max, no per-key test
#pragma unroll
          for (int t = 0; t < IPAGE / 16; ++t)
            m = fmaxf(m, fmaxf(fmaxf(acc[p][t][0], acc[p][t][1]), fmaxf(acc[p][t][2], acc[p][t][3])));
        } else {
#pragma unroll
          for (int t = 0; t < IPAGE / 16; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t * 16 + 4 * grp + i <= vis_to) m = fmaxf(m, acc[p][t][i]);
        }
        m = quarter_reduce<true>(m);
        if (grp == 0 && my_b[p] == cb) sScore[rho[p]][jj] = m == -INFINITY ? m : m * a.scale;
      }
    }
    __syncthreads();  // the last page's buffer is reused by the next request
  }
  __syncthreads();

  // ---- scores out: each row's npg pages are one contiguous segment
  for (int i = tid; i < ITQ * npg; i += IT) {
    const int r = i / npg, jj = i - r * npg;
    const int tok = tok0 + r;
    if (tok < a.total_q)
      a.scores[((int64_t)tok * a.H + h) * a.score_stride + j0 + jj] = sScore[r][jj];
  }
}

// (bv, bj) := the better of (bv, bj) and (ov, oj): higher score, then lower page.
__device__ __forceinline__ void take_better(float &bv, int &bj, float ov, int oj) {
  if (ov > bv || (ov == bv && oj < bj)) {
    bv = ov;
    bj = oj;
  }
}
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, true);
}
template <int CTRL> __device__ __forceinline__ void take_better_dpp(float &bv, int &bj) {
  take_better(bv, bj, __uint_as_float(dpp_u32<CTRL>(__float_as_uint(bv))), (int)dpp_u32<CTRL>((uint32_t)bj));
}
// The wave's best (score, page) on every lane.  The order is total, so any
// combining pattern gives every lane the same winner: DPP within each 16-lane
// row (quad swaps, then rotations by 4 and 8), then the gfx950 row swaps.
__device__ __forceinline__ void wave_best(float &bv, int &bj) {
  take_better_dpp<0xb1>(bv, bj);   // quad_perm [1,0,3,2]
  take_better_dpp<0x4e>(bv, bj);   // quad_perm [2,3,0,1]
  take_better_dpp<0x124>(bv, bj);  // row_ror:4
  take_better_dpp<0x128>(bv, bj);  // row_ror:8
  {
    const auto v = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto j = __builtin_amdgcn_permlane16_swap((uint32_t)bj, (uint32_t)bj, false, false);
    float v0 = __uint_as_float(v[0]);
    int j0 = (int)j[0];
    take_better(v0, j0, __uint_as_float(v[1]), (int)j[1]);
    bv = v0;
    bj = j0;
  }
  {
    const auto v = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto j = __builtin_amdgcn_permlane32_swap((uint32_t)bj, (uint32_t)bj, false, false);
    float v0 = __uint_as_float(v[0]);
    int j0 = (int)j[0];
    take_better(v0, j0, __uint_as_float(v[1]), (int)j[1]);
    bv = v0;
    bj = j0;
  }
}

// One wave per (token, head) row: NPL page scores per lane (page i*64+lane).
template <int NPL>
__global__ void __launch_bounds__(256) k_index_topk(const IndexArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.total_q * a.H) return;
  const int tok = (int)(row / a.H), h = (int)(row - (int64_t)tok * a.H);
  const float *sr = a.scores + row * a.score_stride;
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = i * 64 + lane;
    v[i] = j < a.max_pages ? sr[j] : -INFINITY;
  }
  // slot s of the result is kept by lane s % 64 (register s / 64) and
  // written once at the end, one coalesced store per register
  int32_t res[4] = {-1, -1, -1, -1};
  bool done = false;  // wave-uniform
  for (int s = 0; s < a.top_k && !done; ++s) {
    float bv = -INFINITY;
    int bj = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (v[i] > bv) {  // ascending pages: a tie keeps the lower one
        bv = v[i];
        bj = i * 64 + lane;
      }
    wave_best(bv, bj);
    done = !(bv > -INFINITY);
    if (done) break;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (i * 64 + lane == bj) v[i] = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (s == k * 64 + lane) res[k] = bj;
  }
  int32_t *oi = a.sel_idx + (int64_t)tok * a.sel_stride_tok + (int64_t)h * a.sel_stride_head;
  uint8_t *om = a.sel_mask + (int64_t)tok * a.sel_stride_tok + (int64_t)h * a.sel_stride_head;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = k * 64 + lane;
    if (s < a.top_k) {
      oi[s] = res[k];
      om[s] = res[k] >= 0 ? 1 : 0;
    }
  }
}

// The best (score, page) of each 16-lane row of the wave on every lane of that
// row: the DPP steps of wave_best, which stay within a row.
__device__ __forceinline__ void row16_best(float &bv, int &bj) {
  take_better_dpp<0xb1>(bv, bj);   // quad_perm [1,0,3,2]
  take_better_dpp<0x4e>(bv, bj);   // quad_perm [2,3,0,1]
  take_better_dpp<0x124>(bv, bj);  // row_ror:4
  take_better_dpp<0x128>(bv, bj);  // row_ror:8
}

// Rows of at most 128 pages and top_k <= 64: 16 lanes per (token, head) row,
// four rows per wave, 8 page scores per lane (page i*16 + lane % 16).  The same
// rounds as k_index_topk (arg-max by score, then lower page; the winner is
// removed), with a 16-lane arg-max, so a round costs a quarter of the wave's
// instructions per row.  A row whose scores run out (-inf) stops taking
// slots; the wave runs until all four rows are done.
__global__ void __launch_bounds__(256) k_index_topk16(const IndexArgs a) {
  constexpr int NV = 8;
  const int ll = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = row < (int64_t)a.total_q * a.H;
  const int64_t rr = live ? row : 0;
  const int tok = (int)(rr / a.H), h = (int)(rr - (int64_t)tok * a.H);
  const float *sr = a.scores + rr * a.score_stride;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = i * 16 + ll;
    v[i] = (live && j < a.max_pages) ? sr[j] : -INFINITY;
  }
  // slot s of the row's result is kept by lane s % 16 (register s / 16)
  int32_t res[4] = {-1, -1, -1, -1};
  bool done = false;  // per row (uniform over its 16 lanes)
  for (int s = 0; s < a.top_k; ++s) {
    float bv = -INFINITY;
    int bj = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (v[i] > bv) {  // ascending pages: a tie keeps the lower one
        bv = v[i];
        bj = i * 16 + ll;
      }
    row16_best(bv, bj);
    done = done || !(bv > -INFINITY);
    if (__all(done)) break;
    if (!done) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i * 16 + ll == bj) v[i] = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (s == k * 16 + ll) res[k] = bj;
    }
  }
  if (!live) return;
  int32_t *oi = a.sel_idx + (int64_t)tok * a.sel_stride_tok + (int64_t)h * a.sel_stride_head;
  uint8_t *om = a.sel_mask + (int64_t)tok * a.sel_stride_tok + (int64_t)h * a.sel_stride_head;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = k * 16 + ll;
    if (s < a.top_k) {
      oi[s] = res[k];
      om[s] = res[k] >= 0 ? 1 : 0;
    }
  }
}

__global__ void k_index_zero(uint32_t *err) { *err = 0u; }

}  // namespace

// Static LDS of k_index_scores<D, IPC, RPW> (its __shared__ arrays).
template <int D, int IPC, int RPW> constexpr size_t index_scores_lds() {
  using Gm = IGeom<D>;
  constexpr size_t itq = index_tile_tokens<D, RPW>();
  return 2 * (size_t)Gm::PAGE_BYTES + itq * (IPC + 1) * 4 + 4 * itq * 4 + 4 * 4;
}

size_t index_lds_bytes() {
  // the largest page chunk and tile hold the most scores
  constexpr int pc = kIndexPageChunks[0];
  return index_scores_lds<128, pc, 2>() > index_scores_lds<64, pc, 1>() ? index_scores_lds<128, pc, 2>()
                                                                         : index_scores_lds<64, pc, 1>();
}

namespace {
template <int D, int IPC, int RPW>
hipError_t launch_scores(const IndexArgs &a, int64_t tiles, hipStream_t s) {
  dim3 grid((unsigned)tiles, (unsigned)a.H, (unsigned)((a.max_pages + IPC - 1) / IPC));
  k_index_scores<D, IPC, RPW><<<grid, IGeom<D>::IT, 0, s>>>(a);
  return hipGetLastError();
}
template <int D, int RPW>
hipError_t launch_scores_r(const IndexArgs &a, hipStream_t s) {
  constexpr int itq = index_tile_tokens<D, RPW>();
  const int64_t tiles = (a.total_q + itq - 1) / itq;
  int pc = kIndexPageChunks[0];
  for (int c : kIndexPageChunks) {
    pc = c;
    if (tiles * a.H * ((a.max_pages + c - 1) / c) >= kIndexMinWorkgroups) break;
  }
  switch (pc) {
    case 16: return launch_scores<D, 16, RPW>(a, tiles, s);
    case 8: return launch_scores<D, 8, RPW>(a, tiles, s);
    default: return launch_scores<D, 4, RPW>(a, tiles, s);
  }
}
template <int D>
hipError_t launch_scores_d(const IndexArgs &a, hipStream_t s) {
  // two row tiles per wave for long chunks (1024 tokens or more per
  // request on average) on a grid that still fills the GPU
  if constexpr (D == 128) {
    constexpr int itq2 = index_tile_tokens<D, 2>();
    const int64_t tiles2 = (a.total_q + itq2 - 1) / itq2;
    if ((int64_t)a.total_q >= 1024ll * a.num_seqs &&
        tiles2 * a.H * ((a.max_pages + kIndexPageChunks[0] - 1) / kIndexPageChunks[0]) >= kIndexMinWorkgroups)
      return launch_scores_r<D, 2>(a, s);
  }
  return launch_scores_r<D, 1>(a, s);
}
}  // namespace

hipError_t launch_index_scores(const IndexArgs &a, hipStream_t s) {
  if (a.err_flags) k_index_zero<<<1, 1, 0, s>>>(a.err_flags);
  if (a.total_q == 0) return hipGetLastError();
  return a.D == 64 ? launch_scores_d<64>(a, s) : launch_scores_d<128>(a, s);
}

hipError_t launch_index_topk(const IndexArgs &a, hipStream_t s) {
  const int64_t rows = (int64_t)a.total_q * a.H;
  if (rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (a.max_pages <= 128 && a.top_k <= 64)
    k_index_topk16<<<(unsigned)((rows + 15) / 16), 256, 0, s>>>(a);
  else if (a.max_pages <= 128)
    k_index_topk<2><<<blocks, 256, 0, s>>>(a);
  else if (a.max_pages <= 512)
    k_index_topk<8><<<blocks, 256, 0, s>>>(a);
  else
    k_index_topk<kIndexMaxPages / 64><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace msa
