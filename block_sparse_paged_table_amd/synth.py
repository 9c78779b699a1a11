"""Seeded synthetic inputs for block-sparse paged prefill attention.

This module only *creates* inputs: random query/key/value tensors, paged-cache
layouts with randomly permuted physical pages, per-row page selections, and
the quantised storage formats the kernels consume (FP8 E4M3 queries, NVFP4
keys/values).  It holds none of the method's arithmetic (no dequantisation,
no attention, no combine); both the GPU path and the CPU oracle consume what
it produces, so neither depends on the other.

Workloads follow the shapes of the pages' own cases:
  * MiniMax-AI/MSA PR 21, "K1" and "Combine": paged sparse prefill where each
    query selects 16 pages (its own page, causal, plus history pages) and the
    kernel writes one partial output per selected page;
  * 1Cat-vLLM PR 387 / PR 1236, "Purpose": grouped Page4 routes with 4-token
    microblocks, exact per-row 4-bit masks, nonmonotonic physical pages, a
    partial tail page and all-invalid padding rows.

All randomness comes from numpy's PCG64 ``default_rng(seed)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

# Storage dtypes understood by the library and the oracle.
Q_DTYPES = ("f32", "bf16", "f16", "e4m3")
KV_DTYPES = ("f32", "bf16", "f16", "e4m3", "nvfp4")
TORCH_DTYPE = {
    "f32": torch.float32,
    "bf16": torch.bfloat16,
    "f16": torch.float16,
    "e4m3": torch.float8_e4m3fn,
}


@dataclasses.dataclass
class Problem:
    """One synthetic prefill layer: queries, paged KV cache and selections.

    Row convention: the flat (token, query head) row is ``token * Hq + h``;
    query head ``h`` reads KV head ``h // (Hq // Hkv)``.
    """

    name: str
    num_seqs: int
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    page_size: int
    unit_tokens: int        # page_size for page selections, 4 for microblocks
    num_slots: int          # K selections per (token, KV head)
    slots_per_split: int    # slots merged into one partial slab
    q_dtype: str
    kv_dtype: str
    out_dtype: str
    q: torch.Tensor         # [total_q, Hq, d_qk] in TORCH_DTYPE[q_dtype]
    q_seq: torch.Tensor     # int32 [total_q], request of each token
    q_pos: torch.Tensor     # int32 [total_q], absolute position (-1 = padding)
    seq_lens: torch.Tensor  # int32 [B], KV tokens present per request
    page_table: torch.Tensor  # int32 [B, max_pages], logical -> physical page
    num_phys_pages: int
    # float KV: [P, page, Hkv, d] tensors (possibly strided views);
    # nvfp4 KV: uint8 codes [P, page, Hkv, d/2] (element 2i in the low nibble)
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_sf: Optional[torch.Tensor]  # uint8 E4M3 scales [P, page, Hkv, d/16] (nvfp4)
    v_sf: Optional[torch.Tensor]
    sel_idx: torch.Tensor   # int32 [total_q, Hkv, K], logical unit ids
    sel_mask: torch.Tensor  # uint8 [total_q, Hkv, K]
    sm_scale: float
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    seed: int = 0
    description: str = ""

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def num_rows(self) -> int:
        return self.total_q * self.Hq

    @property
    def num_splits(self) -> int:
        return self.num_slots // self.slots_per_split


# ---------------------------------------------------------------------------
# Storage-format encoders used only to *produce* quantised inputs.
# ---------------------------------------------------------------------------

_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code for each value (ties to the even code, clamp at 6).

    E2M1 magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; the sign is bit 3.
    """
    m = np.minimum(np.abs(y), 6.0)
    code = np.zeros(y.shape, dtype=np.uint8)
    for lower, mid in enumerate(_E2M1_MIDPOINTS):
        # a tie goes to whichever neighbour has an even code
        code += (m > mid) if lower % 2 == 0 else (m >= mid)
    code |= np.signbit(y).astype(np.uint8) << 3
    return code


def quantize_e4m3_tensor(x: torch.Tensor):
    """Per-tensor scaled FP8 E4M3: returns (codes as float8_e4m3fn, scale)."""
    amax = float(x.abs().max())
    scale = amax / 448.0 if amax > 0 else 1.0
    q8 = (x.float() / scale).to(torch.float8_e4m3fn)
    return q8, scale


def quantize_nvfp4(x: np.ndarray):
    """Quantise float values [..., d] to NVFP4 storage.

    Per-tensor FP32 scale g = amax / 448, then for each block of 16
    contiguous elements along d an E4M3 scale s = E4M3(max|x/g| / 6) and
    E2M1 codes of x / (g s).  With this choice every code x scale product is
    at most 6 * 72 = 432, inside the E4M3 range.  Returns (packed codes
    uint8 [..., d/2], scales uint8 [..., d/16], g).
    """
    d = x.shape[-1]
    assert d % 16 == 0
    amax = float(np.abs(x).max())
    g = amax / 448.0 if amax > 0 else 1.0
    y = (x / g).astype(np.float32)
    yb = y.reshape(*y.shape[:-1], d // 16, 16)
    bmax = np.abs(yb).max(axis=-1)
    sf = torch.from_numpy(np.ascontiguousarray(bmax / 6.0)).to(torch.float8_e4m3fn)
    sf_val = sf.float().numpy().astype(np.float32)
    safe = np.where(sf_val > 0, sf_val, 1.0)[..., None]
    codes = _e2m1_encode(np.where(sf_val[..., None] > 0, yb / safe, 0.0))
    codes = codes.reshape(*y.shape[:-1], d)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return (
        torch.from_numpy(np.ascontiguousarray(packed)),
        sf.view(torch.uint8).contiguous(),
        g,
    )


def _randn(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


# ---------------------------------------------------------------------------
# Page-selection problems (one selection = one whole page).
# ---------------------------------------------------------------------------

def build_page_problem(
    *,
    name: str,
    seed: int,
    ctx_lens: Sequence[int],
    chunk_lens: Sequence[int],
    page_size: int,
    Hq: int,
    Hkv: int,
    d: int,
    num_slots: int,
    q_dtype: str,
    kv_dtype: str,
    out_dtype: str,
    select: str = "random",
    history_pages: Optional[int] = None,
    shuffle_slots: bool = False,
    share_sel_across_heads: bool = False,
    pad_rows: int = 0,
    extra_phys_pages: int = 0,
    q_zero: bool = False,
    description: str = "",
) -> Problem:
    """Build a page-selection problem.

    Request b holds ``ctx_lens[b]`` cached tokens followed by
    ``chunk_lens[b]`` new query tokens (query position = ctx + index, so the
    causal diagonal is bottom-right aligned).  Slot 0 of every
    (token, KV head) selects the token's own page; the other slots take up to
    ``history_pages`` (default num_slots - 1) distinct earlier pages drawn
    uniformly without replacement, in draw order.  Unused slots have mask 0
    and index -1.  ``select='all'`` selects every page up to the own page
    (needs num_slots >= pages).  Physical pages are one global random
    permutation; unused page-table entries hold -1.
    """
    assert q_dtype in Q_DTYPES and kv_dtype in KV_DTYPES
    rng = np.random.default_rng(seed)
    B = len(ctx_lens)
    assert len(chunk_lens) == B and Hq % Hkv == 0
    seq_lens = np.array([c + n for c, n in zip(ctx_lens, chunk_lens)], dtype=np.int64)
    pages_per_seq = [(int(s) + page_size - 1) // page_size for s in seq_lens]
    max_pages = max(pages_per_seq)
    total_pages = sum(pages_per_seq) + extra_phys_pages
    perm = rng.permutation(total_pages).astype(np.int32)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        page_table[b, :n] = perm[off:off + n]
        off += n

    # query rows (padding rows at the end, attached to request 0)
    q_seq_l, q_pos_l = [], []
    for b in range(B):
        q_seq_l.append(np.full(chunk_lens[b], b, dtype=np.int32))
        q_pos_l.append(np.arange(ctx_lens[b], ctx_lens[b] + chunk_lens[b], dtype=np.int32))
    q_seq = np.concatenate(q_seq_l + [np.zeros(pad_rows, dtype=np.int32)])
    q_pos = np.concatenate(q_pos_l + [np.full(pad_rows, -1, dtype=np.int32)])
    total_q = len(q_seq)

    # selections
    K = num_slots
    hist = K - 1 if history_pages is None else history_pages
    n_sel_heads = 1 if share_sel_across_heads else Hkv
    sel_idx = np.full((total_q, n_sel_heads, K), -1, dtype=np.int32)
    sel_mask = np.zeros((total_q, n_sel_heads, K), dtype=np.uint8)
    own = np.where(q_pos >= 0, q_pos // page_size, 0).astype(np.int64)
    if select == "random":
        sel_idx[:, :, 0] = own[:, None]
        sel_mask[:, :, 0] = 1
        if hist > 0 and max_pages > 1:
            keys = rng.random((total_q, n_sel_heads, max_pages))
            pages = np.arange(max_pages)[None, None, :]
            keys = np.where(pages < own[:, None, None], keys, np.inf)
            take = min(hist, max_pages)
            order = np.argsort(keys, axis=-1, kind="stable")[:, :, :take]
            chosen_key = np.take_along_axis(keys, order, axis=-1)
            ok = np.isfinite(chosen_key)
            sel_idx[:, :, 1:1 + take] = np.where(ok, order, -1)
            sel_mask[:, :, 1:1 + take] = ok.astype(np.uint8)
    elif select == "all":
        assert K >= max_pages, "select='all' needs a slot per page"
        for p in range(max_pages):
            ok = own >= p
            sel_idx[:, :, p] = np.where(ok, p, -1)[:, None]
            sel_mask[:, :, p] = ok[:, None]
    else:
        raise ValueError(select)
    if shuffle_slots:
        order = np.argsort(rng.random(sel_idx.shape), axis=-1)
        sel_idx = np.take_along_axis(sel_idx, order, axis=-1)
        sel_mask = np.take_along_axis(sel_mask, order, axis=-1)
    if pad_rows:
        # padding rows carry garbage selections that must be ignored
        sel_idx[total_q - pad_rows:] = rng.integers(0, max_pages, (pad_rows, n_sel_heads, K))
        sel_mask[total_q - pad_rows:] = 1
    if share_sel_across_heads:
        sel_idx = np.ascontiguousarray(np.broadcast_to(sel_idx, (total_q, Hkv, K)))
        sel_mask = np.ascontiguousarray(np.broadcast_to(sel_mask, (total_q, Hkv, K)))

    # values
    qf = np.zeros((total_q, Hq, d), np.float32) if q_zero else _randn(rng, (total_q, Hq, d))
    kf = _randn(rng, (total_pages, page_size, Hkv, d))
    vf = _randn(rng, (total_pages, page_size, Hkv, d))
    q_scale = k_scale = v_scale = 1.0
    if q_dtype == "e4m3":
        q, q_scale = quantize_e4m3_tensor(torch.from_numpy(qf))
    else:
        q = torch.from_numpy(qf).to(TORCH_DTYPE[q_dtype])
    k_sf = v_sf = None
    if kv_dtype == "nvfp4":
        k_cache, k_sf, k_scale = quantize_nvfp4(kf)
        v_cache, v_sf, v_scale = quantize_nvfp4(vf)
    elif kv_dtype == "e4m3":
        k_cache, k_scale = quantize_e4m3_tensor(torch.from_numpy(kf))
        v_cache, v_scale = quantize_e4m3_tensor(torch.from_numpy(vf))
    else:
        k_cache = torch.from_numpy(kf).to(TORCH_DTYPE[kv_dtype])
        v_cache = torch.from_numpy(vf).to(TORCH_DTYPE[kv_dtype])

    return Problem(
        name=name, num_seqs=B, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, page_size=page_size,
        unit_tokens=page_size, num_slots=K, slots_per_split=1,
        q_dtype=q_dtype, kv_dtype=kv_dtype, out_dtype=out_dtype,
        q=q.contiguous(),
        q_seq=torch.from_numpy(q_seq), q_pos=torch.from_numpy(q_pos),
        seq_lens=torch.from_numpy(seq_lens.astype(np.int32)),
        page_table=torch.from_numpy(page_table), num_phys_pages=total_pages,
        k_cache=k_cache, v_cache=v_cache, k_sf=k_sf, v_sf=v_sf,
        sel_idx=torch.from_numpy(np.ascontiguousarray(sel_idx)),
        sel_mask=torch.from_numpy(np.ascontiguousarray(sel_mask)),
        sm_scale=1.0 / math.sqrt(d), q_scale=q_scale, k_scale=k_scale, v_scale=v_scale,
        seed=seed, description=description,
    )


# ---------------------------------------------------------------------------
# Paged prefill indexer problems (FP8 queries scored against an FP8 cache).
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class IndexProblem:
    """Queries [total_q, H, d] and a paged cache [pages, page_size, H, d],
    both per-tensor scaled E4M3; the indexer scores every visible page of
    every (token, head) row and keeps the top ``top_k``."""

    name: str
    num_seqs: int
    H: int
    d: int
    page_size: int
    top_k: int
    q: torch.Tensor
    q_seq: torch.Tensor
    q_pos: torch.Tensor
    seq_lens: torch.Tensor
    page_table: torch.Tensor
    num_phys_pages: int
    k_cache: torch.Tensor
    q_scale: float
    k_scale: float
    seed: int = 0
    description: str = ""

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


def build_index_problem(*, name: str, seed: int, ctx_lens: Sequence[int], chunk_lens: Sequence[int],
                        page_size: int, H: int, d: int, top_k: int, pad_rows: int = 0,
                        extra_phys_pages: int = 0, page_bias: float = 0.0,
                        description: str = "") -> IndexProblem:
    """Same request geometry as ``build_page_problem`` (bottom-right aligned
    chunks, one random physical permutation, padding rows at the end).  Values
    N(0, 1); ``page_bias`` adds a per-(page, head) offset along a random query
    direction so that some pages score clearly higher than others."""
    rng = np.random.default_rng(seed)
    B = len(ctx_lens)
    seq_lens = np.array([c + n for c, n in zip(ctx_lens, chunk_lens)], dtype=np.int64)
    pages_per_seq = [(int(x) + page_size - 1) // page_size for x in seq_lens]
    max_pages = max(pages_per_seq)
    total_pages = sum(pages_per_seq) + extra_phys_pages
    perm = rng.permutation(total_pages).astype(np.int32)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        page_table[b, :n] = perm[off:off + n]
        off += n
    q_seq = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(chunk_lens)]
                           + [np.zeros(pad_rows, np.int32)])
    q_pos = np.concatenate([np.arange(c, c + n, dtype=np.int32) for c, n in zip(ctx_lens, chunk_lens)]
                           + [np.full(pad_rows, -1, np.int32)])
    total_q = len(q_seq)
    qf = _randn(rng, (total_q, H, d))
    kf = _randn(rng, (total_pages, page_size, H, d))
    if page_bias:
        u = _randn(rng, (H, d))
        u /= np.linalg.norm(u, axis=-1, keepdims=True)
        qf += 2.0 * u[None]
        kf += (page_bias * rng.standard_normal((total_pages, 1, H, 1))).astype(np.float32) * u[None, None]
    q8, q_scale = quantize_e4m3_tensor(torch.from_numpy(qf))
    k8, k_scale = quantize_e4m3_tensor(torch.from_numpy(kf))
    return IndexProblem(name=name, num_seqs=B, H=H, d=d, page_size=page_size, top_k=top_k,
                        q=q8.contiguous(), q_seq=torch.from_numpy(q_seq),
                        q_pos=torch.from_numpy(q_pos),
                        seq_lens=torch.from_numpy(seq_lens.astype(np.int32)),
                        page_table=torch.from_numpy(page_table), num_phys_pages=total_pages,
                        k_cache=k8.contiguous(), q_scale=q_scale, k_scale=k_scale, seed=seed,
                        description=description)


def make_index_problem(seed: int = 2000) -> IndexProblem:
    """The indexer workload measured beside the attention: the 16K-token
    request of the Q8KV4 workload, 2 indexer heads of dim 128, 16 pages kept."""
    return build_index_problem(
        name="index_q8kv8_16k", seed=seed, ctx_lens=[0], chunk_lens=[16384], page_size=128,
        H=2, d=128, top_k=16, page_bias=1.0,
        description="1 x 16384 tokens, page 128, 2 indexer heads, d 128, E4M3 Q and cache, top 16 pages")


def make_index_short_batch(seed: int = 2004) -> IndexProblem:
    """The indexer on a batch of short chunks over long contexts (the shape
    the adaptive page chunk is for): 8 requests, chunks in {64, 128, 256,
    512}, cached contexts uniform in 16K..128K tokens, 2 heads of dim 128,
    16 pages kept.  Request shapes come from a fixed shape seed."""
    rng = np.random.default_rng(1104)
    chunks = rng.choice([64, 128, 256, 512], size=8)
    ctx = rng.integers(16384, 131072, size=8, endpoint=True)
    return build_index_problem(
        name="index_short_batch", seed=seed, ctx_lens=[int(c) for c in ctx],
        chunk_lens=[int(c) for c in chunks], page_size=128, H=2, d=128, top_k=16, page_bias=1.0,
        description="8 requests, chunks in {64..512}, context U[16K,128K], page 128, 2 indexer "
                    "heads, d 128, E4M3 Q and cache, top 16 pages")


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------

CONFIG_NAMES = (
    "tiny_fp32",
    "bf16_4x4096",
    "q8kv4_16k",
    "grouped_page4_fp16",
    "chunked_batch_q8kv4",
)


def make_config(idx: int, seed: Optional[int] = None, kv_dtype: Optional[str] = None) -> Problem:
    """Synthetic stand-ins for the pages' workloads, seed 1000 + idx.

    ``kv_dtype="e4m3"`` turns the two NVFP4-cache workloads (2 and 4) into
    their FP8-cache (Q8KV8) variants: same shapes, selections and values
    before quantisation."""
    seed = 1000 + idx if seed is None else seed
    if kv_dtype not in (None, "nvfp4", "e4m3") or (kv_dtype == "e4m3" and idx not in (2, 4)):
        raise ValueError(f"no {kv_dtype} variant of workload {idx}")
    fp8 = kv_dtype == "e4m3"
    if idx == 0:
        return build_page_problem(
            name=CONFIG_NAMES[0], seed=seed, ctx_lens=[0], chunk_lens=[512],
            page_size=128, Hq=4, Hkv=1, d=64, num_slots=3, q_dtype="f32",
            kv_dtype="f32", out_dtype="f32",
            description="1 x 512 tokens, page 128, Hkv 1, Hq 4, d 64, FP32, own + 2 earlier pages",
        )
    if idx == 1:
        return build_page_problem(
            name=CONFIG_NAMES[1], seed=seed, ctx_lens=[0] * 4, chunk_lens=[4096] * 4,
            page_size=128, Hq=16, Hkv=1, d=128, num_slots=16, q_dtype="bf16",
            kv_dtype="bf16", out_dtype="bf16",
            description="4 x 4096 tokens, page 128, Hkv 1, Hq 16, d 128, BF16, own + 15 earlier pages",
        )
    if idx == 2:
        return build_page_problem(
            name="q8kv8_16k" if fp8 else CONFIG_NAMES[2], seed=seed, ctx_lens=[0],
            chunk_lens=[16384], page_size=128, Hq=32, Hkv=2, d=128, num_slots=16,
            q_dtype="e4m3", kv_dtype="e4m3" if fp8 else "nvfp4", out_dtype="bf16",
            description=f"1 x 16384 tokens, page 128, Hkv 2, Hq 32, d 128, E4M3 Q, "
                        f"{'E4M3' if fp8 else 'NVFP4'} KV, own + 15 earlier pages per (token, KV head)",
        )
    if idx == 3:
        return make_grouped_page4(seed=seed)
    if idx == 4:
        # request shapes come from a fixed shape seed, so input sets drawn with
        # other seeds (rotated data) keep the same geometry
        rng = np.random.default_rng(1004)
        chunks = rng.choice([128, 256, 512, 1024, 2048, 4096], size=8)
        ctx = rng.integers(8192, 131072, size=8, endpoint=True)
        return build_page_problem(
            name="chunked_batch_q8kv8" if fp8 else CONFIG_NAMES[4], seed=seed + 7919,
            ctx_lens=[int(c) for c in ctx], chunk_lens=[int(c) for c in chunks], page_size=128,
            Hq=16, Hkv=1, d=128, num_slots=16, q_dtype="e4m3",
            kv_dtype="e4m3" if fp8 else "nvfp4", out_dtype="bf16",
            description="8 requests, chunks in {128..4096}, context U[8K,128K], page 128, "
                        f"Hkv 1, Hq 16, d 128, E4M3 Q, {'E4M3' if fp8 else 'NVFP4'} KV, "
                        "own + 15 history pages",
        )
    raise ValueError(idx)


# ---------------------------------------------------------------------------
# Grouped Page4 (microblock) problems.
# ---------------------------------------------------------------------------

def build_microblock_problem(
    *,
    name: str,
    seed: int,
    ctx_len: int,
    chunk_len: int,
    pad_rows: int,
    Hq: int,
    Hkv: int,
    d: int,
    num_slots: int,
    page_size: int = 16,
    unit_tokens: int = 4,
    group_rows: int = 8,
    shared_frac: float = 0.7,
    block16_frac: float = 0.25,
    partial_mask_frac: float = 1.0 / 16,
    interleaved: bool = True,
    spare_pages: int = 4,
    out_dtype: str = "f16",
    description: str = "",
) -> Problem:
    """One prefill chunk with 4-token microblock selections (FP16).

    Every real row selects its own microblock (slot 0, all four mask bits
    set; the causal rule trims it) and ``num_slots - 1`` history units.  Rows
    of the same ``group_rows``-row group share about ``shared_frac`` of their
    history units, drawn from history visible to the whole group; the rest
    are row-specific.  About ``block16_frac`` of the budget is spent as whole
    16-token blocks (four consecutive units, mask 0xF), and a fraction
    ``partial_mask_frac`` of history units carries a random nonzero partial
    4-bit mask.  The KV cache is stored K/V-interleaved
    ``[blocks, 2, page, Hkv, d]`` (FP16) with a random physical order; the
    last page is a partial tail.  Padding rows (q_pos = -1) close the chunk.
    """
    rng = np.random.default_rng(seed)
    assert page_size % unit_tokens == 0 and unit_tokens <= 8
    seq_len = ctx_len + chunk_len
    n_pages = (seq_len + page_size - 1) // page_size
    total_pages = n_pages + spare_pages
    perm = rng.permutation(total_pages).astype(np.int32)
    page_table = perm[:n_pages][None, :].copy()
    total_q = chunk_len + pad_rows
    q_pos = np.concatenate([np.arange(ctx_len, seq_len, dtype=np.int32),
                            np.full(pad_rows, -1, np.int32)])
    q_seq = np.zeros(total_q, np.int32)
    K = num_slots
    upb = page_size // unit_tokens       # units per 16-token block
    sel_idx = np.full((total_q, Hkv, K), -1, np.int32)
    sel_mask = np.zeros((total_q, Hkv, K), np.uint8)
    full_mask = (1 << unit_tokens) - 1

    def draw_units(count, limit_unit, exclude):
        """`count` distinct history units below limit_unit, ~block16_frac as whole blocks."""
        out: list = []
        taken = set(exclude)
        n_blocks = int(round(count * block16_frac)) // upb
        n_block_cap = limit_unit // upb
        if n_block_cap > 0 and n_blocks > 0:
            blocks = rng.choice(n_block_cap, size=min(n_blocks * 2, n_block_cap), replace=False)
            for bl in blocks:
                us = [int(bl) * upb + i for i in range(upb)]
                if any(u in taken for u in us):
                    continue
                out.extend(us)
                taken.update(us)
                if len(out) >= n_blocks * upb:
                    break
        need = count - len(out)
        if need > 0 and limit_unit > 0:
            cand = rng.choice(limit_unit, size=min(limit_unit, need * 2 + 8), replace=False)
            for u in cand:
                u = int(u)
                if u in taken:
                    continue
                out.append(u)
                taken.add(u)
                if len(out) >= count:
                    break
        return out[:count]

    for g in range(Hkv):
        for gs in range(0, chunk_len, group_rows):
            rows = range(gs, min(gs + group_rows, chunk_len))
            first_pos = ctx_len + gs
            group_limit = first_pos // unit_tokens      # units fully before the group
            n_shared = int(round((K - 1) * shared_frac))
            shared = draw_units(n_shared, group_limit, ())
            for r in rows:
                pos = ctx_len + r
                own_u = pos // unit_tokens
                own_limit = own_u  # history strictly before the own unit
                ex = set(shared) | {own_u}
                own_units = draw_units(K - 1 - len(shared), own_limit, ex)
                units = [own_u] + list(shared) + own_units
                masks = [full_mask] * len(units)
                for i in range(1, len(units)):
                    if rng.random() < partial_mask_frac:
                        masks[i] = int(rng.integers(1, full_mask + 1))
                n = len(units)
                sel_idx[r, g, :n] = units
                sel_mask[r, g, :n] = masks
    # padding rows carry garbage selections that must be ignored
    if pad_rows:
        sel_idx[chunk_len:] = rng.integers(0, seq_len // unit_tokens, (pad_rows, Hkv, K))
        sel_mask[chunk_len:] = full_mask

    qf = _randn(rng, (total_q, Hq, d))
    kvf = _randn(rng, (total_pages, 2, page_size, Hkv, d))
    kv = torch.from_numpy(kvf).to(torch.float16)
    if interleaved:
        k_cache, v_cache = kv[:, 0], kv[:, 1]
    else:
        k_cache, v_cache = kv[:, 0].contiguous(), kv[:, 1].contiguous()
    return Problem(
        name=name, num_seqs=1, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, page_size=page_size,
        unit_tokens=unit_tokens, num_slots=K, slots_per_split=K,
        q_dtype="f16", kv_dtype="f16", out_dtype=out_dtype,
        q=torch.from_numpy(qf).to(torch.float16),
        q_seq=torch.from_numpy(q_seq), q_pos=torch.from_numpy(q_pos),
        seq_lens=torch.tensor([seq_len], dtype=torch.int32),
        page_table=torch.from_numpy(page_table), num_phys_pages=total_pages,
        k_cache=k_cache, v_cache=v_cache, k_sf=None, v_sf=None,
        sel_idx=torch.from_numpy(sel_idx), sel_mask=torch.from_numpy(sel_mask),
        sm_scale=1.0 / math.sqrt(d), seed=seed, description=description,
    )


def make_grouped_page4(seed: int = 1003, chunk_len: int = 8120, pad_rows: int = 72,
                       ctx_len: int = 24576, num_slots: int = 512) -> Problem:
    return build_microblock_problem(
        name=CONFIG_NAMES[3], seed=seed, ctx_len=ctx_len, chunk_len=chunk_len,
        pad_rows=pad_rows, Hq=6, Hkv=1, d=256, num_slots=num_slots,
        description=f"{chunk_len}+{pad_rows} rows at positions {ctx_len}.., block 16, unit 4, "
                    f"Hq 6 on 1 latent KV head of dim 256, {num_slots} units/row, FP16",
    )


def make_page4_small_chunk(seed: int = 1005, chunk_len: int = 48, ctx_len: int = 150288,
                           num_slots: int = 512, slots_per_split: int = 32) -> Problem:
    """A chunk below 64 rows on the grouped Page4 geometry (Hq 6 on one KV
    head of dim 256, 4-token units, 512 units per row, FP16), with the
    selections cut into num_slots / slots_per_split splits: the split-k form
    of the microblock route for small chunks (1Cat-vLLM PR 387, section
    "Purpose": the single-row route kept as a many-partition fallback; the
    pages' kernel benchmark runs at 24,240 and 150,288 tokens of context)."""
    p = build_microblock_problem(
        name="page4_small_chunk", seed=seed, ctx_len=ctx_len, chunk_len=chunk_len, pad_rows=0,
        Hq=6, Hkv=1, d=256, num_slots=num_slots,
        description=f"{chunk_len} rows at positions {ctx_len}.., block 16, unit 4, Hq 6 on 1 "
                    f"latent KV head of dim 256, {num_slots} units/row in "
                    f"{num_slots // slots_per_split} splits, FP16",
    )
    return dataclasses.replace(p, slots_per_split=slots_per_split)


def random_partials(seed: int, num_splits: int, num_rows: int, d_v: int,
                    empty_frac: float = 0.1, all_empty_rows: int = 3):
    """Random FP32 partials for a standalone combine test.

    Returns (partial_o [S, rows, d_v], partial_lse [S, rows]) with a fraction
    of slots marked empty (lse = -inf) and a few rows whose every slot is
    empty.
    """
    rng = np.random.default_rng(seed)
    po = rng.standard_normal((num_splits, num_rows, d_v), dtype=np.float32)
    pl = (rng.standard_normal((num_splits, num_rows)) * 3.0 + 2.0).astype(np.float32)
    pl[rng.random((num_splits, num_rows)) < empty_frac] = -np.inf
    if all_empty_rows:
        rows = rng.choice(num_rows, size=min(all_empty_rows, num_rows), replace=False)
        pl[:, rows] = -np.inf
    return torch.from_numpy(po), torch.from_numpy(pl)
