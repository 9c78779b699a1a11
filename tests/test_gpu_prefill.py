"""GPU parity of the page-selection route (plan + attention + combine)
against the FP64 oracle, through the C ABI.

Small problems are compared on every row; the full-size workloads (the
shapes bench.py times, in the same launch configuration) on sampled tokens
that the oracle computes one by one, plus the exact empty-slot pattern over
all rows.  Tolerances are defined in tests/parity.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_paged_table_amd import synth
from block_sparse_paged_table_amd.runner import DeviceProblem
import oracle
from parity import check_combined, check_partials, gpu_rows, rel_l2

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _run(p, **kw):
    dp = DeviceProblem(p, **kw)
    dp.run()
    torch.cuda.synchronize()
    return dp


def _full_parity(p, out_dtype=None, **kw):
    dp = _run(p, out_dtype=out_dtype, **kw)
    ref = oracle.prefill_rows(p)
    po, pl, out, lse = gpu_rows(dp, np.arange(p.total_q))
    r1 = check_partials(p, po, pl, ref)
    r2 = check_combined(p, out, lse, ref, dp.out_dtype)
    assert dp.err_flags() == ref["err"]
    return dp, r1, r2


def _small(seed, **kw):
    args = dict(name="small", seed=seed, ctx_lens=[0, 300], chunk_lens=[700, 450],
                page_size=128, Hq=16, Hkv=1, d=128, num_slots=8, q_dtype="bf16",
                kv_dtype="bf16", out_dtype="f32", pad_rows=5, shuffle_slots=True)
    args.update(kw)
    return synth.build_page_problem(**args)


def test_tiny_fp32_config_all_rows():
    p = synth.make_config(0)
    _full_parity(p)
    _full_parity(p, out_dtype="f32")


@pytest.mark.parametrize("qd,kd,d", [("bf16", "bf16", 128), ("f16", "f16", 128),
                                     ("bf16", "bf16", 64), ("f16", "f16", 64),
                                     ("f32", "f32", 128), ("e4m3", "nvfp4", 128),
                                     ("e4m3", "e4m3", 128), ("e4m3", "e4m3", 64)])
def test_small_all_rows(qd, kd, d):
    p = _small(11, q_dtype=qd, kv_dtype=kd, d=d, Hq=8, Hkv=2)
    _full_parity(p)


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 1), (4, 2), (6, 1), (8, 1), (32, 2), (48, 3)])
def test_head_groupings(Hq, Hkv):
    p = _small(12, Hq=Hq, Hkv=Hkv, d=64, ctx_lens=[129], chunk_lens=[400], num_slots=4)
    _full_parity(p)


@pytest.mark.parametrize("Hq,Hkv,qd,kd", [(16, 2, "e4m3", "nvfp4"), (48, 3, "bf16", "bf16")])
def test_ordering_slices_bitwise_identical(Hq, Hkv, qd, kd):
    """The unit order (slices of the plan) changes scheduling only: every
    written partial, the combined output and the LSE are bitwise equal for any
    slice length, and match the oracle with many slices."""
    # a long context makes many (slice, page, head) lists: the plan's scan
    # runs over several tiles (slices of 1 and 100 tokens, > 8192 lists), in
    # one workgroup at 8 lists per thread (200, 300: 4097-8192 lists at
    # 16 heads) or at 4 (one slice)
    p = _small(21, Hq=Hq, Hkv=Hkv, q_dtype=qd, kv_dtype=kd, ctx_lens=[0, 20000, 1000],
               chunk_lens=[700, 450, 600], num_slots=8)
    _full_parity(p, order_slice_tokens=1)
    ref = _run(p)
    live = ref.partial_lse > -float("inf")
    assert live.any() and not live.all()
    for st in (1, 100, 200, 300, 1 << 20):
        dp = _run(p, order_slice_tokens=st)
        assert torch.equal(dp.partial_lse, ref.partial_lse), st
        assert torch.equal(dp.partial_o[live], ref.partial_o[live]), st
        assert torch.equal(dp.out, ref.out) and torch.equal(dp.lse, ref.lse), st


def _check_own_combine(p, po, pl, out, lse):
    """The GPU combine of the GPU's own (widened) partials equals the oracle's
    combine of the same values at FP32-combine accuracy."""
    po = np.where(np.isfinite(pl)[..., None], po, 0.0)  # empty splits' rows are unspecified
    own_out, own_lse = oracle.combine(po.reshape(-1, p.num_splits, p.d_v).transpose(1, 0, 2),
                                      pl.reshape(-1, p.num_splits).T)
    own_out = own_out.reshape(out.shape)
    own_lse = own_lse.reshape(lse.shape)
    assert np.array_equal(np.isneginf(lse), np.isneginf(own_lse))
    fin = np.isfinite(own_lse)
    assert rel_l2(out, own_out) <= 1e-5 and np.abs(out - own_out).max() <= 1e-5
    assert np.abs(lse[fin] - own_lse[fin]).max() <= 1e-5


@pytest.mark.parametrize("qd,kd", [("bf16", "bf16"), ("f16", "f16"), ("e4m3", "nvfp4"),
                                   ("e4m3", "e4m3")])
@pytest.mark.parametrize("pd", ["f16", "bf16"])
def test_16bit_partials(qd, kd, pd):
    """BF16 / FP16 partial storage: partials within the storage-rounding floor
    of the oracle's; the combine of those partials equals the oracle's combine
    of the same (widened) values; LSEs stay FP32."""
    p = _small(23, q_dtype=qd, kv_dtype=kd, Hq=8, Hkv=2, out_dtype="f32")
    dp = _run(p, partial_dtype=pd)
    assert dp.partial_o.dtype == (torch.float16 if pd == "f16" else torch.bfloat16)
    ref = oracle.prefill_rows(p)
    po, pl, out, lse = gpu_rows(dp, np.arange(p.total_q))
    check_partials(p, po, pl, ref, stored=pd)
    _check_own_combine(p, po, pl, out, lse)
    # same kernel, FP32 partials: the 16-bit ones are their rounding
    dp32 = _run(p)
    live = dp32.partial_lse > -float("inf")
    assert torch.equal(dp.partial_lse, dp32.partial_lse)
    assert torch.equal(dp.partial_o[live], dp32.partial_o[live].to(dp.partial_o.dtype))


def test_fp32_output_and_bf16_output_agree():
    p = _small(13, out_dtype="bf16")
    dp16 = _run(p)
    dp32 = _run(p, out_dtype="f32")
    assert torch.equal(dp16.out, dp32.out.to(torch.bfloat16))
    ref = oracle.prefill_rows(p)
    _, _, out, lse = gpu_rows(dp16, np.arange(p.total_q))
    check_combined(p, out, lse, ref, "bf16")


@pytest.mark.parametrize("qd,kd,d,pad,pd", [("f32", "f32", 64, 32, "f32"), ("e4m3", "nvfp4", 128, 4, "f32"),
                                            ("bf16", "bf16", 128, 12, "f32"), ("e4m3", "e4m3", 64, 4, "f32"),
                                            ("e4m3", "nvfp4", 128, 4, "f16"), ("bf16", "bf16", 64, 8, "bf16"),
                                            ("e4m3", "e4m3", 128, 24, "f16")])
def test_strided_partial_buffer(qd, kd, d, pad, pd):
    """Padded partial rows (row stride d + pad, so rows are not 128-byte
    aligned): the whole-line stores of FP32 partials and the 16-byte stores of
    16-bit partials (8-byte-aligned rows take 8-byte stores) must land on each
    row's own bytes."""
    p = _small(14, q_dtype=qd, kv_dtype=kd, d=d, Hq=8, Hkv=2)
    dp = _run(p, po_row_pad=pad, partial_dtype=pd)
    ref = oracle.prefill_rows(p)
    po, pl, out, lse = gpu_rows(dp, np.arange(p.total_q))
    check_partials(p, po, pl, ref, stored=pd)
    if pd == "f32":
        check_combined(p, out, lse, ref, "f32")
    else:
        # the combine reads the padded 16-bit rows through the same strides
        # (rows 8-byte aligned only when the pad is not a multiple of 8):
        # equal to the oracle's combine of the GPU's own widened partials
        _check_own_combine(p, po, pl, out, lse)


def test_shared_selection_stride_zero():
    p = _small(15, Hq=8, Hkv=2, share_sel_across_heads=True)
    dp = DeviceProblem(p)
    dp.sel_idx = dp.sel_idx[:, :1].expand(-1, p.Hkv, -1)
    dp.sel_mask = dp.sel_mask[:, :1].expand(-1, p.Hkv, -1)
    dp.desc = dp.make_desc()
    assert dp.desc.sel_stride_head == 0
    dp.run()
    torch.cuda.synchronize()
    ref = oracle.prefill_rows(p)
    po, pl, out, lse = gpu_rows(dp, np.arange(p.total_q))
    check_partials(p, po, pl, ref)
    check_combined(p, out, lse, ref, "f32")


def test_error_flags_and_invalid_rows():
    p = _small(16, num_slots=6, Hq=4, Hkv=1, d=64)
    si, sm = p.sel_idx.numpy().copy(), p.sel_mask.numpy().copy()
    qs = p.q_seq.numpy().copy()
    si[3, 0, 2], sm[3, 0, 2] = p.max_pages + 3, 1        # unit beyond the table row
    si[9, 0, 1], sm[9, 0, 1] = -2, 1                     # negative unit
    src = int(np.nonzero(sm[400, 0])[0][0])              # a used slot of token 400
    dst = 5 if src != 5 else 4
    si[400, 0, dst], sm[400, 0, dst] = si[400, 0, src], 1  # duplicate of that slot
    sm[17] = 0                                           # no selection at all
    qs[20] = 9                                           # request that does not exist
    pt = p.page_table.numpy().copy()
    pt[1, 2] = p.num_phys_pages + 11                     # table entry beyond the cache
    p = dataclasses.replace(p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm),
                            q_seq=torch.from_numpy(qs), page_table=torch.from_numpy(pt))
    dp, _, _ = _full_parity(p)
    assert dp.err_flags() == 1 | 2 | 4 | 8


@pytest.mark.parametrize("K", [1, 2, 3, 17, 33, 64, 65, 100])
def test_slot_counts_and_duplicates(K):
    """Slot counts around the plan's lane mapping (a row's K slots on K
    adjacent lanes up to 64 -- 16, 16, 16, 2, 1 and 1 rows per wave here --
    and a whole wave per row beyond), mostly empty slots (few pages exist),
    and a duplicate selection at a late or an early slot."""
    p = _small(40 + K, num_slots=K, Hq=8, Hkv=2, pad_rows=3)
    if K > 1:
        si, sm = p.sel_idx.numpy().copy(), p.sel_mask.numpy().copy()
        t = 600
        src = int(np.nonzero(sm[t, 1])[0][0])
        dst = K - 1 if src != K - 1 else 0
        si[t, 1, dst], sm[t, 1, dst] = si[t, 1, src], 1
        p = dataclasses.replace(p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm))
    dp, _, _ = _full_parity(p)
    assert dp.err_flags() == (8 if K > 1 else 0)


@pytest.mark.parametrize("K", [8, 65])
def test_many_lists_global_count_path(K):
    """More (request, page) lists per ordering slice than the planner's LDS
    histogram holds (130 requests x a 121-page table row = 15730 > 15360):
    the count takes its positions with one global atomic per selection."""
    ctx = [15360] + [0] * 129
    chunk = [64] + [32] * 129
    p = _small(61 + K, num_slots=K, Hq=4, Hkv=1, d=64, ctx_lens=ctx, chunk_lens=chunk, pad_rows=2)
    assert p.num_seqs * p.max_pages * p.Hkv > 15360
    _full_parity(p)


def test_empty_and_all_padding_batches():
    """total_q = 0 launches nothing and touches nothing; a batch of padding rows
    only gives +0 outputs, lse = -inf and every split empty."""
    p = _small(24, Hq=8, Hkv=2)
    empty = dataclasses.replace(p, q=p.q[:0], q_seq=p.q_seq[:0], q_pos=p.q_pos[:0],
                                sel_idx=p.sel_idx[:0], sel_mask=p.sel_mask[:0])
    dp = DeviceProblem(empty)
    dp.run()
    torch.cuda.synchronize()
    assert dp.err_flags() == 0
    pad = dataclasses.replace(p, q_pos=torch.full_like(p.q_pos, -1))
    dp = _run(pad)
    assert torch.all(torch.isneginf(dp.partial_lse)) and torch.all(torch.isneginf(dp.lse))
    assert torch.all(dp.out == 0) and not torch.any(torch.signbit(dp.out.float()))


@pytest.mark.parametrize("qd,kd", [("bf16", "bf16"), ("e4m3", "nvfp4")])
def test_max_slots_255(qd, kd):
    """The page route's largest slot count (slot ids are 8-bit in the plan):
    255 slots, most of them empty or later than the own page."""
    p = _small(25, q_dtype=qd, kv_dtype=kd, Hq=4, Hkv=1, ctx_lens=[3000, 0],
               chunk_lens=[300, 200], num_slots=255, pad_rows=2)
    _full_parity(p)


def test_physical_permutation_bitwise_invariant():
    p = _small(17, extra_phys_pages=5)
    perm = np.random.default_rng(3).permutation(p.num_phys_pages)
    k2, v2 = torch.empty_like(p.k_cache), torch.empty_like(p.v_cache)
    k2[perm], v2[perm] = p.k_cache, p.v_cache
    pt = p.page_table.numpy()
    pt2 = np.where(pt >= 0, perm[np.maximum(pt, 0)], -1).astype(np.int32)
    p2 = dataclasses.replace(p, k_cache=k2, v_cache=v2, page_table=torch.from_numpy(pt2))
    a, b = _run(p), _run(p2)
    assert torch.equal(a.partial_lse, b.partial_lse)
    fin = torch.isfinite(a.partial_lse)
    assert torch.equal(a.partial_o[fin], b.partial_o[fin])
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)


@pytest.mark.parametrize("qd,kd", [("bf16", "bf16"), ("e4m3", "nvfp4")])
def test_three_runs_bitwise_identical(qd, kd):
    p = _small(18, q_dtype=qd, kv_dtype=kd, Hq=16, Hkv=2)
    dp = DeviceProblem(p)
    snaps = []
    for _ in range(3):
        dp.partial_o.fill_(0)
        dp.run()
        torch.cuda.synchronize()
        snaps.append((dp.partial_o.clone(), dp.partial_lse.clone(), dp.out.clone()))
    for s in snaps[1:]:
        assert all(torch.equal(x, y) for x, y in zip(snaps[0], s))


@pytest.mark.parametrize("qd,kd", [("bf16", "bf16"), ("e4m3", "nvfp4")])
def test_graph_capture_replays_match_eager(qd, kd):
    """plan + attention + combine captured in one HIP graph (kernels only, no
    memset nodes); every replay, with eager work and clobbered outputs in
    between, reproduces the eager results bit for bit."""
    p = _small(22, q_dtype=qd, kv_dtype=kd, Hq=16, Hkv=2)
    dp = DeviceProblem(p)
    dp.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dp.partial_lse, dp.partial_o, dp.out, dp.lse)]
    live = ref[0] > -float("inf")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dp.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dp.run()
    torch.cuda.synchronize()
    for i in range(3):
        for t in (dp.partial_o, dp.out, dp.lse, dp.partial_lse):
            t.fill_(float(i + 1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.partial_lse, ref[0]), i
        assert torch.equal(dp.partial_o[live], ref[1][live]), i
        assert torch.equal(dp.out, ref[2]) and torch.equal(dp.lse, ref[3]), i
        assert dp.err_flags() == 0
        dp.run()  # eager work between replays
        torch.cuda.synchronize()


def test_onehot_selection_probe_bitexact():
    """Index probe: K[t, 0] = 128 * (t mod page) and Q[., 0] = 16 give logit
    gaps so large that every partial is exactly the value row of the last
    visible key of its page; V encodes (logical page, offset).  Pins the
    page-table gather, slot -> slab placement and the causal diagonal bit
    for bit."""
    p = _small(19, q_dtype="bf16", kv_dtype="bf16", Hq=4, Hkv=1, d=64, ctx_lens=[77, 0],
               chunk_lens=[500, 333], num_slots=5, pad_rows=0)
    P, page, Hkv, d = p.k_cache.shape
    k = torch.zeros((P, page, Hkv, d), dtype=torch.float32)
    k[:, :, :, 0] = 128.0 * torch.arange(page, dtype=torch.float32)[None, :, None]
    v = torch.zeros((P, page, Hkv, d), dtype=torch.float32)
    inv = {}
    pt = p.page_table.numpy()
    for b in range(p.num_seqs):
        for lp in range(pt.shape[1]):
            if pt[b, lp] >= 0:
                inv[int(pt[b, lp])] = (b, lp)
    for phys, (b, lp) in inv.items():
        v[phys, :, :, 0] = float(b)
        v[phys, :, :, 1] = float(lp)
        v[phys, :, :, 2] = torch.arange(page, dtype=torch.float32)[:, None]
    q = torch.zeros(p.q.shape, dtype=torch.float32)
    q[:, :, 0] = 16.0
    p = dataclasses.replace(p, k_cache=k.to(torch.bfloat16), v_cache=v.to(torch.bfloat16),
                            q=q.to(torch.bfloat16), sm_scale=1.0)
    dp = _run(p)
    po = dp.partial_o.cpu().numpy()
    pl = dp.partial_lse.cpu().numpy()
    si, sm = p.sel_idx.numpy(), p.sel_mask.numpy()
    qpos, qseq, sl = p.q_pos.numpy(), p.q_seq.numpy(), p.seq_lens.numpy()
    checked = 0
    for t in range(p.total_q):
        for j in range(p.num_slots):
            rows = t * p.Hq + np.arange(p.Hq)
            if sm[t, 0, j] == 0:
                assert np.all(np.isneginf(pl[j, rows]))
                continue
            u = int(si[t, 0, j])
            last = min(u * page + page - 1, int(qpos[t]), int(sl[qseq[t]]) - 1)
            expect = np.zeros(d, np.float32)
            expect[0], expect[1], expect[2] = qseq[t], u, last - u * page
            assert np.array_equal(po[j, rows], np.broadcast_to(expect, (p.Hq, d))), (t, j)
            checked += 1
    assert checked > 1000


# ---------------------------------------------------------------- full sizes

def _sample_tokens(p, n=48, seed=0):
    rng = np.random.default_rng(seed)
    T = p.total_q
    fixed = [0, 1, 127, 128, 129, T // 2, T - 2, T - 1]
    picks = set(t for t in fixed if 0 <= t < T)
    picks |= set(int(x) for x in rng.choice(T, size=min(n, T), replace=False))
    return np.array(sorted(picks))


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_full_size_config_sampled(cfg):
    p = synth.make_config(cfg)
    dp = _run(p)
    keep = oracle.make_keep(p)
    # exact empty-slot pattern over every row
    ne = oracle.slot_nonempty(p, keep=keep)                   # [T, Hkv, K]
    G = p.Hq // p.Hkv
    ne_rows = np.repeat(ne, G, axis=1).reshape(p.total_q * p.Hq, p.num_slots).T  # [K, rows]
    gpu_empty = torch.isneginf(dp.partial_lse).cpu().numpy()
    assert np.array_equal(gpu_empty, ne_rows == 0)
    assert dp.err_flags() == 0
    toks = _sample_tokens(p)
    ref = oracle.prefill_rows(p, toks, keep=keep)
    po, pl, out, lse = gpu_rows(dp, toks)
    check_partials(p, po, pl, ref)
    check_combined(p, out, lse, ref, dp.out_dtype)


@pytest.mark.parametrize("cfg,pd", [(2, "f16"), (2, "bf16"), (4, "bf16"), (1, "f16")])
def test_full_size_16bit_partials(cfg, pd):
    """16-bit partial storage at full size, in the launch configuration the
    benchmark's partial-dtype variants time: every live partial is the
    rounding of the same kernel's FP32 partial (whole tensor, bit for bit),
    the LSEs are identical, and sampled rows match the oracle within the
    storage-rounding floor."""
    p = synth.make_config(cfg)
    dp32 = _run(p)
    live = dp32.partial_lse > -float("inf")
    dt = torch.float16 if pd == "f16" else torch.bfloat16
    ref16 = dp32.partial_o[live].to(dt)
    lse32 = dp32.partial_lse.clone()
    del dp32
    torch.cuda.empty_cache()
    dp = _run(p, partial_dtype=pd)
    assert dp.partial_o.dtype == dt
    assert torch.equal(dp.partial_lse, lse32)
    assert torch.equal(dp.partial_o[live], ref16)
    assert dp.err_flags() == 0
    del ref16, lse32
    toks = _sample_tokens(p, n=24)
    keep = oracle.make_keep(p)
    ref = oracle.prefill_rows(p, toks, keep=keep)
    po, pl, out, lse = gpu_rows(dp, toks)
    check_partials(p, po, pl, ref, stored=pd)


@pytest.mark.parametrize("qd,kd,pd", [("e4m3", "nvfp4", "f32"), ("bf16", "bf16", "f16"),
                                      ("e4m3", "e4m3", "bf16"), ("f32", "f32", "f32")])
def test_row_major_partials(qd, kd, pd):
    """partial_o laid out [row][split][d] (split stride d, row stride
    splits * d): the same values as the split-major layout, bit for bit, and
    the combine reads them through the same strides."""
    p = _small(27, q_dtype=qd, kv_dtype=kd, Hq=8, Hkv=2, d=64 if qd == "f32" else 128)
    dp = _run(p, partial_dtype=pd, partial_layout="row")
    assert dp.partial_o.stride(0) == p.d_v and dp.partial_o.stride(1) == p.num_splits * p.d_v
    ref = _run(p, partial_dtype=pd)
    live = ref.partial_lse > -float("inf")
    assert live.any() and not live.all()
    assert torch.equal(dp.partial_lse, ref.partial_lse)
    assert torch.equal(dp.partial_o[live], ref.partial_o[live])
    assert torch.equal(dp.out, ref.out) and torch.equal(dp.lse, ref.lse)
    assert dp.err_flags() == ref.err_flags()
    if pd == "f32":
        oref = oracle.prefill_rows(p)
        po, pl, out, lse = gpu_rows(dp, np.arange(p.total_q))
        check_partials(p, po, pl, oref)
        check_combined(p, out, lse, oref, dp.out_dtype)


@pytest.mark.parametrize("cfg", [2, 4])
def test_full_size_row_major_partials(cfg):
    """The benchmark's partial layout at full size: every partial, the output
    and the LSE equal the split-major run bit for bit; sampled rows against
    the oracle."""
    p = synth.make_config(cfg)
    ref = _run(p)
    live = ref.partial_lse > -float("inf")
    ref_o = ref.partial_o[live].clone()
    ref_l, ref_out, ref_lse = ref.partial_lse.clone(), ref.out.clone(), ref.lse.clone()
    del ref
    torch.cuda.empty_cache()
    dp = _run(p, partial_layout="row")
    assert torch.equal(dp.partial_lse, ref_l)
    assert torch.equal(dp.partial_o[live], ref_o)
    assert torch.equal(dp.out, ref_out) and torch.equal(dp.lse, ref_lse)
    assert dp.err_flags() == 0
    del ref_o
    toks = _sample_tokens(p, n=16)
    oref = oracle.prefill_rows(p, toks, keep=oracle.make_keep(p))
    po, pl, out, lse = gpu_rows(dp, toks)
    check_partials(p, po, pl, oref)
    check_combined(p, out, lse, oref, dp.out_dtype)
