"""GPU parity of the grouped microblock route (4-token units with exact
per-row masks, 8-token groups; one split, or several in its split-k form)
against the FP64 oracle, through the C ABI.  Tolerances are defined in
tests/parity.py."""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_paged_table_amd import synth
from block_sparse_paged_table_amd.runner import DeviceProblem
import oracle
from parity import check_combined, check_partials, gpu_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _mb(seed, **kw):
    args = dict(name="mb", seed=seed, ctx_len=200, chunk_len=45, pad_rows=3, Hq=6, Hkv=1, d=256,
                num_slots=48, page_size=16, spare_pages=3)
    args.update(kw)
    return synth.build_microblock_problem(**args)


def _parity(p, out_dtype=None):
    dp = DeviceProblem(p, out_dtype=out_dtype)
    dp.run()
    torch.cuda.synchronize()
    ref = oracle.prefill_rows(p)
    po, pl, out, lse = gpu_rows(dp, np.arange(p.total_q))
    check_partials(p, po, pl, ref)
    check_combined(p, out, lse, ref, dp.out_dtype)
    assert dp.err_flags() == ref["err"]
    return dp


# head_dim 256 with 8 / 6 / 3 / 2 query heads per KV head: 4 / 3 / 2 / 1 row
# tiles of a group, so every wave loads (4) or 1 / 2 / 3 tileless waves load
@pytest.mark.parametrize("Hq,Hkv,d", [(6, 1, 256), (6, 1, 128), (1, 1, 128), (2, 1, 256),
                                      (8, 1, 128), (12, 2, 256), (3, 3, 128), (8, 1, 256),
                                      (3, 1, 256)])
def test_grouped_small_all_rows(Hq, Hkv, d):
    _parity(_mb(31, Hq=Hq, Hkv=Hkv, d=d))


@pytest.mark.parametrize("ctx_len", [100000, 150000])
def test_grouped_long_context_one_split(ctx_len):
    """One split over contexts of 25K and 37.5K four-token units (the
    planner's bitmap pass, below and above 2^15 units), every row."""
    _parity(_mb(41, ctx_len=ctx_len, chunk_len=37, num_slots=96))


@pytest.mark.parametrize("pd", ["f16", "bf16"])
def test_grouped_16bit_partials(pd):
    """16-bit partial storage on the grouped route: the rounding of the FP32
    partials bit for bit, within the storage floor of the oracle's."""
    p = _mb(35)
    dp = DeviceProblem(p, partial_dtype=pd)
    dp.run()
    dp32 = DeviceProblem(p)
    dp32.run()
    torch.cuda.synchronize()
    assert torch.equal(dp.partial_lse, dp32.partial_lse)
    live = dp32.partial_lse > -float("inf")
    assert torch.equal(dp.partial_o[live], dp32.partial_o[live].to(dp.partial_o.dtype))
    ref = oracle.prefill_rows(p)
    po, pl, _, _ = gpu_rows(dp, np.arange(p.total_q))
    check_partials(p, po, pl, ref, stored=pd)


def test_grouped_contiguous_cache_and_f32_output():
    _parity(_mb(32, interleaved=False), out_dtype="f32")


def test_grouped_ragged_group_and_early_rows():
    # 37 tokens: the last group is partial; the chunk starts at position 0, so
    # early rows see few units and some see nothing but their own
    _parity(_mb(33, ctx_len=0, chunk_len=37, pad_rows=0, num_slots=16))


def test_grouped_errors_and_duplicates():
    p = _mb(34, num_slots=24)
    si, sm = p.sel_idx.numpy().copy(), p.sel_mask.numpy().copy()
    si[2, 0, 5], sm[2, 0, 5] = 10 ** 6, 0xF                   # unit beyond the table
    si[7, 0, 9], sm[7, 0, 9] = si[7, 0, 1], 0x3                 # duplicate unit, other bits
    sm[11] = 0                                                   # row with no selection
    pt = p.page_table.numpy().copy()
    pt[0, 3] = p.num_phys_pages + 4                              # bad physical page
    p = dataclasses.replace(p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm),
                            page_table=torch.from_numpy(pt))
    dp = _parity(p)
    assert dp.err_flags() & (1 | 8)


@pytest.mark.parametrize("spp", [48, 12])
def test_grouped_two_requests_in_one_group(spp):
    """Groups whose 8 tokens belong to two requests (the planner then sorts its
    full 64-bit keys; single-request groups sort 32-bit keys): the tokens from
    13 on become a second request that shares the first one's pages, so its
    rows select the same logical units of an identical cache."""
    p = _mb(37)
    q_seq = p.q_seq.clone()
    q_seq[13:] = torch.where(q_seq[13:] >= 0, torch.ones_like(q_seq[13:]), q_seq[13:])
    p = dataclasses.replace(p, num_seqs=2, q_seq=q_seq, slots_per_split=spp,
                            seq_lens=torch.cat([p.seq_lens, p.seq_lens]),
                            page_table=torch.cat([p.page_table, p.page_table]))
    _parity(p, out_dtype="f32")


def test_grouped_three_runs_bitwise_identical():
    p = _mb(35)
    dp = DeviceProblem(p)
    snaps = []
    for _ in range(3):
        dp.partial_o.fill_(0)
        dp.run()
        torch.cuda.synchronize()
        snaps.append((dp.partial_o.clone(), dp.partial_lse.clone(), dp.out.clone()))
    for s in snaps[1:]:
        assert all(torch.equal(x, y) for x, y in zip(snaps[0], s))


def test_grouped_all_invalid_group_bitwise_zero():
    p = _mb(36, chunk_len=16, pad_rows=8, num_slots=12)
    sm = p.sel_mask.numpy().copy()
    sm[0:8] = 0                                  # a whole group selects nothing
    p = dataclasses.replace(p, sel_mask=torch.from_numpy(sm))
    dp = _parity(p)
    out = dp.out[: 8 * p.Hq].float().cpu().numpy()
    assert np.all(out == 0.0) and not np.signbit(out).any()
    assert torch.all(torch.isneginf(dp.lse[: 8 * p.Hq]))


@pytest.mark.parametrize("spp", [None, 12])
def test_grouped_empty_batch(spp):
    """total_q = 0 on the microblock route (one split, and its split-k form)
    launches nothing past clearing the error word; its buffers are NULL."""
    p = _mb(37, num_slots=48)
    if spp is not None:
        p = dataclasses.replace(p, slots_per_split=spp)
    empty = dataclasses.replace(p, q=p.q[:0], q_seq=p.q_seq[:0], q_pos=p.q_pos[:0],
                                sel_idx=p.sel_idx[:0], sel_mask=p.sel_mask[:0])
    dp = DeviceProblem(empty)
    dp.err.fill_(7)
    dp.run()
    torch.cuda.synchronize()
    assert dp.err_flags() == 0


def test_grouped_full_size_config_sampled():
    p = synth.make_config(3)
    dp = DeviceProblem(p)
    dp.run()
    torch.cuda.synchronize()
    assert dp.err_flags() == 0
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([[0, 1, 7, 8, 4095, 8119, 8120, 8191],
                                     rng.choice(p.total_q, 40, replace=False)]))
    ref = oracle.prefill_rows(p, toks)
    po, pl, out, lse = gpu_rows(dp, toks)
    check_partials(p, po, pl, ref)
    check_combined(p, out, lse, ref, dp.out_dtype)
    # padding rows: +0 output and lse = -inf
    pad = np.nonzero(p.q_pos.numpy() < 0)[0]
    rows = (pad[:, None] * p.Hq + np.arange(p.Hq)[None]).ravel()
    o = dp.out[torch.as_tensor(rows, device="cuda")].float().cpu().numpy()
    assert np.all(o == 0.0) and not np.signbit(o).any()


# ------------------------------------------------------------ split-k form

@pytest.mark.parametrize("spp", [1, 4, 12, 16, 48])
def test_grouped_splits(spp):
    """slots_per_split < num_slots: every (group, KV head, split) is its own
    softmax over the units whose first slot for a row lies in the split."""
    p = dataclasses.replace(_mb(37), slots_per_split=spp)
    dp = _parity(p)
    assert dp.partial_lse.shape[0] == 48 // spp


def test_grouped_split_duplicate_in_later_split():
    p = dataclasses.replace(_mb(38, num_slots=24), slots_per_split=4)
    si, sm = p.sel_idx.numpy().copy(), p.sel_mask.numpy().copy()
    for r in (3, 20, 44):
        si[r, 0, 13], sm[r, 0, 13] = si[r, 0, 2], 0xF   # repeated in split 3: ignored
    si[9, 0, 19], sm[9, 0, 19] = si[9, 0, 17], 0x5       # repeated within split 4
    p = dataclasses.replace(p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm))
    dp = _parity(p)
    assert dp.err_flags() == 8


def test_grouped_splits_ragged_early_rows_and_padding():
    # the chunk starts at position 0: early rows leave most splits empty
    _parity(dataclasses.replace(_mb(39, ctx_len=0, chunk_len=29, pad_rows=5, num_slots=16),
                                slots_per_split=2))


def test_grouped_splits_bitwise_repeatable():
    p = dataclasses.replace(_mb(40), slots_per_split=8)
    dp = DeviceProblem(p)
    snaps = []
    for _ in range(3):
        dp.partial_o.fill_(0)
        dp.run()
        torch.cuda.synchronize()
        snaps.append((dp.partial_o.clone(), dp.partial_lse.clone(), dp.out.clone()))
    for s in snaps[1:]:
        assert all(torch.equal(x, y) for x, y in zip(snaps[0], s))


@pytest.mark.parametrize("ctx_len,spp", [(24240, 32), (150288, 16), (150288, 8)])
def test_page4_small_chunk_workload(ctx_len, spp):
    """The small-chunk workload at its full size (48 rows, 512 units per row;
    16, 32 and 64 splits), every row against the oracle.  Over 150K tokens of
    context 32 and 64 splits take the planner's bitmap pass with more than
    64 KiB of LDS (its latency-mode budget)."""
    p = synth.make_page4_small_chunk(ctx_len=ctx_len, slots_per_split=spp)
    _parity(p)


@pytest.mark.parametrize("spp", [48, 12])
def test_grouped_graph_capture_replays_match_eager(spp):
    """Grouped plan + attention + combine captured in one HIP graph (kernels
    only: the planner clears its counters with a kernel, not a memset node);
    every replay, with eager work and clobbered outputs in between,
    reproduces the eager results bit for bit, one split or split-k."""
    p = dataclasses.replace(_mb(41), slots_per_split=spp)
    dp = DeviceProblem(p)
    dp.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dp.partial_lse, dp.partial_o, dp.out, dp.lse)]
    err = dp.err_flags()
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
        assert dp.err_flags() == err
        dp.run()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("spp", [48, 12])
def test_grouped_row_major_partials(spp):
    """Grouped route with partial_o laid out [row][split][d]: bit for bit the
    split-major results, and the oracle's within tolerance."""
    p = dataclasses.replace(_mb(43), slots_per_split=spp)
    dp = DeviceProblem(p, partial_layout="row")
    dp.run()
    ref = DeviceProblem(p)
    ref.run()
    torch.cuda.synchronize()
    live = ref.partial_lse > -float("inf")
    assert torch.equal(dp.partial_lse, ref.partial_lse)
    assert torch.equal(dp.partial_o[live], ref.partial_o[live])
    assert torch.equal(dp.out, ref.out) and torch.equal(dp.lse, ref.lse)
    oref = oracle.prefill_rows(p)
    po, pl, out, lse = gpu_rows(dp, np.arange(p.total_q))
    check_partials(p, po, pl, oref)
    check_combined(p, out, lse, oref, dp.out_dtype)
