"""msa_sparse_prefill_noalloc (the entry point for callers that cannot
allocate: the plan lives in the library's fixed per-device scratch) against
msa_sparse_prefill with a caller workspace, through the C ABI: the same
partials, LSEs and error flags bit for bit, on two calls in a row whose
second problem is smaller than the first (the scratch keeps the first
call's contents), on the page route (BF16 and E4M3/NVFP4) and on the
grouped microblock route (one split and split-k)."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_paged_table_amd as msa
from block_sparse_paged_table_amd import synth
from block_sparse_paged_table_amd.runner import DeviceProblem

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _page(seed, chunks, qd, kd, **kw):
    args = dict(name="na", seed=seed, ctx_lens=[0, 300][:len(chunks)], chunk_lens=chunks,
                page_size=128, Hq=16, Hkv=2, d=128, num_slots=8, q_dtype=qd, kv_dtype=kd,
                out_dtype="f32", pad_rows=3, shuffle_slots=True)
    args.update(kw)
    return synth.build_page_problem(**args)


def _mb(seed, chunk, spp):
    p = synth.build_microblock_problem(name="na_mb", seed=seed, ctx_len=200, chunk_len=chunk,
                                       pad_rows=3, Hq=6, Hkv=1, d=256, num_slots=48,
                                       page_size=16, spare_pages=3)
    return dataclasses.replace(p, slots_per_split=spp)


def _compare(p, null_err=False):
    ref = DeviceProblem(p)
    ref.prefill()
    dp = DeviceProblem(p)
    dp.partial_o.fill_(float("nan"))
    dp.partial_lse.fill_(float("nan"))
    if null_err:
        dp.desc.err_flags = None
    dp.prefill_noalloc()
    torch.cuda.synchronize()
    assert torch.equal(dp.partial_lse, ref.partial_lse)
    live = ref.partial_lse > -float("inf")
    assert live.any()
    assert torch.equal(dp.partial_o[live], ref.partial_o[live])
    if not null_err:
        assert dp.err_flags() == ref.err_flags()
    # and the combine of its partials gives the same rows
    dp.combine()
    ref.combine()
    torch.cuda.synchronize()
    assert torch.equal(dp.out, ref.out) and torch.equal(dp.lse, ref.lse)


@pytest.mark.parametrize("qd,kd", [("bf16", "bf16"), ("e4m3", "nvfp4")])
def test_noalloc_page_route_two_calls(qd, kd):
    _compare(_page(71, [900, 700], qd, kd))
    _compare(_page(72, [333], qd, kd, Hq=8, num_slots=5), null_err=True)


def test_noalloc_grouped_route_two_calls():
    _compare(_mb(73, 61, 48))
    _compare(_mb(74, 21, 12))


def test_noalloc_errors_flagged():
    p = _page(75, [500], "bf16", "bf16", Hq=4, Hkv=1, num_slots=6)
    si, sm = p.sel_idx.numpy().copy(), p.sel_mask.numpy().copy()
    si[3, 0, 2], sm[3, 0, 2] = p.max_pages + 3, 1
    p = dataclasses.replace(p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm))
    dp = DeviceProblem(p)
    dp.prefill_noalloc()
    torch.cuda.synchronize()
    assert dp.err_flags() == msa.MSA_ERRF_SEL_RANGE
    _compare(p)


def test_noalloc_rejects_problems_beyond_the_scratch():
    p = synth.make_grouped_page4()
    dp = DeviceProblem(p)
    assert dp.ws_bytes > msa.msa_noalloc_scratch_bytes()
    with pytest.raises(msa.MsaError) as e:
        dp.prefill_noalloc()
    assert e.value.status == 3 and "scratch" in str(e.value)
