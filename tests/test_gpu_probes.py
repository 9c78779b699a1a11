"""Bit-exact index probes of the FP8 page routes and the grouped microblock
route on the GPU, through the C ABI: every partial output of the probe
problems of tests/probes.py (known in closed form) must come out bit for
bit, and the oracle must agree with the same closed form.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_paged_table_amd import synth
from block_sparse_paged_table_amd.runner import DeviceProblem
import oracle
import probes

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("kv_dtype,d", [("nvfp4", 128), ("e4m3", 128), ("e4m3", 64)])
def test_fp8_page_onehot_probe_bitexact(kv_dtype, d):
    """Q8KV4 / Q8KV8 page gather, slot -> split placement, causal limit and
    the V-side dequantisation, bit for bit: every live partial equals
    v_scale times the fields of its page's last visible key."""
    p, fdims = probes.page_probe(kv_dtype, d, seed=51 if kv_dtype == "nvfp4" else 52)
    dp = DeviceProblem(p)
    dp.run()
    torch.cuda.synchronize()
    po = dp.partial_o.cpu().numpy()
    pl = dp.partial_lse.cpu().numpy()
    exp = probes.expected_page_rows(p, fdims)
    G = p.Hq // p.Hkv
    checked = 0
    for (t, g, j), row in exp.items():
        rows = t * p.Hq + g * G + np.arange(G)
        if row is None:
            assert np.all(np.isneginf(pl[j, rows])), (t, g, j)
            continue
        assert np.all(np.isfinite(pl[j, rows])), (t, g, j)
        got = po[j, rows]
        assert np.array_equal(got.view(np.uint32), np.broadcast_to(row, got.shape).view(np.uint32)), \
            (t, g, j, got[0, fdims], row[fdims])
        checked += 1
    assert checked > 2000
    # the oracle reproduces the same rows exactly
    ref = oracle.prefill_rows(p, want_single_pass=False)
    for (t, g, j), row in exp.items():
        if row is not None:
            assert np.array_equal(ref["part_o"][t, g * G, j], row), (t, g, j)
        else:
            assert np.isneginf(ref["part_lse"][t, g * G, j])


@pytest.mark.parametrize("spp", [1, 24, 6])
def test_microblock_onehot_probe_bitexact(spp):
    """Grouped route: unit gather through the page table, per-row 4-bit
    masks, causal trim and split placement, bit for bit.  One slot per
    split pins every selected unit; one split pins the union; 6 slots per
    split the split-k form."""
    p = probes.mb_probe(61, spp)
    dp = DeviceProblem(p, out_dtype="f32")
    dp.run()
    torch.cuda.synchronize()
    po = dp.partial_o.cpu().numpy()
    pl = dp.partial_lse.cpu().numpy()
    exp = probes.expected_mb_rows(p)
    G = p.Hq // p.Hkv
    checked = 0
    for (t, g, s), row in exp.items():
        rows = t * p.Hq + g * G + np.arange(G)
        if row is None:
            assert np.all(np.isneginf(pl[s, rows])), (t, g, s)
            continue
        got = po[s, rows]
        assert np.array_equal(got.view(np.uint32), np.broadcast_to(row, got.shape).view(np.uint32)), \
            (t, g, s, got[0, :4], row[:4])
        checked += 1
    assert checked >= p.total_q - 8
    ref = oracle.prefill_rows(p, want_single_pass=False)
    for (t, g, s), row in exp.items():
        if row is not None:
            assert np.array_equal(ref["part_o"][t, g * G, s], row), (t, g, s)
        else:
            assert np.isneginf(ref["part_lse"][t, g * G, s])


@pytest.mark.parametrize("spp", [48, 12])
def test_grouped_physical_permutation_bitwise_invariant(spp):
    """Moving the physical blocks of the interleaved K/V cache (and the page
    table with them) changes no bit of any partial, output or LSE."""
    p = dataclasses.replace(synth.build_microblock_problem(
        name="mb", seed=62, ctx_len=200, chunk_len=45, pad_rows=3, Hq=6, Hkv=1, d=256,
        num_slots=48, page_size=16, spare_pages=5), slots_per_split=spp)
    base = p.k_cache._base
    assert base is not None and base.shape[1] == 2
    perm = np.random.default_rng(4).permutation(p.num_phys_pages)
    base2 = torch.empty_like(base)
    base2[torch.from_numpy(perm)] = base
    pt = p.page_table.numpy()
    pt2 = np.where(pt >= 0, perm[np.maximum(pt, 0)], -1).astype(np.int32)
    p2 = dataclasses.replace(p, k_cache=base2[:, 0], v_cache=base2[:, 1],
                             page_table=torch.from_numpy(pt2))
    a, b = DeviceProblem(p), DeviceProblem(p2)
    a.run()
    b.run()
    torch.cuda.synchronize()
    assert torch.equal(a.partial_lse, b.partial_lse)
    fin = torch.isfinite(a.partial_lse)
    assert fin.any()
    assert torch.equal(a.partial_o[fin], b.partial_o[fin])
    assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse)
