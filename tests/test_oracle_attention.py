"""Pins for the oracle's attention and combine (CPU only).

The oracle (oracle/oracle.c) is checked against things other than itself:
  * dense equivalence -- selecting every visible page must equal dense causal
    attention computed by torch.nn.functional.scaled_dot_product_attention
    (float64, CPU, explicit bottom-right causal mask);
  * the split/combine identity -- merging per-split partials by their LSEs
    equals one softmax over the union of the selected keys
    (MiniMax-AI/MSA PR 21, section "Combine");
  * invariances -- physical page placement and slot order do not change the
    result;
  * closed forms -- zero queries (uniform weights), constant values, a single
    visible key;
  * all-invalid rows give +0 outputs and lse = -inf (1Cat-vLLM PR 387,
    section "Test Result");
  * an independent numpy brute force (oracle/bruteforce.py) on tiny inputs,
    including NVFP4 keys/values, E4M3 queries and 4-token microblocks.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_paged_table_amd import synth
import oracle
from oracle import bruteforce

pytestmark = pytest.mark.usefixtures("oracle_lib")

TOL = 1e-12


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def _small(seed=1, **kw):
    args = dict(name="small", seed=seed, ctx_lens=[5, 0], chunk_lens=[27, 19], page_size=8,
                Hq=4, Hkv=2, d=16, num_slots=3, q_dtype="f32", kv_dtype="f32", out_dtype="f32")
    args.update(kw)
    return synth.build_page_problem(**args)


def _assert_same_finite(a, b, tol=TOL):
    a, b = np.asarray(a), np.asarray(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    fin = np.isfinite(b)
    if fin.any():
        assert np.abs(a[fin] - b[fin]).max() <= tol * max(1.0, np.abs(b[fin]).max())


# ------------------------------------------------------------ dense equivalence

@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("e4m3", "nvfp4"),
                                    ("e4m3", "e4m3")])
def test_dense_equivalence_sdpa(dtypes):
    qd, kd = dtypes
    p = synth.build_page_problem(
        name="dense", seed=11, ctx_lens=[13, 0, 40], chunk_lens=[21, 33, 9], page_size=8,
        Hq=6, Hkv=2, d=32, num_slots=8, q_dtype=qd, kv_dtype=kd, out_dtype="f32",
        select="all", shuffle_slots=True)
    res = oracle.prefill_rows(p)
    q, k, v = bruteforce.values(p)    # library-cast decoding
    pt, seq_lens = p.page_table.numpy(), p.seq_lens.numpy()
    q_seq, q_pos = p.q_seq.numpy(), p.q_pos.numpy()
    G = p.Hq // p.Hkv
    scale = p.sm_scale * p.q_scale * p.k_scale
    for b in range(p.num_seqs):
        L = int(seq_lens[b])
        tpos = np.arange(L)
        phys = pt[b, tpos // p.page_size]
        kl = torch.from_numpy(k[phys, tpos % p.page_size]).permute(1, 0, 2)  # [Hkv, L, d]
        vl = torch.from_numpy(v[phys, tpos % p.page_size] * p.v_scale).permute(1, 0, 2)
        rows = np.nonzero(q_seq == b)[0]
        qq = torch.from_numpy(q[rows]).permute(1, 0, 2)                      # [Hq, n, d]
        mask = torch.from_numpy(tpos[None, :] <= q_pos[rows][:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kl.repeat_interleave(G, 0), vl.repeat_interleave(G, 0),
            attn_mask=mask, scale=scale).permute(1, 0, 2).numpy()
        assert _rel(res["out"][rows], ref) < 1e-12
        assert _rel(res["out1"][rows], ref) < 1e-12


# ------------------------------------------------------------ split / combine

@pytest.mark.parametrize("seed", [1, 2, 3])
def test_split_combine_equals_single_pass(seed):
    p = _small(seed=seed, num_slots=4)
    res = oracle.prefill_rows(p)
    _assert_same_finite(res["lse"], res["lse1"])
    assert _rel(res["out"], res["out1"]) < TOL


def _mb_split(seed, spp, dup_rows=()):
    """Microblock (4-token unit) selections cut into splits of `spp` slots
    (the split-k form of the grouped route, 1Cat-vLLM PR 387, section
    "Purpose": the single-row Page4 route kept as a many-partition
    fallback).  `dup_rows` repeat slot 2's unit in slot 13 (a later split)."""
    p = synth.build_microblock_problem(
        name="mb_split", seed=seed, ctx_len=72, chunk_len=19, pad_rows=2, Hq=4, Hkv=2, d=16,
        num_slots=16, page_size=16, spare_pages=2)
    p = dataclasses.replace(p, slots_per_split=spp)
    if dup_rows:
        si, sm = p.sel_idx.numpy().copy(), p.sel_mask.numpy().copy()
        for r in dup_rows:
            si[r, 0, 13], sm[r, 0, 13] = si[r, 0, 2], 0xF
        p = dataclasses.replace(p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm))
    return p


@pytest.mark.parametrize("spp", [1, 4, 8])
def test_microblock_splits_combine_to_one_split(spp):
    """Merging the per-split partials equals the one-split (spp = K) result,
    and equals the single softmax over the union of the selected keys."""
    split = oracle.prefill_rows(_mb_split(40, spp))
    whole = oracle.prefill_rows(_mb_split(40, 16))
    assert split["part_lse"].shape[2] == 16 // spp
    _assert_same_finite(split["lse"], whole["lse"])
    assert _rel(split["out"], whole["out"]) < TOL
    _assert_same_finite(split["lse"], split["lse1"])
    assert _rel(split["out"], split["out1"]) < TOL


def test_microblock_split_duplicate_in_later_split():
    """A unit selected again in a later split is ignored there (first slot
    wins, over all splits) and flagged."""
    p = _mb_split(41, 4, dup_rows=(3, 10))
    a = oracle.prefill_rows(p)
    b = bruteforce.run(p)
    assert a["err"] == oracle.ERR_DUPLICATE
    _assert_same_finite(a["part_lse"], b["part_lse"])
    fin = np.isfinite(b["part_lse"])
    assert np.abs(a["part_o"][fin] - b["part_o"][fin]).max() < 1e-12
    # the repeated slot adds nothing: same result as with that slot masked off
    sm = p.sel_mask.numpy().copy()
    sm[[3, 10], 0, 13] = 0
    c = oracle.prefill_rows(dataclasses.replace(p, sel_mask=torch.from_numpy(sm)))
    assert c["err"] == 0
    assert np.array_equal(a["part_o"], c["part_o"]) and np.array_equal(a["part_lse"], c["part_lse"])


def test_combine_matches_logaddexp():
    po, pl = synth.random_partials(3, 7, 257, 24, empty_frac=0.3, all_empty_rows=5)
    po = po.numpy().astype(np.float64)
    pl = pl.numpy().astype(np.float64)
    out, lse = oracle.combine(po, pl)
    ref_lse = np.logaddexp.reduce(pl, axis=0)
    _assert_same_finite(lse, ref_lse)
    fin = np.isfinite(ref_lse)
    w = np.where(np.isfinite(pl), np.exp(pl - np.where(fin, ref_lse, 0.0)), 0.0)
    ref = np.einsum("sr,srd->rd", w, po)
    assert np.abs(out[fin] - ref[fin]).max() < 1e-12
    empty = ~fin
    assert empty.sum() >= 5
    assert np.all(out[empty] == 0.0) and not np.signbit(out[empty]).any()


def test_combine_closed_forms():
    rng = np.random.default_rng(0)
    po = rng.standard_normal((5, 4, 8))
    pl = np.full((5, 4), 1.25)
    out, lse = oracle.combine(po, pl)                  # equal weights -> mean
    assert np.abs(out - po.mean(axis=0)).max() < 1e-15
    assert np.abs(lse - (1.25 + np.log(5))).max() < 1e-15
    pl2 = np.full((5, 4), -np.inf)
    pl2[2] = [0.5, -3.0, 7.0, 0.0]                     # one split -> exact copy
    out, lse = oracle.combine(po, pl2)
    assert np.array_equal(out, po[2]) and np.array_equal(lse, pl2[2])


# ------------------------------------------------------------ invariances

def test_physical_permutation_invariance_bitwise():
    p = _small(seed=4, num_slots=3, extra_phys_pages=3)
    rng = np.random.default_rng(9)
    perm = rng.permutation(p.num_phys_pages)
    k2 = torch.empty_like(p.k_cache)
    v2 = torch.empty_like(p.v_cache)
    k2[perm] = p.k_cache
    v2[perm] = p.v_cache
    pt = p.page_table.numpy()
    pt2 = np.where(pt >= 0, perm[np.maximum(pt, 0)], -1).astype(np.int32)
    p2 = dataclasses.replace(p, k_cache=k2, v_cache=v2, page_table=torch.from_numpy(pt2))
    a, b = oracle.prefill_rows(p), oracle.prefill_rows(p2)
    for key in ("part_o", "part_lse", "out", "lse"):
        assert np.array_equal(a[key], b[key])


def test_slot_permutation_moves_slabs():
    p = _small(seed=5, num_slots=4)
    rng = np.random.default_rng(3)
    order = np.argsort(rng.random(p.sel_idx.shape), axis=-1)
    si = np.take_along_axis(p.sel_idx.numpy(), order, -1)
    sm = np.take_along_axis(p.sel_mask.numpy(), order, -1)
    p2 = dataclasses.replace(p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm))
    a, b = oracle.prefill_rows(p), oracle.prefill_rows(p2)
    G = p.Hq // p.Hkv
    for h in range(p.Hq):
        g = h // G
        # slab j of p2 holds slot order[t, g, j] of p
        idx = order[:, g, :]
        assert np.array_equal(b["part_lse"][:, h], np.take_along_axis(a["part_lse"][:, h], idx, 1))
        assert np.array_equal(b["part_o"][:, h],
                              np.take_along_axis(a["part_o"][:, h], idx[..., None], 1))
    _assert_same_finite(a["lse"], b["lse"])
    assert _rel(b["out"], a["out"]) < TOL


# ------------------------------------------------------------ closed forms

def test_zero_query_gives_uniform_mean():
    p = _small(seed=6, q_zero=True, num_slots=3, ctx_lens=[3], chunk_lens=[29])
    res = oracle.prefill_rows(p)
    q_pos, seq_len = p.q_pos.numpy(), int(p.seq_lens[0])
    pt = p.page_table.numpy()[0]
    v = p.v_cache.numpy().astype(np.float64)
    G = p.Hq // p.Hkv
    ps = p.page_size
    checked = 0
    for t in range(p.total_q):
        for g in range(p.Hkv):
            for j in range(p.num_slots):
                u = int(p.sel_idx[t, g, j])
                if p.sel_mask[t, g, j] == 0:
                    assert np.all(np.isneginf(res["part_lse"][t, g * G:(g + 1) * G, j]))
                    continue
                last = min(u * ps + ps - 1, int(q_pos[t]), seq_len - 1)
                toks = np.arange(u * ps, last + 1)
                assert len(toks) > 0
                mean = v[pt[toks // ps], toks % ps, g].mean(axis=0)
                for h in range(g * G, (g + 1) * G):
                    assert abs(res["part_lse"][t, h, j] - np.log(len(toks))) < 1e-13
                    assert np.abs(res["part_o"][t, h, j] - mean).max() < 1e-13
                    checked += 1
    assert checked > 100


def test_constant_values():
    p = _small(seed=7)
    p = dataclasses.replace(p, v_cache=torch.full_like(p.v_cache, 0.375))
    res = oracle.prefill_rows(p)
    fin = np.isfinite(res["part_lse"])
    assert np.abs(res["part_o"][fin] - 0.375).max() < 1e-14
    assert np.abs(res["out"] - 0.375).max() < 1e-14


def test_single_visible_key_exact():
    p = synth.build_page_problem(
        name="one", seed=8, ctx_lens=[0, 0], chunk_lens=[1, 1], page_size=8, Hq=2, Hkv=1, d=16,
        num_slots=2, q_dtype="f32", kv_dtype="f32", out_dtype="f32")
    res = oracle.prefill_rows(p)
    pt = p.page_table.numpy()
    q = p.q.numpy().astype(np.float64)
    k = p.k_cache.numpy().astype(np.float64)
    v = p.v_cache.numpy().astype(np.float64)
    for t in range(2):
        phys = pt[t, 0]
        for h in range(2):
            assert np.array_equal(res["out"][t, h], v[phys, 0, 0])
            logit = p.sm_scale * np.dot(q[t, h], k[phys, 0, 0])
            assert abs(res["lse"][t, h] - logit) < 1e-15


# ------------------------------------------------------------ empty rows, errors

def test_all_invalid_rows_bitwise_zero():
    p = _small(seed=9, pad_rows=3)
    sm = p.sel_mask.numpy().copy()
    sm[4] = 0
    sm[7, 1] = 0
    p = dataclasses.replace(p, sel_mask=torch.from_numpy(sm))
    res = oracle.prefill_rows(p)
    G = p.Hq // p.Hkv
    dead = [(4, h) for h in range(p.Hq)] + [(7, h) for h in range(G, 2 * G)]
    dead += [(t, h) for t in range(p.total_q - 3, p.total_q) for h in range(p.Hq)]
    for t, h in dead:
        o = res["out"][t, h]
        assert np.all(o == 0.0) and not np.signbit(o).any()
        assert np.isneginf(res["lse"][t, h]) and np.all(np.isneginf(res["part_lse"][t, h]))
    assert res["err"] == 0


def test_error_flags_and_duplicate_rule():
    p = _small(seed=10, num_slots=4)
    si, sm = p.sel_idx.numpy().copy(), p.sel_mask.numpy().copy()
    si[3, 0, 1], sm[3, 0, 1] = p.max_pages + 2, 1          # out of range unit
    assert oracle.prefill_rows(dataclasses.replace(
        p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm)))["err"] \
        == oracle.ERR_SEL_RANGE
    # duplicate of slot 0 in slot 2 of token 10: flagged, ignored
    si, sm = p.sel_idx.numpy().copy(), p.sel_mask.numpy().copy()
    si[10, 1, 2], sm[10, 1, 2] = si[10, 1, 0], 1
    dup = dataclasses.replace(p, sel_idx=torch.from_numpy(si), sel_mask=torch.from_numpy(sm))
    r_dup = oracle.prefill_rows(dup)
    assert r_dup["err"] == oracle.ERR_DUPLICATE
    sm2 = sm.copy()
    sm2[10, 1, 2] = 0
    r_clean = oracle.prefill_rows(dataclasses.replace(dup, sel_mask=torch.from_numpy(sm2)))
    assert r_clean["err"] == 0
    assert np.array_equal(r_dup["out"], r_clean["out"])
    # bad physical page in the table
    pt = p.page_table.numpy().copy()
    pt[1, 0] = p.num_phys_pages + 5
    r = oracle.prefill_rows(dataclasses.replace(p, page_table=torch.from_numpy(pt)))
    assert r["err"] == oracle.ERR_PHYS_RANGE
    # query row naming a missing request
    qs = p.q_seq.numpy().copy()
    qs[0] = 7
    r = oracle.prefill_rows(dataclasses.replace(p, q_seq=torch.from_numpy(qs)))
    assert r["err"] == oracle.ERR_QSEQ_RANGE
    assert np.all(np.isneginf(r["lse"][0])) and np.all(r["out"][0] == 0.0)


def test_slot_nonempty_matches_partials():
    p = _small(seed=12, num_slots=4, pad_rows=2)
    ne = oracle.slot_nonempty(p)
    res = oracle.prefill_rows(p)
    G = p.Hq // p.Hkv
    for h in range(p.Hq):
        assert np.array_equal(ne[:, h // G, :] == 1, np.isfinite(res["part_lse"][:, h, :]))


# ------------------------------------------------------------ brute force

def _tiny_cases():
    yield synth.make_config(0)
    yield _small(seed=21)
    yield _small(seed=22, page_size=4, Hq=3, Hkv=1, num_slots=5, shuffle_slots=True, pad_rows=2)
    yield _small(seed=23, Hq=8, Hkv=2, d=32, q_dtype="e4m3", kv_dtype="nvfp4", num_slots=4)
    yield _small(seed=24, q_dtype="bf16", kv_dtype="bf16", share_sel_across_heads=True)
    yield _small(seed=25, q_dtype="f16", kv_dtype="f16", ctx_lens=[30, 3], chunk_lens=[2, 40])
    yield synth.build_microblock_problem(
        name="mb", seed=26, ctx_len=64, chunk_len=21, pad_rows=3, Hq=3, Hkv=1, d=16,
        num_slots=12, page_size=16, spare_pages=2)
    mb = synth.build_microblock_problem(
        name="mb2", seed=27, ctx_len=40, chunk_len=17, pad_rows=1, Hq=2, Hkv=2, d=16,
        num_slots=8, page_size=8, spare_pages=1)
    yield dataclasses.replace(mb, slots_per_split=2)
    yield _small(seed=28, Hq=4, Hkv=2, d=32, q_dtype="e4m3", kv_dtype="e4m3", num_slots=4)
    yield _mb_split(29, 4)
    yield _mb_split(30, 1)


@pytest.mark.parametrize("case", list(range(11)))
def test_bruteforce_agrees(case):
    p = list(_tiny_cases())[case]
    a = oracle.prefill_rows(p)
    b = bruteforce.run(p)
    _assert_same_finite(a["part_lse"], b["part_lse"])
    fin = np.isfinite(b["part_lse"])
    assert np.abs(a["part_o"][fin] - b["part_o"][fin]).max() < 1e-12
    _assert_same_finite(a["lse"], b["lse"])
    assert np.abs(a["out"] - b["out"]).max() < 1e-12
    assert a["err"] == 0
