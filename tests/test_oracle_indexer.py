"""Pins of the oracle's paged prefill indexer (per-page max scores and their
top-k) against what the definition fixes: an independent dense numpy
computation with PyTorch's float8 decoding, a numpy sort for the top-k,
closed forms, causality and invariances.  CPU only."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from block_sparse_paged_table_amd import synth


def _dec(t):
    return t.to(torch.float64).numpy()


def _dense_scores(ip):
    """Scores by dense masked matmuls, one request at a time."""
    q, k = _dec(ip.q), _dec(ip.k_cache)
    pt, sl = ip.page_table.numpy(), ip.seq_lens.numpy()
    q_seq, q_pos = ip.q_seq.numpy(), ip.q_pos.numpy()
    T, H, P = ip.total_q, ip.H, ip.max_pages
    out = np.full((T, H, P), -np.inf)
    for b in range(ip.num_seqs):
        rows = np.nonzero((q_seq == b) & (q_pos >= 0))[0]
        L = int(sl[b])
        if len(rows) == 0 or L == 0:
            continue
        t = np.arange(L)
        keys = k[pt[b, t // ip.page_size], t % ip.page_size]          # [L, H, d]
        vis = t[None, :] <= q_pos[rows][:, None]                      # [n, L]
        for h in range(H):
            s = q[rows, h] @ keys[:, h].T                             # [n, L]
            s = np.where(vis, s, -np.inf)
            npages = (L + ip.page_size - 1) // ip.page_size
            pad = np.full((len(rows), npages * ip.page_size - L), -np.inf)
            s = np.concatenate([s, pad], axis=1).reshape(len(rows), npages, ip.page_size)
            out[rows, h, :npages] = s.max(-1) * ip.q_scale * ip.k_scale
    return out


def _small(seed, **kw):
    args = dict(name="idx", seed=seed, ctx_lens=[100, 0, 37], chunk_lens=[60, 300, 5],
                page_size=16, H=2, d=32, top_k=6, pad_rows=3, extra_phys_pages=4, page_bias=1.0)
    args.update(kw)
    return synth.build_index_problem(**args)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_scores_match_dense_numpy(seed):
    ip = _small(seed)
    sc, err = oracle.index_scores(ip)
    ref = _dense_scores(ip)
    assert err == 0
    assert np.array_equal(np.isneginf(sc), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.abs(sc[fin] - ref[fin]).max() <= 1e-12 * np.abs(ref[fin]).max()


def _numpy_topk(sc, k):
    rows = sc.reshape(-1, sc.shape[-1])
    idx = np.full((rows.shape[0], k), -1, np.int32)
    mask = np.zeros((rows.shape[0], k), np.uint8)
    for r, row in enumerate(rows):
        order = np.lexsort((np.arange(len(row)), -row))   # score desc, index asc
        order = [j for j in order if np.isfinite(row[j])][:k]
        idx[r, :len(order)] = order
        mask[r, :len(order)] = 1
    return idx.reshape(sc.shape[:-1] + (k,)), mask.reshape(sc.shape[:-1] + (k,))


def test_topk_matches_numpy_sort_with_ties():
    rng = np.random.default_rng(5)
    sc = rng.integers(-3, 4, size=(300, 37)).astype(np.float64)   # many exact ties
    sc[rng.random(sc.shape) < 0.3] = -np.inf
    sc[7] = -np.inf                                               # an empty row
    for k in (1, 5, 16, 40):
        a = oracle.topk(sc, k)
        b = _numpy_topk(sc, k)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), k


def test_zero_queries_pick_the_lowest_visible_pages():
    ip = _small(4)
    ip = dataclasses.replace(ip, q=torch.zeros_like(ip.q))
    sc, _ = oracle.index_scores(ip)
    fin = np.isfinite(sc)
    assert np.all(sc[fin] == 0.0)
    idx, mask = oracle.topk(sc, ip.top_k)
    own = np.where(ip.q_pos.numpy() >= 0, ip.q_pos.numpy() // ip.page_size, -1)
    for r in range(ip.total_q):
        n_vis = own[r] + 1
        want = np.arange(min(n_vis, ip.top_k))
        for h in range(ip.H):
            assert np.array_equal(idx[r, h, :len(want)], want)
            assert mask[r, h].sum() == len(want)


def test_onehot_scores_are_last_visible_offsets():
    """K[t, h, 0] = t mod page (exact in E4M3 for page 16), Q[., ., 0] = 1,
    scales 1: a page scores its last visible in-page offset."""
    ip = _small(6, page_size=16)
    P, ps, H, d = ip.k_cache.shape
    k = torch.zeros((P, ps, H, d))
    k[:, :, :, 0] = torch.arange(ps, dtype=torch.float32)[None, :, None]
    q = torch.zeros(ip.q.shape)
    q[:, :, 0] = 1.0
    ip = dataclasses.replace(ip, q=q.to(torch.float8_e4m3fn), k_cache=k.to(torch.float8_e4m3fn),
                             q_scale=1.0, k_scale=1.0)
    sc, _ = oracle.index_scores(ip)
    q_seq, q_pos, sl = ip.q_seq.numpy(), ip.q_pos.numpy(), ip.seq_lens.numpy()
    for r in range(ip.total_q):
        for j in range(ip.max_pages):
            if q_pos[r] < 0 or j * ps > min(q_pos[r], sl[q_seq[r]] - 1):
                assert np.all(np.isneginf(sc[r, :, j]))
            else:
                last = min(j * ps + ps - 1, q_pos[r], sl[q_seq[r]] - 1)
                assert np.all(sc[r, :, j] == last - j * ps)


def test_physical_permutation_invariance():
    ip = _small(7)
    perm = np.random.default_rng(1).permutation(ip.num_phys_pages)
    k2 = torch.empty_like(ip.k_cache)
    k2[perm] = ip.k_cache
    pt = ip.page_table.numpy()
    pt2 = np.where(pt >= 0, perm[np.maximum(pt, 0)], -1).astype(np.int32)
    a, _ = oracle.index_scores(ip)
    b, _ = oracle.index_scores(dataclasses.replace(ip, k_cache=k2, page_table=torch.from_numpy(pt2)))
    assert np.array_equal(a, b)


def test_error_rows_score_nothing():
    ip = _small(8)
    q_seq = ip.q_seq.numpy().copy()
    q_seq[3] = 99
    pt = ip.page_table.numpy().copy()
    pt[1, 2] = 10 ** 6
    sc, err = oracle.index_scores(dataclasses.replace(ip, q_seq=torch.from_numpy(q_seq),
                                                      page_table=torch.from_numpy(pt)))
    assert err == (oracle.ERR_QSEQ_RANGE | oracle.ERR_PHYS_RANGE)
    assert np.all(np.isneginf(sc[3]))
    rows_b1 = np.nonzero((q_seq == 1) & (ip.q_pos.numpy() >= 32))[0]
    assert len(rows_b1) and np.all(np.isneginf(sc[rows_b1, :, 2]))
