"""GPU parity of the paged prefill indexer (per-page max scores and top-k)
against the FP64 oracle, through the C ABI.

Scores: the -inf pattern is exact; finite scores agree within
|gpu - ref| <= 1e-4 * scale * ||q_row|| * max_t ||k_t||, a relative allowance
on the Cauchy-Schwarz bound of sum |q_d k_d|.  The products are exact, but the
FP8 MFMA does not sum a 32-product block as an exact FP32 sum would: errors
of up to 1.8e-5 of that bound were measured for d = 64 (above the 3.8e-6 an
FP32 sum of 64 terms can reach), so the allowance is 1e-4.  Selections: where
the oracle's k-th and (k+1)-th scores are further apart than twice that
bound the selected set must equal the oracle's; everywhere the selection
must be valid (distinct finite pages, as many as there are up to top_k, in
non-increasing GPU-score order, and no unselected page scoring more than a
selected one beyond the bound)."""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_paged_table_amd import synth
from block_sparse_paged_table_amd.runner import DeviceIndexProblem, DeviceProblem
import oracle
from parity import check_combined, check_partials, gpu_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _small(seed, **kw):
    args = dict(name="idx", seed=seed, ctx_lens=[100, 0, 2000], chunk_lens=[60, 300, 170],
                page_size=128, H=2, d=128, top_k=6, pad_rows=5, extra_phys_pages=3, page_bias=1.0)
    args.update(kw)
    return synth.build_index_problem(**args)


def _bounds(ip):
    q = ip.q.to(torch.float64).numpy()
    k = ip.k_cache.to(torch.float64).numpy()
    kmax = np.linalg.norm(k, axis=-1).max()
    return 1e-4 * ip.q_scale * ip.k_scale * np.linalg.norm(q, axis=-1) * kmax   # [T, H]


def _check(ip, dev, tokens=None):
    sub = ip if tokens is None else dataclasses.replace(
        ip, q=ip.q[tokens], q_seq=ip.q_seq[tokens], q_pos=ip.q_pos[tokens])
    toks = np.arange(ip.total_q) if tokens is None else np.asarray(tokens)
    ref, err = oracle.index_scores(sub)
    tol = _bounds(sub)
    H, P, K = ip.H, ip.max_pages, dev.top_k
    g = dev.scores.cpu().numpy()[:, :P].reshape(ip.total_q, H, P)[toks]
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), "finite pattern differs"
    fin = np.isfinite(ref)
    d = np.abs(np.where(fin, np.where(fin, g, 0.0) - np.where(fin, ref, 0.0), 0.0))
    print(f"max score error / bound: {(d / tol[:, :, None]).max():.3g}")
    assert np.all(d <= tol[:, :, None]), f"score error {d.max()} > bound"
    idx = dev.sel_idx.cpu().numpy()[toks]
    mask = dev.sel_mask.cpu().numpy()[toks]
    ridx, rmask = oracle.topk(ref, K)
    exact = 0
    for r in range(len(toks)):
        for h in range(H):
            row, gr, t = ref[r, h], g[r, h], tol[r, h]
            nfin = int(np.isfinite(row).sum())
            nsel = min(K, nfin)
            assert np.array_equal(mask[r, h], (np.arange(K) < nsel).astype(np.uint8))
            sel = idx[r, h, :nsel]
            assert np.all(idx[r, h, nsel:] == -1)
            assert len(set(sel.tolist())) == nsel and np.all(np.isfinite(row[sel]))
            assert np.all(np.diff(gr[sel]) <= 0), "not in descending GPU-score order"
            rest = np.setdiff1d(np.nonzero(np.isfinite(row))[0], sel)
            if nsel and len(rest):
                assert row[rest].max() <= row[sel].min() + 2 * t
            srt = np.sort(row[np.isfinite(row)])[::-1]
            if nfin <= K or srt[K - 1] - srt[K] > 2 * t:
                assert set(sel.tolist()) == set(ridx[r, h, :nsel].tolist())
                exact += 1
    return err, exact


@pytest.mark.parametrize("H,d", [(2, 128), (1, 128), (2, 64), (4, 64)])
def test_index_small_all_rows(H, d):
    ip = _small(41, H=H, d=d)
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    err, exact = _check(ip, dev)
    assert err == 0 and dev.err_flags() == 0
    assert exact > 0


def test_index_scores_only_then_topk_and_wide_pitch():
    ip = _small(42, top_k=9)
    dev = DeviceIndexProblem(ip, score_pad=37)
    dev.scores.fill_(123.0)
    dev.scores_only()
    torch.cuda.synchronize()
    assert torch.all(dev.scores[:, ip.max_pages:] == 123.0)   # pitch padding untouched
    dev.topk()
    torch.cuda.synchronize()
    _check(ip, dev)


def test_index_tiny_chunks_many_requests_and_long_context():
    # tiles span several requests; one request has 40 pages of context
    ip = _small(43, ctx_lens=[0, 5000, 7, 300, 0], chunk_lens=[3, 20, 70, 1, 130], top_k=16)
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    _check(ip, dev)


@pytest.mark.parametrize("top_k", [1, 64])
def test_index_topk16_limits(top_k):
    """The 16-lanes-per-row top-k at its limits: rows of exactly 128 pages,
    one slot and 64 slots (four result registers per lane), on sampled
    tokens of one long request."""
    ip = _small(47, ctx_lens=[16000], chunk_lens=[384], top_k=top_k, H=2)
    assert ip.max_pages == 128
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    err, exact = _check(ip, dev, tokens=[0, 5, 200, 383, 384])
    assert err == 0 and exact > 0


@pytest.mark.parametrize("ctx,chunk,top_k", [
    (9000, 200, 100),   # <= 128 pages, top_k > 64: one wave per row, 2 pages per lane
    (40000, 200, 20),   # 129 .. 512 pages: one wave per row, 8 pages per lane
    (70000, 130, 255),  # > 512 pages and the largest top_k: 32 pages per lane
])
def test_index_topk_wide_rows(ctx, chunk, top_k):
    """The top-k variants for long rows or many slots (rows of at most 128
    pages with top_k <= 64 take 16 lanes per row, covered above), checked on
    sampled tokens of one long request."""
    ip = _small(46, ctx_lens=[ctx], chunk_lens=[chunk], top_k=top_k, H=1)
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    err, exact = _check(ip, dev, tokens=[0, 1, chunk // 2, chunk - 1, chunk])
    assert err == 0 and exact > 0


def test_index_max_pages():
    """A request of exactly the 2048 pages a top-k row can hold (64 lanes x 32
    pages) with the largest top_k, on sampled tokens: the last register slot of
    the last lane holds a live page."""
    ctx, chunk = 2048 * 128 - 130, 130
    ip = _small(48, ctx_lens=[ctx], chunk_lens=[chunk], top_k=255, H=1, pad_rows=2)
    assert ip.max_pages == 2048
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    err, exact = _check(ip, dev, tokens=[0, 77, chunk - 1, chunk])
    assert err == 0 and exact > 0


def test_index_deterministic():
    ip = _small(44)
    dev = DeviceIndexProblem(ip)
    outs = []
    for _ in range(3):
        dev.run()
        torch.cuda.synchronize()
        outs.append((dev.scores.clone(), dev.sel_idx.clone(), dev.sel_mask.clone()))
    for o in outs[1:]:
        assert all(torch.equal(x, y) for x, y in zip(outs[0], o))


def test_index_graph_capture_replays_match_eager():
    """Page scores + top-k captured in one HIP graph (kernels only: the error
    word is cleared by a kernel); every replay, with eager work and clobbered
    outputs in between, reproduces the eager scores and selections."""
    ip = _small(46)
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    ref = (dev.scores.clone(), dev.sel_idx.clone(), dev.sel_mask.clone())
    err = dev.err_flags()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dev.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dev.run()
    torch.cuda.synchronize()
    for i in range(3):
        dev.scores.fill_(float(i + 1))
        dev.sel_idx.fill_(-7)
        dev.sel_mask.fill_(3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(ref, (dev.scores, dev.sel_idx, dev.sel_mask))), i
        assert dev.err_flags() == err
        dev.run()  # eager work between replays
        torch.cuda.synchronize()


def test_index_empty_batch():
    """total_q = 0: the indexer accepts NULL query, score and selection buffers
    and only clears the error word."""
    ip = _small(71)
    empty = dataclasses.replace(ip, q=ip.q[:0], q_seq=ip.q_seq[:0], q_pos=ip.q_pos[:0])
    dev = DeviceIndexProblem(empty)
    assert dev.scores.numel() == 0 and dev.sel_idx.numel() == 0
    dev.err.fill_(7)
    dev.run()
    torch.cuda.synchronize()
    assert dev.err_flags() == 0


def test_index_error_rows():
    ip = _small(45)
    q_seq = ip.q_seq.numpy().copy()
    q_seq[4] = 77
    pt = ip.page_table.numpy().copy()
    pt[2, 3] = 10 ** 6
    bad = dataclasses.replace(ip, q_seq=torch.from_numpy(q_seq), page_table=torch.from_numpy(pt))
    dev = DeviceIndexProblem(bad)
    dev.run()
    torch.cuda.synchronize()
    err, _ = _check(bad, dev)
    assert dev.err_flags() == err == (oracle.ERR_QSEQ_RANGE | oracle.ERR_PHYS_RANGE)
    assert torch.all(dev.sel_mask[4] == 0)


def test_index_full_size_sampled():
    ip = synth.make_index_problem()
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([np.arange(0, 300), np.linspace(0, ip.total_q - 1, 200).astype(int),
                                     np.arange(ip.total_q - 64, ip.total_q)]))
    _, exact = _check(ip, dev, toks)
    assert exact > len(toks)   # most rows are uniquely determined


def _page_chunk(ip):
    """The page chunk the library picks: 16 pages per workgroup, halved (to 4
    at least) while the grid of (64-token tile, head, chunk) workgroups holds
    fewer than 2048."""
    tiles = -(-ip.total_q // 64)
    for pc in (16, 8, 4):
        if tiles * ip.H * -(-ip.max_pages // pc) >= 2048:
            return pc
    return 4


@pytest.mark.parametrize("geo,pc", [
    (dict(ctx_lens=[8192], chunk_lens=[8192]), 16),
    (dict(ctx_lens=[12288], chunk_lens=[4096]), 8),
    (dict(ctx_lens=[30000, 60000, 0], chunk_lens=[64, 100, 30]), 4),
])
def test_index_page_chunk_forms(geo, pc):
    """Each page-chunk form of the scores kernel, on a workload that selects
    it; sampled rows (the first and last tiles and a spread between)."""
    ip = _small(47, H=2, d=128, top_k=16, pad_rows=3, **geo)
    assert _page_chunk(ip) == pc
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([np.arange(0, min(80, ip.total_q)),
                                     np.linspace(0, ip.total_q - 1, 120).astype(int),
                                     np.arange(max(0, ip.total_q - 80), ip.total_q)]))
    _check(ip, dev, toks)


def test_indexer_selections_drive_the_attention():
    """End to end: the GPU indexer's selections are the attention's sel_idx /
    sel_mask (one indexer head per KV head); the attention on them matches
    the oracle on the same selections."""
    geo = dict(seed=46, ctx_lens=[200, 0], chunk_lens=[300, 250], page_size=128, pad_rows=3)
    ip = synth.build_index_problem(name="e2e", H=2, d=128, top_k=5, page_bias=1.0, **geo)
    p = synth.build_page_problem(name="e2e", Hq=8, Hkv=2, d=128, num_slots=5, q_dtype="e4m3",
                                 kv_dtype="e4m3", out_dtype="f32", **geo)
    assert np.array_equal(ip.page_table.numpy(), p.page_table.numpy())
    dev = DeviceIndexProblem(ip)
    dev.run()
    torch.cuda.synchronize()
    p = dataclasses.replace(p, sel_idx=dev.sel_idx.cpu(), sel_mask=dev.sel_mask.cpu())
    dp = DeviceProblem(p)
    dp.run()
    torch.cuda.synchronize()
    ref = oracle.prefill_rows(p)
    po, pl, out, lse = gpu_rows(dp, np.arange(p.total_q))
    check_partials(p, po, pl, ref)
    check_combined(p, out, lse, ref, "f32")
    assert dp.err_flags() == 0
