"""Full-size parity on EVERY row: the four full workloads (BF16 4 x 4096,
Q8KV4 16K-token layer, grouped Page4 8192-row chunk, chunked Q8KV4 batch)
in the launch configuration the benchmark times (row-major partials),
against the FP64 oracle row by row, in token blocks.

Checked over all rows at once (tolerances from tests/parity.py): the exact
empty-split pattern, partial relative L2 and max abs error, partial and
final LSE error, the combined output (16-bit outputs against the rounding
floor of the exact result), +0 outputs and lse = -inf for rows that see
nothing, and the error word.  The measured figures are printed.
"""
import numpy as np
import pytest
import torch

from block_sparse_paged_table_amd import synth
from block_sparse_paged_table_amd.runner import DeviceProblem
import oracle
from parity import gpu_rows, tol_for

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


class _Acc:
    """Sums of squares and maxima over token blocks."""

    def __init__(self):
        self.v = dict(p_err=0.0, p_ref=0.0, p_max=0.0, p_lse=0.0, o_err=0.0, o_ref=0.0,
                      o_floor=0.0, o_max=0.0, o_lse=0.0, rows=0, live=0)

    def add(self, key, x, mode="sum"):
        if mode == "sum":
            self.v[key] += float(x)
        else:
            self.v[key] = max(self.v[key], float(x))


def _round(x, dt):
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdt).double().numpy()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_every_row(cfg):
    p = synth.make_config(cfg)
    tol = tol_for(p)
    dp = DeviceProblem(p, partial_layout="row")
    dp.run()
    torch.cuda.synchronize()
    keep = oracle.make_keep(p)
    acc = _Acc()
    block = max(64, 8192 * 16 // (p.Hq * p.num_splits))
    print(f"\n{p.name}: {p.total_q} tokens x {p.Hq} heads x {p.num_splits} splits, "
          f"blocks of {block} tokens", flush=True)
    for t0 in range(0, p.total_q, block):
        toks = np.arange(t0, min(p.total_q, t0 + block))
        ref = oracle.prefill_rows(p, toks, keep=keep, want_single_pass=False)
        po, pl, out, lse = gpu_rows(dp, toks)
        rpl, rpo = ref["part_lse"], ref["part_o"]
        # empty splits: exactly the oracle's
        assert np.array_equal(np.isneginf(pl), np.isneginf(rpl)), (p.name, t0)
        assert not np.isnan(pl).any() and not np.isnan(out).any()
        fin = np.isfinite(rpl)
        if fin.any():
            a, b = po[fin], rpo[fin]
            acc.add("p_err", ((a - b) ** 2).sum())
            acc.add("p_ref", (b ** 2).sum())
            acc.add("p_max", np.abs(a - b).max(), "max")
            acc.add("p_lse", np.abs(pl[fin] - rpl[fin]).max(), "max")
            acc.add("live", fin.sum())
        # combined rows
        rl, ro = ref["lse"], ref["out"]
        empty = np.isneginf(rl)
        assert np.array_equal(np.isneginf(lse), empty), (p.name, t0)
        if empty.any():
            e = out[empty]
            assert np.all(e == 0.0) and not np.signbit(e).any(), (p.name, t0)
        if (~empty).any():
            acc.add("o_lse", np.abs(lse[~empty] - rl[~empty]).max(), "max")
        acc.add("o_err", ((out - ro) ** 2).sum())
        acc.add("o_ref", (ro ** 2).sum())
        acc.add("o_max", np.abs(out - ro).max(), "max")
        if dp.out_dtype != "f32":
            acc.add("o_floor", ((_round(ro, dp.out_dtype) - ro) ** 2).sum())
        acc.add("rows", out.shape[0] * out.shape[1])
        assert ref["err"] == 0
    assert dp.err_flags() == 0
    v = acc.v
    p_rel = (v["p_err"] / v["p_ref"]) ** 0.5
    o_rel = (v["o_err"] / v["o_ref"]) ** 0.5
    print(f"{p.name}: {v['rows']} rows, {v['live']} live partials: partial rel L2 {p_rel:.3e}, "
          f"max abs {v['p_max']:.3e}, max |d lse| {v['p_lse']:.3e}; output rel L2 {o_rel:.3e} "
          f"(storage floor {(v['o_floor'] / v['o_ref']) ** 0.5:.3e}), max abs {v['o_max']:.3e}, "
          f"max |d lse| {v['o_lse']:.3e}", flush=True)
    assert v["rows"] == p.total_q * p.Hq
    assert p_rel <= tol["rel_l2"] and v["p_max"] <= tol["max_abs"], v
    assert v["p_lse"] <= tol["lse"] and v["o_lse"] <= tol["lse"], v
    if dp.out_dtype == "f32":
        assert o_rel <= tol["rel_l2"] and v["o_max"] <= tol["max_abs"], v
    else:
        assert v["o_err"] ** 0.5 <= v["o_floor"] ** 0.5 + tol["rel_l2"] * v["o_ref"] ** 0.5, v


@pytest.mark.parametrize("cfg", [2, 3, 4, "page4_small_chunk"])
def test_full_size_graph_replay_matches_eager(cfg):
    """The step as the benchmark times it: plan, attention and combine
    captured in one HIP graph and replayed.  Every replay rewrites the live
    partials, the partial LSEs, the outputs and their LSEs bit for bit as the
    eager launches wrote them (whose oracle parity the test above checks);
    between replays the buffers are overwritten by eager work.  The split-k
    small chunk runs its splits in runs merged by an extra combine."""
    p = synth.make_page4_small_chunk() if cfg == "page4_small_chunk" else synth.make_config(cfg)
    dp = DeviceProblem(p, partial_layout="row")
    dp.plan()
    dp.attend()
    dp.combine()
    torch.cuda.synchronize()
    live = torch.isfinite(dp.partial_lse)
    ref = [dp.partial_o.clone(), dp.partial_lse.clone(), dp.out.clone(), dp.lse.clone()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dp.plan()
        dp.attend()
        dp.combine()
    torch.cuda.synchronize()
    for i in range(3):
        for t in (dp.partial_o, dp.partial_lse, dp.out, dp.lse):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.partial_lse, ref[1]), i
        assert torch.equal(dp.partial_o[live], ref[0][live]), i  # partial_o viewed [split][row][d]
        assert torch.equal(dp.out, ref[2]) and torch.equal(dp.lse, ref[3]), i
    print(f"\n{p.name}: 3 graph replays bitwise equal to the eager step", flush=True)
