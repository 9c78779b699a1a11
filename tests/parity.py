"""Shared parity checks for the GPU tests: GPU outputs (through the C ABI)
against the FP64 oracle on the same seeded inputs.

Tolerances (written here, used by every GPU test):
  * FP32 storage (Q, K, V in FP32): the kernels use FP32 MFMA products and
    FP32 accumulation over <= 128 terms; relative L2 <= 1e-5 and max abs
    <= 1e-5 on outputs, |d lse| <= 1e-5.
  * BF16 / FP16 storage: relative L2 <= 1e-3 and max abs <= 2e-3 on FP32
    partials and on the FP32 combine; |d lse| <= 1e-4 (logits are exact
    products accumulated in FP32, |logit| < 20).
  * E4M3 Q / NVFP4 or E4M3 KV: the oracle consumes the identical E4M3
    operands; relative L2 <= 5e-3 and max abs <= 2e-3 on partials and
    combine (the max-abs bound of the 16-bit inputs, applied to the FP8
    path too; every row of the full 16K-token and chunked-batch layers
    measures below 6e-4); |d lse| <= 1e-4.
  * 16-bit outputs of the combine are compared bit for bit with the
    round-to-nearest-even conversion of the GPU's own FP32 combine; end to
    end, ||gpu - ref|| <= ||round(ref) - ref|| + tol * ||ref||.
  * 16-bit partials (BF16 / FP16 storage of partial_o) get the same rule:
    the storage rounding of the exact partial is a floor no kernel can beat,
    so ||gpu - ref|| <= ||round(ref) - ref|| + tol * ||ref|| and
    max|gpu - ref| <= max|round(ref) - ref| + max_abs; the combine of such
    partials is checked against the oracle's combine of the GPU's own
    (widened) partials at FP32-combine accuracy.
Empty splits must hold lse = -inf exactly (their partial rows are
unspecified); rows with no visible key must give +0 outputs and lse = -inf.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {
    "f32": dict(rel_l2=1e-5, max_abs=1e-5, lse=1e-5),
    "bf16": dict(rel_l2=1e-3, max_abs=2e-3, lse=1e-4),
    "f16": dict(rel_l2=1e-3, max_abs=2e-3, lse=1e-4),
    "e4m3": dict(rel_l2=5e-3, max_abs=2e-3, lse=1e-4),
}


def tol_for(p):
    return TOL[p.q_dtype]


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


def gpu_rows(dp, tokens):
    """GPU partials / outputs of the given tokens, reshaped like the oracle's."""
    p = dp.p
    tok = torch.as_tensor(np.asarray(tokens), device=dp.device, dtype=torch.long)
    rows = (tok[:, None] * p.Hq + torch.arange(p.Hq, device=dp.device)[None, :]).reshape(-1)
    po = dp.partial_o[:, rows, :p.d_v].float().cpu().numpy()            # [S, n*Hq, dv]
    pl = dp.partial_lse[:, rows].float().cpu().numpy()                  # [S, n*Hq]
    n = len(tokens)
    po = po.reshape(p.num_splits, n, p.Hq, p.d_v).transpose(1, 2, 0, 3)  # [n, Hq, S, dv]
    pl = pl.reshape(p.num_splits, n, p.Hq).transpose(1, 2, 0)
    out = dp.out[rows].float().cpu().numpy().reshape(n, p.Hq, p.d_v)
    lse = dp.lse[rows].cpu().numpy().reshape(n, p.Hq)
    return po, pl, out, lse


def _round16(x, stored):
    tdt = torch.bfloat16 if stored == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdt).double().numpy()


def check_partials(p, po, pl, ref, tol=None, stored="f32"):
    tol = tol or tol_for(p)
    rpl = ref["part_lse"]
    assert np.array_equal(np.isneginf(pl), np.isneginf(rpl)), "empty-split pattern differs"
    assert not np.isnan(pl).any()
    fin = np.isfinite(rpl)
    if not fin.any():
        return {}
    dl = np.abs(pl[fin] - rpl[fin]).max()
    a, b = po[fin], ref["part_o"][fin]
    r = rel_l2(a, b)
    m = np.abs(a - b).max()
    assert dl <= tol["lse"], f"partial lse err {dl}"
    if stored == "f32":
        assert r <= tol["rel_l2"], f"partial rel L2 {r}"
        assert m <= tol["max_abs"], f"partial max abs {m}"
    else:
        rb = _round16(b, stored)
        floor_l2 = np.linalg.norm(rb - b) / max(np.linalg.norm(b), 1e-300)
        floor_max = np.abs(rb - b).max()
        assert r <= floor_l2 + tol["rel_l2"], f"partial rel L2 {r} (floor {floor_l2})"
        assert m <= floor_max + tol["max_abs"], f"partial max abs {m} (floor {floor_max})"
    return dict(lse=dl, rel_l2=r, max_abs=m)


def check_combined(p, out, lse, ref, out_dtype, tol=None):
    tol = tol or tol_for(p)
    rl = ref["lse"]
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl)), "empty-row pattern differs"
    empty = np.isneginf(rl)
    if empty.any():
        e = out[empty]
        assert np.all(e == 0.0) and not np.signbit(e).any(), "empty rows must be +0"
    fin = ~empty
    res = {}
    if fin.any():
        res["lse"] = np.abs(lse[fin] - rl[fin]).max()
        assert res["lse"] <= tol["lse"], f"lse err {res['lse']}"
    ro = ref["out"]
    if out_dtype == "f32":
        res["rel_l2"] = rel_l2(out, ro)
        res["max_abs"] = np.abs(out - ro).max()
        assert res["rel_l2"] <= tol["rel_l2"], res
        assert res["max_abs"] <= tol["max_abs"], res
    else:
        tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float16
        rounded = torch.from_numpy(ro).to(tdt).double().numpy()
        floor = np.linalg.norm(rounded - ro)
        err = np.linalg.norm(out - ro)
        res["rel_l2"] = err / max(np.linalg.norm(ro), 1e-300)
        assert err <= floor + tol["rel_l2"] * np.linalg.norm(ro), res
    return res
