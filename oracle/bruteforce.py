"""Second, independent oracle for tiny inputs: dense masks in numpy.

TEST INFRASTRUCTURE ONLY.  Written in a different style from ``oracle.c`` so
that a mistake in one is unlikely to be repeated in the other: it builds each
request's logical key/value sequence by indexing the page table with numpy,
forms a dense boolean visibility matrix [tokens x keys] per split from the
selections, and runs a masked softmax with numpy primitives.  Format decoding
uses PyTorch's float8_e4m3fn cast (a library routine) and the E2M1 magnitude
list; products of an E2M1 code and an E4M3 scale are rounded to E4M3 with the
same library cast, which is valid while the product stays within +-448 (the
case for every input the generator produces).

It follows the same definition as the C oracle: MiniMax-AI/MSA PR 21,
sections "K1" and "Combine" (per-page partial output + lse, merged per row)
and 1Cat-vLLM PR 387, section "Purpose" (exact per-row microblock masks).
"""
from __future__ import annotations

import numpy as np
import torch

_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _f8_to_f64(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _nvfp4_values(codes_packed: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """[..., d/2] packed codes + [..., d/16] scales -> float64 [..., d] values."""
    lo = codes_packed & 15
    hi = codes_packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*codes_packed.shape[:-1], -1)
    mag = _E2M1[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    scale = np.repeat(_f8_to_f64(sf), 16, axis=-1)
    prod = torch.from_numpy(val * scale).to(torch.float32)
    return prod.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _np(t):
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.float8_e4m3fn:
            return _f8_to_f64(t.view(torch.uint8).numpy())
        return t.to(torch.float64).numpy() if t.is_floating_point() else t.numpy()
    return np.asarray(t)


def values(problem):
    """Decoded (q [T,Hq,d], k [P,page,Hkv,d], v [P,page,Hkv,d]) in float64."""
    p = problem
    q = _np(p.q)
    if p.kv_dtype == "nvfp4":
        k = _nvfp4_values(p.k_cache.numpy(), p.k_sf.numpy())
        v = _nvfp4_values(p.v_cache.numpy(), p.v_sf.numpy())
    else:
        k, v = _np(p.k_cache), _np(p.v_cache)
    return q, k, v


def run(problem):
    """Returns dict(part_o [T,Hq,S,dv], part_lse [T,Hq,S], out [T,Hq,dv], lse [T,Hq])."""
    p = problem
    q, k, v = values(p)
    T, Hq, dv = q.shape[0], p.Hq, p.d_v
    G = p.Hq // p.Hkv
    S = p.num_slots // p.slots_per_split
    ut, ps = p.unit_tokens, p.page_size
    q_seq, q_pos = p.q_seq.numpy(), p.q_pos.numpy()
    seq_lens, pt = p.seq_lens.numpy(), p.page_table.numpy()
    sel_idx, sel_mask = p.sel_idx.numpy(), p.sel_mask.numpy()
    scale = p.sm_scale * p.q_scale * p.k_scale

    part_o = np.zeros((T, Hq, S, dv))
    part_lse = np.full((T, Hq, S), -np.inf)
    for b in range(p.num_seqs):
        L = int(seq_lens[b])
        rows = np.nonzero((q_seq == b) & (q_pos >= 0))[0]
        if L == 0 or len(rows) == 0:
            continue
        tpos = np.arange(L)
        phys = pt[b, tpos // ps]
        klog = k[phys, tpos % ps]          # [L, Hkv, d]
        vlog = v[phys, tpos % ps] * p.v_scale
        for g in range(p.Hkv):
            # vis[split, row, key]
            vis = np.zeros((S, len(rows), L), dtype=bool)
            for ri, r in enumerate(rows):
                seen = set()
                for j in range(p.num_slots):
                    if sel_mask[r, g, j] == 0:
                        continue
                    u = int(sel_idx[r, g, j])
                    if u in seen:
                        continue
                    seen.add(u)
                    keys = u * ut + np.arange(ut)
                    ok = (keys <= q_pos[r]) & (keys < L)
                    if ut != ps:
                        ok &= ((int(sel_mask[r, g, j]) >> np.arange(ut)) & 1).astype(bool)
                    vis[j // p.slots_per_split, ri, keys[ok]] = True
            for hl in range(G):
                h = g * G + hl
                s = scale * q[rows, h] @ klog[:, g].T          # [rows, L]
                for sp in range(S):
                    m = vis[sp]
                    has = m.any(axis=1)
                    ss = np.where(m, s, -np.inf)
                    mx = np.where(has, ss.max(axis=1), 0.0)
                    e = np.where(m, np.exp(ss - mx[:, None]), 0.0)
                    den = e.sum(axis=1)
                    o = (e @ vlog[:, g]) / np.where(has, den, 1.0)[:, None]
                    part_o[rows, h, sp] = np.where(has[:, None], o, 0.0)
                    part_lse[rows, h, sp] = np.where(has, mx + np.log(np.where(has, den, 1.0)),
                                                     -np.inf)
    # combine with numpy's logaddexp reduction
    lse = np.logaddexp.reduce(part_lse, axis=2)
    w = np.exp(part_lse - np.where(np.isfinite(lse), lse, 0.0)[..., None])
    w = np.where(np.isfinite(part_lse), w, 0.0)
    out = np.einsum("tks,tksd->tkd", w, part_o)
    out = np.where(np.isfinite(lse)[..., None], out, 0.0)
    return dict(part_o=part_o, part_lse=part_lse, out=out, lse=lse)
