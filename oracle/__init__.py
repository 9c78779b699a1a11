"""FP64 CPU oracle for block-sparse paged prefill attention (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never loads it, and it never loads the
GPU library.  The arithmetic lives in ``oracle.c`` (plain C, FP64, OpenMP
over rows); this module only builds it, marshals numpy arrays and exposes:

  * format routines: ``e4m3_decode``, ``e4m3_encode``, ``e2m1_decode``,
    ``nvfp4_dequant`` (E2M1 code x E4M3 scale, rounded once to E4M3);
  * ``prefill_rows(problem, tokens)``: partial outputs / lse per split, their
    LSE combine, and an independent single-pass softmax;
  * ``combine(po, pl)``: the LSE combine on given partials;
  * ``slot_nonempty(problem)``: which slots contribute at least one key;
  * ``index_scores(problem)`` / ``topk(scores, k)``: the paged prefill
    indexer's per-page scores and their top-k selection.

``bruteforce.py`` holds a second, independent numpy implementation for tiny
inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FMT_F64, FMT_E4M3, FMT_NVFP4 = 0, 1, 2
ERR_SEL_RANGE, ERR_PHYS_RANGE, ERR_QSEQ_RANGE, ERR_DUPLICATE = 1, 2, 4, 8


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int), ("total_q", ctypes.c_int), ("Hq", ctypes.c_int),
        ("Hkv", ctypes.c_int), ("d_qk", ctypes.c_int), ("d_v", ctypes.c_int),
        ("page_size", ctypes.c_int), ("unit_tokens", ctypes.c_int),
        ("num_slots", ctypes.c_int), ("slots_per_split", ctypes.c_int),
        ("max_pages", ctypes.c_int), ("pt_stride", ctypes.c_int),
        ("num_phys_pages", ctypes.c_int),
        ("sm_scale", ctypes.c_double), ("q_scale", ctypes.c_double),
        ("k_scale", ctypes.c_double), ("v_scale", ctypes.c_double),
        ("q_seq", ctypes.c_void_p), ("q_pos", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
        ("q_fmt", ctypes.c_int), ("q", ctypes.c_void_p),
        ("kv_fmt", ctypes.c_int), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_sf", ctypes.c_void_p), ("v_sf", ctypes.c_void_p),
        ("sel_idx", ctypes.c_void_p), ("sel_mask", ctypes.c_void_p),
    ]


class _IndexProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int), ("total_q", ctypes.c_int), ("H", ctypes.c_int),
        ("d", ctypes.c_int), ("page_size", ctypes.c_int), ("max_pages", ctypes.c_int),
        ("pt_stride", ctypes.c_int), ("num_phys_pages", ctypes.c_int),
        ("q_scale", ctypes.c_double), ("k_scale", ctypes.c_double),
        ("q_seq", ctypes.c_void_p), ("q_pos", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
    ]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            L.orc_e4m3_decode_n.argtypes = [P, P, ctypes.c_int64]
            L.orc_e4m3_encode_n.argtypes = [P, P, ctypes.c_int64]
            L.orc_e2m1_decode_n.argtypes = [P, P, ctypes.c_int64]
            L.orc_nvfp4_dequant_n.argtypes = [P, P, P, ctypes.c_int64]
            L.orc_combine.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, P, P, P, P]
            L.orc_prefill_rows.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, P, P, P, P, P, P, P]
            L.orc_prefill_rows.restype = ctypes.c_uint32
            L.orc_slot_nonempty.argtypes = [ctypes.POINTER(_Problem), P]
            L.orc_index_scores.argtypes = [ctypes.POINTER(_IndexProblem), P]
            L.orc_index_scores.restype = ctypes.c_uint32
            L.orc_topk_rows.argtypes = [ctypes.c_int64, ctypes.c_int, P, ctypes.c_int, P, P]
            L.orc_abi_version.restype = ctypes.c_int
            _lib = L
        return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ------------------------------------------------------------------ formats

def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_decode_n(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_encode(x) -> np.ndarray:
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_n(_ptr(v), _ptr(out), v.size)
    return out


def e2m1_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e2m1_decode_n(_ptr(c), _ptr(out), c.size)
    return out


def nvfp4_dequant(codes, scales) -> np.ndarray:
    c, s = np.broadcast_arrays(np.asarray(codes, np.uint8), np.asarray(scales, np.uint8))
    c = np.ascontiguousarray(c)
    s = np.ascontiguousarray(s)
    out = np.empty(c.shape, np.uint8)
    lib().orc_nvfp4_dequant_n(_ptr(c), _ptr(s), _ptr(out), c.size)
    return out


# ------------------------------------------------------------------ combine

def combine(po, pl):
    """LSE combine: po [S, rows, d_v], pl [S, rows] -> (out [rows, d_v], lse [rows])."""
    po = np.ascontiguousarray(np.asarray(po, dtype=np.float64))
    pl = np.ascontiguousarray(np.asarray(pl, dtype=np.float64))
    S, rows, dv = po.shape
    assert pl.shape == (S, rows)
    out = np.empty((rows, dv), np.float64)
    lse = np.empty(rows, np.float64)
    lib().orc_combine(S, rows, dv, _ptr(po), _ptr(pl), _ptr(out), _ptr(lse))
    return out, lse


# ---------------------------------------------------------------- attention

def _as_np(t):
    import torch
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        if t.dtype in (torch.bfloat16, torch.float16):
            return t.to(torch.float64).numpy()
        return t.numpy()
    return np.asarray(t)


class _Keep:
    """Holds the numpy buffers a _Problem points into."""

    def __init__(self, problem):
        p = problem
        self.q_seq = np.ascontiguousarray(_as_np(p.q_seq), np.int32)
        self.q_pos = np.ascontiguousarray(_as_np(p.q_pos), np.int32)
        self.seq_lens = np.ascontiguousarray(_as_np(p.seq_lens), np.int32)
        self.page_table = np.ascontiguousarray(_as_np(p.page_table), np.int32)
        self.sel_idx = np.ascontiguousarray(_as_np(p.sel_idx), np.int32)
        self.sel_mask = np.ascontiguousarray(_as_np(p.sel_mask), np.uint8)
        if p.q_dtype == "e4m3":
            self.q = np.ascontiguousarray(_as_np(p.q), np.uint8)
            q_fmt = FMT_E4M3
        else:
            self.q = np.ascontiguousarray(_as_np(p.q), np.float64)
            q_fmt = FMT_F64
        self.k_sf = self.v_sf = None
        if p.kv_dtype == "nvfp4":
            self.k = np.ascontiguousarray(_as_np(p.k_cache), np.uint8)
            self.v = np.ascontiguousarray(_as_np(p.v_cache), np.uint8)
            self.k_sf = np.ascontiguousarray(_as_np(p.k_sf), np.uint8)
            self.v_sf = np.ascontiguousarray(_as_np(p.v_sf), np.uint8)
            kv_fmt = FMT_NVFP4
        elif p.kv_dtype == "e4m3":
            self.k = np.ascontiguousarray(_as_np(p.k_cache), np.uint8)
            self.v = np.ascontiguousarray(_as_np(p.v_cache), np.uint8)
            kv_fmt = FMT_E4M3
        else:
            self.k = np.ascontiguousarray(_as_np(p.k_cache), np.float64)
            self.v = np.ascontiguousarray(_as_np(p.v_cache), np.float64)
            kv_fmt = FMT_F64
        total_q = self.q.shape[0]
        assert self.sel_idx.shape == (total_q, p.Hkv, p.num_slots)
        self.st = _Problem(
            num_seqs=p.num_seqs, total_q=total_q, Hq=p.Hq, Hkv=p.Hkv, d_qk=p.d_qk, d_v=p.d_v,
            page_size=p.page_size, unit_tokens=p.unit_tokens, num_slots=p.num_slots,
            slots_per_split=p.slots_per_split, max_pages=self.page_table.shape[1],
            pt_stride=self.page_table.shape[1], num_phys_pages=p.num_phys_pages,
            sm_scale=p.sm_scale, q_scale=p.q_scale, k_scale=p.k_scale, v_scale=p.v_scale,
            q_seq=_ptr(self.q_seq), q_pos=_ptr(self.q_pos), seq_lens=_ptr(self.seq_lens),
            page_table=_ptr(self.page_table), q_fmt=q_fmt, q=_ptr(self.q), kv_fmt=kv_fmt,
            k=_ptr(self.k), v=_ptr(self.v),
            k_sf=_ptr(self.k_sf) if self.k_sf is not None else None,
            v_sf=_ptr(self.v_sf) if self.v_sf is not None else None,
            sel_idx=_ptr(self.sel_idx), sel_mask=_ptr(self.sel_mask),
        )


def prefill_rows(problem, tokens: Optional[Sequence[int]] = None, want_partials: bool = True,
                 want_single_pass: bool = True, keep: Optional[_Keep] = None):
    """Oracle outputs for the given query tokens (default: all).

    Returns a dict with, for n requested tokens:
      part_o [n, Hq, S, d_v], part_lse [n, Hq, S], out [n, Hq, d_v], lse [n, Hq],
      out1 / lse1 (single-pass softmax over the union), err (ERR_* bits),
      tokens (the token indices).
    """
    k = keep if keep is not None else _Keep(problem)
    total_q = k.q.shape[0]
    toks = np.arange(total_q, dtype=np.int32) if tokens is None else \
        np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(toks)
    Hq, dv, S = problem.Hq, problem.d_v, problem.num_slots // problem.slots_per_split
    res = {"tokens": toks}
    po = np.empty((n, Hq, S, dv)) if want_partials else None
    pl = np.empty((n, Hq, S)) if want_partials else None
    out = np.empty((n, Hq, dv))
    lse = np.empty((n, Hq))
    out1 = np.empty((n, Hq, dv)) if want_single_pass else None
    lse1 = np.empty((n, Hq)) if want_single_pass else None
    nul = None
    err = lib().orc_prefill_rows(
        ctypes.byref(k.st), n, _ptr(toks),
        _ptr(po) if po is not None else nul, _ptr(pl) if pl is not None else nul,
        _ptr(out), _ptr(lse),
        _ptr(out1) if out1 is not None else nul, _ptr(lse1) if lse1 is not None else nul)
    res.update(part_o=po, part_lse=pl, out=out, lse=lse, out1=out1, lse1=lse1, err=int(err))
    return res


def slot_nonempty(problem, keep: Optional[_Keep] = None) -> np.ndarray:
    """uint8 [total_q, Hkv, K]: 1 iff the slot contributes a visible key."""
    k = keep if keep is not None else _Keep(problem)
    total_q = k.q.shape[0]
    ne = np.empty((total_q, problem.Hkv, problem.num_slots), np.uint8)
    lib().orc_slot_nonempty(ctypes.byref(k.st), _ptr(ne))
    return ne


def make_keep(problem) -> _Keep:
    return _Keep(problem)


# ------------------------------------------------------------------ indexer

def index_scores(problem):
    """Per-page indexer scores of an IndexProblem: (scores [total_q, H,
    max_pages] float64, -inf where the page has no visible key; error bits)."""
    p = problem
    q = np.ascontiguousarray(_as_np(p.q), np.uint8)
    k = np.ascontiguousarray(_as_np(p.k_cache), np.uint8)
    q_seq = np.ascontiguousarray(_as_np(p.q_seq), np.int32)
    q_pos = np.ascontiguousarray(_as_np(p.q_pos), np.int32)
    seq_lens = np.ascontiguousarray(_as_np(p.seq_lens), np.int32)
    pt = np.ascontiguousarray(_as_np(p.page_table), np.int32)
    T, H, d = q.shape
    st = _IndexProblem(num_seqs=len(seq_lens), total_q=T, H=H, d=d, page_size=p.page_size,
                       max_pages=pt.shape[1], pt_stride=pt.shape[1],
                       num_phys_pages=p.num_phys_pages, q_scale=p.q_scale, k_scale=p.k_scale,
                       q_seq=_ptr(q_seq), q_pos=_ptr(q_pos), seq_lens=_ptr(seq_lens),
                       page_table=_ptr(pt), q=_ptr(q), k=_ptr(k))
    out = np.empty((T, H, pt.shape[1]), np.float64)
    err = lib().orc_index_scores(ctypes.byref(st), _ptr(out))
    return out, int(err)


def topk(scores, k: int):
    """Top-k of each row of ``scores`` [..., n]: (idx [..., k] int32, mask
    [..., k] uint8); descending score, ties by ascending index, -inf never
    selected (index -1, mask 0)."""
    sc = np.ascontiguousarray(np.asarray(scores, np.float64))
    n = sc.shape[-1]
    rows = sc.size // max(n, 1)
    idx = np.empty(sc.shape[:-1] + (k,), np.int32)
    mask = np.empty(sc.shape[:-1] + (k,), np.uint8)
    lib().orc_topk_rows(rows, n, _ptr(sc), k, _ptr(idx), _ptr(mask))
    return idx, mask

