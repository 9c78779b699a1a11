"""block_sparse_paged_table_amd -- block-sparse paged prefill attention with
per-split partials and a streaming LSE combine, for AMD MI355X (gfx950).

This module is the thin Python binding of the C ABI in ``include/msa.h``
(``lib/libmsa.so``): it marshals arguments only.  Every step of the
computation runs in the HIP kernels of the library; if the library is
missing, every call raises.  PyTorch is used for device memory and streams.

Functions (same names as the C entry points):
  msa_prefill_workspace_bytes(desc) -> int
  msa_prefill_plan(desc, workspace, stream=None)
  msa_prefill_attend(desc, workspace, stream=None)
  msa_sparse_prefill(desc, workspace, stream=None)
  msa_sparse_prefill_noalloc(desc, stream=None)
  msa_combine(partial_o, partial_lse, num_splits, num_rows, head_dim_v, out,
              lse=None, ...strides..., stream=None)
  msa_nvfp4_dequant_e4m3(codes, scales, out, stream=None)
  msa_nvfp4_dequant_f16(codes, scales, out, stream=None)
  msa_device_supported(device) -> bool
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

__all__ = [
    "MSA_F32", "MSA_BF16", "MSA_F16", "MSA_E4M3", "MSA_NVFP4",
    "MSA_ERRF_SEL_RANGE", "MSA_ERRF_PHYS_RANGE", "MSA_ERRF_QSEQ_RANGE", "MSA_ERRF_DUPLICATE",
    "MsaError", "PrefillDesc", "IndexDesc", "library", "library_path", "msa_combine_ex",
    "msa_index_scores", "msa_index_topk", "msa_prefill_index",
    "msa_prefill_workspace_bytes", "msa_prefill_plan", "msa_prefill_attend",
    "msa_sparse_prefill", "msa_sparse_prefill_noalloc", "msa_noalloc_scratch_bytes", "msa_combine", "msa_nvfp4_dequant_e4m3", "msa_nvfp4_dequant_f16",
    "msa_device_supported", "msa_required_lds_bytes", "msa_sparse_prefill_workspace_bytes",
    "msa_abi_version",
]

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "lib", "libmsa.so")

MSA_F32, MSA_BF16, MSA_F16, MSA_E4M3, MSA_NVFP4 = 0, 1, 2, 3, 4
MSA_ERRF_SEL_RANGE, MSA_ERRF_PHYS_RANGE, MSA_ERRF_QSEQ_RANGE, MSA_ERRF_DUPLICATE = 1, 2, 4, 8
STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARG", 2: "MSA_ERR_UNSUPPORTED",
          3: "MSA_ERR_WORKSPACE_TOO_SMALL", 4: "MSA_ERR_HIP"}


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_c_i32, _c_i64, _c_f32, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class PrefillDesc(ctypes.Structure):
    """Mirror of ``msa_prefill_desc`` (include/msa.h), field for field."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_seqs", _c_i32), ("total_q", _c_i32), ("num_q_heads", _c_i32),
        ("num_kv_heads", _c_i32), ("head_dim_qk", _c_i32), ("head_dim_v", _c_i32),
        ("page_size", _c_i32), ("unit_tokens", _c_i32), ("num_slots", _c_i32),
        ("slots_per_split", _c_i32),
        ("sm_scale", _c_f32), ("q_scale", _c_f32), ("k_scale", _c_f32), ("v_scale", _c_f32),
        ("q", _c_p), ("q_dtype", _c_i32), ("q_stride_tok", _c_i64), ("q_stride_head", _c_i64),
        ("q_seq", _c_p), ("q_pos", _c_p), ("seq_lens", _c_p),
        ("k_cache", _c_p), ("v_cache", _c_p), ("kv_dtype", _c_i32),
        ("kv_stride_page_bytes", _c_i64), ("kv_stride_tok_bytes", _c_i64),
        ("kv_stride_head_bytes", _c_i64),
        ("k_sf", _c_p), ("v_sf", _c_p),
        ("sf_stride_page_bytes", _c_i64), ("sf_stride_tok_bytes", _c_i64),
        ("sf_stride_head_bytes", _c_i64),
        ("page_table", _c_p), ("page_table_stride", _c_i64), ("max_pages", _c_i32),
        ("num_phys_pages", _c_i32),
        ("sel_idx", _c_p), ("sel_mask", _c_p), ("sel_stride_tok", _c_i64),
        ("sel_stride_head", _c_i64),
        ("partial_o", _c_p), ("po_split_stride", _c_i64), ("po_row_stride", _c_i64),
        ("partial_lse", _c_p), ("pl_split_stride", _c_i64),
        ("err_flags", _c_p),
        ("order_slice_tokens", ctypes.c_int32),
        ("partial_dtype", ctypes.c_int32),
    ]

    def __init__(self, **kw):
        super().__init__(**kw)
        self.struct_size = ctypes.sizeof(PrefillDesc)


class IndexDesc(ctypes.Structure):
    """Mirror of ``msa_index_desc`` (include/msa.h), field for field."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_seqs", _c_i32), ("total_q", _c_i32), ("num_heads", _c_i32), ("head_dim", _c_i32),
        ("page_size", _c_i32), ("q_scale", _c_f32), ("k_scale", _c_f32),
        ("q", _c_p), ("q_stride_tok", _c_i64), ("q_stride_head", _c_i64),
        ("q_seq", _c_p), ("q_pos", _c_p), ("seq_lens", _c_p),
        ("k_cache", _c_p), ("kv_stride_page_bytes", _c_i64), ("kv_stride_tok_bytes", _c_i64),
        ("kv_stride_head_bytes", _c_i64),
        ("page_table", _c_p), ("page_table_stride", _c_i64), ("max_pages", _c_i32),
        ("num_phys_pages", _c_i32),
        ("scores", _c_p), ("score_stride", _c_i64), ("top_k", _c_i32),
        ("sel_idx", _c_p), ("sel_mask", _c_p), ("sel_stride_tok", _c_i64),
        ("sel_stride_head", _c_i64), ("err_flags", _c_p),
    ]

    def __init__(self, **kw):
        super().__init__(**kw)
        self.struct_size = ctypes.sizeof(IndexDesc)


_lock = threading.Lock()
_lib = None

# (name, restype, argtypes) of every exported symbol
_SIGNATURES = [
    ("msa_prefill_workspace_bytes", ctypes.c_int, [ctypes.POINTER(PrefillDesc), ctypes.POINTER(ctypes.c_size_t)]),
    ("msa_prefill_plan", ctypes.c_int, [ctypes.POINTER(PrefillDesc), _c_p, ctypes.c_size_t, _c_p]),
    ("msa_prefill_attend", ctypes.c_int, [ctypes.POINTER(PrefillDesc), _c_p, ctypes.c_size_t, _c_p]),
    ("msa_sparse_prefill", ctypes.c_int, [ctypes.POINTER(PrefillDesc), _c_p, ctypes.c_size_t, _c_p]),
    ("msa_sparse_prefill_noalloc", ctypes.c_int, [ctypes.POINTER(PrefillDesc), _c_p]),
    ("msa_noalloc_scratch_bytes", ctypes.c_size_t, []),
    ("msa_combine", ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_i32, _c_i64, _c_i32,
                                   _c_p, _c_i32, _c_i64, _c_p, _c_p]),
    ("msa_combine_ex", ctypes.c_int, [_c_p, _c_i32, _c_i64, _c_i64, _c_p, _c_i64, _c_i32, _c_i64,
                                      _c_i32, _c_p, _c_i32, _c_i64, _c_p, _c_p]),
    ("msa_nvfp4_dequant_e4m3", ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_p]),
    ("msa_nvfp4_dequant_f16", ctypes.c_int, [_c_p, _c_p, _c_p, _c_i64, _c_p]),
    ("msa_index_scores", ctypes.c_int, [ctypes.POINTER(IndexDesc), _c_p]),
    ("msa_index_topk", ctypes.c_int, [ctypes.POINTER(IndexDesc), _c_p]),
    ("msa_prefill_index", ctypes.c_int, [ctypes.POINTER(IndexDesc), _c_p]),
    ("msa_device_supported", ctypes.c_int, [ctypes.c_int]),
    ("msa_required_lds_bytes", ctypes.c_size_t, []),
    ("msa_sparse_prefill_workspace_bytes", ctypes.c_size_t, [ctypes.POINTER(PrefillDesc)]),
    ("msa_status_str", ctypes.c_char_p, [ctypes.c_int]),
    ("msa_last_error", ctypes.c_char_p, []),
    ("msa_abi_version", ctypes.c_int, []),
]


def library() -> ctypes.CDLL:
    """Load lib/libmsa.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(library_path):
                raise RuntimeError(
                    f"{library_path} is missing: build it with "
                    "`python -m block_sparse_paged_table_amd.build` (there is no fallback)")
            lib = ctypes.CDLL(library_path)
            for name, res, args in _SIGNATURES:
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def _check(status: int):
    if status != 0:
        raise MsaError(status, library().msa_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def msa_abi_version() -> int:
    return library().msa_abi_version()


def msa_prefill_workspace_bytes(desc: PrefillDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(library().msa_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _ws(workspace):
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def msa_prefill_plan(desc: PrefillDesc, workspace, stream=None):
    p, n = _ws(workspace)
    _check(library().msa_prefill_plan(ctypes.byref(desc), p, n, _stream(stream)))


def msa_prefill_attend(desc: PrefillDesc, workspace, stream=None):
    p, n = _ws(workspace)
    _check(library().msa_prefill_attend(ctypes.byref(desc), p, n, _stream(stream)))


def msa_sparse_prefill(desc: PrefillDesc, workspace, stream=None):
    p, n = _ws(workspace)
    _check(library().msa_sparse_prefill(ctypes.byref(desc), p, n, _stream(stream)))


def msa_sparse_prefill_noalloc(desc: PrefillDesc, stream=None):
    """msa_sparse_prefill on the library's fixed per-device scratch (no
    workspace argument, nothing allocated); calls on one GPU must not overlap."""
    _check(library().msa_sparse_prefill_noalloc(ctypes.byref(desc), _stream(stream)))


def msa_noalloc_scratch_bytes() -> int:
    return library().msa_noalloc_scratch_bytes()


def _combine_args(partial_o, partial_lse, out, po_split_stride, po_row_stride, pl_split_stride,
                  out_dtype, out_row_stride):
    import torch
    codes = {torch.float32: MSA_F32, torch.bfloat16: MSA_BF16, torch.float16: MSA_F16}
    return (partial_o.stride(0) if po_split_stride is None else po_split_stride,
            partial_o.stride(-2) if po_row_stride is None else po_row_stride,
            partial_lse.stride(0) if pl_split_stride is None else pl_split_stride,
            codes[out.dtype] if out_dtype is None else out_dtype,
            out.stride(-2) if out_row_stride is None else out_row_stride,
            codes.get(partial_o.dtype))


def msa_combine(partial_o, partial_lse, num_splits: int, num_rows: int, head_dim_v: int, out,
                lse=None, po_split_stride: Optional[int] = None, po_row_stride: Optional[int] = None,
                pl_split_stride: Optional[int] = None, out_dtype: Optional[int] = None,
                out_row_stride: Optional[int] = None, stream=None):
    """LSE combine of FP32 partials; strides default to those of [S, rows, d] /
    [S, rows] / [rows, d] tensors."""
    pss, prs, lss, odt, ors, _ = _combine_args(partial_o, partial_lse, out, po_split_stride,
                                               po_row_stride, pl_split_stride, out_dtype,
                                               out_row_stride)
    _check(library().msa_combine(_ptr(partial_o), pss, prs, _ptr(partial_lse), lss, num_splits,
                                 num_rows, head_dim_v, _ptr(out), odt, ors, _ptr(lse),
                                 _stream(stream)))


def msa_combine_ex(partial_o, partial_lse, num_splits: int, num_rows: int, head_dim_v: int, out,
                   lse=None, partial_dtype: Optional[int] = None,
                   po_split_stride: Optional[int] = None, po_row_stride: Optional[int] = None,
                   pl_split_stride: Optional[int] = None, out_dtype: Optional[int] = None,
                   out_row_stride: Optional[int] = None, stream=None):
    """LSE combine of FP32, BF16 or FP16 partials (dtype taken from the tensor
    unless given)."""
    pss, prs, lss, odt, ors, pdt = _combine_args(partial_o, partial_lse, out, po_split_stride,
                                                 po_row_stride, pl_split_stride, out_dtype,
                                                 out_row_stride)
    pdt = pdt if partial_dtype is None else partial_dtype
    _check(library().msa_combine_ex(_ptr(partial_o), pdt, pss, prs, _ptr(partial_lse), lss,
                                    num_splits, num_rows, head_dim_v, _ptr(out), odt, ors,
                                    _ptr(lse), _stream(stream)))


def msa_index_scores(desc: IndexDesc, stream=None):
    _check(library().msa_index_scores(ctypes.byref(desc), _stream(stream)))


def msa_index_topk(desc: IndexDesc, stream=None):
    _check(library().msa_index_topk(ctypes.byref(desc), _stream(stream)))


def msa_prefill_index(desc: IndexDesc, stream=None):
    _check(library().msa_prefill_index(ctypes.byref(desc), _stream(stream)))


def msa_nvfp4_dequant_e4m3(codes, scales, out, stream=None):
    _check(library().msa_nvfp4_dequant_e4m3(_ptr(codes), _ptr(scales), _ptr(out), codes.numel(),
                                            _stream(stream)))


def msa_nvfp4_dequant_f16(codes, scales, out, stream=None):
    _check(library().msa_nvfp4_dequant_f16(_ptr(codes), _ptr(scales), _ptr(out), codes.numel(),
                                           _stream(stream)))


def msa_sparse_prefill_workspace_bytes(desc: PrefillDesc) -> int:
    """Workspace bytes, or 0 if the descriptor is rejected."""
    return library().msa_sparse_prefill_workspace_bytes(ctypes.byref(desc))


def msa_required_lds_bytes() -> int:
    return library().msa_required_lds_bytes()


def msa_device_supported(device: int = 0) -> bool:
    return bool(library().msa_device_supported(device))
