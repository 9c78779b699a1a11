"""Device-side harness: puts a synthetic Problem into device memory, builds
the C ABI descriptor, allocates outputs and workspace, and calls the library.

Argument marshalling only; every computation happens in libmsa's kernels.
"""
from __future__ import annotations

import torch

from . import (MSA_BF16, MSA_E4M3, MSA_F16, MSA_F32, MSA_NVFP4, IndexDesc, PrefillDesc,
               msa_combine_ex, msa_index_scores, msa_index_topk, msa_prefill_index,
               msa_prefill_attend, msa_prefill_plan, msa_prefill_workspace_bytes,
               msa_sparse_prefill, msa_sparse_prefill_noalloc)
from .synth import Problem

DTYPE_CODE = {"f32": MSA_F32, "bf16": MSA_BF16, "f16": MSA_F16, "e4m3": MSA_E4M3,
              "nvfp4": MSA_NVFP4}
OUT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _bstrides(t: torch.Tensor):
    es = t.element_size()
    return [s * es for s in t.stride()]


class DeviceProblem:
    """A Problem resident on `device`, with its outputs and workspace."""

    def __init__(self, p: Problem, device: str = "cuda", out_dtype: str = None,
                 partial_o: torch.Tensor = None, partial_lse: torch.Tensor = None,
                 po_row_pad: int = 0, order_slice_tokens: int = 0, partial_dtype: str = "f32",
                 partial_layout: str = "split"):
        self.p = p
        self.order_slice_tokens = order_slice_tokens
        self.partial_dtype = partial_dtype
        dev = torch.device(device)
        self.device = dev
        self.q = p.q.to(dev)
        self.q_seq = p.q_seq.to(dev)
        self.q_pos = p.q_pos.to(dev)
        self.seq_lens = p.seq_lens.to(dev)
        self.page_table = p.page_table.to(dev)
        # K/V keep their layout (strides) on the device
        if p.k_cache.is_contiguous() and p.v_cache.is_contiguous():
            self.k = p.k_cache.to(dev)
            self.v = p.v_cache.to(dev)
        else:  # K/V views of one interleaved tensor: move the base, re-view
            base = p.k_cache._base if p.k_cache._base is not None else p.k_cache
            dbase = base.to(dev)
            off_k = p.k_cache.storage_offset() - base.storage_offset()
            off_v = p.v_cache.storage_offset() - base.storage_offset()
            self.k = torch.as_strided(dbase, p.k_cache.shape, p.k_cache.stride(), off_k)
            self.v = torch.as_strided(dbase, p.v_cache.shape, p.v_cache.stride(), off_v)
            self._kv_base = dbase
        self.k_sf = p.k_sf.to(dev) if p.k_sf is not None else None
        self.v_sf = p.v_sf.to(dev) if p.v_sf is not None else None
        self.sel_idx = p.sel_idx.to(dev)
        self.sel_mask = p.sel_mask.to(dev)
        S, rows, dv = p.num_splits, p.num_rows, p.d_v
        if partial_o is None and partial_layout == "row":
            # [row][split][d]: each row's splits form one contiguous run, which
            # the combine then reads in order; viewed as [split][row][d]
            partial_o = torch.empty((rows, S, dv + po_row_pad), dtype=OUT_TORCH[partial_dtype],
                                    device=dev).permute(1, 0, 2)
        elif partial_o is None:
            if partial_layout != "split":
                raise ValueError(f"partial_layout {partial_layout!r}: 'split' or 'row'")
            partial_o = torch.empty((S, rows, dv + po_row_pad), dtype=OUT_TORCH[partial_dtype],
                                    device=dev)
        if partial_lse is None:
            partial_lse = torch.empty((S, rows), dtype=torch.float32, device=dev)
        # caller-provided buffers must hold every (split, row) the kernels write
        if (partial_o.dim() != 3 or partial_o.shape[0] < S or partial_o.shape[1] < rows
                or partial_o.shape[2] < dv or partial_o.dtype != OUT_TORCH[partial_dtype]):
            raise ValueError(f"partial_o {tuple(partial_o.shape)} too small for {(S, rows, dv)}")
        if partial_lse.dim() != 2 or partial_lse.shape[0] < S or partial_lse.shape[1] < rows:
            raise ValueError(f"partial_lse {tuple(partial_lse.shape)} too small for {(S, rows)}")
        self.partial_o = partial_o
        self.partial_lse = partial_lse
        self.out_dtype = out_dtype or p.out_dtype
        self.out = torch.empty((rows, dv), dtype=OUT_TORCH[self.out_dtype], device=dev)
        self.lse = torch.empty((rows,), dtype=torch.float32, device=dev)
        self.err = torch.zeros((1,), dtype=torch.int32, device=dev)
        self.desc = self.make_desc()
        self.ws_bytes = msa_prefill_workspace_bytes(self.desc)
        self.workspace = torch.empty((max(self.ws_bytes, 256),), dtype=torch.uint8, device=dev)

    def make_desc(self) -> PrefillDesc:
        p = self.p
        kb = _bstrides(self.k)
        d = PrefillDesc(
            num_seqs=p.num_seqs, total_q=p.total_q, num_q_heads=p.Hq, num_kv_heads=p.Hkv,
            head_dim_qk=p.d_qk, head_dim_v=p.d_v, page_size=p.page_size,
            unit_tokens=p.unit_tokens, num_slots=p.num_slots, slots_per_split=p.slots_per_split,
            sm_scale=p.sm_scale, q_scale=p.q_scale, k_scale=p.k_scale, v_scale=p.v_scale,
            q=self.q.data_ptr(), q_dtype=DTYPE_CODE[p.q_dtype],
            q_stride_tok=self.q.stride(0), q_stride_head=self.q.stride(1),
            q_seq=self.q_seq.data_ptr(), q_pos=self.q_pos.data_ptr(),
            seq_lens=self.seq_lens.data_ptr(),
            k_cache=self.k.data_ptr(), v_cache=self.v.data_ptr(), kv_dtype=DTYPE_CODE[p.kv_dtype],
            kv_stride_page_bytes=kb[0], kv_stride_tok_bytes=kb[1], kv_stride_head_bytes=kb[2],
            page_table=self.page_table.data_ptr(), page_table_stride=self.page_table.stride(0),
            max_pages=p.max_pages, num_phys_pages=p.num_phys_pages,
            sel_idx=self.sel_idx.data_ptr(), sel_mask=self.sel_mask.data_ptr(),
            sel_stride_tok=self.sel_idx.stride(0), sel_stride_head=self.sel_idx.stride(1),
            partial_o=self.partial_o.data_ptr(), po_split_stride=self.partial_o.stride(0),
            po_row_stride=self.partial_o.stride(1),
            partial_lse=self.partial_lse.data_ptr(), pl_split_stride=self.partial_lse.stride(0),
            err_flags=self.err.data_ptr(), order_slice_tokens=self.order_slice_tokens,
            partial_dtype=DTYPE_CODE[self.partial_dtype],
        )
        if self.k_sf is not None:
            sb = _bstrides(self.k_sf)
            d.k_sf = self.k_sf.data_ptr()
            d.v_sf = self.v_sf.data_ptr()
            d.sf_stride_page_bytes, d.sf_stride_tok_bytes, d.sf_stride_head_bytes = sb[0], sb[1], sb[2]
        return d

    # -- calls ---------------------------------------------------------------
    def plan(self, stream=None):
        msa_prefill_plan(self.desc, self.workspace, stream)

    def attend(self, stream=None):
        msa_prefill_attend(self.desc, self.workspace, stream)

    def prefill(self, stream=None):
        msa_sparse_prefill(self.desc, self.workspace, stream)

    def prefill_noalloc(self, stream=None):
        msa_sparse_prefill_noalloc(self.desc, stream)

    def combine(self, stream=None, lse: bool = True):
        p = self.p
        msa_combine_ex(self.partial_o, self.partial_lse, p.num_splits, p.num_rows, p.d_v, self.out,
                       self.lse if lse else None, po_row_stride=self.partial_o.stride(1),
                       stream=stream)

    def run(self, stream=None):
        self.prefill(stream)
        self.combine(stream)

    def err_flags(self) -> int:
        return int(self.err.item()) & 0xffffffff


class DeviceIndexProblem:
    """An IndexProblem resident on `device`, with its score and selection
    buffers (scores [total_q * H, max_pages + score_pad], selections
    [total_q, H, top_k])."""

    def __init__(self, ip, device: str = "cuda", top_k: int = None, score_pad: int = 0):
        self.p = ip
        dev = torch.device(device)
        self.device = dev
        self.q = ip.q.to(dev)
        self.q_seq = ip.q_seq.to(dev)
        self.q_pos = ip.q_pos.to(dev)
        self.seq_lens = ip.seq_lens.to(dev)
        self.page_table = ip.page_table.to(dev)
        self.k = ip.k_cache.to(dev)
        self.top_k = top_k or ip.top_k
        T, H = ip.total_q, ip.H
        self.scores = torch.empty((T * H, ip.max_pages + score_pad), dtype=torch.float32, device=dev)
        self.sel_idx = torch.empty((T, H, self.top_k), dtype=torch.int32, device=dev)
        self.sel_mask = torch.empty((T, H, self.top_k), dtype=torch.uint8, device=dev)
        self.err = torch.zeros((1,), dtype=torch.int32, device=dev)
        kb = _bstrides(self.k)
        self.desc = IndexDesc(
            num_seqs=ip.num_seqs, total_q=T, num_heads=H, head_dim=ip.d, page_size=ip.page_size,
            q_scale=ip.q_scale, k_scale=ip.k_scale,
            q=self.q.data_ptr(), q_stride_tok=self.q.stride(0), q_stride_head=self.q.stride(1),
            q_seq=self.q_seq.data_ptr(), q_pos=self.q_pos.data_ptr(),
            seq_lens=self.seq_lens.data_ptr(),
            k_cache=self.k.data_ptr(), kv_stride_page_bytes=kb[0], kv_stride_tok_bytes=kb[1],
            kv_stride_head_bytes=kb[2],
            page_table=self.page_table.data_ptr(), page_table_stride=self.page_table.stride(0),
            max_pages=ip.max_pages, num_phys_pages=ip.num_phys_pages,
            scores=self.scores.data_ptr(), score_stride=self.scores.stride(0), top_k=self.top_k,
            sel_idx=self.sel_idx.data_ptr(), sel_mask=self.sel_mask.data_ptr(),
            sel_stride_tok=self.sel_idx.stride(0), sel_stride_head=self.sel_idx.stride(1),
            err_flags=self.err.data_ptr())

    def scores_only(self, stream=None):
        msa_index_scores(self.desc, stream)

    def topk(self, stream=None):
        msa_index_topk(self.desc, stream)

    def run(self, stream=None):
        msa_prefill_index(self.desc, stream)

    def err_flags(self) -> int:
        return int(self.err.item()) & 0xffffffff

