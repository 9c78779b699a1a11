"""C ABI contract tests that need no GPU: the library loads, exports every
entry point include/msa.h declares, and rejects bad arguments on the host
before anything is enqueued (no device call is made by these tests)."""
import ctypes
import os
import re

import pytest

import block_sparse_paged_table_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # a 256-byte aligned non-null address; never dereferenced


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = msa.library()
    declared = _declared()
    assert {"msa_sparse_prefill", "msa_combine", "msa_prefill_plan", "msa_prefill_attend",
            "msa_prefill_workspace_bytes"} <= declared
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert msa.msa_abi_version() == 1


def _desc(**over):
    d = dict(num_seqs=1, total_q=16, num_q_heads=4, num_kv_heads=1, head_dim_qk=64,
             head_dim_v=64, page_size=128, unit_tokens=128, num_slots=3, slots_per_split=1,
             sm_scale=0.0, q_scale=1.0, k_scale=1.0, v_scale=1.0,
             q=FAKE, q_dtype=msa.MSA_F32, q_stride_tok=256, q_stride_head=64,
             q_seq=FAKE, q_pos=FAKE, seq_lens=FAKE, k_cache=FAKE, v_cache=FAKE,
             kv_dtype=msa.MSA_F32, kv_stride_page_bytes=128 * 256, kv_stride_tok_bytes=256,
             kv_stride_head_bytes=256, page_table=FAKE, page_table_stride=4, max_pages=4,
             num_phys_pages=4, sel_idx=FAKE, sel_mask=FAKE, sel_stride_tok=3, sel_stride_head=3,
             partial_o=FAKE, po_split_stride=64 * 64, po_row_stride=64, partial_lse=FAKE,
             pl_split_stride=64)
    d.update(over)
    return msa.PrefillDesc(**d)


def test_workspace_query_accepts_valid_descriptor():
    assert msa.msa_prefill_workspace_bytes(_desc()) > 0
    # FP8 queries with an FP8 cache (per-tensor scaled) and 16-bit partials
    fp8 = dict(q_dtype=msa.MSA_E4M3, kv_dtype=msa.MSA_E4M3, q_stride_tok=256, q_stride_head=64,
               kv_stride_page_bytes=128 * 64, kv_stride_tok_bytes=64, kv_stride_head_bytes=64)
    for pd in (msa.MSA_F32, msa.MSA_BF16, msa.MSA_F16):
        assert msa.msa_prefill_workspace_bytes(_desc(partial_dtype=pd, **fp8)) > 0


_MICROBLOCK = dict(page_size=16, unit_tokens=4, q_dtype=msa.MSA_F16, kv_dtype=msa.MSA_F16,
                  head_dim_qk=128, head_dim_v=128, num_q_heads=6, q_stride_tok=6 * 128,
                  q_stride_head=128, kv_stride_page_bytes=16 * 256, kv_stride_tok_bytes=256,
                  kv_stride_head_bytes=256, num_slots=8, sel_stride_tok=8, sel_stride_head=8,
                  max_pages=64, page_table_stride=64, po_split_stride=96 * 128, po_row_stride=128,
                  pl_split_stride=96, total_q=1024)


@pytest.mark.parametrize("spp", [8, 4, 2, 1])
def test_microblock_route_takes_any_split_count(spp):
    """Microblock selections may be cut into num_slots / slots_per_split splits
    (the split-k form of the grouped route); on a grid large enough that no
    split is cut into runs (8192 tokens: 1024 groups), the workspace grows
    with the splits (their offsets)."""
    assert msa.msa_prefill_workspace_bytes(_desc(slots_per_split=spp, **_MICROBLOCK)) > 0
    big = dict(_MICROBLOCK, total_q=8192)
    n = msa.msa_prefill_workspace_bytes(_desc(slots_per_split=spp, **big))
    if spp < 8:
        assert n > msa.msa_prefill_workspace_bytes(_desc(slots_per_split=8, **big))


def test_microblock_small_grid_runs_workspace():
    """A small grid cuts each split's list into runs whose FP32 partials live
    in the workspace: 128 groups x 1 split of 64 slots gets 4 runs (4 x 128
    work items fill the 512 the runs may use, 16 slots per run), i.e.
    4 x (1024 x 6 rows) x (128 + 1) x 4 bytes; with 8 slots a run would hold
    fewer than 8 slots, so there are none."""
    wide = dict(_MICROBLOCK, num_slots=64, sel_stride_tok=64, sel_stride_head=64)
    runs = msa.msa_prefill_workspace_bytes(_desc(slots_per_split=64, **wide))
    sub = 4 * 1024 * 6 * 128 * 4 + 4 * 1024 * 6 * 4
    lists = 128 * (8 * 64) * (16 + 8)  # planner stage + lists
    assert sub + lists <= runs <= sub + lists + (1 << 20)
    few = msa.msa_prefill_workspace_bytes(_desc(slots_per_split=8, **_MICROBLOCK))
    assert few < sub


def test_microblock_route_rejects_uneven_splits():
    with pytest.raises(msa.MsaError):
        msa.msa_prefill_workspace_bytes(_desc(slots_per_split=3, **_MICROBLOCK))


@pytest.mark.parametrize("over,status", [
    (dict(q=0), msa.MsaError),
    (dict(num_q_heads=5, num_kv_heads=2), msa.MsaError),
    (dict(q_dtype=msa.MSA_BF16), msa.MsaError),              # mixed dtype pair
    (dict(page_size=64, unit_tokens=64), msa.MsaError),     # page size without a kernel
    (dict(q=FAKE + 4), msa.MsaError),                       # misaligned q
    (dict(kv_stride_tok_bytes=260), msa.MsaError),          # misaligned stride
    (dict(slots_per_split=2, num_slots=4), msa.MsaError),
    (dict(num_slots=4, slots_per_split=3), msa.MsaError),
    (dict(page_table_stride=2), msa.MsaError),
    (dict(po_row_stride=32), msa.MsaError),
    (dict(q_dtype=msa.MSA_E4M3, kv_dtype=msa.MSA_NVFP4, head_dim_qk=128, head_dim_v=128,
          q_stride_tok=512, q_stride_head=128), msa.MsaError),  # NVFP4 without scales
    (dict(partial_dtype=7), msa.MsaError),                  # unknown partial dtype
    (dict(partial_dtype=msa.MSA_F16), msa.MsaError),        # FP32 queries take FP32 partials
])
def test_host_validation_rejects(over, status):
    with pytest.raises(status) as ei:
        msa.msa_prefill_workspace_bytes(_desc(**over))
    assert ei.value.status in (1, 2)
    assert msa.library().msa_last_error().decode()


def test_ordering_slice_hint():
    """order_slice_tokens only sizes the plan's list arrays; negative is rejected."""
    base = msa.msa_prefill_workspace_bytes(_desc(total_q=4096))
    many = msa.msa_prefill_workspace_bytes(_desc(total_q=4096, order_slice_tokens=1))
    assert many > base
    with pytest.raises(msa.MsaError):
        msa.msa_prefill_workspace_bytes(_desc(order_slice_tokens=-1))


def test_struct_size_mismatch_rejected():
    d = _desc()
    d.struct_size = 8
    with pytest.raises(msa.MsaError) as ei:
        msa.msa_prefill_workspace_bytes(d)
    assert ei.value.status == 1


def test_workspace_too_small_rejected_before_launch():
    lib = msa.library()
    d = _desc()
    need = msa.msa_prefill_workspace_bytes(d)
    st = lib.msa_sparse_prefill(ctypes.byref(d), FAKE, need - 1, None)
    assert st == 3  # MSA_ERR_WORKSPACE_TOO_SMALL
    st = lib.msa_prefill_plan(ctypes.byref(d), FAKE + 8, need, None)
    assert st == 1  # misaligned workspace


def test_combine_validation():
    lib = msa.library()
    # zero rows is a no-op success; bad sizes and dtypes are rejected
    assert lib.msa_combine(FAKE, 0, 128, FAKE, 0, 4, 0, 128, FAKE, msa.MSA_BF16, 128, None, None) == 0
    assert lib.msa_combine(FAKE, 0, 128, FAKE, 0, 0, 8, 128, FAKE, msa.MSA_BF16, 128, None, None) == 1
    assert lib.msa_combine(FAKE, 0, 128, FAKE, 0, 4, 8, 126, FAKE, msa.MSA_BF16, 128, None, None) == 1
    assert lib.msa_combine(FAKE, 0, 128, FAKE, 0, 4, 8, 128, FAKE, 7, 128, None, None) == 1
    assert lib.msa_combine(FAKE + 4, 0, 128, FAKE, 0, 4, 8, 128, FAKE, 0, 128, None, None) == 1
    # typed partials: F32 / BF16 / F16 only
    assert lib.msa_combine_ex(FAKE, 3, 0, 128, FAKE, 0, 4, 8, 128, FAKE, 0, 128, None, None) == 1
    assert lib.msa_combine_ex(FAKE, msa.MSA_F16, 0, 128, FAKE, 0, 4, 0, 128, FAKE, 0, 128, None, None) == 0


def test_status_strings():
    lib = msa.library()
    assert lib.msa_status_str(0) == b"MSA_OK"
    assert lib.msa_status_str(3) == b"MSA_ERR_WORKSPACE_TOO_SMALL"


def test_runner_rejects_undersized_partial_buffers():
    """Caller-owned partial buffers are sized by the caller; the harness checks
    them before any descriptor is built (the library only sees pointers)."""
    import torch
    from block_sparse_paged_table_amd import synth
    from block_sparse_paged_table_amd.runner import DeviceProblem
    p = synth.make_config(0)
    small = torch.empty((p.num_splits, p.num_rows - 1, p.d_v), dtype=torch.float32)
    with pytest.raises(ValueError):
        DeviceProblem(p, device="cpu", partial_o=small)
    with pytest.raises(ValueError):
        DeviceProblem(p, device="cpu", partial_lse=torch.empty((p.num_splits, 3)))


def test_rotated_input_sets_share_geometry():
    """Benchmark input sets drawn with other seeds differ in data only."""
    import numpy as np
    from block_sparse_paged_table_amd import synth
    for cfg in (0, 4):
        a, b = synth.make_config(cfg), synth.make_config(cfg, seed=1000 + cfg + 100)
        assert (a.total_q, a.num_rows, a.max_pages) == (b.total_q, b.num_rows, b.max_pages)
        assert np.array_equal(a.seq_lens.numpy(), b.seq_lens.numpy())
        assert not np.array_equal(a.sel_idx.numpy(), b.sel_idx.numpy())


def _idesc(**over):
    d = dict(num_seqs=1, total_q=16, num_heads=2, head_dim=128, page_size=128, q_scale=1.0,
             k_scale=1.0, q=FAKE, q_stride_tok=256, q_stride_head=128, q_seq=FAKE, q_pos=FAKE,
             seq_lens=FAKE, k_cache=FAKE, kv_stride_page_bytes=128 * 256, kv_stride_tok_bytes=256,
             kv_stride_head_bytes=128, page_table=FAKE, page_table_stride=4, max_pages=4,
             num_phys_pages=4, scores=FAKE, score_stride=4, top_k=3, sel_idx=FAKE, sel_mask=FAKE,
             sel_stride_tok=6, sel_stride_head=3)
    d.update(over)
    return msa.IndexDesc(**d)


@pytest.mark.parametrize("over", [
    dict(head_dim=96), dict(page_size=64), dict(score_stride=3), dict(q_scale=0.0),
    dict(max_pages=4096, page_table_stride=4096, score_stride=4096), dict(q=FAKE + 8),
    dict(kv_stride_tok_bytes=200), dict(top_k=0), dict(top_k=300), dict(sel_stride_head=2),
    dict(sel_stride_tok=5), dict(sel_idx=0), dict(struct_size=4)])
def test_index_validation_rejects(over):
    """Indexer descriptors are checked on the host before any launch."""
    d = _idesc(**{k: v for k, v in over.items() if k != "struct_size"})
    if "struct_size" in over:
        d.struct_size = over["struct_size"]
    lib = msa.library()
    calls = [lib.msa_prefill_index, lib.msa_index_topk]
    if not set(over) & {"top_k", "sel_stride_head", "sel_stride_tok", "sel_idx"}:
        calls.append(lib.msa_index_scores)  # (it does not use the selection outputs)
    for fn in calls:  # every case is rejected on the host: nothing is launched
        assert fn(ctypes.byref(d), None) in (1, 2), fn



@pytest.mark.parametrize("layout,pad", [("row", 0), ("split", 0), ("row", 8)])
def test_partial_layouts_describe_their_strides(layout, pad):
    """The device harness builds descriptors on the host: a row-major partial
    buffer ([row][split][d]) is described by split stride d and row stride
    splits * d; a split-major one by row stride d and split stride rows * d
    (padded rows widen both); the workspace does not depend on the layout."""
    from block_sparse_paged_table_amd import synth
    from block_sparse_paged_table_amd.runner import DeviceProblem
    p = synth.make_config(0)
    dp = DeviceProblem(p, device="cpu", partial_layout=layout, po_row_pad=pad)
    S, rows, w = p.num_splits, p.num_rows, p.d_v + pad
    assert tuple(dp.partial_o.shape) == (S, rows, w)
    if layout == "row":
        assert (dp.desc.po_split_stride, dp.desc.po_row_stride) == (w, S * w)
    else:
        assert (dp.desc.po_split_stride, dp.desc.po_row_stride) == (rows * w, w)
    assert dp.ws_bytes == DeviceProblem(p, device="cpu").ws_bytes
    with pytest.raises(ValueError):
        DeviceProblem(p, device="cpu", partial_layout="column")


def _kernel_lds_of_library():
    """{kernel symbol: group_segment_fixed_size} of every gfx950 kernel in
    lib/libmsa.so, read from the code objects' metadata notes: the library's
    .hip_fatbin section holds one offload bundle per source file."""
    import shutil
    import subprocess
    import tempfile
    tools = {t: shutil.which(t) or os.path.join("/opt/rocm/llvm/bin", t)
             for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")}
    if not all(os.path.exists(p) for p in tools.values()):
        pytest.skip("ROCm LLVM tools not found")
    out = {}
    with tempfile.TemporaryDirectory() as td:
        fat = os.path.join(td, "fat.bin")
        subprocess.check_call([tools["llvm-objcopy"], "-O", "binary", "--only-section=.hip_fatbin",
                               msa.library_path, fat])
        data = open(fat, "rb").read()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        starts, i = [], data.find(magic)
        while i >= 0:
            starts.append(i)
            i = data.find(magic, i + 1)
        assert starts, "no offload bundle in libmsa.so"
        for k, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            bundle, co = os.path.join(td, f"b{k}.bin"), os.path.join(td, f"b{k}.co")
            open(bundle, "wb").write(data[a:b])
            subprocess.check_call([tools["clang-offload-bundler"], "--type=o", "--unbundle",
                                   "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                                   f"--input={bundle}", f"--output={co}"])
            notes = subprocess.check_output([tools["llvm-readelf"], "--notes", co], text=True)
            lds = None
            for line in notes.splitlines():
                line = line.strip()
                if line.startswith(".group_segment_fixed_size:"):
                    lds = int(line.split(":")[1])
                elif line.startswith(".name:") and lds is not None:
                    out[line.split(":", 1)[1].strip()] = lds
                    lds = None
    return out


def test_required_lds_covers_every_compiled_kernel():
    """msa_device_supported compares the device's LDS with
    msa_required_lds_bytes(): it must cover the static LDS of every kernel
    the build compiled, and equal the largest one (the FP32 page-route
    attention at head_dim 128, 135,232 bytes; the planners' dynamic LDS is
    smaller)."""
    lds = _kernel_lds_of_library()
    attend = {k: v for k, v in lds.items() if "k1_page_attend" in k}
    assert len(attend) >= 9 and any("k_grouped_attend" in k for k in lds)
    need = msa.msa_required_lds_bytes()
    assert max(lds.values()) <= need
    assert need == max(attend.values()) == 135232


def test_workspace_query_one_value_form():
    """msa_sparse_prefill_workspace_bytes: the workspace size, or 0 for a
    rejected descriptor."""
    d = _desc()
    assert msa.msa_sparse_prefill_workspace_bytes(d) == msa.msa_prefill_workspace_bytes(d)
    assert msa.msa_sparse_prefill_workspace_bytes(_desc(q=0)) == 0
    assert msa.library().msa_last_error().decode()


def test_noalloc_rejects_problems_beyond_its_scratch_before_launch():
    """msa_sparse_prefill_noalloc checks the workspace the descriptor needs
    against its fixed scratch on the host, before touching the device."""
    lib = msa.library()
    assert msa.msa_noalloc_scratch_bytes() == 32 << 20
    big = _desc(total_q=8192, num_slots=512, sel_stride_tok=512, sel_stride_head=512,
                **{k: v for k, v in _MICROBLOCK.items() if k not in ("total_q", "num_slots",
                                                                     "sel_stride_tok", "sel_stride_head")})
    assert msa.msa_prefill_workspace_bytes(big) > msa.msa_noalloc_scratch_bytes()
    assert lib.msa_sparse_prefill_noalloc(ctypes.byref(big), None) == 3  # WORKSPACE_TOO_SMALL
    assert b"scratch" in lib.msa_last_error()
    assert lib.msa_sparse_prefill_noalloc(ctypes.byref(_desc(q=0)), None) == 1


def test_calibration_probes_load_and_validate():
    """The ceiling probes of libmsa_calib.so (not part of the attention
    library) load, export their entry points and reject bad arguments on the
    host; calib_chunk_bytes is host arithmetic."""
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_paged_table_amd", "lib", "libmsa_calib.so"))
    for name in ("calib_read", "calib_write", "calib_gather", "calib_lds", "calib_lds_pattern",
                 "calib_mixed", "calib_chunk_bytes"):
        assert hasattr(lib, name), name
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.calib_lds.argtypes = [P, I32, I32, I32, P]
    assert lib.calib_lds(None, 512, 10, 0, None) == 1   # no sink
    assert lib.calib_lds(FAKE, 0, 10, 0, None) == 1     # empty grid
    assert lib.calib_lds(FAKE, 512, 0, 0, None) == 1    # no iterations
    assert lib.calib_lds(FAKE, 512, 10, 4, None) == 1   # unknown mode
    lib.calib_lds_pattern.argtypes = [P, I32, I32, P, I32, P]
    assert lib.calib_lds_pattern(FAKE, 512, 10, None, 0, None) == 1  # no offset table
    assert lib.calib_lds_pattern(FAKE, 512, 10, FAKE, 2, None) == 1  # unknown read kind
    lib.calib_mixed.argtypes = [P, I64, P, I64, P, I32, I64, I32, P]
    assert lib.calib_mixed(FAKE, 8192, FAKE, 8192 * 6, FAKE, 1, 1, 9, None) == 1      # ratio out of range
    assert lib.calib_mixed(FAKE, 8192, FAKE, 8192 * 5, FAKE, 1, 1, 6, None) == 1      # write array too small
    assert lib.calib_mixed(FAKE, 8191, FAKE, 8192 * 6, FAKE, 1, 1, 6, None) == 1      # read array too small
    lib.calib_chunk_bytes.argtypes = [I64, I32, I32]
    lib.calib_chunk_bytes.restype = I64
    assert lib.calib_chunk_bytes(4 << 30, 2048, 8) == 4 << 30
    assert lib.calib_chunk_bytes((4 << 30) + 4096, 2048, 8) == 4 << 30
