#!/usr/bin/env python3
"""Benchmark of the block-sparse paged prefill hot path on one MI355X.

One step = plan + attention (per-page partial O / LSE) + LSE combine over one
synthetic layer.  Inputs (several rotated sets, so that repeated steps do not
reuse cached Q/KV) are resident in HBM before timing starts.  Prints one JSON
line with whole-step throughput, per-kernel times, the roofline of the
dominant kernel (measured with HIP events on the launch stream) and the CPU
oracle timed on a bounded sample of the same workload.

usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 2]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0               # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0, "f16": 2500.0, "f32": 157.3}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload_stats(p):
    """Algorithmic work of one layer, from the selections (host numpy).

    visible[t, g, j]: keys of slot j of (token t, KV head g) the causal /
    tail rules leave visible (0 = empty slot)."""
    pos = p.q_pos.numpy().astype(np.int64)
    seq = p.q_seq.numpy()
    sl = p.seq_lens.numpy().astype(np.int64)
    valid_row = pos >= 0
    last = np.where(valid_row, np.minimum(pos, sl[np.clip(seq, 0, len(sl) - 1)] - 1), -1)
    si = p.sel_idx.numpy().astype(np.int64)
    sm = p.sel_mask.numpy()
    start = si * p.unit_tokens
    vis = np.clip(last[:, None, None] - start + 1, 0, p.unit_tokens)
    if p.unit_tokens != p.page_size:  # microblocks: count the mask bits in the visible prefix
        prefix = (1 << vis) - 1
        bits = (sm.astype(np.int64) & prefix)
        vis = sum((bits >> i) & 1 for i in range(p.unit_tokens))
    vis = np.where((sm != 0) & (si >= 0), vis, 0)
    G = p.Hq // p.Hkv
    n_vis = int(vis.sum()) * G                      # (row, key) pairs
    per_split = vis.reshape(vis.shape[0], vis.shape[1], p.num_splits, p.slots_per_split).sum(-1)
    nonempty = int((per_split > 0).sum()) * G        # (row, split) partials written
    # cache rows (token, KV head) of the distinct units some valid row selected:
    # the K/V bytes an ideal kernel reads once
    n_units = p.page_table.shape[1] * p.page_size // p.unit_tokens
    seq_ok = valid_row & (seq >= 0) & (seq < len(sl))
    sel = (sm != 0) & (si >= 0) & (si < n_units) & seq_ok[:, None, None]
    ukey = (seq.astype(np.int64)[:, None, None] * p.Hkv + np.arange(p.Hkv)[None, :, None]) * n_units + si
    touched_rows = int(np.unique(ukey[sel]).size) * p.unit_tokens
    # microblock route: every (8-token group, KV head, split) loads each
    # distinct unit its rows selected in that split once (K and V rows)
    gathered = 0
    if p.unit_tokens != p.page_size:
        kvrow = p.k_cache.element_size() * p.d_qk + p.v_cache.element_size() * p.d_v
        T = si.shape[0]
        grp = np.arange(T) // 8
        split = np.arange(p.num_slots) // p.slots_per_split
        gkey = ((grp[:, None, None] * p.Hkv + np.arange(p.Hkv)[None, :, None]) * p.num_splits
                + split[None, None, :]) * (n_units + 1) + si
        gathered = int(np.unique(gkey[sel & (vis > 0)]).size) * p.unit_tokens * kvrow
    return dict(n_visible=n_vis, nonempty=nonempty, touched_kv_rows=touched_rows,
                gathered_kv_bytes=gathered,
                flops=4.0 * p.d_qk * n_vis if p.d_qk == p.d_v else 2.0 * (p.d_qk + p.d_v) * n_vis)


def tensor_bytes(t):
    return t.numel() * t.element_size()


def _calib_lib():
    import ctypes
    path = os.path.join(ROOT, "block_sparse_paged_table_amd", "lib", "libmsa_calib.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build with `python -m block_sparse_paged_table_amd.build`")
    lib = ctypes.CDLL(path)
    P, I64, I32, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
    lib.calib_read.argtypes = [P, I64, P, I32, I32, P]
    lib.calib_write.argtypes = [P, I64, I32, U32, I32, P]
    lib.calib_gather.argtypes = [P, I64, P, I64, P, I32, I32, P]
    lib.calib_lds.argtypes = [P, I32, I32, I32, P]
    lib.calib_mixed.argtypes = [P, I64, P, I64, P, I32, I64, I32, P]
    lib.calib_lds_pattern.argtypes = [P, I32, I32, P, I32, P]
    lib.calib_chunk_bytes.argtypes = [I64, I32, I32]
    lib.calib_chunk_bytes.restype = I64
    return lib


def measure_ceilings(reps=5, buf_gib=4, pool_sweep=False):
    """Best rates this GPU reaches for the access patterns the kernels use
    (probes of libmsa_calib.so, timed with HIP events on the launch stream,
    median of `reps`): a streaming read and a streaming write of a 4 GiB
    buffer, and a gather of 4 KiB microblock units (two 2 KiB runs 8 KiB
    apart) from a 32 MiB K/V pool that stays in the Infinity Cache."""
    import torch
    lib = _calib_lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    nbytes = buf_gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    grids = (256 * 8, 256 * 32)
    sink = torch.zeros(max(grids) * 4, dtype=torch.int32, device="cuda")
    grid = grids[0]

    def timed(fn):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            assert fn() == 0
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    out = {}
    variants = {}
    # writes: grid-stride / chunked non-temporal / chunked write-back
    for g in grids:
        for mode, name in ((0, "stride_nt"), (1, "chunk_nt"), (2, "chunk_wb")):
            nb = nbytes if mode == 0 else lib.calib_chunk_bytes(nbytes, g, 4)
            fn = lambda: lib.calib_write(buf.data_ptr(), nbytes, g, 7, mode, sp)
            timed(fn)
            variants[f"write_{name}_g{g}"] = round(nb / (timed(fn) * 1e-3) / 1e9, 1)
    for g in grids:
        for mode, name in ((0, "stride_nt"), (1, "chunk_nt")):
            nb = nbytes if mode == 0 else lib.calib_chunk_bytes(nbytes, g, 8)
            fn = lambda: lib.calib_read(buf.data_ptr(), nbytes, sink.data_ptr(), g, mode, sp)
            variants[f"read_{name}_g{g}"] = round(nb / (timed(fn) * 1e-3) / 1e9, 1)
    out["hbm_write_gbs"] = max(v for k, v in variants.items() if k.startswith("write"))
    out["hbm_read_gbs"] = max(v for k, v in variants.items() if k.startswith("read"))
    out["variants"] = variants
    del buf
    if pool_sweep:
        # DRAM read and write streams at once, 1 : 6 (the page attention's
        # L2-miss read : write bytes on the 16K Q8KV4 layer).  Not a ceiling of
        # that kernel: its reads are mostly Infinity-Cache hits, and it moves
        # more than this.
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty(3 << 30, dtype=torch.uint8, device="cuda")
        best = 0.0
        for g in grids:
            iters = src.numel() // (g * 8192)
            fn = lambda: lib.calib_mixed(src.data_ptr(), src.numel(), dst.data_ptr(), dst.numel(),
                                         sink.data_ptr(), g, iters, 6, sp)
            timed(fn)
            nb = g * iters * 8192 * 7
            best = max(best, nb / (timed(fn) * 1e-3) / 1e9)
        out["hbm_mixed_1r6w_gbs"] = round(best, 1)
        del src, dst
    rng = np.random.default_rng(9)
    n_units = 1 << 20                           # 4 GiB of 4 KiB units

    def gather(pool_mib, upis):
        pool_blocks = pool_mib * 64             # 16 KiB blocks (16 K rows + 16 V rows)
        pool = torch.randint(0, 255, (pool_blocks * 16384,), dtype=torch.uint8, device="cuda")
        units = torch.from_numpy(rng.integers(0, pool_blocks * 4, n_units).astype(np.int32)).cuda()
        res = {}
        for upi in upis:
            ms = timed(lambda: lib.calib_gather(pool.data_ptr(), pool.numel(), units.data_ptr(),
                                                n_units, sink.data_ptr(), grid, upi, sp))
            res[upi] = n_units * 4096 / (ms * 1e-3) / 1e9
        return res

    # the grouped route's K/V cache size class: 32 MiB (Infinity-Cache resident)
    res = gather(32, (2, 4, 8))
    for upi, gbs in res.items():
        out[f"gather_4k_upi{upi}_gbs"] = round(gbs, 1)
    out["gather_4k_gbs"] = round(max(res.values()), 1)
    # and from a 2 MiB pool, which every XCD's 4 MB L2 holds: the rate of the
    # gathers that hit in L2
    out["gather_4k_l2_gbs"] = round(max(gather(2, (4, 8)).values()), 1)
    # LDS reads of the grouped attention kernel's operands (bytes per clock and
    # CU at the 2.4 GHz peak engine clock; each launch reads 16 KiB per wave
    # and iteration, two 4-wave workgroups per CU)
    lds_grid, lds_iters = 512, 2000
    lds_sink = torch.zeros(lds_grid * 256, dtype=torch.int32, device="cuda")
    lds_bytes = lds_grid * 4 * lds_iters * 16384
    lds = {}
    for mode, name in ((0, "k_frag_b128_bitrev"), (3, "k_frag_b128_rowidx"), (1, "v_frag_tr_b64"),
                       (2, "consecutive_b128")):
        fn = lambda: lib.calib_lds(lds_sink.data_ptr(), lds_grid, lds_iters, mode, sp)
        timed(fn)
        lds[name] = round(lds_bytes / (timed(fn) * 1e-3) / 256 / 2.4e9, 1)
    out["lds_read_bytes_per_clk_cu"] = lds
    if pool_sweep:  # where the gather rate comes from: L2-, cache- or HBM-resident pools
        out["gather_4k_by_pool_mib"] = {m: round(max(gather(m, (4, 8)).values()), 1)
                                        for m in (2, 8, 32, 128, 1024)}
    out["method"] = ("libmsa_calib.so probes, median of %d launches, best variant: 16-byte "
                     "read / write of %d GiB (grid-stride or one chunk per workgroup, %s "
                     "workgroups; writes non-temporal or write-back); 4 KiB-unit gather from a "
                     "32 MiB pool (and from a 2 MiB, L2-resident one), %d units, 2/4/8 units in "
                     "flight per 256-thread workgroup, %d workgroups; LDS operand reads of the "
                     "grouped kernel, 2 x 4 waves per CU"
                     % (reps, buf_gib, "/".join(map(str, grids)), n_units, grid))
    return out


def lds_patterns(reps=5):
    """LDS read throughput (bytes per clock and CU at 2.4 GHz, two 4-wave
    workgroups per CU) of the kernels' MFMA operand reads, each K tile under
    the XOR swizzle it uses and under the one it replaced (calib_lds_pattern;
    the lane offsets follow the kernels' LDS layouts).  Lane l = n + 16 q
    reads A-operand row n; a K row's 16-byte chunk c sits at c ^ swz(row)."""
    import ctypes
    import torch
    lib = _calib_lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    grid, iters = 512, 2000
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    lanes = [(l & 15, l >> 4) for l in range(64)]
    brev4 = lambda x: int("{:04b}".format(x & 15)[::-1], 2)
    # page kernel, 16-bit and FP8 routes: key of A-operand row m in key tile t
    key_of = lambda t, m: (t >> 1) * 32 + (m >> 2) * 8 + (t & 1) * 4 + (m & 3)

    def grouped_k(sw):  # 512-byte rows, 32 per stage, chunk 8 q + c
        return [[n * 512 + (((8 * q + c) ^ sw(n)) << 4) + tile * 8192 for n, q in lanes]
                for tile in range(2) for c in range(8)]

    def page_k(rb, sw):  # rows of rb bytes at key_of, chunk (rb / 64) q + c
        lch = rb // 64
        return [[key_of(t, n) * rb + (((lch * q + c) ^ sw(n)) << 4) for n, q in lanes]
                for t in range(16 // lch) for c in range(lch)][:16]

    def page_f32_k(sw):  # 256-byte rows (d 64), keys 16 t + n, chunk 4 q + c
        return [[(t * 16 + n) * 256 + (((4 * q + c) ^ sw(n)) << 4) for n, q in lanes]
                for t in range(4) for c in range(4)]

    def index_k(sw):  # 128-byte rows, keys 16 t + n, chunk 2 q + c
        return [[(t * 16 + n) * 128 + (((2 * q + c) ^ sw(t * 16 + n)) << 4) for n, q in lanes]
                for t in range(8) for c in range(2)]

    def page_vt():  # V^T rows of 256 bytes (128 keys), row 16 mt + n, chunk (4 kb + q) ^ (row & 15)
        return [[(mt * 16 + n) * 256 + (((4 * kb + q) ^ n) << 4) for n, q in lanes]
                for kb in range(2) for mt in range(8)]

    def grouped_vtr():  # transposed reads of V rows (512 bytes), swizzle 2 (row & 7)
        out = []
        for tile in range(2):
            for mt in range(8):
                row = []
                for l in range(64):
                    vr, vc = (l >> 4) * 4 + ((l >> 2) & 3), l & 3
                    row.append(tile * 8192 + vr * 512 + ((((mt ^ (vr & 7)) << 1) + (vc >> 1)) << 4) + (vc & 1) * 8)
                out.append(row)
        return out

    pats = {
        "consecutive_b128": (0, [[k * 1024 + l * 16 for l in range(64)] for k in range(16)]),
        "grouped_k_d256_bitrev (used)": (0, grouped_k(brev4)),
        "grouped_k_d256_rowidx": (0, grouped_k(lambda n: n)),
        "page_k_fp8_d128 (r^r>>3)&7 (used)": (0, page_k(128, lambda r: (r ^ (r >> 3)) & 7)),
        "page_k_fp8_d128 r>>1": (0, page_k(128, lambda r: r >> 1)),
        "page_k_16bit_d128 (r&3)<<2|r>>2 (used)": (0, page_k(256, lambda r: ((r & 3) << 2) | (r >> 2))),
        "page_k_16bit_d128 r": (0, page_k(256, lambda r: r)),
        "page_k_f32_d64 bitrev (used)": (0, page_f32_k(brev4)),
        "page_k_f32_d64 r": (0, page_f32_k(lambda r: r)),
        "index_k_d128 (k&7)^5(k>>3&1) (used)": (0, index_k(lambda k: (k & 7) ^ (((k >> 3) & 1) * 5))),
        "index_k_d128 k&7": (0, index_k(lambda k: k & 7)),
        "page_vt_b128 (used)": (0, page_vt()),
        "grouped_v_tr_b64 (used)": (1, grouped_vtr()),
    }
    res = {}
    for name, (kind, tab) in pats.items():
        t = np.asarray(tab, dtype=np.int64)
        assert t.shape == (16, 64) and t.max() < 65536 and (t % (16 if kind == 0 else 8) == 0).all(), name
        dev = torch.from_numpy(t.astype(np.int32)).cuda()
        fn = lambda: lib.calib_lds_pattern(sink.data_ptr(), grid, iters, dev.data_ptr(), kind, sp)
        for _ in range(2):
            assert fn() == 0
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            assert fn() == 0
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        nbytes = grid * 4 * iters * 16 * (1024 if kind == 0 else 512)
        res[name] = round(nbytes / (float(np.median(ts)) * 1e-3) / 256 / 2.4e9, 1)
    return res


def cpu_info():
    """Host the CPU baseline ran on: model, logical CPUs and affinity mask."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    aff = sorted(os.sched_getaffinity(0))
    ranges, start = [], None
    for i, c in enumerate(aff):
        if start is None:
            start = c
        if i + 1 == len(aff) or aff[i + 1] != c + 1:
            ranges.append(f"{start}-{c}" if c != start else f"{c}")
            start = None
    return dict(cpu_model=model, nproc=os.cpu_count(), affinity=",".join(ranges))


KERNEL_SOURCES = {"k1_page_attend": "attend_page.hip", "combine_kernel": "combine.hip",
                  "k_grouped_attend": "attend_grouped.hip"}


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this workload, or None when there is none or the kernel's sources
    changed since the counters were taken (hash recorded beside the figure)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "common.h", "launch.h"):
        with open(os.path.join(ROOT, "block_sparse_paged_table_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    for line in open(path):
        parts = line.split()
        if len(parts) == 4 and parts[0] == "traffic:" and parts[1] == kernel:
            return int(parts[2]) if parts[3] == h.hexdigest() else None
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--sets", type=int, default=4,
                    help="rotated input sets (4: the queries and caches of the set in use "
                         "are not left in the 256 MB Infinity Cache by the previous steps)")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens for the CPU oracle leg (0: the whole layer)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kv-dtype", choices=["nvfp4", "e4m3"], default=None,
                    help="cache dtype variant of the Q8 workloads (e4m3: the Q8KV8 route)")
    ap.add_argument("--partial-dtype", choices=["f32", "bf16", "f16"], default="f32",
                    help="partial_o storage (the workloads specify f32)")
    ap.add_argument("--partial-layout", choices=["row", "split"], default="row",
                    help="partial_o layout, through the ABI's split / row strides: "
                         "[row][split][d] (each row's splits one contiguous run, which the "
                         "combine reads in order) or [split][row][d]")
    ap.add_argument("--index", action="store_true",
                    help="time the paged prefill indexer (page scores + top-k) instead")
    ap.add_argument("--index-workload", choices=["16k", "short_batch"], default="16k",
                    help="indexer workload: the 16K-token request, or 8 short chunks over long contexts")
    ap.add_argument("--workload", choices=["page4_small_chunk"], default=None,
                    help="a named workload instead of --config (page4_small_chunk: 48 rows, "
                         "512 microblocks per row in splits, the split-k microblock route)")
    ap.add_argument("--slots-per-split", type=int, default=0,
                    help="microblock workloads: slots merged into one split (0 = the workload's)")
    ap.add_argument("--slice-tokens", type=int, default=0,
                    help="order_slice_tokens of the descriptor (0 = chosen by the library)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times), to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters against known bytes")
    ap.add_argument("--lds-patterns", action="store_true",
                    help="measure the LDS read throughput of the kernels' operand read patterns "
                         "under their K-tile swizzles and print it as JSON")
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph",
                    help="timed steps replayed from HIP graphs captured per input set (default), "
                         "or launched kernel by kernel; per-kernel times always come from an "
                         "eager pass with events")
    ap.add_argument("--calibrate", action="store_true",
                    help="only measure the ceilings (HBM read, HBM write, cache-resident "
                         "4 KiB gather, LDS operand reads) and print them as one JSON line")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the live ceiling measurement of the normal run")
    args = ap.parse_args()
    if args.calibrate:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps(measure_ceilings(pool_sweep=True)), flush=True)
        return
    if args.lds_patterns:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps({"lds_read_bytes_per_clk_cu": lds_patterns()}), flush=True)
        return
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "copies": 3}), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the method shards without exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.index:
        return bench_index(args)

    import torch
    from block_sparse_paged_table_amd import synth
    from block_sparse_paged_table_amd.runner import DeviceProblem

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = args.config
    if args.workload == "page4_small_chunk":
        log(f"generating {args.sets} input sets of {args.workload}")
        kw = {"slots_per_split": args.slots_per_split} if args.slots_per_split else {}
        probs = [synth.make_page4_small_chunk(seed=1005 + 100 * i, **kw) for i in range(args.sets)]
    else:
        log(f"generating {args.sets} input sets of config {cfg} ({synth.CONFIG_NAMES[cfg]})")
        probs = [synth.make_config(cfg, seed=1000 + cfg + 100 * i, kv_dtype=args.kv_dtype)
                 for i in range(args.sets)]
        if args.slots_per_split:
            if probs[0].unit_tokens == probs[0].page_size:
                sys.exit("--slots-per-split applies to microblock workloads only")
            probs = [dataclasses.replace(p, slots_per_split=args.slots_per_split) for p in probs]
    p0 = probs[0]
    st = workload_stats(p0)
    for p in probs[1:]:  # rotated sets share the output buffers: same geometry only
        assert (p.total_q, p.num_rows, p.num_splits, p.d_v) == \
            (p0.total_q, p0.num_rows, p0.num_splits, p0.d_v), "input sets differ in shape"
    # one partial buffer / output shared by all sets (the biggest allocations)
    pd = args.partial_dtype
    dps = [DeviceProblem(probs[0], order_slice_tokens=args.slice_tokens, partial_dtype=pd,
                         partial_layout=args.partial_layout)]
    for p in probs[1:]:
        dps.append(DeviceProblem(p, partial_o=dps[0].partial_o, partial_lse=dps[0].partial_lse,
                                 order_slice_tokens=args.slice_tokens, partial_dtype=pd))
    for dp in dps[1:]:
        dp.out, dp.lse = dps[0].out, dps[0].lse
    torch.cuda.synchronize()
    log("inputs resident; warmup")

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        dps[i % len(dps)].run()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        dp = dps[i % len(dps)]
        e = ev[i]
        e[0].record(stream)
        dp.plan()
        e[1].record(stream)
        dp.attend()
        e[2].record(stream)
        dp.combine()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel times: median of the K launches (the mean beside it)
    t_plan = [e[0].elapsed_time(e[1]) for e in ev]
    t_attn = [e[1].elapsed_time(e[2]) for e in ev]
    t_comb = [e[2].elapsed_time(e[3]) for e in ev]
    plan_ms, attn_ms, comb_ms = (float(np.median(t)) for t in (t_plan, t_attn, t_comb))
    step_ms = float(np.median([e[0].elapsed_time(e[3]) for e in ev]))
    means = {k: round(float(np.mean(t)), 4) for k, t in
             (("plan", t_plan), ("attention", t_attn), ("combine", t_comb))}
    ms_per_step = wall * 1e3 / K
    log(f"plan {plan_ms:.3f} ms, attention {attn_ms:.3f} ms, combine {comb_ms:.3f} ms (medians), "
        f"step(events) {step_ms:.3f} ms, step(wall) {ms_per_step:.3f} ms")
    ms_per_step_eager = ms_per_step
    if args.launch == "graph":
        # the same steps replayed from HIP graphs, one per input set (plan,
        # attention and combine captured from the library's own launches: no
        # allocation, no memset), so the step pays no per-kernel launch gaps
        graphs = []
        for dp in dps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                dp.plan()
                dp.attend()
                dp.combine()
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / K
        log(f"step(wall, graph replay) {ms_per_step:.3f} ms")
    ceil = None
    if not args.no_ceilings:
        log("measuring the read / write / gather ceilings")
        ceil = measure_ceilings()

    # algorithmic bytes per launch
    p, dp = p0, dps[0]
    S, rows, dv = p.num_splits, p.num_rows, p.d_v
    out_b = dp.out.element_size()
    kv_bytes = sum(tensor_bytes(t) for t in (dp.k, dp.v) if t is not None)
    kv_bytes += sum(tensor_bytes(t) for t in (dp.k_sf, dp.v_sf) if t is not None)
    cache_rows = p.num_phys_pages * p.page_size * p.Hkv
    kv_bytes = int(kv_bytes * min(1.0, st["touched_kv_rows"] / cache_rows))  # touched units only
    pe = dp.partial_o.element_size()
    wname = p.name + ("" if pd == "f32" else f"+{pd}_partials")
    if args.partial_layout == "split":
        wname += "+split_major_partials"
    if args.slots_per_split:
        wname += f"+{p.num_splits}_splits"
    attn_bytes = pe * dv * st["nonempty"] + 4 * st["nonempty"] + tensor_bytes(dp.q) + kv_bytes
    comb_bytes = pe * dv * st["nonempty"] + 4 * rows * S + out_b * rows * dv + 4 * rows
    attn_tflops = st["flops"] / (attn_ms * 1e-3) / 1e12
    attn_gbs = attn_bytes / (attn_ms * 1e-3) / 1e9
    comb_gbs = comb_bytes / (comb_ms * 1e-3) / 1e9
    mfma_dtype = {"e4m3": "fp8", "bf16": "bf16", "f16": "f16", "f32": "f32"}[p.q_dtype]
    dominant = "attention" if attn_ms >= comb_ms else "combine"
    grouped = p.unit_tokens != p.page_size
    # the grouped route gathers its units' K/V rows from a cache that stays on
    # chip: its binding ceiling is the cache-resident gather, not HBM
    gather_bytes = st["gathered_kv_bytes"]
    gather_gbs = gather_bytes / (attn_ms * 1e-3) / 1e9
    if dominant == "attention" and grouped:
        # The gathers are served by the L2 where they hit and by the Infinity
        # Cache where they miss: the ceiling is the measured gather rate of each
        # level, weighted by the kernel's own L2-miss bytes (its recorded
        # FETCH_SIZE + WRITE_SIZE traffic; the writes are a few percent).
        # Without a current record, the Infinity-Cache rate alone.
        traffic = recorded_traffic("k_grouped_attend", wname)
        peak, source = None, None
        if ceil and traffic is not None and traffic < gather_bytes:
            hit = gather_bytes - traffic
            t_floor = hit / (ceil["gather_4k_l2_gbs"] * 1e9) + traffic / (ceil["gather_4k_gbs"] * 1e9)
            peak = round(gather_bytes / t_floor / 1e9, 1)
            source = ("measured 4 KiB-unit gather ceilings, L2-resident (%.0f GB/s) for the %.2f GB "
                      "that hit in L2 and Infinity-Cache-resident (%.0f GB/s) for the %.2f GB that "
                      "miss (recorded L2-miss traffic)" % (ceil["gather_4k_l2_gbs"], hit / 1e9,
                                                           ceil["gather_4k_gbs"], traffic / 1e9))
        elif ceil:
            peak = ceil["gather_4k_gbs"]
            source = "measured 4 KiB-unit gather ceiling (Infinity-Cache resident)"
        roof = dict(kernel="k_grouped_attend", bound="gather", achieved=round(gather_gbs, 1),
                    peak=peak, unit="GB/s", frac=round(gather_gbs / peak, 4) if peak else None,
                    peak_source=source, traffic=traffic, alg_bytes=gather_bytes,
                    hbm_alg_bytes=attn_bytes,
                    mfma_frac=round(attn_tflops / MFMA_PEAK_TFLOPS[mfma_dtype], 4))
    elif dominant == "attention":
        roof = dict(kernel="k1_page_attend", bound="hbm", achieved=round(attn_gbs, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(attn_gbs / HBM_PEAK_GBS, 4),
                    traffic=recorded_traffic("k1_page_attend", wname), alg_bytes=attn_bytes)
        if ceil:  # its bytes are almost all partial writes
            roof.update(ceiling=ceil["hbm_write_gbs"], ceiling_kind="measured HBM write",
                        frac_of_ceiling=round(attn_gbs / ceil["hbm_write_gbs"], 4))

    else:
        roof = dict(kernel="combine_kernel", bound="hbm", achieved=round(comb_gbs, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(comb_gbs / HBM_PEAK_GBS, 4),
                    traffic=recorded_traffic("combine_kernel", wname), alg_bytes=comb_bytes)
        if ceil:
            roof.update(ceiling=ceil["hbm_read_gbs"], ceiling_kind="measured HBM read",
                        frac_of_ceiling=round(comb_gbs / ceil["hbm_read_gbs"], 4))

    cpu = None
    if not args.no_cpu:
        import oracle
        n = min(args.cpu_sample, p.total_q) if args.cpu_sample > 0 else p.total_q
        toks = np.linspace(0, p.total_q - 1, n).astype(np.int32)
        keep = oracle.make_keep(p)
        sub = workload_stats_subset(p, toks)
        log(f"CPU oracle on {n} tokens")
        t = time.perf_counter()
        # the layer's result: every split's partial and their combine, per row
        oracle.prefill_rows(p, toks, want_partials=False, want_single_pass=False, keep=keep)
        dt = time.perf_counter() - t
        cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
        what = "the whole layer" if n == p.total_q else f"{n} of {p.total_q} query tokens (evenly spaced)"
        cpu = dict(value=round(sub / dt / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
                   sample=f"{what}: all heads and slots, partials + combine; {dt:.2f} s, "
                          f"FP64 C oracle, OpenMP", seconds=round(dt, 2), **cpu_info())

    res = {
        "metric": "sparse-prefill attn TFLOP/s over selected tokens + combine HBM GB/s, 1 GPU",
        "value": round(st["flops"] / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": mfma_dtype, "data": "synthetic",
        "launch": {"timed": "hip_graph_replay" if args.launch == "graph" else "eager",
                   "ms_per_step_eager": round(ms_per_step_eager, 4),
                   "note": "per-kernel times and the roofline come from the eager pass's events"},
        "config": {"workload": wname,
                   "description": p.description, "partial_dtype": pd, "partial_layout": args.partial_layout, "total_q": p.total_q,
                   "Hq": p.Hq, "Hkv": p.Hkv, "head_dim": p.d_qk, "page_size": p.page_size,
                   "slots": p.num_slots, "splits": p.num_splits, "input_sets": len(dps)},
        "kernels_ms": {"plan": round(plan_ms, 4), "attention": round(attn_ms, 4),
                       "combine": round(comb_ms, 4), "stat": "median of the timed steps",
                       "mean": means},
        "ceilings": ceil,
        "attention": {"tflops": round(attn_tflops, 2),
                      "mfma_frac": round(attn_tflops / MFMA_PEAK_TFLOPS[mfma_dtype], 4),
                      "hbm_gbs": round(attn_gbs, 1), "alg_bytes": attn_bytes,
                      "gathered_kv_gbs": round(gather_gbs, 1) if grouped else None,
                      "flops": st["flops"], "visible_keys": st["n_visible"]},
        "combine": {"gbs": round(comb_gbs, 1), "hbm_frac": round(comb_gbs / HBM_PEAK_GBS, 4),
                    "alg_bytes": comb_bytes,
                    "read_ceiling_frac": round(comb_gbs / ceil["hbm_read_gbs"], 4) if ceil else None,
                    "traffic": recorded_traffic("combine_kernel", wname)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def index_visible_keys(ip):
    """(token, head) x visible key pairs the indexer scores."""
    pos = ip.q_pos.numpy().astype(np.int64)
    sl = ip.seq_lens.numpy().astype(np.int64)
    seq = ip.q_seq.numpy()
    last = np.where(pos >= 0, np.minimum(pos, sl[np.clip(seq, 0, len(sl) - 1)] - 1), -1)
    return int((last + 1).sum()) * ip.H


def bench_index(args):
    """The indexer workload: page scores + top-k per step, rotated inputs."""
    import torch
    from block_sparse_paged_table_amd import synth
    from block_sparse_paged_table_amd.runner import DeviceIndexProblem
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.index_workload == "short_batch":
        ips = [synth.make_index_short_batch(seed=2004 + 100 * i) for i in range(args.sets)]
    else:
        ips = [synth.make_index_problem(seed=2000 + 100 * i) for i in range(args.sets)]
    devs = [DeviceIndexProblem(ip) for ip in ips]
    ip = ips[0]
    for i in range(args.warmup):
        devs[i % len(devs)].run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        d = devs[i % len(devs)]
        ev[i][0].record(stream)
        d.scores_only()
        ev[i][1].record(stream)
        d.topk()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    tk_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms = wall * 1e3 / K
    nvis = index_visible_keys(ip)
    flops = 2.0 * ip.d * nvis
    score_bytes = ip.total_q * ip.H * ip.max_pages * 4
    sc_tflops = flops / (sc_ms * 1e-3) / 1e12
    log(f"scores {sc_ms:.4f} ms, top-k {tk_ms:.4f} ms, step(wall) {ms:.4f} ms")
    cpu = None
    if not args.no_cpu:
        import dataclasses
        import oracle
        n = min(args.cpu_sample // 4, ip.total_q)
        toks = np.linspace(0, ip.total_q - 1, n).astype(np.int64)
        sub = dataclasses.replace(ip, q=ip.q[toks], q_seq=ip.q_seq[toks], q_pos=ip.q_pos[toks])
        t = time.perf_counter()
        sc, _ = oracle.index_scores(sub)
        oracle.topk(sc, ip.top_k)
        dt = time.perf_counter() - t
        cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
        cpu = dict(value=round(2.0 * ip.d * index_visible_keys(sub) / dt / 1e12, 6), unit="TFLOP/s",
                   cores=cores, kind="oracle",
                   sample=f"{n} of {ip.total_q} query tokens (evenly spaced), all heads and pages; "
                          f"{dt:.2f} s, FP64 C oracle, OpenMP")
    res = {
        "metric": "prefill indexer page-score TFLOP/s over visible keys (scores + top-k), 1 GPU",
        "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": ip.name, "description": ip.description, "total_q": ip.total_q,
                   "heads": ip.H, "head_dim": ip.d, "page_size": ip.page_size,
                   "top_k": ip.top_k, "input_sets": len(devs)},
        "kernels_ms": {"scores": round(sc_ms, 4), "topk": round(tk_ms, 4)},
        "roofline": dict(kernel="k_index_scores", bound="mfma", achieved=round(sc_tflops, 2),
                         peak=MFMA_PEAK_TFLOPS["fp8"], unit="TFLOP/s",
                         frac=round(sc_tflops / MFMA_PEAK_TFLOPS["fp8"], 4), traffic=None,
                         alg_bytes=score_bytes + ip.q.numel() + ip.k_cache.numel()),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def workload_stats_subset(p, toks):
    import dataclasses
    import torch
    sub = dataclasses.replace(p, q=p.q[toks], q_seq=p.q_seq[toks], q_pos=p.q_pos[toks],
                              sel_idx=p.sel_idx[toks], sel_mask=p.sel_mask[toks])
    return workload_stats(sub)["flops"]


if __name__ == "__main__":
    main()
