"""Probe problems whose every partial output is known in closed form
(shared by the CPU pins of the oracle and the GPU probes of the kernels).

Keys are built so that, inside every split, the key with the highest
position dominates the softmax by a logit gap so large that every other
weight is exactly zero (in FP32 on the device, and in FP64 too: the gaps
exceed 745): each partial output is then the value row of the last key its
split sees.  Value rows encode where their key lives (request, logical page
or unit, offset, KV head), so a wrong page-table gather, a wrong slot ->
split placement, a wrong causal limit or a wrong microblock mask bit changes
the bits.  The expected rows are written down from the selections alone.

Page route, FP8 (MiniMax-AI/MSA PR 21, sections "K1" and "Build the prefill
for SM107"): E4M3 queries equal to 448 in every dimension; the key at
in-page offset o holds dimension values summing to o (2.0 in the first
o // 2 dimensions, 1.0 in the next one if o is odd); with sm_scale 2 the
logits are 896 o.  Value fields are small integers, exact in E4M3 (and, for
NVFP4, carried by a block scale times the code of 1.0).

Microblock route (1Cat-vLLM PR 387, section "Purpose"): FP16 queries
(1, 16, 512, 0, ...) against keys (64 (t mod 16), 64 ((t / 16) mod 32),
64 (t / 512), 0, ...) give the dot product 64 t at absolute position t,
exact in FP32; sm_scale 16 makes consecutive positions 1024 apart.
"""
import dataclasses

import numpy as np
import torch

from block_sparse_paged_table_amd import synth

E4M3 = torch.float8_e4m3fn


def e4m3_bytes(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(E4M3).view(torch.uint8).numpy()


def page_probe(kv_dtype, d, seed):
    p = synth.build_page_problem(
        name="fp8_probe", seed=seed, ctx_lens=[77, 0, 1000], chunk_lens=[500, 333, 260],
        page_size=128, Hq=8, Hkv=2, d=d, num_slots=6, q_dtype="e4m3", kv_dtype=kv_dtype,
        out_dtype="f32", pad_rows=3, shuffle_slots=True, extra_phys_pages=2)
    P, page, Hkv = p.num_phys_pages, p.page_size, p.Hkv
    # keys: dimension values summing to the in-page offset
    kval = np.zeros((P, page, Hkv, d), np.float32)
    for o in range(page):
        kval[:, o, :, :o // 2] = 2.0
        if o % 2:
            kval[:, o, :, o // 2] = 1.0
    # values: (request, logical page // 16, logical page % 16, offset // 16,
    # offset % 16, KV head) in six fields
    fields = np.zeros((P, page, Hkv, 6), np.float32)
    pt = p.page_table.numpy()
    for b in range(p.num_seqs):
        for lp in range(pt.shape[1]):
            ph = int(pt[b, lp])
            if ph >= 0:
                fields[ph, :, :, 0] = b
                fields[ph, :, :, 1] = lp // 16
                fields[ph, :, :, 2] = lp % 16
    fields[:, :, :, 3] = (np.arange(page) // 16)[None, :, None]
    fields[:, :, :, 4] = (np.arange(page) % 16)[None, :, None]
    fields[:, :, :, 5] = np.arange(Hkv)[None, None, :]
    fdims = [16 * i for i in range(6)] if kv_dtype == "nvfp4" else list(range(6))
    if kv_dtype == "nvfp4":
        # K: codes of 2.0 (0b0100) and 1.0 (0b0010), every block scale 1.0
        kc = np.where(kval == 2.0, 4, np.where(kval == 1.0, 2, 0)).astype(np.uint8)
        ksf = np.full((P, page, Hkv, d // 16), 0x38, np.uint8)
        # V: one element of code 1.0 per field block, the block scale = the field
        vc = np.zeros((P, page, Hkv, d), np.uint8)
        vsf = np.full((P, page, Hkv, d // 16), 0x38, np.uint8)
        for i, dim in enumerate(fdims):
            vc[..., dim] = 2
            vsf[..., dim // 16] = e4m3_bytes(fields[..., i])
        pack = lambda c: torch.from_numpy(np.ascontiguousarray(c[..., 0::2] | (c[..., 1::2] << 4)))
        p = dataclasses.replace(p, k_cache=pack(kc), v_cache=pack(vc), k_sf=torch.from_numpy(ksf),
                                v_sf=torch.from_numpy(vsf))
    else:
        vval = np.zeros((P, page, Hkv, d), np.float32)
        for i, dim in enumerate(fdims):
            vval[..., dim] = fields[..., i]
        p = dataclasses.replace(p, k_cache=torch.from_numpy(kval).to(E4M3),
                                v_cache=torch.from_numpy(vval).to(E4M3))
    q = torch.full(p.q.shape, 448.0).to(E4M3)
    return dataclasses.replace(p, q=q, q_scale=1.0, k_scale=1.0, v_scale=0.25, sm_scale=2.0), fdims


def expected_page_rows(p, fdims):
    """Expected partial row of every (token, KV head, slot): v_scale times the
    fields of the slot's last visible key, or None for an empty slot."""
    si, sm = p.sel_idx.numpy(), p.sel_mask.numpy()
    qpos, qseq, sl = p.q_pos.numpy(), p.q_seq.numpy(), p.seq_lens.numpy()
    page = p.page_size
    exp = {}
    for t in range(p.total_q):
        for g in range(p.Hkv):
            for j in range(p.num_slots):
                if sm[t, g, j] == 0 or qpos[t] < 0:
                    exp[t, g, j] = None
                    continue
                u = int(si[t, g, j])
                last = min(u * page + page - 1, int(qpos[t]), int(sl[qseq[t]]) - 1)
                if last < u * page:
                    exp[t, g, j] = None
                    continue
                off = last - u * page
                row = np.zeros(p.d_v, np.float32)
                for dim, f in zip(fdims, (qseq[t], u // 16, u % 16, off // 16, off % 16, g)):
                    row[dim] = f * p.v_scale
                exp[t, g, j] = row
    return exp


def mb_probe(seed, spp, **kw):
    args = dict(name="mb_probe", seed=seed, ctx_len=300, chunk_len=61, pad_rows=3, Hq=6, Hkv=2,
                d=128, num_slots=24, page_size=16, spare_pages=3, partial_mask_frac=0.3)
    args.update(kw)
    p = synth.build_microblock_problem(**args)
    base = p.k_cache._base if p.k_cache._base is not None else None
    P, page, Hkv, d = p.num_phys_pages, p.page_size, p.Hkv, p.d_qk
    kv = np.zeros((P, 2, page, Hkv, d), np.float32)
    pt = p.page_table.numpy()[0]
    for lp, ph in enumerate(pt):
        if ph < 0:
            continue
        t = lp * page + np.arange(page)
        kv[ph, 0, :, :, 0] = (64 * (t % 16))[:, None]
        kv[ph, 0, :, :, 1] = (64 * ((t // 16) % 32))[:, None]
        kv[ph, 0, :, :, 2] = (64 * (t // 512))[:, None]
        kv[ph, 1, :, :, 0] = (t % 16)[:, None]
        kv[ph, 1, :, :, 1] = ((t // 16) % 64)[:, None]
        kv[ph, 1, :, :, 2] = (t // 1024)[:, None]
        kv[ph, 1, :, :, 3] = np.arange(Hkv)[None, :]
    kvt = torch.from_numpy(kv).to(torch.float16)
    assert base is not None  # the builder's interleaved layout
    q = torch.zeros(p.q.shape, dtype=torch.float32)
    q[..., 0], q[..., 1], q[..., 2] = 1.0, 16.0, 512.0
    return dataclasses.replace(p, k_cache=kvt[:, 0], v_cache=kvt[:, 1], q=q.to(torch.float16),
                               sm_scale=16.0, slots_per_split=spp)


def expected_mb_rows(p):
    """Per (token, KV head, split): the fields of the highest visible position
    among the split's valid, first-occurrence units (mask bits, causal and
    tail rules), or None."""
    si, sm = p.sel_idx.numpy(), p.sel_mask.numpy()
    qpos, sl = p.q_pos.numpy(), int(p.seq_lens.numpy()[0])
    ut, S = p.unit_tokens, p.num_splits
    exp = {}
    for t in range(p.total_q):
        for g in range(p.Hkv):
            best = [-1] * S
            seen = set()
            for j in range(p.num_slots):
                if sm[t, g, j] == 0 or qpos[t] < 0:
                    continue
                u = int(si[t, g, j])
                if u in seen:
                    continue
                seen.add(u)
                for i in range(ut):
                    x = u * ut + i
                    if (sm[t, g, j] >> i) & 1 and x <= qpos[t] and x < sl:
                        best[j // p.slots_per_split] = max(best[j // p.slots_per_split], x)
            for s in range(S):
                if best[s] < 0:
                    exp[t, g, s] = None
                else:
                    x = best[s]
                    row = np.zeros(p.d_v, np.float32)
                    row[:4] = (x % 16, (x // 16) % 64, x // 1024, g)
                    exp[t, g, s] = row
    return exp
