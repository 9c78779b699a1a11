"""GPU parity tests for the standalone kernels, through the C ABI:
the exact NVFP4 dequantisation and the LSE combine."""
import numpy as np
import pytest
import torch

import block_sparse_paged_table_amd as msa
from block_sparse_paged_table_amd import synth
import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def test_device_supported():
    assert msa.msa_device_supported(0)


def _all_finite_pairs():
    """All 16 codes x 254 finite E4M3 scales, each pair repeated four times in
    a row so that element i = 4 * pair + pos reaches the device lookups at
    every position pos of a 4-code word."""
    scales = np.array([s for s in range(256) if s not in (0x7F, 0xFF)], np.uint8)
    cc, ss = np.meshgrid(np.arange(16, dtype=np.uint8), scales, indexing="ij")
    return np.repeat(cc.ravel(), 4), np.repeat(ss.ravel(), 4)


def test_nvfp4_dequant_exhaustive_bitexact():
    """K side (E4M3 operand of the QK product): all 4064 finite (code, scale)
    pairs at every lookup position, bit for bit (signed zeros, saturation
    beyond 448 included) against the oracle's exact rounding."""
    cc, ss = _all_finite_pairs()
    ref = oracle.nvfp4_dequant(cc, ss)
    codes = torch.from_numpy(cc.copy()).cuda()
    sc = torch.from_numpy(ss.copy()).cuda()
    out = torch.empty_like(codes)
    msa.msa_nvfp4_dequant_e4m3(codes, sc, out)
    got = out.cpu().numpy()
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, [(int(cc[i]), int(ss[i]), i % 4, int(got[i]), int(ref[i]))
                           for i in bad[:10]]


def test_nvfp4_dequant_f16_exhaustive_bitexact():
    """V side (FP16 operand of the PV product, converted through the FP16
    tables the attention kernel uses): all 4064 finite (code, scale) pairs at
    every lookup position equal the oracle's E4M3 rounding widened to FP16,
    bit for bit (signed zeros and saturation included)."""
    cc, ss = _all_finite_pairs()
    ref = oracle.e4m3_decode(oracle.nvfp4_dequant(cc, ss)).astype(np.float16).view(np.uint16)
    codes = torch.from_numpy(cc.copy()).cuda()
    sc = torch.from_numpy(ss.copy()).cuda()
    out = torch.empty(codes.shape, dtype=torch.int16, device="cuda")
    msa.msa_nvfp4_dequant_f16(codes, sc, out)
    got = out.cpu().numpy().view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, [(int(cc[i]), int(ss[i]), i % 4, hex(got[i]), hex(ref[i]))
                           for i in bad[:10]]
    # the K-side bytes decode to the same values
    k8 = torch.empty_like(codes)
    msa.msa_nvfp4_dequant_e4m3(codes, sc, k8)
    kv = oracle.e4m3_decode(k8.cpu().numpy()).astype(np.float16).view(np.uint16)
    assert np.array_equal(kv, got)


@pytest.mark.parametrize("S,rows,dv", [(1, 333, 128), (3, 1000, 64), (16, 4099, 128),
                                       (20, 517, 256), (7, 64, 512), (16, 100, 4)])
def test_combine_matches_oracle(S, rows, dv):
    po, pl = synth.random_partials(100 + S, S, rows, dv, empty_frac=0.2, all_empty_rows=4)
    ref_out, ref_lse = oracle.combine(po.numpy(), pl.numpy())
    po_d, pl_d = po.cuda(), pl.cuda()
    out32 = torch.empty((rows, dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    msa.msa_combine(po_d, pl_d, S, rows, dv, out32, lse)
    torch.cuda.synchronize()
    o, l = out32.cpu().numpy(), lse.cpu().numpy()
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), empty)
    assert np.all(o[empty] == 0.0) and not np.signbit(o[empty]).any()
    fin = ~empty
    assert np.abs(l[fin] - ref_lse[fin]).max() < 2e-6 * max(1.0, np.abs(ref_lse[fin]).max())
    assert np.abs(o[fin] - ref_out[fin]).max() < 2e-6 * max(1.0, np.abs(ref_out).max())
    # 16-bit outputs are the RNE conversion of the same FP32 result
    for dt in (torch.bfloat16, torch.float16):
        o16 = torch.empty((rows, dv), dtype=dt, device="cuda")
        msa.msa_combine(po_d, pl_d, S, rows, dv, o16)
        assert torch.equal(o16, out32.to(dt))


@pytest.mark.parametrize("S,rows,dv", [(16, 1000, 128), (3, 257, 64), (40, 130, 256)])
@pytest.mark.parametrize("pdt", [torch.float16, torch.bfloat16])
def test_combine_16bit_partials(S, rows, dv, pdt):
    """msa_combine_ex on BF16 / FP16 partials equals the oracle's combine of
    the same values widened to FP64, at FP32-combine accuracy."""
    po, pl = synth.random_partials(200 + S, S, rows, dv, empty_frac=0.2, all_empty_rows=3)
    po16 = po.to(pdt)
    ref_out, ref_lse = oracle.combine(po16.double().numpy(), pl.numpy())
    out = torch.empty((rows, dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    msa.msa_combine_ex(po16.cuda(), pl.cuda(), S, rows, dv, out, lse)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), empty)
    assert np.all(o[empty] == 0.0) and not np.signbit(o[empty]).any()
    fin = ~empty
    assert np.abs(l[fin] - ref_lse[fin]).max() < 2e-6 * max(1.0, np.abs(ref_lse[fin]).max())
    assert np.abs(o[fin] - ref_out[fin]).max() < 2e-6 * max(1.0, np.abs(ref_out).max())


def test_combine_strided_buffers():
    """Wider row pitch, a split stride larger than the slab, and an output
    pitch: other entries stay untouched."""
    S, rows, dv = 5, 301, 128
    po, pl = synth.random_partials(7, S, rows, dv)
    big = torch.full((S, rows + 9, dv + 32), 7.0, dtype=torch.float32, device="cuda")
    big[:, :rows, :dv] = po.cuda()
    plb = torch.full((S, rows + 5), 3.0, dtype=torch.float32, device="cuda")
    plb[:, :rows] = pl.cuda()
    out = torch.full((rows, dv + 64), -5.0, dtype=torch.bfloat16, device="cuda")
    msa.msa_combine(big, plb, S, rows, dv, out, None, po_split_stride=big.stride(0),
                    po_row_stride=big.stride(1), pl_split_stride=plb.stride(0),
                    out_row_stride=out.stride(0))
    ref = torch.empty((rows, dv), dtype=torch.bfloat16, device="cuda")
    msa.msa_combine(po.cuda(), pl.cuda(), S, rows, dv, ref)
    assert torch.equal(out[:, :dv], ref)
    assert torch.all(out[:, dv:] == -5.0)


def test_combine_deterministic_repeat():
    S, rows, dv = 16, 2048, 128
    po, pl = synth.random_partials(9, S, rows, dv)
    po_d, pl_d = po.cuda(), pl.cuda()
    outs = []
    for _ in range(3):
        o = torch.empty((rows, dv), dtype=torch.float32, device="cuda")
        msa.msa_combine(po_d, pl_d, S, rows, dv, o)
        outs.append(o)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
