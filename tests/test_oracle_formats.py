"""Pins for the oracle's number-format routines (CPU only).

Each check ties the oracle to something other than itself: PyTorch's
float8_e4m3fn cast (a library routine), IEEE half-precision multiplication in
numpy, closed-form values of the formats, and exhaustive enumeration.

Passage: MiniMax-AI/MSA PR 21, section "Build the prefill for SM107" -- an
NVFP4 element is an E2M1 code times an E4M3 scale; the product is exact in
FP16 and the only rounding is the final conversion to E4M3.
"""
import fractions

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.usefixtures("oracle_lib")

FINITE_SCALES = np.array([s for s in range(256) if s not in (0x7F, 0xFF)], np.uint8)


def _torch_f8(x_f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_for_all_codes(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle_lib.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_e4m3_closed_forms(oracle_lib):
    d = oracle_lib.e4m3_decode
    assert d([0x7E])[0] == 448.0            # largest finite
    assert d([0x01])[0] == 2.0 ** -9        # smallest subnormal
    assert d([0x07])[0] == 7 * 2.0 ** -9    # largest subnormal
    assert d([0x08])[0] == 2.0 ** -6        # smallest normal
    assert d([0x38])[0] == 1.0
    assert d([0x39])[0] == 1.125
    z = d([0x80])[0]
    assert z == 0.0 and np.signbit(z)
    assert np.isnan(d([0x7F])[0]) and np.isnan(d([0xFF])[0])


def test_e4m3_encode_roundtrip_and_ties(oracle_lib):
    codes = FINITE_SCALES
    vals = oracle_lib.e4m3_decode(codes)
    assert np.array_equal(oracle_lib.e4m3_encode(vals), codes)
    # midpoints between neighbouring non-negative codes go to the even code
    pos = vals[(codes < 0x7E)]
    nxt = oracle_lib.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    mids = (pos + nxt) / 2
    enc = oracle_lib.e4m3_encode(mids)
    lower = np.arange(0, 0x7E, dtype=np.uint8)
    expect = np.where(lower % 2 == 0, lower, lower + 1)
    assert np.array_equal(enc, expect)
    assert np.array_equal(oracle_lib.e4m3_encode(-mids), expect | 0x80)


def test_e4m3_encode_matches_torch_rne_in_range(oracle_lib):
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 40,
        (rng.random(5000).astype(np.float32) * 2 ** -6),       # subnormal range
        np.float32(448.0) * rng.random(2000).astype(np.float32),
    ])
    assert np.array_equal(oracle_lib.e4m3_encode(x.astype(np.float64)), _torch_f8(x))


def test_e4m3_encode_saturates(oracle_lib):
    e = oracle_lib.e4m3_encode
    assert list(e([449.0, 463.99, 464.0, 480.0, 1e9, np.inf])) == [0x7E] * 6
    assert list(e([-449.0, -1e9, -np.inf])) == [0xFE] * 3
    assert e([np.nan])[0] == 0x7F
    assert e([-0.0])[0] == 0x80 and e([-(2.0 ** -11)])[0] == 0x80


def test_e2m1_closed_forms(oracle_lib):
    mags = oracle_lib.e2m1_decode(np.arange(8, dtype=np.uint8))
    assert list(mags) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    neg = oracle_lib.e2m1_decode(np.arange(8, 16, dtype=np.uint8))
    assert list(neg) == [-m for m in mags]
    assert np.signbit(neg[0])


def _products(oracle_lib):
    codes = np.arange(16, dtype=np.uint8)
    e2 = oracle_lib.e2m1_decode(codes)
    sc = oracle_lib.e4m3_decode(FINITE_SCALES)
    return codes, e2, sc, e2[:, None] * sc[None, :]


def test_nvfp4_product_exact_in_fp16(oracle_lib):
    """Every code x finite-scale product is exact in IEEE half precision."""
    _, e2, sc, prod = _products(oracle_lib)
    f16 = (e2.astype(np.float16)[:, None] * sc.astype(np.float16)[None, :]).astype(np.float64)
    assert np.array_equal(f16, prod)
    assert np.array_equal(np.signbit(f16), np.signbit(prod))


def test_nvfp4_product_significant_bits(oracle_lib):
    """The product has at most 6 significant bits (fits FP16's 11)."""
    _, _, _, prod = _products(oracle_lib)

    def sig(x):
        n = fractions.Fraction(abs(float(x))).numerator
        while n and n % 2 == 0:
            n //= 2
        return n.bit_length()

    bits = np.vectorize(sig)(prod)
    assert bits.max() == 6


def test_nvfp4_dequant_exhaustive(oracle_lib):
    """All 16 x 254 (code, finite scale) pairs.

    (a) in-range products equal PyTorch's float8_e4m3fn cast of the exact
        product (library RNE);
    (b) the FP16-path result (round the FP16 product) equals the direct
        rounding of the exact product bit for bit, signed zeros included;
    (c) products beyond 448 saturate to +-448; there are 252 of them.
    """
    codes, e2, sc, prod = _products(oracle_lib)
    cc, ss = np.meshgrid(codes, FINITE_SCALES, indexing="ij")
    got = oracle_lib.nvfp4_dequant(cc, ss)
    inr = np.abs(prod) <= 448
    ref = _torch_f8(prod.astype(np.float32))
    assert np.array_equal(got[inr], ref[inr])
    f16 = (e2.astype(np.float16)[:, None] * sc.astype(np.float16)[None, :]).astype(np.float64)
    assert np.array_equal(oracle_lib.e4m3_encode(f16), got)
    over = ~inr
    assert over.sum() == 252
    assert np.all(got[over & (prod > 0)] == 0x7E)
    assert np.all(got[over & (prod < 0)] == 0xFE)
    # signed zero: code 8 (-0) times a scale is a zero whose sign is the XOR
    # of the two signs (IEEE product), kept through the rounding
    neg_scale = FINITE_SCALES >= 0x80
    assert np.all(got[8][~neg_scale] == 0x80) and np.all(got[8][neg_scale] == 0x00)
    assert np.all(got[0][~neg_scale] == 0x00) and np.all(got[0][neg_scale] == 0x80)
