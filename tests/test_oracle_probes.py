"""The oracle against the closed-form probe problems of tests/probes.py:
every partial output of the FP8 page routes (E4M3 queries with an NVFP4 or
E4M3 cache) and of the microblock route (per-row 4-bit masks; one split,
one slot per split, and the split-k form) equals the value row of the last
visible key of its split, exactly, and every empty split has lse = -inf.
A dropped mask bit, an off-by-one causal limit, a wrong page-table lookup
or a wrong slot -> split mapping in the oracle fails here."""
import numpy as np
import pytest

import probes


def _check(p, exp, ref):
    G = p.Hq // p.Hkv
    n = 0
    for (t, g, s), row in exp.items():
        for hl in range(G):
            if row is None:
                assert np.isneginf(ref["part_lse"][t, g * G + hl, s]), (t, g, s)
            else:
                assert np.array_equal(ref["part_o"][t, g * G + hl, s], row), (t, g, s)
                n += 1
    return n


@pytest.mark.parametrize("kv_dtype,d", [("nvfp4", 128), ("e4m3", 128), ("e4m3", 64)])
def test_oracle_fp8_page_probe(oracle_lib, kv_dtype, d):
    p, fdims = probes.page_probe(kv_dtype, d, seed=51)
    ref = oracle_lib.prefill_rows(p, want_single_pass=False)
    assert ref["err"] == 0
    assert _check(p, probes.expected_page_rows(p, fdims), ref) > 20000


@pytest.mark.parametrize("spp", [1, 24, 6])
def test_oracle_microblock_probe(oracle_lib, spp):
    p = probes.mb_probe(61, spp)
    ref = oracle_lib.prefill_rows(p, want_single_pass=False)
    assert ref["err"] == 0
    assert _check(p, probes.expected_mb_rows(p), ref) > 300
