"""Oracle number formats pinned to the pages' fixed facts and to brute force over all codes.

Pins: "混合精度与 FP8 训练" sections 2.2, 3 and 8.1; Ascend 950 format guide section 2.1;
"NVIDIA：Blackwell GPU MXFP8 预训练最佳实践" section 4.2; torch's own fp8 decoders (library).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

E4M3, E5M2, E8M0 = O.E4M3, O.E5M2, O.E8M0


def all_decoded(fmt):
    return np.array([O.decode(fmt, c) for c in range(256)])


def finite_nonneg(fmt):
    v = all_decoded(fmt)[:128]
    return v[np.isfinite(v)]


@pytest.fixture(scope="module")
def facts(golden_dir):
    with open(os.path.join(golden_dir, "w3_format_facts.json")) as f:
        return json.load(f)


def test_decode_matches_torch_for_all_codes():
    for fmt, dt in ((E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)):
        codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
        ref = codes.view(dt).to(torch.float64).numpy()
        ours = all_decoded(fmt)
        nan_ref, nan_ours = np.isnan(ref), np.isnan(ours)
        assert np.array_equal(nan_ref, nan_ours)
        assert np.array_equal(ref[~nan_ref], ours[~nan_ours])
        # signed zero survives
        assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e8m0_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = all_decoded(E8M0)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], ours[:255])
    assert ours[0] == 2.0 ** -127 and ours[127] == 1.0 and ours[254] == 2.0 ** 127


def test_counts_and_ascending_codes():
    # E4M3: 0x00..0x7E finite (0x7F is the single NaN); E5M2: 0x00..0x7B finite (0x7C inf).
    assert O.num_finite_nonneg(E4M3) == 127
    assert O.num_finite_nonneg(E5M2) == 124
    for fmt in (E4M3, E5M2):
        v = finite_nonneg(fmt)
        assert len(v) == O.num_finite_nonneg(fmt)
        assert np.all(np.diff(v) > 0), "codes must ascend with value"


def test_special_codes():
    d4 = all_decoded(E4M3)
    nan4 = [c for c in range(256) if np.isnan(d4[c])]
    assert nan4 == [0x7F, 0xFF]                     # only S.1111.111
    assert not np.any(np.isinf(d4))                 # no infinities
    d5 = all_decoded(E5M2)
    assert d5[0x7C] == np.inf and d5[0xFC] == -np.inf
    assert [c for c in range(256) if np.isnan(d5[c])] == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]


def test_e4m3_range_facts(facts):
    f = facts["e4m3"]
    v = finite_nonneg(E4M3)
    assert O.max_finite(E4M3) == f["max"] == v[-1] == O.decode(E4M3, 0x7E)
    assert v[1] == f["min_subnormal"] == 2.0 ** -9
    normals = v[v >= 2.0 ** -6]
    assert normals[0] == f["min_normal"]
    top = v[v >= 256]
    assert list(top) == f["top_binade_values"]       # the 7 values the all-ones exponent adds
    # without the all-ones exponent the maximum would be 240 (IEEE-style E4M3)
    assert v[v < 256][-1] == f["max_without_top_binade"]
    assert abs(math.log2(f["max"] / f["min_subnormal"]) - f["binades"]) < 0.01
    lo, hi = f["exponent_range"]
    exps = sorted({math.frexp(x)[1] - 1 for x in v[1:]})
    assert exps[0] == lo and exps[-1] == hi and len(exps) == hi - lo + 1 == 18


def test_e5m2_range_facts(facts):
    f = facts["e5m2"]
    v = finite_nonneg(E5M2)
    assert O.max_finite(E5M2) == v[-1] == 57344.0 == O.decode(E5M2, 0x7B)
    assert v[1] == 2.0 ** -16
    lo, hi = f["exponent_range"]
    exps = sorted({math.frexp(x)[1] - 1 for x in v[1:]})
    assert exps[0] == lo and exps[-1] == hi and len(exps) == 32
    b4 = math.log2(448 / 2.0 ** -9)
    b5 = math.log2(57344 / 2.0 ** -16)
    assert round(b5 / b4, 1) == f["binade_ratio_vs_e4m3"]


def test_values_per_binade(facts):
    for fmt, key in ((E4M3, "e4m3"), (E5M2, "e5m2")):
        v = finite_nonneg(fmt)
        per = facts[key]["values_per_binade"]
        mb = 3 if fmt == E4M3 else 2
        assert per == 2 ** mb
        for k in range(-6 if fmt == E4M3 else -14, 8 if fmt == E4M3 else 15):
            n = np.count_nonzero((v >= 2.0 ** k) & (v < 2.0 ** (k + 1)))
            assert n == per, (fmt, k, n)
        if fmt == E4M3:   # top binade [256, 512) holds 7 (the eighth pattern is NaN)
            assert np.count_nonzero(v >= 256) == 7


def test_interior_values_of_1_2(golden_dir):
    with open(os.path.join(golden_dir, "w2_interior_values.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(7)
    pts = rng.uniform(1.0, 2.0, g["points"])
    for fmt, want in ((E4M3, g["e4m3_interior"]), (E5M2, None)):
        landed = sorted({O.decode(fmt, O.encode(fmt, p)) for p in pts})
        interior = [x for x in landed if 1.0 < x < 2.0]
        if want is not None:
            assert interior == want
        else:
            assert len(interior) == g["e5m2_interior_count"]
    b = g["binades_log2_max_over_min_subnormal"]
    assert round(math.log2(448 / 2.0 ** -9)) == b["e4m3"]
    assert round(math.log2(57344 / 2.0 ** -16)) == b["e5m2"]


def test_encode_decode_roundtrip_all_finite_codes():
    for fmt in (E4M3, E5M2):
        for c in range(256):
            v = O.decode(fmt, c)
            if not np.isfinite(v):
                continue
            assert O.encode(fmt, v) == c, (fmt, hex(c))
