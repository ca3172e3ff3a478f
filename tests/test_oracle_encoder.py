"""Oracle encoder sat_rne8 and the scaled cast fl32(x*S) -> fp8.

Pins:
  * the 0.1 worked example ("混合精度与 FP8 训练" section 2.3, tests/golden/w1_point_one.json);
  * textbook round-to-nearest-even ties (same page, section 4.1);
  * exhaustive agreement over all 65536 BF16 inputs times a set of scales with (a) an
    independent bit-manipulation encoder written below and (b) torch's float8 casts, which
    round to nearest even but do not saturate, so they are fed values clamped to +-max first;
  * the RNE error bound: at most half a spacing for unsaturated values (section 3).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from synthetic import bf16_bits, bf16_to_f32

E4M3, E5M2 = O.E4M3, O.E5M2
FMT = {E4M3: dict(mbits=3, bias=7, maxbits=0x43E00000, maxcode=0x7E, max=448.0, torch=torch.float8_e4m3fn),
       E5M2: dict(mbits=2, bias=15, maxbits=0x47600000, maxcode=0x7B, max=57344.0, torch=torch.float8_e5m2)}


def bit_encoder(y, fmt):
    """Independent saturating RNE fp32 -> fp8 by integer manipulation of the fp32 bits."""
    p = FMT[fmt]
    u = np.ascontiguousarray(y, dtype=np.float32).view(np.uint32).astype(np.int64)
    sign = (u >> 24) & 0x80
    a = u & 0x7FFFFFFF
    mb, bias = p["mbits"], p["bias"]
    out = np.zeros(a.shape, np.int64)
    sat = a >= p["maxbits"]
    E = (a >> 23) - 127
    emin = 1 - bias
    normal = (~sat) & (E >= emin)
    sh = 23 - mb
    r = a + ((1 << (sh - 1)) - 1) + ((a >> sh) & 1)
    code_n = (r >> sh) - ((127 - bias) << mb)
    sub = (~sat) & (~normal) & (a >= 0x00800000)
    sig = (a & 0x7FFFFF) | 0x800000
    shift = np.clip(23 + emin - mb - E, 1, 40)
    q = sig >> shift
    rem = sig & ((np.int64(1) << shift) - 1)
    half = np.int64(1) << (shift - 1)
    q = q + ((rem > half) | ((rem == half) & ((q & 1) == 1)))
    out = np.where(sat, p["maxcode"], np.where(normal, code_n, np.where(sub, q, 0)))
    return (out | sign).astype(np.uint8)


def torch_encoder(y, fmt):
    p = FMT[fmt]
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).clamp(-p["max"], p["max"])
    return t.to(p["torch"]).view(torch.uint8).numpy()


def test_point_one_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "w1_point_one.json")) as f:
        g = json.load(f)
    # BF16 of 0.1 (pins the input generator's rounding): exponent field 123, mantissa 77
    b = int(bf16_bits(np.array([g["value"]], np.float32))[0])
    assert b >> 7 == g["bf16"]["exponent_field"] and b & 0x7F == g["bf16"]["mantissa_field"]
    assert float(bf16_to_f32(np.array([b], np.uint16))[0]) == g["bf16"]["value"]
    e4 = (g["e4m3"]["exponent_field"] << 3) | g["e4m3"]["mantissa_field"]
    for y in (g["value"], float(np.float32(g["value"])), g["bf16"]["value"]):
        assert O.encode(E4M3, y) == e4 == 0x1D
        assert O.encode(E5M2, y) == 0x2E
    assert O.decode(E4M3, 0x1D) == g["e4m3"]["value"]
    assert O.decode(E5M2, 0x2E) == g["e5m2"]["value"]
    assert O.decode(E5M2, 0x2E) == (1 + g["e5m2"]["mantissa_field"] / 4) * 2.0 ** -4
    assert round(abs(g["e4m3"]["value"] - 0.1) / 0.1 * 100, 1) == g["e4m3"]["relative_error_pct"]
    assert round(abs(g["e5m2"]["value"] - 0.1) / 0.1 * 100, 2) == g["e5m2"]["relative_error_pct"]


def test_ties_to_even():
    # midpoints between neighbours go to the code with an even mantissa
    assert O.encode(E4M3, 1.0625) == 0x38      # between 1.0 (0x38) and 1.125 (0x39)
    assert O.encode(E4M3, 1.1875) == 0x3A      # between 1.125 (0x39) and 1.25 (0x3A)
    assert O.encode(E4M3, 2.0 ** -10) == 0x00  # between 0 and 2^-9
    assert O.encode(E4M3, 3 * 2.0 ** -10) == 0x02
    assert O.encode(E4M3, -1.0625) == 0xB8
    assert O.encode(E5M2, 1.125) == 0x3C       # between 1.0 (0x3C) and 1.25 (0x3D)
    assert O.encode(E5M2, 1.375) == 0x3E
    assert O.encode(E4M3, 464.0) == 0x7E       # above max: saturates, never NaN
    assert O.encode(E5M2, 61440.0) == 0x7B
    assert O.encode(E4M3, float("inf")) == 0x7E and O.encode(E4M3, float("-inf")) == 0xFE


def test_signed_zero_and_underflow():
    assert O.encode(E4M3, -0.0) == 0x80
    assert O.encode(E4M3, -1e-6) == 0x80
    assert O.encode(E5M2, -1e-9) == 0x80
    assert O.encode(E4M3, 0.0) == 0x00


def test_nan_gives_nan_code():
    for fmt in (E4M3, E5M2):
        assert np.isnan(O.decode(fmt, O.encode(fmt, float("nan"))))


def _scale_set():
    rng = np.random.default_rng(11)
    s = [1.0, 22400.0, float(np.float32(448 / 20)), float(np.float32(448 / 50))]
    s += [2.0 ** -k for k in range(-127, 128)]
    s += list((2.0 ** rng.uniform(-40, 40, 1000)).astype(np.float32))
    return np.array(s, np.float32)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scaled_cast_exhaustive_bf16(fmt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f32(bits)
    ok = ~np.isnan(x)
    xb, xf = bits[ok], x[ok]
    for s in _scale_set():
        q = O.cast(xb, fmt, s)
        with np.errstate(over="ignore"):
            y = xf * np.float32(s)      # IEEE fp32 product, correctly rounded
        assert np.array_equal(q, bit_encoder(y, fmt)), s
        assert np.array_equal(q, torch_encoder(y, fmt)), s


def test_encoder_random_fp32_vs_independent():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    y = u.view(np.float32)
    y = y[np.isfinite(y)]
    for fmt in (E4M3, E5M2):
        q = O.encode_f32(fmt, y)
        assert np.array_equal(q, bit_encoder(y, fmt))
        assert np.array_equal(q, torch_encoder(y, fmt))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_error_at_most_half_spacing(fmt):
    rng = np.random.default_rng(3)
    mx = O.max_finite(fmt)
    y = (rng.uniform(-1, 1, 200_000) * mx).astype(np.float32)
    q = O.encode_f32(fmt, y)
    v = np.array([O.decode(fmt, c) for c in range(256)])
    got = v[q]
    fin = np.array(sorted(set(np.abs(v[np.isfinite(v)]))))
    idx = np.clip(np.searchsorted(fin, np.abs(y), side="right") - 1, 0, len(fin) - 2)
    spacing = fin[idx + 1] - fin[idx]
    assert np.all(np.abs(got - y) <= spacing / 2)
    mb = 3 if fmt == E4M3 else 2
    normal = np.abs(y) >= fin[np.searchsorted(fin, 2.0 ** (-6 if fmt == E4M3 else -14))]
    rel = np.abs(got - y)[normal] / np.abs(y)[normal]
    assert np.all(rel <= 2.0 ** -(mb + 1))
