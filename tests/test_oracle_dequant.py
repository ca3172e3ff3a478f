"""CPU pins of the oracle's dequantization and quantization error statistics.

What fixes them, from outside the oracle:
  * tests/golden/w4_scaling_example.json ("混合精度与 FP8 训练" section 8.1): the code 22 with
    S = 22400 de-scales to about 0.000982, a 1.8% error against 0.001;
  * tests/golden/w5_delayed_failure.json (same page, section 8.2.1): the saturated 448 with
    S = 22.4 de-scales to 20, and that element counts as saturated;
  * closed forms: with S = 2^k de-scaling is decode(q) * 2^-k exactly; an MX element is exactly
    decode(q) * 2^(byte-127); a value already on the scaled fp8 grid survives the round trip
    unchanged and contributes no noise;
  * the exact rational quotient decode(q)/S rounded to fp32 (Fraction arithmetic, no float
    division) for every code and random scales;
  * round to nearest even's error bound: relative error <= 2^-(m+1) for values in the normal
    range ("混合精度与 FP8 训练" sections 3 and 4.1);
  * torch's float32 -> bfloat16 conversion (round to nearest even) for the BF16 output;
  * exact rational sums (Fractions) for the signal and noise of small tensors, and counts
    enumerated directly; round-up MX never saturates ("NVIDIA：Blackwell GPU MXFP8 预训练最佳实践"
    section 4.1), OCP round-down saturates a block maximum exactly when its significand
    exceeds 1.75.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from synthetic import bf16_bits, bf16_to_f32, small_tensor

E4M3, E5M2 = O.E4M3, O.E5M2
FMTS = [E4M3, E5M2]
MBITS = {E4M3: 3, E5M2: 2}


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def finite_codes(fmt):
    return [c for c in range(256) if math.isfinite(O.decode(fmt, c))]


def f32_rne(fr):
    """The fp32 value nearest to the rational fr (ties to even), found from the two fp32
    neighbours of a first guess with exact Fraction distances."""
    if fr == 0:
        return np.float32(0.0)
    g = np.float32(float(fr))
    if not np.isfinite(g):
        return g
    cands = {g, np.nextafter(g, np.float32(np.inf)), np.nextafter(g, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - fr)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_worked_example_descale(golden_dir):
    g = load(golden_dir, "w4_scaling_example.json")
    code = O.encode(E4M3, g["scaled_e4m3_value"])
    deq = O.dequant_one(E4M3, code, np.float32(g["scale"]))
    assert round(deq, 6) == g["dequantized"]
    assert round(abs(deq - g["value"]) / g["value"] * 100, 1) == g["dequantized_relative_error_pct"]
    assert O.dequant_scaled(np.array([code], np.uint8), E4M3, g["scale"])[0] == np.float32(deq)


def test_worked_example_saturation(golden_dir):
    g = load(golden_dir, "w5_delayed_failure.json")
    s = np.float32(448 / g["history_amax"])
    x = np.array([g["spike"], 1.0, 0.0], np.float32)
    q = O.cast(x, E4M3, s)
    assert O.decode(E4M3, q[0]) == g["saturated"]
    xh = O.dequant_scaled(q, E4M3, s)
    assert round(float(xh[0]), 4) == g["dequantized"]
    st = O.stats_scaled(x, q, E4M3, s)
    assert st["saturated"] == 1 and st["count"] == 3 and st["nonzero"] == 2 and st["zeroed"] == 0
    # the spike keeps 20 of 50: 60% of it is lost
    assert round((g["spike"] - float(xh[0])) / g["spike"], 2) == 0.6


@pytest.mark.parametrize("fmt", FMTS)
def test_descale_power_of_two_is_exact(fmt):
    for k in range(-30, 31):
        s = np.float32(2.0 ** k)
        for c in range(256):
            v = O.decode(fmt, c)
            got = O.dequant_one(fmt, c, s)
            if math.isnan(v):
                assert math.isnan(got)
            else:
                assert got == np.float32(v * 2.0 ** -k), (fmt, c, k)


@pytest.mark.parametrize("fmt", FMTS)
def test_descale_equals_exact_rational_rounding(fmt):
    rng = np.random.default_rng(17)
    scales = (2.0 ** rng.uniform(-60, 60, 120)).astype(np.float32)
    scales = np.concatenate([scales, np.float32([22400.0, 22.4, 8.96, 3.0, 7.0, 1.0 / 3.0])])
    for s in scales:
        for c in finite_codes(fmt):
            want = f32_rne(Fraction(O.decode(fmt, c)) / Fraction(float(s)))
            assert O.dequant_one(fmt, c, s) == want, (fmt, c, float(s))


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_descale_closed_form(fmt):
    for b in range(256):
        for c in range(256):
            got = O.dequant_mx_one(fmt, c, b)
            v = O.decode(fmt, c)
            if b == 255 or math.isnan(v):
                assert math.isnan(got)
            else:
                with np.errstate(over="ignore"):
                    assert got == np.float32(math.ldexp(v, b - 127)), (fmt, c, b)
    q = np.arange(64, dtype=np.uint8).reshape(1, 64)
    s = np.array([[127 - 6, 130]], np.uint8)
    want = np.array([np.float32(math.ldexp(O.decode(fmt, c), -6 if c < 32 else 3)) for c in range(64)], np.float32)
    got = O.dequant_mx(q, s, fmt)[0]
    assert np.array_equal(got, want, equal_nan=True)


@pytest.mark.parametrize("fmt", FMTS)
def test_round_trip_on_the_grid(fmt):
    """Values already on the scaled fp8 grid come back unchanged, with zero noise."""
    for k in (-12, 0, 7):
        s = np.float32(2.0 ** k)
        x = np.array([O.decode(fmt, c) * 2.0 ** -k for c in finite_codes(fmt)], np.float32)
        q = O.cast(x, fmt, s)
        assert np.array_equal(O.dequant_scaled(q, fmt, s), x)
        st = O.stats_scaled(x, q, fmt, s)
        assert st["noise"] == 0.0 and st["zeroed"] == 0 and st["saturated"] == 0


@pytest.mark.parametrize("fmt", FMTS)
def test_round_trip_error_bound(fmt):
    """RNE: in the normal range the relative error of the scaled value is at most 2^-(m+1)."""
    x = bf16_to_f32(small_tensor(64, 512, seed=5))
    q, amax, s, _ = O.quantize_per_tensor(x, fmt)
    xh = O.dequant_scaled(q, fmt, s)
    y = (x.astype(np.float64) * np.float64(s)).astype(np.float32).astype(np.float64)   # fl32(x*S)
    tiny = {E4M3: 2.0 ** -6, E5M2: 2.0 ** -14}[fmt]                 # smallest normal value
    normal = (np.abs(y) >= tiny) & (np.abs(y) <= O.max_finite(fmt))
    dq = np.array([O.decode(fmt, c) for c in q.ravel()]).reshape(q.shape)
    rel = np.abs(dq[normal] - y[normal]) / np.abs(y[normal])
    assert rel.max() <= 2.0 ** -(MBITS[fmt] + 1)
    assert np.count_nonzero(normal) > 0.9 * x.size
    # and the de-scaled value is that code over S, rounded once to fp32
    assert np.array_equal(xh, (dq / np.float64(s)).astype(np.float32))


def test_bf16_output_matches_torch():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, 2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    edge = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000, 0x80008001, 0x3F808000,
                     0x3F818000, 0x00000001, 0x007FFFFF], np.uint32)
    f = np.concatenate([u, ties, edge]).view(np.float32)
    f = f[np.isfinite(f)]
    got = O.to_bf16(f)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert O.to_bf16(np.array([np.nan], np.float32))[0] & 0x7FFF > 0x7F80


def exact_stats(x64, xh):
    """Signal and noise as exact rationals, counts by enumeration."""
    fin = np.isfinite(x64)
    sig = sum(Fraction(float(v)) ** 2 for v in x64[fin])
    noi = sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(x64[fin], xh[fin].astype(np.float64)))
    nz = fin & (x64 != 0)
    return sig, noi, int(fin.sum()), int(nz.sum()), int((nz & (xh == 0)).sum()), int((~fin).sum())


def check_sums(st, sig, noi, n):
    tol = (n + 4) * 2.0 ** -52
    assert abs(st["signal"] - float(sig)) <= tol * float(sig) + 1e-300
    assert abs(st["noise"] - float(noi)) <= tol * max(float(noi), 1e-300) + 1e-300


@pytest.mark.parametrize("fmt", FMTS)
def test_stats_per_tensor_and_block_brute_force(fmt):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((37, 256)) * np.where(rng.random((37, 256)) < 0.05, 1e-10, 1.0)).astype(np.float32)
    x[3, :7] = 0.0
    x[5, 9] = np.inf
    x[6, 1] = np.nan
    xf = x.copy()
    xf[~np.isfinite(xf)] = 0.0
    q, amax, s, _ = O.quantize_per_tensor(xf, fmt)
    st = O.stats_scaled(x, q, fmt, s)
    xh = O.dequant_scaled(q, fmt, s)
    sig, noi, cnt, nz, zd, nf = exact_stats(x.astype(np.float64).ravel(), xh.ravel())
    assert (st["count"], st["nonzero"], st["zeroed"], st["nonfinite"]) == (cnt, nz, zd, nf) == (cnt, nz, zd, 2)
    assert st["zeroed"] > 0
    check_sums(st, sig, noi, cnt)
    qb, sb, _, _ = O.quantize_block(xf, 1, 128, fmt)
    stb = O.stats_block(x, qb, 1, 128, fmt, sb)
    xhb = O.dequant_block(qb, 1, 128, fmt, sb)
    sig, noi, cnt, nz, zd, nf = exact_stats(x.astype(np.float64).ravel(), xhb.ravel())
    assert (stb["count"], stb["nonzero"], stb["zeroed"], stb["nonfinite"]) == (cnt, nz, zd, nf)
    check_sums(stb, sig, noi, cnt)
    # finer groups lose less: the per-group result has less noise than the per-tensor one
    assert stb["noise"] < st["noise"]


@pytest.mark.parametrize("fmt", FMTS)
def test_stats_mx_saturation_rule(fmt):
    """Round-up never saturates; OCP round-down saturates a block maximum exactly when its
    significand exceeds 1.75 (and nothing else in a block whose other values are small)."""
    rng = np.random.default_rng(9)
    rows = 64
    x = (rng.standard_normal((rows, 32)) * 0.01).astype(np.float32)
    sig = rng.uniform(1.0, 2.0, rows).astype(np.float32)
    x[:, 0] = sig * np.float32(2.0 ** 3)
    xb = bf16_bits(x)
    top = bf16_to_f32(xb)[:, 0] / 8.0
    q_up, s_up, _, _, _ = O.quantize_mx(xb, fmt, O.ROUND_UP, col=False)
    assert O.stats_mx(xb, q_up, s_up, fmt)["saturated"] == 0
    q_dn, s_dn, _, _, _ = O.quantize_mx(xb, fmt, O.ROUND_DOWN, col=False)
    st = O.stats_mx(xb, q_dn, s_dn, fmt)
    assert st["saturated"] == int((top > 1.75).sum()) > 0
    xh = O.dequant_mx(q_dn, s_dn, fmt)
    s_, n_, cnt, nz, zd, nf = exact_stats(bf16_to_f32(xb).astype(np.float64).ravel(), xh.ravel())
    assert (st["count"], st["nonzero"], st["zeroed"], st["nonfinite"]) == (cnt, nz, zd, nf)
    check_sums(st, s_, n_, cnt)


def test_stats_degenerate():
    z = np.zeros((4, 64), np.float32)
    q = O.cast(z, E4M3, np.float32(1.0))
    st = O.stats_scaled(z, q, E4M3, 1.0)
    assert st == {"signal": 0.0, "noise": 0.0, "count": 256, "nonzero": 0, "zeroed": 0, "saturated": 0, "nonfinite": 0}
    # a value far below the grid is zeroed and is all noise
    x = np.array([[1e-12, 1.0]], np.float32)
    q = O.cast(x, E4M3, np.float32(1.0))
    st = O.stats_scaled(x, q, E4M3, 1.0)
    assert st["zeroed"] == 1 and st["nonzero"] == 2
    assert st["noise"] == float(np.float32(1e-12)) ** 2
