"""CPU pins of the NVFP4 oracle's two quotients, each rounded once from its exact value.

"混合精度与 FP8 训练" (hs-black.github.io) section 13.2: a block of 16 takes the scale amax/6
stored in E4M3, every element is divided by the stored block scale and rounded to E2M1, and an fp32
tensor scale S_t extends E4M3's range. The oracle's reading (R17): e_b = E4M3(amax_b * S_t / 6) and
code = E2M1(x * S_t / decode(e_b)), each the nearest value of the exact quotient with ties to the
even code.

The reference here is a brute-force search over exact rationals (fractions.Fraction): every
non-negative value of the format is tried and the nearest one taken, ties to the even code; nothing
of the oracle's binary search or midpoint test is reused. The separating cases are inputs whose
exact quotient lies within 2^-24 (relative) of a midpoint, where rounding the quotient to fp32
first (or multiplying by a rounded reciprocal) lands on the midpoint and the tie goes the other way.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

f32 = np.float32
MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]       # between consecutive E2M1 values


def nearest_code(fmt, q):
    """Code of the format value nearest to the rational |q| (ties: the even code)."""
    n = 8 if fmt == O.E2M1 else 127
    a = abs(q)
    best, best_d = None, None
    for c in range(n):
        d = abs(a - Fraction(O.decode(fmt, c)))
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def exact_element(x, s_t, e):
    dec = Fraction(O.decode(O.E4M3, e))
    sign = 8 if np.signbit(x) else 0
    if dec == 0:
        return sign
    return sign | nearest_code(O.E2M1, Fraction(float(x)) * Fraction(float(s_t)) / dec)


def exact_block(amax_b, s_t):
    return nearest_code(O.E4M3, Fraction(float(amax_b)) * Fraction(float(s_t)) / 6)


def test_tie_from_the_definition():
    """x / decode(e_b) = 1.25 exactly (S_t = 1): the tie between 1.0 and 1.5 goes to 1.0 (code 2).
    Multiplying by fl32(1 / decode(e_b)) instead lands above 1.25 and gives 1.5."""
    e = O.encode(O.E4M3, 15 / 512)
    assert O.decode(O.E4M3, e) == 15 / 512
    x = 75 / 2048                                  # 1.25 * 15/512, exact in BF16 and fp32
    assert O.nvfp4_element(x, 1.0, e) == 2 == exact_element(f32(x), f32(1.0), e)
    r = f32(f32(1.0) / f32(15 / 512))
    assert O.encode(O.E2M1, float(f32(f32(x) * r))) == 3   # the reciprocal form rounds twice


@pytest.mark.parametrize("m", MIDPOINTS)
def test_every_midpoint_tie_goes_to_the_even_code(m):
    lower = MIDPOINTS.index(m)                     # the midpoint lies between codes lower, lower + 1
    even = lower if lower % 2 == 0 else lower + 1
    for e in (1, 7, 8, 23, 56, 100, 0x7E):        # subnormal, normal and the largest block scales
        dec = O.decode(O.E4M3, e)
        x = f32(m * dec)                           # 3 x 4 significant bits: exact
        assert float(x) == m * dec
        assert O.nvfp4_element(float(x), 1.0, e) == even == exact_element(x, f32(1.0), e), (m, e)
        assert O.nvfp4_element(-float(x), 1.0, e) == 8 | even, (m, e)
        # one fp32 step either side leaves the tie
        up, dn = np.nextafter(x, f32(np.inf)), np.nextafter(x, f32(0))
        assert O.nvfp4_element(float(up), 1.0, e) == lower + 1 == exact_element(up, f32(1.0), e), (m, e)
        assert O.nvfp4_element(float(dn), 1.0, e) == lower == exact_element(dn, f32(1.0), e), (m, e)


def test_elements_near_midpoints_under_tensor_scales():
    """x * S_t / decode(e_b) within a few fp32 steps of each midpoint, for random tensor scales:
    the oracle equals the brute force every time, and at least one input separates it from the
    two-rounding form fl32(x * fl32(S_t / decode(e_b)))."""
    rng = np.random.default_rng(5)
    separated = 0
    for _ in range(1500):
        A = f32(rng.uniform(1, 2) * 2.0 ** int(rng.integers(-6, 6)))
        s_t = O.nvfp4_tensor_scale(float(A))
        e = int(rng.integers(1, 127))
        dec = O.decode(O.E4M3, e)
        x0 = f32(MIDPOINTS[int(rng.integers(0, 7))] * dec / float(s_t))
        for x in (np.nextafter(np.nextafter(x0, f32(0)), f32(0)), np.nextafter(x0, f32(0)), x0,
                  np.nextafter(x0, f32(np.inf))):
            x = f32(x)
            got = O.nvfp4_element(float(x), s_t, e)
            assert got == exact_element(x, s_t, e), (float(x), s_t, e)
            two = O.encode(O.E2M1, float(f32(x * f32(f32(s_t) / f32(dec)))))
            separated += two != got
    assert separated > 0


# (tensor amax, block amax): amax_b * S_t / 6 lies within 2^-24 of an E4M3 midpoint; found by a
# search over fp32 inputs, checked here against the brute force
BLOCK_CASES = [(1.6369616985321045, 0.001941151567734778),      # 0.5312500026 -> 0.5625 (code 49)
               (14.52682876586914, 0.0015832987846806645),      # 0.0488281274 -> code 21
               (110.69795227050781, 0.055982157588005066)]      # 0.2265625107 -> code 39


@pytest.mark.parametrize("A,a", BLOCK_CASES)
def test_block_scale_rounds_once(A, a):
    A, a = f32(A), f32(a)
    s_t = O.nvfp4_tensor_scale(float(A))
    assert s_t == f32(f32(2688.0) / A)
    e = O.nvfp4_block(float(a), s_t)
    assert e == exact_block(a, s_t)
    two = O.encode(O.E4M3, float(min(f32(f32(a / f32(6.0)) * s_t), f32(448.0))))
    assert two == e - 1                          # rounding amax_b / 6 to fp32 first lands on the tie


def test_block_scales_random_and_saturating():
    rng = np.random.default_rng(9)
    for _ in range(2000):
        A = f32(rng.uniform(1, 2) * 2.0 ** int(rng.integers(-40, 40)))
        s_t = O.nvfp4_tensor_scale(float(A))
        a = f32(float(A) * rng.uniform(0, 1.5) ** 3)   # some above A: the code saturates at 448
        assert O.nvfp4_block(float(a), s_t) == exact_block(a, s_t), (float(A), float(a))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_whole_tensor_against_brute_force(dtype):
    """Every block code and every element code of a small tensor with a wide spread of block
    magnitudes (so some block scales are E4M3 subnormals or zero) equals the brute force."""
    rng = np.random.default_rng(11 if dtype == "fp32" else 12)
    v = (rng.standard_normal((6, 64)) * np.exp(rng.uniform(-14, 4, (6, 4))).repeat(16, axis=1)).astype(np.float32)
    if dtype == "bf16":
        from synthetic import bf16_bits
        x = bf16_bits(v)
        xv = (x.astype(np.uint32) << 16).view(np.float32)
    else:
        x, xv = v, v
    q, s_blk, s_t, a, nf = O.quantize_nvfp4(x)
    assert nf == 0 and a == np.abs(xv).max() and s_t == O.nvfp4_tensor_scale(float(a))
    codes = O.unpack_fp4(q)
    for r in range(xv.shape[0]):
        for g in range(xv.shape[1] // 16):
            blk = xv[r, 16 * g:16 * g + 16]
            e = exact_block(np.abs(blk).max(), s_t)
            assert s_blk[r, g] == e, (r, g)
            for k in range(16):
                assert codes[r, 16 * g + k] == exact_element(blk[k], s_t, e), (r, g, k)
