"""CPU pins of the power-of-two group scales and the 1x128 -> 128x1 re-grouping
("混合精度与 FP8 训练" sections 10.4 and 10.5).

  * closed form of the power-of-two scale over every positive finite BF16 amax: S is a power of
    two, amax * S <= F8max and amax * 2S > F8max (unless S sits at the 2^127 clamp); the pages'
    MX example (amax 5.3, each element multiplied by 64) fixes 5.3 -> 64;
  * a tensor that is one group: the power-of-two block result equals the plain cast with that
    power of two;
  * the reason the pages give for power-of-two scales: re-grouping adds no error. Every element
    whose re-scaled value (its 1x128 value times its 128x1 scale) is in the normal fp8 range
    de-scales to exactly the value the 1x128 codes de-scaled to (only values pushed into the
    subnormal range can move); with Eq.(1) scales the same re-grouping changes many values;
  * the transposed layout: element (c, r) of the result belongs to element (r, c) of the input.
"""
import math

import numpy as np
import pytest

import oracle as O
from synthetic import bf16_to_f32, small_tensor, token_activation

E4M3, E5M2 = O.E4M3, O.E5M2
FMTS = [E4M3, E5M2]
MIN_NORMAL = {E4M3: 2.0 ** -6, E5M2: 2.0 ** -14}


@pytest.mark.parametrize("fmt", FMTS)
def test_pow2_scale_closed_form(fmt):
    f8max = O.max_finite(fmt)
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    amax = bf16_to_f32(bits).astype(np.float64)
    for a in amax:
        s = O.scale_pow2(fmt, a)
        m, e = math.frexp(s)
        assert m == 0.5, (a, s)                           # a power of two
        assert a * s <= f8max
        assert a * 2 * s > f8max or s == 2.0 ** 127
    assert O.scale_pow2(fmt, 0.0) == 1.0 and O.scale_pow2(fmt, float("inf")) == 1.0
    assert O.scale_pow2(E4M3, 5.3) == 64.0                # the pages' MX example: x 64


@pytest.mark.parametrize("fmt", FMTS)
def test_pow2_single_group_is_the_plain_cast(fmt):
    x = small_tensor(1, 128, seed=21)
    q, s, a, _ = O.quantize_block_ex(x, 1, 128, fmt, pow2=True)
    assert s.shape == (1, 1)
    assert s[0, 0] == O.scale_pow2(fmt, float(O.amax(x)))
    assert np.array_equal(q, O.cast(x, fmt, s[0, 0]))
    q1, s1, _, _ = O.quantize_block_ex(x, 1, 128, fmt, pow2=False)
    q2, s2, _, _ = O.quantize_block(x, 1, 128, fmt)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)   # pow2=False is quantize_block


def regroup(x, fmt, pow2):
    q, s, _, _ = O.quantize_block_ex(x, 1, 128, fmt, pow2=pow2)
    first = O.dequant_block(q, 1, 128, fmt, s)                   # what the 1x128 codes mean
    qT, sT, nf = O.requant_1x128_to_128x1(q, s, fmt, fmt, pow2)
    second = O.dequant_block(qT, 1, 128, fmt, sT)                # what the 128x1 codes mean
    return first, second, qT, sT


@pytest.mark.parametrize("fmt", FMTS)
def test_pow2_regrouping_adds_no_error(fmt):
    x = token_activation(384, 512, seed=7)
    first, second, qT, sT = regroup(x, fmt, pow2=True)
    assert qT.shape == (512, 384) and sT.shape == (512, 3)
    back = second.T
    s2 = np.repeat(sT, 128, axis=1)[:, :384].T                   # the 128x1 scale of each element
    normal = np.abs(first.astype(np.float64) * s2) >= MIN_NORMAL[fmt]   # re-scaled value is normal
    assert np.array_equal(back[normal], first[normal])
    assert normal.mean() > 0.9
    moved = ~normal & (back != first)
    assert np.all(np.abs(back[moved] - first[moved]) <= np.abs(first[moved]) + 1e-38)   # only underflow


@pytest.mark.parametrize("fmt", FMTS)
def test_eq1_regrouping_does_add_error(fmt):
    x = token_activation(384, 512, seed=7)
    first, second, _, _ = regroup(x, fmt, pow2=False)
    changed = np.count_nonzero(second.T != first)
    assert changed > 0.05 * x.size                       # why the pages take powers of two


def test_transposed_layout():
    x = small_tensor(256, 256, seed=4)
    q, s, _, _ = O.quantize_block_ex(x, 1, 128, E4M3, pow2=True)
    qT, sT, _ = O.requant_1x128_to_128x1(q, s, E4M3, E4M3, True)
    xt = np.ascontiguousarray(bf16_to_f32(x).T)
    qd, sd, _, _ = O.quantize_block_ex(O.dequant_block(q, 1, 128, E4M3, s).T.copy(), 1, 128, E4M3, pow2=True)
    assert np.array_equal(qT, qd) and np.array_equal(sT, sd)
    # the column groups of the original: scalesT[c][g] covers rows 128g .. 128g+127 of column c
    col = xt[5, 128:256].astype(np.float64)
    assert sT[5, 1] == O.scale_pow2(E4M3, float(np.max(np.abs(O.dequant_block(q, 1, 128, E4M3, s)[128:256, 5]))))
    assert np.max(np.abs(col)) > 0
