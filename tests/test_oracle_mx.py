"""Oracle MX (1x32 blocks, E8M0 shared scale) pinned to closed forms, brute force and invariants.

Pins ("混合精度与 FP8 训练" section 13.1; "NVIDIA：Blackwell GPU MXFP8 预训练最佳实践" section 4.1):
  * round-down X = floor(log2 amax) - emax, checked by its defining inequality for every
    positive finite BF16 amax;
  * round-up X = ceil(log2(amax/destmax)), checked by its defining inequality (the smallest X
    with amax/2^X <= destmax) for every positive finite BF16 amax; so round-up never saturates;
  * closed form: X_up - X_down is 1 exactly when the significand of amax exceeds 1.75
    (destmax = 1.75 * 2^emax for both formats), else 0;
  * a zero block gives X = -127 and all-zero bytes (tests/golden/w7_mx_zero_block.json);
  * columnwise(X) == rowwise(X^T) with numpy's transpose; dual == two single-direction calls;
  * torch's float8_e8m0fnu decoder agrees with the scale bytes.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from synthetic import bf16_to_f32, mx_gradient, small_tensor

E4M3, E5M2 = O.E4M3, O.E5M2
DOWN, UP = O.ROUND_DOWN, O.ROUND_UP


def positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)   # all positive finite
    return bf16_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_exponent_definitions_exhaustive(fmt):
    destmax = O.max_finite(fmt)
    em = O.emax(fmt)
    assert destmax == 1.75 * 2.0 ** em
    n_diff = 0
    for a in positive_bf16():
        xd = O.mx_exponent(fmt, DOWN, a)
        xu = O.mx_exponent(fmt, UP, a)
        fl = math.floor(math.log2(a))
        # round-down: 2^(X+emax) <= amax < 2^(X+emax+1), unless clamped at -127
        if fl - em >= -127:
            assert 2.0 ** (xd + em) <= a < 2.0 ** (xd + em + 1)
        else:
            assert xd == -127
        # round-up: amax/2^X <= destmax < amax/2^(X-1), unless clamped at -127
        if xu > -127:
            assert a / 2.0 ** xu <= destmax < a / 2.0 ** (xu - 1)
        else:
            assert a / 2.0 ** -127 <= destmax
        if xd > -127:
            sig = a / 2.0 ** fl
            assert xu - xd == (1 if sig > 1.75 else 0)
            n_diff += xu - xd
    assert n_diff > 0


def test_zero_block(golden_dir):
    with open(os.path.join(golden_dir, "w7_mx_zero_block.json")) as f:
        g = json.load(f)
    x = np.zeros((32, 64), np.float32)
    x[3, 7] = -0.0
    x[5, 40] = 2.5                    # only row 5's second block and column 40 are non-zero
    for fmt in (E4M3, E5M2):
        for rnd in (DOWN, UP):
            assert O.mx_exponent(fmt, rnd, g["amax"]) == g["X"]
            qr, sr, qc, sc, nf = O.quantize_mx(x, fmt, rnd)
            assert nf == 0
            assert sr[3, 0] == g["X"] + 127 == 0 and qr[3, 7] == 0x00     # -0 in a zero block -> 0x00
            assert sc[7, 0] == 0 and qc[7, 3] == 0x00
            assert sr[5, 1] != 0 and sc[40, 0] != 0
            assert np.count_nonzero(qr) == 1 and np.count_nonzero(qc) == 1


def _bf16_tensor(rows, cols, seed):
    return small_tensor(rows, cols, seed=seed)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rnd", [DOWN, UP])
def test_col_equals_row_of_transpose_and_dual(fmt, rnd):
    x = mx_gradient(96, 160, seed=9)
    qr, sr, qc, sc, _ = O.quantize_mx(x, fmt, rnd)
    qr2, sr2, _, _, _ = O.quantize_mx(np.ascontiguousarray(x.T), fmt, rnd, col=False)
    assert np.array_equal(qc, qr2) and np.array_equal(sc, sr2)
    a, b, _, _, _ = O.quantize_mx(x, fmt, rnd, col=False)
    _, _, c, d, _ = O.quantize_mx(x, fmt, rnd, row=False)
    assert np.array_equal(a, qr) and np.array_equal(b, sr) and np.array_equal(c, qc) and np.array_equal(d, sc)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rnd", [DOWN, UP])
def test_block_rule_by_hand(fmt, rnd):
    """Each row block equals: X from the block amax, then sat_rne8(x / 2^X) elementwise."""
    x = mx_gradient(4, 128, seed=2)
    xf = bf16_to_f32(x).astype(np.float64)
    qr, sr, _, _, _ = O.quantize_mx(x, fmt, rnd, col=False)
    destmax = O.max_finite(fmt)
    for r in range(4):
        for g in range(4):
            blk = xf[r, 32 * g:32 * g + 32]
            X = O.mx_exponent(fmt, rnd, np.max(np.abs(blk)))
            assert sr[r, g] == X + 127
            want = [O.encode(fmt, v / 2.0 ** X) for v in blk]
            assert list(qr[r, 32 * g:32 * g + 32]) == want
            if rnd == UP:    # never saturates
                assert np.max(np.abs(blk)) / 2.0 ** X <= destmax


def test_e8m0_bytes_decode_with_torch():
    x = mx_gradient(64, 64, seed=4)
    _, sr, _, sc, _ = O.quantize_mx(x, E4M3, UP)
    for s in (sr, sc):
        t = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        assert np.array_equal(t, np.array([O.decode(O.E8M0, b) for b in s.reshape(-1)]).reshape(s.shape))


def test_error_bound_unsaturated():
    """|q*2^X - x| <= half the fp8 spacing at x/2^X ("混合精度与 FP8 训练" section 3)."""
    x = mx_gradient(64, 256, seed=12)
    xf = bf16_to_f32(x).astype(np.float64)
    for fmt in (E4M3, E5M2):
        qr, sr, _, _, _ = O.quantize_mx(x, fmt, UP, col=False)
        mb = 3 if fmt == E4M3 else 2
        X = sr.astype(np.int64) - 127
        scale = np.repeat(2.0 ** X, 32, axis=1)
        dec = np.array([O.decode(fmt, c) for c in range(256)])[qr] * scale
        y = np.abs(xf / scale)
        e = np.floor(np.log2(np.maximum(y, 2.0 ** -30)))
        e = np.maximum(e, -6 if fmt == E4M3 else -14)
        spacing = 2.0 ** (e - mb) * scale
        assert np.all(np.abs(dec - xf) <= spacing / 2)


def test_fp32_input_matches_bf16_widened():
    x = mx_gradient(64, 96, seed=21)
    xf = bf16_to_f32(x)
    for fmt in (E4M3, E5M2):
        a = O.quantize_mx(x, fmt, UP)
        b = O.quantize_mx(xf, fmt, UP)
        for u, v in zip(a[:4], b[:4]):
            assert np.array_equal(u, v)


def test_nonfinite_flag_and_nan_scale():
    x = np.ones((32, 32), np.float32)
    x[4, 9] = np.inf
    qr, sr, qc, sc, nf = O.quantize_mx(x, E4M3, UP)
    assert nf == 1 and sr[4, 0] == 0xFF and sc[9, 0] == 0xFF
    assert sr[5, 0] == 127 - 8 and sc[8, 0] == 127 - 8
