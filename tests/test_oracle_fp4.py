"""CPU pins of the FP4 oracle: E2M1 elements, MXFP4 (1x32, E8M0) and NVFP4 (1x16, E4M3 block
scale and an fp32 tensor scale).

Pages: "混合精度与 FP8 训练" sections 13.1 (MX rule, emax of E2M1 = 2, the amax 5.3 block: scale
1, 5.3 -> 6, 13% error) and 13.2 (E2M1 values 0, 0.5, 1, 1.5, 2, 3, 4, 6; NVFP4 blocks of 16 with
an E4M3 scale that can align the block maximum to 6; 5.3/6 = 0.883 -> 0.875, 5.3/0.875 = 6.06 ->
6, de-scaled 5.25, under 1% error; 4.5 bits per element); the Ascend 950 guide section 2.4
(MXFP4 = 32 FP4 values + one shared scale).

  * E2M1 decode = the pages' value list; encode against an independent round-half-even on the
    integer grid of each binade (numpy rint) for every BF16 value and for hand ties;
  * MXFP4: the 5.3 example in both rounding modes; emax 2; round-up minus round-down exponent =
    [significand > 1.5] over every positive BF16 amax; round-up never saturates; columnwise =
    rowwise of the transpose; the nibble order of the packing;
  * NVFP4: the 5.3 example; the block holding the tensor amax gets E4M3's 448; in every block
    whose scale is a normal E4M3 value the largest element encodes to +-6; scaling the tensor by
    2^k leaves codes and block scales unchanged and divides S_t by 2^k; 4.5 bits per element;
    de-scaling error within one E2M1 half-spacing of the block.
"""
import numpy as np
import pytest

import oracle as O
from synthetic import bf16_bits, bf16_to_f32, small_tensor

E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_values():
    assert [O.decode(O.E2M1, c) for c in range(8)] == E2M1_VALUES
    assert [O.decode(O.E2M1, c) for c in range(8, 16)] == [-v for v in E2M1_VALUES]
    assert O.max_finite(O.E2M1) == 6.0 and O.num_finite_nonneg(O.E2M1) == 8


def rint_e2m1(v):
    """Independent encoder: round half to even on the integer grid of the value's binade."""
    a = abs(float(v))
    if a >= 6.0:
        code = 7
    elif a < 2.0:
        code = int(np.rint(a * 2.0))            # grid 0.5: code = 2a (0..4)
    elif a < 4.0:
        code = int(np.rint(a)) + 2              # grid 1: values 2, 3, 4 = codes 4, 5, 6
    else:
        code = min(int(np.rint(a / 2.0)) + 4, 7)   # grid 2: values 4, 6 (8 saturates to 6)
    return code | (8 if np.signbit(v) else 0)


def test_e2m1_encode_hand_ties():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 6.5: 7, 1e9: 7, -0.0: 8, -0.2: 8,
            -0.3: 9, -5.0001: 15}
    for v, c in ties.items():
        assert O.encode(O.E2M1, v) == c, v


def test_e2m1_encode_every_bf16():
    bits = np.arange(0x10000, dtype=np.uint32)
    vals = ((bits << 16).view(np.float32))
    fin = vals[np.isfinite(vals)]
    got = O.encode_f32(O.E2M1, fin)
    want = np.array([rint_e2m1(v) for v in fin], np.uint8)
    assert np.array_equal(got, want)


def test_mxfp4_worked_example():
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [5.3, -1.0, 0.2, 2.9]
    xb = bf16_bits(x)
    for rnd in (O.ROUND_DOWN, O.ROUND_UP):
        q, s, _, _, nf = O.quantize_mxfp4(xb, rnd, col=False)
        assert s[0, 0] == 127 and nf == 0                   # floor(log2 5.3) - 2 = 0: scale 1
        codes = O.unpack_fp4(q)[0]
        assert codes[0] == 7 and O.decode(O.E2M1, codes[0]) == 6.0
        v = float(bf16_to_f32(xb)[0, 0])
        assert abs(6.0 - v) / v == pytest.approx(0.13, abs=0.005)
        assert list(codes[1:4]) == [10, 0, 5]                # -1 -> 0b1010, 0.2 -> 0, 2.9 -> 3


def test_mxfp4_exponent_rules_every_bf16_amax():
    assert O.mx_exponent(O.E2M1, O.ROUND_DOWN, 4.0) == 0 and O.mx_exponent(O.E2M1, O.ROUND_DOWN, 8.0) == 1
    amaxes = bf16_to_f32(np.arange(1, 0x7F80, dtype=np.uint16))
    for a in amaxes[::7]:
        a = float(a)
        d = O.mx_exponent(O.E2M1, O.ROUND_DOWN, a)
        u = O.mx_exponent(O.E2M1, O.ROUND_UP, a)
        m, e = np.frexp(a)                                   # a = m 2^e, significand 2m in [1, 2)
        if -127 < d and u < 127:
            assert d == e - 1 - 2
            assert u - d == (1 if 2 * m > 1.5 else 0), a
            assert a / 2.0 ** u <= 6.0


def test_mxfp4_col_is_row_of_transpose_and_packing():
    x = small_tensor(64, 96, seed=11, scale=3.0)
    for rnd in (O.ROUND_DOWN, O.ROUND_UP):
        qr, sr, qc, sc, _ = O.quantize_mxfp4(x, rnd)
        qt, st, _, _, _ = O.quantize_mxfp4(np.ascontiguousarray(x.T), rnd, col=False)
        assert np.array_equal(qc, qt) and np.array_equal(sc, st)
        assert qr.shape == (64, 48) and qc.shape == (96, 32)
        # element 2j in the low nibble, 2j+1 in the high nibble
        codes = O.quantize_mx(x, O.E2M1, rnd, col=False)[0]
        assert np.array_equal(qr & 0xF, codes[:, 0::2]) and np.array_equal(qr >> 4, codes[:, 1::2])
        assert np.array_equal(O.unpack_fp4(qr), codes)


def test_nvfp4_worked_example():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2688.0                                  # tensor amax 448 * 6 gives S_t = 1
    x[0, 16] = 5.3
    x[0, 17] = -0.4
    q, s_blk, s_t, a, nf = O.quantize_nvfp4(x)
    assert s_t == 1.0 and a == 2688.0 and nf == 0
    assert O.decode(O.E4M3, s_blk[0, 1]) == 0.875     # 5.3 / 6 = 0.883 -> 0.875
    codes = O.unpack_fp4(q)[0]
    assert codes[16] == 7                             # 5.3 / 0.875 = 6.06 -> 6
    assert O.dequant_nvfp4_one(codes[16], s_blk[0, 1], s_t) == 5.25
    assert abs(5.25 - 5.3) / 5.3 < 0.01
    assert O.decode(O.E4M3, s_blk[0, 0]) == 448.0     # the block holding the tensor amax
    # 4.5 bits per element: 16 codes (8 bytes) + one scale byte per block
    assert (q.nbytes + s_blk.nbytes) * 8 / x.size == 4.5


def nvfp4_real(x):
    return bf16_to_f32(x) if x.dtype == np.uint16 else x


@pytest.mark.parametrize("seed,scale", [(1, 1.0), (2, 1e-3), (3, 300.0)])
def test_nvfp4_block_maximum_on_top_and_error_bound(seed, scale):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((48, 128)) * np.exp(rng.uniform(-3, 3, (48, 1)))).astype(np.float32) * np.float32(scale)
    q, s_blk, s_t, a, _ = O.quantize_nvfp4(x)
    codes = O.unpack_fp4(q)
    xr = nvfp4_real(x)
    top = 0
    for r in range(x.shape[0]):
        for g in range(x.shape[1] // 16):
            blk = xr[r, 16 * g:16 * g + 16]
            cb = codes[r, 16 * g:16 * g + 16]
            dec = O.decode(O.E4M3, s_blk[r, g])
            if dec >= 2.0 ** -6:                      # a normal E4M3 block scale
                assert O.decode(O.E2M1, cb[np.argmax(np.abs(blk))] & 7) == 6.0, (r, g)
                top += 1
                # de-scaled error within one E2M1 half-spacing (at most 1) of the block scale
                xh = np.array([O.dequant_nvfp4_one(c, s_blk[r, g], s_t) for c in cb])
                assert np.all(np.abs(xh - blk) <= (dec / s_t) * (1 + 2 ** -20) + np.abs(blk) * 2 ** -20)
    assert top > 0
    assert O.decode(O.E4M3, s_blk.reshape(-1)[np.argmax(np.abs(xr).reshape(-1)) // 16]) == 448.0


@pytest.mark.parametrize("k", [-20, -3, 1, 7])
def test_nvfp4_power_of_two_invariance(k):
    x = (np.random.default_rng(4).standard_normal((16, 64)) * 5.0).astype(np.float32)
    q0, s0, t0, _, _ = O.quantize_nvfp4(x)
    q1, s1, t1, _, _ = O.quantize_nvfp4(x * np.float32(2.0 ** k))
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
    assert t1 == np.float32(t0 * 2.0 ** -k)


def test_nvfp4_zero_and_negligible_blocks():
    x = np.zeros((1, 48), np.float32)
    x[0, 0] = 1000.0
    x[0, 16] = -1e-6                                  # scale underflows E4M3: signed zero codes
    x[0, 33] = -0.0
    q, s_blk, s_t, _, _ = O.quantize_nvfp4(x)
    codes = O.unpack_fp4(q)[0]
    assert s_blk[0, 1] == 0 and s_blk[0, 2] == 0
    assert codes[16] == 8 and codes[17] == 0 and codes[33] == 8 and codes[32] == 0


def test_nvfp4_nonfinite():
    x = np.ones((2, 32), np.float32)
    x[1, 20] = np.nan
    q, s_blk, s_t, a, nf = O.quantize_nvfp4(x)
    assert nf == 1 and s_t == 1.0 and s_blk[1, 1] == 0x7F
    assert s_blk[0, 0] != 0x7F


def test_nvfp4_caller_amax():
    x = (np.random.default_rng(8).standard_normal((8, 64)) * 3.0).astype(np.float32)
    ref = O.quantize_nvfp4(x)
    same = O.quantize_nvfp4(x, amax_in=-float(ref[3]))        # the magnitude is used
    assert all(np.array_equal(a, b) for a, b in zip(ref[:2], same[:2])) and ref[2] == same[2]
    # an amax below the data's: block scales saturate at 448 and the top codes at +-6
    q, s_blk, s_t, a, _ = O.quantize_nvfp4(x, amax_in=float(ref[3]) / 8)
    assert a == np.float32(ref[3] / 8) and s_t == O.nvfp4_tensor_scale(a)
    top = np.abs(x).reshape(-1, 16).max(axis=1) > a
    assert np.all(s_blk.reshape(-1)[top] == 0x7E)


def test_nvfp4_tiny_tensor_scale_overflow():
    """With the tensor amax in the fp32 subnormal range S_t overflows to FLT_MAX (Eq.(1)'s rule).
    The element quotient x * S_t / decode(e_b) is still exact: the block's largest element lands
    on 6 and de-scales back to about its value; a block whose scale underflows E4M3 keeps signed
    zero codes."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.float32(1e-40)
    x[0, 16] = np.float32(3e-45)
    q, s_blk, s_t, _, _ = O.quantize_nvfp4(x)
    codes = O.unpack_fp4(q)[0]
    fmax = np.finfo(np.float32).max
    assert s_t == fmax
    e = O.nvfp4_block(1e-40, s_t)
    assert s_blk[0, 0] == e and O.decode(O.E4M3, e) == 3 / 512          # 1e-40 * FLT_MAX / 6 = 0.00567
    assert codes[0] == 7 and np.all(codes[1:16] == 0)
    xh = O.dequant_nvfp4_one(codes[0], e, s_t)
    assert abs(xh - float(x[0, 0])) / float(x[0, 0]) < 0.04            # 6 * (3/512) / FLT_MAX
    assert O.nvfp4_block(3e-45, s_t) == 0 == s_blk[0, 1]                 # below E4M3's range
    assert np.all(codes[16:] == 0)


def _golden(golden_dir, name):
    import json
    import os
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_golden_e2m1_values(golden_dir):
    g = _golden(golden_dir, "w10_e2m1_values.json")
    assert [O.decode(O.E2M1, c) for c in range(8)] == g["values"]


def test_golden_mxfp4_example(golden_dir):
    g = _golden(golden_dir, "w8_mxfp4_example.json")
    assert O.emax(O.E2M1) == g["emax_e2m1"]
    assert O.mx_exponent(O.E2M1, O.ROUND_DOWN, g["amax"]) == g["shared_exponent"]
    assert 2.0 ** g["shared_exponent"] == g["scale"]
    assert O.decode(O.E2M1, O.encode(O.E2M1, g["amax"] / g["scale"])) == g["rounded_amax"]
    err = abs(g["rounded_amax"] - g["amax"]) / g["amax"]
    assert round(100 * err) == g["relative_error_pct"]


def test_golden_nvfp4_example(golden_dir):
    g = _golden(golden_dir, "w9_nvfp4_example.json")
    e = O.nvfp4_block(g["amax"], 1.0)                  # S_t = 1, as in the example
    assert round(g["amax"] / 6, 3) == g["block_scale_exact"]
    assert O.decode(O.E4M3, e) == g["block_scale_e4m3"]
    assert round(g["amax"] / g["block_scale_e4m3"], 2) == g["scaled_amax"]
    code = O.nvfp4_element(g["amax"], 1.0, e)
    assert O.decode(O.E2M1, code) == g["rounded_amax"]
    assert O.dequant_nvfp4_one(code, e, 1.0) == g["dequantized"]
    assert abs(g["dequantized"] - g["amax"]) / g["amax"] * 100 < g["relative_error_below_pct"]
    assert (g["block_size"] * 4 + 8) / g["block_size"] == g["bits_per_element"]
