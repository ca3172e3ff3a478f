"""GPU parity of the power-of-two group scales and of the 1x128 -> 128x1 re-grouping
("混合精度与 FP8 训练" sections 10.4-10.5) against the oracle: codes and fp32 scales bit for bit.

  * power-of-two 1x128 / 128x128 quantization for every positive finite BF16 value as a group
    amax, on ragged shapes, on FP32 input and on the full 8192x7168 activation;
  * the re-grouping for every (input format, output format, scale rule) on ragged shapes (rows
    and columns multiples of 16, partial 128-row groups), and on the full 8192x7168 activation
    quantized with power-of-two scales, where it also adds no error (values re-scaled into the
    normal range de-scale to exactly their 1x128 values);
  * tiles mixing power-of-two and general row scales, and non-finite columns next to finite
    ones, on every code;
  * non-finite groups set the flag.
"""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import bf16_to_f32, small_tensor, token_activation
from qf8_test_utils import assert_bytes_equal, host, parallel_row_slabs, to_device

pytestmark = pytest.mark.gpu
FMTS = [O.E4M3, O.E5M2]
MIN_NORMAL = {O.E4M3: 2.0 ** -6, O.E5M2: 2.0 ** -14}


def check_block_pow2(x, br, fmt, tag):
    q, s, _ = qf8.quantize_block(to_device(x), br, 128, fmt, pow2_scales=True)
    wq, ws, _, _ = O.quantize_block_ex(x, br, 128, fmt, pow2=True)
    assert_bytes_equal(host(s).view(np.uint32), ws.view(np.uint32), "scales", tag)
    assert_bytes_equal(host(q), wq, "q", tag)


@pytest.mark.parametrize("fmt", FMTS)
def test_pow2_every_bf16_amax(fmt):
    amaxes = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((len(amaxes), 128), np.uint16)
    x[:, 0] = amaxes
    x[:, 77] = amaxes | 0x8000
    x[:, 5] = amaxes >> 1
    check_block_pow2(x, 1, fmt, " [all amax, pow2]")


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("shape", [(1, 128), (3, 200), (130, 264), (300, 8)])
def test_pow2_small_shapes(shape, br):
    for fmt in FMTS:
        check_block_pow2(small_tensor(*shape, seed=shape[0] * 3 + br), br, fmt, f" [{shape} br={br}]")


def test_pow2_fp32_input():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 260)) * 10.0 ** rng.uniform(-30, 30, (64, 1))).astype(np.float32)
    for br in (1, 128):
        check_block_pow2(x, br, O.E4M3, f" [fp32 br={br}]")


def check_requant(q, s, fin, fout, pow2, tag):
    qT, sT = qf8.requantize_1x128_to_128x1(to_device(q), torch.from_numpy(s).cuda(), fin, fout, pow2_scales=pow2)
    wqT, wsT, _ = O.requant_1x128_to_128x1(q, s, fin, fout, pow2)
    assert_bytes_equal(host(sT).view(np.uint32), wsT.view(np.uint32), "scalesT", tag)
    assert_bytes_equal(host(qT), wqT, "qT", tag)


@pytest.mark.parametrize("shape", [(128, 128), (16, 16), (48, 160), (272, 400), (512, 144)])
def test_requant_small(shape):
    x = small_tensor(*shape, seed=shape[0] + shape[1])
    for fin in FMTS:
        for pow2 in (True, False):
            q, s, _, _ = O.quantize_block_ex(x, 1, 128, fin, pow2=pow2)
            for fout in FMTS:
                check_requant(q, s, fin, fout, pow2, f" [{shape} {fin}->{fout} pow2={pow2}]")


@pytest.mark.parametrize("fin", FMTS)
def test_requant_mixed_row_scales_and_nonfinite_columns(fin):
    """Tiles where some waves see only power-of-two row scales and others do not (rows 20..27
    and 150..151 get general scales; 208 rows leave a partial second tile of 80), and where a few
    columns hold NaN or Inf codes, so that waves with and without non-finite columns meet in one
    tile: every scale and every code but the NaN ones (non-finite input is outside the bit-exact
    contract; Inf still saturates to +-F8max and is compared) against the oracle, for both output
    formats and scale rules."""
    x = small_tensor(208, 384, seed=31)
    q, s, _, _ = O.quantize_block_ex(x, 1, 128, fin, pow2=True)
    s = s.copy()
    s[20:28] *= np.float32(1.5)
    s[150:152] *= np.float32(0.7)
    q = q.copy()
    nan_code = 0x7F if fin == O.E4M3 else 0x7E
    q[5, 9] = nan_code
    q[130, 200] = 0x80 | nan_code
    if fin == O.E5M2:
        q[60, 300] = 0x7C                                    # +Inf
        q[207, 301] = 0xFC                                   # -Inf
    nan_at = [(5, 9), (130, 200)]                            # NaN codes are outside the contract
    for pow2 in (True, False):
        for fout in FMTS:
            tag = f" [mixed {fin}->{fout} pow2={pow2}]"
            qT, sT = qf8.requantize_1x128_to_128x1(to_device(q), torch.from_numpy(s).cuda(), fin, fout,
                                                   pow2_scales=pow2)
            wqT, wsT, _ = O.requant_1x128_to_128x1(q, s, fin, fout, pow2)
            got, want = host(qT).copy(), wqT.copy()
            for r, c in nan_at:
                got[c, r] = want[c, r] = 0
            assert_bytes_equal(host(sT).view(np.uint32), wsT.view(np.uint32), "scalesT", tag)
            assert_bytes_equal(got, want, "qT (NaN positions excluded)", tag)


def test_requant_nonfinite_flag():
    x = small_tensor(128, 128, seed=2)
    q, s, _, _ = O.quantize_block_ex(x, 1, 128, O.E4M3, pow2=True)
    q[7, 3] = 0x7F                                           # an E4M3 NaN code
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    qT, sT = qf8.requantize_1x128_to_128x1(to_device(q), torch.from_numpy(s).cuda(), O.E4M3, O.E4M3, nonfinite=nf)
    torch.cuda.synchronize()
    assert int(nf.item()) == 1 and host(sT)[3, 0] == 1.0


@pytest.fixture(scope="module")
def activation():
    return token_activation()


def test_full_activation_pow2_regrouping(activation):
    x = activation
    fmt = O.E4M3
    q, s, _ = qf8.quantize_block(to_device(x), 1, 128, fmt, pow2_scales=True, want_amax=False)
    qT, sT = qf8.requantize_1x128_to_128x1(q, s, fmt, fmt, pow2_scales=True)
    qh, sh, qTh, sTh = host(q), host(s), host(qT), host(sT)
    rows, cols = x.shape
    # 1x128 pass, sampled rows against the oracle
    for r0 in (0, 4096, rows - 64):
        wq, ws, _, _ = O.quantize_block_ex(x[r0:r0 + 64], 1, 128, fmt, pow2=True)
        assert_bytes_equal(qh[r0:r0 + 64], wq, "q", f" [rows {r0}..]")
        assert_bytes_equal(sh[r0:r0 + 64].view(np.uint32), ws.view(np.uint32), "scales", f" [rows {r0}..]")
    # the re-grouping, every column, in slabs of 512 columns (4 scale columns each)
    def slab(c0, c1):
        wqT, wsT, _ = O.requant_1x128_to_128x1(np.ascontiguousarray(qh[:, c0:c1]),
                                               np.ascontiguousarray(sh[:, c0 // 128:c1 // 128]), fmt, fmt, True)
        return wqT, wsT
    parts = parallel_row_slabs(lambda a, b: slab(a * 512, b * 512), cols // 512, 1)
    assert_bytes_equal(qTh, np.concatenate([p[0] for p in parts]), "qT", " [8192x7168]")
    assert_bytes_equal(sTh.view(np.uint32), np.concatenate([p[1] for p in parts]).view(np.uint32), "scalesT", "")
    # no added error on the GPU result either (sampled column slab)
    c0, c1 = 1024, 1536
    first = O.dequant_block(np.ascontiguousarray(qh[:, c0:c1]), 1, 128, fmt, np.ascontiguousarray(sh[:, c0 // 128:c1 // 128]))
    second = O.dequant_block(qTh[c0:c1], 1, 128, fmt, sTh[c0:c1]).T
    s2 = np.repeat(sTh[c0:c1], 128, axis=1)[:, :rows].T
    normal = np.abs(first.astype(np.float64) * s2) >= MIN_NORMAL[fmt]
    assert np.array_equal(second[normal], first[normal]) and normal.mean() > 0.9
