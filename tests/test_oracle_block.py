"""Oracle fine-grained (1x128 per-token-group, 128x128 block) scaling.

Pins ("混合精度与 FP8 训练" sections 8.1 and 10.2): each group is quantized by the per-tensor
rule on its own, so
  * a group covering the whole tensor equals per-tensor current scaling;
  * 1x128 groups on a [R][128] tensor equal per-row per-tensor scaling;
  * 128x128 blocks stay valid under transpose: quantizing X^T gives the transposed codes and
    the transposed scale grid;
  * partial groups at the right and bottom edges follow the same rule on their elements.
"""
import numpy as np
import pytest

import oracle as O
from synthetic import bf16_to_f32, block_weight, small_tensor, token_activation

E4M3, E5M2 = O.E4M3, O.E5M2


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_whole_tensor_group_is_per_tensor(fmt):
    x = token_activation(64, 96, seed=3)
    q, s, a, nf = O.quantize_block(x, 64, 96, fmt)
    q2, a2, s2, nf2 = O.quantize_per_tensor(x, fmt)
    assert np.array_equal(q, q2) and s[0, 0] == s2 and a[0, 0] == a2 and nf == nf2 == 0


def test_1x128_is_per_row_per_tensor():
    x = token_activation(16, 128, seed=4)
    q, s, a, _ = O.quantize_block(x, 1, 128, E4M3)
    assert s.shape == (16, 1)
    for r in range(16):
        qr, ar, sr, _ = O.quantize_per_tensor(x[r:r + 1], E4M3)
        assert np.array_equal(q[r], qr[0]) and s[r, 0] == sr and a[r, 0] == ar


def test_128x128_transpose_invariance():
    x = block_weight(256, 384, seed=5)
    q, s, a, _ = O.quantize_block(x, 128, 128, E4M3)
    qt, st, at, _ = O.quantize_block(np.ascontiguousarray(x.T), 128, 128, E4M3)
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T) and np.array_equal(at, a.T)


@pytest.mark.parametrize("br,bc", [(1, 128), (128, 128)])
def test_group_rule_by_hand_with_ragged_edges(br, bc):
    rows, cols = (3, 200) if br == 1 else (150, 200)
    x = small_tensor(rows, cols, seed=6)
    xf = bf16_to_f32(x).astype(np.float64)
    q, s, a, _ = O.quantize_block(x, br, bc, E4M3)
    assert s.shape == (-(-rows // br), -(-cols // bc))
    for bi in range(s.shape[0]):
        for bj in range(s.shape[1]):
            blk = xf[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
            am = np.max(np.abs(blk))
            assert a[bi, bj] == am
            sg = np.float32(448.0 / am)
            assert s[bi, bj] == sg
            want = np.array([O.encode(E4M3, float(np.float32(v * np.float64(sg)))) for v in blk.reshape(-1)])
            got = q[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc].reshape(-1)
            assert np.array_equal(got, want)


def test_zero_group_scale_is_one():
    x = np.zeros((2, 256), np.float32)
    x[1, 130] = 3.0
    q, s, a, _ = O.quantize_block(x, 1, 128, E4M3)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert s[1, 1] == np.float32(448 / 3.0) and q[1, 130] == 0x7E


def test_tiny_amax_scale_saturates_to_flt_max():
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 2.0 ** -140            # 448 / amax overflows fp32
    _, s, _, _ = O.quantize_block(x, 1, 128, E4M3)
    assert s[0, 0] == np.finfo(np.float32).max
