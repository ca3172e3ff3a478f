"""GPU parity of quantize_block (1x128 per-token groups, 128x128 weight blocks) against the CPU
oracle: bit-exact codes, fp32 group scales and group amax.

  * every positive finite BF16 value as a group amax (one 1x128 group each), which also pins
    the device division S = fl32(F8max/amax) over the whole BF16 range;
  * small shapes with ragged right and bottom edges, BF16 and FP32 input;
  * the full 8192x7168 token-activation workload (1x128) and 7168x18432 weight (128x128).
"""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import block_weight, small_tensor, token_activation
from qf8_test_utils import assert_bytes_equal, host, parallel_row_slabs, to_device

pytestmark = pytest.mark.gpu
FMTS = [O.E4M3, O.E5M2]


def run_block(x, br, fmt):
    xd = to_device(x)
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    q = torch.full(x.shape, 0xA5, dtype=torch.uint8, device="cuda")
    q, s, a = qf8.quantize_block(xd, br, 128, fmt, q=q, nonfinite=nf)
    torch.cuda.synchronize()
    return host(q), host(s), host(a), int(nf.item())


def check(x, br, fmt, tag=""):
    g = run_block(x, br, fmt)
    w = O.quantize_block(x, br, 128, fmt)
    assert_bytes_equal(g[0], w[0], "q", tag)
    assert_bytes_equal(g[1], w[1], "scales", tag)
    assert_bytes_equal(g[2], w[2], "amax", tag)
    assert g[3] == w[3]


@pytest.mark.parametrize("fmt", FMTS)
def test_every_bf16_amax_as_group_amax(fmt):
    amaxes = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((len(amaxes), 128), np.uint16)
    x[:, 0] = amaxes
    x[:, 77] = amaxes | 0x8000
    x[:, 5] = amaxes >> 1
    check(x, 1, fmt, " [all amax]")


@pytest.mark.parametrize("shape", [(1, 128), (3, 200), (16, 1024), (37, 136), (300, 8)])
@pytest.mark.parametrize("fmt", FMTS)
def test_1x128_small(shape, fmt):
    check(token_activation(*shape, seed=sum(shape)), 1, fmt, f" [{shape}]")


@pytest.mark.parametrize("shape", [(128, 128), (150, 200), (256, 384), (129, 1032), (7, 64)])
@pytest.mark.parametrize("fmt", FMTS)
def test_128x128_small(shape, fmt):
    check(block_weight(*shape, seed=sum(shape)), 128, fmt, f" [{shape}]")


@pytest.mark.parametrize("br", [1, 128])
def test_fp32_input(br):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((140, 260)) * rng.standard_t(3, (140, 1))).astype(np.float32)
    for fmt in FMTS:
        check(x, br, fmt, " [fp32]")


def test_zero_and_tiny_groups():
    x = np.zeros((130, 256), np.uint16)
    x[0, 200] = 0x0001
    x[129, 1] = 0x8000
    for br in (1, 128):
        check(x, br, O.E4M3, f" [zeros br={br}]")


def test_nonfinite_flag():
    x = small_tensor(4, 256, seed=2)
    x[1, 130] = 0x7F80
    g = run_block(x, 1, O.E4M3)
    assert g[3] == 1 and np.isinf(g[2][1, 1]) and g[1][1, 1] == 1.0


@pytest.fixture(scope="module")
def activation():
    return token_activation()


@pytest.fixture(scope="module")
def weight():
    return block_weight()


def test_full_size_1x128_activation(activation):
    x = activation
    g = run_block(x, 1, O.E4M3)
    parts = parallel_row_slabs(lambda r0, r1: O.quantize_block(x[r0:r1], 1, 128, O.E4M3), x.shape[0], 512)
    for i, name in enumerate(("q", "scales", "amax")):
        assert_bytes_equal(g[i], np.concatenate([p[i] for p in parts], axis=0), name, " [8192x7168 1x128]")


def test_full_size_128x128_weight(weight):
    x = weight
    g = run_block(x, 128, O.E4M3)
    parts = parallel_row_slabs(lambda r0, r1: O.quantize_block(x[r0:r1], 128, 128, O.E4M3), x.shape[0], 512)
    for i, name in enumerate(("q", "scales", "amax")):
        assert_bytes_equal(g[i], np.concatenate([p[i] for p in parts], axis=0), name, " [7168x18432 128x128]")
