"""GPU parity of quantize_mx_dual (MX 1x32 blocks, E8M0 scales) against the CPU oracle.

Every comparison is byte-exact on fp8 codes and E8M0 scale bytes:
  * an exhaustive domain: for every BF16 amax exponent (and mantissas on both sides of the 1.75
    round-up boundary) blocks holding every BF16 magnitude not above that amax, with random
    signs, in both directions, E4M3/E5M2 x round-down/round-up;
  * small and ragged shapes spanning several 128 x 512 tiles, BF16 and FP32 input,
    single-direction calls, an all-zero block and -0;
  * the full 16384 x 4096 gradient workload in all four variants (the configuration the
    benchmark times), compared over every byte.
"""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import mx_gradient, small_tensor
from qf8_test_utils import assert_bytes_equal, host, parallel_row_slabs, to_device

pytestmark = pytest.mark.gpu

VARIANTS = [(f, r) for f in (O.E4M3, O.E5M2) for r in (O.ROUND_DOWN, O.ROUND_UP)]
VID = [f"{'e4m3' if f == 0 else 'e5m2'}-{'down' if r == 0 else 'up'}" for f, r in VARIANTS]


def run_gpu(x, fmt, rnd, row=True, col=True):
    xd = to_device(x)
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows, cols = x.shape
    # poison outputs so that any byte the kernel fails to write shows up
    out = {}
    if row:
        out["q_row"] = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device="cuda")
        out["s_row"] = torch.full((rows, cols // 32), 0xA5, dtype=torch.uint8, device="cuda")
    if col:
        out["q_colT"] = torch.full((cols, rows), 0xA5, dtype=torch.uint8, device="cuda")
        out["s_colT"] = torch.full((cols, rows // 32), 0xA5, dtype=torch.uint8, device="cuda")
    r = qf8.quantize_mx_dual(xd, fmt, rnd, rowwise=row, colwise=col, nonfinite=nf, **out)
    torch.cuda.synchronize()
    return [None if t is None else host(t) for t in r] + [int(nf.item())]


def check(x, fmt, rnd, row=True, col=True, tag=""):
    g = run_gpu(x, fmt, rnd, row, col)
    w = O.quantize_mx(x, fmt, rnd, row=row, col=col)
    for i, name in enumerate(("q_row", "s_row", "q_colT", "s_colT")):
        if w[i] is None:
            assert g[i] is None
            continue
        assert_bytes_equal(g[i], w[i], name, f" [{tag} fmt={fmt} rnd={rnd} shape={x.shape}]")
    assert g[4] == w[4]


def exhaustive_blocks(seed=0):
    """[G, 32] BF16 blocks: for each amax A (every exponent field, mantissas 0x00/0x60/0x61/0x7F
    and a few subnormals) every BF16 magnitude <= A, 31 per block next to A, random signs, A at
    a varying position."""
    rng = np.random.default_rng(seed)
    mags = np.arange(0, 0x7F80, dtype=np.uint32)
    amaxes = [a for e in range(1, 255) for a in ((e << 7) | 0x00, (e << 7) | 0x60, (e << 7) | 0x61, (e << 7) | 0x7F)]
    amaxes += [0x0001, 0x0040, 0x007F]
    blocks = []
    for a in amaxes:
        below = mags[: a + 1]
        ng = -(-len(below) // 31)
        body = np.resize(below, ng * 31).reshape(ng, 31)
        blk = np.concatenate([np.full((ng, 1), a, np.uint32), body], axis=1)
        blocks.append(blk)
    b = np.concatenate(blocks, axis=0)
    b |= (rng.integers(0, 2, b.shape, dtype=np.uint32) << 15)
    shift = np.arange(b.shape[0]) % 32
    cols = (np.arange(32)[None, :] - shift[:, None]) % 32
    b = np.take_along_axis(b, cols, axis=1)
    pad = (-b.shape[0]) % 64
    if pad:
        b = np.concatenate([b, np.zeros((pad, 32), np.uint32)], axis=0)
    return b.astype(np.uint16)


@pytest.fixture(scope="module")
def exhaustive():
    return exhaustive_blocks()


@pytest.mark.parametrize("fmt,rnd", VARIANTS, ids=VID)
def test_exhaustive_rowwise(exhaustive, fmt, rnd):
    check(exhaustive, fmt, rnd, row=True, col=False, tag="exhaustive-row")


@pytest.mark.parametrize("fmt,rnd", VARIANTS, ids=VID)
def test_exhaustive_columnwise(exhaustive, fmt, rnd):
    xt = np.ascontiguousarray(exhaustive.T)          # [32, G]: each column is one block
    check(xt, fmt, rnd, row=False, col=True, tag="exhaustive-col")


SHAPES = [(32, 32), (64, 96), (128, 512), (256, 1024), (160, 544), (96, 1056), (384, 2048)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fmt,rnd", VARIANTS, ids=VID)
def test_dual_small_bf16(shape, fmt, rnd):
    x = mx_gradient(*shape, seed=sum(shape))
    check(x, fmt, rnd, tag="dual-bf16")


@pytest.mark.parametrize("shape", [(32, 32), (64, 288), (160, 544)])
@pytest.mark.parametrize("fmt,rnd", VARIANTS, ids=VID)
def test_dual_small_fp32(shape, fmt, rnd):
    rng = np.random.default_rng(5)
    x = (rng.laplace(0, 1e-3, shape) * np.where(rng.random(shape) < 0.01, 1e4, 1.0)).astype(np.float32)
    check(x, fmt, rnd, tag="dual-fp32")


@pytest.mark.parametrize("fmt,rnd", VARIANTS, ids=VID)
def test_single_direction_and_ragged(fmt, rnd):
    check(small_tensor(37, 64, seed=3), fmt, rnd, row=True, col=False, tag="row-ragged-rows")
    check(small_tensor(130, 96, seed=4), fmt, rnd, row=True, col=False, tag="row-ragged-rows")
    check(small_tensor(64, 40, seed=5), fmt, rnd, row=False, col=True, tag="col-narrow")
    check(small_tensor(96, 520, seed=6), fmt, rnd, row=False, col=True, tag="col-ragged-cols")


@pytest.mark.parametrize("fmt,rnd", VARIANTS, ids=VID)
def test_rowwise_ragged_rows_fp32(fmt, rnd):
    """Rowwise codes leave two rows at a time through lane pairs; with an odd number of rows in a
    wave the pair's second row lies outside the tensor. FP32 input (the 8-byte pieces)."""
    rng = np.random.default_rng(9)
    for shape in [(37, 64), (130, 96), (1, 32)]:
        x = (rng.standard_normal(shape) * np.exp(rng.uniform(-3, 3, (shape[0], 1)))).astype(np.float32)
        check(x, fmt, rnd, row=True, col=False, tag=f"row-ragged-rows-fp32 {shape}")


def test_zero_blocks_and_negative_zero():
    x = np.zeros((64, 64), np.uint16)
    x[3, 5] = 0x8000                     # -0 inside an all-zero block -> 0x00
    x[40, 40] = 0x4000                   # 2.0
    x[41, 41] = 0x8001                   # negative subnormal
    for fmt, rnd in VARIANTS:
        check(x, fmt, rnd, tag="zeros")


def test_extreme_magnitudes():
    x = np.zeros((64, 64), np.uint16)
    x[0, :] = 0x7F7F                     # largest finite BF16
    x[1, :] = 0x0001                     # smallest subnormal BF16
    x[2, 0:32] = 0x7F7F
    x[2, 1] = 0x0001                     # tiny value next to huge amax underflows to (signed) zero
    x[5, :] = 0x80FF
    for fmt, rnd in VARIANTS:
        check(x, fmt, rnd, tag="extremes")


def test_nonfinite_sets_flag_and_nan_scale():
    x = small_tensor(64, 64, seed=9)
    x[7, 9] = 0x7F80                     # +Inf
    x[50, 33] = 0x7FC1                   # NaN
    g = run_gpu(x, O.E4M3, O.ROUND_UP)
    w = O.quantize_mx(x, O.E4M3, O.ROUND_UP)
    assert g[4] == 1 and w[4] == 1
    assert g[1][7, 0] == 0xFF and g[1][50, 1] == 0xFF and g[3][9, 0] == 0xFF and g[3][33, 1] == 0xFF
    # blocks without the non-finite values stay bit-exact
    ok_row = np.ones(g[1].shape, bool)
    ok_row[7, 0] = ok_row[50, 1] = False
    assert np.array_equal(g[1][ok_row], w[1][ok_row])
    qr_ok = np.repeat(ok_row, 32, axis=1)
    assert np.array_equal(g[0][qr_ok], w[0][qr_ok])


@pytest.fixture(scope="module")
def gradient_full():
    return mx_gradient()


@pytest.mark.parametrize("fmt,rnd", VARIANTS, ids=VID)
def test_full_size_gradient(gradient_full, fmt, rnd):
    x = gradient_full
    rows, cols = x.shape
    g = run_gpu(x, fmt, rnd)
    slab = 1024

    def one(r0, r1):
        return O.quantize_mx(x[r0:r1], fmt, rnd)

    parts = parallel_row_slabs(one, rows, slab)
    assert_bytes_equal(g[0], np.concatenate([p[0] for p in parts], axis=0), "q_row", " [16384x4096]")
    assert_bytes_equal(g[1], np.concatenate([p[1] for p in parts], axis=0), "s_row", " [16384x4096]")
    assert_bytes_equal(g[2], np.concatenate([p[2] for p in parts], axis=1), "q_colT", " [16384x4096]")
    assert_bytes_equal(g[3], np.concatenate([p[3] for p in parts], axis=1), "s_colT", " [16384x4096]")
    assert g[4] == 0
