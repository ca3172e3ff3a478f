"""Scale outputs that are not 16-byte aligned.

The ABI puts no alignment requirement on the E8M0 / E4M3 scale arrays (s_row, s_colT, s_blk).
The kernels gather these bytes and store them in whole words or 16-byte pieces when the array
is aligned, and byte by byte when it is not (or when a tile or pass is ragged). These tests
hand every scale array in at an odd address (a view one byte into a poisoned buffer), compare
the bytes with the CPU oracle, and check that the guard bytes on both sides are untouched:
MXFP8 rowwise-only and dual, MXFP4 rowwise-only, and NVFP4 with a caller amax and with the
measured amax (below and above the single-pass size of 2^22 elements).
"""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import mx_gradient
from qf8_test_utils import assert_bytes_equal, host, to_device

pytestmark = pytest.mark.gpu

POISON = 0xA5


def odd_view(shape):
    """A contiguous uint8 tensor of `shape` starting one byte into a poisoned buffer (with one
    guard byte after it), and the buffer."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2,), POISON, dtype=torch.uint8, device="cuda")
    return buf[1:1 + n].view(*shape), buf


def check_guards(buf, what):
    b = host(buf)
    assert b[0] == POISON and b[-1] == POISON, f"{what}: a byte outside the array was written"


@pytest.mark.parametrize("shape", [(128, 256), (256, 512), (160, 544), (96, 4096)])
@pytest.mark.parametrize("fmt", [O.E4M3, O.E5M2], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("dual", [False, True], ids=["rowwise", "dual"])
def test_mxfp8_odd_scale_arrays(shape, fmt, dual):
    rows, cols = shape
    x = mx_gradient(rows, cols, seed=rows + cols)
    xd = to_device(x)
    q_row = torch.full((rows, cols), POISON, dtype=torch.uint8, device="cuda")
    s_row, sbuf_r = odd_view((rows, cols // 32))
    out = {"q_row": q_row, "s_row": s_row}
    if dual:
        out["q_colT"] = torch.full((cols, rows), POISON, dtype=torch.uint8, device="cuda")
        out["s_colT"], sbuf_c = odd_view((cols, rows // 32))
    for rnd in (O.ROUND_DOWN, O.ROUND_UP):
        r = qf8.quantize_mx_dual(xd, fmt, rnd, rowwise=True, colwise=dual, **out)
        torch.cuda.synchronize()
        w = O.quantize_mx(x, fmt, rnd, row=True, col=dual)
        tag = f" [shape={shape} fmt={fmt} rnd={rnd} dual={dual}]"
        assert_bytes_equal(host(r[0]), w[0], "q_row", tag)
        assert_bytes_equal(host(r[1]), w[1], "s_row", tag)
        check_guards(sbuf_r, "s_row" + tag)
        if dual:
            assert_bytes_equal(host(r[2]), w[2], "q_colT", tag)
            assert_bytes_equal(host(r[3]), w[3], "s_colT", tag)
            check_guards(sbuf_c, "s_colT" + tag)


@pytest.mark.parametrize("shape", [(128, 512), (160, 544), (64, 4096)])
def test_mxfp4_rowwise_odd_scale_array(shape):
    rows, cols = shape
    x = mx_gradient(rows, cols, seed=rows * 3 + cols)
    xd = to_device(x)
    q_row = torch.full((rows, cols // 2), POISON, dtype=torch.uint8, device="cuda")
    s_row, sbuf = odd_view((rows, cols // 32))
    for rnd in (O.ROUND_DOWN, O.ROUND_UP):
        r = qf8.quantize_mxfp4_dual(xd, rnd, rowwise=True, colwise=False, q_row=q_row, s_row=s_row)
        torch.cuda.synchronize()
        w = O.quantize_mxfp4(x, rnd, row=True, col=False)
        tag = f" [shape={shape} rnd={rnd}]"
        assert_bytes_equal(host(r[0]), w[0], "q_row", tag)
        assert_bytes_equal(host(r[1]), w[1], "s_row", tag)
        check_guards(sbuf, "s_row" + tag)


@pytest.mark.parametrize("shape", [(64, 4096), (33, 48), (1000, 1008), (2048, 2048), (2049, 2064)])
@pytest.mark.parametrize("caller_amax", [False, True], ids=["measured", "caller"])
def test_nvfp4_odd_scale_array(shape, caller_amax):
    rows, cols = shape
    x = mx_gradient(rows, cols, seed=rows + 7 * cols)
    xd = to_device(x)
    amax = float(O.quantize_nvfp4(x)[3]) if caller_amax else None       # the measured tensor amax
    ain = None if amax is None else torch.tensor([amax], dtype=torch.float32, device="cuda")
    q = torch.full((rows, cols // 2), POISON, dtype=torch.uint8, device="cuda")
    s_blk, sbuf = odd_view((rows, cols // 16))
    st = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    qf8.quantize_nvfp4(xd, amax_in=ain, q=q, s_blk=s_blk, tensor_scale=st)
    torch.cuda.synchronize()
    w = O.quantize_nvfp4(x, amax_in=amax)
    tag = f" [shape={shape} caller_amax={caller_amax}]"
    assert np.float32(st.item()) == w[2], tag
    assert_bytes_equal(host(s_blk), w[1], "s_blk", tag)
    assert_bytes_equal(host(q), w[0], "q", tag)
    check_guards(sbuf, "s_blk" + tag)
