"""Memory hygiene of the GPU library: every output byte is written, nothing past an output is
touched, and repeated calls give identical bytes (all maxima are order-free)."""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import mx_gradient, small_tensor, token_activation
from qf8_test_utils import assert_bytes_equal, host, to_device

pytestmark = pytest.mark.gpu
CANARY = 4096


def guarded(n, fill=0xA5):
    """uint8 device buffer of n bytes followed by a canary region; returns (view, full)."""
    full = torch.full((n + CANARY,), 0x5A, dtype=torch.uint8, device="cuda")
    full[:n] = fill
    return full[:n], full


def canary_ok(full, n):
    return bool(torch.all(full[n:] == 0x5A).item())


def test_mx_dual_canaries_and_repeat():
    x = mx_gradient(160, 544, seed=1)
    rows, cols = x.shape
    xd = to_device(x)
    bufs = {k: guarded(n) for k, n in (("q_row", rows * cols), ("s_row", rows * cols // 32),
                                       ("q_colT", rows * cols), ("s_colT", rows * cols // 32))}
    views = dict(q_row=bufs["q_row"][0].view(rows, cols), s_row=bufs["s_row"][0].view(rows, cols // 32),
                 q_colT=bufs["q_colT"][0].view(cols, rows), s_colT=bufs["s_colT"][0].view(cols, rows // 32))
    outs = []
    for _ in range(2):
        qf8.quantize_mx_dual(xd, qf8.E4M3, qf8.ROUND_DOWN, **views)
        torch.cuda.synchronize()
        outs.append([host(v).copy() for v in views.values()])
    for k, (v, full) in bufs.items():
        assert canary_ok(full, v.numel()), k
    w = O.quantize_mx(x, O.E4M3, O.ROUND_DOWN)
    for a, b, c, name in zip(outs[0], outs[1], w, views):
        assert np.array_equal(a, b), name
        assert_bytes_equal(a, c, name)


def test_per_tensor_and_block_canaries():
    x = small_tensor(33, 65 * 8, seed=2)
    n = x.size
    xd = to_device(x)
    qv, qfull = guarded(n)
    qf8.quantize_per_tensor(xd, qf8.E5M2, q=qv.view(x.shape))
    torch.cuda.synchronize()
    assert canary_ok(qfull, n)
    assert_bytes_equal(host(qv).reshape(x.shape), O.quantize_per_tensor(x, O.E5M2)[0], "q")
    xa = token_activation(33, 520, seed=3)
    qv, qfull = guarded(xa.size)
    sfull = torch.full((33 * 5 + 64,), -7.0, dtype=torch.float32, device="cuda")
    qf8.quantize_block(to_device(xa), 1, 128, qf8.E4M3, q=qv.view(xa.shape), scales=sfull[:33 * 5].view(33, 5))
    torch.cuda.synchronize()
    assert canary_ok(qfull, xa.size) and bool(torch.all(sfull[33 * 5:] == -7.0).item())
    w = O.quantize_block(xa, 1, 128, O.E4M3)
    assert_bytes_equal(host(qv).reshape(xa.shape), w[0], "q")
    assert_bytes_equal(host(sfull[:33 * 5]).reshape(33, 5), w[1], "scales")


def test_repeat_identical_per_tensor_large():
    x = small_tensor(1024, 4096, seed=4)
    xd = to_device(x)
    a = [host(qf8.quantize_per_tensor(xd, qf8.E4M3)[0]) for _ in range(3)]
    assert np.array_equal(a[0], a[1]) and np.array_equal(a[1], a[2])


def test_per_tensor_single_pass_canaries():
    """The single-pass kernel on a ragged length: nothing written past q, every byte of q written."""
    n = qf8.ONEPASS_MIN_ELEMS + 13
    x = small_tensor(1, n, seed=9)
    qv, qfull = guarded(n)
    qf8.quantize_per_tensor(to_device(x), qf8.E4M3, q=qv.view(x.shape))
    torch.cuda.synchronize()
    assert canary_ok(qfull, n)
    assert_bytes_equal(host(qv).reshape(x.shape), O.quantize_per_tensor(x, O.E4M3)[0], "q")
