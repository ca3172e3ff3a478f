"""quantize_per_tensor_noalloc (the workspace-free entry point for callers that cannot allocate)
against quantize_per_tensor with a caller workspace, through the C ABI: codes, amax, scale and the
non-finite flag identical, on calls in a row on the library's one scratch array: an 8192x8192
BF16 activation (single-pass kernel, grid barrier in the scratch), then a smaller 256x512 tensor
(two-kernel path, partial maxima in the scratch), then FP32 and E5M2 inputs of both sizes, and the
large one again (the array left zero by every call)."""
import ctypes

import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
from synthetic import per_tensor_activation, per_tensor_small
from qf8_test_utils import host, to_device

pytestmark = pytest.mark.gpu


def run_noalloc(xd, fmt):
    rows, cols = xd.shape
    q = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device="cuda")
    am = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    sc = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    vp = ctypes.c_void_p
    dtype = 0 if xd.dtype == torch.bfloat16 else 1
    st = qf8._load().quantize_per_tensor_noalloc(vp(xd.data_ptr()), dtype, rows, cols, fmt, vp(q.data_ptr()),
                                                 vp(am.data_ptr()), vp(sc.data_ptr()), vp(nf.data_ptr()),
                                                 vp(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qf8.qf8_status_string(st)
    torch.cuda.synchronize()
    return host(q), np.float32(am.item()), np.float32(sc.item()), int(nf.item())


def run_with_workspace(xd, fmt):
    ws = qf8.workspace(xd)
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    q, am, sc = qf8.quantize_per_tensor(xd, fmt, nonfinite=nf, ws=ws)
    torch.cuda.synchronize()
    return host(q), np.float32(am.item()), np.float32(sc.item()), int(nf.item())


def check(x, fmt, tag):
    print(f"noalloc case: {tag}", flush=True)
    xd = to_device(x)
    got = run_noalloc(xd, fmt)
    want = run_with_workspace(xd, fmt)
    assert got[1] == want[1] and got[2] == want[2] and got[3] == want[3], (tag, got[1:], want[1:])
    assert np.array_equal(got[0], want[0]), f"{tag}: codes differ at {np.argwhere(got[0] != want[0])[:3].tolist()}"


def test_noalloc_matches_workspace_entry_point():
    big = per_tensor_activation()                       # 8192x8192 BF16: single-pass kernel
    small = per_tensor_small(256, 512, seed=1)          # 256x512 BF16: partial maxima + cast
    check(big, qf8.E4M3, "8192x8192 bf16 e4m3")
    check(small, qf8.E4M3, "256x512 bf16 e4m3 (smaller, second call)")
    rng = np.random.default_rng(7)
    check((rng.standard_normal((2048, 2048)) * 3).astype(np.float32), qf8.E5M2, "2048x2048 fp32 e5m2")
    check((rng.standard_normal((33, 48)) * 1e-3).astype(np.float32), qf8.E4M3, "33x48 fp32 e4m3")
    check(big, qf8.E5M2, "8192x8192 bf16 e5m2 (the array left zero by the calls before)")


def test_noalloc_argument_errors():
    """Argument errors are reported before the scratch array is touched."""
    f = qf8._load().quantize_per_tensor_noalloc
    fake = ctypes.c_void_p(0x10000)
    assert f(fake, 0, 4, 4, 7, fake, fake, fake, None, None) == -2        # bad fmt
    assert f(fake, 0, -1, 4, 0, fake, fake, fake, None, None) == -3       # bad shape
    assert f(fake, 0, 4, 4, 0, None, fake, fake, None, None) == -1        # no output
    assert f(ctypes.c_void_p(0x10008), 0, 4, 4, 0, fake, fake, fake, None, None) == -4
