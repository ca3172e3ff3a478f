"""GPU parity of quantize_per_tensor and qf8_cast_scaled against the CPU oracle (bit-exact codes,
amax and fp32 scale).

  * the device encoder: every BF16 input times 1259 scales (powers of two over the whole fp32
    exponent range, the pages' worked-example scales, random scales), and random FP32 inputs;
  * the scale division: every positive finite BF16 amax -> S = fl32(F8max/amax);
  * the 256x512 workload and the full 8192x8192 activation workload, E4M3 and E5M2;
  * ragged and degenerate sizes: empty, one element, lengths that are not multiples of the
    16-byte vector, all-zero input, amax so small that F8max/amax overflows, Inf/NaN flag.
"""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import bf16_to_f32, per_tensor_activation, per_tensor_small, small_tensor
from qf8_test_utils import (assert_bytes_equal, holder_lib, host, parallel_row_slabs, time_beside_holders,
                             to_device)

pytestmark = pytest.mark.gpu
FMTS = [O.E4M3, O.E5M2]


def scale_set():
    rng = np.random.default_rng(11)
    s = [1.0, 22400.0, float(np.float32(448 / 20)), float(np.float32(448 / 50))]
    s += [2.0 ** -k for k in range(-127, 128)]
    s += list((2.0 ** rng.uniform(-40, 40, 1000)).astype(np.float32))
    return np.array(s, np.float32)


@pytest.mark.parametrize("fmt", FMTS)
def test_cast_exhaustive_bf16_times_scales(fmt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[~np.isnan(bf16_to_f32(bits))]
    xd = to_device(bits)
    q = torch.empty(len(bits), dtype=torch.uint8, device="cuda")
    sd = torch.empty(1, dtype=torch.float32, device="cuda")
    for s in scale_set():
        sd.fill_(float(s))
        qf8.qf8_cast_scaled(xd, fmt, sd, q=q)
        assert_bytes_equal(host(q), O.cast(bits, fmt, s), "q", f" [scale={s!r}]")


@pytest.mark.parametrize("fmt", FMTS)
def test_cast_random_fp32(fmt):
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32).copy()
    x[~np.isfinite(x)] = 0.0
    xd = to_device(x)
    sd = torch.empty(1, dtype=torch.float32, device="cuda")
    for s in (1.0, 2.0 ** -100, 2.0 ** 100, 3.0e-20, 7.5e15):
        sd.fill_(s)
        q = qf8.qf8_cast_scaled(xd, fmt, sd)
        assert_bytes_equal(host(q), O.cast(x, fmt, np.float32(s)), "q", f" [fp32 scale={s}]")


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_for_every_bf16_amax(fmt):
    # one 1x128 group per amax value would also do; here a per-tensor call per value is too slow,
    # so the block kernel's group scales (same division) are checked in test_gpu_block.py and the
    # per-tensor path is checked on a spread of amax values
    for a in (0x0001, 0x0080, 0x3C00, 0x3F80, 0x4000, 0x43E0, 0x43E1, 0x7F7F, 0x1234, 0x0A0A):
        x = np.array([[a, 0x0000, a | 0x8000, 0x3F80 if a > 0x3F80 else 0x0000]], np.uint16)
        q, am, s = qf8.quantize_per_tensor(to_device(x), fmt)
        wq, wa, ws, _ = O.quantize_per_tensor(x, fmt)
        assert am.item() == wa and np.float32(s.item()) == ws, hex(a)
        assert_bytes_equal(host(q), wq, "q", f" [amax bits {a:#x}]")


def run_pt(x, fmt):
    xd = to_device(x)
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    q = torch.full(x.shape, 0xA5, dtype=torch.uint8, device="cuda")
    q, am, s = qf8.quantize_per_tensor(xd, fmt, q=q, nonfinite=nf)
    torch.cuda.synchronize()
    return host(q), np.float32(am.item()), np.float32(s.item()), int(nf.item())


@pytest.mark.parametrize("fmt", FMTS)
def test_small_workload(fmt):
    x = per_tensor_small()
    q, am, s, nf = run_pt(x, fmt)
    wq, wa, ws, wnf = O.quantize_per_tensor(x, fmt)
    assert (am, s, nf) == (wa, ws, wnf)
    assert_bytes_equal(q, wq, "q")


@pytest.mark.parametrize("shape", [(0, 0), (1, 1), (1, 7), (3, 5), (7, 9), (1, 1031), (13, 333), (1, 8 * 1024 * 1024 + 3)])
@pytest.mark.parametrize("fmt", FMTS)
def test_ragged_sizes(shape, fmt):
    x = small_tensor(*shape, seed=shape[0] * 7 + shape[1]) if shape[0] * shape[1] else np.zeros(shape, np.uint16)
    q, am, s, nf = run_pt(x, fmt)
    wq, wa, ws, wnf = O.quantize_per_tensor(x, fmt)
    assert (am, s, nf) == (wa, ws, wnf)
    assert_bytes_equal(q, wq, "q", f" [{shape}]")


@pytest.mark.parametrize("fmt", FMTS)
def test_fp32_input(fmt):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((100, 37)) * np.where(rng.random((100, 37)) < 0.01, 300, 1)).astype(np.float32)
    q, am, s, nf = run_pt(x, fmt)
    wq, wa, ws, wnf = O.quantize_per_tensor(x, fmt)
    assert (am, s, nf) == (wa, ws, wnf)
    assert_bytes_equal(q, wq, "q")


def test_degenerate_amax():
    z = np.zeros((4, 64), np.uint16)
    z[1, 3] = 0x8000
    q, am, s, nf = run_pt(z, O.E4M3)
    assert am == 0 and s == 1.0 and nf == 0
    assert_bytes_equal(q, O.quantize_per_tensor(z, O.E4M3)[0], "q")
    tiny = np.zeros((2, 16), np.uint16)
    tiny[0, 0] = 0x0003                   # subnormal amax: F8max/amax overflows fp32
    q, am, s, nf = run_pt(tiny, O.E4M3)
    assert s == np.finfo(np.float32).max
    assert_bytes_equal(q, O.quantize_per_tensor(tiny, O.E4M3)[0], "q")


def test_nonfinite_flag():
    x = small_tensor(8, 64, seed=1)
    x[2, 2] = 0x7F80
    q, am, s, nf = run_pt(x, O.E4M3)
    assert nf == 1 and np.isinf(am) and s == 1.0
    x[2, 2] = 0xFFC0
    q, am, s, nf = run_pt(x, O.E5M2)
    assert nf == 1 and np.isnan(am)


@pytest.fixture(scope="module")
def activation_full():
    return per_tensor_activation()


@pytest.mark.parametrize("fmt", FMTS)
def test_full_size_activation(activation_full, fmt):
    x = activation_full
    q, am, s, nf = run_pt(x, fmt)
    wa = np.float32(O.amax(x))
    ws = np.float32(O.scale_from_amax(fmt, wa))
    assert am == wa and s == ws and nf == 0
    parts = parallel_row_slabs(lambda r0, r1: O.cast(x[r0:r1], fmt, ws), x.shape[0], 512)
    assert_bytes_equal(q, np.concatenate(parts, axis=0), "q", " [8192x8192]")


# ---- the single-pass kernel (tensors of ONEPASS_MIN_ELEMS elements and more) ----------------

def onchip_capacity_elems(dtype_bytes):
    """Elements the single-pass kernel keeps on chip: one 512-thread workgroup per CU, 64 slabs
    of 512 16-byte vectors each."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return min(cus, 512) * 512 * 64 * (16 // dtype_bytes)


def oracle_flat(x, fmt):
    """Oracle per-tensor result for a large tensor, its cast split over flat slabs in threads."""
    flat = x.reshape(-1)
    wa = np.float32(O.amax(flat))
    ws = np.float32(O.scale_from_amax(fmt, wa))
    step = 1 << 22
    parts = parallel_row_slabs(lambda i0, i1: O.cast(flat[i0 * step:i1 * step], fmt, ws), (flat.size + step - 1) // step, 1)
    return np.concatenate(parts).reshape(x.shape), wa, ws


def barrier_words(ws):
    return host(ws.view(torch.int32)[:qf8.BARRIER_WORDS]).astype(np.int64)


def run_with_ws(x, fmt, ws):
    xd = to_device(x)
    q = torch.full(x.shape, 0xA5, dtype=torch.uint8, device="cuda")
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    q, am, s = qf8.quantize_per_tensor(xd, fmt, q=q, nonfinite=nf, ws=ws)
    torch.cuda.synchronize()
    return host(q), np.float32(am.item()), np.float32(s.item()), int(nf.item())


def check_big(x, fmt, ws, tag):
    q, am, s, nf = run_with_ws(x, fmt, ws)
    wq, wa, wsc = oracle_flat(x, fmt)
    assert (am, s, nf) == (wa, wsc, 0), tag
    assert_bytes_equal(q, wq, "q", f" [{tag}]")
    words = barrier_words(ws)
    words[2] = 0                                     # the timeout override is the caller's
    assert not words.any(), f"barrier region not left zero [{tag}]"


def test_onepass_threshold_and_capacity_bf16():
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    cap = onchip_capacity_elems(2)
    for n, seed in ((qf8.ONEPASS_MIN_ELEMS - 1, 1), (qf8.ONEPASS_MIN_ELEMS, 2), (cap + 8, 3), (cap + cap // 2 + 5, 4)):
        print(f"onepass bf16 n={n}", flush=True)
        x = small_tensor(1, n, seed=seed)
        check_big(x, O.E4M3 if seed % 2 else O.E5M2, ws, f"bf16 n={n}")


def test_onepass_fp32():
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    rng = np.random.default_rng(8)
    cap = onchip_capacity_elems(4)
    for shape in ((cap // 4096, 4096), (1, cap + cap // 3 + 3)):
        print(f"onepass fp32 {shape}", flush=True)
        x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(3.0)).astype(np.float32)
        check_big(x, O.E4M3, ws, f"fp32 {shape}")


@pytest.mark.parametrize("ticks", [1, 100])
def test_onepass_give_up_path(activation_full, ticks):
    """Force waiting workgroups to give up at the grid barrier (timeout override in workspace
    word 2): 1 tick (10 ns) times every waiter out at once and repeatedly, so that nearly all
    give up; 100 ticks (1 us) lets part of them give up. Their slabs are then cast by the
    released workgroups together. Same bytes, barrier left clean."""
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    ws.view(torch.int32)[2] = ticks
    check_big(activation_full, O.E4M3, ws, f"give-up after {ticks} ticks")
    ws.view(torch.int32)[2] = 0
    check_big(activation_full, O.E4M3, ws, "default timeout after a give-up run")


@pytest.mark.parametrize("grid", [1, 17, 250, 300])
def test_onepass_other_grids(grid):
    """The single-pass kernel with other workgroup counts: one workgroup; 17 and 250 (the last
    barrier group of 16 is ragged: 1 and 10 workgroups); 300 on a 256-CU device, where 44
    workgroups only become resident after waiters have given up, and the released workgroups
    cast the given-up slabs. A tensor above the 128 MiB held on chip by 256 workgroups also streams slabs."""
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    qf8.qf8_set_onepass_grid(grid)
    try:
        for n, seed in ((qf8.ONEPASS_MIN_ELEMS + 24, 31 + grid), ((3 << 22) + 5, 32 + grid)):
            print(f"onepass grid={grid} n={n}", flush=True)
            x = small_tensor(1, n, seed=seed)
            check_big(x, O.E4M3 if seed % 2 else O.E5M2, ws, f"grid {grid}, n={n}")
    finally:
        qf8.qf8_set_onepass_grid(0)


@pytest.mark.parametrize("holders,size", [(8, "8192x8192"), (64, "8192x8192"), (8, "beyond the held capacity")])
def test_onepass_beside_cu_holders(activation_full, holders, size):
    """A kernel on another stream holds 48 KiB of LDS on `holders` CUs for 3 ms (so one workgroup
    of the single-pass kernel no longer fits on those CUs) while a single-pass call runs: that
    many workgroups cannot become resident. About as many waiters give up, on every shader
    engine, the late workgroups take their CUs, and the others share the given-up slabs (beyond
    the held capacity those include slabs that are streamed twice). The bytes, the amax and the
    scale are unchanged, the workspace is left zero, and the call ends within the give-up
    timeout (~53 us at 8192x8192) plus a few uncontended calls: it is timed with events on its
    stream and must end in under 1 ms, long before the holder (a design where every waiter gives
    up after 1 ms and one workgroup casts all of their slabs took 2.8-4.5 ms)."""
    lib = holder_lib()
    if size == "8192x8192":
        x = activation_full
    else:
        x = small_tensor(1, onchip_capacity_elems(2) + onchip_capacity_elems(2) // 3 + 5, seed=61)
    xd = to_device(x)
    ws = qf8.workspace(xd)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    am = torch.empty(1, dtype=torch.float32, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    wq, wa, wsc = oracle_flat(x, O.E4M3)
    times = []
    for rep in range(3):
        print(f"beside {holders} CU holders, {size}, rep {rep}", flush=True)
        q.fill_(0xA5)
        times.append(time_beside_holders(lib, holders, lambda: qf8.quantize_per_tensor(xd, O.E4M3, q=q, amax=am, scale=sc,
                                                                                       ws=ws)))
        assert np.float32(am.item()) == wa and np.float32(sc.item()) == wsc, rep
        assert_bytes_equal(host(q), wq, "q", f" [beside {holders} CU holders, {size}, rep {rep}]")
        words = barrier_words(ws)
        words[2] = 0
        assert not words.any(), "barrier region not left zero"
    print(f"call times beside {holders} CU holders, {size} (us): {[round(t) for t in times]}", flush=True)
    assert max(times) < 1000.0, times


def test_onepass_workspace_reuse():
    """One workspace across calls of both paths and several sizes, in a row on one stream."""
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    for n, seed in ((5 << 20, 11), (1000, 12), (6 << 20 | 3, 13), (5 << 20, 14)):
        x = small_tensor(1, n, seed=seed)
        check_big(x, O.E4M3, ws, f"reuse n={n}")


def test_onepass_beside_a_busy_stream(activation_full):
    """The single-pass kernel while another stream keeps CUs busy with a long fp32 matmul: some
    workgroups may not be resident when the others reach the grid barrier, so waiters can give
    up and the released workgroups cast their slabs. The bytes must not depend on it."""
    x = activation_full
    xd = to_device(x)
    ws = qf8.workspace(xd)
    a = torch.randn(8192, 8192, device="cuda")
    b = torch.randn(8192, 8192, device="cuda")
    busy = torch.cuda.Stream()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    results = []
    for rep in range(3):
        with torch.cuda.stream(busy):
            c = a @ b                                     # several milliseconds of work
        with torch.cuda.stream(side):
            q, am, sc = qf8.quantize_per_tensor(xd, O.E4M3, ws=ws)
        torch.cuda.synchronize()
        results.append((host(q), float(am.item()), float(sc.item())))
        del c
    wa = np.float32(O.amax(x))
    wsc = np.float32(O.scale_from_amax(O.E4M3, wa))
    parts = parallel_row_slabs(lambda r0, r1: O.cast(x[r0:r1], O.E4M3, wsc), x.shape[0], 512)
    want = np.concatenate(parts, axis=0)
    for rep, (q, am, sc) in enumerate(results):
        assert np.float32(am) == wa and np.float32(sc) == wsc, rep
        assert_bytes_equal(q, want, "q", f" [beside a busy stream, rep {rep}]")
    words = barrier_words(ws)
    words[2] = 0
    assert not words.any(), "barrier region not left zero"
