"""Helpers shared by the GPU parity tests: device transfer, byte comparison, parallel oracle runs."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ORACLE_THREADS = min(16, os.cpu_count() or 1)


def to_device(x, device="cuda"):
    """numpy uint16 (BF16 bits), float32 or uint8 -> contiguous CUDA tensor holding the same bytes."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    if x.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    raise TypeError(x.dtype)


def host(t):
    return t.cpu().numpy()


def assert_bytes_equal(got, want, name, extra=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    if np.array_equal(got.view(np.uint8) if got.dtype != np.uint8 else got,
                      want.view(np.uint8) if want.dtype != np.uint8 else want):
        return
    g8 = got.reshape(-1).view(np.uint8) if got.dtype != np.uint8 else got.reshape(-1)
    w8 = want.reshape(-1).view(np.uint8) if want.dtype != np.uint8 else want.reshape(-1)
    bad = np.nonzero(g8 != w8)[0]
    i = int(bad[0])
    idx = np.unravel_index(i // max(1, got.dtype.itemsize), got.shape)
    raise AssertionError(f"{name}{extra}: {len(bad)} differing bytes; first at index {tuple(int(v) for v in idx)}: "
                         f"got {got.reshape(-1)[i // max(1, got.dtype.itemsize)]!r} "
                         f"want {want.reshape(-1)[i // max(1, want.dtype.itemsize)]!r}")


def parallel_row_slabs(fn, rows, slab):
    """Run fn(r0, r1) over row slabs [r0, r1) of height `slab` (the oracle is single-threaded C;
    ctypes releases the GIL, so slabs run concurrently). Returns the list of results in order."""
    bounds = [(r, min(r + slab, rows)) for r in range(0, rows, slab)]
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        return list(ex.map(lambda b: fn(*b), bounds))


def holder_lib():
    """The CU-holding kernel of the contention tests (tests/contention/holder.hip, built by
    __graft_entry__.build()): holder_launch(grid, lds_bytes, microseconds, sink, stream)."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "contention", "libholder.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.holder_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.holder_launch.restype = ctypes.c_int
    return lib


_HOLD_STREAMS = []


def time_beside_holders(lib, holders, call, hold_us=3000, lds=48 * 1024):
    """Launches the holder on its own stream (holders workgroups, each with lds bytes of LDS, for
    hold_us microseconds), then call() on another stream after a ~20 us delay that lets the
    holder's workgroups start first. Returns call()'s time in microseconds from HIP events on its
    stream, after a device synchronize. call() must allocate nothing: an allocation on the
    stream between the events would be timed too."""
    if not _HOLD_STREAMS:
        _HOLD_STREAMS.extend([torch.cuda.Stream(), torch.cuda.Stream(), torch.zeros(1, dtype=torch.int32, device="cuda")])
    hold, side, sink = _HOLD_STREAMS
    torch.cuda.synchronize()
    assert lib.holder_launch(holders, lds, hold_us, sink.data_ptr(), hold.cuda_stream) == 0
    with torch.cuda.stream(side):
        torch.cuda._sleep(50000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(side)
        call()
        e1.record(side)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3
