"""FP8 tensor quantization on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libqf8.so`` (C ABI in ``include/qf8.h``): the functions below carry the
C names, marshal torch tensors into device pointers and the current HIP stream, allocate output
tensors when none are given, and raise ``QF8Error`` on a non-zero status. Every step of the
quantization runs in the library's HIP kernels; there is no CPU path. torch supplies device
memory and streams only.

Formats: ``E4M3`` (max 448) and ``E5M2`` (max 57344), OCP encodings. Inputs: ``torch.bfloat16``
or ``torch.float32`` CUDA tensors, contiguous, 2-D ``[rows, cols]`` (1-D tensors count as one
row). Outputs are ``torch.uint8`` tensors of raw fp8 / E8M0 bytes.
"""
import ctypes
import os

import torch  # loaded first: the library binds to the HIP runtime torch has already loaded

__all__ = [
    "E4M3", "E5M2", "ROUND_DOWN", "ROUND_UP", "QF8Error", "library_path",
    "qf8_status_string", "qf8_workspace_bytes", "qf8_set_onepass_grid", "qf8_cast_scaled", "quantize_per_tensor",
    "DelayedState", "qf8_delayed_init", "qf8_delayed_init_ex", "qf8_delayed_reset", "quantize_delayed",
    "EST_MAX", "EST_RECENT", "EST_MEAN", "DELAYED_SPLIT_AMAX",
    "quantize_block", "quantize_mx_dual", "quantize_mxfp4_dual", "quantize_nvfp4", "dequantize_mxfp4",
    "dequantize_nvfp4",
]

E4M3, E5M2 = 0, 1
ROUND_DOWN, ROUND_UP = 0, 1
FLAG_POW2_SCALES = 1
EST_MAX, EST_RECENT, EST_MEAN = 0, 1, 2   # delayed-scaling estimators (qf8_estimator)
DELAYED_SPLIT_AMAX = 1                    # qf8_delayed_flags
_BF16, _FP32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqf8.so")
_lib = None


class QF8Error(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {qf8_status_string(status)} ({status})")


class _DelayedStruct(ctypes.Structure):
    _fields_ = [("history", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("hist_len", ctypes.c_int32), ("interval", ctypes.c_int32), ("n_guard", ctypes.c_int32),
                ("fmt", ctypes.c_int32), ("step", ctypes.c_int64), ("magic", ctypes.c_int32),
                ("estimator", ctypes.c_int32), ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run `python -m mx_block_scaled_amax_amd.build` "
                          "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sigs = {
        "qf8_status_string": (ctypes.c_char_p, [i32]),
        "qf8_workspace_bytes": (sz, [i64, i64, i32]),
        "qf8_workspace_init": (i32, [vp, sz, vp]),
        "qf8_set_onepass_grid": (i32, [i32]),
        "qf8_cast_scaled": (i32, [vp, i32, i64, i32, vp, vp, vp]),
        "quantize_per_tensor": (i32, [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, sz, vp]),
        "quantize_per_tensor_noalloc": (i32, [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp]),
        "qf8_delayed_init": (i32, [ctypes.POINTER(_DelayedStruct), vp, vp, vp, i32, i32, i32, i32, vp]),
        "qf8_delayed_init_ex": (i32, [ctypes.POINTER(_DelayedStruct), vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]),
        "qf8_delayed_reset": (i32, [ctypes.POINTER(_DelayedStruct), vp]),
        "quantize_delayed": (i32, [vp, i32, i64, i64, i32, ctypes.POINTER(_DelayedStruct), vp, vp, vp, vp, vp, sz, vp]),
        "quantize_block": (i32, [vp, i32, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp]),
        "quantize_block_ex": (i32, [vp, i32, i64, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
        "requantize_1x128_to_128x1": (i32, [vp, vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]),
        "quantize_mx_dual": (i32, [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp]),
        "quantize_mxfp4_dual": (i32, [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp]),
        "quantize_nvfp4": (i32, [vp, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "dequantize_mxfp4": (i32, [vp, vp, i64, i64, vp, i32, vp]),
        "dequantize_nvfp4": (i32, [vp, vp, vp, i64, i64, vp, i32, vp]),
        "dequantize_scaled": (i32, [vp, i64, i32, vp, vp, i32, vp, i32, vp, vp, sz, vp]),
        "dequantize_block": (i32, [vp, i64, i64, i32, i32, i32, vp, vp, i32, vp, i32, vp, vp, sz, vp]),
        "dequantize_mx": (i32, [vp, vp, i64, i64, i32, vp, i32, vp, i32, vp, vp, sz, vp]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def qf8_status_string(status):
    return _load().qf8_status_string(int(status)).decode()


def _check(status, what):
    if status != 0:
        raise QF8Error(status, what)


def _dtype_code(x):
    if x.dtype == torch.bfloat16:
        return _BF16
    if x.dtype == torch.float32:
        return _FP32
    raise TypeError(f"input must be torch.bfloat16 or torch.float32, got {x.dtype}")


def _dev_tensor(x, name):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor; the library has no CPU path")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x


def _rows_cols(x):
    if x.dim() == 1:
        return 1, x.shape[0]
    if x.dim() != 2:
        raise ValueError("expected a 1-D or 2-D tensor")
    return x.shape[0], x.shape[1]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev_tensor(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}")
    return t


def qf8_workspace_bytes(rows, cols, dtype=torch.bfloat16):
    return _load().qf8_workspace_bytes(rows, cols, _BF16 if dtype == torch.bfloat16 else _FP32)


# Mirrors of two library constants, for tests: the number of leading u32 words of a workspace
# that every call leaves zero (grid-barrier header line, 512 release lines and 256 amax slot
# lines, 32 words each), and the element count from which quantize_per_tensor uses the
# single-pass kernel.
BARRIER_WORDS = 32 + 512 * 32 + 256 * 32
ONEPASS_MIN_ELEMS = 1 << 22


def qf8_set_onepass_grid(grid):
    """Workgroups of the single-pass kernel on the current device (1..512), 0 = one per CU."""
    _check(_load().qf8_set_onepass_grid(int(grid)), "qf8_set_onepass_grid")


def qf8_workspace_init(ws, stream=None):
    """Zero-fill a workspace (uint8 device tensor) on the stream, as it must be before first use."""
    _dev_tensor(ws, "ws")
    _check(_load().qf8_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream, ws.device)),
           "qf8_workspace_init")
    return ws


def workspace(x, stream=None):
    """A zero-initialised device workspace for quantize_per_tensor / quantize_delayed on x. It
    may be reused by any number of later calls ordered on one stream."""
    rows, cols = _rows_cols(x)
    ws = torch.empty(qf8_workspace_bytes(rows, cols, x.dtype), dtype=torch.uint8, device=x.device)
    return qf8_workspace_init(ws, stream)


def qf8_cast_scaled(x, fmt, scale, q=None, stream=None):
    """q = sat_rne8(fl32(x * scale)); scale is a 1-element float32 device tensor."""
    _dev_tensor(x, "x")
    _dev_tensor(scale, "scale")
    q = _out(q, tuple(x.shape), torch.uint8, x.device, "q")
    _check(_load().qf8_cast_scaled(_ptr(x), _dtype_code(x), x.numel(), fmt, _ptr(scale), _ptr(q),
                                   _stream(stream, x.device)), "qf8_cast_scaled")
    return q


def quantize_per_tensor(x, fmt, q=None, amax=None, scale=None, nonfinite=None, ws=None, stream=None):
    """Per-tensor current scaling. Returns (q, amax, scale) as device tensors."""
    _dev_tensor(x, "x")
    rows, cols = _rows_cols(x)
    dev = x.device
    q = _out(q, tuple(x.shape), torch.uint8, dev, "q")
    amax = _out(amax, (1,), torch.float32, dev, "amax")
    scale = _out(scale, (1,), torch.float32, dev, "scale")
    ws = workspace(x) if ws is None else _dev_tensor(ws, "ws")
    _check(_load().quantize_per_tensor(_ptr(x), _dtype_code(x), rows, cols, fmt, _ptr(q), _ptr(amax), _ptr(scale),
                                       _ptr(nonfinite), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream, dev)), "quantize_per_tensor")
    return q, amax, scale


class DelayedState:
    """Device state of per-tensor delayed scaling: history FIFO, meta (count, head), next scale."""

    def __init__(self, hist_len, interval, n_guard, fmt, device="cuda", stream=None, estimator=None, split=False):
        self.history = torch.zeros(hist_len, dtype=torch.float32, device=device)
        self.meta = torch.zeros(4, dtype=torch.int32, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        self.struct = _DelayedStruct()
        self.device = self.history.device
        if estimator is None and not split:
            qf8_delayed_init(self, hist_len, interval, n_guard, fmt, stream)
        else:
            qf8_delayed_init_ex(self, hist_len, interval, n_guard, fmt, estimator or EST_MAX,
                                DELAYED_SPLIT_AMAX if split else 0, stream)

    @property
    def step(self):
        return self.struct.step

    @step.setter
    def step(self, v):
        self.struct.step = int(v)

    def history_list(self):
        """History oldest-first (synchronizes)."""
        count, head = (int(v) for v in self.meta[:2].cpu())
        h = self.history.cpu().tolist()
        n = self.struct.hist_len
        return [h[(head + i) % n] for i in range(count)]


def qf8_delayed_init(state, hist_len, interval, n_guard, fmt, stream=None):
    _check(_load().qf8_delayed_init(ctypes.byref(state.struct), _ptr(state.history), _ptr(state.meta),
                                    _ptr(state.scale), hist_len, interval, n_guard, fmt,
                                    _stream(stream, state.device)), "qf8_delayed_init")


def qf8_delayed_init_ex(state, hist_len, interval, n_guard, fmt, estimator, flags=0, stream=None):
    _check(_load().qf8_delayed_init_ex(ctypes.byref(state.struct), _ptr(state.history), _ptr(state.meta),
                                       _ptr(state.scale), hist_len, interval, n_guard, fmt, estimator, flags,
                                       _stream(stream, state.device)), "qf8_delayed_init_ex")


def qf8_delayed_reset(state, stream=None):
    _check(_load().qf8_delayed_reset(ctypes.byref(state.struct), _stream(stream, state.device)), "qf8_delayed_reset")


def quantize_delayed(x, state, q=None, scale_used=None, amax_out=None, nonfinite=None, ws=None, stream=None):
    """One delayed-scaling iteration in the state's format. Returns q; scale_used / amax_out are
    filled when given."""
    _dev_tensor(x, "x")
    rows, cols = _rows_cols(x)
    q = _out(q, tuple(x.shape), torch.uint8, x.device, "q")
    ws = workspace(x) if ws is None else _dev_tensor(ws, "ws")
    _check(_load().quantize_delayed(_ptr(x), _dtype_code(x), rows, cols, state.struct.fmt, ctypes.byref(state.struct),
                                    _ptr(q),
                                    _ptr(scale_used), _ptr(amax_out), _ptr(nonfinite), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream, x.device)), "quantize_delayed")
    return q


def quantize_block(x, block_rows, block_cols, fmt, q=None, scales=None, amax=None, nonfinite=None, stream=None,
                   want_amax=True, pow2_scales=False):
    """1x128 or 128x128 group scaling (power-of-two group scales with pow2_scales).
    Returns (q, scales, amax-or-None)."""
    _dev_tensor(x, "x")
    rows, cols = _rows_cols(x)
    gshape = (-(-rows // block_rows), -(-cols // block_cols))
    q = _out(q, tuple(x.shape), torch.uint8, x.device, "q")
    scales = _out(scales, gshape, torch.float32, x.device, "scales")
    if amax is None and want_amax:
        amax = torch.empty(gshape, dtype=torch.float32, device=x.device)
    _check(_load().quantize_block_ex(_ptr(x), _dtype_code(x), rows, cols, block_rows, block_cols, fmt,
                                     FLAG_POW2_SCALES if pow2_scales else 0, _ptr(q), _ptr(scales), _ptr(amax),
                                     _ptr(nonfinite), _stream(stream, x.device)), "quantize_block_ex")
    return q, scales, amax


def requantize_1x128_to_128x1(q, scales, fmt_in, fmt_out, pow2_scales=True, qT=None, scalesT=None, nonfinite=None,
                              stream=None):
    """Re-group 1x128-quantized q [rows][cols] (with its group scales) into 128x1 groups, stored
    transposed. Returns (qT [cols][rows], scalesT [cols][ceil(rows/128)])."""
    _dev_tensor(q, "q")
    _dev_tensor(scales, "scales")
    rows, cols = _rows_cols(q)
    dev = q.device
    qT = _out(qT, (cols, rows), torch.uint8, dev, "qT")
    scalesT = _out(scalesT, (cols, -(-rows // 128)), torch.float32, dev, "scalesT")
    _check(_load().requantize_1x128_to_128x1(_ptr(q), _ptr(scales), rows, cols, fmt_in, fmt_out,
                                             FLAG_POW2_SCALES if pow2_scales else 0, _ptr(qT), _ptr(scalesT),
                                             _ptr(nonfinite), _stream(stream, dev)), "requantize_1x128_to_128x1")
    return qT, scalesT


def quantize_mx_dual(x, fmt, rnd, rowwise=True, colwise=True, q_row=None, s_row=None, q_colT=None, s_colT=None,
                     nonfinite=None, stream=None):
    """MX 1x32 quantization. Returns (q_row, s_row, q_colT, s_colT); a direction not asked for is None."""
    _dev_tensor(x, "x")
    rows, cols = _rows_cols(x)
    dev = x.device
    if rowwise:
        q_row = _out(q_row, (rows, cols), torch.uint8, dev, "q_row")
        s_row = _out(s_row, (rows, cols // 32), torch.uint8, dev, "s_row")
    else:
        q_row = s_row = None
    if colwise:
        q_colT = _out(q_colT, (cols, rows), torch.uint8, dev, "q_colT")
        s_colT = _out(s_colT, (cols, rows // 32), torch.uint8, dev, "s_colT")
    else:
        q_colT = s_colT = None
    _check(_load().quantize_mx_dual(_ptr(x), _dtype_code(x), rows, cols, fmt, rnd, _ptr(q_row), _ptr(s_row),
                                    _ptr(q_colT), _ptr(s_colT), _ptr(nonfinite), _stream(stream, dev)),
           "quantize_mx_dual")
    return q_row, s_row, q_colT, s_colT


def quantize_mxfp4_dual(x, rnd, rowwise=True, colwise=True, q_row=None, s_row=None, q_colT=None, s_colT=None,
                        nonfinite=None, stream=None):
    """MXFP4 (E2M1, 1x32 E8M0). Codes packed two per byte. Returns (q_row [rows][cols/2], s_row,
    q_colT [cols][rows/2], s_colT); a direction not asked for is None."""
    _dev_tensor(x, "x")
    rows, cols = _rows_cols(x)
    dev = x.device
    if rowwise:
        q_row = _out(q_row, (rows, cols // 2), torch.uint8, dev, "q_row")
        s_row = _out(s_row, (rows, cols // 32), torch.uint8, dev, "s_row")
    else:
        q_row = s_row = None
    if colwise:
        q_colT = _out(q_colT, (cols, rows // 2), torch.uint8, dev, "q_colT")
        s_colT = _out(s_colT, (cols, rows // 32), torch.uint8, dev, "s_colT")
    else:
        q_colT = s_colT = None
    _check(_load().quantize_mxfp4_dual(_ptr(x), _dtype_code(x), rows, cols, rnd, _ptr(q_row), _ptr(s_row),
                                       _ptr(q_colT), _ptr(s_colT), _ptr(nonfinite), _stream(stream, dev)),
           "quantize_mxfp4_dual")
    return q_row, s_row, q_colT, s_colT


def quantize_nvfp4(x, amax_in=None, q=None, s_blk=None, tensor_scale=None, amax_out=None, nonfinite=None, ws=None,
                   stream=None):
    """NVFP4 (E2M1, 1x16 E4M3 block scales, fp32 tensor scale). Returns (q [rows][cols/2] packed,
    s_blk [rows][cols/16], tensor_scale [1]). amax_in: optional device fp32 tensor amax."""
    _dev_tensor(x, "x")
    rows, cols = _rows_cols(x)
    dev = x.device
    q = _out(q, (rows, cols // 2), torch.uint8, dev, "q")
    s_blk = _out(s_blk, (rows, cols // 16), torch.uint8, dev, "s_blk")
    tensor_scale = _out(tensor_scale, (1,), torch.float32, dev, "tensor_scale")
    if amax_in is None and ws is None:
        ws = workspace(x)
    _check(_load().quantize_nvfp4(_ptr(x), _dtype_code(x), rows, cols, _ptr(amax_in), _ptr(q), _ptr(s_blk),
                                  _ptr(tensor_scale), _ptr(amax_out), _ptr(nonfinite), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream(stream, dev)),
           "quantize_nvfp4")
    return q, s_blk, tensor_scale



def _fp4_out(out, out_dtype, rows, cols, dev):
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    return _out(out, (rows, cols), out_dtype, dev, "out")


def dequantize_mxfp4(q, sb, out_dtype=torch.bfloat16, out=None, stream=None):
    """MXFP4 de-scaling: q [rows][cols/2] packed, sb [rows][cols/32] E8M0 -> out [rows][cols]."""
    _dev_tensor(q, "q")
    _dev_tensor(sb, "sb")
    rows, cols = q.shape[0], q.shape[1] * 2
    out = _fp4_out(out, out_dtype, rows, cols, q.device)
    _check(_load().dequantize_mxfp4(_ptr(q), _ptr(sb), rows, cols, _ptr(out),
                                    _BF16 if out.dtype == torch.bfloat16 else _FP32,
                                    _stream(stream, q.device)), "dequantize_mxfp4")
    return out


def dequantize_nvfp4(q, s_blk, tensor_scale, out_dtype=torch.bfloat16, out=None, stream=None):
    """NVFP4 de-scaling: q [rows][cols/2] packed, s_blk [rows][cols/16] E4M3, tensor_scale [1]."""
    _dev_tensor(q, "q")
    _dev_tensor(s_blk, "s_blk")
    _dev_tensor(tensor_scale, "tensor_scale")
    rows, cols = q.shape[0], q.shape[1] * 2
    out = _fp4_out(out, out_dtype, rows, cols, q.device)
    _check(_load().dequantize_nvfp4(_ptr(q), _ptr(s_blk), _ptr(tensor_scale), rows, cols, _ptr(out),
                                    _BF16 if out.dtype == torch.bfloat16 else _FP32,
                                    _stream(stream, q.device)), "dequantize_nvfp4")
    return out


# ---- dequantization and error statistics ------------------------------------------------------

STATS_FIELDS = ("signal", "noise", "count", "nonzero", "zeroed", "saturated", "nonfinite")


def stats_to_dict(stats):
    """Read a qf8_error_stats device tensor (8 x int64) back to the host (synchronizes)."""
    import numpy as np
    raw = stats.detach().cpu().numpy().view(np.uint8)
    f = raw[:16].view(np.float64)
    i = raw[16:].view(np.int64)
    return {"signal": float(f[0]), "noise": float(f[1]), "count": int(i[0]), "nonzero": int(i[1]),
            "zeroed": int(i[2]), "saturated": int(i[3]), "nonfinite": int(i[4])}


def _dq_common(q, out_dtype, out, shape, x, want_out, ws, dev):
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    out_code = _BF16 if out_dtype == torch.bfloat16 else _FP32
    if want_out:
        out = _out(out, shape, out_dtype, dev, "out")
    else:
        out = None
    stats = None
    x_code = 0
    if x is not None:
        _dev_tensor(x, "x")
        if tuple(x.shape) != tuple(shape):
            raise ValueError(f"x must have the shape of q, {tuple(shape)}")
        x_code = _dtype_code(x)
        stats = torch.zeros(8, dtype=torch.int64, device=dev)
        if ws is None:
            ws = torch.empty(_load().qf8_workspace_bytes(1, 1, 0), dtype=torch.uint8, device=dev)
        else:
            _dev_tensor(ws, "ws")
    if out is None and stats is None:
        raise ValueError("nothing to do: ask for the output (want_out) or pass x for statistics")
    return out, out_code, stats, x_code, ws


def dequantize_scaled(q, fmt, scale, out_dtype=torch.bfloat16, out=None, x=None, want_out=True, ws=None, stream=None):
    """xhat = fl32(decode(q) / scale) for a per-tensor (or delayed) result; scale is a 1-element
    float32 device tensor. With x (the source tensor), also error statistics. Returns
    (out or None, stats device tensor or None)."""
    _dev_tensor(q, "q")
    _dev_tensor(scale, "scale")
    dev = q.device
    out, oc, stats, xc, ws = _dq_common(q, out_dtype, out, tuple(q.shape), x, want_out, ws, dev)
    _check(_load().dequantize_scaled(_ptr(q), q.numel(), fmt, _ptr(scale), _ptr(out), oc, _ptr(x), xc, _ptr(stats),
                                     _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream, dev)),
           "dequantize_scaled")
    return out, stats


def dequantize_block(q, block_rows, block_cols, fmt, scales, out_dtype=torch.bfloat16, out=None, x=None,
                     want_out=True, ws=None, stream=None):
    """Per-group de-scaling of a quantize_block result (groups of block_rows x block_cols)."""
    _dev_tensor(q, "q")
    _dev_tensor(scales, "scales")
    rows, cols = _rows_cols(q)
    dev = q.device
    out, oc, stats, xc, ws = _dq_common(q, out_dtype, out, tuple(q.shape), x, want_out, ws, dev)
    _check(_load().dequantize_block(_ptr(q), rows, cols, block_rows, block_cols, fmt, _ptr(scales), _ptr(out), oc,
                                    _ptr(x), xc, _ptr(stats), _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(stream, dev)), "dequantize_block")
    return out, stats


def dequantize_mx(q, s, fmt, out_dtype=torch.bfloat16, out=None, x=None, want_out=True, ws=None, stream=None):
    """MX de-scaling of q [rows][cols] with E8M0 bytes s [rows][cols/32] (a rowwise result, or a
    columnwise one in its transposed layout; then x is the source transposed)."""
    _dev_tensor(q, "q")
    _dev_tensor(s, "s")
    rows, cols = _rows_cols(q)
    dev = q.device
    out, oc, stats, xc, ws = _dq_common(q, out_dtype, out, tuple(q.shape), x, want_out, ws, dev)
    _check(_load().dequantize_mx(_ptr(q), _ptr(s), rows, cols, fmt, _ptr(out), oc, _ptr(x), xc, _ptr(stats),
                                 _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream, dev)), "dequantize_mx")
    return out, stats
