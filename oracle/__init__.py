"""CPU oracle for FP8 tensor quantization (test infrastructure).

A plain, slow C implementation (``qf8_oracle.c``) of what the quantization path computes,
wrapped with ctypes. Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package; the product path never does. It shares no code
with the GPU library (``mx_block_scaled_amax_amd``), and neither imports the other.

Arrays: BF16 tensors are ``numpy.uint16`` arrays of raw bit patterns, FP32 tensors are
``numpy.float32`` arrays. Formats: 0 = E4M3, 1 = E5M2, 2 = E8M0 (decode only).
MX rounding: 0 = OCP round-down, 1 = round-up.
"""
import ctypes
import os
import subprocess

import numpy as np

E4M3, E5M2, E8M0, E2M1 = 0, 1, 2, 3
ROUND_DOWN, ROUND_UP = 0, 1
EST_MAX, EST_RECENT, EST_MEAN = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qf8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqf8_oracle.so")
_lib = None

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def build():
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.qf8o_decode.restype = ctypes.c_double
    lib.qf8o_decode.argtypes = [ctypes.c_int, ctypes.c_uint]
    lib.qf8o_encode.restype = ctypes.c_uint
    lib.qf8o_encode.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.qf8o_num_finite_nonneg.restype = ctypes.c_int
    lib.qf8o_num_finite_nonneg.argtypes = [ctypes.c_int]
    lib.qf8o_max_finite.restype = ctypes.c_double
    lib.qf8o_max_finite.argtypes = [ctypes.c_int]
    lib.qf8o_amax.restype = ctypes.c_double
    lib.qf8o_amax.argtypes = [_c_void_p, ctypes.c_int, _i64]
    lib.qf8o_scale_from_amax.restype = ctypes.c_float
    lib.qf8o_scale_from_amax.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.qf8o_cast_one.restype = ctypes.c_uint
    lib.qf8o_cast_one.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_float]
    lib.qf8o_cast.restype = None
    lib.qf8o_cast.argtypes = [_c_void_p, ctypes.c_int, _i64, ctypes.c_int, ctypes.c_float, _c_void_p]
    lib.qf8o_encode_f32.restype = None
    lib.qf8o_encode_f32.argtypes = [ctypes.c_int, _c_void_p, _i64, _c_void_p]
    lib.qf8o_quantize_per_tensor.restype = None
    lib.qf8o_quantize_per_tensor.argtypes = [_c_void_p, ctypes.c_int, _i64, _i64, ctypes.c_int,
                                             _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.qf8o_delayed_sizeof.restype = ctypes.c_size_t
    lib.qf8o_delayed_init.restype = ctypes.c_int
    lib.qf8o_delayed_init.argtypes = [_c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.qf8o_delayed_reset.restype = None
    lib.qf8o_delayed_reset.argtypes = [_c_void_p]
    lib.qf8o_delayed_estimate.restype = ctypes.c_float
    lib.qf8o_delayed_estimate.argtypes = [_c_void_p]
    lib.qf8o_delayed_scale.restype = ctypes.c_float
    lib.qf8o_delayed_scale.argtypes = [_c_void_p]
    lib.qf8o_delayed_step.restype = None
    lib.qf8o_delayed_step.argtypes = [_c_void_p, _c_void_p, ctypes.c_int, _i64, _i64,
                                      _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.qf8o_delayed_set_estimator.restype = ctypes.c_int
    lib.qf8o_delayed_set_estimator.argtypes = [_c_void_p, ctypes.c_int]
    lib.qf8o_delayed_set_split.restype = ctypes.c_int
    lib.qf8o_delayed_set_split.argtypes = [_c_void_p, ctypes.c_int]
    lib.qf8o_delayed_piece.restype = None
    lib.qf8o_delayed_piece.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64, _c_void_p, _c_void_p]
    lib.qf8o_delayed_get.restype = None
    lib.qf8o_delayed_get.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.qf8o_quantize_block.restype = None
    lib.qf8o_quantize_block.argtypes = [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.c_int,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.qf8o_emax.restype = ctypes.c_int
    lib.qf8o_emax.argtypes = [ctypes.c_int]
    lib.qf8o_mx_exponent.restype = ctypes.c_int
    lib.qf8o_mx_exponent.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double]
    lib.qf8o_quantize_mx.restype = None
    lib.qf8o_quantize_mx.argtypes = [_c_void_p, ctypes.c_int, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                     _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.qf8o_dequant_one.restype = ctypes.c_float
    lib.qf8o_dequant_one.argtypes = [ctypes.c_int, ctypes.c_uint, ctypes.c_float]
    lib.qf8o_dequant_mx_one.restype = ctypes.c_float
    lib.qf8o_dequant_mx_one.argtypes = [ctypes.c_int, ctypes.c_uint, ctypes.c_uint]
    lib.qf8o_dequant_scaled.restype = None
    lib.qf8o_dequant_scaled.argtypes = [_c_void_p, _i64, ctypes.c_int, ctypes.c_float, _c_void_p]
    lib.qf8o_dequant_block.restype = None
    lib.qf8o_dequant_block.argtypes = [_c_void_p, _i64, _i64, _i64, _i64, ctypes.c_int, _c_void_p, _c_void_p]
    lib.qf8o_dequant_mx.restype = None
    lib.qf8o_dequant_mx.argtypes = [_c_void_p, _c_void_p, _i64, _i64, ctypes.c_int, _c_void_p]
    lib.qf8o_pack_fp4.restype = None
    lib.qf8o_pack_fp4.argtypes = [_c_void_p, _i64, _c_void_p]
    lib.qf8o_unpack_fp4.restype = None
    lib.qf8o_unpack_fp4.argtypes = [_c_void_p, _i64, _c_void_p]
    lib.qf8o_nvfp4_tensor_scale.restype = ctypes.c_float
    lib.qf8o_nvfp4_tensor_scale.argtypes = [ctypes.c_double]
    lib.qf8o_nvfp4_block.restype = ctypes.c_uint
    lib.qf8o_nvfp4_block.argtypes = [ctypes.c_double, ctypes.c_float]
    lib.qf8o_nvfp4_element.restype = ctypes.c_uint
    lib.qf8o_nvfp4_element.argtypes = [ctypes.c_double, ctypes.c_float, ctypes.c_uint]
    lib.qf8o_encode_ratio.restype = ctypes.c_uint
    lib.qf8o_encode_ratio.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
    lib.qf8o_quantize_nvfp4.restype = None
    lib.qf8o_quantize_nvfp4.argtypes = [_c_void_p, ctypes.c_int, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p]
    lib.qf8o_dequant_mxfp4_one.restype = ctypes.c_float
    lib.qf8o_dequant_mxfp4_one.argtypes = [ctypes.c_uint, ctypes.c_uint]
    lib.qf8o_dequant_nvfp4_one.restype = ctypes.c_float
    lib.qf8o_dequant_nvfp4_one.argtypes = [ctypes.c_uint, ctypes.c_uint, ctypes.c_float]
    lib.qf8o_dequant_nvfp4.restype = None
    lib.qf8o_dequant_nvfp4.argtypes = [_c_void_p, _c_void_p, _i64, _i64, ctypes.c_float, _c_void_p]
    lib.qf8o_dequant_mxfp4.restype = None
    lib.qf8o_dequant_mxfp4.argtypes = [_c_void_p, _c_void_p, _i64, _i64, _c_void_p]
    lib.qf8o_f32_to_bf16.restype = None
    lib.qf8o_f32_to_bf16.argtypes = [_c_void_p, _i64, _c_void_p]
    lib.qf8o_stats_scaled.restype = None
    lib.qf8o_stats_scaled.argtypes = [_c_void_p, ctypes.c_int, _c_void_p, _i64, ctypes.c_int, ctypes.c_float,
                                      _c_void_p, _c_void_p]
    lib.qf8o_stats_block.restype = None
    lib.qf8o_stats_block.argtypes = [_c_void_p, ctypes.c_int, _c_void_p, _i64, _i64, _i64, _i64, ctypes.c_int,
                                     _c_void_p, _c_void_p, _c_void_p]
    lib.qf8o_stats_mx.restype = None
    lib.qf8o_stats_mx.argtypes = [_c_void_p, ctypes.c_int, _c_void_p, _c_void_p, _i64, _i64, ctypes.c_int,
                                  _c_void_p, _c_void_p]
    lib.qf8o_scale_pow2.restype = ctypes.c_float
    lib.qf8o_scale_pow2.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.qf8o_quantize_block_ex.restype = None
    lib.qf8o_quantize_block_ex.argtypes = [_c_void_p, ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                           _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    lib.qf8o_requant_1x128_to_128x1.restype = None
    lib.qf8o_requant_1x128_to_128x1.argtypes = [_c_void_p, _c_void_p, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_c_void_p)


def _dtype_code(x):
    if x.dtype == np.uint16:
        return 0
    if x.dtype == np.float32:
        return 1
    raise TypeError("oracle inputs are uint16 (bf16 bits) or float32 arrays")


def _contig(x):
    return np.ascontiguousarray(x)


def decode(fmt, code):
    return _load().qf8o_decode(fmt, int(code))


def encode(fmt, y):
    return _load().qf8o_encode(fmt, float(y))


def encode_f32(fmt, y):
    y = _contig(np.asarray(y, dtype=np.float32))
    q = np.empty(y.shape, np.uint8)
    _load().qf8o_encode_f32(fmt, _ptr(y), y.size, _ptr(q))
    return q


def num_finite_nonneg(fmt):
    return _load().qf8o_num_finite_nonneg(fmt)


def max_finite(fmt):
    return _load().qf8o_max_finite(fmt)


def emax(fmt):
    return _load().qf8o_emax(fmt)


def amax(x):
    x = _contig(x)
    return _load().qf8o_amax(_ptr(x), _dtype_code(x), x.size)


def scale_from_amax(fmt, a):
    return _load().qf8o_scale_from_amax(fmt, float(a))


def cast_one(fmt, x, scale):
    return _load().qf8o_cast_one(fmt, float(x), float(np.float32(scale)))


def cast(x, fmt, scale):
    """q = sat_rne8(fl32(x * scale)) elementwise."""
    x = _contig(x)
    q = np.empty(x.shape, np.uint8)
    _load().qf8o_cast(_ptr(x), _dtype_code(x), x.size, fmt, float(np.float32(scale)), _ptr(q))
    return q


def quantize_per_tensor(x, fmt):
    """Returns (q, amax, scale, nonfinite)."""
    x = _contig(x)
    rows, cols = (x.shape[0], int(np.prod(x.shape[1:]))) if x.ndim >= 2 else (1, x.size)
    q = np.empty(x.shape, np.uint8)
    am = np.zeros(1, np.float32)
    sc = np.zeros(1, np.float32)
    nf = np.zeros(1, np.int32)
    _load().qf8o_quantize_per_tensor(_ptr(x), _dtype_code(x), rows, cols, fmt, _ptr(q), _ptr(am), _ptr(sc), _ptr(nf))
    return q, am[0], sc[0], int(nf[0])


def delayed_piece(step, interval, n):
    """[lo, hi) of the piece a split-mode step measures (R15)."""
    lo = np.zeros(1, np.int64)
    hi = np.zeros(1, np.int64)
    _load().qf8o_delayed_piece(step, interval, n, _ptr(lo), _ptr(hi))
    return int(lo[0]), int(hi[0])


class Delayed:
    """Delayed-scaling state machine (amax history FIFO, Interval, 2^-N margin)."""

    def __init__(self, hist_len, interval, n_guard, fmt, estimator=0, split=False):
        """estimator: 0 max of the history, 1 most recent entry, 2 mean (R14).
        split: measure one of `interval` pieces of the tensor per step and append the window's
        maximum on update steps (R15)."""
        lib = _load()
        self._buf = np.zeros(lib.qf8o_delayed_sizeof(), np.uint8)
        if lib.qf8o_delayed_init(_ptr(self._buf), hist_len, interval, n_guard, fmt) != 0:
            raise ValueError("bad delayed-scaling configuration")
        if lib.qf8o_delayed_set_estimator(_ptr(self._buf), estimator) != 0:
            raise ValueError("bad estimator")
        if lib.qf8o_delayed_set_split(_ptr(self._buf), 1 if split else 0) != 0:
            raise ValueError("bad split flag")
        self.hist_len = hist_len
        self.fmt = fmt

    def reset(self):
        _load().qf8o_delayed_reset(_ptr(self._buf))

    def estimate(self):
        return _load().qf8o_delayed_estimate(_ptr(self._buf))

    def next_scale(self):
        return _load().qf8o_delayed_scale(_ptr(self._buf))

    def step(self, x):
        """One iteration. Returns (q, scale_used, amax, nonfinite)."""
        x = _contig(x)
        rows, cols = (x.shape[0], int(np.prod(x.shape[1:]))) if x.ndim >= 2 else (1, x.size)
        q = np.empty(x.shape, np.uint8)
        s = np.zeros(1, np.float32)
        a = np.zeros(1, np.float32)
        nf = np.zeros(1, np.int32)
        _load().qf8o_delayed_step(_ptr(self._buf), _ptr(x), _dtype_code(x), rows, cols, _ptr(q), _ptr(s), _ptr(a), _ptr(nf))
        return q, s[0], a[0], int(nf[0])

    def state(self):
        """Returns (history oldest-first as float32 array, count, step)."""
        h = np.zeros(self.hist_len, np.float32)
        c = np.zeros(1, np.int32)
        st = np.zeros(1, np.int64)
        _load().qf8o_delayed_get(_ptr(self._buf), _ptr(h), _ptr(c), _ptr(st))
        return h[:c[0]].copy(), int(c[0]), int(st[0])


def quantize_block(x, br, bc, fmt):
    """Returns (q, scales, amax, nonfinite); scales/amax are [ceil(R/br)][ceil(C/bc)]."""
    x = _contig(x)
    rows, cols = x.shape
    gr, gc = -(-rows // br), -(-cols // bc)
    q = np.empty(x.shape, np.uint8)
    sc = np.zeros((gr, gc), np.float32)
    am = np.zeros((gr, gc), np.float32)
    nf = np.zeros(1, np.int32)
    _load().qf8o_quantize_block(_ptr(x), _dtype_code(x), rows, cols, br, bc, fmt, _ptr(q), _ptr(sc), _ptr(am), _ptr(nf))
    return q, sc, am, int(nf[0])


def mx_exponent(fmt, rnd, a):
    return _load().qf8o_mx_exponent(fmt, rnd, float(a))


def quantize_mx(x, fmt, rnd, row=True, col=True):
    """Returns (q_row, s_row, q_colT, s_colT, nonfinite); a direction not asked for is None."""
    x = _contig(x)
    rows, cols = x.shape
    q_row = np.empty((rows, cols), np.uint8) if row else None
    s_row = np.empty((rows, cols // 32), np.uint8) if row else None
    q_colT = np.empty((cols, rows), np.uint8) if col else None
    s_colT = np.empty((cols, rows // 32), np.uint8) if col else None
    nf = np.zeros(1, np.int32)
    _load().qf8o_quantize_mx(_ptr(x), _dtype_code(x), rows, cols, fmt, rnd, _ptr(q_row), _ptr(s_row),
                             _ptr(q_colT), _ptr(s_colT), _ptr(nf))
    return q_row, s_row, q_colT, s_colT, int(nf[0])


# ---- dequantization and error statistics --------------------------------------------------

STATS_FIELDS = ("count", "nonzero", "zeroed", "saturated", "nonfinite")


def dequant_one(fmt, code, scale):
    """fl32(decode(code) / scale)."""
    return _load().qf8o_dequant_one(fmt, int(code), float(np.float32(scale)))


def dequant_mx_one(fmt, code, sbyte):
    """fl32(decode(code) * 2^(sbyte - 127)); NaN for sbyte 0xFF."""
    return _load().qf8o_dequant_mx_one(fmt, int(code), int(sbyte))


def dequant_scaled(q, fmt, scale):
    """Per-tensor (or delayed) dequantization: float32 array of q's shape."""
    q = np.ascontiguousarray(q, np.uint8)
    out = np.empty(q.shape, np.float32)
    _load().qf8o_dequant_scaled(_ptr(q), q.size, fmt, float(np.float32(scale)), _ptr(out))
    return out


def dequant_block(q, br, bc, fmt, scales):
    q = np.ascontiguousarray(q, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    rows, cols = q.shape
    out = np.empty(q.shape, np.float32)
    _load().qf8o_dequant_block(_ptr(q), rows, cols, br, bc, fmt, _ptr(scales), _ptr(out))
    return out


def dequant_mx(q, s, fmt):
    """q [rows][cols] with blocks of 32 along rows, s [rows][cols/32] E8M0 bytes."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    rows, cols = q.shape
    out = np.empty(q.shape, np.float32)
    _load().qf8o_dequant_mx(_ptr(q), _ptr(s), rows, cols, fmt, _ptr(out))
    return out


def to_bf16(f):
    """float32 array -> BF16 bit patterns (uint16), round to nearest even."""
    f = np.ascontiguousarray(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().qf8o_f32_to_bf16(_ptr(f), f.size, _ptr(out))
    return out


def _stats_dict(sums, counts):
    d = {"signal": float(sums[0]), "noise": float(sums[1])}
    d.update({k: int(v) for k, v in zip(STATS_FIELDS, counts)})
    return d


def stats_scaled(x, q, fmt, scale):
    x = _contig(x)
    q = np.ascontiguousarray(q, np.uint8)
    sums, counts = np.zeros(2, np.float64), np.zeros(5, np.int64)
    _load().qf8o_stats_scaled(_ptr(x), _dtype_code(x), _ptr(q), x.size, fmt, float(np.float32(scale)),
                              _ptr(sums), _ptr(counts))
    return _stats_dict(sums, counts)


def stats_block(x, q, br, bc, fmt, scales):
    x = _contig(x)
    q = np.ascontiguousarray(q, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    rows, cols = x.shape
    sums, counts = np.zeros(2, np.float64), np.zeros(5, np.int64)
    _load().qf8o_stats_block(_ptr(x), _dtype_code(x), _ptr(q), rows, cols, br, bc, fmt, _ptr(scales),
                             _ptr(sums), _ptr(counts))
    return _stats_dict(sums, counts)


def stats_mx(x, q, s, fmt):
    """x in the layout of q (for a columnwise result: x transposed)."""
    x = _contig(x)
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    rows, cols = x.shape
    sums, counts = np.zeros(2, np.float64), np.zeros(5, np.int64)
    _load().qf8o_stats_mx(_ptr(x), _dtype_code(x), _ptr(q), _ptr(s), rows, cols, fmt, _ptr(sums), _ptr(counts))
    return _stats_dict(sums, counts)


# ---- power-of-two group scales and the 1x128 -> 128x1 re-grouping ----------------------------

def scale_pow2(fmt, a):
    """Largest power of two S with a * S <= F8max (1 for a = 0 or non-finite)."""
    return _load().qf8o_scale_pow2(fmt, float(a))


def quantize_block_ex(x, br, bc, fmt, pow2):
    """quantize_block with Eq.(1) scales (pow2 False) or power-of-two scales (pow2 True).
    Returns (q, scales, amax, nonfinite)."""
    x = _contig(x)
    rows, cols = x.shape
    gr, gc = -(-rows // br), -(-cols // bc)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((gr, gc), np.float32)
    a = np.empty((gr, gc), np.float32)
    nf = np.zeros(1, np.int32)
    _load().qf8o_quantize_block_ex(_ptr(x), _dtype_code(x), rows, cols, br, bc, fmt, int(bool(pow2)), _ptr(q),
                                   _ptr(s), _ptr(a), _ptr(nf))
    return q, s, a, int(nf[0])


def requant_1x128_to_128x1(q, scales, fmt_in, fmt_out, pow2_out):
    """De-scale q [rows][cols] (1x128 groups), transpose, quantize again in 1x128 groups of the
    transpose. Returns (qT [cols][rows], scalesT [cols][ceil(rows/128)], nonfinite)."""
    q = np.ascontiguousarray(q, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    rows, cols = q.shape
    tmp = np.empty(rows * cols, np.float32)
    qT = np.empty((cols, rows), np.uint8)
    sT = np.empty((cols, -(-rows // 128)), np.float32)
    nf = np.zeros(1, np.int32)
    _load().qf8o_requant_1x128_to_128x1(_ptr(q), _ptr(scales), rows, cols, fmt_in, fmt_out, int(bool(pow2_out)),
                                        _ptr(tmp), _ptr(qT), _ptr(sT), _ptr(nf))
    return qT, sT, int(nf[0])


# ---- FP4 (R16 MXFP4, R17 NVFP4) -----------------------------------------------------------------

def pack_fp4(codes):
    """4-bit codes (one per byte, even count along the last axis) -> bytes, c[2j] | c[2j+1] << 4."""
    c = np.ascontiguousarray(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] // 2,), np.uint8)
    _load().qf8o_pack_fp4(_ptr(c), c.size, _ptr(out))
    return out


def unpack_fp4(packed):
    p = np.ascontiguousarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    _load().qf8o_unpack_fp4(_ptr(p), out.size, _ptr(out))
    return out


def quantize_mxfp4(x, rnd, row=True, col=True):
    """Returns (q_row [rows][cols/2], s_row, q_colT [cols][rows/2], s_colT, nonfinite), packed."""
    q_row, s_row, q_colT, s_colT, nf = quantize_mx(x, E2M1, rnd, row, col)
    return (pack_fp4(q_row) if row else None, s_row, pack_fp4(q_colT) if col else None, s_colT, nf)


def nvfp4_tensor_scale(a):
    return _load().qf8o_nvfp4_tensor_scale(float(a))


def nvfp4_block(amax_b, s_t):
    """E4M3 block-scale code of one block: amax_b * S_t / 6 rounded once (R17)."""
    return int(_load().qf8o_nvfp4_block(float(amax_b), float(np.float32(s_t))))


def nvfp4_element(x, s_t, e):
    """E2M1 code of one element under block-scale code e: x * S_t / decode(e) rounded once (R17)."""
    return int(_load().qf8o_nvfp4_element(float(x), float(np.float32(s_t)), int(e)))


def encode_ratio(fmt, num, den):
    """sat_rne of the exact quotient num / den (products of num's format values with den exact)."""
    return int(_load().qf8o_encode_ratio(int(fmt), float(num), float(den)))


def quantize_nvfp4(x, amax_in=None):
    """Returns (q [rows][cols/2] packed, s_blk [rows][cols/16] E4M3 codes, S_t, amax, nonfinite).
    amax_in: a tensor amax to use in place of the measured one."""
    x = _contig(x)
    ain = None if amax_in is None else np.array([amax_in], np.float32)
    rows, cols = x.shape
    codes = np.empty((rows, cols), np.uint8)
    s_blk = np.empty((rows, cols // 16), np.uint8)
    st = np.zeros(1, np.float32)
    a = np.zeros(1, np.float32)
    nf = np.zeros(1, np.int32)
    _load().qf8o_quantize_nvfp4(_ptr(x), _dtype_code(x), rows, cols, _ptr(ain), _ptr(codes), _ptr(s_blk), _ptr(st),
                                _ptr(a), _ptr(nf))
    return pack_fp4(codes), s_blk, np.float32(st[0]), np.float32(a[0]), int(nf[0])


def dequant_mxfp4(q, s):
    """q [rows][cols/2] packed, s [rows][cols/32] E8M0 -> float32 [rows][cols]."""
    codes = unpack_fp4(q)
    s = np.ascontiguousarray(s, np.uint8)
    rows, cols = codes.shape
    out = np.empty((rows, cols), np.float32)
    _load().qf8o_dequant_mxfp4(_ptr(codes), _ptr(s), rows, cols, _ptr(out))
    return out


def dequant_nvfp4(q, s_blk, s_t):
    """q [rows][cols/2] packed, s_blk [rows][cols/16] E4M3, S_t -> float32 [rows][cols]."""
    codes = unpack_fp4(q)
    s_blk = np.ascontiguousarray(s_blk, np.uint8)
    rows, cols = codes.shape
    out = np.empty((rows, cols), np.float32)
    _load().qf8o_dequant_nvfp4(_ptr(codes), _ptr(s_blk), rows, cols, float(np.float32(s_t)), _ptr(out))
    return out


def dequant_nvfp4_one(code, e_code, s_t):
    return _load().qf8o_dequant_nvfp4_one(int(code), int(e_code), float(np.float32(s_t)))


def dequant_mxfp4_one(code, sbyte):
    return _load().qf8o_dequant_mxfp4_one(int(code), int(sbyte))
