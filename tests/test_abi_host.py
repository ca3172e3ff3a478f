"""Host-side checks of libqf8.so (no GPU needed, nothing is launched): the library loads, exports
every function include/qf8.h declares, and rejects bad arguments with the documented status
before touching the device."""
import ctypes
import os
import re

import pytest

import mx_block_scaled_amax_amd as qf8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qf8.h")

OK, NULL, ENUM, SHAPE, ALIGN, WS, STATE = 0, -1, -2, -3, -4, -5, -6
FAKE = ctypes.c_void_p(0x10000)          # 16-byte aligned, never dereferenced (rejected first)
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{]*\)\s*;", text)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def lib():
    qf8._load()
    return qf8._lib


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"quantize_per_tensor", "quantize_delayed", "quantize_block", "quantize_mx_dual"} <= set(names)
    L = ctypes.CDLL(qf8.library_path())
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(-7, 1):
        assert qf8.qf8_status_string(s)
    assert "unknown" in qf8.qf8_status_string(-99)
    assert qf8.qf8_workspace_bytes(8192, 8192) >= 2048 * 4


def test_set_onepass_grid_range():
    """The grid is range-checked before any HIP call."""
    f = lib().qf8_set_onepass_grid
    assert f(-1) == SHAPE
    assert f(513) == SHAPE
    assert f(1 << 30) == SHAPE


def test_mx_argument_errors():
    f = lib().quantize_mx_dual
    assert f(FAKE, 0, 64, 64, 2, 0, FAKE, FAKE, None, None, None, None) == ENUM    # bad fmt
    assert f(FAKE, 3, 64, 64, 0, 0, FAKE, FAKE, None, None, None, None) == ENUM    # bad dtype
    assert f(FAKE, 0, 64, 64, 0, 5, FAKE, FAKE, None, None, None, None) == ENUM    # bad rounding
    assert f(FAKE, 0, 64, 64, 0, 0, None, None, None, None, None, None) == NULL    # no direction
    assert f(FAKE, 0, 64, 64, 0, 0, FAKE, None, None, None, None, None) == NULL    # q without scales
    assert f(FAKE, 0, 64, 48, 0, 0, FAKE, FAKE, None, None, None, None) == SHAPE   # rowwise cols % 32
    assert f(FAKE, 0, 40, 64, 0, 0, None, None, FAKE, FAKE, None, None) == SHAPE   # colwise rows % 32
    assert f(FAKE, 0, -1, 64, 0, 0, FAKE, FAKE, None, None, None, None) == SHAPE
    assert f(MISALIGNED, 0, 64, 64, 0, 0, FAKE, FAKE, None, None, None, None) == ALIGN
    assert f(None, 0, 64, 64, 0, 0, FAKE, FAKE, None, None, None, None) == NULL
    # columnwise FP8 is limited to 2^23 rows (one tile's output must stay below 2^31 bytes)
    assert f(FAKE, 0, (1 << 23) + 32, 256, 0, 0, None, None, FAKE, FAKE, None, None) == SHAPE


def test_fp4_argument_errors():
    f = lib().quantize_mxfp4_dual
    assert f(FAKE, 3, 64, 64, 0, FAKE, FAKE, None, None, None, None) == ENUM       # bad dtype
    assert f(FAKE, 0, 64, 64, 5, FAKE, FAKE, None, None, None, None) == ENUM       # bad rounding
    assert f(FAKE, 0, 64, 64, 0, None, None, None, None, None, None) == NULL       # no direction
    assert f(FAKE, 0, 64, 64, 0, None, None, FAKE, None, None, None) == NULL       # q without scales
    assert f(FAKE, 0, 64, 48, 0, FAKE, FAKE, None, None, None, None) == SHAPE      # rowwise cols % 32
    assert f(FAKE, 0, 40, 64, 0, None, None, FAKE, FAKE, None, None) == SHAPE      # colwise rows % 32
    assert f(FAKE, 0, 64, 36, 0, None, None, FAKE, FAKE, None, None) == SHAPE      # BF16 cols % 8
    assert f(FAKE, 0, (1 << 24) + 32, 32, 0, FAKE, FAKE, None, None, None, None) == SHAPE
    assert f(MISALIGNED, 0, 64, 64, 0, FAKE, FAKE, None, None, None, None) == ALIGN
    assert f(None, 0, 64, 64, 0, FAKE, FAKE, None, None, None, None) == NULL
    assert f(None, 0, 0, 64, 0, FAKE, FAKE, None, None, None, None) == OK          # empty: nothing to do
    g = lib().quantize_nvfp4
    assert g(FAKE, 2, 4, 16, None, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == ENUM
    assert g(FAKE, 0, 4, 24, None, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == SHAPE   # cols % 16
    assert g(FAKE, 0, 4, 16, None, FAKE, None, FAKE, None, None, FAKE, 1 << 20, None) == NULL    # no s_blk
    assert g(FAKE, 0, 4, 16, None, FAKE, FAKE, None, None, None, FAKE, 1 << 20, None) == NULL    # no S_t out
    assert g(FAKE, 0, 4, 16, None, FAKE, FAKE, FAKE, None, None, None, 0, None) == WS            # amax pass needs ws
    assert g(FAKE, 0, 4, 16, None, FAKE, FAKE, FAKE, None, None, FAKE, 64, None) == WS
    assert g(FAKE, 0, 4, 16, None, MISALIGNED, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == ALIGN


def test_per_tensor_argument_errors():
    f = lib().quantize_per_tensor
    fl = ctypes.c_void_p(0x20000)
    assert f(FAKE, 0, 4, 4, 7, FAKE, fl, fl, None, FAKE, 1 << 20, None) == ENUM
    assert f(FAKE, 0, 4, 4, 0, FAKE, None, fl, None, FAKE, 1 << 20, None) == NULL
    assert f(FAKE, 0, 4, 4, 0, FAKE, fl, fl, None, FAKE, 16, None) == WS
    assert f(FAKE, 0, 4, 4, 0, FAKE, fl, fl, None, None, 1 << 20, None) == WS
    assert f(FAKE, 0, 4, 4, 0, MISALIGNED, fl, fl, None, FAKE, 1 << 20, None) == ALIGN
    assert f(FAKE, 0, -4, 4, 0, FAKE, fl, fl, None, FAKE, 1 << 20, None) == SHAPE
    g = lib().qf8_cast_scaled
    assert g(FAKE, 0, 0, 0, None, None, None) == OK          # empty: nothing to do
    assert g(FAKE, 0, 10, 0, None, FAKE, None) == NULL
    assert g(FAKE, 0, -1, 0, fl, FAKE, None) == SHAPE


def test_block_argument_errors():
    f = lib().quantize_block
    assert f(FAKE, 0, 128, 128, 2, 128, 0, FAKE, FAKE, None, None, None) == SHAPE   # block rows
    assert f(FAKE, 0, 128, 128, 1, 64, 0, FAKE, FAKE, None, None, None) == SHAPE    # block cols
    assert f(FAKE, 0, 128, 132, 1, 128, 0, FAKE, FAKE, None, None, None) == SHAPE   # cols % 8 (bf16)
    assert f(FAKE, 0, 128, 128, 1, 128, 0, FAKE, None, None, None, None) == NULL
    assert f(FAKE, 0, 0, 128, 1, 128, 0, None, None, None, None, None) == OK        # empty


def test_delayed_state_errors():
    st = qf8._DelayedStruct()
    L = lib()
    ref = ctypes.byref(st)
    assert L.quantize_delayed(FAKE, 0, 4, 4, 0, ref, FAKE, None, None, None, FAKE, 1 << 20, None) == STATE  # not initialised
    assert L.qf8_delayed_init(ref, FAKE, FAKE, FAKE, 0, 1, 0, 0, None) == STATE       # hist_len 0
    assert L.qf8_delayed_init(ref, FAKE, FAKE, FAKE, 16, 0, 0, 0, None) == STATE      # interval 0
    assert L.qf8_delayed_init(ref, FAKE, FAKE, FAKE, 16, 1, 65, 0, None) == STATE     # n_guard too large
    assert L.qf8_delayed_init(ref, FAKE, FAKE, FAKE, 16, 1, 0, 9, None) == ENUM
    assert L.qf8_delayed_init(ref, None, FAKE, FAKE, 16, 1, 0, 0, None) == NULL
    assert L.qf8_delayed_reset(None, None) == NULL
    # estimator outside qf8_estimator: init_ex refuses it before touching the device, and a
    # state whose estimator field was overwritten is refused before any launch
    assert L.qf8_delayed_init_ex(ref, FAKE, FAKE, FAKE, 16, 1, 0, 0, 3, 0, None) == ENUM
    assert L.qf8_delayed_init_ex(ref, FAKE, FAKE, FAKE, 16, 1, 0, 0, -1, 0, None) == ENUM
    assert L.qf8_delayed_init_ex(ref, FAKE, FAKE, FAKE, 16, 1, 0, 0, 0, 2, None) == ENUM      # unknown flag
    st.history = st.meta = st.scale = FAKE
    st.hist_len, st.interval, st.n_guard, st.fmt, st.step = 16, 1, 0, 0, 0
    st.magic, st.estimator = 0x51463844, 3
    assert L.quantize_delayed(FAKE, 0, 4, 4, 0, ref, FAKE, None, None, None, FAKE, 1 << 20, None) == STATE
    assert L.qf8_delayed_reset(ref, None) == STATE
    st.estimator, st.flags = 0, 4
    assert L.quantize_delayed(FAKE, 0, 4, 4, 0, ref, FAKE, None, None, None, FAKE, 1 << 20, None) == STATE
    # the call's format must be the state's: a mismatch is refused before any launch
    st.flags = 0
    assert L.quantize_delayed(FAKE, 0, 4, 4, 1, ref, FAKE, None, None, None, FAKE, 1 << 20, None) == STATE
    assert L.quantize_delayed(FAKE, 0, 4, 4, 7, ref, FAKE, None, None, None, FAKE, 1 << 20, None) == ENUM


def test_no_cpu_path():
    import torch
    with pytest.raises(TypeError):
        qf8.quantize_mx_dual(torch.zeros(32, 32, dtype=torch.bfloat16), qf8.E4M3, qf8.ROUND_UP)


def test_workspace_argument_errors():
    L = lib()
    need = qf8.qf8_workspace_bytes(64, 64)
    assert need >= qf8.BARRIER_WORDS * 4 + 16384 * 4
    assert L.qf8_workspace_init(None, need, None) == NULL
    assert L.qf8_workspace_init(FAKE, need - 4, None) == WS
    assert L.qf8_workspace_init(MISALIGNED, need, None) == ALIGN
    fl = ctypes.c_void_p(0x20000)
    f = L.quantize_per_tensor
    assert f(FAKE, 0, 4, 4, 0, FAKE, fl, fl, None, MISALIGNED, need, None) == ALIGN   # ws 16-byte aligned


def test_dequant_argument_errors():
    L = lib()
    fl = ctypes.c_void_p(0x20000)
    need = qf8.qf8_workspace_bytes(1, 1)
    f = L.dequantize_scaled
    assert f(FAKE, 64, 7, fl, FAKE, 0, None, 0, None, None, 0, None) == ENUM            # fmt
    assert f(FAKE, 64, 0, fl, FAKE, 5, None, 0, None, None, 0, None) == ENUM            # out dtype
    assert f(FAKE, 64, 0, fl, None, 0, None, 0, None, None, 0, None) == NULL            # no out, no stats
    assert f(FAKE, 64, 0, None, FAKE, 0, None, 0, None, None, 0, None) == NULL          # no scale
    assert f(FAKE, 64, 0, fl, None, 0, None, 0, FAKE, FAKE, need, None) == NULL         # stats without x
    assert f(FAKE, 64, 0, fl, None, 0, FAKE, 0, FAKE, FAKE, 16, None) == WS             # small workspace
    assert f(FAKE, 64, 0, fl, None, 0, FAKE, 9, FAKE, FAKE, need, None) == ENUM         # x dtype
    assert f(MISALIGNED, 64, 0, fl, FAKE, 0, None, 0, None, None, 0, None) == ALIGN
    assert f(FAKE, -1, 0, fl, FAKE, 0, None, 0, None, None, 0, None) == SHAPE
    assert f(FAKE, 1 << 33, 0, fl, FAKE, 0, None, 0, None, None, 0, None) == SHAPE
    assert f(FAKE, 0, 0, fl, FAKE, 0, None, 0, None, None, 0, None) == OK               # empty: nothing to do
    g = L.dequantize_block
    assert g(FAKE, 128, 128, 2, 128, 0, fl, FAKE, 0, None, 0, None, None, 0, None) == SHAPE   # block rows
    assert g(FAKE, 128, 130, 1, 128, 0, fl, FAKE, 0, None, 0, None, None, 0, None) == SHAPE   # cols % 4
    assert g(FAKE, 128, 128, 1, 128, 0, None, FAKE, 0, None, 0, None, None, 0, None) == NULL  # scales
    h = L.dequantize_mx
    assert h(FAKE, FAKE, 64, 48, 0, FAKE, 0, None, 0, None, None, 0, None) == SHAPE      # cols % 32
    assert h(FAKE, None, 64, 64, 0, FAKE, 0, None, 0, None, None, 0, None) == NULL       # scale bytes


def test_block_ex_and_requant_argument_errors():
    L = lib()
    f = L.quantize_block_ex
    assert f(FAKE, 0, 128, 128, 1, 128, 0, 2, FAKE, FAKE, None, None, None) == ENUM       # unknown flag
    assert f(FAKE, 0, 128, 128, 1, 64, 0, 1, FAKE, FAKE, None, None, None) == SHAPE
    g = L.requantize_1x128_to_128x1
    assert g(FAKE, FAKE, 128, 128, 0, 3, 1, FAKE, FAKE, None, None) == ENUM               # fmt_out
    assert g(FAKE, FAKE, 128, 120, 0, 0, 1, FAKE, FAKE, None, None) == SHAPE              # cols % 16
    assert g(FAKE, FAKE, 136, 128, 0, 0, 1, FAKE, FAKE, None, None) == SHAPE              # rows % 16
    assert g(FAKE, FAKE, 128, 128, 0, 0, 1, FAKE, None, None, None) == NULL               # scalesT
    assert g(FAKE, FAKE, 0, 128, 0, 0, 1, None, None, None, None) == OK                   # empty
    assert g(MISALIGNED, FAKE, 128, 128, 0, 0, 1, FAKE, FAKE, None, None) == ALIGN


def test_fp4_dequant_argument_errors():
    f = lib().dequantize_mxfp4
    assert f(FAKE, FAKE, 4, 64, FAKE, 2, None) == ENUM                 # bad out dtype
    assert f(FAKE, FAKE, 4, 48, FAKE, 0, None) == SHAPE                # cols % 32
    assert f(None, FAKE, 4, 64, FAKE, 0, None) == NULL
    assert f(FAKE, FAKE, 4, 64, MISALIGNED, 0, None) == ALIGN
    assert f(None, None, 0, 64, None, 0, None) == OK                   # empty
    g = lib().dequantize_nvfp4
    assert g(FAKE, FAKE, FAKE, 4, 64, FAKE, 7, None) == ENUM
    assert g(FAKE, FAKE, FAKE, 4, 40, FAKE, 0, None) == SHAPE          # cols % 16
    assert g(FAKE, FAKE, None, 4, 64, FAKE, 0, None) == NULL           # no tensor scale
    assert g(MISALIGNED, FAKE, FAKE, 4, 64, FAKE, 0, None) == ALIGN
    assert g(FAKE, FAKE, FAKE, 1 << 20, 1 << 16, FAKE, 0, None) == SHAPE   # 2^36 elements
