"""GPU parity of the dequantization kernels and the quantization error statistics against the
CPU oracle.

  * every fp8 code of both formats de-scaled by exactly pinned scales (1, 2^k, the pages' 22400
    and 22.4, random), FP32 output bit for bit and BF16 output equal to the oracle's fp32
    result rounded to nearest even;
  * MX: every code under every E8M0 byte (0xFF gives NaN);
  * random codes and scales on a tensor large enough that every workgroup walks several tiles
    (each scaling mode, sampled row bands bit-exact);
  * round trips through the GPU quantizers on ragged shapes and on the full workloads
    (per-tensor 8192x8192, 1x128 8192x7168, 128x128 7168x18432, MX dual 16384x4096 rowwise and
    columnwise): the de-scaled tensors are bit-exact against the oracle on every element;
  * statistics: counts exact, fp64 sums within the summation-order bound (n * 2^-52 relative),
    the same bits on repeated calls, non-finite inputs counted and excluded (in whole tiles of
    several workgroups and in a partial one, BF16 and FP32 x, every scaling mode), empty input.
"""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import bf16_to_f32, block_weight, mx_gradient, per_tensor_activation, small_tensor, token_activation
from qf8_test_utils import assert_bytes_equal, host, parallel_row_slabs, to_device

pytestmark = pytest.mark.gpu
FMTS = [O.E4M3, O.E5M2]
F32 = torch.float32
BF16 = torch.bfloat16


def f32_host(t):
    return t.detach().cpu().numpy().astype(np.float32)


def bf16_host(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def assert_f32_equal(got, want, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    g, w = got[~gn].view(np.uint32), want[~wn].view(np.uint32)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{what}: {bad.size} values differ, first {got[~gn][bad[0]]!r} vs {want[~wn][bad[0]]!r}"


def assert_bf16_of(got_bits, want_f32, what):
    wb = O.to_bf16(want_f32)
    nan = np.isnan(np.asarray(want_f32, np.float32))
    assert np.array_equal(((got_bits & 0x7FFF) > 0x7F80), nan), f"{what}: NaN positions differ"
    assert_bytes_equal(got_bits[~nan].view(np.uint8), wb[~nan].view(np.uint8), what)


def dev_scale(s):
    return torch.tensor([np.float32(s)], dtype=F32, device="cuda")


@pytest.mark.parametrize("fmt", FMTS)
def test_every_code_every_pinned_scale(fmt):
    codes = np.tile(np.arange(256, dtype=np.uint8), 3)          # 768 codes: whole units and no tail
    qd = to_device(codes)
    rng = np.random.default_rng(12)
    scales = [1.0, 22400.0, float(np.float32(448 / 20)), 2.0 ** -20, 2.0 ** 17, 3.0, 1 / 3.0]
    scales += list((2.0 ** rng.uniform(-50, 50, 40)).astype(np.float32))
    for s in scales:
        sd = dev_scale(s)
        want = O.dequant_scaled(codes, fmt, s)
        o32, _ = qf8.dequantize_scaled(qd, fmt, sd, out_dtype=F32)
        assert_f32_equal(f32_host(o32), want, f"fp32 scale {s!r}")
        o16, _ = qf8.dequantize_scaled(qd, fmt, sd, out_dtype=BF16)
        assert_bf16_of(bf16_host(o16), want, f"bf16 scale {s!r}")


@pytest.mark.parametrize("n", [1, 3, 5, 4097, 1000003])
def test_scaled_ragged_lengths(n):
    rng = np.random.default_rng(n)
    codes = rng.integers(0, 256, n, dtype=np.uint64).astype(np.uint8)
    s = np.float32(rng.uniform(0.01, 100.0))
    for fmt in FMTS:
        o, _ = qf8.dequantize_scaled(to_device(codes), fmt, dev_scale(s), out_dtype=F32)
        assert_f32_equal(f32_host(o), O.dequant_scaled(codes, fmt, s), f"n={n}")


@pytest.mark.parametrize("n", [1, 17, 4097, 1000003, 5 * 1048576 + 11])
def test_scaled_ragged_lengths_with_stats(n):
    """Statistics on lengths that leave a partial last tile and a tail of n % 16 elements (the
    largest also gives whole tiles to several workgroups), BF16 x with a few outliers."""
    rng = np.random.default_rng(n + 7)
    x = small_tensor(1, n, seed=n).reshape(-1)
    x[rng.integers(0, n, max(1, n // 1000))] = 0x4780              # 65536: saturates below
    codes = rng.integers(0, 256, n, dtype=np.uint64).astype(np.uint8)
    codes[(codes & 0x7F) >= 0x7C] = 0x10            # no Inf/NaN codes, so the noise sum stays finite
    s = np.float32(rng.uniform(0.5, 8.0))
    for fmt in FMTS:
        o, st = qf8.dequantize_scaled(to_device(codes), fmt, dev_scale(s), out_dtype=BF16, x=to_device(x))
        want = O.stats_scaled(x, codes, fmt, s)
        assert np.isfinite(want["noise"])
        check_stats(qf8.stats_to_dict(st), want, f"n={n}")
        assert_bf16_of(bf16_host(o), O.dequant_scaled(codes, fmt, s), f"n={n}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_every_code_every_byte(fmt):
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))       # row r: all 256 codes
    s = np.tile(np.arange(256, dtype=np.uint8)[:, None], (1, 8))  # every block of row r: byte r
    want = O.dequant_mx(q, s, fmt)
    o, _ = qf8.dequantize_mx(to_device(q), to_device(s), fmt, out_dtype=F32)
    assert_f32_equal(f32_host(o), want, "mx fp32")
    o16, _ = qf8.dequantize_mx(to_device(q), to_device(s), fmt, out_dtype=BF16)
    assert_bf16_of(bf16_host(o16), want, "mx bf16")


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("shape", [(1, 128), (7, 264), (130, 512), (257, 392)])
def test_block_round_trip_small(shape, br):
    x = small_tensor(*shape, seed=shape[0] + br)
    for fmt in FMTS:
        q, sc = qf8.quantize_block(to_device(x), br, 128, fmt)[:2]
        qh, sch = host(q), host(sc)
        want = O.dequant_block(qh, br, 128, fmt, sch)
        o, st = qf8.dequantize_block(q, br, 128, fmt, sc, out_dtype=F32, x=to_device(x))
        assert_f32_equal(f32_host(o), want, f"block {shape} br={br}")
        check_stats(qf8.stats_to_dict(st), O.stats_block(x, qh, br, 128, fmt, sch), f"block {shape}")


def check_stats(got, want, what):
    for k in ("count", "nonzero", "zeroed", "saturated", "nonfinite"):
        assert got[k] == want[k], f"{what}: {k} {got[k]} vs {want[k]}"
    tol = (want["count"] + 64) * 2.0 ** -52
    for k in ("signal", "noise"):
        assert abs(got[k] - want[k]) <= tol * abs(want[k]) + 1e-300, f"{what}: {k} {got[k]!r} vs {want[k]!r}"


def oracle_stats_slabs(fn, rows, slab=512):
    """Oracle statistics over row slabs in threads, merged (counts exact; sums re-associated)."""
    parts = parallel_row_slabs(fn, rows, slab)
    out = {k: 0 for k in ("count", "nonzero", "zeroed", "saturated", "nonfinite")}
    out["signal"] = out["noise"] = 0.0
    for p in parts:
        for k in out:
            out[k] += p[k]
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_per_tensor_full_round_trip_and_stats(fmt):
    x = per_tensor_activation()
    xd = to_device(x)
    q, am, s = qf8.quantize_per_tensor(xd, fmt)
    ws = qf8.workspace(xd)
    o, st = qf8.dequantize_scaled(q, fmt, s, out_dtype=BF16, x=xd, ws=ws)
    o2, st2 = qf8.dequantize_scaled(q, fmt, s, out_dtype=BF16, x=xd, ws=ws)
    assert torch.equal(st, st2) and torch.equal(o, o2)          # deterministic
    qh, sh = host(q), np.float32(s.item())
    rows = x.shape[0]
    ob = bf16_host(o)
    for r0 in (0, 4096, rows - 512):
        want = O.dequant_scaled(qh[r0:r0 + 512], fmt, sh)
        assert_bf16_of(ob[r0:r0 + 512], want, f"per-tensor rows {r0}..")
    want = oracle_stats_slabs(lambda a, b: O.stats_scaled(x[a:b], qh[a:b], fmt, sh), rows)
    got = qf8.stats_to_dict(st)
    check_stats(got, want, "per-tensor 8192x8192")
    assert got["count"] == x.size and got["saturated"] <= 1
    sqnr = 10 * np.log10(got["signal"] / got["noise"])
    assert 25 < sqnr < 60


@pytest.mark.parametrize("fmt", FMTS)
def test_block_full_round_trip_and_stats(fmt):
    for make, br in ((token_activation, 1), (block_weight, 128)):
        x = make()
        xd = to_device(x)
        q, sc = qf8.quantize_block(xd, br, 128, fmt)[:2]
        o, st = qf8.dequantize_block(q, br, 128, fmt, sc, out_dtype=BF16, x=xd)
        qh, sch = host(q), host(sc)
        ob = bf16_host(o)
        r0 = 128 * 13
        want = O.dequant_block(qh[r0:r0 + 256], br, 128, fmt, sch[r0 // br:(r0 + 256 + br - 1) // br])
        assert_bf16_of(ob[r0:r0 + 256], want, f"block br={br}")
        gs = sch.shape[1]
        want_st = oracle_stats_slabs(
            lambda a, b: O.stats_block(x[a:b], qh[a:b], br, 128, fmt, sch[a // br:(b + br - 1) // br]),
            x.shape[0], 1024 if br == 128 else 512)
        check_stats(qf8.stats_to_dict(st), want_st, f"block {x.shape} br={br}")
        del xd, q, o


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rnd", [O.ROUND_DOWN, O.ROUND_UP])
def test_mx_dual_full_round_trip_and_stats(rnd, fmt):
    x = mx_gradient()
    xd = to_device(x)
    q_row, s_row, q_colT, s_colT = qf8.quantize_mx_dual(xd, fmt, rnd)
    o_r, st_r = qf8.dequantize_mx(q_row, s_row, fmt, out_dtype=BF16, x=xd)
    xt = xd.t().contiguous()
    o_c, st_c = qf8.dequantize_mx(q_colT, s_colT, fmt, out_dtype=BF16, x=xt)
    qr, sr, qc, scT = host(q_row), host(s_row), host(q_colT), host(s_colT)
    orb, ocb = bf16_host(o_r), bf16_host(o_c)
    for r0 in (0, 9000):
        assert_bf16_of(orb[r0:r0 + 256], O.dequant_mx(qr[r0:r0 + 256], sr[r0:r0 + 256], fmt), f"mx row {r0}")
    for c0 in (0, 3000):
        assert_bf16_of(ocb[c0:c0 + 64], O.dequant_mx(qc[c0:c0 + 64], scT[c0:c0 + 64], fmt), f"mx colT {c0}")
    want_r = oracle_stats_slabs(lambda a, b: O.stats_mx(x[a:b], qr[a:b], sr[a:b], fmt), x.shape[0], 1024)
    check_stats(qf8.stats_to_dict(st_r), want_r, "mx rowwise")
    xT = np.ascontiguousarray(x.T)
    want_c = oracle_stats_slabs(lambda a, b: O.stats_mx(xT[a:b], qc[a:b], scT[a:b], fmt), xT.shape[0], 256)
    check_stats(qf8.stats_to_dict(st_c), want_c, "mx columnwise")
    got = qf8.stats_to_dict(st_r)
    if rnd == O.ROUND_UP:
        assert got["saturated"] == 0                  # round-up never saturates
    elif fmt == O.E4M3:
        assert got["saturated"] > 0


def test_stats_nonfinite_and_empty():
    x = small_tensor(16, 64, seed=3)
    xf = bf16_to_f32(x)
    q, am, s = qf8.quantize_per_tensor(to_device(x), O.E4M3)
    xbad = x.copy()
    xbad[0, 0] = 0x7F80      # Inf
    xbad[1, 1] = 0xFFC0      # NaN
    _, st = qf8.dequantize_scaled(q, O.E4M3, s, x=to_device(xbad), want_out=False)
    got = qf8.stats_to_dict(st)
    want = O.stats_scaled(xbad, host(q), O.E4M3, np.float32(s.item()))
    check_stats(got, want, "nonfinite")
    assert got["nonfinite"] == 2 and got["count"] == xf.size - 2
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    _, st = qf8.dequantize_scaled(e, O.E4M3, s, x=torch.empty(0, dtype=BF16, device="cuda"), want_out=False)
    assert qf8.stats_to_dict(st) == {"signal": 0.0, "noise": 0.0, "count": 0, "nonzero": 0, "zeroed": 0,
                                     "saturated": 0, "nonfinite": 0}


# 16384 x 20480 codes: 41,943,040 eight-code units in 40,960 workgroup tiles of 1024 units on the
# de-scaling grid of 16384 workgroups, so workgroups 0..8191 walk three tiles and the others two
# (both halves of the prefetching loop and both of its exits). Row bands checked: one of the first
# tiles, one of the second and the last rows (third tiles).
BIG_ROWS, BIG_COLS = 16384, 20480
BIG_BANDS = ((0, 64), (8000, 8064), (BIG_ROWS - 64, BIG_ROWS))


@pytest.mark.parametrize("mode", ["scaled", "block", "mx"])
def test_dequant_several_tiles_per_workgroup(mode):
    """Random codes of every value (NaN codes included) and random scales: de-scaling alone, BF16
    output, on a tensor large enough for several tiles per workgroup; sampled row bands bit-exact."""
    rng = np.random.default_rng(77)
    q = rng.integers(0, 256, (BIG_ROWS, BIG_COLS), dtype=np.uint8)
    qd = to_device(q)
    fmt = O.E5M2 if mode == "block" else O.E4M3
    if mode == "scaled":
        s = np.float32(rng.uniform(0.01, 1000.0))
        o, _ = qf8.dequantize_scaled(qd, fmt, dev_scale(s), out_dtype=BF16)
        want = lambda r0, r1: O.dequant_scaled(q[r0:r1], fmt, s)
    elif mode == "block":
        sc = (2.0 ** rng.integers(-20, 21, (BIG_ROWS, BIG_COLS // 128))).astype(np.float32)
        sc *= rng.choice(np.array([1.0, 1.0, 3.0, 0.7], np.float32), sc.shape)
        o, _ = qf8.dequantize_block(qd, 1, 128, fmt, to_device(sc), out_dtype=BF16)
        want = lambda r0, r1: O.dequant_block(q[r0:r1], 1, 128, fmt, sc[r0:r1])
    else:
        sb = rng.integers(0, 256, (BIG_ROWS, BIG_COLS // 32), dtype=np.uint8)
        o, _ = qf8.dequantize_mx(qd, to_device(sb), fmt, out_dtype=BF16)
        want = lambda r0, r1: O.dequant_mx(q[r0:r1], sb[r0:r1], fmt)
    for r0, r1 in BIG_BANDS:
        assert_bf16_of(bf16_host(o[r0:r1]), want(r0, r1), f"{mode} rows {r0}..{r1}")
    del o, qd


def test_dequant_several_tiles_per_workgroup_4_code_units():
    """The 4-code units on a tensor where every workgroup walks several tiles: MX to FP32 (one
    16-byte FP32 piece per unit) and groups to BF16 on rows that are only a multiple of 4 codes
    long (8-byte pieces); sampled row bands bit-exact."""
    rng = np.random.default_rng(78)
    q = rng.integers(0, 256, (BIG_ROWS, BIG_COLS), dtype=np.uint8)
    sb = rng.integers(0, 256, (BIG_ROWS, BIG_COLS // 32), dtype=np.uint8)
    o, _ = qf8.dequantize_mx(to_device(q), to_device(sb), O.E5M2, out_dtype=F32)
    for r0, r1 in BIG_BANDS:
        assert_f32_equal(f32_host(o[r0:r1]), O.dequant_mx(q[r0:r1], sb[r0:r1], O.E5M2), f"mx fp32 rows {r0}..{r1}")
    del o
    cols = BIG_COLS + 4                                   # cols % 8 == 4
    q4 = rng.integers(0, 256, (BIG_ROWS, cols), dtype=np.uint8)
    sc = (2.0 ** rng.integers(-20, 21, (BIG_ROWS, (cols + 127) // 128))).astype(np.float32)
    o, _ = qf8.dequantize_block(to_device(q4), 1, 128, O.E4M3, to_device(sc), out_dtype=BF16)
    for r0, r1 in BIG_BANDS:
        assert_bf16_of(bf16_host(o[r0:r1]), O.dequant_block(q4[r0:r1], 1, 128, O.E4M3, sc[r0:r1]),
                       f"block 4-code rows {r0}..{r1}")
    del o


def check_stats_nan_aware(got, want, what):
    """check_stats where a NaN sum (a NaN de-scaled element next to a finite x) must be NaN in both."""
    for k in ("signal", "noise"):
        if np.isnan(want[k]):
            assert np.isnan(got[k]), f"{what}: {k} {got[k]!r}, want NaN"
    check_stats({k: (0.0 if k in ("signal", "noise") and np.isnan(want[k]) else v) for k, v in got.items()},
                {k: (0.0 if k in ("signal", "noise") and np.isnan(v) else v) for k, v in want.items()}, what)


# 2051 x 4128 = 529,158 sixteen-code units: 2067 whole workgroup tiles of 256 units and a partial
# one of 6 units, over a statistics grid of 1024 workgroups (so workgroups 0..18 take three tiles)
NF_ROWS, NF_COLS = 2051, 4128
NF_TILE = 256 * 16


def nonfinite_inputs(xdt):
    """The clean x and a copy with Inf/NaN in whole tiles of several workgroups (first, second and
    third tile of a workgroup) and in the partial last tile; Inf and NaN of both signs."""
    x = small_tensor(NF_ROWS, NF_COLS, seed=11)
    bad = x.copy()
    flat = bad.reshape(-1)
    n = flat.size
    pos = {5 * NF_TILE + 77: 0x7F80, 5 * NF_TILE + 78: 0xFF80, 1724 * NF_TILE + 4000: 0x7FC0,
           2051 * NF_TILE + 9: 0xFFC0, n - 5: 0x7F80}
    for p, v in pos.items():
        flat[p] = v
    if xdt == "f32":
        return bf16_to_f32(x), bf16_to_f32(bad)
    return x, bad


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["scaled", "block", "mx"])
def test_stats_nonfinite_in_whole_tiles(mode, xdt):
    """Inf/NaN inside whole tiles, where a wave sums without the per-element filter and starts
    over once its sum turns non-finite, beside waves and workgroups without them, plus one in
    the partial last tile (filtered per element). MX also puts the NaN scale byte 0xFF on one
    block of a whole tile: its elements de-scale to NaN and make the noise sum NaN."""
    x, bad = nonfinite_inputs(xdt)
    xd, badd = to_device(x), to_device(bad)
    fmt = O.E4M3
    if mode == "scaled":
        q, _, s = qf8.quantize_per_tensor(xd, fmt)
        o, st = qf8.dequantize_scaled(q, fmt, s, out_dtype=F32, x=badd)
        qh, sh = host(q), np.float32(s.item())
        want = O.stats_scaled(bad, qh, fmt, sh)
        want_o = O.dequant_scaled(qh, fmt, sh)
    elif mode == "block":
        q, sc = qf8.quantize_block(xd, 1, 128, fmt)[:2]
        o, st = qf8.dequantize_block(q, 1, 128, fmt, sc, out_dtype=F32, x=badd)
        qh, sch = host(q), host(sc)
        want = O.stats_block(bad, qh, 1, 128, fmt, sch)
        want_o = O.dequant_block(qh, 1, 128, fmt, sch)
    else:
        q, s_row = qf8.quantize_mx_dual(xd, fmt, O.ROUND_DOWN, colwise=False)[:2]
        c0 = 700 * NF_TILE + 100                               # a block inside workgroup 700's first tile
        s_row[c0 // NF_COLS, (c0 % NF_COLS) // 32] = 0xFF
        o, st = qf8.dequantize_mx(q, s_row, fmt, out_dtype=F32, x=badd)
        qh, sh = host(q), host(s_row)
        want = O.stats_mx(bad, qh, sh, fmt)
        want_o = O.dequant_mx(qh, sh, fmt)
        assert np.isnan(want["noise"])
    got = qf8.stats_to_dict(st)
    check_stats_nan_aware(got, want, f"{mode} {xdt} non-finite")
    assert got["nonfinite"] == 5
    assert_f32_equal(f32_host(o), want_o, f"{mode} {xdt} output beside non-finite x")
    # the same tensor without the non-finite values: the clean sums, all elements counted
    _, st2 = (qf8.dequantize_scaled(q, fmt, s, x=xd, want_out=False) if mode == "scaled" else
              qf8.dequantize_block(q, 1, 128, fmt, sc, x=xd, want_out=False) if mode == "block" else
              qf8.dequantize_mx(q, s_row, fmt, x=xd, want_out=False))
    want2 = (O.stats_scaled(x, qh, fmt, sh) if mode == "scaled" else O.stats_block(x, qh, 1, 128, fmt, sch)
             if mode == "block" else O.stats_mx(x, qh, sh, fmt))
    check_stats_nan_aware(qf8.stats_to_dict(st2), want2, f"{mode} {xdt} clean")
    assert qf8.stats_to_dict(st2)["count"] == x.size


def test_delayed_spike_saturation_counted():
    """The pages' delayed-scaling failure: a 50 under S = 22.4 saturates (counted) and comes
    back as 20."""
    x = np.full((4, 64), 1.0, np.float32)
    x[2, 5] = 50.0
    sd = dev_scale(448 / 20)
    q = qf8.qf8_cast_scaled(to_device(x), O.E4M3, sd)
    o, st = qf8.dequantize_scaled(q, O.E4M3, sd, out_dtype=F32, x=to_device(x))
    assert round(float(f32_host(o)[2, 5]), 4) == 20.0
    got = qf8.stats_to_dict(st)
    assert got["saturated"] == 1
    check_stats(got, O.stats_scaled(x, host(q), O.E4M3, np.float32(448 / 20)), "spike")
