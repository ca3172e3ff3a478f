"""GPU parity of the FP4 quantizers against the CPU oracle, byte-exact on packed E2M1 codes and on
the scale bytes (E8M0 for MXFP4, E4M3 for NVFP4) and bit-exact on the NVFP4 tensor scale.

MXFP4 (quantize_mxfp4_dual):
  * an exhaustive domain: for every BF16 amax exponent (mantissas on both sides of the 1.5
    round-up boundary) blocks holding every BF16 magnitude not above that amax, random signs,
    rowwise and columnwise, both rounding modes;
  * small and ragged shapes over several 128-row tiles, BF16 and FP32, single directions,
    all-zero blocks and -0, extreme magnitudes, Inf/NaN (flag and 0xFF scale);
  * the full 16384 x 4096 gradient workload in both rounding modes, every byte.
NVFP4 (quantize_nvfp4):
  * blocks whose amax spans the E4M3 block-scale range under S_t = 1 (a 2688 in the tensor),
    each holding every BF16 magnitude down to amax / 4096 with random signs;
  * quotients x * S_t / decode(e_b) on and next to every E2M1 midpoint, fp32 and BF16, unit and
    random tensor scales, through both kernels (the oracle rounds each quotient once);
  * random BF16 and FP32 tensors of several shapes (S_t != 1), a caller-given amax equal to and
    below the measured one, an all-zero tensor, a tensor with a subnormal amax, Inf/NaN;
  * the full 16384 x 4096 workload, every byte.
"""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import bf16_bits, mx_gradient, small_tensor
from qf8_test_utils import assert_bytes_equal, holder_lib, host, parallel_row_slabs, time_beside_holders, to_device

pytestmark = pytest.mark.gpu

RND = [O.ROUND_DOWN, O.ROUND_UP]
RID = ["down", "up"]


# ---- MXFP4 -------------------------------------------------------------------------------------

def run_mx(x, rnd, row=True, col=True):
    xd = to_device(x)
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows, cols = x.shape
    out = {}                                  # poisoned, so that any byte left unwritten shows
    if row:
        out["q_row"] = torch.full((rows, cols // 2), 0xA5, dtype=torch.uint8, device="cuda")
        out["s_row"] = torch.full((rows, cols // 32), 0xA5, dtype=torch.uint8, device="cuda")
    if col:
        out["q_colT"] = torch.full((cols, rows // 2), 0xA5, dtype=torch.uint8, device="cuda")
        out["s_colT"] = torch.full((cols, rows // 32), 0xA5, dtype=torch.uint8, device="cuda")
    r = qf8.quantize_mxfp4_dual(xd, rnd, rowwise=row, colwise=col, nonfinite=nf, **out)
    torch.cuda.synchronize()
    return [None if t is None else host(t) for t in r] + [int(nf.item())]


def check_mx(x, rnd, row=True, col=True, tag=""):
    g = run_mx(x, rnd, row, col)
    w = O.quantize_mxfp4(x, rnd, row=row, col=col)
    for i, name in enumerate(("q_row", "s_row", "q_colT", "s_colT")):
        if w[i] is None:
            assert g[i] is None
            continue
        assert_bytes_equal(g[i], w[i], name, f" [{tag} rnd={rnd} shape={x.shape}]")
    assert g[4] == w[4]


def exhaustive_blocks(seed=0):
    """[G, 32] BF16 blocks: for each amax A (every exponent field, mantissas 0x00/0x40/0x41/0x7F
    and a few subnormals) every BF16 magnitude <= A, 31 per block next to A, random signs, A at
    a varying position."""
    rng = np.random.default_rng(seed)
    mags = np.arange(0, 0x7F80, dtype=np.uint32)
    amaxes = [a for e in range(1, 255) for a in ((e << 7) | 0x00, (e << 7) | 0x40, (e << 7) | 0x41, (e << 7) | 0x7F)]
    amaxes += [0x0001, 0x0040, 0x007F]
    blocks = []
    for a in amaxes:
        below = mags[: a + 1]
        ng = -(-len(below) // 31)
        body = np.resize(below, ng * 31).reshape(ng, 31)
        blocks.append(np.concatenate([np.full((ng, 1), a, np.uint32), body], axis=1))
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


@pytest.mark.parametrize("rnd", RND, ids=RID)
def test_mxfp4_exhaustive_rowwise(exhaustive, rnd):
    check_mx(exhaustive, rnd, row=True, col=False, tag="exhaustive-row")


@pytest.mark.parametrize("rnd", RND, ids=RID)
def test_mxfp4_exhaustive_columnwise(exhaustive, rnd):
    check_mx(np.ascontiguousarray(exhaustive.T), rnd, row=False, col=True, tag="exhaustive-col")


@pytest.mark.parametrize("shape", [(32, 32), (64, 96), (128, 512), (256, 1024), (160, 544), (96, 1056), (416, 800),
                                   (544, 256)])
@pytest.mark.parametrize("rnd", RND, ids=RID)
def test_mxfp4_dual_small_bf16(shape, rnd):
    check_mx(mx_gradient(*shape, seed=sum(shape)), rnd, tag="dual-bf16")


@pytest.mark.parametrize("shape", [(32, 32), (64, 288), (160, 544), (288, 160)])
@pytest.mark.parametrize("rnd", RND, ids=RID)
def test_mxfp4_dual_small_fp32(shape, rnd):
    rng = np.random.default_rng(5)
    x = (rng.laplace(0, 1e-3, shape) * np.where(rng.random(shape) < 0.01, 1e4, 1.0)).astype(np.float32)
    check_mx(x, rnd, tag="dual-fp32")


@pytest.mark.parametrize("rnd", RND, ids=RID)
def test_mxfp4_single_direction_and_ragged(rnd):
    check_mx(small_tensor(37, 64, seed=3), rnd, row=True, col=False, tag="row-ragged-rows")
    check_mx(small_tensor(130, 96, seed=4), rnd, row=True, col=False, tag="row-ragged-rows")
    check_mx(small_tensor(64, 40, seed=5), rnd, row=False, col=True, tag="col-narrow")
    check_mx(small_tensor(96, 520, seed=6), rnd, row=False, col=True, tag="col-ragged-cols")
    check_mx(small_tensor(320, 288, seed=8), rnd, row=False, col=True, tag="col-two-tile-rows")
    x = (np.random.default_rng(7).standard_normal((96, 36)) * 10).astype(np.float32)
    check_mx(x, rnd, row=False, col=True, tag="col-fp32-ragged")
    rng = np.random.default_rng(9)
    for shape in [(37, 64), (130, 96), (1, 32)]:          # FP32 rows in pairs, the second one missing
        x = (rng.standard_normal(shape) * np.exp(rng.uniform(-3, 3, (shape[0], 1)))).astype(np.float32)
        check_mx(x, rnd, row=True, col=False, tag=f"row-ragged-rows-fp32 {shape}")


def test_mxfp4_zero_blocks_and_extremes():
    x = np.zeros((64, 64), np.uint16)
    x[3, 5] = 0x8000                     # -0 inside an all-zero block -> zero codes
    x[40, 40] = 0x4000
    x[41, 41] = 0x8001                   # negative subnormal
    x[0, 32:] = 0x7F7F                   # largest finite BF16
    x[1, 32:] = 0x0001                   # smallest subnormal
    x[2, 32] = 0x7F7F
    x[2, 33] = 0x0001
    x[5, 32:] = 0x80FF
    for rnd in RND:
        check_mx(x, rnd, tag="zeros-extremes")


def test_mxfp4_nonfinite():
    x = small_tensor(64, 64, seed=9)
    x[7, 9] = 0x7F80
    x[50, 33] = 0x7FC1
    g = run_mx(x, O.ROUND_UP)
    w = O.quantize_mxfp4(x, O.ROUND_UP)
    assert g[4] == 1 and w[4] == 1
    assert g[1][7, 0] == 0xFF and g[1][50, 1] == 0xFF and g[3][9, 0] == 0xFF and g[3][33, 1] == 0xFF
    ok = np.ones(g[1].shape, bool)
    ok[7, 0] = ok[50, 1] = False
    assert np.array_equal(g[1][ok], w[1][ok])
    qok = np.repeat(ok, 16, axis=1)      # 16 packed bytes per block of 32
    assert np.array_equal(g[0][qok], w[0][qok])


@pytest.fixture(scope="module")
def gradient_full():
    return mx_gradient()


@pytest.mark.parametrize("rnd", RND, ids=RID)
def test_mxfp4_full_size_gradient(gradient_full, rnd):
    x = gradient_full
    rows, cols = x.shape
    g = run_mx(x, rnd)
    parts = parallel_row_slabs(lambda r0, r1: O.quantize_mxfp4(x[r0:r1], rnd), rows, 1024)
    assert_bytes_equal(g[0], np.concatenate([p[0] for p in parts], axis=0), "q_row", " [16384x4096]")
    assert_bytes_equal(g[1], np.concatenate([p[1] for p in parts], axis=0), "s_row", " [16384x4096]")
    assert_bytes_equal(g[2], np.concatenate([p[2] for p in parts], axis=1), "q_colT", " [16384x4096]")
    assert_bytes_equal(g[3], np.concatenate([p[3] for p in parts], axis=1), "s_colT", " [16384x4096]")
    assert g[4] == 0


# ---- NVFP4 -------------------------------------------------------------------------------------

def run_nv(x, amax_in=None):
    xd = to_device(x)
    rows, cols = x.shape
    q = torch.full((rows, cols // 2), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, cols // 16), 0xA5, dtype=torch.uint8, device="cuda")
    st = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    a = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    ain = None if amax_in is None else torch.tensor([amax_in], dtype=torch.float32, device="cuda")
    qf8.quantize_nvfp4(xd, amax_in=ain, q=q, s_blk=s, tensor_scale=st, amax_out=a, nonfinite=nf)
    torch.cuda.synchronize()
    return host(q), host(s), np.float32(st.item()), np.float32(a.item()), int(nf.item())


def check_nv(x, amax_in=None, tag=""):
    g = run_nv(x, amax_in)
    w = O.quantize_nvfp4(x, amax_in=amax_in)
    extra = f" [{tag} shape={x.shape}]"
    assert g[2] == w[2], f"tensor scale{extra}: {g[2]!r} vs {w[2]!r}"
    assert g[3] == w[3] and g[4] == w[4], extra
    assert_bytes_equal(g[1], w[1], "s_blk", extra)
    assert_bytes_equal(g[0], w[0], "q", extra)
    return g


def nv_domain(seed=1):
    """[G, 16] BF16 blocks under S_t = 1: a 2688 in the first block; block amaxes with every
    exponent from 2^-10 to 2^10 and mantissas 0x00/0x20/0x40/0x41/0x55/0x7F, each block holding
    15 BF16 magnitudes between amax / 4096 and amax (all of them over consecutive blocks)."""
    rng = np.random.default_rng(seed)
    blocks = [np.array([0x4528] + [0] * 15, np.uint32)]          # 2688.0
    for e in range(127 - 10, 127 + 11):                          # amax < 2048 < 2688
        for m in (0x00, 0x20, 0x40, 0x41, 0x55, 0x7F):
            a = (e << 7) | m
            lo = a - (12 << 7)
            below = np.arange(max(lo, 0), a + 1, dtype=np.uint32)
            ng = -(-len(below) // 15)
            body = np.resize(below, ng * 15).reshape(ng, 15)
            blocks.append(np.concatenate([np.full((ng, 1), a, np.uint32), body], axis=1).reshape(-1))
    b = np.concatenate(blocks).reshape(-1, 16)
    b |= (rng.integers(0, 2, b.shape, dtype=np.uint32) << 15)
    b[0, 0] = 0x4528
    pad = (-b.shape[0]) % 8
    if pad:
        b = np.concatenate([b, np.zeros((pad, 16), np.uint32)], axis=0)
    return b.reshape(-1, 128).astype(np.uint16)


def test_nvfp4_block_scale_domain():
    x = nv_domain()
    g = check_nv(x, tag="domain")
    assert g[2] == 1.0


@pytest.mark.parametrize("shape", [(1, 16), (16, 16), (64, 256), (33, 48), (1000, 1008)])
def test_nvfp4_random_bf16(shape):
    x = mx_gradient(*shape, seed=sum(shape) + 1)
    check_nv(x, tag="bf16")


@pytest.mark.parametrize("shape,scale", [((32, 64), 1.0), ((129, 496), 1e-4), ((7, 4096), 3e5)])
def test_nvfp4_random_fp32(shape, scale):
    rng = np.random.default_rng(shape[0])
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-4, 4, (shape[0], 1))) * scale).astype(np.float32)
    check_nv(x, tag="fp32")


def test_nvfp4_caller_amax():
    x = mx_gradient(64, 256, seed=12)
    a = float(O.amax(x))
    check_nv(x, amax_in=a, tag="amax_in=measured")
    check_nv(x, amax_in=-a, tag="amax_in=-measured")
    check_nv(x, amax_in=a / 16, tag="amax_in=measured/16")
    check_nv(x, amax_in=a * 1000, tag="amax_in=measured*1000")


def test_nvfp4_zero_tiny_and_nonfinite():
    check_nv(np.zeros((4, 64), np.uint16), tag="zeros")
    t = np.zeros((2, 32), np.float32)
    t[0, 0] = np.float32(1e-40)
    t[1, 16] = np.float32(-3e-45)
    t[1, 17] = np.float32(-0.0)
    check_nv(t, tag="tiny")
    x = small_tensor(16, 64, seed=3)
    x[5, 20] = 0x7FC0
    x[9, 63] = 0xFF80
    g = run_nv(x)
    w = O.quantize_nvfp4(x)
    assert g[4] == 1 and w[4] == 1 and g[2] == w[2] == 1.0
    assert g[1][5, 1] == 0x7F and g[1][9, 3] == 0x7F
    ok = np.ones(g[1].shape, bool)
    ok[5, 1] = ok[9, 3] = False
    assert np.array_equal(g[1][ok], w[1][ok])
    assert np.array_equal(g[0][np.repeat(ok, 8, axis=1)], w[0][np.repeat(ok, 8, axis=1)])


def test_nvfp4_full_size(gradient_full):
    x = gradient_full
    rows, _ = x.shape
    g = run_nv(x)
    a = float(O.amax(x))
    parts = parallel_row_slabs(lambda r0, r1: O.quantize_nvfp4(x[r0:r1], amax_in=a), rows, 1024)
    assert g[2] == parts[0][2] and g[3] == np.float32(a) and g[4] == 0
    assert_bytes_equal(g[1], np.concatenate([p[1] for p in parts], axis=0), "s_blk", " [16384x4096]")
    assert_bytes_equal(g[0], np.concatenate([p[0] for p in parts], axis=0), "q", " [16384x4096]")


def run_nv_ws(x, ws):
    xd = to_device(x)
    rows, cols = x.shape
    q = torch.full((rows, cols // 2), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, cols // 16), 0xA5, dtype=torch.uint8, device="cuda")
    st = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    a = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    nf = torch.zeros(1, dtype=torch.int32, device="cuda")
    qf8.quantize_nvfp4(xd, q=q, s_blk=s, tensor_scale=st, amax_out=a, nonfinite=nf, ws=ws)
    torch.cuda.synchronize()
    return host(q), host(s), np.float32(st.item()), np.float32(a.item()), int(nf.item())


def check_nv_big(x, ws, tag):
    """Large inputs (the single-pass path from 2^22 elements), compared on every byte; the oracle
    runs on row slabs with the whole tensor's amax."""
    g = run_nv_ws(x, ws)
    a = float(O.amax(x))
    parts = parallel_row_slabs(lambda r0, r1: O.quantize_nvfp4(x[r0:r1], amax_in=a), x.shape[0], 256)
    assert g[2] == parts[0][2] and g[3] == np.float32(a) and g[4] == 0, tag
    assert_bytes_equal(g[1], np.concatenate([p[1] for p in parts], axis=0), "s_blk", f" [{tag}]")
    assert_bytes_equal(g[0], np.concatenate([p[0] for p in parts], axis=0), "q", f" [{tag}]")
    words = host(ws.view(torch.int32)[:qf8.BARRIER_WORDS]).copy()
    words[2] = 0                                   # the give-up timeout override a test may set
    assert not words.any(), f"workspace not left zero [{tag}]"


def test_nvfp4_single_pass_threshold_and_fp32():
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    check_nv_big(mx_gradient(1, (1 << 22) - 16, seed=21), ws, "2^22 - 16 elements (amax pass)")
    check_nv_big(mx_gradient(1, 1 << 22, seed=22), ws, "2^22 elements (single pass)")
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((4096, 8192)) * np.exp(rng.uniform(-2, 2, (4096, 1)))).astype(np.float32)
    check_nv_big(x, ws, "4096x8192 fp32 (beyond the held capacity)")


def test_nvfp4_single_pass_ragged_scale_groups():
    """Single-pass sizes with ragged ends: the vector count is not a multiple of the 8 (BF16) or
    16 (FP32) vectors that one 16-lane row of a wave holds, so the last rows run partly out of
    range; BF16 and FP32, every byte compared."""
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    check_nv_big(mx_gradient(2049, 2064, seed=24), ws, "2049x2064 bf16 (vectors % 8 = 2)")
    rng = np.random.default_rng(25)
    x = (rng.standard_normal((1025, 4112)) * np.exp(rng.uniform(-2, 2, (1025, 1)))).astype(np.float32)
    check_nv_big(x, ws, "1025x4112 fp32 (vectors % 16 = 4)")


@pytest.mark.parametrize("ticks", [1, 100])
def test_nvfp4_single_pass_give_up(gradient_full, ticks):
    """Waiting workgroups forced to give up at the grid barrier: the released ones cast their slabs."""
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    ws.view(torch.int32)[2] = ticks
    check_nv_big(gradient_full, ws, f"give-up after {ticks} ticks")
    ws.view(torch.int32)[2] = 0
    check_nv_big(gradient_full[:2048], ws, "default timeout after a give-up run")


def test_nvfp4_single_pass_beside_cu_holders(gradient_full):
    """The single-pass NVFP4 kernel (16384x4096 BF16, 108 MiB held on chip) while a kernel on
    another stream holds 48 KiB of LDS on 8 CUs for 3 ms: about as many waiters give up, per
    shader engine, and the released workgroups cast their slabs. Same bytes as the oracle, the
    workspace left zero, and the call ends in under 1 ms (events on its stream)."""
    lib = holder_lib()
    x = gradient_full
    xd = to_device(x)
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    a = float(O.amax(x))
    parts = parallel_row_slabs(lambda r0, r1: O.quantize_nvfp4(x[r0:r1], amax_in=a), x.shape[0], 256)
    wq = np.concatenate([p[0] for p in parts], axis=0)
    wsb = np.concatenate([p[1] for p in parts], axis=0)
    q = torch.empty(wq.shape, dtype=torch.uint8, device="cuda")
    sb = torch.empty(wsb.shape, dtype=torch.uint8, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    times = []
    for rep in range(3):
        print(f"nvfp4 single pass beside 8 CU holders, rep {rep}", flush=True)
        q.fill_(0xA5)
        sb.fill_(0xA5)
        times.append(time_beside_holders(lib, 8, lambda: qf8.quantize_nvfp4(xd, q=q, s_blk=sb, tensor_scale=ts, ws=ws)))
        assert np.float32(ts.item()) == parts[0][2], rep
        assert_bytes_equal(host(sb), wsb, "s_blk", f" [beside 8 CU holders, rep {rep}]")
        assert_bytes_equal(host(q), wq, "q", f" [beside 8 CU holders, rep {rep}]")
        words = host(ws.view(torch.int32)[:qf8.BARRIER_WORDS]).copy()
        words[2] = 0
        assert not words.any(), "workspace not left zero"
    print(f"call times (us): {[round(t) for t in times]}", flush=True)
    assert max(times) < 1000.0, times


@pytest.mark.parametrize("grid", [17, 300])
def test_nvfp4_single_pass_other_grids(grid):
    """Other workgroup counts of the single-pass kernel: a ragged last barrier group (17), and
    more workgroups than fit at once on a 256-CU device (300: the late ones run once waiters have
    given up, whose slabs the released workgroups cast)."""
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    qf8.qf8_set_onepass_grid(grid)
    try:
        check_nv_big(mx_gradient(2048, 4096, seed=40 + grid), ws, f"grid {grid}")
    finally:
        qf8.qf8_set_onepass_grid(0)


MIDPOINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]          # between consecutive E2M1 values


def nv_tie_tensor(rows, cols, seed, dtype, unit_scale):
    """A tensor whose blocks put x * S_t / decode(e_b) on and next to the E2M1 midpoints, where
    one rounding of the exact quotient decides the code. Element [0, 0] is the tensor amax A:
    2688 (S_t = 1) when unit_scale, else a random A. Every block takes a random E4M3 code e,
    holds its amax 6 * decode(e) / S_t and elements m * decode(e) / S_t for random midpoints m,
    exact or moved by up to two steps of the input format (fp32 or BF16), with random signs."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    A = f32(2688.0) if unit_scale else f32(rng.uniform(1, 2) * 2.0 ** int(rng.integers(-8, 8)))
    s_t = O.nvfp4_tensor_scale(float(A))
    nb = rows * cols // 16
    e = rng.integers(1, 127, nb)
    dec = np.array([O.decode(O.E4M3, c) for c in range(128)])[e]
    m = np.array(MIDPOINTS)[rng.integers(0, 7, (nb, 16))]
    x = (m * dec[:, None] / float(s_t)).astype(np.float32)
    x[:, 0] = (6.0 * dec / float(s_t)).astype(np.float32)
    if dtype == "bf16":
        bits = (x.view(np.uint32) >> 16).astype(np.int32)        # exact: at most 7 significant bits
        bits[:, 1:] += rng.integers(-2, 3, (nb, 15))
        bits |= rng.integers(0, 2, bits.shape) << 15
        out = bits.astype(np.uint16).reshape(rows, cols)
        out[0, 0] = 0x4528                                        # 2688.0
        return out
    u = x.view(np.int32)
    u[:, 1:] += rng.integers(-2, 3, (nb, 15)).astype(np.int32)
    x = u.view(np.float32) * np.where(rng.integers(0, 2, x.shape) == 1, f32(-1), f32(1))
    x = x.reshape(rows, cols)
    x[0, 0] = A
    return x


@pytest.mark.parametrize("dtype,unit", [("fp32", True), ("fp32", False), ("bf16", True)])
def test_nvfp4_midpoint_ties_streaming(dtype, unit):
    """Quotients on and within two input steps of every E2M1 midpoint (and block amaxes on E4M3
    midpoints' neighbours), through the streaming kernel: every byte equals the oracle, which
    rounds each quotient once."""
    x = nv_tie_tensor(96, 512, seed=31 + unit, dtype=dtype, unit_scale=unit)
    g = check_nv(x, tag=f"ties {dtype} unit_scale={unit}")
    if unit:
        assert g[2] == 1.0


@pytest.mark.parametrize("dtype,unit", [("fp32", False), ("bf16", True)])
def test_nvfp4_midpoint_ties_single_pass(dtype, unit):
    """The same construction at 2^22 elements, through the single-pass kernel (the tensor held on
    chip across its grid barrier; the elements whose two estimates disagree are recomputed
    exactly from the vector still in registers or LDS, before its store)."""
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    x = nv_tie_tensor(2048, 2048, seed=35 + unit, dtype=dtype, unit_scale=unit)
    check_nv_big(x, ws, f"ties {dtype} unit_scale={unit} 2048x2048")



def nv_overflow_tensor(rows, cols, seed, dtype):
    """A tensor amax A = 2^-120, so small that 2688 / A exceeds FLT_MAX: S_t is held at FLT_MAX,
    and S_t / decode(e_b) overflows for every block code below about 1. Block amaxes A * 2^-u
    with u uniform in [0, 12] put about half of the blocks there; each block holds its amax,
    uniform magnitudes below it (fp32 subnormals among them), 5% zeros, and random signs."""
    rng = np.random.default_rng(seed)
    nb = rows * cols // 16
    ab = 2.0 ** -120 * 2.0 ** -rng.uniform(0, 12, nb)
    v = rng.uniform(0, 1, (nb, 16)) * ab[:, None]
    v[:, 0] = ab
    v[:, 1:][rng.random((nb, 15)) < 0.05] = 0.0
    x = (v * np.where(rng.integers(0, 2, v.shape) == 1, -1.0, 1.0)).astype(np.float32).reshape(rows, cols)
    x[0, 0] = np.float32(2.0 ** -120)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)      # truncation: 2^-120 stays the amax
    return x


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_nvfp4_single_pass_overflowing_factors(dtype):
    """Blocks whose element factor S_t / decode(e_b) overflows get the factors (0, Inf): their two
    code estimates are 0 and +-6, never adjacent, so every nonzero element goes through the exact
    search, and zeros keep their signs. Streaming kernel (96x512) and single-pass kernel (2^22
    elements), every byte compared."""
    check_nv(nv_overflow_tensor(96, 512, seed=40, dtype=dtype), tag=f"overflowing factors {dtype}")
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    x = nv_overflow_tensor(2048, 2048, seed=41, dtype=dtype)
    g = run_nv_ws(x, ws)
    assert g[2] == np.finfo(np.float32).max, g[2]
    check_nv_big(x, ws, f"overflowing factors {dtype} 2048x2048")

# ---- FP4 de-scaling ------------------------------------------------------------------------------

def _f32_equal(got, want, what):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    g, w = got[~gn].view(np.uint32), want[~wn].view(np.uint32)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{what}: {bad.size} values differ, first {got[~gn][bad[0]]!r} vs {want[~wn][bad[0]]!r}"


def _bf16_of(got_bits, want_f32, what):
    wb = O.to_bf16(want_f32)
    nan = np.isnan(np.asarray(want_f32, np.float32))
    assert np.array_equal(((got_bits & 0x7FFF) > 0x7F80), nan), f"{what}: NaN positions differ"
    assert_bytes_equal(got_bits[~nan].view(np.uint8), wb[~nan].view(np.uint8), what)


def _both_outputs(run, want, what):
    out32 = run(torch.float32)
    torch.cuda.synchronize()
    _f32_equal(out32.cpu().numpy(), want, what + " fp32")
    out16 = run(torch.bfloat16)
    torch.cuda.synchronize()
    _bf16_of(out16.cpu().view(torch.int16).numpy().view(np.uint16), want, what + " bf16")


def test_dequant_mxfp4_every_code_pair_every_scale_byte():
    """256 rows x 512 columns: each row's 256 code bytes are all byte values (every ordered pair
    of codes), and the 16 scale bytes of row r are (r + 17 b) mod 256: every code with every
    E8M0 byte, 0xFF (NaN) included."""
    rows, cols = 256, 512
    q = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    sb = ((np.arange(rows)[:, None] + 17 * np.arange(cols // 32)[None, :]) % 256).astype(np.uint8)
    want = O.dequant_mxfp4(q, sb)
    qd, sd = to_device(q), to_device(sb)
    _both_outputs(lambda dt: qf8.dequantize_mxfp4(qd, sd, out_dtype=dt), want, "mxfp4 exhaustive")


@pytest.mark.parametrize("s_t", [1.0, 3.7, 2688.0 / 5.3, 1e-30, 7.9e-36, 1e30, 3.4028235e38])
def test_dequant_nvfp4_every_code_every_block_scale(s_t):
    """128 rows x 512 columns: every code byte in every row, and the 32 block-scale codes of row r
    are (r + 5 b) mod 128: every E2M1 code with every E4M3 scale code (0x7F, NaN, included)."""
    rows, cols = 128, 512
    q = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    sb = ((np.arange(rows)[:, None] + 5 * np.arange(cols // 16)[None, :]) % 128).astype(np.uint8)
    want = O.dequant_nvfp4(q, sb, s_t)
    qd, sd = to_device(q), to_device(sb)
    st = torch.tensor([np.float32(s_t)], dtype=torch.float32, device="cuda")
    _both_outputs(lambda dt: qf8.dequantize_nvfp4(qd, sd, st, out_dtype=dt), want, f"nvfp4 exhaustive S_t={s_t}")


def test_dequant_fp4_round_trip_full(gradient_full):
    """Quantize the 16384 x 4096 workload on the GPU, de-scale on the GPU, and compare with the
    oracle's de-scaling of the same codes (both MXFP4 directions and NVFP4)."""
    xd = to_device(gradient_full)
    q_row, s_row, q_colT, s_colT = qf8.quantize_mxfp4_dual(xd, O.ROUND_DOWN)
    for q, s, name in ((q_row, s_row, "mxfp4 rowwise"), (q_colT, s_colT, "mxfp4 columnwise")):
        want = O.dequant_mxfp4(host(q), host(s))
        _both_outputs(lambda dt: qf8.dequantize_mxfp4(q, s, out_dtype=dt), want, name)
    qn, sn, st = qf8.quantize_nvfp4(xd)
    want = O.dequant_nvfp4(host(qn), host(sn), np.float32(st.item()))
    _both_outputs(lambda dt: qf8.dequantize_nvfp4(qn, sn, st, out_dtype=dt), want, "nvfp4")
