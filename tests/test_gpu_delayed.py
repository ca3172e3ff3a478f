"""GPU parity of quantize_delayed (device-resident amax history) against the oracle state machine.

  * the hand-computed sequence of the oracle tests (history 3, Interval 2, N_guard 1) and the
    delayed-spike worked example: codes, scales, amax, history after every step;
  * long random sequences with several (history, Interval, N_guard) settings, both formats;
  * reset (restart with current scaling), checkpoint/resume of the state, non-finite steps;
  * the estimators (maximum, most recent, mean as the fp32 sum oldest to newest): hand
    sequence, long histories (64 and 1024 entries) that wrap several times, an input whose mean
    depends on the summation order, and a history whose fp32 sum overflows;
  * the amax split over the Interval steps (one piece of the flattened tensor measured per step,
    the window's maximum appended on update steps): a hand sequence, pieces that start and end
    inside 16-byte vectors and in the scalar tail, BF16 and FP32, every estimator, Inf/NaN in
    and out of the measured piece, and the full drifting workload;
  * the full drifting-std workload: 100 iterations of 4096x14336 (history 16, Interval 5,
    N_guard 3, E4M3); every step's scale and amax bit-exact against the oracle state machine,
    and the codes of several steps compared on every byte.
"""
import numpy as np
import pytest
import torch

import mx_block_scaled_amax_amd as qf8
import oracle as O
from synthetic import bf16_bits, delayed_base, delayed_sigmas, delayed_step_input, small_tensor
from qf8_test_utils import assert_bytes_equal, host, to_device

pytestmark = pytest.mark.gpu


class Pair:
    """A GPU delayed state and the oracle state machine driven with the same inputs."""

    def __init__(self, hist_len, interval, n_guard, fmt, estimator=None, split=False):
        self.g = qf8.DelayedState(hist_len, interval, n_guard, fmt, estimator=estimator, split=split)
        self.o = O.Delayed(hist_len, interval, n_guard, fmt, estimator=estimator or 0, split=split)
        self.fmt = fmt
        self.nf = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.s = torch.zeros(1, dtype=torch.float32, device="cuda")
        self.a = torch.zeros(1, dtype=torch.float32, device="cuda")

    def step(self, x, tag=""):
        self.nf.zero_()
        xd = to_device(x)
        q = qf8.quantize_delayed(xd, self.g, scale_used=self.s, amax_out=self.a, nonfinite=self.nf)
        torch.cuda.synchronize()
        wq, ws, wa, wnf = self.o.step(x)
        assert np.float32(self.s.item()) == ws, f"scale {tag}: {self.s.item()!r} vs {ws!r}"
        a = np.float32(self.a.item())
        assert (a == wa) or (np.isnan(a) and np.isnan(wa)), f"amax {tag}"
        assert int(self.nf.item()) == wnf
        if not wnf:
            assert_bytes_equal(host(q), wq, "q", f" [{tag}]")
        h, c, st = self.o.state()
        assert self.g.history_list() == list(h), f"history {tag}"
        assert self.g.step == st
        return q


def tensor_with_amax(a):
    return np.array([[a, -a / 2, 0.3 * a, -0.01 * a]], np.float32)


def test_hand_sequence():
    p = Pair(3, 2, 1, O.E4M3)
    for t, a in enumerate([4, 8, 2, 16, 1, 32, 64, 0.5, 0.25, 128, 2]):
        p.step(tensor_with_amax(a), f"t={t}")


def test_spike_example():
    p = Pair(16, 1, 0, O.E4M3)
    p.step(np.array([[20.0, 1.0, -3.0]], np.float32), "t=0")
    q = p.step(np.array([[50.0, 1.0]], np.float32), "t=1")
    assert host(q)[0, 0] == 0x7E                       # 50 * 22.4 saturates to 448


@pytest.mark.parametrize("hist,interval,guard,fmt", [(16, 5, 3, O.E4M3), (1, 1, 0, O.E5M2), (4, 3, 2, O.E4M3),
                                                     (64, 7, 10, O.E5M2)])
def test_random_sequences(hist, interval, guard, fmt):
    rng = np.random.default_rng(hist * 100 + interval)
    p = Pair(hist, interval, guard, fmt)
    base = small_tensor(33, 72, seed=hist)
    basef = (base.astype(np.uint32) << 16).view(np.float32)
    for t in range(40):
        x = bf16_bits(basef * np.float32(2.0 ** rng.uniform(-6, 6)))
        p.step(x, f"t={t}")


ESTIMATORS = [qf8.EST_MAX, qf8.EST_RECENT, qf8.EST_MEAN]


@pytest.mark.parametrize("est", ESTIMATORS)
def test_estimator_hand_sequence(est):
    p = Pair(3, 2, 1, O.E4M3, est)
    assert p.g.struct.estimator == est
    for t, a in enumerate([4, 8, 2, 16, 1, 32, 64, 0.5, 0.25, 128, 2, 3]):
        p.step(tensor_with_amax(a), f"est={est} t={t}")


@pytest.mark.parametrize("est", ESTIMATORS)
@pytest.mark.parametrize("hist,interval,steps", [(64, 1, 150), (1024, 1, 1100), (1024, 3, 60)])
def test_estimator_long_histories(est, hist, interval, steps):
    """Histories of 64 and 1024 entries: the mean sums up to 1024 fp32 values in FIFO order, and
    the ring wraps (150 steps through 64 entries, 1100 through 1024)."""
    rng = np.random.default_rng(7 * hist + est)
    p = Pair(hist, interval, 2, O.E4M3 if est != qf8.EST_RECENT else O.E5M2, est)
    basef = (small_tensor(8, 40, seed=hist + est).astype(np.uint32) << 16).view(np.float32)
    for t in range(steps):
        p.step(bf16_bits(basef * np.float32(2.0 ** rng.uniform(-20, 20))), f"est={est} t={t}")


def test_mean_summation_order():
    """History 2^24, 1, 1, 1 (then wrapping): in fp32 the oldest-to-newest sum stays 2^24 (each +1
    is a tie to even), so the next step casts with 448 / 2^22; newest-to-oldest would sum to
    2^24 + 4 and give another scale."""
    p = Pair(4, 1, 0, O.E4M3, qf8.EST_MEAN)
    for t, a in enumerate([2.0 ** 24, 1.0, 1.0, 1.0]):
        p.step(tensor_with_amax(a), f"t={t}")
    p.step(tensor_with_amax(3.0), "t=4")
    assert np.float32(p.s.item()) == np.float32(448.0 * 2.0 ** -22)
    for t, a in enumerate([2.0 ** 24, 1.0, 1.0, 5.0], start=5):
        p.step(tensor_with_amax(a), f"t={t}")


def test_mean_sum_overflow():
    """Two amaxes near the largest BF16 value overflow the fp32 sum; the estimate is infinite and
    the scale falls back to 1 (with the margin), on both sides."""
    p = Pair(4, 1, 1, O.E5M2, qf8.EST_MEAN)
    big = float(np.float32(3.3e38))
    for t, a in enumerate([big, big, 2.0, 4.0, 8.0, 16.0]):
        p.step(bf16_bits(tensor_with_amax(a)), f"t={t}")
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(big) + np.float32(big))


def row(*v):
    return np.array([v], np.float32)


def test_split_hand_sequence():
    p = Pair(4, 2, 0, O.E4M3, split=True)
    assert p.g.struct.flags == qf8.DELAYED_SPLIT_AMAX
    for t, x in enumerate([row(1, 2, 3, 4), row(8, 1, 100, 1), row(100, 1, 2, 16), row(1, 1, 1, 1),
                           row(0.5, 0.5, 0.5, 2), row(3, 0, 0, 0)]):
        p.step(x, f"t={t}")
    assert p.g.history_list() == [4.0, 16.0, 2.0]


def outlier_steps(rng, shape, steps, fp32):
    """Random tensors whose few large entries move from step to step, so the piece amaxes differ
    from the whole amax and from each other."""
    for _ in range(steps):
        x = rng.standard_normal(shape).astype(np.float32) * np.float32(2.0 ** rng.uniform(-6, 6))
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=3, replace=False)
        flat[idx] *= np.float32(rng.uniform(10, 1000))
        yield x if fp32 else bf16_bits(x)


@pytest.mark.parametrize("est", ESTIMATORS)
@pytest.mark.parametrize("interval,shape,fp32", [(5, (33, 73), False), (3, (7, 5), False), (7, (129, 1001), True),
                                                 (4, (301, 4096), False), (2, (1, 3), True), (6, (1024, 999), False)])
def test_split_random_sequences(est, interval, shape, fp32):
    """Pieces of 2409 elements cut in 5 (boundaries inside vectors, 1-element tail), 35 in 3,
    129129 fp32 in 7, a multi-run tensor in 4, 3 elements in 2, and 1023K elements in 6."""
    rng = np.random.default_rng(interval * 1000 + shape[1] + est)
    p = Pair(6, interval, 1, O.E4M3 if est != qf8.EST_MEAN else O.E5M2, est, split=True)
    for t, x in enumerate(outlier_steps(rng, shape, 3 * interval + 2, fp32)):
        p.step(x, f"t={t}")


def test_split_nonfinite_inside_and_outside_the_piece():
    p = Pair(4, 2, 0, O.E4M3, split=True)
    base = small_tensor(16, 40, seed=9)
    x = base.copy()
    p.step(x, "t=0")
    x = base.copy()
    x[2, 5] = 0x7FC0                                   # NaN in piece [0, 320) at step 1
    p.step(x, "nan inside")
    p.step(base, "window dropped")
    assert len(p.g.history_list()) == 1
    x = base.copy()
    x[12, 1] = 0x7F80                                  # Inf outside piece [0, 320) at step 3
    p.step(x, "inf outside")
    p.step(base, "window appended")
    assert len(p.g.history_list()) == 2


def test_split_full_size_drifting_workload():
    """The 4096x14336 drifting workload with the amax split over Interval = 5 steps (pieces of
    11744051 or 11744052 elements): every step's scale, amax and history, codes of three steps."""
    z = delayed_base()
    sig = delayed_sigmas()
    zd = torch.from_numpy(z).cuda()
    st = qf8.DelayedState(16, 5, 3, qf8.E4M3, split=True)
    orc = O.Delayed(16, 5, 3, O.E4M3, split=True)
    s = torch.zeros(1, dtype=torch.float32, device="cuda")
    a = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = qf8.workspace(zd)
    q = torch.empty(z.shape, dtype=torch.uint8, device="cuda")
    for t in range(11):
        xd = (zd * float(sig[t])).to(torch.bfloat16)
        qf8.quantize_delayed(xd, st, q=q, scale_used=s, amax_out=a, ws=ws)
        torch.cuda.synchronize()
        wq, ws_o, wa_o, _ = orc.step(delayed_step_input(z, sig[t]))
        assert np.float32(a.item()) == wa_o, f"amax t={t}"
        assert np.float32(s.item()) == ws_o, f"scale t={t}"
        if t in (0, 4, 10):
            assert_bytes_equal(host(q), wq, "q", f" [4096x14336 split t={t}]")
        assert st.history_list() == list(orc.state()[0]), f"history t={t}"


def test_reset_and_resume():
    p = Pair(4, 2, 3, O.E4M3)
    rng = np.random.default_rng(3)
    xs = [small_tensor(16, 64, seed=i) for i in range(12)]
    for t in range(5):
        p.step(xs[t], f"t={t}")
    # checkpoint: copy the device state and host counter
    ck = (p.g.history.clone(), p.g.meta.clone(), p.g.scale.clone(), p.g.step)
    ock = O.Delayed(4, 2, 3, O.E4M3)
    ock._buf[:] = p.o._buf
    for t in range(5, 9):
        p.step(xs[t], f"t={t}")
    after = [host(qf8.quantize_delayed(to_device(xs[9]), p.g)).copy()]
    # resume from the checkpoint into a fresh state and replay: identical results
    r = Pair(4, 2, 3, O.E4M3)
    r.g.history.copy_(ck[0]); r.g.meta.copy_(ck[1]); r.g.scale.copy_(ck[2]); r.g.step = ck[3]
    r.o = ock
    for t in range(5, 9):
        r.step(xs[t], f"resume t={t}")
    assert np.array_equal(host(qf8.quantize_delayed(to_device(xs[9]), r.g)), after[0])
    # reset: next step is current scaling, history restarts
    qf8.qf8_delayed_reset(p.g)
    p.o.reset()
    p.step(xs[10], "after reset")
    assert p.g.history_list() == [float(np.float32(O.amax(xs[10])))]


def test_nonfinite_step_not_pushed():
    p = Pair(4, 1, 0, O.E4M3)
    p.step(small_tensor(8, 64, seed=1), "t=0")
    x = small_tensor(8, 64, seed=2)
    x[3, 3] = 0x7FC0
    p.step(x, "nan step")
    x[3, 3] = 0xFF80
    p.step(x, "inf step")
    p.step(small_tensor(8, 64, seed=3), "t=3")


def test_fp32_and_ragged():
    p = Pair(8, 2, 1, O.E5M2)
    rng = np.random.default_rng(6)
    for t in range(8):
        x = (rng.standard_normal((13, 29)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        p.step(x, f"t={t}")


def test_full_size_drifting_workload():
    """100 steps of the 4096x14336 drifting workload (H=16, I=5, N=3). On 11 steps (update steps
    and the reuse steps after them, early, middle and late) the oracle's state machine takes the
    real tensor and its codes, scale and amax are compared with the GPU's; on the other steps it
    takes a one-element surrogate with the same amax, bf16(sigma * max|Z|) (rounding is monotone
    and odd), so that its history, scale and step count still follow every step."""
    z = delayed_base()
    sig = delayed_sigmas()
    zd = torch.from_numpy(z).cuda()
    st = qf8.DelayedState(16, 5, 3, qf8.E4M3)
    orc = O.Delayed(16, 5, 3, O.E4M3)
    s = torch.zeros(1, dtype=torch.float32, device="cuda")
    a = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = qf8.workspace(zd)                                   # zero-filled once, reused every step
    q = torch.empty(z.shape, dtype=torch.uint8, device="cuda")
    zmax = float(np.max(np.abs(z)))
    full_steps = {0, 1, 5, 6, 10, 25, 50, 51, 55, 95, 99}
    rows = np.random.default_rng(0).choice(z.shape[0], 64, replace=False)
    for t in range(100):
        xd = (zd * float(sig[t])).to(torch.bfloat16)          # = bf16(fl32(sigma_t * Z))
        qf8.quantize_delayed(xd, st, q=q, scale_used=s, amax_out=a, ws=ws)
        torch.cuda.synchronize()
        if t in (0, 50):   # the device-side input generation reproduces the host generator
            assert np.array_equal(host(xd.view(torch.int16)).view(np.uint16)[rows],
                                  delayed_step_input(z[rows], sig[t]))
        # amax of bf16(sigma*Z) is bf16(sigma*max|Z|): rounding is monotone and odd
        want_amax = np.float32((np.uint32(bf16_bits(np.array([np.float32(sig[t]) * np.float32(zmax)]))[0]) << 16).view(np.float32))
        if t in full_steps:
            print(f"delayed 4096x14336 step {t}: oracle on the whole tensor", flush=True)
            wq, ws_o, wa_o, wnf = orc.step(delayed_step_input(z, sig[t]))
            assert wnf == 0
            assert_bytes_equal(host(q), wq, "q", f" [4096x14336 t={t}]")
        else:
            _, ws_o, wa_o, _ = orc.step(bf16_bits(np.array([[np.float32(sig[t]) * np.float32(zmax)]], np.float32)))
        assert np.float32(a.item()) == want_amax == wa_o, f"amax t={t}"
        assert np.float32(s.item()) == ws_o, f"scale t={t}"
        h, c, stp = orc.state()
        assert st.step == stp
    assert st.history_list() == list(orc.state()[0])


def test_workspace_clean_after_steps():
    """The fused steps' amax slots and the step-0 barrier are left zero in the workspace, so one
    workspace serves consecutive states and sizes (large: single-pass step 0; small: two kernels)."""
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    for rows, cols, split in ((2048, 4096, False), (13, 29, False), (2048, 4096, True), (13, 29, True)):
        p = Pair(8, 2, 1, O.E4M3, split=split)
        for t in range(5):
            x = small_tensor(rows, cols, seed=100 + t)
            xd = to_device(x)
            q = qf8.quantize_delayed(xd, p.g, ws=ws)
            torch.cuda.synchronize()
            wq, _, _, _ = p.o.step(x)
            assert_bytes_equal(host(q), wq, "q", f" [{rows}x{cols} split={split} t={t}]")
            words = host(ws.view(torch.int32)[:qf8.BARRIER_WORDS])
            assert not words.any(), f"workspace not left zero [{rows}x{cols} split={split} t={t}]"


@pytest.mark.parametrize("interval", [1, 3, 5])
def test_reuse_steps_without_diagnostics(interval):
    """Steps called with no scale_used / amax_out / nonfinite: reuse steps are the cast alone.
    Codes and history still follow the oracle at every step, and the workspace stays clean."""
    rng = np.random.default_rng(40 + interval)
    st = qf8.DelayedState(8, interval, 2, qf8.E4M3)
    orc = O.Delayed(8, interval, 2, O.E4M3)
    ws = qf8.workspace(torch.empty(1, device="cuda"))
    base = (small_tensor(129, 1000, seed=interval).astype(np.uint32) << 16).view(np.float32)
    for t in range(4 * interval + 3):
        x = bf16_bits(base * np.float32(2.0 ** rng.uniform(-8, 8)))
        q = qf8.quantize_delayed(to_device(x), st, ws=ws)
        torch.cuda.synchronize()
        wq, _, _, _ = orc.step(x)
        assert_bytes_equal(host(q), wq, "q", f" [I={interval} t={t}]")
        assert st.history_list() == list(orc.state()[0]), f"history I={interval} t={t}"
    assert not host(ws.view(torch.int32)[:qf8.BARRIER_WORDS]).any()


def test_full_size_without_diagnostics_on_reuse_steps():
    """The drifting workload with diagnostics asked for on update steps only (reuse steps are the
    cast alone): every step's codes on sampled rows, the scale of update steps, the history."""
    z = delayed_base()
    sig = delayed_sigmas()
    zd = torch.from_numpy(z).cuda()
    st = qf8.DelayedState(16, 5, 3, qf8.E4M3)
    orc = O.Delayed(16, 5, 3, O.E4M3)
    s = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = qf8.workspace(zd)
    q = torch.empty(z.shape, dtype=torch.uint8, device="cuda")
    rows = np.random.default_rng(1).choice(z.shape[0], 32, replace=False)
    zmax = float(np.max(np.abs(z)))
    for t in range(21):
        xd = (zd * float(sig[t])).to(torch.bfloat16)
        update = t % 5 == 0
        qf8.quantize_delayed(xd, st, q=q, scale_used=s if update else None, ws=ws)
        torch.cuda.synchronize()
        _, s_o, _, _ = orc.step(bf16_bits(np.array([[np.float32(sig[t]) * np.float32(zmax)]], np.float32)))
        if update:
            assert np.float32(s.item()) == s_o, f"scale t={t}"
        want = O.cast(delayed_step_input(z[rows], sig[t]), O.E4M3, s_o)
        assert_bytes_equal(host(q)[rows], want, "q", f" [sampled rows t={t}]")
    assert st.history_list() == list(orc.state()[0])
