"""CPU pins of the delayed-scaling estimator rules ("HiFloat8：高性能训练之路" section 1.2: the
amax estimate is the maximum of the history buffer, or another rule such as the most recent
entry or the mean).

  * a hand-computed sequence (history 3, Interval 1, no margin) under all three rules: the
    scale each step uses is F8max over the rule's value of the history before the step;
  * the mean's summation order is fixed (oldest to newest, fp32): with entries 2^24, 1, 1 that
    order gives 2^24 (each +1 is a tie that rounds back), newest-first would give 2^24 + 2;
  * most recent after the FIFO wrapped, and with Interval > 1 (only update steps append);
  * long histories (64 and 1024 entries, more steps than entries): max and mean against plain
    numpy over the last entries.
"""
import numpy as np
import pytest

import oracle as O

E4M3 = O.E4M3


def tensor_with_amax(a):
    return np.array([[a, -a / 2, 0.0]], np.float32)


@pytest.mark.parametrize("est", [O.EST_MAX, O.EST_RECENT, O.EST_MEAN])
def test_hand_sequence(est):
    amaxes = [4.0, 8.0, 2.0, 16.0, 1.0, 32.0]
    d = O.Delayed(3, 1, 0, E4M3, estimator=est)
    hist = []
    for t, a in enumerate(amaxes):
        _, s, got_a, _ = d.step(tensor_with_amax(a))
        assert got_a == a
        if t == 0:
            want = np.float32(448.0 / a)                           # step 0: current scaling
        else:
            h = np.array(hist, np.float32)
            if est == O.EST_MAX:
                e = h.max()
            elif est == O.EST_RECENT:
                e = h[-1]
            else:
                acc = np.float32(0.0)
                for v in h:
                    acc = np.float32(acc + v)
                e = np.float32(acc / np.float32(len(h)))
            want = np.float32(448.0 / np.float64(e))
        assert s == want, (est, t)
        hist = (hist + [a])[-3:]
    assert list(d.state()[0]) == hist


def test_mean_sums_oldest_to_newest_in_fp32():
    d = O.Delayed(3, 1, 0, E4M3, estimator=O.EST_MEAN)
    for a in (16777216.0, 1.0, 1.0):
        d.step(tensor_with_amax(a))
    assert d.estimate() == np.float32(16777216.0 / 3)            # 2^24 + 1 + 1 stays 2^24 in fp32
    assert d.estimate() != np.float32(16777218.0 / 3)            # the newest-first order


def test_recent_after_wrap_and_interval():
    d = O.Delayed(2, 1, 0, E4M3, estimator=O.EST_RECENT)
    for a in (4.0, 8.0, 2.0):
        d.step(tensor_with_amax(a))
    assert d.estimate() == 2.0 and list(d.state()[0]) == [8.0, 2.0]
    d = O.Delayed(4, 3, 0, E4M3, estimator=O.EST_RECENT)
    for a in (4.0, 8.0, 2.0, 16.0, 1.0):                         # appends at steps 0 and 3
        d.step(tensor_with_amax(a))
    assert list(d.state()[0]) == [4.0, 16.0] and d.estimate() == 16.0


@pytest.mark.parametrize("hist_len", [64, 1024])
def test_long_history(hist_len):
    rng = np.random.default_rng(hist_len)
    a = (2.0 ** rng.uniform(-10, 10, hist_len + 300)).astype(np.float32)
    dm = O.Delayed(hist_len, 1, 0, E4M3, estimator=O.EST_MAX)
    da = O.Delayed(hist_len, 1, 0, E4M3, estimator=O.EST_MEAN)
    for v in a:
        dm.step(tensor_with_amax(v))
        da.step(tensor_with_amax(v))
    last = a[-hist_len:]
    assert dm.estimate() == last.max()
    acc = np.float32(0.0)
    for v in last:
        acc = np.float32(acc + v)
    assert da.estimate() == np.float32(acc / np.float32(hist_len))
