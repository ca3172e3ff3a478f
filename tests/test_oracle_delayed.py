"""Oracle delayed-scaling state machine ("HiFloat8：高性能训练之路" section 1.2 and 5.2;
"混合精度与 FP8 训练" sections 8.2 and 8.2.1).

Pins: a hand-computed sequence (history length 3, Interval 2, N_guard 1, E4M3) whose amax
values are powers of two so that every scale is exact; the failure example of section 8.2.1 is
pinned in test_oracle_pins.py. Invariants: S is constant between update steps, the history never
holds more than its capacity, the estimate is the maximum of the retained pushes, a reset makes
the next step current scaling, and a non-finite amax is flagged and never pushed.
"""
import numpy as np

import oracle as O

E4M3 = O.E4M3


def tensor_with_amax(a):
    return np.array([[a, -a / 2, 0.3 * a, -0.01 * a]], np.float32)


def test_hand_computed_sequence():
    d = O.Delayed(hist_len=3, interval=2, n_guard=1, fmt=E4M3)
    amaxes = [4, 8, 2, 16, 1, 32, 64, 0.5, 0.25, 128, 2]
    # step 0: current scaling 448/4 = 112 (no margin), then push 4
    # steps 1..6: estimate 4 -> 448/4 * 2^-1 = 56; pushes at steps 2 (2), 4 (1), 6 (64, drops 4)
    # steps 7..10: estimate 64 -> 448/64 * 2^-1 = 3.5; push at 8 (0.25, drops 2), 10 (2, drops 1);
    # the 128 of step 9 is never pushed (not an update step)
    want_s = [112, 56, 56, 56, 56, 56, 56, 3.5, 3.5, 3.5, 3.5]
    want_h = [[4], [4], [4, 2], [4, 2], [4, 2, 1], [4, 2, 1], [2, 1, 64], [2, 1, 64], [1, 64, 0.25],
              [1, 64, 0.25], [64, 0.25, 2]]
    for t, a in enumerate(amaxes):
        x = tensor_with_amax(a)
        q, s, am, nf = d.step(x)
        assert s == want_s[t], t
        assert am == a and nf == 0
        assert np.array_equal(q, O.cast(x, E4M3, s))
        h, c, st = d.state()
        assert list(h) == want_h[t] and c == len(want_h[t]) and st == t + 1
    assert d.next_scale() == np.float32(448 / 64 / 2)


def test_reset_restarts_with_current_scaling():
    d = O.Delayed(hist_len=4, interval=1, n_guard=3, fmt=E4M3)
    for a in (1.0, 2.0, 4.0):
        d.step(tensor_with_amax(a))
    d.reset()
    h, c, st = d.state()
    assert c == 0 and st == 0
    q, s, am, _ = d.step(tensor_with_amax(7.0))
    assert s == np.float32(448 / 7.0)          # Eq.(1), no 2^-N margin
    assert d.next_scale() == np.float32(np.float32(448 / 7.0) / 8)


def test_nonfinite_is_flagged_and_not_pushed():
    d = O.Delayed(hist_len=4, interval=1, n_guard=0, fmt=E4M3)
    d.step(tensor_with_amax(2.0))
    x = tensor_with_amax(3.0)
    x[0, 2] = np.nan
    q, s, am, nf = d.step(x)
    assert nf == 1 and np.isnan(am)
    h, c, _ = d.state()
    assert list(h) == [2.0]
    x[0, 2] = np.inf
    _, _, am, nf = d.step(x)
    assert nf == 1 and am == np.inf and d.state()[0].tolist() == [2.0]


def test_scale_constant_between_updates_and_capacity():
    rng = np.random.default_rng(1)
    d = O.Delayed(hist_len=5, interval=3, n_guard=2, fmt=E4M3)
    pushed = []
    prev = None
    for t in range(40):
        a = float(np.float32(2.0 ** rng.uniform(-3, 3)))
        q, s, am, _ = d.step(tensor_with_amax(a))
        if t > 0 and (t - 1) % 3 != 0:
            assert s == prev                    # no push since the previous step
        if t % 3 == 0:
            pushed.append(am)
        h, c, _ = d.state()
        assert c == min(len(pushed), 5) and list(h) == pushed[-5:]
        prev = d.next_scale()
        want = np.float32(np.float32(448 / max(pushed[-5:])) * np.float32(0.25))
        assert prev == want
