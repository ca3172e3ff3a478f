"""CPU pins of the split amax of delayed scaling ("HiFloat8：高性能训练之路", the section comparing
HiF8 with FP8 and MXFP8: with a larger margin the amax can be updated every Interval steps and
its computation spread over those steps by cutting the tensor into equal sub-tensors, one per
step).

Reading: step t >= 1 measures piece (t - 1) mod I of the flattened tensor, piece k being
[floor(k n / I), floor((k+1) n / I)); the window's maximum is appended on the update step
t % I == 0; a window with an Inf/NaN piece appends nothing; amax_out and nonfinite still cover
the whole tensor.

  * a sequence worked by hand (4 elements, I = 2) in which split and whole-tensor updates append
    different values;
  * Inf/NaN inside the measured piece (window dropped) and outside it (flag only);
  * I = 1 reduces to whole-tensor updates; an input that repeats every step gives the
    whole-tensor history for any I (the maximum over the pieces is the whole amax);
  * the pieces of one window partition [0, n) into near-equal consecutive ranges, also when
    n < I (empty pieces).
"""
import numpy as np
import pytest

import oracle as O

E4M3 = O.E4M3


def row(*v):
    return np.array([v], np.float32)


def test_hand_sequence():
    d = O.Delayed(4, 2, 0, E4M3, split=True)
    steps = [
        # x,                         scale used,  amax_out, history after the step
        (row(1, 2, 3, 4),            448 / 4,     4,        [4]),        # current scaling, push 4
        (row(8, 1, 100, 1),          448 / 4,     100,      [4]),        # piece [0,2): 8
        (row(100, 1, 2, 16),         448 / 4,     100,      [4, 16]),    # piece [2,4): 16 -> push 16
        (row(1, 1, 1, 1),            448 / 16,    1,        [4, 16]),    # piece [0,2): 1
        (row(0.5, 0.5, 0.5, 2),      448 / 16,    2,        [4, 16, 2]), # piece [2,4): 2 -> push 2
        (row(3, 0, 0, 0),            448 / 16,    3,        [4, 16, 2]),
    ]
    for t, (x, s_want, a_want, h_want) in enumerate(steps):
        _, s, a, nf = d.step(x)
        assert s == np.float32(s_want), t
        assert a == np.float32(a_want) and nf == 0, t
        h, _, _ = d.state()
        assert list(h) == h_want, t
    # whole-tensor updates append the full amax of steps 2 and 4 instead
    w = O.Delayed(4, 2, 0, E4M3)
    for x, *_ in steps[:5]:
        w.step(x)
    assert list(w.state()[0]) == [4, 100, 2]


def test_nonfinite_inside_and_outside_the_piece():
    d = O.Delayed(4, 2, 0, E4M3, split=True)
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    d.step(row(1, 2, 3, 4))                                        # history [4]
    _, _, a, nf = d.step(row(nan, 1, 1, 1))                        # NaN inside piece [0,2)
    assert nf == 1 and np.isnan(a)
    _, _, _, nf = d.step(row(1, 1, 5, 6))                          # window ends: dropped
    assert nf == 0 and list(d.state()[0]) == [4]
    _, _, a, nf = d.step(row(2, 3, inf, 1))                        # Inf outside piece [0,2)
    assert nf == 1 and np.isinf(a)
    d.step(row(50, 50, 7, 1))                                      # piece [2,4): 7 -> push max(3, 7)
    assert list(d.state()[0]) == [4, 7]


@pytest.mark.parametrize("est", [O.EST_MAX, O.EST_RECENT, O.EST_MEAN])
def test_interval_one_is_whole_tensor(est):
    rng = np.random.default_rng(5 + est)
    a = O.Delayed(8, 1, 2, O.E5M2, estimator=est, split=True)
    b = O.Delayed(8, 1, 2, O.E5M2, estimator=est)
    for t in range(20):
        x = (rng.standard_normal((5, 7)) * 2.0 ** rng.uniform(-8, 8)).astype(np.float32)
        qa, sa, aa, na = a.step(x)
        qb, sb, ab, nb = b.step(x)
        assert sa == sb and aa == ab and na == nb and np.array_equal(qa, qb), t
        assert np.array_equal(a.state()[0], b.state()[0])


@pytest.mark.parametrize("interval,shape", [(3, (5, 7)), (4, (1, 3)), (5, (2, 64)), (7, (3, 3))])
def test_repeated_input_gives_whole_history(interval, shape):
    rng = np.random.default_rng(interval)
    a = O.Delayed(6, interval, 1, E4M3, split=True)
    b = O.Delayed(6, interval, 1, E4M3)
    for t in range(4 * interval + 2):
        if t % interval == 1 or interval == 1 or t == 0:
            x = (rng.standard_normal(shape) * 2.0 ** rng.uniform(-4, 4)).astype(np.float32)
        # x is held for the whole window t = mI+1 .. (m+1)I, so every piece sees the same tensor
        qa, sa, _, _ = a.step(x)
        qb, sb, _, _ = b.step(x)
        assert sa == sb and np.array_equal(qa, qb), t
    assert np.array_equal(a.state()[0], b.state()[0])


@pytest.mark.parametrize("n,interval", [(4, 2), (10, 3), (3, 4), (0, 3), (1, 1), (1000003, 7), (2 ** 33 + 5, 9)])
def test_pieces_partition(n, interval):
    for start in (1, 1 + 5 * interval):                             # any window
        pieces = [O.delayed_piece(t, interval, n) for t in range(start, start + interval)]
        assert pieces[0][0] == 0 and pieces[-1][1] == n
        for (lo0, hi0), (lo1, hi1) in zip(pieces, pieces[1:]):
            assert hi0 == lo1
        sizes = [hi - lo for lo, hi in pieces]
        assert max(sizes) - min(sizes) <= 1 and min(sizes) == n // interval
