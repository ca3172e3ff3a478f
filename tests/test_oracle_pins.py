"""Oracle per-tensor scaling and the delayed-scaling failure pinned to the pages' worked examples.

  * tests/golden/w4_scaling_example.json: "混合精度与 FP8 训练" section 8.1 (amax 0.02, value 0.001);
  * tests/golden/w5_delayed_failure.json: same page, section 8.2.1 (history 20, spike 50);
  * tests/golden/w6_mx_example.json: same page, section 13.1 (MX block with amax 5.3).
"""
import json
import os

import numpy as np
import pytest

import oracle as O

E4M3 = O.E4M3


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_scaling_example(golden_dir):
    g = load(golden_dir, "w4_scaling_example.json")
    # unscaled: 0.001 is about half the subnormal spacing 2^-9 and rounds up to it
    q0 = O.encode(E4M3, g["value"])
    assert O.decode(E4M3, q0) == g["unscaled_e4m3_value"]
    assert round(abs(O.decode(E4M3, q0) - g["value"]) / g["value"] * 100) == g["unscaled_relative_error_pct"]
    # per-tensor current scaling of the fp32 tensor [amax, value]
    x = np.array([g["amax"], g["value"]], np.float32)
    q, amax, s, nf = O.quantize_per_tensor(x, E4M3)
    assert nf == 0
    assert amax == np.float32(g["amax"])
    assert s == g["scale"]                                   # fl32(448 / fl32(0.02)) is exactly 22400
    assert abs(float(np.float32(g["value"]) * s) - g["scaled_value"]) < 1e-5
    assert O.decode(E4M3, q[1]) == g["scaled_e4m3_value"]     # spacing 2 in [16, 32)
    assert q[0] == 0x7E                                       # amax maps onto 448
    deq = O.decode(E4M3, q[1]) / s
    assert round(deq, 6) == g["dequantized"]
    assert round(abs(deq - g["value"]) / g["value"] * 100, 1) == g["dequantized_relative_error_pct"]


def test_delayed_failure_example(golden_dir):
    g = load(golden_dir, "w5_delayed_failure.json")
    # Two iterations of delayed scaling with no margin (the page's TE form, margin 0), Interval 1.
    d = O.Delayed(hist_len=16, interval=1, n_guard=0, fmt=E4M3)
    x0 = np.array([g["history_amax"], 1.0, -3.0], np.float32)
    q0, s0, a0, _ = d.step(x0)                      # step 0: current scaling, pushes amax 20
    assert a0 == g["history_amax"]
    s1 = d.next_scale()
    assert abs(s1 - g["scale"]) < 1e-5 and s1 == np.float32(448 / 20)
    x1 = np.array([g["spike"], 1.0], np.float32)
    q1, su, a1, _ = d.step(x1)                      # step 1: reuses S = 22.4, then pushes 50
    assert su == s1
    assert abs(float(np.float32(g["spike"]) * su) - g["scaled_spike"]) < 1e-3
    assert O.decode(E4M3, q1[0]) == g["saturated"]   # saturates instead of overflowing
    assert round(O.decode(E4M3, q1[0]) / su, 4) == g["dequantized"]
    s2 = d.next_scale()
    assert abs(s2 - g["next_scale"]) < 1e-6 and s2 == np.float32(448 / 50)
    hist, count, step = d.state()
    assert list(hist) == [20.0, 50.0] and count == 2 and step == 2


def test_mx_example(golden_dir):
    g = load(golden_dir, "w6_mx_example.json")
    assert O.emax(E4M3) == g["emax_e4m3"]
    for rnd in (O.ROUND_DOWN, O.ROUND_UP):
        X = O.mx_exponent(E4M3, rnd, g["amax"])
        assert X == g["shared_exponent"] == g["floor_log2_amax"] - g["emax_e4m3"]
        assert 2.0 ** -X == g["multiplier"]
    assert round(g["amax"] * g["multiplier"]) == g["scaled_amax"] <= g["e4m3_max"]
    # a block of 32 whose amax is (the BF16 of) 5.3: byte 121, no element saturates
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = g["amax"]
    x[0, 9] = -1.0
    q, s, _, _, nf = O.quantize_mx(x, E4M3, O.ROUND_UP, col=False)
    assert nf == 0 and s[0, 0] == 127 + g["shared_exponent"] == 121
    assert O.decode(E4M3, q[0, 5]) < g["e4m3_max"]
    assert O.decode(E4M3, q[0, 9]) == -64.0
