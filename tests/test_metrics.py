"""The parity gates themselves (CPU): a correctly rounded result passes, an
error of one extra unit in the accumulation fails."""
import numpy as np

import workloads as W
from convcheck import G1_TOL, half_ulp, metrics


def test_half_ulp_values():
    assert half_ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -8
    assert half_ulp(np.array([1.0]), "f16")[0] == 2.0 ** -11
    assert half_ulp(np.array([3.0]), "bf16")[0] == 2.0 ** -7
    assert half_ulp(np.array([1e-9]), "f16")[0] == 2.0 ** -25     # subnormal range


def test_correctly_rounded_results_pass_even_when_S_equals_y():
    """S = |r|, the hardest case.  f16: G1 is the gate as written, and one
    rounding (at most 2^-11 of |y|) stays below 2e-3.  bf16: one rounding
    alone can exceed 2e-3, so G1 counts only the error beyond it."""
    r = np.random.default_rng(0).uniform(0.1, 100.0, 20000)
    for dt in ("f16", "bf16"):
        y = W.Tensor.quantise(r, dt).f64()
        m = metrics(y, r, np.abs(r), dt)
        assert m["nrmse"] == 0.0
        if dt == "f16":
            assert m["g1"] == m["g1_raw"] <= 2.0 ** -11 < G1_TOL[dt]
        else:
            assert m["g1"] == 0.0 and m["g1_raw"] > G1_TOL[dt]


def test_accumulation_error_is_caught():
    r = np.random.default_rng(1).uniform(0.5, 1.0, 1000)
    s = np.abs(r) * 10
    for dt in ("f16", "bf16"):
        y = W.Tensor.quantise(r * (1 + 0.05), dt).f64()  # a 5 % error before rounding
        m = metrics(y, r, s, dt)
        assert m["g1"] > G1_TOL[dt]


def test_f32_gate_is_plain_relative_error():
    r = np.linspace(-1, 1, 101)
    y = r + 2e-6
    m = metrics(y, r, np.full_like(r, 0.1), "f32")
    assert abs(m["g1"] - 2e-6 / (0.1 + 1e-6)) < 1e-12
