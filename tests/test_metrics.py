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
    r = np.random.default_rng(0).uniform(0.1, 100.0, 20000)
    for dt in ("f16", "bf16"):
        y = W.Tensor.quantise(r, dt).f64()
        m = metrics(y, r, np.abs(r), dt)          # S = |r|: the hardest case
        assert m["g1"] == 0.0 and m["nrmse"] == 0.0
        if dt == "bf16":   # one bf16 rounding alone can exceed the 2e-3 bound
            assert m["g1_raw"] > G1_TOL[dt]


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
