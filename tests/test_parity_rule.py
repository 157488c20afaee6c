"""The comparison rule itself: tolerance formula and NaN handling."""
import numpy as np

import oracle


def test_bf16_ulp_values():
    assert oracle.ulp_bf16(1.0) == 2.0 ** -7
    assert oracle.ulp_bf16(1.5) == 2.0 ** -7
    assert oracle.ulp_bf16(-3.0) == 2.0 ** -6
    assert oracle.ulp_bf16(0.0) == 2.0 ** -133
    assert oracle.ulp_bf16(2.0 ** -130) == 2.0 ** -133     # subnormal range: fixed spacing


def test_tolerance_bar():
    D = np.array([100.0, -2.0, 0.0])
    S = np.array([1000.0, 50.0, 10.0])
    assert np.allclose(oracle.tolerance(D, S, "f32"), [1e-2, 5e-4, 1e-4])
    assert np.allclose(oracle.tolerance(D, S, "bf16"), [1e-2 + 0.5, 5e-4 + 2 ** -6, 1e-4 + 2 ** -133])


def test_ratio_pass_fail_and_nan():
    D = np.array([[1.0, np.nan], [3.0, 4.0]])
    S = np.array([[10.0, np.nan], [10.0, 10.0]])
    g = D.copy()
    assert oracle.parity_ratio(np.where(np.isnan(g), np.nan, g), D, S, "f32") == 0.0
    g2 = g.copy()
    g2[0, 0] += 1e-4
    assert abs(oracle.parity_ratio(g2, D, S, "f32") - 1.0) < 1e-9
    g3 = g.copy()
    g3[1, 1] += 2e-4
    assert oracle.parity_ratio(g3, D, S, "f32") > 1.0
    g4 = g.copy()
    g4[0, 1] = 0.0               # finite where NaN is required
    assert oracle.parity_ratio(g4, D, S, "f32") == float("inf")
    g5 = g.copy()
    g5[1, 0] = np.nan            # NaN where a finite value is required
    assert oracle.parity_ratio(g5, D, S, "f32") == float("inf")


def test_ratio_rejects_invalid_tolerance():
    D = np.array([1.0, 2.0])
    for S in (np.array([10.0, -1.0]), np.array([10.0, np.nan]), np.array([np.inf, 1.0])):
        for out in ("f32", "bf16"):
            try:
                oracle.parity_ratio(D, D, S, out)
            except ValueError:
                continue
            raise AssertionError(f"accepted S = {S} for {out}")
    for rel in (0.0, -1e-5, np.nan, np.inf):
        try:
            oracle.parity_ratio(D, D, np.array([1.0, 1.0]), "f32", rel=rel)
        except ValueError:
            continue
        raise AssertionError(f"accepted rel = {rel}")


def test_zero_tolerance_needs_exact_match():
    D = np.array([0.0, 3.0])
    S = np.array([0.0, 10.0])
    assert oracle.parity_ratio(np.array([0.0, 3.0]), D, S, "f32") == 0.0
    assert oracle.parity_ratio(np.array([-0.0, 3.0]), D, S, "f32") == 0.0
    assert oracle.parity_ratio(np.array([1e-30, 3.0]), D, S, "f32") == float("inf")
    # bf16 output always has the ulp term, so S = 0 still has a positive bar
    assert oracle.parity_ratio(np.array([2.0 ** -134, 3.0]), D, S, "bf16") <= 1.0
