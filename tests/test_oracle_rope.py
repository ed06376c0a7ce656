"""Pins of the oracle's RoPE (MAC-Attention blog, "Match (1)": a product of
independent 2x2 rotations of pairs (x[2j], x[2j+1])), against facts that do
not depend on how it is written: position 0 is the identity, each pair keeps
its length, dot products depend only on the position difference, a single
pair rotates by exactly pos * base^(-2j/d), and rotations compose."""
import math

import numpy as np
import pytest


@pytest.mark.parametrize("d", [8, 64, 128])
def test_rope_invariants(oracle_lib, d):
    rng = np.random.default_rng(d)
    x, y = rng.standard_normal(d), rng.standard_normal(d)
    base = 5e5
    assert np.array_equal(oracle_lib.rope(x, 0, base), x)
    for pos in (1, 77, 4096, 262143):
        rx = oracle_lib.rope(x, pos, base)
        # each pair keeps its length
        np.testing.assert_allclose(np.hypot(rx[0::2], rx[1::2]), np.hypot(x[0::2], x[1::2]),
                                   rtol=1e-13)
        # relative position: <R(m) x, R(n) y> = <R(m - n) x, y>
        for n in (0, 5, pos // 2):
            lhs = float(rx @ oracle_lib.rope(y, n, base))
            rhs = float(oracle_lib.rope(x, pos - n, base) @ y)
            assert abs(lhs - rhs) < 1e-10 * (1 + abs(lhs))


def test_rope_single_pair_angle(oracle_lib):
    """d = 8, unit vector in pair j: the pair turns by pos * base^(-2j/d)."""
    d, base = 8, 10000.0
    for j in range(d // 2):
        x = np.zeros(d)
        x[2 * j] = 1.0
        for pos in (1, 3, 1000):
            y = oracle_lib.rope(x, pos, base)
            ang = pos * base ** (-2.0 * j / d)
            assert abs(y[2 * j] - math.cos(ang)) < 1e-12
            assert abs(y[2 * j + 1] - math.sin(ang)) < 1e-12
            others = np.delete(y, [2 * j, 2 * j + 1])
            assert not others.any()


def test_rope_composes(oracle_lib):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(64)
    a = oracle_lib.rope(oracle_lib.rope(x, 300, 5e5), 45, 5e5)
    np.testing.assert_allclose(a, oracle_lib.rope(x, 345, 5e5), atol=1e-12)
