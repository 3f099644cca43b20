"""Pins of the output head (oracle/layer.py: softcap, lm_head_softcap): closed
forms of cap * tanh(z / cap) and a brute-force logit loop that fixes the
orientation of the head weight ([V][D] rows)."""
import math

import numpy as np

from oracle import layer as L


def test_softcap_closed_forms():
    cap = 30.0
    assert L.softcap(0.0, cap) == 0.0
    # tanh(atanh(1/2)) = 1/2: the cap halves at z = cap * atanh(1/2) = 15 ln 3
    assert abs(L.softcap(15.0 * math.log(3.0), cap) - 15.0) < 1e-12
    # odd, monotone, bounded by the cap and saturating towards it
    z = np.linspace(-400, 400, 8001)
    y = L.softcap(z, cap)
    np.testing.assert_array_equal(y, -L.softcap(-z, cap))
    assert np.all(np.diff(y) > 0) and np.all(np.abs(y) < cap)
    assert cap - L.softcap(400.0, cap) < 1e-9
    # near zero: z - z^3 / (3 cap^2) + 2 z^5 / (15 cap^4), remainder below the
    # next term of the alternating series, 17 z^7 / (315 cap^6)
    for v in (1e-3, 0.1, 1.0, 2.0):
        series = v - v ** 3 / (3 * cap ** 2) + 2 * v ** 5 / (15 * cap ** 4)
        assert abs(L.softcap(v, cap) - series) <= 17 / 315 * v ** 7 / cap ** 6 + 1e-15
    # cap 0: no cap
    np.testing.assert_array_equal(L.softcap(z, 0.0), z)


def test_lm_head_brute_force():
    g = np.random.default_rng(0)
    x = g.standard_normal((3, 7))
    w = g.standard_normal((11, 7))             # [V][D]
    got = L.lm_head_softcap(x, w, 2.5)
    for t in range(3):
        for v in range(11):
            z = sum(x[t, d] * w[v, d] for d in range(7))
            assert abs(got[t, v] - 2.5 * math.tanh(z / 2.5)) < 1e-12
    np.testing.assert_allclose(L.lm_head_softcap(x, w, 0.0), x @ w.T, rtol=0, atol=1e-13)
