"""Pins for oracle/uos.py: the UOS objective and its minimiser 7.25.

E(x) at grid points and Delta(q) are checked against closed forms derived by
hand from the definition (every cell of width w contributes w^3/12); the
numeric J sweep must land on the boundary the pages state; Lemma 1's
derivative formula is checked by finite differences; and J is tied to the
block quantiser's scale rule by Monte Carlo over log-uniform block maxima.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import mxfp4, uos

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_E_closed_forms():
    # cells [0,.5],[.5,1],[1,1.5],[1.5,2] (w=.5), [2,3],[3,4] (w=1), [4,6] (w=2): w^3/12 each
    xs = np.array([0.5, 2.0, 3.0, 4.0, 6.0, 7.0, 8.0])
    want = np.array([1 / 96, 4 / 96, 1 / 8, 5 / 24, 7 / 8, 7 / 8 + 1 / 3, 7 / 8 + 8 / 3])
    assert np.allclose(uos.E(xs), want, rtol=0, atol=1e-14)
    for x in (1.3, 3.7, 6.6):
        assert abs(uos.E(x)[0] - uos.E_quad(x)) < 1e-13


def test_delta_closed_form_branches():
    q = np.array([6.0, 6.5, 7.0, 7.2, 7.25, 7.3, 7.5, 8.0])
    first = -1.0 / (8 * q ** 3)                                  # on [6, 7]: negative
    second = (4 * q - 29) * (4 * q - 27) / (8 * q ** 3)          # on [7, 8]
    want = np.where(q <= 7.0, first, second)
    assert np.allclose(uos.delta(q), want, rtol=0, atol=1e-13)
    g = GOLD["delta_second_branch_factor"]["value"]
    lo, hi = g["interval"]
    assert not (lo <= g["root_outside_interval"] <= hi)
    qs = np.linspace(6.0, 8.0, 2001)
    d = uos.delta(qs)
    assert (d[qs < 7.25 - 1e-9] < 0).all() and (d[qs > 7.25 + 1e-9] > 0).all()
    b = GOLD["uos_boundary"]["value"]
    assert abs(uos.delta(b["numerator"] / b["denominator"])[0]) < 1e-15


@pytest.mark.parametrize("name", list(uos.DENSITIES))
def test_J_minimum_is_7_25_for_every_density(name):
    h = uos.DENSITIES[name]
    qs = np.round(np.arange(6.0, 8.0 + 1e-9, 0.005), 3)
    Js = np.array([uos.J(q, h) for q in qs])
    assert qs[np.argmin(Js)] == GOLD["j_minimum_all_densities"]["value"]


def test_J_matches_adaptive_quadrature():
    for q in (6.3, 7.25, 7.9):
        assert abs(uos.J(q) - uos.J_quad(q)) < 1e-12


def test_lemma1_derivative_sign():
    for name, h in uos.DENSITIES.items():
        for q in (6.2, 6.9, 7.1, 7.4, 7.8):
            eps = 1e-4
            num = (uos.J(q + eps, h) - uos.J(q - eps, h)) / (2 * eps)
            formula = float(h(math.log2(q))) * uos.delta(q)[0] / (q * math.log(2))
            assert abs(num - formula) < 1e-7 * max(1.0, abs(formula)) + 1e-9, (name, q)


def test_J_is_mean_D_of_normalised_max_under_the_scale_rule():
    # log-uniform block maxima, scaled by the oracle's own ceiling rule: the mean of D(X_q)
    # must equal J(q) with h = 1 (Monte Carlo, 400k samples)
    rng = np.random.default_rng(21)
    M = np.exp2(rng.uniform(-10, 10, 400_000))
    for q in (6.0, 7.25):
        e = mxfp4.scale_exponent(M, mxfp4.rule_ceil(q))
        X = np.ldexp(M, -e)
        Dx = uos.D(X)
        mc, se = Dx.mean(), Dx.std() / math.sqrt(len(Dx))
        assert abs(mc - uos.J(q)) < 5 * se
