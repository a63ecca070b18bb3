"""Pins of the oracle's exact-d codebook ("O Que E TurboQuant?", Como
Funciona, Estagio 1: after the rotation each coordinate of the unit vector
follows Beta((d-1)/2, (d-1)/2) on [-1, 1], and the Lloyd-Max quantiser is
optimised for that law).  Coordinates are scaled by sqrt(d), so the density
is proportional to (1 - y^2/d)^((d-3)/2) on [-sqrt d, sqrt d].  CPU only."""
from math import exp, lgamma, pi, sqrt

import numpy as np
import pytest

import oracle as O


@pytest.mark.parametrize("d", [16, 128])
def test_total_mass_closed_form(d):
    # int (1 - y^2/d)^((d-3)/2) dy = sqrt(d) B(1/2, (d-1)/2)
    want = sqrt(d) * exp(lgamma(0.5) + lgamma((d - 1) / 2) - lgamma(d / 2))
    assert abs(O.beta_mass(d, -sqrt(d), sqrt(d)) / want - 1) < 1e-12


@pytest.mark.parametrize("d", [16, 128])
def test_one_bit_centroids_are_the_mean_absolute_coordinate(d):
    # E|u_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)) for a uniform unit vector
    want = sqrt(d) * exp(lgamma(d / 2) - lgamma((d + 1) / 2)) / sqrt(pi)
    c, _ = O.lloyd_max_beta(1, d)
    np.testing.assert_allclose(c, [-want, want], rtol=1e-11)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_centroids_are_cell_means_by_brute_force(bits):
    """Each centroid is the conditional mean of its cell, checked with a
    plain trapezoid rule on a 2e6-point grid (independent of the oracle's
    quadrature)."""
    d = 128
    c, _ = O.lloyd_max_beta(bits, d)
    t = np.concatenate([[-sqrt(d)], (c[1:] + c[:-1]) / 2, [sqrt(d)]])
    for j in range(len(c)):
        y = np.linspace(t[j], t[j + 1], 2_000_001)
        g = np.clip(1 - y * y / d, 0, None) ** ((d - 3) / 2)
        assert abs(np.trapezoid(y * g, y) / np.trapezoid(g, y) - c[j]) < 1e-9


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_symmetric_increasing_and_better_than_gaussian_tables(bits):
    c, t = O.tables_f32_beta(bits)
    assert np.all(np.diff(c) > 0) and np.array_equal(c, -c[::-1])
    cg, tg = O.tables_f32(bits)
    # optimal for its own law: lower MSE there than the N(0,1) tables
    assert O.beta_mse(bits, c, t) < O.beta_mse(bits, cg, tg)
    # lighter tails than N(0,1) at the same variance: with two or more levels
    # per side the outer centroid moves inwards (at 1 bit it is E|y|, larger)
    assert (c[-1] < cg[-1]) == (bits >= 2)


def test_large_d_approaches_the_gaussian_tables():
    for bits in (2, 3):
        cb, _ = O.lloyd_max_beta(bits, 1 << 20)
        cg, _ = O.lloyd_max(bits)
        np.testing.assert_allclose(cb, cg, rtol=2e-5)
