"""Pins of the oracle's Gaussian Lloyd-Max tables (CPU only).

Lloyd-Max centroids for N(0,1) (PolarQuant page, Technical summary sec. 2;
TurboQuant page, Como Funciona, Estagio 1; codebooks precomputed per bit
width: TurboQuant page, Como Implementar)."""
import json
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_constants.json")))


def test_one_bit_closed_form():
    c, _ = O.lloyd_max(1)
    assert abs(c[1] - np.sqrt(2 / np.pi)) < 1e-12 and abs(c[0] + np.sqrt(2 / np.pi)) < 1e-12
    assert abs(O.gauss_mse(1, c, [0.0]) - (1 - 2 / np.pi)) < 1e-12
    assert abs(c[1] - GOLD["lloyd_max_b1_centroid"]["value"]) < 5e-5


def test_two_bit_printed():
    c, _ = O.lloyd_max(2)
    want = GOLD["lloyd_max_b2_centroids"]["value"]
    tol = GOLD["lloyd_max_b2_centroids"]["abs_tol"]
    assert abs(c[2] - want[0]) < tol[0] and abs(c[3] - want[1]) < tol[1]
    assert abs(c[1] + want[0]) < tol[0] and abs(c[0] + want[1]) < tol[1]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_printed_and_by_quadrature(bits):
    c, _ = O.lloyd_max(bits)
    t = (c[1:] + c[:-1]) / 2
    mse = O.gauss_mse(bits, c, t)
    want = GOLD["lloyd_max_mse"]["value"][str(bits)]
    assert abs(mse - want) / want < GOLD["lloyd_max_mse"]["rel_tol"]
    # the closed-form cell integral against numerical quadrature
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    q = sum(integrate.quad(lambda x, cj=cj: (x - cj) ** 2 * stats.norm.pdf(x), a, b,
                           epsabs=1e-14, epsrel=1e-12)[0]
            for a, b, cj in zip(edges[:-1], edges[1:], c))
    assert abs(q - mse) < 1e-10


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_centroid_condition_by_quadrature(bits):
    """Each centroid is the conditional mean of its cell (checked numerically)."""
    c, _ = O.lloyd_max(bits)
    t = (c[1:] + c[:-1]) / 2
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for a, b, cj in zip(edges[:-1], edges[1:], c):
        m1 = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b, epsabs=1e-15, epsrel=1e-13)[0]
        m0 = integrate.quad(stats.norm.pdf, a, b, epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(m1 / m0 - cj) < 1e-9
    assert np.allclose(c, -c[::-1], atol=1e-13)


@pytest.mark.parametrize("bits", [3, 4])
def test_textbook_levels(bits):
    c, _ = O.lloyd_max(bits)
    want = GOLD["max1960_levels"]["value"][str(bits)]
    assert np.max(np.abs(c[len(c) // 2:] - want)) < GOLD["max1960_levels"]["abs_tol"]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_unique_fixed_point(bits):
    """The N(0,1) density is log-concave, so Lloyd's fixed point is unique."""
    L = 1 << bits
    ref, _ = O.lloyd_max(bits, tol=1e-16, max_iter=20000)
    rng = np.random.default_rng(bits)
    for init in (np.linspace(-1, 1, L), np.sort(rng.standard_normal(L) * 3), np.linspace(-4, 0.5, L)):
        c, _ = O.lloyd_max(bits, init=init, tol=1e-16, max_iter=20000)
        assert np.max(np.abs(c - ref)) < 1e-12


def test_mse_on_gaussian_samples():
    """10^7 N(0,1) samples (numpy seed 0) through the fp32 tables."""
    y = np.random.default_rng(0).standard_normal(10_000_000)
    for bits in (1, 2, 3, 4):
        _, yh = O.scalar_quantize(y, bits)
        mse = np.mean((y - yh) ** 2)
        want = GOLD["lloyd_max_mse"]["value"][str(bits)]
        assert abs(mse - want) / want < GOLD["lloyd_max_mse"]["rel_tol"], (bits, mse)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_fp32_tables_and_bucket_rule(bits):
    c32, t32 = O.tables_f32(bits)
    c, _ = O.lloyd_max(bits)
    assert np.array_equal(c32, c.astype(np.float32))
    assert np.array_equal(t32, ((c32[1:].astype(np.float64) + c32[:-1]) / 2).astype(np.float32))
    # symmetric tables: mirrored entries are exact negatives; middle threshold is 0
    assert np.array_equal(c32, -c32[::-1]) and t32[len(t32) // 2] == 0.0
    # counting thresholds == nearest centroid (independent formulation), away from ties
    y = np.random.default_rng(5).standard_normal(200_000) * 1.5
    idx, _ = O.scalar_quantize(y, bits)
    nn = np.argmin(np.abs(y[:, None] - c32[None, :].astype(np.float64)), axis=1)
    far = np.min(np.abs(y[:, None] - t32[None, :]), axis=1) > 1e-6
    assert np.array_equal(idx[far], nn[far])
    # exact tie goes to the lower cell
    ti, _ = O.scalar_quantize(t32.astype(np.float64), bits)
    assert np.array_equal(ti, np.arange(len(t32)))
