"""Pins of the oracle's decision-band flags (CPU only).

Every code-parity test accepts a GPU difference only where the oracle flags
the decision as within 1e-5 of a boundary, so the flags themselves are pinned
here with inputs built at a known distance from a boundary:

  - scalar codes (PolarQuant page, sec. 2; TurboQuant page, Estagio 1): a
    rotated coordinate within 1e-5 of a threshold;
  - QJL signs (TurboQuant page, Estagio 2): a projection (S r)_j within
    1e-5 * gamma of zero;
  - NSN vector codes (NSNQuant page, Metodologia sec. 3, nearest codebook
    entry): a sub-vector within 1e-5 of the bisecting hyperplane of its
    nearest entry and another.

Each case puts points at 0.5e-5 (flagged) and 2e-5 (not flagged) from a
boundary, plus one exact tie, and checks both the flag and the code.  A
statistical test bounds the flagged fraction on random vectors, and the
exact-d MSE integral is pinned against an independent quadrature and a
Monte-Carlo estimate."""
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle as O
from tests.test_oracle_hadamard import sylvester

H128 = sylvester(128).astype(np.float64)
BAND = O.BAND
GOLDEN_CB = os.path.join(os.path.dirname(__file__), "golden", "vq_codebook_256x8.txt")


def x_for_rotated(y, signs):
    """An input vector whose rotated unit vector is y (||y||^2 = d):
    y = H (D .* x / ||x||) with x = D .* H y / d, since H H = d I."""
    x = signs * (H128 @ y) / 128.0
    np.testing.assert_allclose(np.linalg.norm(x), 1.0, rtol=1e-14)
    return x


def complete_norm(y, free):
    """Set coordinate `free` so that ||y||^2 = d (it must stay far from every
    threshold; the caller checks)."""
    rest = np.sum(np.delete(y, free) ** 2)
    y[free] = np.sqrt(128.0 - rest)
    return y


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_quantize_flags_at_known_distances(bits):
    c, t = O.tables_f32(bits)
    t = t.astype(np.float64)
    rng = np.random.default_rng(bits)
    signs = np.where(rng.integers(0, 2, 128) == 1, 1, -1).astype(np.int8)
    y = np.zeros(128)
    # far from every threshold: the centroids themselves (margin >= half a gap)
    y[:] = c[rng.integers(0, len(c), 128)].astype(np.float64) * 0.5
    offsets = [+0.5e-5, -0.5e-5, +2e-5, -2e-5, 0.0]
    want_flag = [1, 1, 0, 0, 1]
    j = len(t) // 2  # a threshold near the middle (0 for odd counts)
    for k, off in enumerate(offsets):
        y[k] = t[j] + off
    y = complete_norm(y, 127)
    dist = np.min(np.abs(y[5:, None] - t[None, :]), axis=1)
    assert dist.min() > 1e-3  # the other coordinates are far from every threshold
    r = O.quantize(x_for_rotated(y, signs)[None, None, None], signs[None], bits, want_y=True)
    np.testing.assert_allclose(r["y"][0, 0, 0], y, atol=1e-13)
    fl = r["flags"][0, 0, 0]
    assert list(fl[:5]) == want_flag
    assert not fl[5:].any()
    idx = r["idx"][0, 0, 0]
    # above the threshold: cell j + 1; below or exactly on it: cell j
    assert list(idx[:4]) == [j + 1, j, j + 1, j]
    assert idx[4] in (j, j + 1)  # rounding of the construction decides an exact tie
    assert np.array_equal(idx[5:], np.searchsorted(t, y[5:], side="left"))


def test_quantize_flagged_fraction_matches_the_band_mass():
    """On random Gaussian vectors the rotated coordinates follow the law of
    sqrt(d) u_1 for a uniform unit vector u; the flagged fraction must match
    sum_j P(|y - t_j| < band) = sum_j 2 band g(t_j) to Poisson accuracy."""
    bits, n = 3, 40_000
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 1, n, 128))
    signs = np.where(rng.integers(0, 2, (1, 128)) == 1, 1, -1).astype(np.int8)
    r = O.quantize(x, signs, bits)
    _, t = O.tables_f32(bits)
    d = 128
    # density of y = sqrt(d) u_1: (u_1 + 1)/2 ~ Beta((d-1)/2, (d-1)/2)
    g = stats.beta.pdf((t / np.sqrt(d) + 1) / 2, (d - 1) / 2, (d - 1) / 2) / (2 * np.sqrt(d))
    expect = 2 * BAND * g.sum() * n * d
    got = int(r["flags"].sum())
    assert abs(got - expect) < 5 * np.sqrt(expect) + 1, (got, expect)
    assert 50 < expect < 400


def test_qjl_flags_at_known_distances():
    """S a signed permutation, so z = S r is known exactly."""
    d = m = 128
    bits = 2
    c, _ = O.tables_f32(bits)
    rng = np.random.default_rng(7)
    perm = rng.permutation(m)
    sg = np.where(rng.integers(0, 2, m) == 1, 1.0, -1.0)
    S = np.zeros((m, d))
    S[np.arange(m), perm] = sg
    idx = rng.integers(0, 4, d).astype(np.int32)
    r = np.where(rng.integers(0, 2, d) == 1, 1.0, -1.0) * rng.uniform(1e-3, 2e-2, d)
    # z_j = sg_j r_perm(j): put chosen multiples of gamma at z_0 .. z_4
    frac = np.array([0.5e-5, -0.5e-5, 2e-5, -2e-5, 0.0])
    small = perm[:5]
    others = np.setdiff1d(np.arange(d), small)
    gamma = np.sqrt(np.sum(r[others] ** 2) / (1 - np.sum(frac ** 2)))
    r[small] = sg[:5] * frac * gamma
    y = c[idx].astype(np.float64) + np.sqrt(d) * r
    q = O.qjl(y[None], idx[None], S, bits)
    np.testing.assert_allclose(q["gamma"][0], np.linalg.norm(r), rtol=1e-13)
    np.testing.assert_allclose(q["gamma"][0], gamma, rtol=1e-12)
    fl = q["flags"][0]
    assert list(fl[:5]) == [1, 1, 0, 0, 1]
    assert not fl[5:].any()
    bits_out = np.unpackbits(q["signs"][0], bitorder="little")
    z = sg * r[perm]
    assert list(bits_out[:4]) == [1, 0, 1, 0]
    assert bits_out[4] == 1  # sign(0) = +1
    assert np.array_equal(bits_out[5:], (z[5:] >= 0).astype(np.uint8))


def codebook():
    return np.loadtxt(GOLDEN_CB, dtype=np.float32).reshape(256, 8).astype(np.float64)


def test_nsn_flags_at_known_distances():
    """With the mean given as zero, x = H z / d encodes to z exactly (NSN's
    normalisations are then the identity on z, ||z||^2 = d).  Sub-vector s
    sits at distance delta_s from the bisector of an entry p and its nearest
    neighbour q, on p's side; such a point has p and q as its two nearest
    entries (any entry nearer to the midpoint would be nearer to p than q is)."""
    C = codebook()
    D2 = ((C[:, None] - C[None]) ** 2).sum(-1)
    np.fill_diagonal(D2, np.inf)
    nearest = np.argmin(D2, axis=1)
    deltas = [0.5e-5, 2e-5, 0.5e-5, 2e-5, 0.1, 0.0, 0.5e-5, 2e-5, 0.1, 0.5e-5, 2e-5, 0.0, 0.5e-5, 2e-5, 0.1]
    want_flag = [1 if dl < BAND else 0 for dl in deltas]
    z = np.zeros(128)
    ps, qs = [], []
    for s, dl in enumerate(deltas):
        p = (37 * s + 5) % 256
        q = nearest[p]
        n = (C[p] - C[q]) / np.linalg.norm(C[p] - C[q])
        z[8 * s:8 * s + 8] = 0.5 * (C[p] + C[q]) + dl * n
        ps.append(p)
        qs.append(q)
    # the last sub-vector takes the remaining norm, along a direction whose
    # nearest entry wins by a wide margin (checked by brute force)
    R = np.sqrt(128.0 - np.sum(z[:120] ** 2))
    for cand in range(256):
        v = C[cand] / np.linalg.norm(C[cand]) * R
        dd = np.sort(((v - C) ** 2).sum(-1))
        if dd[1] - dd[0] > 0.1:
            z[120:] = v
            break
    else:
        pytest.fail("no far sub-vector found")
    x = H128 @ z / 128.0
    r = O.nsn_vq(x[None, None], C, o_given=np.zeros((1, 128)), want_z=True)
    np.testing.assert_allclose(r["z"][0, 0], z, atol=1e-13)
    fl = r["flags"][0, 0]
    codes = r["codes"][0, 0]
    assert list(fl[:15]) == want_flag
    assert fl[15] == 0
    for s, dl in enumerate(deltas):
        if dl > 0:
            assert codes[s] == ps[s], s
        else:
            assert codes[s] in (ps[s], qs[s]), s
    assert codes[15] == np.argmin(((z[120:] - C) ** 2).sum(-1))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_beta_mse_against_independent_quadrature(bits):
    """kvqo_beta_mse(c, t) = E (y - c[idx(y)])^2 under the law of sqrt(d) u_1,
    checked with scipy's adaptive quadrature of the normalised density."""
    d = 128
    c, t = O.tables_f32_beta(bits)
    c, t = c.astype(np.float64), t.astype(np.float64)
    r = np.sqrt(d)
    pdf = lambda y: stats.beta.pdf((y / r + 1) / 2, (d - 1) / 2, (d - 1) / 2) / (2 * r)  # noqa: E731
    edges = np.concatenate([[-r], t, [r]])
    want = 0.0
    for j in range(len(c)):
        v, _ = integrate.quad(lambda y: (y - c[j]) ** 2 * pdf(y), edges[j], edges[j + 1], epsabs=1e-14,
                              epsrel=1e-12, limit=200)
        want += v
    got = O.beta_mse(bits, c, t)
    assert abs(got / want - 1) < 1e-9, (got, want)
    # the Gaussian tables under the same law: same integral, other centroids
    cg, tg = (a.astype(np.float64) for a in O.tables_f32(bits))
    eg = np.concatenate([[-r], tg, [r]])
    wg = sum(integrate.quad(lambda y: (y - cg[j]) ** 2 * pdf(y), eg[j], eg[j + 1], epsabs=1e-14,
                            epsrel=1e-12, limit=200)[0] for j in range(len(cg)))
    assert abs(O.beta_mse(bits, cg, tg) / wg - 1) < 1e-9


def test_beta_mse_against_monte_carlo_on_unit_vectors():
    """The same MSE estimated from 8e6 coordinates of uniform unit vectors."""
    d, bits = 128, 3
    rng = np.random.default_rng(2024)
    g = rng.standard_normal((62_500, d))
    y = np.sqrt(d) * g / np.linalg.norm(g, axis=1, keepdims=True)
    c, t = O.tables_f32_beta(bits)
    idx = np.searchsorted(t.astype(np.float64), y, side="left")
    est = np.mean((y - c.astype(np.float64)[idx]) ** 2)
    assert abs(est / O.beta_mse(bits, c, t) - 1) < 3e-3
