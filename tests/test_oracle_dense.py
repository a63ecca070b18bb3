"""Pins of the oracle's dense-rotation path ("O Que E TurboQuant?", Como
Funciona, Estagio 1: a random orthogonal transformation from the QR
decomposition of a Gaussian matrix).  The strong pins use the orthogonal
matrix Q = H diag(D) / sqrt(d), with which the dense path must reproduce the
randomized-Hadamard path exactly.  CPU only."""
import numpy as np
import pytest

import oracle as O
from calibration_free_kv_amd import synth


def hadamard_Q(signs_row):
    return O.hadamard_matrix(128).astype(np.float64) * signs_row[None, :].astype(np.float64) / np.sqrt(128)


def test_generator_is_orthogonal():
    Q = synth.random_orthogonal(3)
    np.testing.assert_allclose(Q.T @ Q, np.eye(128), atol=1e-12)
    Qh = hadamard_Q(synth.random_signs(np.random.default_rng(0), 1)[0])
    np.testing.assert_allclose(Qh.T @ Qh, np.eye(128), atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_hadamard_as_dense_matrix_reproduces_the_hadamard_path(bits):
    inp = synth.make("l8b32k", T=200)
    x, signs = inp["k"][:, :1], inp["signs_k"][:1]
    Q = hadamard_Q(signs[0])
    a = O.quantize(x, signs, bits, want_y=True)
    b = O.quantize_dense(x, Q, bits, want_y=True)
    np.testing.assert_allclose(b["y"], a["y"], atol=1e-12)
    bad = (a["idx"] != b["idx"]) & (a["flags"] == 0)
    assert not bad.any()
    np.testing.assert_allclose(b["norms"], a["norms"], rtol=1e-15)
    np.testing.assert_allclose(O.dequant_dense(a["codes"][0, 0, 5], a["norms"][0, 0, 5], Q, bits),
                               O.dequant(a["codes"][0, 0, 5], a["norms"][0, 0, 5], signs[0], bits), atol=1e-12)
    q = inp["q"][:, :4]
    for route in (0, 1):
        np.testing.assert_allclose(O.logits_dense(q, a["codes"], a["norms"], Q, bits, route=route),
                                   O.logits(q, a["codes"], a["norms"], signs, bits), rtol=1e-11, atol=1e-11)
    v = O.quantize(inp["v"][:, :1], signs, bits)
    np.testing.assert_allclose(O.attention_dense(q, a["codes"], a["norms"], v["codes"], v["norms"], Q, bits),
                               O.attention(q, a["codes"], a["norms"], v["codes"], v["norms"], signs, signs, bits),
                               rtol=1e-11, atol=1e-11)


def test_random_rotation_error_matches_the_gaussian_mse():
    """With a Haar-random Q the rotated coordinates are close to N(0,1), so the
    relative reconstruction error approaches the Lloyd-Max MSE per coordinate."""
    Q = synth.random_orthogonal(5)
    x = synth.random_tensor(6, (1, 1, 3000, 128)).astype(np.float64)
    r = O.quantize_dense(x, Q, 3)
    err = 0.0
    for t in range(0, 3000, 10):
        xh = O.dequant_dense(r["codes"][0, 0, t], r["norms"][0, 0, t], Q, 3)
        err += np.sum((xh - x[0, 0, t]) ** 2) / np.sum(x[0, 0, t] ** 2)
    c, t_ = O.tables_f32(3)
    mse = O.gauss_mse(3, c.astype(np.float64), t_.astype(np.float64))
    assert abs(err / 300 / mse - 1) < 0.1


def test_dense_logit_routes_agree():
    Q = synth.random_orthogonal(7)
    inp = synth.make("l8b32k", T=50)
    r = O.quantize_dense(inp["k"][:, :2], Q, 3)
    q = inp["q"][:, :8]
    a = O.logits_dense(q, r["codes"], r["norms"], Q, 3, route=0)
    b = O.logits_dense(q, r["codes"], r["norms"], Q, 3, route=1)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------- dense rotation + QJL residual
def test_dense_qjl_with_hadamard_matrix_reproduces_the_hadamard_qjl_path():
    """TurboQuant's two stages (Como Funciona, Estagio 1 + 2) with Q = H diag(D)
    / sqrt(d): the same rotated coordinates, hence the same residual signs and
    gamma, and the same QJL-corrected logits on both routes."""
    inp = synth.make("long128k_qjl", T=120)
    x, signs = inp["k"][:, :1], inp["signs_k"][:1]
    S = inp["S"].astype(np.float64)
    Q = hadamard_Q(signs[0])
    for bits in (1, 2, 3):
        a = O.quantize(x, signs, bits, want_y=True)
        b = O.quantize_dense(x, Q, bits, want_y=True)
        same = (a["idx"] == b["idx"]).all(-1)  # keys without a boundary flip
        qa = O.qjl(a["y"], a["idx"], S, bits)
        qb = O.qjl(b["y"], b["idx"], S, bits)
        np.testing.assert_allclose(qb["gamma"][same], qa["gamma"][same], rtol=1e-11)
        flag = qa["flags"].astype(bool)[same]
        bits_a = np.unpackbits(qa["signs"][same], axis=-1, bitorder="little")
        bits_b = np.unpackbits(qb["signs"][same], axis=-1, bitorder="little")
        assert not ((bits_a != bits_b) & ~flag).any()
        q = inp["q"][:, :4]
        ref = O.logits(q, a["codes"], a["norms"], signs, bits, qjl_signs=qa["signs"], gamma=qa["gamma"], S=S)
        for route in (0, 1):
            np.testing.assert_allclose(
                O.logits_dense(q, a["codes"], a["norms"], Q, bits, route=route, qjl_signs=qa["signs"],
                               gamma=qa["gamma"], S=S), ref, rtol=1e-11, atol=1e-11)


def test_dense_qjl_logit_routes_agree():
    Q = synth.random_orthogonal(11)
    rng = np.random.default_rng(12)
    k = rng.standard_normal((1, 2, 30, 128))
    S = rng.standard_normal((128, 128))
    r = O.quantize_dense(k, Q, 2, want_y=True)
    o = O.qjl(r["y"], r["idx"], S, 2)
    q = rng.standard_normal((1, 8, 128))
    a = O.logits_dense(q, r["codes"], r["norms"], Q, 2, route=0, qjl_signs=o["signs"], gamma=o["gamma"], S=S)
    b = O.logits_dense(q, r["codes"], r["norms"], Q, 2, route=1, qjl_signs=o["signs"], gamma=o["gamma"], S=S)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


def test_dense_qjl_estimator_is_unbiased():
    """Over independent projections S the corrected logit averages to the exact
    <q, k> under a Haar-random rotation too; the MSE-only logit is biased."""
    Q = synth.random_orthogonal(13)
    rng = np.random.default_rng(14)
    k = rng.standard_normal((1, 1, 1, 128)) * np.exp(rng.standard_normal(128))
    # a query along the key, where the MSE-only shrinkage (about 1 - MSE_1) shows
    q = (k[0, 0] / np.linalg.norm(k) + 0.3 * rng.standard_normal((1, 128)) / np.sqrt(128))[None]
    r = O.quantize_dense(k, Q, 1, want_y=True)
    exact = float(q[0, 0] @ k[0, 0, 0])
    mse_only = O.logits_dense(q, r["codes"], r["norms"], Q, 1)[0, 0, 0]
    est = []
    for _ in range(600):
        S = rng.standard_normal((128, 128))
        o = O.qjl(r["y"], r["idx"], S, 1)
        est.append(O.logits_dense(q, r["codes"], r["norms"], Q, 1, qjl_signs=o["signs"], gamma=o["gamma"],
                                  S=S)[0, 0, 0])
    est = np.array(est)
    se = est.std(ddof=1) / np.sqrt(len(est))
    assert abs(est.mean() - exact) < 4 * se
    assert abs(mse_only - exact) > 4 * se
