"""Pins of the oracle's logits, attention and QJL residual (CPU only).

Scores read straight from the indices with the query rotated once
(TurboQuant page, Como Implementar); 1-bit QJL residual correcting the
inner-product bias (TurboQuant page, Estagio 2)."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle as O
from calibration_free_kv_amd import synth
from tests.test_oracle_quantize import H128, dequant_dense


def _setup(bits, T=200, seed=0):
    rng = np.random.default_rng(seed)
    B, Hkv, Hq = 2, 2, 8
    k = rng.standard_normal((B, Hkv, T, 128)) * np.exp(rng.standard_normal((Hkv, 1, 128)))
    v = rng.standard_normal((B, Hkv, T, 128)) * np.exp(rng.standard_normal((Hkv, 1, 128)))
    q = rng.standard_normal((B, Hq, 128))
    sk = np.where(rng.integers(0, 2, (Hkv, 128)) == 1, 1, -1).astype(np.int8)
    sv = np.where(rng.integers(0, 2, (Hkv, 128)) == 1, 1, -1).astype(np.int8)
    rk = O.quantize(k, sk, bits, want_y=True)
    rv = O.quantize(v, sv, bits)
    return dict(k=k, v=v, q=q, sk=sk, sv=sv, rk=rk, rv=rv, B=B, Hkv=Hkv, Hq=Hq, T=T)


def _dense_keys(s, bits, which="k"):
    r, sg = (s["rk"], s["sk"]) if which == "k" else (s["rv"], s["sv"])
    c32, _ = O.tables_f32(bits)
    out = np.zeros(s[which].shape)
    for b in range(s["B"]):
        for g in range(s["Hkv"]):
            out[b, g] = dequant_dense(r["idx"][b, g], r["norms"][b, g], sg[g].astype(np.float64), c32)
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_logit_routes_agree_and_match_dense(bits):
    s = _setup(bits)
    l0 = O.logits(s["q"], s["rk"]["codes"], s["rk"]["norms"], s["sk"], bits, route=0)
    l1 = O.logits(s["q"], s["rk"]["codes"], s["rk"]["norms"], s["sk"], bits, route=1)
    kh = _dense_keys(s, bits)
    G = s["Hq"] // s["Hkv"]
    ref = np.einsum("bhd,bhtd->bht", s["q"], np.repeat(kh, G, axis=1))
    scale = np.linalg.norm(s["q"], axis=-1)[..., None] * np.repeat(s["rk"]["norms"], G, axis=1)
    assert np.max(np.abs(l0 - l1) / scale) < 1e-12
    assert np.max(np.abs(l1 - ref) / scale) < 1e-12


@pytest.mark.parametrize("bits", [2, 3])
def test_attention_matches_dense_softmax(bits):
    s = _setup(bits, T=150, seed=4)
    out = O.attention(s["q"], s["rk"]["codes"], s["rk"]["norms"], s["rv"]["codes"],
                      s["rv"]["norms"], s["sk"], s["sv"], bits)
    kh, vh = _dense_keys(s, bits, "k"), _dense_keys(s, bits, "v")
    G = s["Hq"] // s["Hkv"]
    lg = np.einsum("bhd,bhtd->bht", s["q"], np.repeat(kh, G, axis=1)) / np.sqrt(128)
    ref = np.einsum("bht,bhtd->bhd", softmax(lg, axis=-1), np.repeat(vh, G, axis=1))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)


def test_attention_special_cases():
    s = _setup(3, T=40, seed=9)
    args = (s["rk"]["codes"], s["rk"]["norms"], s["rv"]["codes"], s["rv"]["norms"], s["sk"], s["sv"], 3)
    vh = _dense_keys(s, 3, "v")
    G = s["Hq"] // s["Hkv"]
    # T = 1: output is the only value
    one = O.attention(s["q"], s["rk"]["codes"][:, :, :1], s["rk"]["norms"][:, :, :1],
                      s["rv"]["codes"][:, :, :1], s["rv"]["norms"][:, :, :1], s["sk"], s["sv"], 3)
    np.testing.assert_allclose(one, np.repeat(vh[:, :, 0], G, axis=1), rtol=1e-12, atol=1e-12)
    # zero query: equal logits, output is the mean value
    z = O.attention(np.zeros_like(s["q"]), *args)
    np.testing.assert_allclose(z, np.repeat(vh.mean(axis=2), G, axis=1), rtol=1e-12, atol=1e-12)
    # one dominant logit: a huge scale picks the arg-max key's value
    big = O.attention(s["q"], *args, sm_scale=1e6)
    l1 = O.logits(s["q"], s["rk"]["codes"], s["rk"]["norms"], s["sk"], 3)
    am = np.argmax(l1, axis=-1)
    for b in range(s["B"]):
        for h in range(s["Hq"]):
            np.testing.assert_allclose(big[b, h], vh[b, h // G, am[b, h]], rtol=1e-9, atol=1e-9)


def _qjl_setup(bits, m, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((1, 1, 1, 128))
    s = np.where(rng.integers(0, 2, (1, 128)) == 1, 1, -1).astype(np.int8)
    r = O.quantize(k, s, bits, want_y=True)
    q = rng.standard_normal((1, 1, 128))
    return k, s, r, q


def test_qjl_bits_and_gamma_by_definition():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((1, 2, 30, 128))
    s = np.where(rng.integers(0, 2, (2, 128)) == 1, 1, -1).astype(np.int8)
    S = rng.standard_normal((128, 128))
    r = O.quantize(k, s, 2, want_y=True)
    out = O.qjl(r["y"], r["idx"], S, 2)
    c32, _ = O.tables_f32(2)
    res = (r["y"] - c32[r["idx"]]) / np.sqrt(128)
    np.testing.assert_allclose(out["gamma"], np.linalg.norm(res, axis=-1), rtol=1e-13)
    z = res @ S.T
    bits = (z >= 0).astype(np.uint8)
    assert np.array_equal(out["signs"], np.packbits(bits, axis=-1, bitorder="little"))


@pytest.mark.parametrize("bits", [1, 2])
def test_qjl_estimator_is_unbiased(bits):
    """Over independent projections S the QJL-corrected logit averages to the
    exact <q, k>; the MSE-only logit is shrunk by 1 - MSE_b."""
    k, s, r, q = _qjl_setup(bits, 128, seed=40 + bits)
    exact = float(q[0, 0] @ k[0, 0, 0])
    mse_only = O.logits(q, r["codes"], r["norms"], s, bits)[0, 0, 0]
    rng = np.random.default_rng(7)
    est = []
    for _ in range(600):
        S = rng.standard_normal((128, 128))
        o = O.qjl(r["y"], r["idx"], S, bits)
        est.append(O.logits(q, r["codes"], r["norms"], s, bits, qjl_signs=o["signs"],
                            gamma=o["gamma"], S=S)[0, 0, 0])
    est = np.array(est)
    se = est.std(ddof=1) / np.sqrt(len(est))
    assert abs(est.mean() - exact) < 4 * se
    # the bias of the plain MSE logit is far outside that band
    assert abs(mse_only - exact) > 4 * se
    # variance bound: Var <= (pi/2) rho^2 gamma^2 ||R q||^2 / m
    gamma = O.qjl(r["y"], r["idx"], rng.standard_normal((128, 128)), bits)["gamma"][0, 0, 0]
    bound = np.pi / 2 * r["norms"][0, 0, 0] ** 2 * gamma ** 2 * np.sum(q ** 2) / 128
    assert est.var(ddof=1) < 1.2 * bound


def test_qjl_variance_shrinks_with_m():
    k, s, r, q = _qjl_setup(1, 0, seed=77)
    rng = np.random.default_rng(8)
    var = []
    for m in (32, 512):
        est = []
        for _ in range(300):
            S = rng.standard_normal((m, 128))
            o = O.qjl(r["y"], r["idx"], S, 1)
            est.append(O.logits(q, r["codes"], r["norms"], s, 1, qjl_signs=o["signs"],
                                gamma=o["gamma"], S=S)[0, 0, 0])
        var.append(np.var(est))
    assert var[1] < var[0] / 8  # ~1/m scaling (16x fewer -> at least 8x smaller)


def test_qjl_logit_routes_agree():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 2, 25, 128))
    s = np.where(rng.integers(0, 2, (2, 128)) == 1, 1, -1).astype(np.int8)
    S = rng.standard_normal((128, 128))
    r = O.quantize(k, s, 2, want_y=True)
    o = O.qjl(r["y"], r["idx"], S, 2)
    q = rng.standard_normal((1, 8, 128))
    a = O.logits(q, r["codes"], r["norms"], s, 2, route=0, qjl_signs=o["signs"], gamma=o["gamma"], S=S)
    b = O.logits(q, r["codes"], r["norms"], s, 2, route=1, qjl_signs=o["signs"], gamma=o["gamma"], S=S)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)
