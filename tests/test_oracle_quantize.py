"""Pins of the oracle's quantiser, packing and dequantiser (CPU only).

Per-vector L2 norm kept, normalised vector rotated by the random-sign
Walsh-Hadamard transform, coordinates bucketed against Gaussian Lloyd-Max
thresholds (PolarQuant page, sec. 2; TurboQuant page, Estagio 1)."""
import json
import os

import numpy as np
import pytest

import oracle as O
from calibration_free_kv_amd import synth
from tests.test_oracle_hadamard import sylvester

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_constants.json")))
H128 = sylvester(128).astype(np.float64)


def test_pack_layout_hand_example():
    idx = np.zeros(128, np.int32)
    idx[:3] = [1, 5, 7]
    rec = O.pack(idx, 3)
    # coordinate i occupies bits [3i, 3i+3) of the record, LSB first
    assert rec.shape == (48,) and rec[0] == 0xE9 and rec[1] == 0x01 and not rec[2:].any()


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_pack_roundtrip(bits):
    idx = np.random.default_rng(bits).integers(0, 1 << bits, (5, 128)).astype(np.int32)
    rec = O.pack(idx, bits)
    assert rec.shape == (5, 16 * bits)
    assert np.array_equal(O.unpack(rec, 128, bits), idx)
    # bit-level check against an independent numpy formulation
    bitstream = ((idx[:, :, None] >> np.arange(bits)) & 1).reshape(5, -1)
    assert np.array_equal(np.packbits(bitstream, axis=1, bitorder="little"), rec)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_against_dense_nearest_centroid(bits):
    inp = synth.make("tiny", T=300)
    x = inp["k"].astype(np.float64)
    D = inp["signs_k"][0].astype(np.float64)
    r = O.quantize(x, inp["signs_k"], bits, want_y=True)
    xv = x[0, 0]
    rho = np.linalg.norm(xv, axis=1)
    np.testing.assert_allclose(r["norms"][0, 0], rho, rtol=1e-14)
    y = (H128 @ (D[:, None] * (xv / rho[:, None]).T)).T
    np.testing.assert_allclose(r["y"][0, 0], y, atol=1e-12)
    c32, t32 = O.tables_f32(bits)
    nn = np.argmin(np.abs(y[..., None] - c32.astype(np.float64)), axis=-1)
    flagged = r["flags"][0, 0].astype(bool)
    assert np.array_equal(r["idx"][0, 0][~flagged], nn[~flagged])
    assert np.array_equal(O.unpack(r["codes"], 128, bits), r["idx"])
    # rotated coordinates have unit mean square exactly: ||y||^2 = d
    np.testing.assert_allclose(np.sum(y ** 2, axis=1), 128.0, rtol=1e-12)


def test_scale_invariance_and_zero_vector():
    x = synth.random_tensor(7, (1, 1, 64, 128)).astype(np.float64)
    x[0, 0, 5] = 0.0
    s = np.where(np.random.default_rng(1).integers(0, 2, (1, 128)) == 1, 1, -1)
    for bits in (1, 2, 3, 4):
        a = O.quantize(x, s, bits)
        b = O.quantize(x * 8.0, s, bits)
        assert np.array_equal(a["codes"], b["codes"])
        np.testing.assert_allclose(b["norms"], 8.0 * a["norms"], rtol=1e-15)
        # zero vector: u = 0, y = 0, every index = #{t_j < 0} = 2^(b-1) - 1
        assert a["norms"][0, 0, 5] == 0.0
        assert np.all(a["idx"][0, 0, 5] == (1 << (bits - 1)) - 1)


def dequant_dense(idx, rho, D, c32):
    return rho[:, None] * (D[None, :] * (c32[idx].astype(np.float64) @ H128.T)) / 128.0


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequant_matches_dense(bits):
    inp = synth.make("tiny", T=50)
    r = O.quantize(inp["k"], inp["signs_k"], bits)
    c32, _ = O.tables_f32(bits)
    ref = dequant_dense(r["idx"][0, 0], r["norms"][0, 0], inp["signs_k"][0].astype(np.float64), c32)
    for t in range(50):
        got = O.dequant(r["codes"][0, 0, t], r["norms"][0, 0, t], inp["signs_k"][0], bits)
        np.testing.assert_allclose(got, ref[t], rtol=1e-12, atol=1e-12)


def test_cosine_three_bits_matches_page():
    """Mean cosine between a vector and its reconstruction ~ sqrt(1 - MSE_3)
    = 0.9826; the TurboQuant page reports 0.983+ at 3 bits."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((1, 1, 4000, 128))
    s = np.where(rng.integers(0, 2, (1, 128)) == 1, 1, -1)
    r = O.quantize(x, s, 3)
    c32, _ = O.tables_f32(3)
    xh = dequant_dense(r["idx"][0, 0], r["norms"][0, 0], s[0].astype(np.float64), c32)
    xv = x[0, 0]
    cos = np.sum(xh * xv, 1) / np.linalg.norm(xh, axis=1) / np.linalg.norm(xv, axis=1)
    page = GOLD["turboquant_cosine_3bit"]["value"]
    assert abs(cos.mean() - page) < 2e-3
    assert abs(cos.mean() - np.sqrt(1 - 0.0345478)) < 1.5e-3


@pytest.mark.parametrize("bits,mse", [(1, 0.363380), (2, 0.117482), (3, 0.0345478)])
def test_mse_only_inner_product_bias(bits, mse):
    """<q, k_hat> shrinks <q, k> by the factor 1 - MSE_b on average (the bias
    the QJL residual is there to correct, TurboQuant page, Estagio 2)."""
    rng = np.random.default_rng(100 + bits)
    n = 6000
    k = rng.standard_normal((1, 1, n, 128))
    q = rng.standard_normal(128)
    s = np.where(rng.integers(0, 2, (1, 128)) == 1, 1, -1)
    r = O.quantize(k, s, bits)
    c32, _ = O.tables_f32(bits)
    kh = dequant_dense(r["idx"][0, 0], r["norms"][0, 0], s[0].astype(np.float64), c32)
    exact = k[0, 0] @ q
    approx = kh @ q
    slope = np.sum(approx * exact) / np.sum(exact * exact)
    assert abs(slope - (1 - mse)) < 0.01
