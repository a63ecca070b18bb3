"""Pins of the oracle's attention over a cache split into a quantised prefix
and a full-precision residual window (NSNQuant page, "Detalhes de
Implementacao": following KIVI, the residual is quantised and appended when
it fills).  CPU only.

The strong pins use plain softmax attention over explicit vectors, which
involves no part of the method: a residual-only cache, and a prefix whose
vectors are exactly what their codes reconstruct."""
import numpy as np
import pytest

import oracle as O
from calibration_free_kv_amd import synth


def plain_attention(q, K, V, scale):
    """q [Hq,d]; K, V [Hkv,N,d] -> [Hq,d] (GQA: query head h reads KV head h // (Hq/Hkv))."""
    G = q.shape[0] // K.shape[0]
    out = np.zeros_like(q)
    for h in range(q.shape[0]):
        s = scale * K[h // G] @ q[h]
        w = np.exp(s - s.max())
        out[h] = w @ V[h // G] / w.sum()
    return out


def exact_vectors(rng, bits, signs, n):
    """n vectors per head equal to what their codes reconstruct:
    rho D .* H c[idx] / d; returns (codes, norms, vectors)."""
    H_, d = signs.shape
    c, _ = O.tables_f32(bits)
    idx = rng.integers(0, 1 << bits, size=(1, H_, n, d))
    rho = rng.uniform(0.5, 3.0, size=(1, H_, n))
    Hm = O.hadamard_matrix(d).astype(np.float64)
    y = c.astype(np.float64)[idx]
    vec = rho[..., None] * signs[None, :, None, :] * (y @ Hm.T) / d
    return O.pack(idx, bits), rho, vec


@pytest.mark.parametrize("bits", [2, 3])
def test_residual_only_is_plain_attention(bits):
    rng = np.random.default_rng(1)
    kt, vt = rng.standard_normal((2, 1, 2, 9, 128))
    q = rng.standard_normal((1, 4, 128))
    s = np.ones((2, 128), np.int8)
    empty_c = np.zeros((1, 2, 0, 16 * bits), np.uint8)
    got = O.attention_stream(q, empty_c, np.zeros((1, 2, 0)), empty_c, np.zeros((1, 2, 0)), kt, vt, s, s, bits)
    np.testing.assert_allclose(got[0], plain_attention(q[0], kt[0], vt[0], 1 / np.sqrt(128)), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_exact_prefix_then_residual_is_plain_attention(bits):
    rng = np.random.default_rng(2)
    sk, sv = synth.random_signs(rng, 2), synth.random_signs(rng, 2)
    kc, kn, kx = exact_vectors(rng, bits, sk, 7)
    vc, vn, vx = exact_vectors(rng, bits, sv, 7)
    kt, vt = rng.standard_normal((2, 1, 2, 5, 128))
    q = rng.standard_normal((1, 8, 128)) * 0.3
    got = O.attention_stream(q, kc, kn, vc, vn, kt, vt, sk, sv, bits, sm_scale=0.2)
    K = np.concatenate([kx[0], kt[0]], axis=1)
    V = np.concatenate([vx[0], vt[0]], axis=1)
    np.testing.assert_allclose(got[0], plain_attention(q[0], K, V, 0.2), rtol=1e-11, atol=1e-11)


def test_no_residual_equals_prefix_attention():
    inp = synth.make("l8b32k", T=40)
    r_k = O.quantize(inp["k"], inp["signs_k"], 3)
    r_v = O.quantize(inp["v"], inp["signs_v"], 3)
    empty = np.zeros((1, 8, 0, 128))
    a = O.attention_stream(inp["q"], r_k["codes"], r_k["norms"], r_v["codes"], r_v["norms"], empty, empty,
                           inp["signs_k"], inp["signs_v"], 3)
    b = O.attention(inp["q"], r_k["codes"], r_k["norms"], r_v["codes"], r_v["norms"], inp["signs_k"],
                    inp["signs_v"], 3)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_moving_exact_tokens_into_the_residual_changes_nothing():
    rng = np.random.default_rng(3)
    sk, sv = synth.random_signs(rng, 1), synth.random_signs(rng, 1)
    kc, kn, kx = exact_vectors(rng, 3, sk, 6)
    vc, vn, vx = exact_vectors(rng, 3, sv, 6)
    q = rng.standard_normal((1, 2, 128)) * 0.3
    a = O.attention_stream(q, kc, kn, vc, vn, np.zeros((1, 1, 0, 128)), np.zeros((1, 1, 0, 128)), sk, sv, 3)
    b = O.attention_stream(q, kc[:, :, :4], kn[:, :, :4], vc[:, :, :4], vn[:, :, :4], kx[:, :, 4:], vx[:, :, 4:],
                           sk, sv, 3)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
