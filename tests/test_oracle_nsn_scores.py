"""Pins of the oracle's attention over NSN-VQ codes (CPU only).

The score kernels of the NSNQuant page ("Detalhes de Implementacao") fold the
byproducts s1, s2, o into attention; reconstruction inverts Metodologia 1-2:
x_hat = s1 (s2 H zq / sqrt(d) + o).  The strong pins build a codebook whose
entries ARE the sub-vectors of the exact transform z of some tokens, so the
codes reconstruct those tokens exactly; then logits and attention must equal
the plain inner products and the plain softmax attention over the original
vectors, which involve no part of the method."""
import os

import numpy as np

import oracle as O
from calibration_free_kv_amd import synth

GOLDEN_CB = os.path.join(os.path.dirname(__file__), "golden", "vq_codebook_256x8.txt")


def _codebook():
    return np.loadtxt(GOLDEN_CB, dtype=np.float32).reshape(256, 8)


def _exact_codes(x, first):
    """Codes naming entries first, first+1, ... that hold the sub-vectors of
    the exact transform of x [H,T,d]; returns (codes [1,H,T,16], s1, s2, o,
    entries [H*T*16, 8])."""
    r = O.nsn_vq(x, _codebook(), want_z=True)
    H, T, d = x.shape
    entries = r["z"].reshape(H * T * 16, 8)
    codes = (first + np.arange(H * T * 16)).reshape(1, H, T, 16).astype(np.uint8)
    return codes, r["s1"][None], r["s2"][None], r["o"][None], entries


def _lognormal_tokens(seed, H, T):
    x = synth.random_tensor(seed, (H, T, 128)).astype(np.float64)
    x *= np.exp(np.random.default_rng(seed + 100).standard_normal((H, 1, 128)))
    return x.astype(np.float16).astype(np.float64)


def test_logits_of_exact_codes_are_plain_inner_products():
    x = _lognormal_tokens(1, 2, 8)
    x[1, 3] = 0.0  # zero token: s1 = 0, the key reconstructs to 0
    codes, s1, s2, o, ent = _exact_codes(x, 0)
    cb = ent  # 2 heads x 8 tokens x 16 sub-vectors = 256 entries
    q = synth.random_tensor(2, (1, 4, 128)).astype(np.float64)  # 2 query heads per KV head
    want = np.einsum("hd,htd->ht", q[0], np.repeat(x, 2, axis=0))[None]
    scale = np.linalg.norm(q, axis=-1)[..., None] * np.repeat(np.linalg.norm(x, axis=-1), 2, axis=0)[None]
    for route in (1, 2):
        got = O.nsn_logits(q, codes, s1, s2, o, cb, route=route)
        assert np.abs(got - want).max() <= 1e-12 * scale.max(), route
    assert np.all(O.nsn_logits(q, codes, s1, s2, o, cb)[:, 2:4, 3] == 0.0)


def test_attention_of_exact_codes_is_plain_softmax_attention():
    xk = _lognormal_tokens(3, 1, 8)
    xv = _lognormal_tokens(4, 1, 8)
    kc, ks1, ks2, ko, ek = _exact_codes(xk, 0)
    vc, vs1, vs2, vo, ev = _exact_codes(xv, 128)
    cb = np.concatenate([ek, ev])
    q = synth.random_tensor(5, (1, 4, 128)).astype(np.float64) * 0.2
    for sm in (None, 0.01):
        got = O.nsn_attention(q, kc, ks1, ks2, ko, vc, vs1, vs2, vo, cb, sm_scale=sm)
        scale = 1 / np.sqrt(128) if sm is None else sm
        s = scale * q[0] @ xk[0].T  # [4, 8]
        w = np.exp(s - s.max(axis=1, keepdims=True))
        want = (w @ xv[0]) / w.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(got[0], want, rtol=1e-11, atol=1e-11 * np.abs(xv).max())


def test_logit_routes_agree_on_random_codes():
    c = synth.random_nsn_codes(6, (2, 3, 50))
    q = synth.random_tensor(7, (2, 12, 128)).astype(np.float64)
    cb = _codebook()
    a = O.nsn_logits(q, c["codes"], c["s1"], c["s2"], c["o"], cb, route=1)
    b = O.nsn_logits(q, c["codes"], c["s1"], c["s2"], c["o"], cb, route=2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(a).max())


def test_attention_special_cases():
    c = synth.random_nsn_codes(8, (1, 2, 40))
    v = synth.random_nsn_codes(9, (1, 2, 40))
    cb = _codebook()
    args = (c["codes"], c["s1"], c["s2"], c["o"], v["codes"], v["s1"], v["s2"], v["o"], cb)
    # the reconstructed values, written out from the stated inverse
    H = O.hadamard_matrix(128)
    zq = cb.astype(np.float64)[v["codes"].astype(np.int64)].reshape(1, 2, 40, 128)
    vh = v["s1"][..., None] * (v["s2"][..., None] * (zq @ H.T) / np.sqrt(128) + v["o"][:, :, None, :])
    # zero query: uniform weights, the mean value vector
    out = O.nsn_attention(np.zeros((1, 8, 128)), *args)
    np.testing.assert_allclose(out[0], np.repeat(vh[0].mean(axis=1), 4, axis=0), rtol=1e-12, atol=1e-12)
    # one token: its value vector
    first = lambda e: (e["codes"][:, :, :1], e["s1"][:, :, :1], e["s2"][:, :, :1], e["o"])
    q = synth.random_tensor(10, (1, 8, 128)).astype(np.float64)
    out = O.nsn_attention(q, *first(c), *first(v), cb)
    np.testing.assert_allclose(out[0], np.repeat(vh[0, :, 0], 4, axis=0), rtol=1e-12, atol=1e-12)
    # a huge scale selects the value of the largest logit
    lg = O.nsn_logits(q, c["codes"], c["s1"], c["s2"], c["o"], cb)
    out = O.nsn_attention(q, *args, sm_scale=1e6)
    best = lg.argmax(axis=-1)[0]
    np.testing.assert_allclose(out[0], vh[0, np.arange(8) // 4, best], rtol=1e-9, atol=1e-9)
