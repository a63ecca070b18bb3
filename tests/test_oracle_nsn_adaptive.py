"""Pins of the oracle's adaptive scale for NSN-VQ codes (CPU only).

NSNQuant page, Metodologia sec. 3, "Ajuste de Escala": the quantised vector
is rescaled so that its component along the original vector is preserved,
leaving only an error orthogonal to it.  Reading: with z the transformed
token and zq its selected codebook entries, alpha = ||z||^2 / <z, zq> and the
stored s2 becomes alpha * s2, so the usual reconstruction
x_hat = s1 (s2 H zq / sqrt(d) + o) carries the scaled entries."""
import os

import numpy as np

import oracle as O
from calibration_free_kv_amd import synth
from tests.test_oracle_hadamard import sylvester

GOLDEN_CB = os.path.join(os.path.dirname(__file__), "golden", "vq_codebook_256x8.txt")
H128 = sylvester(128).astype(np.float64)


def _codebook():
    return np.loadtxt(GOLDEN_CB, dtype=np.float32).reshape(256, 8).astype(np.float64)


def test_error_is_orthogonal_to_the_shifted_token():
    """x - s1 o = s1 s2 H z / sqrt(d); with the scaled entries the error
    x_hat - x is orthogonal to it in the original space, for every token."""
    x = synth.make("nsn_vq", T=200)["x"].astype(np.float64)
    cb = _codebook()
    r = O.nsn_vq(x, cb, adaptive=True)
    plain = O.nsn_vq(x, cb)
    assert np.array_equal(r["codes"], plain["codes"])  # the scale does not change the codes
    np.testing.assert_array_equal(r["s1"], plain["s1"])
    H, T, d = x.shape
    worst = 0.0
    ratios = []
    for h in range(H):
        for t in range(0, T, 7):
            zq = cb[r["codes"][h, t].astype(np.int64)].reshape(d)
            xh = O.nsn_reconstruct(zq, r["s1"][h, t], r["s2"][h, t], r["o"][h])
            xc = x[h, t] - r["s1"][h, t] * r["o"][h]
            worst = max(worst, abs(np.dot(xh - x[h, t], xc)) / np.dot(xc, xc))
            # without the scale the error has a component along xc
            xp = O.nsn_reconstruct(zq, plain["s1"][h, t], plain["s2"][h, t], plain["o"][h])
            ratios.append(np.dot(xp - plain["s1"][h, t] * plain["o"][h], xc) / np.dot(xc, xc))
    assert worst < 1e-12
    # the plain entries shrink the token along itself (k-means centroids sit
    # inside their cells), which the scale undoes: alpha > 1 on average
    assert np.mean(ratios) < 0.95
    assert np.mean(r["s2"] / plain["s2"]) > 1.02


def test_token_proportional_to_its_entries_is_reconstructed_exactly():
    """If z is c times a concatenation of entries that stay nearest after the
    scaling, the scaled entries are z itself (alpha = c): lossless."""
    cb = _codebook()
    d = 128
    # entries j whose nearest entry is still j after scaling by a c near 1
    chosen = []
    for j in range(256):
        ok = all(np.argmin(((c * cb[j] - cb) ** 2).sum(-1)) == j for c in (0.9, 1.0, 1.1, 1.2))
        if ok:
            chosen.append(j)
        if len(chosen) == 16:
            break
    assert len(chosen) == 16
    zq = cb[chosen].reshape(d)
    c = np.sqrt(d) / np.linalg.norm(zq)
    assert 0.9 < c < 1.2
    z = c * zq
    x = H128 @ z / 128.0  # with the mean given as zero, x encodes to z exactly
    r = O.nsn_vq(x[None, None], cb, o_given=np.zeros((1, d)), want_z=True, adaptive=True)
    assert list(r["codes"][0, 0]) == chosen
    plain = O.nsn_vq(x[None, None], cb, o_given=np.zeros((1, d)))
    np.testing.assert_allclose(r["s2"][0, 0] / plain["s2"][0, 0], c, rtol=1e-12)
    xh = O.nsn_reconstruct(zq, r["s1"][0, 0], r["s2"][0, 0], np.zeros(d))
    np.testing.assert_allclose(xh, x, atol=1e-13)


def test_degenerate_tokens_keep_their_scale():
    """A token equal to the mean (b = 0, z = 0) has <z, zq> = 0: alpha = 1."""
    x = synth.make("nsn_vq", T=1)["x"].astype(np.float64)
    cb = _codebook()
    r = O.nsn_vq(x, cb, adaptive=True)
    p = O.nsn_vq(x, cb)
    np.testing.assert_array_equal(r["s2"], p["s2"])
