"""Pins of the oracle's 4-bit double quantisation of the NSN byproducts
(NSNQuant page, Metodologia sec. 3, "Double Quantization": o, s1 and the
codebook entries stored with 4 bits).  The page gives no scheme; the reading
is the uniform min-max quantiser of a block (lo = min, step = range / 15,
round to nearest), s1 in blocks of 32 tokens, o in one block per head, the
codebook in one block.  CPU only."""
import os

import numpy as np
import pytest

import oracle as O
from tests.test_oracle_hadamard import sylvester

GOLDEN_CB = os.path.join(os.path.dirname(__file__), "golden", "vq_codebook_256x8.txt")
H128 = sylvester(128).astype(np.float64)


def codebook():
    return np.loadtxt(GOLDEN_CB, dtype=np.float32).reshape(256, 8).astype(np.float64)


def test_dq4_error_bound_and_extremes():
    rng = np.random.default_rng(1)
    for n in (2, 17, 128, 2048):
        v = rng.standard_normal(n) * 3 + 1
        c, lo, step, _ = O.dq4(v)
        assert c.max() <= 15
        vh = lo + c * step
        assert np.all(np.abs(vh - v) <= step / 2 * (1 + 1e-12))
        assert lo == v.min() and step == (v.max() - v.min()) / 15
        assert c[np.argmin(v)] == 0 and c[np.argmax(v)] == 15
        assert vh[np.argmin(v)] == lo


def test_dq4_reproduces_values_on_its_grid():
    """Values lo + k step (step a power of two, so the grid is exact) come back
    with code k, including both ends."""
    rng = np.random.default_rng(2)
    k = rng.integers(0, 16, 200)
    k[:2] = (0, 15)
    v = -3.0 + k * 0.25
    c, lo, step, fl = O.dq4(v)
    assert lo == -3.0 and step == 0.25
    assert np.array_equal(c, k) and not fl.any()


def test_dq4_constant_block():
    c, lo, step, fl = O.dq4(np.full(40, 2.5))
    assert step == 0.0 and lo == 2.5 and not c.any() and not fl.any()


def test_dq4_flags_at_known_distances():
    """u = (v - lo) / step at 0.5e-4 (flagged) and 2e-4 (not) from a half-integer."""
    base = np.array([0.0, 15.0, 3.5 + 0.5e-4, 3.5 - 0.5e-4, 7.5 + 2e-4, 7.5 - 2e-4, 11.0])
    v = 1.0 + base * 0.125
    c, lo, step, fl = O.dq4(v)
    assert lo == 1.0 and step == 0.125
    assert list(fl) == [0, 0, 1, 1, 0, 0, 0]
    assert list(c) == [0, 15, 4, 3, 8, 7, 11]


def test_nibble_packing_round_trip_and_layout():
    c = np.array([[1, 2, 3], [15, 0, 7]], np.uint8)
    p = O.pack_nibbles(c)
    assert p.tolist() == [[0x21, 0x03], [0x0F, 0x07]]
    assert np.array_equal(O.unpack_nibbles(p, 3), c)


def test_nsn_dq_encoding_inverts_with_the_quantised_mean():
    """x_t = s1_t (s2_t H z_t / sqrt(d) + o_hat) holds exactly with the
    unquantised z: the shift used the 4-bit mean o_hat, not o."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 40, 128)) * np.exp(rng.standard_normal((2, 1, 128)))
    r = O.nsn_vq_dq(x, codebook(), want_z=True)
    assert np.abs(r["o_hat"] - r["o"]).max() > 1e-3  # the quantised mean differs from o
    assert np.all(np.abs(r["o_hat"] - r["o"]) <= r["o_step"][:, None] / 2 * (1 + 1e-12))
    for h in range(2):
        for t in (0, 17, 39):
            xr = r["s1"][h, t] * (r["s2"][h, t] * (H128 @ r["z"][h, t]) / np.sqrt(128) + r["o_hat"][h])
            np.testing.assert_allclose(xr, x[h, t], rtol=0, atol=1e-12 * np.abs(x[h, t]).max())
    # the encoder with the exact mean gives other s2 and z (the shift moved)
    r0 = O.nsn_vq(x, codebook(), want_z=True)
    assert np.abs(r0["s2"] - r["s2"]).max() > 1e-6


def test_nsn_dq_s1_blocks():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 70, 128)) * np.exp(rng.standard_normal((3, 1, 128)))
    r = O.nsn_vq_dq(x, codebook())
    assert r["s1_lo"].shape == (3, 3)  # blocks of 32, 32 and 6 tokens
    for h in range(3):
        for b, sl in enumerate((slice(0, 32), slice(32, 64), slice(64, 70))):
            s1 = r["s1"][h, sl]
            assert r["s1_lo"][h, b] == s1.min()
            np.testing.assert_allclose(r["s1_lo"][h, b] + 15 * r["s1_step"][h, b], s1.max(), rtol=1e-14)
            assert np.all(np.abs(r["s1_hat"][h, sl] - s1) <= r["s1_step"][h, b] / 2 * (1 + 1e-12))
    assert np.array_equal(O.unpack_nibbles(r["s1q"], 70), r["s1_codes"])
    assert np.array_equal(O.unpack_nibbles(r["oq"], 128), r["o_codes"])


def test_nsn_dq_single_token_and_zero_token():
    """One token: its a equals o, o_hat differs from it by < step/2 per channel,
    so b = a - o_hat is the rounding residue; s1 is one block of one value
    (step 0, stored exactly).  A zero token keeps s1 = 0."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 1, 128))
    r = O.nsn_vq_dq(x, codebook())
    assert r["s1_step"][0, 0] == 0 and r["s1_hat"][0, 0] == r["s1"][0, 0]
    np.testing.assert_allclose(r["s2"][0, 0], np.linalg.norm(r["o"][0] - r["o_hat"][0]) / np.sqrt(128), rtol=1e-12)
    x = rng.standard_normal((1, 33, 128))
    x[0, 5] = 0
    r = O.nsn_vq_dq(x, codebook())
    assert r["s1"][0, 5] == 0 and r["s1_codes"][0, 5] == 0 and r["s1_hat"][0, 5] == 0


@pytest.mark.parametrize("seed", [6, 7])
def test_dq_s1_only_rescales_the_reconstruction(seed):
    """The 4-bit s1 multiplies the whole reconstruction, so per token the
    change is |s1_hat - s1| / s1 of ||x_hat||, at most half a step."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, 64, 128)) * np.exp(rng.standard_normal((1, 1, 128)))
    r = O.nsn_vq_dq(x, codebook())
    C = codebook()
    for t in (0, 31, 63):
        zq = C[r["codes"][0, t].astype(np.int64)].reshape(128)
        a = O.nsn_reconstruct(zq, r["s1"][0, t], r["s2"][0, t], r["o_hat"][0])
        b = O.nsn_reconstruct(zq, r["s1_hat"][0, t], r["s2"][0, t], r["o_hat"][0])
        bound = abs(r["s1_hat"][0, t] - r["s1"][0, t]) * np.linalg.norm(a) / max(r["s1"][0, t], 1e-300)
        assert np.linalg.norm(b - a) <= bound * (1 + 1e-10) + 1e-12


def test_dq_codebook():
    c, lo, step, fl, cbh = O.dq_codebook(codebook())
    assert len(np.unique(cbh)) <= 16
    assert np.all(np.abs(cbh - codebook()) <= step / 2 * (1 + 1e-12))
    assert lo == codebook().min()
