"""Pins of the oracle's gain-shape residual quantisation (GSRQ page:
gain-shape k-means keeps the gain apart from the shape; GSKM stages in a
residual quantisation pipeline give GSRQ, below 1 bit per element).  The
reading: the NSN front end (NSNQuant page, Metodologia 1-2), 32-dim
sub-vectors, two stages of 256 unit shapes and 16 gain levels each (24 bits
per 32 elements = 0.75 bit per element).  CPU only."""
import os

import numpy as np
import pytest

import oracle as O
from calibration_free_kv_amd import synth
from tests.test_oracle_hadamard import sylvester

HERE = os.path.dirname(__file__)
GOLDEN_CB = os.path.join(HERE, "golden", "vq_codebook_256x8.txt")
GOLDEN_GSRQ = os.path.join(HERE, "golden", "gsrq_tables_256x32.txt")
H128 = sylvester(128).astype(np.float64)


def tables():
    """The fixture: stage 1 shapes (256 lines), levels (1 line), stage 2 alike."""
    lines = [ln.split() for ln in open(GOLDEN_GSRQ) if not ln.startswith("#")]
    return dict(S1=np.array(lines[0:256], dtype=np.float32), G1=np.array(lines[256], dtype=np.float32),
                S2=np.array(lines[257:513], dtype=np.float32), G2=np.array(lines[513], dtype=np.float32))


def test_front_end_equals_the_nsn_encoder_steps():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 50, 128)) * np.exp(rng.standard_normal((2, 1, 128)))
    x[1, 7] = 0
    f = O.nsn_front(x)
    cb = np.loadtxt(GOLDEN_CB, dtype=np.float32).reshape(256, 8)
    r = O.nsn_vq(x, cb, want_z=True)
    for k in ("s1", "s2", "o", "z"):
        np.testing.assert_array_equal(f[k], r[k])


def test_gskm_shapes_objective_and_fixed_point():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3000, 16))
    S, obj = O.gskm(x, rng.choice(3000, 32, replace=False), passes=8)
    np.testing.assert_allclose(np.linalg.norm(S, axis=1), 1.0, rtol=1e-13)
    assert np.all(np.diff(obj) >= -1e-12) and obj[-1] > obj[0]
    # K = n: every sample keeps its own direction, objective = mean norm
    y = rng.standard_normal((5, 4))
    S, obj = O.gskm(y, np.arange(5), passes=3)
    np.testing.assert_allclose(S, y / np.linalg.norm(y, axis=1, keepdims=True), atol=1e-15)
    np.testing.assert_allclose(obj, np.linalg.norm(y, axis=1).mean(), rtol=1e-14)


def test_gskm_one_step_closed_form():
    """Two clusters of directions in 2-D: after a pass each shape is the unit
    vector along its cell's sum (the maximiser of the summed projection)."""
    x = np.array([[1.0, 0.1], [2.0, -0.1], [1.5, 0.2], [0.1, 1.0], [-0.2, 3.0]])
    S, obj = O.gskm(x, np.array([0, 3]), passes=1)
    a, b = x[:3].sum(0), x[3:].sum(0)
    np.testing.assert_allclose(S[0], a / np.linalg.norm(a), atol=1e-15)
    np.testing.assert_allclose(S[1], b / np.linalg.norm(b), atol=1e-15)
    e0 = x[0] / np.linalg.norm(x[0])
    e1 = x[3] / np.linalg.norm(x[3])
    want = np.mean([max(v @ e0, v @ e1) for v in x])
    np.testing.assert_allclose(obj[0], want, rtol=1e-14)


def test_lloyd_1d_two_points_and_fixed_point():
    v = np.array([1.0] * 30 + [5.0] * 70)
    np.testing.assert_allclose(O.lloyd_1d(v, 2, passes=5), [1.0, 5.0])
    rng = np.random.default_rng(3)
    g = rng.standard_normal(20000) + 3
    lv = O.lloyd_1d(g, 8, passes=300)
    t = 0.5 * (lv[1:] + lv[:-1])
    cell = np.searchsorted(t, g, side="left")
    for k in range(8):
        np.testing.assert_allclose(lv[k], g[cell == k].mean(), rtol=1e-9)
    assert np.all(np.diff(lv) > 0)


def axis_tables(m=32, L=16):
    """Shapes = the signed unit axes (K = 2m), levels on an exact grid."""
    S = np.concatenate([np.eye(m), -np.eye(m)])
    G = 0.5 + 0.25 * np.arange(L)
    return dict(S1=S, G1=G, S2=S, G2=G / 16)  # every stage-2 level below every stage-1 level


def test_encode_recovers_exact_two_stage_vectors():
    """z = G1[c1] e_a + G2[c2] e_b (a != b) is reproduced exactly, with the
    codes that name it."""
    tab = axis_tables()
    rng = np.random.default_rng(4)
    z, want = [], []
    for _ in range(200):
        a, b = rng.choice(32, 2, replace=False)
        sa, sb = rng.choice([0, 32], 2)
        c1, c2 = rng.integers(0, 16, 2)
        v = np.zeros(32)
        v[a] = tab["G1"][c1] * (1 if sa == 0 else -1)
        v[b] = tab["G2"][c2] * (1 if sb == 0 else -1)
        z.append(v)
        want.append((a + sa, b + sb, c1 | (c2 << 4)))
    codes, zhat, fl = O.gsrq_encode(np.array(z), tab)
    assert np.array_equal(codes, np.array(want, dtype=np.uint8))
    np.testing.assert_array_equal(zhat, np.array(z))
    assert not fl.any()


def test_encode_flags_at_known_distances():
    """Two shapes whose projections differ by 0.5e-5 (flagged) or 2e-5 (not),
    and a projection 0.5e-5 from a gain threshold."""
    tab = axis_tables()
    t = 0.5 * (tab["G1"][5] + tab["G1"][6])
    z = np.zeros((4, 32))
    z[0, 0], z[0, 1] = 1.9, 1.9 - 0.5e-5
    z[1, 0], z[1, 1] = 1.9, 1.9 - 2e-5
    z[2, 3] = t + 0.5e-5
    z[3, 3] = t + 2e-5
    codes, zhat, fl = O.gsrq_encode(z, tab)
    assert list(fl & 1) == [1, 0, 0, 0]
    assert list(fl & 2) == [0, 0, 2, 0]
    assert codes[0, 0] == 0 and codes[1, 0] == 0  # the larger projection wins
    assert codes[2, 2] & 15 == 6 and codes[3, 2] & 15 == 6  # above the threshold: the upper level


def test_record_layout_and_reproduction_from_the_tables():
    tab = tables()
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 20, 128)) * np.exp(rng.standard_normal((1, 1, 128)))
    r = O.gsrq_vq(x, tab)
    rec = r["codes"][0]
    assert rec.shape == (20, 12)
    for t in (0, 7, 19):
        zq = np.concatenate([tab["G1"][rec[t, 8 + s] & 15] * tab["S1"][rec[t, s]].astype(np.float64)
                             + tab["G2"][rec[t, 8 + s] >> 4] * tab["S2"][rec[t, 4 + s]].astype(np.float64)
                             for s in range(4)])
        np.testing.assert_allclose(zq, r["zhat"][0, t], atol=1e-12)


def test_fixture_tables_and_the_second_stage_gain():
    """Unit shapes, increasing levels; on held-out N(0, I_32) sub-vectors the
    second stage lowers the error, and both stages beat zero."""
    tab = tables()
    for k in (1, 2):
        np.testing.assert_allclose(np.linalg.norm(tab["S%d" % k].astype(np.float64), axis=1), 1.0, atol=1e-6)
        assert np.all(np.diff(tab["G%d" % k]) > 0)
    z = synth.gaussian_samples(99, 4000, dim=32)
    _, zh2, _ = O.gsrq_encode(z, tab)
    one = dict(tab, G2=np.zeros(16, np.float32))
    _, zh1, _ = O.gsrq_encode(z, one)
    e2 = np.mean((z - zh2) ** 2)
    e1 = np.mean((z - zh1) ** 2)
    assert e2 < e1 < 1.0
    assert e1 - e2 > 0.05


def test_nsn_identity_with_the_exact_rotated_vector():
    """x = s1 (s2 H z / sqrt(d) + o) with z unquantised: the front end inverts."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 9, 128))
    f = O.nsn_front(x)
    for t in range(9):
        xr = f["s1"][0, t] * (f["s2"][0, t] * (H128 @ f["z"][0, t]) / np.sqrt(128) + f["o"][0])
        np.testing.assert_allclose(xr, x[0, t], atol=1e-12)


@pytest.mark.parametrize("G", [1, 4])
def test_logit_routes_agree_and_attention_special_cases(G):
    tab = tables()
    rng = np.random.default_rng(7)
    Hkv, T = 2, 40
    xk = rng.standard_normal((Hkv, T, 128)) * np.exp(rng.standard_normal((Hkv, 1, 128)))
    xv = rng.standard_normal((Hkv, T, 128))
    k, v = O.gsrq_vq(xk, tab), O.gsrq_vq(xv, tab)
    lead = lambda a: a[None]  # noqa: E731
    q = rng.standard_normal((1, Hkv * G, 128))
    a = O.gsrq_logits(q, lead(k["codes"]), lead(k["s1"]), lead(k["s2"]), lead(k["o"]), tab, route=1)
    b = O.gsrq_logits(q, lead(k["codes"]), lead(k["s1"]), lead(k["s2"]), lead(k["o"]), tab, route=2)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)
    # a zero query weighs every token equally: the mean reconstruction
    out = O.gsrq_attention(np.zeros_like(q), lead(k["codes"]), lead(k["s1"]), lead(k["s2"]), lead(k["o"]),
                           lead(v["codes"]), lead(v["s1"]), lead(v["s2"]), lead(v["o"]), tab)
    for g in range(Hkv):
        vh = np.array([O.nsn_reconstruct(v["zhat"][g, t], v["s1"][g, t], v["s2"][g, t], v["o"][g]) for t in range(T)])
        np.testing.assert_allclose(out[0, g * G], vh.mean(0), atol=1e-12)
    # one token: its reconstruction
    one = O.gsrq_attention(q, lead(k["codes"][:, :1]), lead(k["s1"][:, :1]), lead(k["s2"][:, :1]), lead(k["o"]),
                           lead(v["codes"][:, :1]), lead(v["s1"][:, :1]), lead(v["s2"][:, :1]), lead(v["o"]), tab)
    np.testing.assert_allclose(one[0, 0], O.nsn_reconstruct(v["zhat"][0, 0], v["s1"][0, 0], v["s2"][0, 0],
                                                            v["o"][0]), atol=1e-12)
