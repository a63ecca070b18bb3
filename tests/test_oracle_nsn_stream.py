"""Pins of the oracle's NSN-VQ streaming-cache attention (CPU only).

NSNQuant page, Detalhes de Implementacao, "Residuos": following KIVI the
cache is a quantised part plus a full-precision residual that is quantised
and appended when it fills.  Read with Metodologia sec. 1, every flushed group
is one NSN call with its own channel mean, so packed token t reconstructs with
the mean of its group t / Gs; the window tokens are used as they are."""
import os

import numpy as np

import oracle as O
from calibration_free_kv_amd import synth

GOLDEN_CB = os.path.join(os.path.dirname(__file__), "golden", "vq_codebook_256x8.txt")


def _cb():
    return np.loadtxt(GOLDEN_CB, dtype=np.float32).reshape(256, 8).astype(np.float64)


def encode_groups(x, Gs):
    """x [B, Hkv, T, d] -> codes/s1/s2 [B, Hkv, T, ...] and means [B, Hkv, T/Gs, d],
    each group of Gs tokens one NSN-VQ call (as a flush encodes it)."""
    B, Hkv, T, d = x.shape
    cb = _cb()
    out = dict(codes=np.zeros((B, Hkv, T, 16), np.uint8), s1=np.zeros((B, Hkv, T)), s2=np.zeros((B, Hkv, T)),
               o=np.zeros((B, Hkv, T // Gs, d)))
    for g in range(T // Gs):
        r = O.nsn_vq(x[:, :, g * Gs:(g + 1) * Gs].reshape(B * Hkv, Gs, d), cb)
        out["codes"][:, :, g * Gs:(g + 1) * Gs] = r["codes"].reshape(B, Hkv, Gs, 16)
        out["s1"][:, :, g * Gs:(g + 1) * Gs] = r["s1"].reshape(B, Hkv, Gs)
        out["s2"][:, :, g * Gs:(g + 1) * Gs] = r["s2"].reshape(B, Hkv, Gs)
        out["o"][:, :, g] = r["o"].reshape(B, Hkv, d)
    return out


def data(seed, B, Hkv, T, G=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, B, Hkv, T, 128)) * np.exp(rng.standard_normal((2, 1, Hkv, 1, 128)))
    q = rng.standard_normal((B, Hkv * G, 128))
    return x[0], x[1], q


def stream(q, k, v, kt, vt, Gs, sm_scale=None):
    return O.nsn_attention_stream(q, k["codes"], k["s1"], k["s2"], k["o"], v["codes"], v["s1"], v["s2"], v["o"],
                                  kt, vt, _cb(), Gs, sm_scale=sm_scale)


def recon(e, Gs):
    """Reconstructions x_hat of every packed token (each with its group's mean)."""
    B, Hkv, T, _ = e["codes"].shape
    cb = _cb()
    out = np.zeros((B, Hkv, T, 128))
    for b in range(B):
        for g in range(Hkv):
            for t in range(T):
                zq = cb[e["codes"][b, g, t].astype(np.int64)].reshape(128)
                out[b, g, t] = O.nsn_reconstruct(zq, e["s1"][b, g, t], e["s2"][b, g, t], e["o"][b, g, t // Gs])
    return out


def test_one_group_without_window_is_the_plain_nsn_decode():
    K, V, q = data(1, 2, 2, 96)
    k, v = encode_groups(K, 96), encode_groups(V, 96)
    empty = np.zeros((2, 2, 0, 128))
    got = stream(q, k, v, empty, empty, 96)
    want = O.nsn_attention(q, k["codes"], k["s1"], k["s2"], k["o"][:, :, 0], v["codes"], v["s1"], v["s2"],
                           v["o"][:, :, 0], _cb())
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_window_only_is_plain_softmax_attention():
    K, V, q = data(2, 1, 2, 40)
    e = encode_groups(K[:, :, :0], 8)
    got = stream(q, e, e, K, V, 8)
    s = np.einsum("bhd,bhtd->bht", q, np.repeat(K, 4, axis=1)) / np.sqrt(128)
    w = np.exp(s - s.max(-1, keepdims=True))
    want = np.einsum("bht,bhtd->bhd", w, np.repeat(V, 4, axis=1)) / w.sum(-1)[..., None]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_each_group_reads_its_own_mean():
    """The last group's tokens moved into the window as their reconstructions
    change nothing; neither does swapping two groups (codes, scales and mean
    slots together): attention does not depend on token order."""
    Gs = 32
    K, V, q = data(3, 1, 2, 3 * Gs)
    k, v = encode_groups(K, Gs), encode_groups(V, Gs)
    empty = np.zeros((1, 2, 0, 128))
    full = stream(q, k, v, empty, empty, Gs)
    cut = lambda e: {n: (a[:, :, :2] if n == "o" else a[:, :, :2 * Gs]) for n, a in e.items()}  # noqa: E731
    kr, vr = recon(k, Gs)[:, :, 2 * Gs:], recon(v, Gs)[:, :, 2 * Gs:]
    np.testing.assert_allclose(stream(q, cut(k), cut(v), kr, vr, Gs), full, rtol=1e-12, atol=1e-12)

    def swap(e):
        o = {n: a.copy() for n, a in e.items()}
        for n in ("codes", "s1", "s2"):
            o[n][:, :, :Gs], o[n][:, :, Gs:2 * Gs] = e[n][:, :, Gs:2 * Gs], e[n][:, :, :Gs]
        o["o"][:, :, 0], o["o"][:, :, 1] = e["o"][:, :, 1], e["o"][:, :, 0]
        return o
    np.testing.assert_allclose(stream(q, swap(k), swap(v), empty, empty, Gs), full, rtol=1e-12, atol=1e-12)
    # and the means matter: giving every group the first group's mean changes the result
    k0 = {n: a.copy() for n, a in k.items()}
    k0["o"][:, :, 1:] = k["o"][:, :, :1]
    assert np.abs(stream(q, k0, v, empty, empty, Gs) - full).max() > 1e-3
