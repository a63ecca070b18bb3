"""Every (mode, bit width, query heads per KV head) that kvq_create and the
score dispatchers accept, against the CPU oracle at small ragged sizes, and
the decode cases where one key takes essentially all of the softmax weight.

Both sides score the same codes written by the oracle's encoders (no GPU
output feeds the oracle).  Logits within 1e-3 ||q|| ||k|| (and at fp32
level, 1e-5); attention outputs within 2e-3 max-abs."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]

GOLDEN_CB = os.path.join(os.path.dirname(__file__), "golden", "vq_codebook_256x8.txt")


def kv_inputs(seed, B, Hkv, T):
    """Lognormal-scaled K and V [B, Hkv, T, 128] fp16 and their sign diagonals."""
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((B, Hkv, T, 128)) * np.exp(rng.standard_normal((1, Hkv, 1, 128)))).astype(np.float16)
    v = (rng.standard_normal((B, Hkv, T, 128)) * np.exp(rng.standard_normal((1, Hkv, 1, 128)))).astype(np.float16)
    sk = synth.random_signs(rng, Hkv)
    sv = synth.random_signs(rng, Hkv)
    return k, v, sk, sv


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_logit_err(lg, ref, q, norms, G):
    scale = np.linalg.norm(q.astype(np.float64), axis=-1)[..., None] * np.repeat(norms.astype(np.float64), G, axis=1)
    return (np.abs(lg - ref) / np.maximum(scale, 1e-30)).max()


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_mse_logits_every_width_and_group(bits, G):
    B, Hkv, T = 2, 2, 333
    k, _, sk, sv = kv_inputs(100 + 10 * bits + G, B, Hkv, T)
    q = synth.random_tensor(7 + G, (B, Hkv * G, 128))
    r = O.quantize(k, sk, bits)
    kn = r["norms"].astype(np.float32)
    ctx = kvq.Context(Hkv, bits, sk, sv)
    lg = to_np(ctx.logits(dev(q), dev(r["codes"]), dev(kn)))
    ref = O.logits(q, r["codes"], kn.astype(np.float64), sk, bits)
    err = rel_logit_err(lg, ref, q, kn, G)
    assert err <= 1e-5, (bits, G, err)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_mse_decode_every_width_and_group(bits, G):
    B, Hkv, T = 2, 2, 1333
    k, v, sk, sv = kv_inputs(200 + 10 * bits + G, B, Hkv, T)
    q = synth.random_tensor(17 + G, (B, Hkv * G, 128))
    rk, rv = O.quantize(k, sk, bits), O.quantize(v, sv, bits)
    kn, vn = rk["norms"].astype(np.float32), rv["norms"].astype(np.float32)
    ctx = kvq.Context(Hkv, bits, sk, sv)
    out = to_np(ctx.attn_decode(dev(q), dev(rk["codes"]), dev(kn), dev(rv["codes"]), dev(vn)))
    ref = O.attention(q, rk["codes"], kn.astype(np.float64), rv["codes"], vn.astype(np.float64), sk, sv, bits)
    err = np.abs(out - ref).max()
    assert err <= 2e-3, (bits, G, err)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_qjl_logits_every_width_and_group(bits, G):
    B, Hkv, T = 1, 2, 555
    k, _, sk, sv = kv_inputs(300 + 10 * bits + G, B, Hkv, T)
    S = np.random.default_rng(31).standard_normal((128, 128)).astype(np.float16).astype(np.float32)
    q = synth.random_tensor(27 + G, (B, Hkv * G, 128))
    r = O.quantize(k, sk, bits, want_y=True)
    qj = O.qjl(r["y"], r["idx"], S, bits)
    kn, gm = r["norms"].astype(np.float32), qj["gamma"].astype(np.float32)
    ctx = kvq.Context(Hkv, bits, sk, sv, mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=S)
    lg = to_np(ctx.logits(dev(q), dev(r["codes"]), dev(kn), dev(qj["signs"]), dev(gm)))
    ref = O.logits(q, r["codes"], kn.astype(np.float64), sk, bits, qjl_signs=qj["signs"],
                   gamma=gm.astype(np.float64), S=S)
    err = rel_logit_err(lg, ref, q, kn, G)
    assert err <= 1e-5, (bits, G, err)


@pytest.mark.parametrize("G", [1, 2, 4])
def test_dense_one_bit_decode_and_logits(G):
    B, Hkv, T, bits = 1, 2, 900, 1
    k, v, _, _ = kv_inputs(400 + G, B, Hkv, T)
    Q = synth.random_orthogonal(60 + G).astype(np.float32)
    Qd = Q.astype(np.float64)
    q = synth.random_tensor(37 + G, (B, Hkv * G, 128))
    rk, rv = O.quantize_dense(k, Qd, bits), O.quantize_dense(v, Qd, bits)
    kn, vn = rk["norms"].astype(np.float32), rv["norms"].astype(np.float32)
    ctx = kvq.Context(Hkv, bits, rot_Q=Q)
    lg = to_np(ctx.logits(dev(q), dev(rk["codes"]), dev(kn)))
    assert rel_logit_err(lg, O.logits_dense(q, rk["codes"], kn.astype(np.float64), Qd, bits), q, kn, G) <= 1e-5
    out = to_np(ctx.attn_decode(dev(q), dev(rk["codes"]), dev(kn), dev(rv["codes"]), dev(vn)))
    ref = O.attention_dense(q, rk["codes"], kn.astype(np.float64), rv["codes"], vn.astype(np.float64), Qd, bits)
    assert np.abs(out - ref).max() <= 2e-3


def test_stream_one_bit():
    B, Hkv, T, R, bits = 1, 2, 700, 40, 1
    k, v, sk, sv = kv_inputs(500, B, Hkv, T + R)
    q = synth.random_tensor(47, (B, 8, 128))
    rk, rv = O.quantize(k[:, :, :T], sk, bits), O.quantize(v[:, :, :T], sv, bits)
    kn, vn = rk["norms"].astype(np.float32), rv["norms"].astype(np.float32)
    kt, vt = np.ascontiguousarray(k[:, :, T:]), np.ascontiguousarray(v[:, :, T:])
    ctx = kvq.Context(Hkv, bits, sk, sv)
    out = to_np(ctx.attn_decode_stream(dev(q), dev(rk["codes"]), dev(kn), dev(rv["codes"]), dev(vn), T, dev(kt),
                                       dev(vt), R))
    ref = O.attention_stream(q, rk["codes"], kn.astype(np.float64), rv["codes"], vn.astype(np.float64), kt, vt,
                             sk, sv, bits)
    assert np.abs(out - ref).max() <= 2e-3


# ----------------------------------------------------------------------------- one dominant key
def plant(x, q, G, first=100, step=37):
    """Key t_h = first + step h of KV head h // G becomes 4 q_h, so that its
    logit for query head h (about 4 ||q_h||^2) stands far above the others."""
    for h in range(q.shape[1]):
        x[0, h // G, first + step * h] = (q[0, h].astype(np.float32) * 4).astype(np.float16)


def dominant_scale(lg):
    """A softmax scale under which, for every query head, the largest logit
    exceeds the runner-up by at least 40 (weight of the rest below 1e-14 of it)."""
    s = np.sort(lg, axis=-1)
    gap = (s[..., -1] - s[..., -2]).min()
    assert gap > 50, gap  # the planted keys dominate by far more than the logits' rounding
    return float(40.0 / gap)


def test_mse_decode_one_dominant_key():
    """A decode whose softmax puts all weight on one key returns that key's
    dequantised value, v_hat = rho D .* H c[idx] / d."""
    B, Hkv, T, bits, G = 1, 2, 2000, 3, 4
    k, v, sk, sv = kv_inputs(600, B, Hkv, T)
    q = synth.random_tensor(57, (B, Hkv * G, 128))
    plant(k, q, G)
    rk, rv = O.quantize(k, sk, bits), O.quantize(v, sv, bits)
    kn, vn = rk["norms"].astype(np.float32), rv["norms"].astype(np.float32)
    lg = O.logits(q, rk["codes"], kn.astype(np.float64), sk, bits)
    sm = dominant_scale(lg)
    ctx = kvq.Context(Hkv, bits, sk, sv)
    out = to_np(ctx.attn_decode(dev(q), dev(rk["codes"]), dev(kn), dev(rv["codes"]), dev(vn), sm_scale=sm))
    ref = O.attention(q, rk["codes"], kn.astype(np.float64), rv["codes"], vn.astype(np.float64), sk, sv, bits,
                      sm_scale=sm)
    assert np.abs(out - ref).max() <= 2e-3
    for h in range(Hkv * G):
        g, t = h // G, int(np.argmax(lg[0, h]))
        vh = O.dequant(rv["codes"][0, g, t], float(vn[0, g, t]), sv[g], bits)
        np.testing.assert_allclose(out[0, h], vh, atol=1e-4 * np.abs(vh).max())


def test_stream_decode_one_dominant_key():
    """The dominant key in the fp16 window for some heads, in the packed
    prefix for others."""
    B, Hkv, T, R, bits, G = 1, 2, 900, 30, 2, 4
    k, v, sk, sv = kv_inputs(700, B, Hkv, T + R)
    q = synth.random_tensor(67, (B, Hkv * G, 128))
    plant(k, q, G, first=10, step=97)
    rk, rv = O.quantize(k[:, :, :T], sk, bits), O.quantize(v[:, :, :T], sv, bits)
    kn, vn = rk["norms"].astype(np.float32), rv["norms"].astype(np.float32)
    kt, vt = np.ascontiguousarray(k[:, :, T:]), np.ascontiguousarray(v[:, :, T:])
    kt[0, 0, 5] = (q[0, 0].astype(np.float32) * 5).astype(np.float16)  # head 0 prefers window token 5
    lq = O.logits(q, rk["codes"], kn.astype(np.float64), sk, bits)
    kw = kt.astype(np.float64)[:, np.arange(Hkv * G) // G]          # [B, Hq, R, d]
    lw = (kw * q.astype(np.float64)[:, :, None, :]).sum(-1)          # window logits
    lg = np.concatenate([lq, lw], axis=-1)
    sm = dominant_scale(lg)
    ctx = kvq.Context(Hkv, bits, sk, sv)
    out = to_np(ctx.attn_decode_stream(dev(q), dev(rk["codes"]), dev(kn), dev(rv["codes"]), dev(vn), T, dev(kt),
                                       dev(vt), R, sm_scale=sm))
    ref = O.attention_stream(q, rk["codes"], kn.astype(np.float64), rv["codes"], vn.astype(np.float64), kt, vt,
                             sk, sv, bits, sm_scale=sm)
    assert np.abs(out - ref).max() <= 2e-3
    where = np.argmax(lg[0], axis=-1)
    assert (where >= T).any() and (where < T).any()
    for h in range(Hkv * G):
        g, t = h // G, int(where[h])
        want = vt[0, g, t - T].astype(np.float64) if t >= T else O.dequant(rv["codes"][0, g, t], float(vn[0, g, t]),
                                                                           sv[g], bits)
        np.testing.assert_allclose(out[0, h], want, atol=1e-4 * np.abs(want).max())


def test_nsn_decode_one_dominant_key():
    B, Hkv, T, G = 1, 2, 1500, 4
    cb = np.loadtxt(GOLDEN_CB, dtype=np.float32).reshape(256, 8)

    q = synth.random_tensor(77, (B, Hkv * G, 128))

    def enc(seed, planted=False):
        x = synth.random_tensor(seed, (B * Hkv, T, 128)).astype(np.float64)
        x *= np.exp(np.random.default_rng(seed + 1).standard_normal((B * Hkv, 1, 128)))
        x = x.astype(np.float16)
        if planted:
            plant(x[None], q, G)
        r = O.nsn_vq(x, cb)
        return dict(codes=r["codes"].reshape(B, Hkv, T, 16), s1=r["s1"].astype(np.float32).reshape(B, Hkv, T),
                    s2=r["s2"].astype(np.float32).reshape(B, Hkv, T), o=r["o"].astype(np.float32).reshape(B, Hkv, 128))

    kk, vv = enc(800, planted=True), enc(802)
    lg = O.nsn_logits(q, kk["codes"], kk["s1"], kk["s2"], kk["o"], cb)
    sm = dominant_scale(lg)
    ctx = kvq.Context(Hkv, 1, mode=kvq.KVQ_MODE_NSN_VQ, vq_codebook=cb)
    out = to_np(ctx.nsn_attn_decode(dev(q), {n: dev(a) for n, a in kk.items()}, {n: dev(a) for n, a in vv.items()},
                                    sm_scale=sm))
    ref = O.nsn_attention(q, kk["codes"], kk["s1"], kk["s2"], kk["o"], vv["codes"], vv["s1"], vv["s2"], vv["o"], cb,
                          sm_scale=sm)
    assert np.abs(out - ref).max() <= 2e-3
    for h in range(Hkv * G):
        g, t = h // G, int(np.argmax(lg[0, h]))
        zq = cb.astype(np.float64)[vv["codes"][0, g, t].astype(np.int64)].reshape(128)
        want = O.nsn_reconstruct(zq, float(vv["s1"][0, g, t]), float(vv["s2"][0, g, t]), vv["o"][0, g])
        np.testing.assert_allclose(out[0, h], want, atol=1e-4 * np.abs(want).max())
