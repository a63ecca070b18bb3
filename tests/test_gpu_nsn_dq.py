"""GPU parity of the double-quantised NSN-VQ path (NSNQuant page, Metodologia
sec. 3, "Double Quantization": o, s1 and the codebook entries in 4 bits)
against the CPU oracle.

Encoder: the 4-bit codes of the means and of s1 are exact except values whose
rounding lies within 1e-4 of a step of a half-integer (flagged by the oracle;
there the GPU's code must be the oracle's or its neighbour, and a differing
mean code is followed by the oracle's encoding with that admissible mean);
the (lo, step) pairs within 1e-5; VQ codes exact outside the 1e-5 bisector
band.  Scoring: the GPU reads 4-bit byproducts written by the oracle's
encoder or drawn by the seeded generator; the oracle scores their
dequantised values.  No GPU output feeds the oracle."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import needs_gpu, to_np
from tests.test_gpu_nsn import bisector_excess

pytestmark = [pytest.mark.gpu, needs_gpu]

GOLDEN_CB = os.path.join(os.path.dirname(__file__), "golden", "vq_codebook_256x8.txt")


def codebook():
    return np.loadtxt(GOLDEN_CB, dtype=np.float32).reshape(256, 8)


def ctx_for(H, options=0):
    return kvq.Context(H, 1, mode=kvq.KVQ_MODE_NSN_VQ, vq_codebook=codebook(), nsn_options=options)


def check_dq4(g_codes, g_lo, g_step, r_codes, r_lo, r_step, r_flags, what):
    np.testing.assert_allclose(g_lo, r_lo, rtol=1e-5, atol=1e-6, err_msg=what + " lo")
    np.testing.assert_allclose(g_step, r_step, rtol=1e-5, atol=1e-7, err_msg=what + " step")
    diff = g_codes.astype(int) - r_codes.astype(int)
    assert not (diff != 0)[r_flags == 0].any(), "%s: %d codes differ away from a rounding tie" % (
        what, int(((diff != 0) & (r_flags == 0)).sum()))
    assert np.abs(diff).max() <= 1
    return int((diff != 0).sum())


def check_encoder(x, cb, g, adaptive=False):
    """The GPU's double-quantised encoding of x [H,T,d] against the oracle's."""
    H, T, _ = x.shape
    ref = O.nsn_vq_dq(x, cb, want_z=True, adaptive=adaptive)
    g_oc = O.unpack_nibbles(g["oq"], 128)
    n_o = check_dq4(g_oc, g["op"][:, 0], g["op"][:, 1], ref["o_codes"], ref["o_lo"], ref["o_step"], ref["o_flags"],
                    "means")
    if n_o:
        # a mean code on a rounding tie went the other way: the oracle encodes
        # with that admissible quantised mean (its own lo and step)
        alt = ref["o_lo"][:, None] + g_oc * ref["o_step"][:, None]
        ref = O.nsn_vq_dq(x, cb, want_z=True, adaptive=adaptive, o_hat=alt)
    g_sc = O.unpack_nibbles(g["s1q"], T)
    n_s = check_dq4(g_sc, g["s1p"][..., 0], g["s1p"][..., 1], ref["s1_codes"], ref["s1_lo"], ref["s1_step"],
                    ref["s1_flags"], "s1")
    mism = g["codes"] != ref["codes"]
    assert not (mism & (ref["flags"] == 0)).any(), "VQ codes differ outside the 1e-5 band"
    if mism.any():
        ex = bisector_excess(ref["z"], cb, g["codes"].astype(np.int64), ref["codes"].astype(np.int64))
        assert ex[mism].max() < O.BAND
    assert int(mism.sum()) <= int(ref["flags"].sum()) // 2 + 2
    # with the adaptive scale a boundary flip changes the token's alpha: compare the others
    tok = ~mism.any(-1) if adaptive else np.ones(mism.shape[:-1], bool)
    np.testing.assert_allclose(g["s2"][tok], ref["s2"][tok], rtol=1e-5, atol=1e-6)
    return n_o, n_s, int(mism.sum())


@pytest.mark.parametrize("T", [1, 31, 33, 700, 2049])
def test_nsn_dq_encoder(T):
    x = synth.make("nsn_vq", T=T)["x"]
    ctx = ctx_for(x.shape[0])
    g = {k: to_np(v) for k, v in ctx.nsn_vq_quantize_dq(torch.from_numpy(x).cuda()).items()}
    print("T=%d code differences (means, s1, vq): %s" % (T, check_encoder(x, codebook(), g)))


def test_nsn_dq_encoder_degenerate_tokens():
    """A zero token (s1 = 0) and a block of equal norms (step 0)."""
    x = synth.make("nsn_vq", T=96)["x"]
    x[1, 40] = 0
    x[2, 64:96] = x[2, 64]  # one block of 32 identical tokens: s1 step 0
    ctx = ctx_for(x.shape[0])
    g = {k: to_np(v) for k, v in ctx.nsn_vq_quantize_dq(torch.from_numpy(x).cuda()).items()}
    check_encoder(x, codebook(), g)
    assert g["s1p"][2, 2, 1] == 0
    assert O.unpack_nibbles(g["s1q"], 96)[1, 40] == 0


def test_nsn_dq_codebook_option_and_adaptive_scale():
    """KVQ_NSN_DQ_CODEBOOK: the context encodes with the 4-bit codebook, as the
    oracle does with its own double quantisation of the same entries; with
    the adaptive scale and the 4-bit byproducts on top."""
    x = synth.make("nsn_vq", T=500)["x"]
    # both sides decide the codebook's codes in double with the same formula,
    # so even values near a rounding tie (flagged) get the same code
    c, lo, step, fl, cbh = O.dq_codebook(codebook())
    ctx = ctx_for(x.shape[0], kvq.KVQ_NSN_DQ_CODEBOOK | kvq.KVQ_NSN_ADAPTIVE_SCALE)
    g = {k: to_np(v) for k, v in ctx.nsn_vq_quantize_dq(torch.from_numpy(x).cuda()).items()}
    print(check_encoder(x, cbh, g, adaptive=True))
    ctx2 = ctx_for(x.shape[0], kvq.KVQ_NSN_DQ_CODEBOOK)
    g2 = {k: to_np(v) for k, v in ctx2.nsn_vq_quantize(torch.from_numpy(x).cuda()).items()}
    ref = O.nsn_vq(x, cbh)
    assert not ((g2["codes"] != ref["codes"]) & (ref["flags"] == 0)).any()


def dequant(e):
    """The oracle's reading of 4-bit byproducts: s1 and o as lo + code step."""
    T = e["codes"].shape[-2]
    sc = O.unpack_nibbles(e["s1q"], T).astype(np.float64)
    blk = np.arange(T) // 32
    p = e["s1p"].astype(np.float64)
    s1 = p[..., blk, 0] + sc * p[..., blk, 1]
    oc = O.unpack_nibbles(e["oq"], 128).astype(np.float64)
    op = e["op"].astype(np.float64)
    return s1, op[..., 0:1] + oc * op[..., 1:2]


def oracle_dq_encoded(seed, B, Hkv, T):
    x = synth.random_tensor(seed, (B * Hkv, T, 128)).astype(np.float64)
    x *= np.exp(np.random.default_rng(seed + 1000).standard_normal((B * Hkv, 1, 128)))
    r = O.nsn_vq_dq(x.astype(np.float16), codebook())
    f32 = lambda a: a.astype(np.float32)  # noqa: E731
    return dict(codes=r["codes"].reshape(B, Hkv, T, 16), s1q=r["s1q"].reshape(B, Hkv, -1),
                s1p=f32(np.stack([r["s1_lo"], r["s1_step"]], -1)).reshape(B, Hkv, -1, 2),
                s2=f32(r["s2"]).reshape(B, Hkv, T), oq=r["oq"].reshape(B, Hkv, 64),
                op=f32(np.stack([r["o_lo"], r["o_step"]], -1)).reshape(B, Hkv, 2))


def on_gpu(e):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in e.items()}


@pytest.mark.parametrize("G", [1, 4, 8])
def test_nsn_dq_logits(G):
    B, Hkv, T = 2, 2, 777
    e = oracle_dq_encoded(90, B, Hkv, T)
    q = synth.random_tensor(91, (B, Hkv * G, 128))
    lg = to_np(ctx_for(Hkv).nsn_logits_dq(torch.from_numpy(q).cuda(), on_gpu(e)))
    s1, o = dequant(e)
    ref = O.nsn_logits(q, e["codes"], s1, e["s2"], o, codebook())
    scale = np.linalg.norm(q.astype(np.float64), axis=-1)[..., None] * np.repeat(s1 * np.sqrt(128), G, axis=1)
    err = (np.abs(lg - ref) / np.maximum(scale, 1e-30)).max()
    print("G=%d max rel err %.3g" % (G, err))
    assert err <= 1e-5


@pytest.mark.parametrize("T", [1, 50, 3001])
def test_nsn_dq_decode(T):
    k, v = oracle_dq_encoded(92, 1, 8, T), oracle_dq_encoded(93, 1, 8, T)
    q = synth.random_tensor(94, (1, 32, 128))
    ctx = ctx_for(8)
    got = to_np(ctx.nsn_attn_decode_dq(torch.from_numpy(q).cuda(), on_gpu(k), on_gpu(v)))
    ks1, ko = dequant(k)
    vs1, vo = dequant(v)
    want = O.nsn_attention(q, k["codes"], ks1, k["s2"], ko, v["codes"], vs1, v["s2"], vo, codebook())
    err = np.abs(got - want).max()
    print("T=%d max abs err %.3g" % (T, err))
    assert err <= 2e-3


def test_nsn_dq_decode_full_size_and_splits():
    """8 KV heads x 65536 tokens drawn by the seeded generator, 32 query heads;
    every output checked; split counts agree."""
    k = synth.random_nsn_dq_codes(95, (1, 8, 65536))
    v = synth.random_nsn_dq_codes(96, (1, 8, 65536))
    q = synth.random_tensor(97, (1, 32, 128))
    ctx = ctx_for(8)
    kg, vg, qg = on_gpu(k), on_gpu(v), torch.from_numpy(q).cuda()
    got = to_np(ctx.nsn_attn_decode_dq(qg, kg, vg))
    ks1, ko = dequant(k)
    vs1, vo = dequant(v)
    want = O.nsn_attention(q, k["codes"], ks1, k["s2"], ko, v["codes"], vs1, v["s2"], vo, codebook())
    err = np.abs(got - want).max()
    print("full size max abs err %.3g" % err)
    assert err <= 2e-3
    for n in (1, 7, 100000):
        np.testing.assert_allclose(to_np(ctx.nsn_attn_decode_dq(qg, kg, vg, n_split=n)), got, rtol=1e-4, atol=1e-5)


def test_nsn_dq_encode_then_decode():
    """The GPU encodes K and V with double quantisation and decodes; the oracle
    decodes its own encoding of the same tokens."""
    Hkv, T = 2, 640
    xk = synth.make("nsn_vq", T=T)["x"][:Hkv]
    xv = synth.make("nsn_vq", T=T)["x"][Hkv:2 * Hkv]
    ctx = ctx_for(Hkv)
    kg = ctx.nsn_vq_quantize_dq(torch.from_numpy(np.ascontiguousarray(xk)).cuda())
    vg = ctx.nsn_vq_quantize_dq(torch.from_numpy(np.ascontiguousarray(xv)).cuda())
    lead = lambda e: {n: t.unsqueeze(0) for n, t in e.items()}  # noqa: E731
    q = synth.random_tensor(98, (1, 4 * Hkv, 128))
    got = to_np(ctx.nsn_attn_decode_dq(torch.from_numpy(q).cuda(), lead(kg), lead(vg)))
    rk, rv = O.nsn_vq_dq(xk, codebook()), O.nsn_vq_dq(xv, codebook())
    want = O.nsn_attention(q, rk["codes"][None], rk["s1_hat"][None], rk["s2"][None], rk["o_hat"][None],
                           rv["codes"][None], rv["s1_hat"][None], rv["s2"][None], rv["o_hat"][None], codebook())
    err = np.abs(got - want).max()
    print("max abs err %.3g" % err)
    assert err <= 2e-3
