"""GPU parity of gain-shape residual quantisation (GSRQ page: gain-shape
k-means stages in a residual quantisation pipeline, below 1 bit per element;
read as two stages of 256 unit shapes and 16 gain levels over 32-dim
sub-vectors of the NSN-normalised rotated vector) against the CPU oracle.

Encoder: s1, s2, o within 1e-5; per sub-vector the shape and gain indices of
both stages exact except decisions the oracle flags as within 1e-5 of a tie
(a flagged stage-1 decision taken the other way changes stage 2, which is
then not compared); a differing flagged shape must project within 1e-5 of the
oracle's.  Scoring: both sides read records written by the oracle's encoder
or drawn by the seeded generator.  No GPU output feeds the oracle."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gsrq_tables_256x32.txt")


def tables():
    lines = [ln.split() for ln in open(GOLDEN) if not ln.startswith("#")]
    return dict(S1=np.array(lines[0:256], dtype=np.float32), G1=np.array(lines[256], dtype=np.float32),
                S2=np.array(lines[257:513], dtype=np.float32), G2=np.array(lines[513], dtype=np.float32))


def ctx_for(H):
    return kvq.Context(H, 1, mode=kvq.KVQ_MODE_GSRQ, gsrq_tables=tables())


def split(rec):
    """records [..., 12] -> (j1, j2, c1, c2) [..., 4]"""
    return rec[..., 0:4], rec[..., 4:8], rec[..., 8:12] & 15, rec[..., 8:12] >> 4


def check_codes(z, got, ref, flags, tab):
    """Compare the GPU's records with the oracle's (both [n, 12]) for the oracle's
    rotated vectors z [n, 128] and flags [n, 4]."""
    gj1, gj2, gc1, gc2 = split(got)
    rj1, rj2, rc1, rc2 = split(ref)
    f1 = (flags & 3) != 0   # a stage-1 decision near a tie
    f2 = (flags & 12) != 0
    s1_diff = (gj1 != rj1) | (gc1 != rc1)
    assert not (s1_diff & ~f1).any(), "%d stage-1 decisions differ away from a tie" % int((s1_diff & ~f1).sum())
    zs = z.reshape(-1, 4, 32).astype(np.float64)
    S1 = tab["S1"].astype(np.float64)
    for n, sv in zip(*np.nonzero(gj1 != rj1)):
        pg, pr = zs[n, sv] @ S1[gj1[n, sv]], zs[n, sv] @ S1[rj1[n, sv]]
        assert pr - pg < O.BAND, ("GPU shape projects farther than the band from the best", pr - pg)
    s2_diff = ((gj2 != rj2) | (gc2 != rc2)) & ~s1_diff
    assert not (s2_diff & ~f2).any(), "%d stage-2 decisions differ away from a tie" % int((s2_diff & ~f2).sum())
    n_diff = int((s1_diff | s2_diff).sum())
    assert n_diff <= int((f1 | f2).sum()) // 2 + 2
    return n_diff, int((f1 | f2).sum())


@pytest.mark.parametrize("T", [1, 63, 700, 2049])
def test_gsrq_encoder(T):
    x = synth.make("nsn_vq", T=T)["x"]
    tab = tables()
    g = {k: to_np(v) for k, v in ctx_for(x.shape[0]).gsrq_quantize(torch.from_numpy(x).cuda()).items()}
    ref = O.gsrq_vq(x, tab)
    np.testing.assert_allclose(g["o"], ref["o"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(g["s1"], ref["s1"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(g["s2"], ref["s2"], rtol=1e-5, atol=1e-6)
    print("T=%d code differences / flagged: %s" % (T, check_codes(ref["z"].reshape(-1, 128), g["codes"].reshape(-1, 12),
                                                                 ref["codes"].reshape(-1, 12),
                                                                 ref["flags"].reshape(-1, 4), tab)))


def test_gsrq_encoder_degenerate_tokens():
    x = synth.make("nsn_vq", T=80)["x"]
    x[1, 3] = 0
    tab = tables()
    g = {k: to_np(v) for k, v in ctx_for(x.shape[0]).gsrq_quantize(torch.from_numpy(x).cuda()).items()}
    ref = O.gsrq_vq(x, tab)
    assert g["s1"][1, 3] == 0
    check_codes(ref["z"].reshape(-1, 128), g["codes"].reshape(-1, 12), ref["codes"].reshape(-1, 12),
                ref["flags"].reshape(-1, 4), tab)


def test_gsrq_encoder_full_size_sampled():
    x = synth.make("nsn_vq")["x"]
    tab = tables()
    g = {k: to_np(v) for k, v in ctx_for(8).gsrq_quantize(torch.from_numpy(x).cuda()).items()}
    a = x.astype(np.float64)
    nx = np.linalg.norm(a, axis=-1, keepdims=True)
    o_ref = (np.sqrt(128) * a / np.where(nx > 0, nx, 1)).mean(axis=1)
    np.testing.assert_allclose(g["o"], o_ref, rtol=1e-5, atol=1e-6)
    t_sel = np.random.default_rng(3).choice(x.shape[1], 512, replace=False)
    ref = O.gsrq_vq(x[:, t_sel], tab, o_given=o_ref)
    np.testing.assert_allclose(g["s2"][:, t_sel], ref["s2"], rtol=1e-5, atol=1e-6)
    print(check_codes(ref["z"].reshape(-1, 128), g["codes"][:, t_sel].reshape(-1, 12), ref["codes"].reshape(-1, 12),
                      ref["flags"].reshape(-1, 4), tab))


def oracle_encoded(seed, B, Hkv, T):
    x = synth.random_tensor(seed, (B * Hkv, T, 128)).astype(np.float64)
    x *= np.exp(np.random.default_rng(seed + 1000).standard_normal((B * Hkv, 1, 128)))
    r = O.gsrq_vq(x.astype(np.float16), tables())
    f32 = lambda a: a.astype(np.float32)  # noqa: E731
    return dict(codes=r["codes"].reshape(B, Hkv, T, 12), s1=f32(r["s1"]).reshape(B, Hkv, T),
                s2=f32(r["s2"]).reshape(B, Hkv, T), o=f32(r["o"]).reshape(B, Hkv, 128))


def on_gpu(e):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in e.items()}


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gsrq_logits(G):
    B, Hkv, T = 2, 2, 777
    e = oracle_encoded(100, B, Hkv, T)
    q = synth.random_tensor(101, (B, Hkv * G, 128))
    ge = on_gpu(e)
    lg = to_np(ctx_for(Hkv).gsrq_logits(torch.from_numpy(q).cuda(), ge["codes"], ge["s1"], ge["s2"], ge["o"]))
    ref = O.gsrq_logits(q, e["codes"], e["s1"], e["s2"], e["o"], tables())
    scale = np.linalg.norm(q.astype(np.float64), axis=-1)[..., None] * np.repeat(
        e["s1"].astype(np.float64) * np.sqrt(128), G, axis=1)
    err = (np.abs(lg - ref) / np.maximum(scale, 1e-30)).max()
    print("G=%d max rel err %.3g" % (G, err))
    assert err <= 1e-5


def decode_ref(q, k, v, sm_scale=None):
    return O.gsrq_attention(q, k["codes"], k["s1"], k["s2"], k["o"], v["codes"], v["s1"], v["s2"], v["o"], tables(),
                            sm_scale=sm_scale)


@pytest.mark.parametrize("G,T", [(4, 1), (4, 50), (1, 1000), (2, 3001), (4, 3001)])
def test_gsrq_decode(G, T):
    Hkv = 4
    k, v = oracle_encoded(102, 1, Hkv, T), oracle_encoded(103, 1, Hkv, T)
    q = synth.random_tensor(104, (1, Hkv * G, 128))
    got = to_np(ctx_for(Hkv).gsrq_attn_decode(torch.from_numpy(q).cuda(), on_gpu(k), on_gpu(v)))
    err = np.abs(got - decode_ref(q, k, v)).max()
    print("G=%d T=%d max abs err %.3g" % (G, T, err))
    assert err <= 2e-3


def test_gsrq_decode_full_size_and_splits():
    """8 KV heads x 65536 tokens of stand-in records, 32 query heads; every
    output checked; split counts agree; a larger softmax scale."""
    k = synth.random_gsrq_codes(105, (1, 8, 65536))
    v = synth.random_gsrq_codes(106, (1, 8, 65536))
    q = synth.random_tensor(107, (1, 32, 128))
    ctx = ctx_for(8)
    kg, vg, qg = on_gpu(k), on_gpu(v), torch.from_numpy(q).cuda()
    got = to_np(ctx.gsrq_attn_decode(qg, kg, vg))
    err = np.abs(got - decode_ref(q, k, v)).max()
    print("full size max abs err %.3g" % err)
    assert err <= 2e-3
    for n in (1, 7, 100000):
        np.testing.assert_allclose(to_np(ctx.gsrq_attn_decode(qg, kg, vg, n_split=n)), got, rtol=1e-4, atol=1e-5)
    got = to_np(ctx.gsrq_attn_decode(qg, kg, vg, sm_scale=0.5))
    assert np.abs(got - decode_ref(q, k, v, sm_scale=0.5)).max() <= 2e-3


def test_gsrq_encode_then_decode():
    Hkv, T = 2, 640
    xk = np.ascontiguousarray(synth.make("nsn_vq", T=T)["x"][:Hkv])
    xv = np.ascontiguousarray(synth.make("nsn_vq", T=T)["x"][Hkv:2 * Hkv])
    ctx = ctx_for(Hkv)
    kg = {n: t.unsqueeze(0) for n, t in ctx.gsrq_quantize(torch.from_numpy(xk).cuda()).items()}
    vg = {n: t.unsqueeze(0) for n, t in ctx.gsrq_quantize(torch.from_numpy(xv).cuda()).items()}
    q = synth.random_tensor(108, (1, 4 * Hkv, 128))
    got = to_np(ctx.gsrq_attn_decode(torch.from_numpy(q).cuda(), kg, vg))
    rk, rv = O.gsrq_vq(xk, tables()), O.gsrq_vq(xv, tables())
    want = O.gsrq_attention(q, rk["codes"][None], rk["s1"][None], rk["s2"][None], rk["o"][None], rv["codes"][None],
                            rv["s1"][None], rv["s2"][None], rv["o"][None], tables())
    err = np.abs(got - want).max()
    print("max abs err %.3g" % err)
    assert err <= 2e-3
