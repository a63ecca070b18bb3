"""GPU parity of the streaming NSN-VQ cache (kvq_nsn_flush,
kvq_nsn_attn_decode_stream) against the CPU oracle.

NSNQuant page, Detalhes de Implementacao: recent tokens stay in a
full-precision window that is quantised when it fills (as in KIVI); each flush
of Gs tokens is one NSN-VQ encoding with its own channel means.  Decode
inputs are written by the oracle's encoder (small cases) or drawn by the
seeded generator (full size); both sides read the same codes, fp32
byproducts and fp16 window.  No GPU output feeds the oracle.  Attention
outputs within 2e-3 max-abs; flushed codes exact except sub-vectors within
1e-5 of a bisecting hyperplane."""
import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import needs_gpu, to_np
from tests.test_gpu_nsn import compare
from tests.test_gpu_nsn_scores import codebook, ctx_for, on_gpu, query

pytestmark = [pytest.mark.gpu, needs_gpu]


def raw_tokens(seed, B, Hkv, T):
    """fp16 tokens with lognormal per-channel scales (outlier channels)."""
    x = synth.random_tensor(seed, (B, Hkv, T, 128)).astype(np.float64)
    x *= np.exp(np.random.default_rng(seed + 1000).standard_normal((B, Hkv, 1, 128)))
    return x.astype(np.float16)


def encode_groups(x, Gs, T_cap):
    """The oracle's encoding of x [B, Hkv, T, d] in flush groups of Gs tokens,
    byproducts rounded to fp32, in arrays of capacity T_cap."""
    B, Hkv, T, d = x.shape
    out = dict(codes=np.zeros((B, Hkv, T_cap, 16), np.uint8), s1=np.zeros((B, Hkv, T_cap), np.float32),
               s2=np.zeros((B, Hkv, T_cap), np.float32), o=np.zeros((B, Hkv, T_cap // Gs, d), np.float32))
    for g in range(T // Gs):
        r = O.nsn_vq(x[:, :, g * Gs:(g + 1) * Gs].reshape(B * Hkv, Gs, d), codebook())
        sl = slice(g * Gs, (g + 1) * Gs)
        out["codes"][:, :, sl] = r["codes"].reshape(B, Hkv, Gs, 16)
        out["s1"][:, :, sl] = r["s1"].reshape(B, Hkv, Gs)
        out["s2"][:, :, sl] = r["s2"].reshape(B, Hkv, Gs)
        out["o"][:, :, g] = r["o"].reshape(B, Hkv, d)
    return out


def reference(q, k, v, T, Gs, kt, vt, R, sm_scale=None):
    sub = lambda e: {n: (a[:, :, :T // Gs] if n == "o" else a[:, :, :T]) for n, a in e.items()}  # noqa: E731
    ks, vs = sub(k), sub(v)
    return O.nsn_attention_stream(q, ks["codes"], ks["s1"], ks["s2"], ks["o"], vs["codes"], vs["s1"], vs["s2"],
                                  vs["o"], kt[:, :, :R], vt[:, :, :R], codebook(), Gs, sm_scale=sm_scale)


def gpu_decode(ctx, q, k, v, T, Gs, kt, vt, R, **kw):
    return to_np(ctx.nsn_attn_decode_stream(torch.from_numpy(q).cuda(), on_gpu(k), on_gpu(v), T, Gs,
                                            torch.from_numpy(kt).cuda(), torch.from_numpy(vt).cuda(), R, **kw))


@pytest.mark.parametrize("G,T,R", [(4, 0, 70), (4, 128, 0), (1, 640, 128), (2, 1280, 1), (4, 1280, 100)])
def test_nsn_stream_decode(G, T, R):
    B, Hkv, Gs, R_cap = 2, 2, 128, 192
    T_cap = T + 2 * Gs
    k = encode_groups(raw_tokens(30, B, Hkv, T), Gs, T_cap)
    v = encode_groups(raw_tokens(31, B, Hkv, T), Gs, T_cap)
    kt, vt = raw_tokens(32, B, Hkv, R_cap), raw_tokens(33, B, Hkv, R_cap)
    q = query(34, B, Hkv * G)
    got = gpu_decode(ctx_for(Hkv), q, k, v, T, Gs, kt, vt, R)
    err = np.abs(got - reference(q, k, v, T, Gs, kt, vt, R)).max()
    print("G=%d T=%d R=%d max abs err %.3g" % (G, T, R, err))
    assert err <= 2e-3


def test_nsn_stream_split_cap_and_invariance():
    """40 groups of 64 tokens: a split holds at most 32 groups, so one
    requested split becomes two; every split count gives the same output."""
    B, Hkv, Gs, T, R = 1, 2, 64, 40 * 64, 30
    k = encode_groups(raw_tokens(40, B, Hkv, T), Gs, T)
    v = encode_groups(raw_tokens(41, B, Hkv, T), Gs, T)
    kt, vt = raw_tokens(42, B, Hkv, 64), raw_tokens(43, B, Hkv, 64)
    q = query(44, B, Hkv * 4)
    ctx = ctx_for(Hkv)
    outs = [gpu_decode(ctx, q, k, v, T, Gs, kt, vt, R, n_split=n) for n in (1, 3, 7, 100000)]
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-4, atol=1e-5)
    assert np.abs(outs[0] - reference(q, k, v, T, Gs, kt, vt, R)).max() <= 2e-3
    got = gpu_decode(ctx, q, k, v, T, Gs, kt, vt, R, sm_scale=0.3)
    assert np.abs(got - reference(q, k, v, T, Gs, kt, vt, R, sm_scale=0.3)).max() <= 2e-3


def test_nsn_stream_full_size():
    """8 KV heads x 65536 packed tokens in 512 groups of 128, a window of 100,
    32 query heads; every output checked."""
    B, Hkv, Gs, T, R = 1, 8, 128, 65536, 100
    k = synth.random_nsn_codes(50, (B, Hkv, T), n_groups=T // Gs)
    v = synth.random_nsn_codes(51, (B, Hkv, T), n_groups=T // Gs)
    kt, vt = raw_tokens(52, B, Hkv, 128), raw_tokens(53, B, Hkv, 128)
    q = query(54, B, Hkv * 4)
    got = gpu_decode(ctx_for(Hkv), q, k, v, T, Gs, kt, vt, R)
    err = np.abs(got - reference(q, k, v, T, Gs, kt, vt, R)).max()
    print("full size max abs err %.3g" % err)
    assert err <= 2e-3


def test_nsn_flush_parity_and_untouched_positions():
    B, Hkv, Gs, R_cap, T_cap, T0 = 2, 2, 128, 192, 512, 256
    kt, vt = raw_tokens(60, B, Hkv, R_cap), raw_tokens(61, B, Hkv, R_cap)
    ctx = ctx_for(Hkv)
    k, v = ctx.nsn_stream_alloc(B, T_cap, Gs)
    for e in (k, v):
        e["codes"].fill_(0xAB)
        e["s1"].fill_(-1.0)
        e["s2"].fill_(-2.0)
        e["o"].fill_(-7.0)
    ctx.nsn_flush(torch.from_numpy(kt).cuda(), torch.from_numpy(vt).cuda(), Gs, k, v, T0)
    torch.cuda.synchronize()
    g = T0 // Gs
    for e, x in ((k, kt), (v, vt)):
        h = {n: to_np(a) for n, a in e.items()}
        xs = x[:, :, :Gs].reshape(B * Hkv, Gs, 128)
        got = dict(codes=h["codes"][:, :, T0:T0 + Gs].reshape(B * Hkv, Gs, 16),
                   s1=h["s1"][:, :, T0:T0 + Gs].reshape(B * Hkv, Gs),
                   s2=h["s2"][:, :, T0:T0 + Gs].reshape(B * Hkv, Gs))
        print(compare(xs, codebook(), got))
        np.testing.assert_allclose(h["o"][:, :, g].reshape(B * Hkv, 128), O.nsn_vq(xs, codebook())["o"], rtol=1e-5,
                                   atol=1e-6)
        rest = np.ones(T_cap, bool)
        rest[T0:T0 + Gs] = False
        assert np.all(h["codes"][:, :, rest] == 0xAB)
        assert np.all(h["s1"][:, :, rest] == -1.0) and np.all(h["s2"][:, :, rest] == -2.0)
        other = np.arange(T_cap // Gs) != g
        assert np.all(h["o"][:, :, other] == -7.0)


def test_nsn_stream_flushes_then_decode():
    """Three windows flushed one after another, then a decode step with a
    partly filled window: the GPU's own encodings against the oracle's
    encodings of the same tokens."""
    B, Hkv, Gs, R_cap, T_cap, G = 1, 2, 128, 128, 512, 4
    ctx = ctx_for(Hkv)
    k, v = ctx.nsn_stream_alloc(B, T_cap, Gs)
    raw_k = raw_tokens(70, B, Hkv, 3 * Gs)
    raw_v = raw_tokens(71, B, Hkv, 3 * Gs)
    for f in range(3):
        wk = torch.from_numpy(np.ascontiguousarray(raw_k[:, :, f * Gs:(f + 1) * Gs])).cuda()
        wv = torch.from_numpy(np.ascontiguousarray(raw_v[:, :, f * Gs:(f + 1) * Gs])).cuda()
        ctx.nsn_flush(wk, wv, Gs, k, v, f * Gs)
    kt, vt = raw_tokens(72, B, Hkv, R_cap), raw_tokens(73, B, Hkv, R_cap)
    q = query(74, B, Hkv * G)
    got = to_np(ctx.nsn_attn_decode_stream(torch.from_numpy(q).cuda(), k, v, 3 * Gs, Gs, torch.from_numpy(kt).cuda(),
                                           torch.from_numpy(vt).cuda(), 50))
    ko, vo = encode_groups(raw_k, Gs, T_cap), encode_groups(raw_v, Gs, T_cap)
    # codes of the GPU flushes: exact but for boundary sub-vectors
    mism = sum(int((to_np(e["codes"])[:, :, :3 * Gs] != r["codes"][:, :, :3 * Gs]).sum()) for e, r in ((k, ko), (v, vo)))
    print("boundary code differences", mism)
    assert mism <= 8
    err = np.abs(got - reference(q, ko, vo, 3 * Gs, Gs, kt, vt, 50)).max()
    print("max abs err %.3g" % err)
    assert err <= 2e-3


def test_nsn_stream_validation():
    ctx = ctx_for(2)
    k, v = ctx.nsn_stream_alloc(1, 256, 128)
    q = torch.from_numpy(query(80, 1, 8)).cuda()
    w = torch.zeros((1, 2, 128, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:  # T not a multiple of the group size
        ctx.nsn_attn_decode_stream(q, k, v, 100, 128, w, w, 10)
    assert e.value.status == kvq.KVQ_E_INVAL
    with pytest.raises(kvq.KvqError):  # group size not a multiple of 64
        ctx.nsn_flush(w, w, 96, k, v, 0)
    with pytest.raises(kvq.KvqError):  # 8 query heads per KV head
        ctx.nsn_attn_decode_stream(torch.from_numpy(query(81, 1, 16)).cuda(), k, v, 128, 128, w, w, 10)
