"""GPU parity of kvq_logits and kvq_attn_decode against the CPU oracle.

Both sides score the SAME packed codes and fp32 norms, written by the
oracle's quantizer (the GPU consumes them), so decision-boundary flips in
quantisation cannot leak into these tolerances: logits within
1e-3 * ||q|| ||k||, attention outputs within 2e-3 max-abs."""
import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def oracle_codes(x, signs, bits):
    """Packed codes and fp32 norms from the oracle's quantizer, on the GPU."""
    r = O.quantize(x, signs, bits)
    return dict(codes=torch.from_numpy(r["codes"]).cuda(),
                norms=torch.from_numpy(r["norms"].astype(np.float32)).cuda())


def quantized(name, bits, T=None, B=None):
    inp = synth.make(name, T=T, B=B)
    ctx = kvq.Context(inp["Hkv"], bits, inp["signs_k"], inp["signs_v"])
    k = oracle_codes(inp["k"], inp["signs_k"], bits)
    v = oracle_codes(inp["v"], inp["signs_v"], bits) if "v" in inp else None
    return inp, ctx, k, v


def check_logits(inp, ctx, k, bits, label):
    q = torch.from_numpy(inp["q"]).cuda()
    lg = to_np(ctx.logits(q, k["codes"], k["norms"]))
    codes, norms = to_np(k["codes"]), to_np(k["norms"]).astype(np.float64)
    ref = O.logits(inp["q"], codes, norms, inp["signs_k"], bits)
    G = inp["Hq"] // inp["Hkv"]
    scale = (np.linalg.norm(inp["q"].astype(np.float64), axis=-1)[..., None] *
             np.repeat(norms, G, axis=1))
    err = np.abs(lg - ref) / np.maximum(scale, 1e-30)
    assert err.max() <= 1e-3, (label, err.max())
    assert err.max() <= 1e-5, (label, "fp32-level agreement expected", err.max())
    return err.max()


def test_logits_tiny_full():
    inp, ctx, k, _ = quantized("tiny", 3)
    print("tiny logits max rel err", check_logits(inp, ctx, k, 3, "tiny"))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_logits_gqa_ragged(bits):
    inp, ctx, k, _ = quantized("l8b32k", bits, T=777, B=2)
    check_logits(inp, ctx, k, bits, "l8b32k T=777 B=2")


def decode_ref(inp, k, v, bits, b_sel=None):
    kc, kn = to_np(k["codes"]), to_np(k["norms"]).astype(np.float64)
    vc, vn = to_np(v["codes"]), to_np(v["norms"]).astype(np.float64)
    q = inp["q"]
    if b_sel is not None:
        kc, kn, vc, vn, q = kc[b_sel], kn[b_sel], vc[b_sel], vn[b_sel], q[b_sel]
    return O.attention(q, kc, kn, vc, vn, inp["signs_k"], inp["signs_v"], bits)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("T", [1, 50, 1000, 3001])
def test_decode_ragged(bits, T):
    inp, ctx, k, v = quantized("l8b32k", bits, T=T)
    out = to_np(ctx.attn_decode(torch.from_numpy(inp["q"]).cuda(), k["codes"], k["norms"], v["codes"], v["norms"]))
    ref = decode_ref(inp, k, v, bits)
    err = np.abs(out - ref).max()
    assert err <= 2e-3, (bits, T, err)


def test_decode_l8b32k_full_size():
    for bits in (2, 3, 4):
        inp, ctx, k, v = quantized("l8b32k", bits)
        out = to_np(ctx.attn_decode(torch.from_numpy(inp["q"]).cuda(), k["codes"], k["norms"], v["codes"],
                                    v["norms"]))
        err = np.abs(out - decode_ref(inp, k, v, bits)).max()
        print("l8b32k full decode b=%d max abs err %.3g" % (bits, err))
        assert err <= 2e-3


def test_decode_batch16_full_size_sampled():
    inp, ctx, k, v = quantized("batch16", 3)
    out = to_np(ctx.attn_decode(torch.from_numpy(inp["q"]).cuda(), k["codes"], k["norms"], v["codes"], v["norms"]))
    sel = np.array([0, 7, 15])
    ref = decode_ref(inp, k, v, 3, b_sel=sel)
    err = np.abs(out[sel] - ref).max()
    print("batch16 decode max abs err %.3g" % err)
    assert err <= 2e-3


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_decode_several_tiles_per_wave(bits):
    """One split per (batch, KV head): each wave of the block runs several
    64-token tiles (the next tile's records loaded while the current one is
    scored), the last one ragged."""
    inp, ctx, k, v = quantized("l8b32k", bits, T=3001)
    out = to_np(ctx.attn_decode(torch.from_numpy(inp["q"]).cuda(), k["codes"], k["norms"], v["codes"], v["norms"],
                                n_split=1))
    err = np.abs(out - decode_ref(inp, k, v, bits)).max()
    assert err <= 2e-3, (bits, err)


def test_decode_split_invariance():
    inp, ctx, k, v = quantized("l8b32k", 3, T=5000)
    q = torch.from_numpy(inp["q"]).cuda()
    outs = [to_np(ctx.attn_decode(q, k["codes"], k["norms"], v["codes"], v["norms"], n_split=n))
            for n in (1, 2, 7, 64)]
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-4, atol=1e-5)


def test_decode_zero_query_is_mean_value():
    inp, ctx, k, v = quantized("l8b32k", 3, T=300)
    inp["q"] = np.zeros_like(inp["q"])
    out = to_np(ctx.attn_decode(torch.from_numpy(inp["q"]).cuda(), k["codes"], k["norms"], v["codes"], v["norms"]))
    np.testing.assert_allclose(out, decode_ref(inp, k, v, 3), atol=2e-3)


def test_decode_workspace_reuse_and_too_small():
    inp, ctx, k, v = quantized("l8b32k", 2, T=700)
    q = torch.from_numpy(inp["q"]).cuda()
    ws = ctx.decode_ws(1, 32, 700)
    a = to_np(ctx.attn_decode(q, k["codes"], k["norms"], v["codes"], v["norms"], ws=ws))
    b = to_np(ctx.attn_decode(q, k["codes"], k["norms"], v["codes"], v["norms"], ws=ws))
    assert np.array_equal(a, b)  # counters were left at zero by the first call
    with pytest.raises(kvq.KvqError) as e:
        ctx.attn_decode(q, k["codes"], k["norms"], v["codes"], v["norms"], ws=ws[:16])
    assert e.value.status == kvq.KVQ_E_WORKSPACE


def test_decode_split_request_is_clamped():
    """More splits than 512 (or than 64-token chunks) are clamped, not overrun."""
    inp, ctx, k, v = quantized("l8b32k", 2, T=33000)
    q = torch.from_numpy(inp["q"]).cuda()
    ref = to_np(ctx.attn_decode(q, k["codes"], k["norms"], v["codes"], v["norms"]))
    big = to_np(ctx.attn_decode(q, k["codes"], k["norms"], v["codes"], v["norms"], n_split=100000))
    np.testing.assert_allclose(big, ref, rtol=1e-4, atol=1e-5)


def test_group_sizes_without_kernels_are_rejected_on_the_host():
    """Decode is built for 1, 2 and 4 query heads per KV head, logits for 1, 2,
    4 and 8: other divisible ratios are KVQ_E_UNSUPPORTED (nothing launched),
    a ratio that does not divide is KVQ_E_INVAL."""
    inp, ctx, k, v = quantized("l8b32k", 3, T=100)
    args = (k["codes"], k["norms"], v["codes"], v["norms"])
    for hq, status in ((24, kvq.KVQ_E_UNSUPPORTED), (64, kvq.KVQ_E_UNSUPPORTED), (12, kvq.KVQ_E_INVAL)):
        q = torch.zeros((1, hq, 128), dtype=torch.float16, device="cuda")
        with pytest.raises(kvq.KvqError) as e:
            ctx.attn_decode(q, *args)
        assert e.value.status == status, hq
    for hq, status in ((24, kvq.KVQ_E_UNSUPPORTED), (40, kvq.KVQ_E_UNSUPPORTED), (12, kvq.KVQ_E_INVAL)):
        q = torch.zeros((1, hq, 128), dtype=torch.float16, device="cuda")
        with pytest.raises(kvq.KvqError) as e:
            ctx.logits(q, k["codes"], k["norms"])
        assert e.value.status == status, hq
    q8 = torch.from_numpy(np.repeat(inp["q"], 2, axis=1)).cuda()  # 64 query heads: 8 per KV head
    lg = to_np(ctx.logits(q8, k["codes"], k["norms"]))
    np.testing.assert_array_equal(lg[:, 0::2], lg[:, 1::2])
