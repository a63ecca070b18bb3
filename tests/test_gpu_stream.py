"""GPU parity of the streaming cache (kvq_attn_decode_stream, kvq_flush)
against the CPU oracle: a quantised prefix held in arrays with spare
capacity, followed by a full-precision residual window.

Decode scores codes and fp32 norms written by the oracle's quantizer (the
unused capacity holds random bytes, which must not be read); attention
outputs within 2e-3 max-abs.  Flush is compared with the oracle's encoding
of the window: exact indices except coordinates within 1e-5 of a threshold,
norms to 1e-5, and every other position of the packed arrays untouched."""
import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import bound_mismatches, boundary_mismatches, needs_gpu, to_np, unpack_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def cache(seed, bits, B, Hkv, T, T_cap, R, R_cap, Hq):
    """Packed prefix (oracle codes, random bytes past T) and fp16 windows
    (random rows past R); returns (inp, device arrays, host arrays)."""
    inp = synth.make("l8b32k", T=max(T, 1), B=B)
    inp = dict(k=inp["k"][:, :Hkv], v=inp["v"][:, :Hkv], signs_k=inp["signs_k"][:Hkv], signs_v=inp["signs_v"][:Hkv])
    rng = np.random.default_rng(seed)
    rec = 16 * bits
    kc = rng.integers(0, 256, size=(B, Hkv, T_cap, rec), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(B, Hkv, T_cap, rec), dtype=np.uint8)
    kn = rng.uniform(1, 2, size=(B, Hkv, T_cap)).astype(np.float32)
    vn = rng.uniform(1, 2, size=(B, Hkv, T_cap)).astype(np.float32)
    if T > 0:
        rk = O.quantize(inp["k"][:, :, :T], inp["signs_k"], bits)
        rv = O.quantize(inp["v"][:, :, :T], inp["signs_v"], bits)
        kc[:, :, :T], vc[:, :, :T] = rk["codes"], rv["codes"]
        kn[:, :, :T], vn[:, :, :T] = rk["norms"], rv["norms"]
    kt = synth.random_tensor(seed + 1, (B, Hkv, R_cap, 128), scale=2.0)
    vt = synth.random_tensor(seed + 2, (B, Hkv, R_cap, 128), scale=2.0)
    q = synth.random_tensor(seed + 3, (B, Hq, 128))
    host = dict(kc=kc, vc=vc, kn=kn, vn=vn, kt=kt, vt=vt, q=q)
    dev = {k: torch.from_numpy(v).cuda() for k, v in host.items()}
    return inp, dev, host


def run_case(bits, B, Hkv, Hq, T, T_cap, R, R_cap, seed=1, sm_scale=None):
    inp, d, h = cache(seed, bits, B, Hkv, T, T_cap, R, R_cap, Hq)
    ctx = kvq.Context(Hkv, bits, inp["signs_k"], inp["signs_v"])
    out = to_np(ctx.attn_decode_stream(d["q"], d["kc"], d["kn"], d["vc"], d["vn"], T, d["kt"], d["vt"], R,
                                       sm_scale=sm_scale or 0.0))
    ref = O.attention_stream(h["q"], h["kc"][:, :, :T], h["kn"][:, :, :T].astype(np.float64), h["vc"][:, :, :T],
                             h["vn"][:, :, :T].astype(np.float64), h["kt"][:, :, :R], h["vt"][:, :, :R],
                             inp["signs_k"], inp["signs_v"], bits, sm_scale=sm_scale)
    return np.abs(out - ref).max()


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("T,R", [(0, 1), (0, 100), (1, 0), (300, 64), (3001, 128), (5000, 1)])
def test_stream_decode(bits, T, R):
    err = run_case(bits, 1, 8, 32, T, T + 77, R, R + 13)
    print("b=%d T=%d R=%d max abs err %.3g" % (bits, T, R, err))
    assert err <= 2e-3


@pytest.mark.parametrize("G", [1, 2])
def test_stream_decode_groups_batch_scale(G):
    assert run_case(3, 2, 4, 4 * G, 2000, 2048, 70, 128, seed=5, sm_scale=0.3) <= 2e-3


def test_stream_decode_full_size():
    """32704 quantised tokens (of 32768 slots) and a 64-token window, 8 KV
    heads, 32 query heads: the decode workload with its residual."""
    err = run_case(3, 1, 8, 32, 32704, 32768, 64, 128, seed=7)
    print("full size max abs err %.3g" % err)
    assert err <= 2e-3


def test_stream_decode_workspace_reuse_and_validation():
    inp, d, h = cache(9, 3, 1, 8, 500, 600, 20, 32, 32)
    ctx = kvq.Context(8, 3, inp["signs_k"], inp["signs_v"])
    ws = ctx.stream_ws(1, 32, 600)
    a = to_np(ctx.attn_decode_stream(d["q"], d["kc"], d["kn"], d["vc"], d["vn"], 500, d["kt"], d["vt"], 20, ws=ws))
    b = to_np(ctx.attn_decode_stream(d["q"], d["kc"], d["kn"], d["vc"], d["vn"], 500, d["kt"], d["vt"], 20, ws=ws))
    assert np.array_equal(a, b)
    for T, R in ((601, 0), (500, 33), (0, 0), (-1, 5)):
        with pytest.raises(kvq.KvqError) as e:
            ctx.attn_decode_stream(d["q"], d["kc"], d["kn"], d["vc"], d["vn"], T, d["kt"], d["vt"], R, ws=ws)
        assert e.value.status == kvq.KVQ_E_INVAL, (T, R)
    with pytest.raises(kvq.KvqError) as e:
        ctx.attn_decode_stream(d["q"], d["kc"], d["kn"], d["vc"], d["vn"], 500, d["kt"], d["vt"], 20, ws=ws[:512])
    assert e.value.status == kvq.KVQ_E_WORKSPACE


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_flush_matches_oracle_and_touches_nothing_else(bits):
    B, Hkv, T_cap, R_cap, R, T0 = 2, 8, 400, 64, 50, 123
    inp = synth.make("l8b32k", T=1, B=B)
    ctx = kvq.Context(Hkv, bits, inp["signs_k"], inp["signs_v"])
    kt = synth.random_tensor(11, (B, Hkv, R_cap, 128), scale=3.0)
    vt = synth.random_tensor(12, (B, Hkv, R_cap, 128), scale=0.5)
    kt[1, 3, 7] = 0  # a zero vector
    rng = np.random.default_rng(13)
    kc0 = rng.integers(0, 256, size=(B, Hkv, T_cap, 16 * bits), dtype=np.uint8)
    vc0 = rng.integers(0, 256, size=(B, Hkv, T_cap, 16 * bits), dtype=np.uint8)
    kn0 = rng.uniform(1, 2, size=(B, Hkv, T_cap)).astype(np.float32)
    vn0 = rng.uniform(1, 2, size=(B, Hkv, T_cap)).astype(np.float32)
    g = {k: torch.from_numpy(v.copy()).cuda() for k, v in dict(kc=kc0, vc=vc0, kn=kn0, vn=vn0).items()}
    ctx.flush(torch.from_numpy(kt).cuda(), torch.from_numpy(vt).cuda(), R, g["kc"], g["kn"], g["vc"], g["vn"], T0)
    got = {k: to_np(v) for k, v in g.items()}
    sel = slice(T0, T0 + R)
    for name, x, signs, c0, n0 in (("k", kt, inp["signs_k"], kc0, kn0), ("v", vt, inp["signs_v"], vc0, vn0)):
        ref = O.quantize(x[:, :, :R], signs, bits, want_y=True)
        gi = unpack_np(got[name + "c"][:, :, sel], bits)
        m, f = boundary_mismatches(gi, ref, O.tables_f32(bits)[1], "flush " + name)
        bound_mismatches(m, f, "flush " + name)
        np.testing.assert_allclose(got[name + "n"][:, :, sel], ref["norms"], rtol=1e-5, atol=1e-30)
        keep = np.ones(T_cap, bool)
        keep[sel] = False
        assert np.array_equal(got[name + "c"][:, :, keep], c0[:, :, keep]), name
        assert np.array_equal(got[name + "n"][:, :, keep], n0[:, :, keep]), name
    assert got["kn"][1, 3, T0 + 7] == 0
    with pytest.raises(kvq.KvqError) as e:
        ctx.flush(torch.from_numpy(kt).cuda(), torch.from_numpy(vt).cuda(), R, g["kc"], g["kn"], g["vc"], g["vn"],
                  T_cap - R + 1)
    assert e.value.status == kvq.KVQ_E_INVAL
