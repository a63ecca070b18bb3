"""GPU parity of the MSE path with the exact-d codebook (KVQ_CODEBOOK_BETA:
Lloyd-Max for Beta((d-1)/2, (d-1)/2) on [-1, 1] scaled by sqrt(d), the
TurboQuant page's Stage 1) against the CPU oracle.  The kernels are those of
the N(0,1) tables; only the tables differ, and the library builds them with
its own quadrature (compared with the oracle's to fp32 rounding)."""
import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import bound_mismatches, boundary_mismatches, needs_gpu, to_np, unpack_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def beta_ctx(inp, bits):
    return kvq.Context(inp["Hkv"], bits, inp["signs_k"], inp["signs_v"], codebook=kvq.KVQ_CODEBOOK_BETA)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_library_tables_equal_oracle_tables(bits):
    inp = synth.make("l8b32k", T=1)
    c, t = beta_ctx(inp, bits).tables()
    co, to = O.tables_f32_beta(bits)
    np.testing.assert_allclose(c, co, rtol=3e-7, atol=0)
    np.testing.assert_allclose(t, to, rtol=3e-7, atol=1e-30)
    assert not np.array_equal(c, O.tables_f32(bits)[0])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_beta(bits):
    inp = synth.make("l8b32k", T=777)
    ctx = beta_ctx(inp, bits)
    out = ctx.quantize(kvq.KVQ_KIND_K, torch.from_numpy(inp["k"]).cuda())
    r = check_codes_beta(inp["k"], inp["signs_k"], bits, to_np(out["codes"]), to_np(out["norms"]))
    print(r)


def check_codes_beta(x, signs, bits, codes, norms):
    ref = O.quantize(x, signs, bits, codebook="beta", want_y=True)
    gi = unpack_np(codes, bits)
    m, f = boundary_mismatches(gi, ref, O.tables_f32_beta(bits)[1], "beta")
    bound_mismatches(m, f, "beta")
    np.testing.assert_allclose(norms, ref["norms"], rtol=1e-5, atol=1e-30)
    return dict(mismatch_at_boundary=m, flagged=f)


@pytest.mark.parametrize("bits", [2, 3])
def test_decode_and_logits_beta(bits):
    inp = synth.make("l8b32k", T=1500)
    ctx = beta_ctx(inp, bits)
    rk = O.quantize(inp["k"], inp["signs_k"], bits, codebook="beta")
    rv = O.quantize(inp["v"], inp["signs_v"], bits, codebook="beta")
    kn, vn = rk["norms"].astype(np.float32), rv["norms"].astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    q = dev(inp["q"])
    out = to_np(ctx.attn_decode(q, dev(rk["codes"]), dev(kn), dev(rv["codes"]), dev(vn)))
    ref = O.attention(inp["q"], rk["codes"], kn.astype(np.float64), rv["codes"], vn.astype(np.float64),
                      inp["signs_k"], inp["signs_v"], bits, codebook="beta")
    assert np.abs(out - ref).max() <= 2e-3
    lg = to_np(ctx.logits(q, dev(rk["codes"]), dev(kn)))
    lref = O.logits(inp["q"], rk["codes"], kn.astype(np.float64), inp["signs_k"], bits, codebook="beta")
    scale = np.linalg.norm(inp["q"].astype(np.float64), axis=-1)[..., None] * np.repeat(kn, 4, axis=1)
    assert (np.abs(lg - lref) / scale).max() <= 1e-5


def test_beta_rejected_for_nsn():
    cb = np.zeros((256, 8), np.float32)
    with pytest.raises(kvq.KvqError) as e:
        kvq.Context(2, 1, mode=kvq.KVQ_MODE_NSN_VQ, vq_codebook=cb, codebook=kvq.KVQ_CODEBOOK_BETA)
    assert e.value.status == kvq.KVQ_E_INVAL
