"""kvq_attn_decode_noalloc (the decode entry point that allocates nothing and
takes no workspace) against kvq_attn_decode, through the C ABI.

Both entry points score the same packed codes (written by the oracle's
quantizer) and run the same kernels, the no-allocation one on the library's
fixed per-device scratch.  Two calls in a row, the second smaller, so that the
second runs on scratch the first left behind.  Bar: attention outputs within
2e-3 max-abs of the existing entry point (and of the oracle)."""
import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def encoded(inp, bits, Q=None):
    if Q is None:
        rk = O.quantize(inp["k"], inp["signs_k"], bits)
        rv = O.quantize(inp["v"], inp["signs_v"], bits)
    else:
        rk = O.quantize_dense(inp["k"], Q.astype(np.float64), bits)
        rv = O.quantize_dense(inp["v"], Q.astype(np.float64), bits)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    return (dev(rk["codes"]), dev(rk["norms"].astype(np.float32)), dev(rv["codes"]),
            dev(rv["norms"].astype(np.float32)))


def oracle_out(inp, enc, bits, Q=None):
    kc, kn, vc, vn = [to_np(t) for t in enc]
    kn, vn = kn.astype(np.float64), vn.astype(np.float64)
    if Q is None:
        return O.attention(inp["q"], kc, kn, vc, vn, inp["signs_k"], inp["signs_v"], bits)
    return O.attention_dense(inp["q"], kc, kn, vc, vn, Q.astype(np.float64), bits)


@pytest.mark.parametrize("dense", [False, True])
def test_noalloc_equals_workspace_decode_twice(dense):
    bits = 3
    Q = synth.random_orthogonal(50).astype(np.float32) if dense else None
    for B, T in ((2, 5000), (1, 700)):  # the second call is smaller
        inp = synth.make("l8b32k", T=T, B=B)
        ctx = kvq.Context(8, bits, inp["signs_k"], inp["signs_v"], rot_Q=Q)
        enc = encoded(inp, bits, Q)
        q = torch.from_numpy(inp["q"]).cuda()
        ref = to_np(ctx.attn_decode(q, *enc))
        got = to_np(ctx.attn_decode_noalloc(q, *enc))
        err = float(np.abs(got - ref).max())
        print("dense=%s B=%d T=%d max |noalloc - workspace| %.3g" % (dense, B, T, err))
        assert err <= 2e-3
        assert float(np.abs(got - oracle_out(inp, enc, bits, Q)).max()) <= 2e-3


def test_noalloc_repeats_and_rejects_oversize():
    inp = synth.make("l8b32k", T=300)
    ctx = kvq.Context(8, 2, inp["signs_k"], inp["signs_v"])
    enc = encoded(inp, 2)
    q = torch.from_numpy(inp["q"]).cuda()
    a = to_np(ctx.attn_decode_noalloc(q, *enc))
    b = to_np(ctx.attn_decode_noalloc(q, *enc))
    assert np.array_equal(a, b)  # the counters were left at zero
    # 512 x 32 query heads need 520 bytes each even at one split: above the scratch
    qb = torch.zeros((512, 32, 128), dtype=torch.float16, device="cuda")
    kc = torch.zeros((512, 8, 1, 32), dtype=torch.uint8, device="cuda")
    kn = torch.ones((512, 8, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        ctx.attn_decode_noalloc(qb, kc, kn, kc, kn)
    assert e.value.status == kvq.KVQ_E_WORKSPACE
