"""GPU parity of kvq_quantize against the CPU oracle (through the C ABI).

Codes must be bit-exact except at coordinates within 1e-5 of a decision
threshold (counted); norms within 1e-5 relative."""
import numpy as np
import pytest
import torch

from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import check_codes, needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def run(x_np, signs_k, signs_v, bits, kind=kvq.KVQ_KIND_K):
    H = x_np.shape[1]
    ctx = kvq.Context(H, bits, signs_k, signs_v)
    x = torch.from_numpy(x_np).cuda()
    out = ctx.quantize(kind, x)
    return to_np(out["codes"]), to_np(out["norms"]), ctx, x, out


def test_tiny_full():
    inp = synth.make("tiny")
    codes, norms, *_ = run(inp["k"], inp["signs_k"], inp["signs_v"], 3)
    r = check_codes(inp["k"], inp["signs_k"], 3, codes, norms, label="tiny")
    print("tiny", r)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("kind", [kvq.KVQ_KIND_K, kvq.KVQ_KIND_V])
def test_l8b32k_ragged(bits, kind):
    inp = synth.make("l8b32k", T=1000)
    x = inp["k"] if kind == kvq.KVQ_KIND_K else inp["v"]
    signs = inp["signs_k"] if kind == kvq.KVQ_KIND_K else inp["signs_v"]
    codes, norms, *_ = run(x, inp["signs_k"], inp["signs_v"], bits, kind)
    print(bits, kind, check_codes(x, signs, bits, codes, norms, label="l8b32k T=1000"))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_l8b32k_full_size_sampled(bits):
    inp = synth.make("l8b32k")
    rng = np.random.default_rng(bits)
    for kind, x, signs in ((0, inp["k"], inp["signs_k"]), (1, inp["v"], inp["signs_v"])):
        codes, norms, *_ = run(x, inp["signs_k"], inp["signs_v"], bits, kind)
        n = 4096
        where = (np.zeros(n, int), rng.integers(0, 8, n), rng.integers(0, x.shape[2], n))
        print(bits, kind, check_codes(x, signs, bits, codes, norms, where=where, label="l8b32k full"))


def test_batch16_full_size_sampled():
    inp = synth.make("batch16", with_v=False)
    codes, norms, *_ = run(inp["k"], inp["signs_k"], inp["signs_v"], 3)
    rng = np.random.default_rng(0)
    n = 4096
    where = (rng.integers(0, 16, n), rng.integers(0, 8, n), rng.integers(0, 8192, n))
    print(check_codes(inp["k"], inp["signs_k"], 3, codes, norms, where=where, label="batch16"))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1, 31, 32, 33, 63, 64, 65, 129])
def test_edges(bits, T):
    rng = np.random.default_rng(T * 10 + bits)
    x = (rng.standard_normal((2, 3, T, 128)) * np.exp(rng.standard_normal((3, 1, 128)))).astype(np.float16)
    x[0, 0, 0] = 0.0                      # zero vector
    if T > 2:
        x[1, 2, 1] = np.float16(6e-8)     # subnormal-only vector
        x[1, 1, 2, :4] = np.float16(65504.0)  # largest fp16
    sk = np.where(rng.integers(0, 2, (3, 128)) == 1, 1, -1).astype(np.int8)
    codes, norms, *_ = run(x, sk, sk, bits)
    check_codes(x, sk, bits, codes, norms, label="edges")
    from tests.gpu_util import unpack_np
    assert norms[0, 0, 0] == 0.0
    assert np.all(unpack_np(codes[0, 0, 0], bits) == (1 << (bits - 1)) - 1)


def test_empty_and_validation():
    inp = synth.make("tiny", T=64)
    ctx = kvq.Context(1, 3, inp["signs_k"], inp["signs_v"])
    x = torch.from_numpy(inp["k"]).cuda()
    c = torch.empty((1, 1, 64, 48), dtype=torch.uint8, device="cuda")
    n = torch.empty((1, 1, 64), dtype=torch.float32, device="cuda")
    kvq.kvq_quantize(ctx, 0, x, 1, 1, 0, c, n)  # T = 0 is a valid empty call
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_quantize(ctx, 0, x, 1, 2, 64, c, n)  # wrong number of heads
    assert e.value.status == kvq.KVQ_E_INVAL
    with pytest.raises(kvq.KvqError):
        kvq.kvq_quantize(ctx, 2, x, 1, 1, 64, c, n)  # bad kind


def test_deterministic():
    inp = synth.make("l8b32k", T=2048)
    ctx = kvq.Context(8, 3, inp["signs_k"], inp["signs_v"])
    x = torch.from_numpy(inp["k"]).cuda()
    a = ctx.quantize(0, x)
    b = ctx.quantize(0, x)
    torch.cuda.synchronize()
    assert torch.equal(a["codes"], b["codes"]) and torch.equal(a["norms"], b["norms"])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantize_kv_fused_equals_separate(bits):
    inp = synth.make("l8b32k", T=1500, B=2)
    ctx = kvq.Context(8, bits, inp["signs_k"], inp["signs_v"])
    k = torch.from_numpy(inp["k"]).cuda()
    v = torch.from_numpy(inp["v"]).cuda()
    ko, vo = ctx.quantize_kv(k, v)
    ks = ctx.quantize(kvq.KVQ_KIND_K, k)
    vs = ctx.quantize(kvq.KVQ_KIND_V, v)
    torch.cuda.synchronize()
    for a, b in ((ko, ks), (vo, vs)):
        assert torch.equal(a["codes"], b["codes"]) and torch.equal(a["norms"], b["norms"])
    check_codes(inp["v"], inp["signs_v"], bits, to_np(vo["codes"]), to_np(vo["norms"]), label="fused V")


@pytest.mark.parametrize("seed", [0, 0xDEADBEEFCAFEF00D])
def test_seeded_signs_match_oracle(seed):
    """A context given a seed instead of sign arrays draws D_K and D_V with
    SplitMix64; the library's draw equals the oracle's own generator, and the
    codes of K and V follow that D."""
    import oracle as O

    inp = synth.make("l8b32k", T=300)
    H = inp["k"].shape[1]
    ctx = kvq.Context(H, 3, None, None, seed=seed)
    sk, sv = ctx.signs()
    ok, ov = O.seeded_signs(seed, H, 0), O.seeded_signs(seed, H, 1)
    assert np.array_equal(sk, ok) and np.array_equal(sv, ov)
    for kind, x, signs in ((kvq.KVQ_KIND_K, inp["k"], ok), (kvq.KVQ_KIND_V, inp["v"], ov)):
        out = ctx.quantize(kind, torch.from_numpy(x).cuda())
        check_codes(x, signs, 3, to_np(out["codes"]), to_np(out["norms"]), label="seeded")
    # explicit arrays are returned as given
    ctx2 = kvq.Context(H, 3, inp["signs_k"], None, seed=seed)
    sk2, sv2 = ctx2.signs()
    assert np.array_equal(sk2, inp["signs_k"]) and np.array_equal(sv2, ov)
