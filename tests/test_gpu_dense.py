"""GPU parity of the dense-rotation mode (a caller-given orthogonal Q in place
of the randomized Hadamard transform) against the CPU oracle.

The orthogonal matrices are seeded Haar draws (QR of a Gaussian matrix),
rounded to fp32 once; the library and the oracle receive the same fp32
entries.  Quantisation: exact indices except coordinates within 1e-5 of a
threshold (the oracle's flags), norms to 1e-5.  Scoring reads the oracle's
codes: logits within 1e-5 ||q|| ||k||, attention outputs within 2e-3."""
import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import bound_mismatches, boundary_mismatches, needs_gpu, to_np, unpack_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def rot(seed):
    return synth.random_orthogonal(seed).astype(np.float32)


def check_dense_codes(x, Q, bits, codes, norms, codebook="gauss"):
    ref = O.quantize_dense(x, Q.astype(np.float64), bits, codebook=codebook, want_y=True)
    gi = unpack_np(to_np(codes), bits)
    _, t = O.tables_f32_beta(bits) if codebook == "beta" else O.tables_f32(bits)
    m, f = boundary_mismatches(gi, ref, t, "dense")
    bound_mismatches(m, f, "dense")
    np.testing.assert_allclose(to_np(norms), ref["norms"], rtol=1e-5, atol=1e-30)
    return m, f


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_quantize_dense_ragged(bits):
    """2 x 8 x 777 vectors: 194 full groups of 64 and a ragged one."""
    inp = synth.make("l8b32k", T=777, B=2)
    Q = rot(30 + bits)
    ctx = kvq.Context(8, bits, rot_Q=Q)
    x = inp["k"].copy()
    x[1, 5, 776] = 0  # a zero vector: every coordinate at 0
    r = ctx.quantize(kvq.KVQ_KIND_K, torch.from_numpy(x).cuda())
    print("bits=%d (mismatches, flagged) = %s" % (bits, check_dense_codes(x, Q, bits, r["codes"], r["norms"])))
    assert to_np(r["norms"])[1, 5, 776] == 0


@pytest.mark.parametrize("T", [1, 63, 1000])
def test_quantize_kv_dense_and_beta_codebook(T):
    inp = synth.make("l8b32k", T=T)
    Q = rot(40)
    for cb, name in ((kvq.KVQ_CODEBOOK_GAUSS, "gauss"), (kvq.KVQ_CODEBOOK_BETA, "beta")):
        ctx = kvq.Context(8, 3, rot_Q=Q, codebook=cb)
        ko, vo = ctx.quantize_kv(torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda())
        check_dense_codes(inp["k"], Q, 3, ko["codes"], ko["norms"], codebook=name)
        check_dense_codes(inp["v"], Q, 3, vo["codes"], vo["norms"], codebook=name)


def test_quantize_dense_full_size_sampled():
    """The full l8b32k cache (8 x 32768 keys): 4096 sampled vectors checked."""
    inp = synth.make("l8b32k")
    Q = rot(41)
    ctx = kvq.Context(8, 3, rot_Q=Q)
    r = ctx.quantize(kvq.KVQ_KIND_K, torch.from_numpy(inp["k"]).cuda())
    t = np.sort(np.random.default_rng(42).choice(inp["k"].shape[2], 512, replace=False))
    check_dense_codes(inp["k"][:, :, t], Q, 3, r["codes"][:, :, torch.from_numpy(t).cuda()],
                      r["norms"][:, :, torch.from_numpy(t).cuda()])


def oracle_dense_codes(x, Q, bits):
    r = O.quantize_dense(x, Q.astype(np.float64), bits)
    return r["codes"], r["norms"].astype(np.float32)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_logits_dense(bits):
    inp = synth.make("l8b32k", T=777, B=2)
    Q = rot(50)
    kc, kn = oracle_dense_codes(inp["k"], Q, bits)
    ctx = kvq.Context(8, bits, rot_Q=Q)
    lg = to_np(ctx.logits(torch.from_numpy(inp["q"]).cuda(), torch.from_numpy(kc).cuda(),
                          torch.from_numpy(kn).cuda()))
    ref = O.logits_dense(inp["q"], kc, kn.astype(np.float64), Q.astype(np.float64), bits)
    scale = np.linalg.norm(inp["q"].astype(np.float64), axis=-1)[..., None] * np.repeat(kn.astype(np.float64), 4,
                                                                                       axis=1)
    err = np.abs(lg - ref) / np.maximum(scale, 1e-30)
    print("bits=%d max rel err %.3g" % (bits, err.max()))
    assert err.max() <= 1e-5


def decode_case(bits, T, B=1, Hkv=8, Hq=32, seed=60, n_split=0):
    inp = synth.make("l8b32k", T=T, B=B)
    Q = rot(seed)
    k, v = inp["k"][:, :Hkv], inp["v"][:, :Hkv]
    q = inp["q"][:, :Hq]
    kc, kn = oracle_dense_codes(k, Q, bits)
    vc, vn = oracle_dense_codes(v, Q, bits)
    ctx = kvq.Context(Hkv, bits, rot_Q=Q)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out = to_np(ctx.attn_decode(g(q), g(kc), g(kn), g(vc), g(vn), n_split=n_split))
    ref = O.attention_dense(q, kc, kn.astype(np.float64), vc, vn.astype(np.float64), Q.astype(np.float64), bits)
    return np.abs(out - ref).max()


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("T", [1, 50, 3001])
def test_decode_dense(bits, T):
    err = decode_case(bits, T)
    print("bits=%d T=%d max abs err %.3g" % (bits, T, err))
    assert err <= 2e-3


@pytest.mark.parametrize("G", [1, 2])
def test_decode_dense_groups_batch_splits(G):
    for n_split in (0, 1, 5):
        assert decode_case(3, 2000, B=2, Hkv=4, Hq=4 * G, seed=61, n_split=n_split) <= 2e-3


def test_decode_dense_full_size():
    """8 KV heads x 32768 tokens, 32 query heads, every output checked."""
    err = decode_case(3, None, seed=62)
    print("full size max abs err %.3g" % err)
    assert err <= 2e-3


def test_hadamard_matrix_as_dense_rotation_matches_hadamard_path():
    """Q = H diag(D) / sqrt(d) makes the dense mode the Hadamard mode: the
    same codes (away from thresholds) and the same logits and outputs."""
    inp = synth.make("l8b32k", T=1500)
    Hm = O.hadamard_matrix(128).astype(np.float64)
    out = {}
    for dense in (False, True):
        # one Q serves all heads, so use the same signs for every head and both kinds
        s = np.repeat(inp["signs_k"][:1], 8, axis=0)
        Q = (Hm * s[0][None, :].astype(np.float64) / np.sqrt(128)).astype(np.float32)
        ctx = kvq.Context(8, 3, s, s, rot_Q=Q if dense else None)
        ko, vo = ctx.quantize_kv(torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda())
        q = torch.from_numpy(inp["q"]).cuda()
        out[dense] = dict(k=unpack_np(to_np(ko["codes"]), 3), kn=to_np(ko["norms"]),
                          lg=to_np(ctx.logits(q, ko["codes"], ko["norms"])),
                          o=to_np(ctx.attn_decode(q, ko["codes"], ko["norms"], vo["codes"], vo["norms"])))
    a, b = out[False], out[True]
    assert np.mean(a["k"] != b["k"]) < 1e-4
    np.testing.assert_allclose(b["kn"], a["kn"], rtol=1e-6)
    same = np.all(a["k"] == b["k"], axis=-1)  # keys whose codes agree
    scale = np.linalg.norm(inp["q"].astype(np.float64), axis=-1)[..., None] * np.repeat(a["kn"], 4, axis=1)
    diff = np.abs(a["lg"] - b["lg"]) / scale
    assert diff[np.repeat(same, 4, axis=1)].max() <= 1e-5


def test_dense_validation():
    Q = rot(70)
    with pytest.raises(kvq.KvqError) as e:  # the NSN-VQ mode keeps its own transform
        kvq.Context(2, 1, mode=kvq.KVQ_MODE_NSN_VQ, vq_codebook=np.ones((256, 8), np.float32), rot_Q=Q)
    assert e.value.status == kvq.KVQ_E_UNSUPPORTED
    bad = Q.copy()
    bad[3, 4] = np.nan
    with pytest.raises(kvq.KvqError) as e:
        kvq.Context(2, 3, rot_Q=bad)
    assert e.value.status == kvq.KVQ_E_INVAL
    ctx = kvq.Context(2, 3, rot_Q=Q)
    kc = torch.zeros((1, 2, 64, 48), dtype=torch.uint8, device="cuda")
    kn = torch.ones((1, 2, 64), dtype=torch.float32, device="cuda")
    kt = torch.zeros((1, 2, 16, 128), dtype=torch.float16, device="cuda")
    q = torch.zeros((1, 8, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:  # the streaming cache is Hadamard-only
        ctx.attn_decode_stream(q, kc, kn, kc, kn, 10, kt, kt, 4)
    assert e.value.status == kvq.KVQ_E_UNSUPPORTED
    with pytest.raises(kvq.KvqError) as e:
        ctx.flush(kt, kt, 4, kc, kn, kc, kn, 0)
    assert e.value.status == kvq.KVQ_E_UNSUPPORTED


def test_quantize_kv_dense_equals_two_calls_and_is_deterministic():
    """One K+V launch gives the bits of two single-list calls (the same
    per-vector arithmetic), and repeated calls give the same bits."""
    inp = synth.make("l8b32k", T=333, B=2)
    ctx = kvq.Context(8, 3, rot_Q=rot(80))
    k, v = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    ko, vo = ctx.quantize_kv(k, v)
    k1 = ctx.quantize(kvq.KVQ_KIND_K, k)
    v1 = ctx.quantize(kvq.KVQ_KIND_V, v)
    ko2, _ = ctx.quantize_kv(k, v)
    for a, b in ((ko, k1), (vo, v1), (ko, ko2)):
        assert torch.equal(a["codes"], b["codes"])
        assert torch.equal(a["norms"], b["norms"])


# --------------------------------------------------------------------------- dense rotation + QJL residual
def check_dense_qjl(x, Q, S, bits, g, where=None):
    """Codes (valid at flagged coordinates), norms, and for every key the QJL
    sign bits and gamma of the residual in the dense-rotated space, against
    the oracle (a key whose codes flipped at a flagged coordinate is compared
    with the oracle's QJL of that admissible code)."""
    from tests.test_gpu_qjl import admissible_qjl
    B, H, T, _ = x.shape
    if where is None:
        bb, hh, tt = [a.ravel() for a in np.meshgrid(np.arange(B), np.arange(H), np.arange(T), indexing="ij")]
    else:
        bb, hh, tt = where
    xs = x[bb, hh, tt][None, None]
    ref = O.quantize_dense(xs, Q.astype(np.float64), bits, want_y=True)
    gi = unpack_np(g["codes"][bb, hh, tt], bits)[None, None]
    m, f = boundary_mismatches(gi, ref, O.tables_f32(bits)[1], "dense qjl codes")
    bound_mismatches(m, f, "dense qjl codes")
    np.testing.assert_allclose(g["norms"][bb, hh, tt], ref["norms"][0, 0], rtol=1e-5, atol=1e-30)
    S64 = S.astype(np.float64)
    q = O.qjl(ref["y"], ref["idx"], S64, bits)
    r_gamma, r_flags = q["gamma"][0, 0].copy(), q["flags"][0, 0].copy()
    r_bits = np.unpackbits(q["signs"][0, 0], axis=-1, bitorder="little")
    for v in np.flatnonzero(~(gi[0, 0] == ref["idx"][0, 0]).all(-1)):
        alt = admissible_qjl(ref["y"][0, 0, v], ref["idx"][0, 0, v], ref["flags"][0, 0, v], S64, bits, gi[0, 0, v])
        r_gamma[v] = alt["gamma"][0]
        r_bits[v] = np.unpackbits(alt["signs"][0], bitorder="little")
        r_flags[v] = alt["flags"][0]
    np.testing.assert_allclose(g["qjl_gamma"][bb, hh, tt], r_gamma, rtol=1e-5, atol=1e-7)
    g_bits = np.unpackbits(g["qjl_signs"][bb, hh, tt], axis=-1, bitorder="little")
    bad = (g_bits != r_bits) & (r_flags == 0)
    assert not bad.any(), "%d sign bits differ outside the 1e-5*gamma band" % int(bad.sum())
    nm = int((g_bits != r_bits).sum())
    assert nm <= int(r_flags.sum()) // 2 + 2, (nm, int(r_flags.sum()))
    return m, nm


def run_dense_qjl(x, Q, S, bits, signs_k, signs_v):
    ctx = kvq.Context(x.shape[1], bits, signs_k, signs_v, mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=S, rot_Q=Q)
    out = ctx.quantize(kvq.KVQ_KIND_K, torch.from_numpy(x).cuda())
    return ctx, {k: to_np(v) for k, v in out.items()}


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_dense_qjl_quantize_ragged(bits):
    """2 x 8 x 333 keys (ragged groups of 64), a zero key."""
    inp = synth.make("long128k_qjl", T=333, B=2)
    x = inp["k"].copy()
    x[1, 2, 7] = 0
    Q = rot(80 + bits)
    ctx, g = run_dense_qjl(x, Q, inp["S"], bits, inp["signs_k"], inp["signs_v"])
    print("bits=%d (code mismatches, sign mismatches) = %s" % (bits, check_dense_qjl(x, Q, inp["S"], bits, g)))
    assert g["norms"][1, 2, 7] == 0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_dense_qjl_general_fp32_projection(bits):
    """An S that is not exactly fp16: the kernel adds the e_hi . S_lo pass
    (these instances spill registers to scratch)."""
    inp = synth.make("long128k_qjl", T=200)
    S = np.random.default_rng(6).standard_normal((128, 128)).astype(np.float32)
    Q = rot(85)
    ctx, g = run_dense_qjl(inp["k"], Q, S, bits, inp["signs_k"], inp["signs_v"])
    print("bits=%d (code mismatches, sign mismatches) = %s" % (bits, check_dense_qjl(inp["k"], Q, S, bits, g)))


def test_dense_qjl_full_size_sampled():
    """The long-context keys (8 x 131072) with the dense rotation and the QJL
    residual: 2048 sampled keys checked."""
    inp = synth.make("long128k_qjl")
    Q = rot(86)
    ctx, g = run_dense_qjl(inp["k"], Q, inp["S"], 2, inp["signs_k"], inp["signs_v"])
    rng = np.random.default_rng(4)
    n = 2048
    where = (np.zeros(n, int), rng.integers(0, 8, n), rng.integers(0, inp["T"], n))
    print(check_dense_qjl(inp["k"], Q, inp["S"], 2, g, where=where))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_dense_qjl_logits(bits):
    """Logits with the QJL term in the rotated space, on the oracle's codes."""
    inp = synth.make("long128k_qjl", T=900)
    Q = rot(90 + bits)
    S = inp["S"]
    r = O.quantize_dense(inp["k"], Q.astype(np.float64), bits, want_y=True)
    qj = O.qjl(r["y"], r["idx"], S.astype(np.float64), bits)
    kn, gm = r["norms"].astype(np.float32), qj["gamma"].astype(np.float32)
    ctx = kvq.Context(8, bits, mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=S, rot_Q=Q)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    lg = to_np(ctx.logits(dev(inp["q"]), dev(r["codes"]), dev(kn), dev(qj["signs"]), dev(gm)))
    ref = O.logits_dense(inp["q"], r["codes"], kn.astype(np.float64), Q.astype(np.float64), bits,
                         qjl_signs=qj["signs"], gamma=gm.astype(np.float64), S=S.astype(np.float64))
    scale = np.linalg.norm(inp["q"].astype(np.float64), axis=-1)[..., None] * np.repeat(kn.astype(np.float64), 4, axis=1)
    err = (np.abs(lg - ref) / scale).max()
    assert err <= 1e-5, err
