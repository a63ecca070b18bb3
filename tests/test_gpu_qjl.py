"""GPU parity of the QJL residual path (kvq_quantize in MSE_QJL mode and
kvq_logits with the QJL term) against the CPU oracle.

Sign bits and gamma are compared on every vector: exact except bits whose
projection lies within 1e-5 * gamma of zero.  A vector whose GPU indices
differ from the oracle's at flagged coordinates (an admissible code: each
such coordinate in the neighbouring cell across a threshold within 1e-5) is
compared with the oracle's QJL residual of that admissible code.  The logit tests score codes
written by the oracle (small cases) or drawn by the seeded generator (full
size); no GPU output feeds the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import check_codes, needs_gpu, to_np, unpack_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def run_qjl(inp, bits, S):
    ctx = kvq.Context(inp["Hkv"], bits, inp["signs_k"], inp["signs_v"], mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=S)
    k = torch.from_numpy(inp["k"]).cuda()
    out = ctx.quantize(kvq.KVQ_KIND_K, k)
    return ctx, {n: to_np(t) for n, t in out.items()}, out


def admissible_qjl(y, idx, flags, S, bits, gi):
    """The oracle's QJL results for every admissible code vector of one key:
    each flagged coordinate (within 1e-5 of a threshold) in its own cell or in
    the neighbouring cell across that threshold.  Returns the alternative
    whose indices equal the GPU's `gi` (the GPU's choice among them)."""
    _, t = O.tables_f32(bits)
    fpos = np.flatnonzero(flags)
    assert len(fpos) <= 8, "too many flagged coordinates in one key"
    alts = []
    for mask in range(1 << len(fpos)):
        alt = idx.copy()
        for k, i in enumerate(fpos):
            if mask >> k & 1:
                # the other side of the threshold y[i] is near
                j = int(np.argmin(np.abs(y[i] - t.astype(np.float64))))
                alt[i] = j if idx[i] == j + 1 else j + 1
        alts.append(alt)
    for alt in alts:
        if np.array_equal(alt, gi):
            return O.qjl(y[None], alt[None], S, bits)
    raise AssertionError("GPU indices are not an admissible code of the key")


def check_qjl(inp, bits, S, o, where=None):
    """Sign bits and gamma of every key: exact (gamma to 1e-5) except bits
    whose projection lies within 1e-5 * gamma of zero.  A key whose GPU
    indices differ from the oracle's at flagged coordinates is compared with
    the oracle's QJL of those indices (its residual is a different vector)."""
    x = inp["k"]
    B, H, T, _ = x.shape
    if where is None:
        bb, hh, tt = [a.ravel() for a in np.meshgrid(np.arange(B), np.arange(H), np.arange(T), indexing="ij")]
    else:
        bb, hh, tt = where
    mism = flipped = flagged = 0
    for h in np.unique(hh):
        sel = hh == h
        xs = x[bb[sel], h, tt[sel]][None, None]
        ref = O.quantize(xs, inp["signs_k"][h:h + 1], bits, want_y=True)
        q = O.qjl(ref["y"], ref["idx"], S, bits)
        gi = unpack_np(o["codes"][bb[sel], h, tt[sel]], bits)
        g_gamma = o["qjl_gamma"][bb[sel], h, tt[sel]]
        g_bits = np.unpackbits(o["qjl_signs"][bb[sel], h, tt[sel]], axis=-1, bitorder="little")
        r_gamma = q["gamma"][0, 0].copy()
        r_bits = np.unpackbits(q["signs"][0, 0], axis=-1, bitorder="little")
        r_flags = q["flags"][0, 0].copy()
        for v in np.flatnonzero(~(gi == ref["idx"][0, 0]).all(-1)):
            alt = admissible_qjl(ref["y"][0, 0, v], ref["idx"][0, 0, v], ref["flags"][0, 0, v], S, bits, gi[v])
            r_gamma[v] = alt["gamma"][0]
            r_bits[v] = np.unpackbits(alt["signs"][0], bitorder="little")
            r_flags[v] = alt["flags"][0]
            flipped += 1
        np.testing.assert_allclose(g_gamma, r_gamma, rtol=1e-5, atol=1e-7)
        bad = (g_bits != r_bits) & (r_flags == 0)
        assert not bad.any(), "%d sign bits differ outside the 1e-5*gamma band" % int(bad.sum())
        mism += int((g_bits != r_bits).sum())
        flagged += int(r_flags.sum())
    assert mism <= flagged // 2 + 2, (mism, flagged)
    return mism, flipped


def oracle_qjl_codes(inp, bits):
    """Codes, fp32 norms, sign bits and fp32 gamma of every key, from the oracle."""
    r = O.quantize(inp["k"], inp["signs_k"], bits, want_y=True)
    q = O.qjl(r["y"], r["idx"], inp["S"], bits)
    return dict(codes=r["codes"], norms=r["norms"].astype(np.float32), qjl_signs=q["signs"],
                qjl_gamma=q["gamma"].astype(np.float32))


def check_qjl_logits(inp, ctx, c, t=None):
    g = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in c.items()}
    lg = to_np(ctx.logits(torch.from_numpy(inp["q"]).cuda(), g["codes"], g["norms"], g["qjl_signs"],
                          g["qjl_gamma"]))
    sub = (lambda a: a) if t is None else (lambda a: a[:, :, t])
    ref = O.logits(inp["q"], sub(c["codes"]), sub(c["norms"]).astype(np.float64), inp["signs_k"], 2,
                   qjl_signs=sub(c["qjl_signs"]), gamma=sub(c["qjl_gamma"]).astype(np.float64), S=inp["S"])
    G = inp["Hq"] // inp["Hkv"]
    scale = np.linalg.norm(inp["q"].astype(np.float64), axis=-1)[..., None] * np.repeat(sub(c["norms"]), G, axis=1)
    err = np.abs(sub(lg) - ref) / np.maximum(scale, 1e-30)
    assert err.max() <= 1e-3
    assert err.max() <= 1e-5, err.max()
    return err.max()


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_qjl_quantize_ragged(bits):
    inp = synth.make("long128k_qjl", T=700)
    ctx, o, _ = run_qjl(inp, bits, inp["S"])
    check_codes(inp["k"], inp["signs_k"], bits, o["codes"], o["norms"], label="qjl codes")
    print("boundary sign mismatches", check_qjl(inp, bits, inp["S"], o))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_qjl_general_fp32_projection(bits):
    """S not representable in fp16: the kernel adds the e_hi * S_lo pass
    (at b = 3 that instance spills two registers to scratch)."""
    inp = synth.make("long128k_qjl", T=300)
    S = np.random.default_rng(5).standard_normal((128, 128)).astype(np.float32)
    ctx, o, _ = run_qjl(inp, bits, S)
    check_codes(inp["k"], inp["signs_k"], bits, o["codes"], o["norms"], label="qjl codes, fp32 S")
    check_qjl(inp, bits, S, o)


def test_qjl_full_size_sampled():
    inp = synth.make("long128k_qjl")
    ctx, o, _ = run_qjl(inp, 2, inp["S"])
    rng = np.random.default_rng(3)
    n = 4096
    where = (np.zeros(n, int), rng.integers(0, 8, n), rng.integers(0, inp["T"], n))
    check_codes(inp["k"], inp["signs_k"], 2, o["codes"], o["norms"], where=where, label="qjl full")
    check_qjl(inp, 2, inp["S"], o, where=where)


def test_qjl_zero_vector():
    inp = synth.make("long128k_qjl", T=65)
    inp["k"][0, 3, 7] = 0
    ctx, o, _ = run_qjl(inp, 2, inp["S"])
    check_qjl(inp, 2, inp["S"], o)
    assert o["norms"][0, 3, 7] == 0


@pytest.mark.parametrize("T", [1000, 4097])
def test_qjl_logits(T):
    inp = synth.make("long128k_qjl", T=T)
    ctx = kvq.Context(inp["Hkv"], 2, inp["signs_k"], inp["signs_v"], mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=inp["S"])
    print("max rel err", check_qjl_logits(inp, ctx, oracle_qjl_codes(inp, 2)))


def test_qjl_logits_full_size_sampled():
    """All 8 x 131072 keys as drawn by the seeded generator (uniform codes and
    sign bits, lognormal norms and gamma); the oracle scores 2048 of them."""
    inp = synth.make("long128k_qjl")
    c = synth.random_codes(11, (1, inp["Hkv"], inp["T"]), 2, qjl_m=128)
    ctx = kvq.Context(inp["Hkv"], 2, inp["signs_k"], inp["signs_v"], mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=inp["S"])
    t = np.random.default_rng(9).integers(0, inp["T"], 2048)
    print("max rel err", check_qjl_logits(inp, ctx, c, t=t))
