"""The bounds-checked debug build (libkvq_debug.so, compiled with KVQ_DEBUG).

A child process loads it (KVQ_LIB) and runs the paths on seeded inputs: K
and V quantised in one launch at b = 1..4 over a ragged token count, logits,
decode with automatic splits, with one split (several tiles per wave) and
without allocation, the streaming decode and its flush; NSN-VQ (plain and
adaptive scale) and GSRQ encoders with logits and decode from their records;
the dense rotation; the QJL quantiser and its logits.  The check records
are read after every call.  No check may fail, and every result must equal,
bit for bit, the one the release library gives in this process: the checks
and the NaN fill of LDS change no arithmetic, and a kernel that read LDS it
never wrote would differ."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "calibration_free_kv_amd", "libkvq_debug.so")


def run_cases():
    """Results of the calls through whichever library this process loaded,
    and the failed checks {call: record}."""
    res, fails = {}, {}

    def take(name):
        torch.cuda.synchronize()
        v = kvq.debug_take()
        if v:
            fails[name] = v

    T = 3001
    inp = synth.make("l8b32k", T=T)
    k = torch.from_numpy(inp["k"]).cuda()
    v = torch.from_numpy(inp["v"]).cuda()
    q = torch.from_numpy(inp["q"]).cuda()
    for bits in (1, 2, 3, 4):
        ctx = kvq.Context(inp["Hkv"], bits, inp["signs_k"], inp["signs_v"])
        ko, vo = ctx.quantize_kv(k, v)
        take("quantize_kv b=%d" % bits)
        for name, t in (("kc", ko["codes"]), ("kn", ko["norms"]), ("vc", vo["codes"]), ("vn", vo["norms"])):
            res["%s%d" % (name, bits)] = to_np(t)
        res["lg%d" % bits] = to_np(ctx.logits(q, ko["codes"], ko["norms"]))
        take("logits b=%d" % bits)
        for ns in (0, 1):
            res["dec%d_%d" % (bits, ns)] = to_np(ctx.attn_decode(q, ko["codes"], ko["norms"], vo["codes"],
                                                                 vo["norms"], n_split=ns))
            take("attn_decode b=%d n_split=%d" % (bits, ns))
        res["dna%d" % bits] = to_np(ctx.attn_decode_noalloc(q, ko["codes"], ko["norms"], vo["codes"], vo["norms"]))
        take("attn_decode_noalloc b=%d" % bits)
        # streaming cache: the first T - R tokens packed, the last R in the fp16 window
        R, Tp = 100, T - 100
        kt = k[:, :, Tp:].contiguous()
        vt = v[:, :, Tp:].contiguous()
        res["st%d" % bits] = to_np(ctx.attn_decode_stream(q, ko["codes"], ko["norms"], vo["codes"], vo["norms"], Tp,
                                                          kt, vt, R))
        take("attn_decode_stream b=%d" % bits)
        g = {n: t.clone() for n, t in (("kc", ko["codes"]), ("kn", ko["norms"]), ("vc", vo["codes"]),
                                       ("vn", vo["norms"]))}
        ctx.flush(kt, vt, R, g["kc"], g["kn"], g["vc"], g["vn"], Tp)
        take("flush b=%d" % bits)
        for n, t in g.items():
            res["fl%s%d" % (n, bits)] = to_np(t)
        ctx.close()
    # NSN-VQ (plain and adaptive scale), GSRQ: encoders over the 8 heads of K and
    # V, logits and decode from their records
    cb = np.loadtxt(os.path.join(ROOT, "tests", "golden", "vq_codebook_256x8.txt"), dtype=np.float32).reshape(256, 8)
    lines = [ln.split() for ln in open(os.path.join(ROOT, "tests", "golden", "gsrq_tables_256x32.txt"))
             if not ln.startswith("#")]
    gt = dict(S1=np.array(lines[0:256], dtype=np.float32), G1=np.array(lines[256], dtype=np.float32),
              S2=np.array(lines[257:513], dtype=np.float32), G2=np.array(lines[513], dtype=np.float32))
    H = inp["Hkv"]

    def per_head(e, rec):
        return dict(codes=e["codes"].view(1, H, T, rec), s1=e["s1"].view(1, H, T), s2=e["s2"].view(1, H, T),
                    o=e["o"].view(1, H, 128))

    for name, ctx, rec in (("nsn", kvq.Context(H, 1, mode=kvq.KVQ_MODE_NSN_VQ, vq_codebook=cb), 16),
                           ("nsna", kvq.Context(H, 1, mode=kvq.KVQ_MODE_NSN_VQ, vq_codebook=cb,
                                                nsn_options=kvq.KVQ_NSN_ADAPTIVE_SCALE), 16),
                           ("gsrq", kvq.Context(H, 1, mode=kvq.KVQ_MODE_GSRQ, gsrq_tables=gt), 12)):
        enc = ctx.gsrq_quantize if name == "gsrq" else ctx.nsn_vq_quantize
        ek, ev = enc(k[0]), enc(v[0])
        take(name + " encode")
        for n, t in ek.items():
            res["%s_%s" % (name, n)] = to_np(t)
        kd, vd = per_head(ek, rec), per_head(ev, rec)
        lg = ctx.gsrq_logits(q, **kd) if name == "gsrq" else ctx.nsn_logits(q, **kd)
        res[name + "_lg"] = to_np(lg)
        take(name + " logits")
        dec = ctx.gsrq_attn_decode if name == "gsrq" else ctx.nsn_attn_decode
        res[name + "_dec"] = to_np(dec(q, kd, vd))
        take(name + " decode")
        ctx.close()
    # dense rotation: quantize K and V, decode
    ctx = kvq.Context(H, 3, rot_Q=synth.random_orthogonal(5).astype(np.float32))
    ko, vo = ctx.quantize_kv(k, v)
    take("dense quantize_kv")
    res["dense_kc"], res["dense_kn"] = to_np(ko["codes"]), to_np(ko["norms"])
    res["dense_dec"] = to_np(ctx.attn_decode(q, ko["codes"], ko["norms"], vo["codes"], vo["norms"]))
    take("dense decode")
    ctx.close()
    qi = synth.make("long128k_qjl", T=T)
    ctx = kvq.Context(qi["Hkv"], 2, qi["signs_k"], qi["signs_v"], mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=qi["S"])
    qo = ctx.quantize(kvq.KVQ_KIND_K, torch.from_numpy(qi["k"]).cuda())
    take("quantize qjl")
    for n, t in qo.items():
        res["qjl_" + n] = to_np(t)
    res["qjl_lg"] = to_np(ctx.logits(torch.from_numpy(qi["q"]).cuda(), qo["codes"], qo["norms"], qo["qjl_signs"],
                                     qo["qjl_gamma"]))
    take("logits qjl")
    ctx.close()
    return res, fails


def test_debug_build_checks_pass_and_results_match(tmp_path):
    assert os.path.exists(DEBUG_LIB), "libkvq_debug.so is built with libkvq.so"
    assert not kvq.debug_build() and kvq.debug_take() == 0  # the release library in this process
    out = str(tmp_path / "debug.npz")
    child = ("import sys; sys.path.insert(0, %r)\n"
             "import numpy as np\n"
             "from calibration_free_kv_amd import kvq\n"
             "from tests.test_gpu_debug import run_cases\n"
             "assert kvq.debug_build()\n"
             "res, fails = run_cases()\n"
             "np.savez(%r, **res)\n"
             "print('failed checks:', fails)\n"
             "sys.exit(1 if fails else 0)\n") % (ROOT, out)
    env = dict(os.environ, KVQ_LIB=DEBUG_LIB)
    print("child process: debug build", flush=True)
    r = subprocess.run([sys.executable, "-c", child], env=env, capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    got = np.load(out)
    want, fails = run_cases()
    assert not fails
    assert sorted(got.files) == sorted(want)
    for name in want:
        assert np.array_equal(got[name], want[name], equal_nan=True), name
    print("%d results equal between the debug and release builds" % len(want))
