"""Throughput of the KV-cache quantisation hot path on one MI355X.

Main line (one step): quantise the K and the V cache of one Llama-3-8B-shaped
attention layer (batch 1, 8 KV heads x 128, 32768 tokens, fp16) to 3-bit codes
with kvq_quantize_kv, then one decode step of attention for its 32 query heads
(GQA 4) read straight from codes with kvq_attn_decode.  Inputs are synthetic
(seeded N(0,1) x per-channel lognormal(0,1) scales) and resident in HBM before
timing starts.  The steps rotate over 4 input/output sets (645 MB, more than
twice the 256 MB last-level cache); the decode of step s reads the codes of
set s + 2, written two steps earlier, so they are not served from that cache.
The decode runs on a second stream (default priority) and overlaps the
quantize of the same step: events order each decode after the quantize that
wrote its codes and each quantize after the last decode that read the set it
overwrites.

value = (K and V vectors quantised + keys scored) per second of the whole step.
roofline = the dominant kernel (kvq_quantize_kv): algorithmic bytes per launch
(fp16 input, packed codes, fp32 norms) / mean launch duration from HIP events
recorded on the stream the kernels run on, in a pass before the warm-up and
timed steps: as many launches of the kernel as there are timed steps, back
to back over the same rotating sets, replayed from a captured HIP graph
between two events, after 100 ms of untimed replays (the GPU's clocks settle
under load) (events between the kernels would otherwise sit inside
the timed steps, and an event around every launch adds its own marker and
dispatch gap).  traffic = HBM bytes per launch from the committed rocprofv3
counter record for the same kernel source, or null when the kernel source
has changed since the counters were taken.

rows = every step of the path on its own workload (all sizes full), timed the
same way (warmed graph replays over rotating buffer sets, the last launch
checked against an eager one), each with its algorithmic bytes (and flops
where the matrix cores do the work) and the fraction of the matching MI355X
peak.  The two 4096-vector rows measure latency instead: events around each
eager launch.

cpu_baseline = the CPU oracle (plain C, double precision) on the same step,
once on one thread and once on every host thread the process is given (the
unchanged oracle on (batch, KV head) slices from a thread pool); the value is
the all-thread rate, with the thread count and the CPU model.  Rows carry
their own single-thread oracle sample rates.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, GB/s
FP16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
D = 128
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "kvq_quantize_kv_l8b32k_b3_traffic.md")
TRACE_RECORD = os.path.join(ROOT, "profiles", "kvq_step_l8b32k_b3_kernel_trace.md")
QUANT_SRC = os.path.join(ROOT, "calibration_free_kv_amd", "csrc", "kvq_quantize.hip")


def rec_bytes(bits):
    return 16 * bits + 4  # packed codes + fp32 norm per vector


def quant_bytes(n_vec, bits, qjl=False):
    """fp16 read + codes and norm written (+ 16 B signs and 4 B gamma with QJL)."""
    return n_vec * (2 * D + rec_bytes(bits) + (20 if qjl else 0))


def decode_bytes(n_tok_heads, bits):
    return n_tok_heads * 2 * rec_bytes(bits)  # K and V records of every (token, KV head)


def logits_bytes(n_keys, Hq_per_kv, bits, qjl=False):
    return n_keys * (rec_bytes(bits) + (20 if qjl else 0) + 4 * Hq_per_kv)


def nsn_bytes(n_vec):
    return n_vec * (2 * D + 16 + 8)  # x read once (algorithmic), codes + s1 + s2 written


def source_sha(path):
    """sha256 of a source's code: comments and blank lines removed, so that a
    record stays valid across edits of comments only."""
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in txt.splitlines()]
    return hashlib.sha256("\n".join(ln for ln in lines if ln.strip()).encode()).hexdigest()


def read_record(path, key):
    """A value of a committed rocprofv3 record, if the record is current (its
    code_sha256 is that of the quantize kernel's source code)."""
    try:
        txt = open(path).read()
    except OSError:
        return None
    m = dict(re.findall(r"^- (\w+): `?([^`\n]+)`?$", txt, re.M))
    if m.get("code_sha256") != source_sha(QUANT_SRC):
        return None
    try:
        return float(m[key])
    except (KeyError, ValueError):
        return None


def read_traffic():
    """Bytes per launch from the committed counter record, if it is current."""
    return read_record(TRAFFIC_RECORD, "traffic_bytes_per_launch")


class Timer:
    """Mean duration of launches, from HIP events on the launching stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def run(self, launch, reps, warmup):
        torch = self.torch
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record(self.stream)
            launch(warmup + i)
            ev[i][1].record(self.stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        return float(ms.mean()), float(np.percentile(ms, 10)), float(np.percentile(ms, 90))


def run_graph(timer, launch, reps, per_graph=10, check=None, warm_s=0.1):
    """Mean duration of back-to-back launches replayed from a HIP graph (no
    host launch cost in the timed region): per_graph launches are captured
    once; each timed replay is bracketed by events.  check(), if given,
    compares the replayed result with an eager one.  Before the timed
    replays the graph is replayed, untimed, for warm_s seconds: capturing and
    instantiating it leaves the GPU idle long enough for its clocks to drop,
    and they take tens of milliseconds of load to settle again."""
    torch = timer.torch
    for i in range(3):
        launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            launch(i)
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        if check is not None:
            check()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        g.replay()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(timer.stream)
        g.replay()
        ev[i][1].record(timer.stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev]) / per_graph
    del g
    return float(ms.mean()), float(np.percentile(ms, 10)), float(np.percentile(ms, 90))


def eager_check(timer, launch, i, outs):
    """check() for run_graph: the tensors outs, as the replays left them,
    equal what an eager launch(i) writes (i = the graph's last launch, the
    last writer of outs)."""
    torch = timer.torch

    def check():
        got = [t.clone() for t in outs]
        launch(i)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(got, outs)), "graph replay differs from the eager launch"
    return check


def row(ms, p10, p90, nbytes=None, flops=None, **extra):
    r = {"ms": ms, "p10_ms": p10, "p90_ms": p90}
    if nbytes is not None:
        gbs = nbytes / (ms * 1e-3) / 1e9
        r.update({"bytes_per_launch": nbytes, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS})
    if flops is not None:
        tf = flops / (ms * 1e-3) / 1e12
        r.update({"flops_per_launch": flops, "TFLOP/s": tf, "frac_fp16_mfma": tf / FP16_MFMA_TFLOPS})
    r.update(extra)
    return r


def oracle_rate(fn, units, budget_s=2.0):
    """units per second of the oracle on a bounded sample (repeats until budget_s)."""
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 3:
            return reps * units / el


# --------------------------------------------------------------------------- main step
def host_threads():
    """Host threads for the all-core oracle run: the CPU share the process is
    given (OMP_NUM_THREADS where set, else the affinity mask)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_step(inp, bits, threads):
    """One step of the oracle on the workload: quantise K and V, decode
    attention from the codes.  With threads > 1 the unchanged oracle runs on
    (batch, KV head) slices from a thread pool (its C routines run without
    the interpreter lock)."""
    import oracle as O
    B, Hkv, T = inp["k"].shape[:3]
    G = inp["Hq"] // Hkv
    jobs = [(b, h) for b in range(B) for h in range(Hkv)]

    def one(job):
        b, h = job
        sl = (slice(b, b + 1), slice(h, h + 1))
        rk = O.quantize(inp["k"][sl], inp["signs_k"][h:h + 1], bits)
        rv = O.quantize(inp["v"][sl], inp["signs_v"][h:h + 1], bits)
        return O.attention(inp["q"][b:b + 1, G * h:G * h + G], rk["codes"], rk["norms"], rv["codes"],
                           rv["norms"], inp["signs_k"][h:h + 1], inp["signs_v"][h:h + 1], bits)

    if threads == 1:
        for j in jobs:
            one(j)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, jobs))


def cpu_baseline(inp, bits, budget_s=10.0):
    """The oracle on the same workload: one thread, then all the host threads
    the process is given (the reported value)."""
    B, Hkv, T = inp["k"].shape[:3]
    n = B * Hkv * T
    out = {}
    for threads in (1, host_threads()):
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle_step(inp, bits, threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 3:
                break
        out[threads] = (reps, el, reps * 3 * n / el)
    thr = max(out)
    reps, el, rate = out[thr]
    return {"value": rate, "unit": "vectors/s", "cores": thr, "kind": "oracle",
            "sample": "%d full step(s) of the same workload (quantise %d K + %d V vectors, decode attention over "
                      "%d keys), %.1f s on %d thread(s); one thread: %.3g vectors/s" % (
                          reps, n, n, n, el, thr, out[1][2]),
            "single_thread_value": out[1][2], "cpu_model": cpu_model()}


def trace_roofline(qb):
    """The same roofline from the committed rocprofv3 kernel trace of this step
    (kernel durations only, without the gaps between launches that the events
    include), or None when the kernel source has changed since the trace."""
    us = read_record(TRACE_RECORD, "quantize_avg_us")
    if us is None:
        return None
    gbs = qb / (us * 1e-6) / 1e9
    return {"ms_per_launch": us * 1e-3, "achieved": gbs, "frac": gbs / HBM_PEAK_GBS,
            "source": "profiles/" + os.path.basename(TRACE_RECORD)}


def main_step(torch, kvq, synth, args, dev, timer):
    bits = 3
    inp = synth.make("l8b32k")
    B, Hkv, T = inp["k"].shape[:3]
    Hq = inp["Hq"]
    n = B * Hkv * T
    ctx = kvq.Context(Hkv, bits, inp["signs_k"], inp["signs_v"], device=dev.index)
    k0 = torch.from_numpy(inp["k"]).to(dev)
    v0 = torch.from_numpy(inp["v"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    nset = 4
    sets = []
    for _ in range(nset):
        sets.append(dict(k=k0.clone(), v=v0.clone(),
                         kc=torch.empty((B, Hkv, T, 16 * bits), dtype=torch.uint8, device=dev),
                         kn=torch.empty((B, Hkv, T), dtype=torch.float32, device=dev),
                         vc=torch.empty((B, Hkv, T, 16 * bits), dtype=torch.uint8, device=dev),
                         vn=torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)))
    del k0, v0
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = ctx.decode_ws(B, Hq, T)
    stream = torch.cuda.current_stream(dev)
    for st in sets:  # every set holds valid codes before the first timed decode
        kvq.kvq_quantize_kv(ctx, st["k"], st["v"], B, Hkv, T, st["kc"], st["kn"], st["vc"], st["vn"])
    torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # Per-kernel durations for the roofline, measured first: K launches of
    # each kernel back to back over the rotating sets, captured once into a
    # HIP graph and replayed between two events on the launching stream, so
    # neither the host's launch cost nor an event between two launches sits
    # in the interval (an event around every launch adds its marker and the
    # dispatch gap to each one).
    def qlaunch(i):
        st = sets[i % nset]
        kvq.kvq_quantize_kv(ctx, st["k"], st["v"], B, Hkv, T, st["kc"], st["kn"], st["vc"], st["vn"])

    def dlaunch(i):
        sd = sets[i % nset]
        kvq.kvq_attn_decode(ctx, q, B, Hq, T, sd["kc"], sd["kn"], sd["vc"], sd["vn"], 0.0, out, ws)

    last = (args.steps - 1) % nset

    def check_quantize():  # the replay's codes of the last set equal an eager launch's
        got = sets[last]["kc"].clone(), sets[last]["vn"].clone()
        qlaunch(last)
        torch.cuda.synchronize()
        assert torch.equal(got[0], sets[last]["kc"]) and torch.equal(got[1], sets[last]["vn"]), \
            "graph replay differs from the eager launch"

    def check_decode():
        got = out.clone()
        dlaunch(last)
        torch.cuda.synchronize()
        assert torch.equal(got, out), "graph replay differs from the eager launch"

    # (run_graph replays each graph untimed for 100 ms first: the GPU's
    # clocks settle under load, and the timed steps after this pass see them
    # settled too; cold, the first replays of the quantize graph measured
    # 40.4 us per launch against 35.2 us after 100 ms of launches)
    q_ms = run_graph(timer, qlaunch, 5, args.steps, check=check_quantize)[0]
    d_ms = run_graph(timer, dlaunch, 5, args.steps, check=check_decode)[0]

    # The timed steps put each step's decode on a second stream, where it
    # overlaps the same step's quantize (they touch different buffer sets):
    # decode s waits for quantize s - 2, which wrote the codes it reads, and
    # quantize s waits for decode s - 2, the last reader of the set it
    # overwrites.  Both streams have the default priority.
    dstream = torch.cuda.Stream(device=dev)
    evq = {}
    evd = {}

    def step2(s):
        st = sets[s % nset]
        sd = sets[(s + nset // 2) % nset]
        if s - nset // 2 in evd:
            stream.wait_event(evd[s - nset // 2])
        kvq.kvq_quantize_kv(ctx, st["k"], st["v"], B, Hkv, T, st["kc"], st["kn"], st["vc"], st["vn"])
        evq[s] = torch.cuda.Event()
        evq[s].record(stream)
        if s - nset // 2 in evq:
            dstream.wait_event(evq[s - nset // 2])
        with torch.cuda.stream(dstream):
            kvq.kvq_attn_decode(ctx, q, B, Hq, T, sd["kc"], sd["kn"], sd["vc"], sd["vn"], 0.0, out, ws)
        evd[s] = torch.cuda.Event()
        evd[s].record(dstream)

    for s in range(args.warmup):
        step2(s)
    torch.cuda.synchronize()
    # The K timed steps carry no timing events of their own (an event between
    # the kernels would order them).
    t_start, t_end = E(), E()
    torch.cuda.synchronize()
    t_start.record(stream)
    dstream.wait_event(t_start)
    for s in range(args.steps):
        step2(args.warmup + s)
    done = torch.cuda.Event()
    done.record(dstream)
    stream.wait_event(done)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    evq.clear()
    evd.clear()


    qb = quant_bytes(2 * n, bits)
    db = decode_bytes(n, bits)
    q_gbs = qb / (q_ms * 1e-3) / 1e9
    d_gbs = db / (d_ms * 1e-3) / 1e9
    res = {
        "metric": "KV vectors quantized/s + keys scored/s (decode), % of HBM roofline, 1 GPU",
        "value": 3 * n / (ms_step * 1e-3),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped layer: batch %d, %d KV heads x 128, %d query heads, %d tokens, "
                               "%d-bit codes; quantise K+V, one decode step" % (B, Hkv, Hq, T, bits),
                   "bits": bits, "tokens": T, "kv_heads": Hkv, "q_heads": Hq, "batch": B, "buffer_sets": nset},
        "roofline": {"bound": "hbm", "achieved": q_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": q_gbs / HBM_PEAK_GBS, "traffic": read_traffic(), "kernel": "kvq_quantize_kv",
                     "bytes_per_launch": qb, "ms_per_launch": q_ms, "trace": trace_roofline(qb)},
        "kernels": {
            "kvq_quantize_kv": {"ms": q_ms, "GB/s": q_gbs, "frac_hbm": q_gbs / HBM_PEAK_GBS,
                                "vectors_per_s": 2 * n / (q_ms * 1e-3)},
            "kvq_attn_decode": {"ms": d_ms, "GB/s": d_gbs, "frac_hbm": d_gbs / HBM_PEAK_GBS,
                                "keys_per_s": n / (d_ms * 1e-3), "bytes_per_launch": db},
        },
        "step_frac_hbm": (qb + db) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    cpu_inp = inp
    del sets
    torch.cuda.empty_cache()
    return res, cpu_inp


# --------------------------------------------------------------------------- rows
def rows(torch, kvq, synth, dev, timer, reps, oracle_rates):
    import oracle as O
    out = {}
    rng_sets = lambda total_bytes: max(2, int(np.ceil(600e6 / max(total_bytes, 1))))  # noqa: E731

    def graph(launch, per_graph, outs):
        # launches 0 .. per_graph - 1 back to back from a warmed graph replay,
        # checked against an eager launch of the last one
        return run_graph(timer, launch, reps, per_graph, check=eager_check(timer, launch, per_graph - 1, outs))

    # l8b32k: quantize K+V and decode at b = 2, 3, 4
    inp = synth.make("l8b32k")
    B, Hkv, T = inp["k"].shape[:3]
    Hq, n = inp["Hq"], B * Hkv * T
    k0 = torch.from_numpy(inp["k"]).to(dev)
    v0 = torch.from_numpy(inp["v"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    xs = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(3)]
    for bits in (2, 3, 4):
        ctx = kvq.Context(Hkv, bits, inp["signs_k"], inp["signs_v"], device=dev.index)
        ns = rng_sets(decode_bytes(n, bits))
        cs = [[torch.empty((B, Hkv, T, 16 * bits), dtype=torch.uint8, device=dev),
               torch.empty((B, Hkv, T), dtype=torch.float32, device=dev),
               torch.empty((B, Hkv, T, 16 * bits), dtype=torch.uint8, device=dev),
               torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)] for _ in range(ns)]

        def quant(i):
            k, v = xs[i % len(xs)]
            c = cs[i % ns]
            kvq.kvq_quantize_kv(ctx, k, v, B, Hkv, T, c[0], c[1], c[2], c[3])
        out["quantize_kv_l8b32k_b%d" % bits] = row(*graph(quant, ns, cs[ns - 1]), nbytes=quant_bytes(2 * n, bits),
                                                    units_per_launch=2 * n, unit="vectors")
        outb = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        ws = ctx.decode_ws(B, Hq, T)

        def dec(i):
            c = cs[i % ns]
            kvq.kvq_attn_decode(ctx, q, B, Hq, T, c[0], c[1], c[2], c[3], 0.0, outb, ws)
        out["attn_decode_l8b32k_b%d" % bits] = row(*graph(dec, ns, [outb]), nbytes=decode_bytes(n, bits),
                                                    units_per_launch=n, unit="keys", buffer_sets=ns)
        del cs, ctx
    sub = {k: v[:, :, :2048] for k, v in inp.items() if k in ("k", "v")}
    oracle_rates["quantize_kv_l8b32k_b3"] = oracle_rate(
        lambda: O.quantize(sub["k"], inp["signs_k"], 3), B * Hkv * 2048)
    rq = O.quantize(sub["k"], inp["signs_k"], 3)
    rv = O.quantize(sub["v"], inp["signs_v"], 3)
    oracle_rates["attn_decode_l8b32k_b3"] = oracle_rate(
        lambda: O.attention(inp["q"], rq["codes"], rq["norms"], rv["codes"], rv["norms"], inp["signs_k"],
                            inp["signs_v"], 3), B * Hkv * 2048)
    # dense rotation (one Haar-random Q for every head), 3 bits
    ctx = kvq.Context(Hkv, 3, device=dev.index, rot_Q=synth.random_orthogonal(44).astype(np.float32))
    ns = rng_sets(decode_bytes(n, 3))
    cs = [[torch.empty((B, Hkv, T, 48), dtype=torch.uint8, device=dev),
           torch.empty((B, Hkv, T), dtype=torch.float32, device=dev),
           torch.empty((B, Hkv, T, 48), dtype=torch.uint8, device=dev),
           torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)] for _ in range(ns)]

    def quantd(i):
        k, v = xs[i % len(xs)]
        c = cs[i % ns]
        kvq.kvq_quantize_kv(ctx, k, v, B, Hkv, T, c[0], c[1], c[2], c[3])
    # the rotation on the matrix cores: 128 x 128 products, high and low parts of Q
    out["quantize_kv_dense_l8b32k_b3"] = row(*graph(quantd, ns, cs[ns - 1]), nbytes=quant_bytes(2 * n, 3),
                                             flops=2 * n * 2 * 2 * D * D, units_per_launch=2 * n, unit="vectors")
    outb = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = ctx.decode_ws(B, Hq, T)

    def decd(i):
        c = cs[i % ns]
        kvq.kvq_attn_decode(ctx, q, B, Hq, T, c[0], c[1], c[2], c[3], 0.0, outb, ws)
    out["attn_decode_dense_l8b32k_b3"] = row(*graph(decd, ns, [outb]), nbytes=decode_bytes(n, 3),
                                             units_per_launch=n, unit="keys", buffer_sets=ns)
    del cs, ctx
    del xs, k0, v0
    torch.cuda.empty_cache()

    # batch16: decode at b = 3 (and its quantize)
    inp = synth.make("batch16")
    B, Hkv, T = inp["k"].shape[:3]
    Hq, n = inp["Hq"], B * Hkv * T
    ctx = kvq.Context(Hkv, 3, inp["signs_k"], inp["signs_v"], device=dev.index)
    k0 = torch.from_numpy(inp["k"]).to(dev)
    v0 = torch.from_numpy(inp["v"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    ns = rng_sets(decode_bytes(n, 3))
    cs = [[torch.empty((B, Hkv, T, 48), dtype=torch.uint8, device=dev),
           torch.empty((B, Hkv, T), dtype=torch.float32, device=dev),
           torch.empty((B, Hkv, T, 48), dtype=torch.uint8, device=dev),
           torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)] for _ in range(ns)]

    def quant16(i):
        c = cs[i % ns]
        kvq.kvq_quantize_kv(ctx, k0, v0, B, Hkv, T, c[0], c[1], c[2], c[3])
    out["quantize_kv_batch16_b3"] = row(*graph(quant16, ns, cs[ns - 1]), nbytes=quant_bytes(2 * n, 3),
                                        units_per_launch=2 * n, unit="vectors")
    outb = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = ctx.decode_ws(B, Hq, T)

    def dec16(i):
        c = cs[i % ns]
        kvq.kvq_attn_decode(ctx, q, B, Hq, T, c[0], c[1], c[2], c[3], 0.0, outb, ws)
    out["attn_decode_batch16_b3"] = row(*graph(dec16, ns, [outb]), nbytes=decode_bytes(n, 3),
                                        units_per_launch=n, unit="keys", buffer_sets=ns)
    del cs, k0, v0, ctx
    torch.cuda.empty_cache()

    # long128k_qjl: quantize K with the QJL residual, logits for 32 query heads
    inp = synth.make("long128k_qjl")
    B, Hkv, T = inp["k"].shape[:3]
    Hq, n = inp["Hq"], B * Hkv * T
    ctx = kvq.Context(Hkv, 2, inp["signs_k"], inp["signs_v"], mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=inp["S"],
                      device=dev.index)
    k0 = torch.from_numpy(inp["k"]).to(dev)
    ks = [k0, k0.clone()]
    q = torch.from_numpy(inp["q"]).to(dev)
    lb = logits_bytes(n, Hq // Hkv, 2, qjl=True)
    ns = rng_sets(lb)
    cs = [dict(codes=torch.empty((B, Hkv, T, 32), dtype=torch.uint8, device=dev),
               norms=torch.empty((B, Hkv, T), dtype=torch.float32, device=dev),
               qjl_signs=torch.empty((B, Hkv, T, 16), dtype=torch.uint8, device=dev),
               qjl_gamma=torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)) for _ in range(ns)]

    def qjl(i):
        c = cs[i % ns]
        kvq.kvq_quantize(ctx, kvq.KVQ_KIND_K, ks[i % 2], B, Hkv, T, c["codes"], c["norms"], c["qjl_signs"],
                         c["qjl_gamma"])
    out["quantize_qjl_long128k_b2"] = row(*graph(qjl, ns, list(cs[ns - 1].values())), nbytes=quant_bytes(n, 2, qjl=True),
                                          flops=n * 2 * D * D, units_per_launch=n, unit="vectors",
                                          note="flops = the S r projection, 2 d^2 per key")
    lo = [torch.empty((B, Hq, T), dtype=torch.float32, device=dev) for _ in range(2)]

    def lg(i):
        c = cs[i % ns]
        kvq.kvq_logits(ctx, q, B, Hq, T, c["codes"], c["norms"], c["qjl_signs"], c["qjl_gamma"], lo[i % 2])
    out["logits_qjl_long128k_b2"] = row(*graph(lg, ns, [lo[(ns - 1) % 2]]), nbytes=lb, units_per_launch=n * Hq,
                                        unit="logits", buffer_sets=ns)
    # the same workload with the dense rotation (TurboQuant's Estagio 1 + 2)
    Qd = synth.random_orthogonal(31).astype(np.float32)
    ctxd = kvq.Context(Hkv, 2, inp["signs_k"], inp["signs_v"], mode=kvq.KVQ_MODE_MSE_QJL, qjl_S=inp["S"],
                       rot_Q=Qd, device=dev.index)

    def qjld(i):
        c = cs[i % ns]
        kvq.kvq_quantize(ctxd, kvq.KVQ_KIND_K, ks[i % 2], B, Hkv, T, c["codes"], c["norms"], c["qjl_signs"],
                         c["qjl_gamma"])
    out["quantize_qjl_dense_long128k_b2"] = row(*graph(qjld, ns, list(cs[ns - 1].values())), nbytes=quant_bytes(n, 2, qjl=True),
                                                flops=n * 2 * (2 * D * D + 2 * D * D), units_per_launch=n,
                                                unit="vectors",
                                                note="flops = rotation (Q as two fp16 parts) and projection "
                                                     "(e as two fp16 parts), 2 d^2 each per part")

    def lgd(i):
        c = cs[i % ns]
        kvq.kvq_logits(ctxd, q, B, Hq, T, c["codes"], c["norms"], c["qjl_signs"], c["qjl_gamma"], lo[i % 2])
    out["logits_qjl_dense_long128k_b2"] = row(*graph(lgd, ns, [lo[(ns - 1) % 2]]), nbytes=lb, units_per_launch=n * Hq,
                                              unit="logits", buffer_sets=ns)
    del ctxd
    kk = inp["k"][:, :, :1024]

    def oracle_qjl():
        r = O.quantize(kk, inp["signs_k"], 2, want_y=True)
        return r, O.qjl(r["y"], r["idx"], inp["S"], 2)
    oracle_rates["quantize_qjl_long128k_b2"] = oracle_rate(oracle_qjl, B * Hkv * 1024)
    r, rj = oracle_qjl()
    oracle_rates["logits_qjl_long128k_b2"] = oracle_rate(
        lambda: O.logits(inp["q"], r["codes"], r["norms"], inp["signs_k"], 2, 1, rj["signs"], rj["gamma"], inp["S"]),
        B * Hq * 1024)
    del ks, k0, cs, lo, ctx
    torch.cuda.empty_cache()

    # tiny: latency of quantize and logits (one head, 4096 keys)
    inp = synth.make("tiny")
    B, Hkv, T = inp["k"].shape[:3]
    ctx = kvq.Context(Hkv, 3, inp["signs_k"], inp["signs_v"], device=dev.index)
    k0 = torch.from_numpy(inp["k"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    c = ctx.quantize(kvq.KVQ_KIND_K, k0)
    lt = torch.empty((B, inp["Hq"], T), dtype=torch.float32, device=dev)
    out["quantize_tiny_b3"] = row(*timer.run(lambda i: ctx.quantize(kvq.KVQ_KIND_K, k0, out=c), reps, 5),
                                  nbytes=quant_bytes(T, 3), note="latency-bound (4096 vectors)")
    out["logits_tiny_b3"] = row(*timer.run(lambda i: kvq.kvq_logits(ctx, q, B, inp["Hq"], T, c["codes"], c["norms"],
                                                                    None, None, lt), reps, 5),
                                nbytes=logits_bytes(T, 1, 3), note="latency-bound (4096 logits)")
    del ctx

    # nsn_vq: NSN + Hadamard + 8-dim VQ over 8 heads x 65536 tokens
    inp = synth.make("nsn_vq")
    H, T = inp["x"].shape[:2]
    cb = np.loadtxt(os.path.join(ROOT, "tests", "golden", "vq_codebook_256x8.txt"), dtype=np.float32).reshape(256, 8)
    ctx = kvq.Context(H, 1, mode=kvq.KVQ_MODE_NSN_VQ, vq_codebook=cb, device=dev.index)
    x0 = torch.from_numpy(inp["x"]).to(dev)
    xsn = [x0] + [x0.clone() for _ in range(3)]
    o = ctx.nsn_vq_quantize(x0)
    ws = torch.empty(int(kvq.lib().kvq_nsn_vq_ws_bytes(ctx.handle, H, T)), dtype=torch.uint8, device=dev)
    def nenc(i):
        ctx.nsn_vq_quantize(xsn[i % 4], out=o, ws=ws)
    out["nsn_vq_8x65536"] = row(*graph(nenc, 4, list(o.values())),
                                nbytes=nsn_bytes(H * T), flops=H * T * 16 * 256 * 8 * 2, units_per_launch=H * T,
                                unit="vectors", note="three launches (stats, mean, search); x is read twice; "
                                "flops = exhaustive distances 16 x 256 x 8 x 2 per vector")
    oracle_rates["nsn_vq_8x65536"] = oracle_rate(lambda: O.nsn_vq(inp["x"][:1, :1024], cb), 1024)
    # with the adaptive scale and the cosine-refined codebook
    cbc = np.loadtxt(os.path.join(ROOT, "tests", "golden", "vq_codebook_256x8_cos.txt"),
                     dtype=np.float32).reshape(256, 8)
    ctxa = kvq.Context(H, 1, mode=kvq.KVQ_MODE_NSN_VQ, vq_codebook=cbc, nsn_options=kvq.KVQ_NSN_ADAPTIVE_SCALE,
                       device=dev.index)
    def nenca(i):
        ctxa.nsn_vq_quantize(xsn[i % 4], out=o, ws=ws)
    out["nsn_vq_adaptive_8x65536"] = row(*graph(nenca, 4, list(o.values())),
                                         nbytes=nsn_bytes(H * T), flops=H * T * 16 * 256 * 8 * 2,
                                         units_per_launch=H * T, unit="vectors",
                                         note="adaptive scale folded into s2, cosine-refined codebook")
    del xsn, x0, ctxa

    # NSN-VQ scoring from codes: logits and one decode step, 8 KV heads x 65536
    # keys, 32 query heads; stand-in encoded K and V from the seeded generator
    Hq = 32
    n = H * T
    per_set = n * 2 * (16 + 8)
    ns = rng_sets(per_set)
    dv = lambda e: {k: torch.from_numpy(v).to(dev) for k, v in e.items()}  # noqa: E731
    kv = [(dv(synth.random_nsn_codes(40 + 2 * i, (1, H, T))), dv(synth.random_nsn_codes(41 + 2 * i, (1, H, T))))
          for i in range(ns)]
    qn = torch.from_numpy(synth.random_tensor(42, (1, Hq, D))).to(dev)
    lgo = torch.empty((1, Hq, T), dtype=torch.float32, device=dev)
    dout = torch.empty((1, Hq, D), dtype=torch.float32, device=dev)
    wsd = ctx.nsn_decode_ws(1, Hq, T)

    def nlg(i):
        ctx.nsn_logits(qn, **kv[i % ns][0], out=lgo)

    def ndec(i):
        ctx.nsn_attn_decode(qn, kv[i % ns][0], kv[i % ns][1], ws=wsd, out=dout)

    def same(fn, res):
        def check():
            got = res.clone()
            fn(0)
            torch.cuda.synchronize()
            assert torch.equal(got, res), "graph replay differs from the eager launch"
        return check
    last = ns - 1
    out["nsn_logits_8x65536_g4"] = row(*run_graph(timer, nlg, reps, ns, check=same(lambda i: nlg(last), lgo)),
                                       nbytes=n * (16 + 8 + 4 * Hq // H), units_per_launch=n, unit="keys",
                                       buffer_sets=ns, note="16 table lookups per key serve 4 heads")
    out["nsn_attn_decode_8x65536_g4"] = row(*run_graph(timer, ndec, reps, ns, check=same(lambda i: ndec(last), dout)),
                                            nbytes=n * 2 * (16 + 8), units_per_launch=n, unit="keys",
                                            buffer_sets=ns, note="two launches (splits, merge)")
    e = synth.random_nsn_codes(40, (1, H, 1024))
    f = synth.random_nsn_codes(41, (1, H, 1024))
    qh = synth.random_tensor(42, (1, Hq, D))
    oracle_rates["nsn_logits_8x65536_g4"] = oracle_rate(
        lambda: O.nsn_logits(qh, e["codes"], e["s1"], e["s2"], e["o"], cb), H * 1024)
    oracle_rates["nsn_attn_decode_8x65536_g4"] = oracle_rate(
        lambda: O.nsn_attention(qh, e["codes"], e["s1"], e["s2"], e["o"], f["codes"], f["s1"], f["s2"], f["o"], cb),
        H * 1024)
    del kv

    # double-quantised byproducts (4-bit s1 per 32 tokens, 4-bit means): the
    # encoder over 8 heads x 65536 tokens and decode from such codes
    x0 = torch.from_numpy(inp["x"]).to(dev)
    xsn = [x0] + [x0.clone() for _ in range(3)]
    odq = ctx.nsn_vq_quantize_dq(x0)
    wsq = torch.empty(int(kvq.lib().kvq_nsn_vq_dq_ws_bytes(ctx.handle, H, T)), dtype=torch.uint8, device=dev)
    dq_meta = H * T * (0.5 + 8 / 32) + H * (64 + 8)  # s1 nibbles and block pairs, mean nibbles and pairs
    def nencq(i):
        ctx.nsn_vq_quantize_dq(xsn[i % 4], out=odq, ws=wsq)
    out["nsn_vq_dq_8x65536"] = row(*graph(nencq, 4, list(odq.values())),
                                   nbytes=H * T * (2 * D + 16 + 4) + dq_meta, flops=H * T * 16 * 256 * 8 * 2,
                                   units_per_launch=H * T, unit="vectors",
                                   note="three launches; 4-bit s1 (32-token blocks) and means")
    del xsn, x0
    per_set = n * 2 * (16 + 4.75)
    ns = rng_sets(per_set)
    kvd = [(dv(synth.random_nsn_dq_codes(70 + 2 * i, (1, H, T))), dv(synth.random_nsn_dq_codes(71 + 2 * i, (1, H, T))))
           for i in range(ns)]

    def ndecq(i):
        ctx.nsn_attn_decode_dq(qn, kvd[i % ns][0], kvd[i % ns][1], ws=wsd, out=dout)
    last = ns - 1
    out["nsn_attn_decode_dq_8x65536_g4"] = row(
        *run_graph(timer, ndecq, reps, ns, check=same(lambda i: ndecq(last), dout)),
        nbytes=n * 2 * (16 + 4.75), units_per_launch=n, unit="keys", buffer_sets=ns,
        note="s1 read as 4-bit codes with per-block pairs")
    del kvd

    # gain-shape residual quantisation on the NSN front end (12-byte records):
    # the encoder over 8 heads x 65536 tokens, logits and decode from
    # stand-in records
    gl = [ln.split() for ln in open(os.path.join(ROOT, "tests", "golden", "gsrq_tables_256x32.txt"))
          if not ln.startswith("#")]
    gtab = dict(S1=np.array(gl[0:256], np.float32), G1=np.array(gl[256], np.float32),
                S2=np.array(gl[257:513], np.float32), G2=np.array(gl[513], np.float32))
    ctxg = kvq.Context(H, 1, mode=kvq.KVQ_MODE_GSRQ, gsrq_tables=gtab, device=dev.index)
    x0 = torch.from_numpy(inp["x"]).to(dev)
    xsn = [x0] + [x0.clone() for _ in range(3)]
    og = ctxg.gsrq_quantize(x0)
    wsg = torch.empty(int(kvq.lib().kvq_gsrq_ws_bytes(ctxg.handle, H, T)), dtype=torch.uint8, device=dev)
    def genc(i):
        ctxg.gsrq_quantize(xsn[i % 4], out=og, ws=wsg)
    out["gsrq_8x65536"] = row(*graph(genc, 4, list(og.values())),
                              nbytes=H * T * (2 * D + 12 + 8), flops=H * T * 2 * 4 * 256 * 32 * 2,
                              units_per_launch=H * T, unit="vectors",
                              note="three launches (stats, mean, search); two stages of 256 shapes per 32-dim "
                              "sub-vector on the vector ALUs; x is read twice")
    del xsn, x0
    n = H * T
    ns = rng_sets(n * 2 * (12 + 8))
    kvg = [(dv(synth.random_gsrq_codes(110 + 2 * i, (1, H, T))), dv(synth.random_gsrq_codes(111 + 2 * i, (1, H, T))))
           for i in range(ns)]

    def glg(i):
        e = kvg[i % ns][0]
        ctxg.gsrq_logits(qn, e["codes"], e["s1"], e["s2"], e["o"], out=lgo)

    def gdec(i):
        ctxg.gsrq_attn_decode(qn, kvg[i % ns][0], kvg[i % ns][1], ws=wsd, out=dout)
    last = ns - 1
    out["gsrq_logits_8x65536_g4"] = row(*run_graph(timer, glg, reps, ns, check=same(lambda i: glg(last), lgo)),
                                        nbytes=n * (12 + 8 + 4 * Hq // H), units_per_launch=n, unit="keys",
                                        buffer_sets=ns, note="8 table lookups per key serve 4 heads")
    out["gsrq_attn_decode_8x65536_g4"] = row(*run_graph(timer, gdec, reps, ns, check=same(lambda i: gdec(last), dout)),
                                             nbytes=n * 2 * (12 + 8), units_per_launch=n, unit="keys",
                                             buffer_sets=ns, note="two launches (splits, merge)")
    del kvg, ctxg

    # streaming NSN-VQ cache: 65408 packed tokens in flush groups of 128 (each
    # with its own means) plus a 100-token fp16 window, 8 KV heads, 32 query
    # heads; and the flush of one 128-token group of the window
    Gs, T_cap, T_s, R_cap, R_s = 128, 65536, 65408, 128, 100
    n = H * T_s
    ns = rng_sets(n * 2 * (16 + 8))
    kvs = [(dv(synth.random_nsn_codes(80 + 2 * i, (1, H, T_cap), n_groups=T_cap // Gs)),
            dv(synth.random_nsn_codes(81 + 2 * i, (1, H, T_cap), n_groups=T_cap // Gs))) for i in range(ns)]
    wins = [(torch.from_numpy(synth.random_tensor(84 + 2 * i, (1, H, R_cap, D))).to(dev),
             torch.from_numpy(synth.random_tensor(85 + 2 * i, (1, H, R_cap, D))).to(dev)) for i in range(ns)]
    wss = ctx.nsn_stream_ws(1, Hq, T_cap)
    wsf = torch.empty(int(kvq.lib().kvq_nsn_flush_ws_bytes(ctx.handle, 1, Gs)), dtype=torch.uint8, device=dev)

    def nsdec(i):
        k, v = kvs[i % ns]
        kt, vt = wins[i % ns]
        ctx.nsn_attn_decode_stream(qn, k, v, T_s, Gs, kt, vt, R_s, ws=wss, out=dout)

    def nsflush(i):
        k, v = kvs[i % ns]
        kt, vt = wins[i % ns]
        ctx.nsn_flush(kt, vt, Gs, k, v, T_s, ws=wsf)
    last = ns - 1
    out["nsn_attn_decode_stream_8x65408_g4"] = row(
        *run_graph(timer, nsdec, reps, ns, check=same(lambda i: nsdec(last), dout)),
        nbytes=n * 2 * (16 + 8) + H * (T_s // Gs) * 2 * D * 4 + H * R_s * 2 * 2 * D, units_per_launch=n + H * R_s,
        unit="keys", buffer_sets=ns, note="per-group means; three launches (window, splits, merge)")
    out["nsn_flush_group128"] = row(*run_graph(timer, nsflush, reps, ns), nbytes=2 * H * Gs * (2 * D + 24),
                                    units_per_launch=2 * H * Gs, unit="vectors", buffer_sets=ns,
                                    note="K and V, three launches each; latency-bound (2048 vectors)")
    del kvs, wins, ctx

    # streaming cache: decode over 32704 packed tokens (of 32768 slots) plus a
    # 64-token fp16 window, and the flush of a 64-token window (b = 3, 8 KV
    # heads, 32 query heads); stand-in packed codes from the seeded generator
    inp = synth.make("l8b32k", T=1)
    Hkv, Hq, T_cap, T_s, R_cap, R_s = 8, 32, 32768, 32704, 128, 64
    ctx = kvq.Context(Hkv, 3, inp["signs_k"], inp["signs_v"], device=dev.index)
    n = Hkv * T_s
    ns = rng_sets(n * 2 * rec_bytes(3))
    dv = lambda e: {k: torch.from_numpy(v).to(dev) for k, v in e.items()}  # noqa: E731
    k0, v0 = dv(synth.random_codes(60, (1, Hkv, T_cap), 3)), dv(synth.random_codes(61, (1, Hkv, T_cap), 3))
    kt0 = torch.from_numpy(synth.random_tensor(90, (1, Hkv, R_cap, D))).to(dev)
    vt0 = torch.from_numpy(synth.random_tensor(91, (1, Hkv, R_cap, D))).to(dev)
    cl = lambda e: {k: v.clone() for k, v in e.items()}  # noqa: E731
    pk = [(cl(k0), cl(v0)) for _ in range(ns)]
    win = [(kt0.clone(), vt0.clone()) for _ in range(ns)]
    qs = torch.from_numpy(synth.random_tensor(43, (1, Hq, D))).to(dev)
    sout = torch.empty((1, Hq, D), dtype=torch.float32, device=dev)
    sws = ctx.stream_ws(1, Hq, T_cap)

    def sdec(i):
        k, v = pk[i % ns]
        kt, vt = win[i % ns]
        ctx.attn_decode_stream(qs, k["codes"], k["norms"], v["codes"], v["norms"], T_s, kt, vt, R_s, ws=sws, out=sout)

    def sflush(i):
        k, v = pk[i % ns]
        kt, vt = win[i % ns]
        ctx.flush(kt, vt, R_s, k["codes"], k["norms"], v["codes"], v["norms"], T_s)
    last = ns - 1
    out["attn_decode_stream_l8b32k_b3"] = row(
        *run_graph(timer, sdec, reps, ns, check=same(lambda i: sdec(last), sout)),
        nbytes=n * 2 * rec_bytes(3) + Hkv * R_s * 2 * 2 * D, units_per_launch=n + Hkv * R_s, unit="keys",
        buffer_sets=ns, note="32704 packed + 64 fp16 window tokens per KV head; two launches")
    out["flush_window64_b3"] = row(*run_graph(timer, sflush, reps, ns), nbytes=quant_bytes(2 * Hkv * R_s, 3),
                                   units_per_launch=2 * Hkv * R_s, unit="vectors", buffer_sets=ns,
                                   note="latency-bound (1024 vectors)")
    del pk, win, ctx
    torch.cuda.empty_cache()
    return out


def calibrate_copy(torch, dev, nbytes=256 << 20, reps=3):
    """A plain device copy of known size, for scaling rocprofv3's byte counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy": {"bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes,
                                         "copies": reps}}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--row-reps", type=int, default=20)
    ap.add_argument("--no-rows", action="store_true", help="time only the main step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true", help="run a 256 MiB device copy and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    from calibration_free_kv_amd import kvq, synth

    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        calibrate_copy(torch, dev)
        return
    timer = Timer(torch, torch.cuda.current_stream(dev))
    res, cpu_inp = main_step(torch, kvq, synth, args, dev, timer)
    if not args.no_rows:
        orates = {}
        res["rows"] = rows(torch, kvq, synth, dev, timer, args.row_reps, orates)
        for k, v in orates.items():
            res["rows"][k]["oracle_units_per_s"] = v
            res["rows"][k]["oracle_cores"] = 1
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cpu_inp, 3)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
