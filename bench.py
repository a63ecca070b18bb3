"""Throughput of the KV-cache quantisation hot path on one MI355X.

One step = quantise the K and the V cache of one Llama-3-8B-shaped attention
layer (batch 1, 8 KV heads x 128, 32768 tokens, fp16) to b-bit codes with
kvq_quantize, then one decode step of attention for its 32 query heads
(GQA 4) read straight from the codes with kvq_attn_decode.  Inputs are
synthetic (seeded N(0,1) x per-channel lognormal(0,1) scales) and resident in
HBM before timing starts; the step rotates over several input/output sets
larger than twice the 256 MiB last-level cache, so data are not served from it.

Prints one JSON line.  value = (K and V vectors quantised + keys scored) per
second of the whole step.  The roofline object refers to kvq_quantize, the
dominant kernel: algorithmic bytes per launch (fp16 input, packed codes and
fp32 norms) divided by its mean launch duration from HIP events recorded on
the kernels' stream during the timed steps.  cpu_baseline times the CPU
oracle (plain C, double precision, one thread) on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def algorithmic_bytes(n_vec, bits):
    quant = 2 * n_vec * (256 + 16 * bits + 4)      # per launch (K and V together)
    decode = n_vec * 2 * (16 * bits + 4)           # K and V records of every token
    return quant, decode


def cpu_baseline(inp, bits, budget_s=10.0):
    import oracle as O
    B, Hkv, T = inp["k"].shape[:3]
    t0 = time.perf_counter()
    reps = 0
    while True:
        rk = O.quantize(inp["k"], inp["signs_k"], bits)
        rv = O.quantize(inp["v"], inp["signs_v"], bits)
        O.attention(inp["q"], rk["codes"], rk["norms"], rv["codes"], rv["norms"], inp["signs_k"],
                    inp["signs_v"], bits)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 3:
            break
    n = B * Hkv * T
    return {"value": reps * 3 * n / el, "unit": "vectors/s", "cores": 1, "kind": "oracle",
            "sample": "%d full step(s) of the same workload (quantise %d K + %d V vectors, decode "
                      "attention over %d keys), %.1f s, single thread" % (reps, n, n, n, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--bits", type=int, default=3, choices=[2, 3, 4])
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    from calibration_free_kv_amd import kvq, synth

    dev = torch.device("cuda", 0)
    bits = args.bits
    inp = synth.make("l8b32k")
    B, Hkv, T = inp["k"].shape[:3]
    Hq = inp["Hq"]
    n = B * Hkv * T
    ctx = kvq.Context(Hkv, bits, inp["signs_k"], inp["signs_v"], device=0)
    k0 = torch.from_numpy(inp["k"]).to(dev)
    v0 = torch.from_numpy(inp["v"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    sets = []
    for i in range(args.sets):
        sets.append(dict(k=k0.clone(), v=v0.clone(),
                         kc=torch.empty((B, Hkv, T, 16 * bits), dtype=torch.uint8, device=dev),
                         kn=torch.empty((B, Hkv, T), dtype=torch.float32, device=dev),
                         vc=torch.empty((B, Hkv, T, 16 * bits), dtype=torch.uint8, device=dev),
                         vn=torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)))
    del k0, v0
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    ws = ctx.decode_ws(B, Hq, T)
    torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    stream = torch.cuda.current_stream(dev)

    def step(s, ev=None):
        st = sets[s % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        kvq.kvq_quantize_kv(ctx, st["k"], st["v"], B, Hkv, T, st["kc"], st["kn"], st["vc"], st["vn"])
        if ev is not None:
            ev[1].record(stream)
        kvq.kvq_attn_decode(ctx, q, B, Hq, T, st["kc"], st["kn"], st["vc"], st["vn"], 0.0, out, ws)
        if ev is not None:
            ev[2].record(stream)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    evs = [[E() for _ in range(3)] for _ in range(args.steps)]
    t_start, t_end = E(), E()
    t_start.record(stream)
    for s in range(args.steps):
        step(s, evs[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    q_ms = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    d_ms = np.mean([e[1].elapsed_time(e[2]) for e in evs])

    qb, db = algorithmic_bytes(n, bits)
    q_gbs = qb / (q_ms * 1e-3) / 1e9
    d_gbs = db / (d_ms * 1e-3) / 1e9
    value = 3 * n / (ms_step * 1e-3)
    res = {
        "metric": "KV vectors quantized/s + keys scored/s (decode), % of HBM roofline, 1 GPU",
        "value": value,
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
        "config": {"workload": "Llama-3-8B-shaped layer: batch %d, %d KV heads x 128, %d query heads, "
                               "%d tokens, %d-bit codes; quantise K+V, one decode step" % (B, Hkv, Hq, T, bits),
                   "bits": bits, "tokens": T, "kv_heads": Hkv, "q_heads": Hq, "batch": B,
                   "buffer_sets": args.sets},
        "roofline": {"bound": "hbm", "achieved": q_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": q_gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "kvq_quantize",
                     "bytes_per_launch": qb, "ms_per_launch": q_ms},
        "kernels": {
            "kvq_quantize": {"ms": q_ms, "GB/s": q_gbs, "frac_hbm": q_gbs / HBM_PEAK_GBS,
                             "vectors_per_s": 2 * n / (q_ms * 1e-3), "launch": "kvq_quantize_kv (K and V)"},
            "kvq_attn_decode": {"ms": d_ms, "GB/s": d_gbs, "frac_hbm": d_gbs / HBM_PEAK_GBS,
                                "keys_per_s": n / (d_ms * 1e-3), "bytes_per_launch": db},
        },
        "step_frac_hbm": (qb + db) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, bits)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
