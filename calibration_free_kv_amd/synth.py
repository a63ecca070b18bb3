"""Seeded synthetic inputs for the KV-cache quantisation path.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic.  The GPU path and the CPU oracle both consume what it
produces, so the same bits reach both.  Random quantities the method itself
draws (the random-sign diagonals D of the randomized Hadamard transform, the
Gaussian QJL projection S, the k-means seed points) are produced here too and
passed to both sides as inputs.

Workloads (the shapes of one Llama-3-8B-like attention layer and its
variants; sizes given with each):

  tiny           1 KV head x 4096 tokens, d=128, K ~ N(0,1) with 4 outlier
                 channels scaled x20; one query head; 3-bit codes
  l8b32k         batch 1, 8 KV heads, 32 query heads (GQA 4), 32768 tokens;
                 K and V = N(0,1) x per-channel lognormal(0,1) scale;
                 2-, 3- and 4-bit codes; one decode step
  batch16        batch 16 x 8192 tokens, otherwise as l8b32k; 3-bit codes
  long128k_qjl   batch 1, 131072 tokens, 8 KV heads, 32 query heads;
                 2-bit codes + 1-bit QJL residual with a 128x128 projection
  nsn_vq         8 heads x 65536 tokens, NSN + Hadamard + 8-dim VQ with a
                 256-entry codebook

Recipe: each workload has a seed (its position in the list above);
``numpy.random.SeedSequence(seed).spawn(8)`` gives independent PCG64
streams for [K data, V data, K scales, V scales, query, D_K, D_V, S].  Values
are drawn in float64 and cast once to float16 (round to nearest even).  The
lognormal scale is one factor per (tensor, KV head, channel), shared by all
tokens and batch entries.  The QJL projection S has N(0,1) entries rounded to
the nearest fp16 value.  The tiny workload's 4 outlier channels are the
first 4 entries of a permutation of 128 drawn with seed 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 128


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hkv: int
    Hq: int
    T: int
    bits: tuple
    dist: str  # "outlier" or "lognormal"
    qjl: bool = False
    nsn: bool = False
    kinds: tuple = ("K", "V")
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1, 1, 4096, (3,), "outlier", kinds=("K",)),
    "l8b32k": Workload("l8b32k", 1, 1, 8, 32, 32768, (2, 3, 4), "lognormal"),
    "batch16": Workload("batch16", 2, 16, 8, 32, 8192, (3,), "lognormal"),
    "long128k_qjl": Workload("long128k_qjl", 3, 1, 8, 32, 131072, (2,), "lognormal", qjl=True,
                             kinds=("K",)),
    "nsn_vq": Workload("nsn_vq", 4, 1, 8, 8, 65536, (1,), "lognormal", nsn=True, kinds=("K",)),
}


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(8)]


def _kv(rng_data, rng_scale, B, H, T, dist, chunk_tokens=4096):
    out = np.empty((B, H, T, D), np.float16)
    if dist == "lognormal":
        scale = np.exp(rng_scale.standard_normal((H, D)))
    else:
        scale = np.ones((H, D))
        ch = np.random.Generator(np.random.PCG64(0)).permutation(D)[:4]
        scale[:, ch] = 20.0
    for b in range(B):
        for h in range(H):
            for t0 in range(0, T, chunk_tokens):
                t1 = min(T, t0 + chunk_tokens)
                x = rng_data.standard_normal((t1 - t0, D)) * scale[h]
                out[b, h, t0:t1] = x.astype(np.float16)
    return out


def random_signs(rng, H, d=D):
    return np.where(rng.integers(0, 2, size=(H, d)) == 1, 1, -1).astype(np.int8)


def make(name: str, T: int | None = None, B: int | None = None, with_v: bool | None = None):
    """Inputs of a workload; T and B may be shrunk for oracle-sized tests.

    Returns dict with k (and v) [B,Hkv,T,128] fp16, q [B,Hq,128] fp16,
    signs_k / signs_v [Hkv,128] int8 (+-1), S [128,128] fp32 (QJL) and
    x [Hkv,T,128] fp16 for the NSN workload."""
    w = WORKLOADS[name]
    T = w.T if T is None else T
    B = w.B if B is None else B
    r = _streams(w.seed)
    out = dict(workload=w, B=B, T=T, Hkv=w.Hkv, Hq=w.Hq)
    if w.nsn:
        out["x"] = _kv(r[0], r[2], 1, w.Hkv, T, w.dist)[0]
        return out
    out["k"] = _kv(r[0], r[2], B, w.Hkv, T, w.dist)
    if with_v if with_v is not None else ("V" in w.kinds):
        out["v"] = _kv(r[1], r[3], B, w.Hkv, T, w.dist)
    out["q"] = r[4].standard_normal((B, w.Hq, D)).astype(np.float16)
    out["signs_k"] = random_signs(r[5], w.Hkv)
    out["signs_v"] = random_signs(r[6], w.Hkv)
    if w.qjl:
        # N(0,1) entries rounded to the nearest fp16 value (then held as fp32)
        out["S"] = r[7].standard_normal((D, D)).astype(np.float16).astype(np.float32)
    return out


def gaussian_samples(seed: int, n: int, dim: int = 8):
    """N(0, I_dim) samples (float64) and K distinct seed indices for k-means."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((n, dim))


def kmeans_init(seed: int, n: int, K: int = 256):
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    return rng.choice(n, size=K, replace=False).astype(np.int64)


def random_tensor(seed: int, shape, scale: float = 1.0, dtype=np.float16):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(shape) * scale).astype(dtype)


def random_codes(seed: int, lead, bits: int, qjl_m: int = 0):
    """Stand-in encoded keys for scoring at full size (no quantizer involved):
    uniform packed code bytes [*lead, 16*bits], norms exp(N(3.4, 0.25^2)) (the
    spread of ||x|| for the lognormal-scaled 128-vectors above), and with
    qjl_m > 0 uniform sign bytes [*lead, qjl_m/8] and gamma ~ U(0.2, 0.5)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lead = tuple(lead)
    out = dict(codes=rng.integers(0, 256, size=lead + (16 * bits,), dtype=np.uint8),
               norms=np.exp(rng.normal(3.4, 0.25, size=lead)).astype(np.float32))
    if qjl_m:
        out["qjl_signs"] = rng.integers(0, 256, size=lead + (qjl_m // 8,), dtype=np.uint8)
        out["qjl_gamma"] = rng.uniform(0.2, 0.5, size=lead).astype(np.float32)
    return out


def random_nsn_codes(seed: int, lead, d: int = D, sub: int = 8, o_scale: float = 0.5, n_groups=None):
    """Stand-in NSN-VQ encoded vectors (no quantizer involved): entry indices
    uniform over 256 [*lead, d/sub] u8, s1 = exp(N(1, 0.25^2)), s2 ~ U(0.6, 1.0)
    (both fp32 [*lead]), and channel means o ~ N(0, o_scale^2) fp32
    [*lead[:-1], d] (one per head; larger than zero-mean data gives, so that
    the mean term is exercised), or [*lead[:-1], n_groups, d] (one per flush
    group of a streaming cache)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lead = tuple(lead)
    og = () if n_groups is None else (int(n_groups),)
    return dict(codes=rng.integers(0, 256, size=lead + (d // sub,), dtype=np.uint8),
                s1=np.exp(rng.normal(1.0, 0.25, size=lead)).astype(np.float32),
                s2=rng.uniform(0.6, 1.0, size=lead).astype(np.float32),
                o=(rng.standard_normal(lead[:-1] + og + (d,)) * o_scale).astype(np.float32))


def random_nsn_dq_codes(seed: int, lead, d: int = D, sub: int = 8, block: int = 32):
    """Stand-in NSN-VQ encoded vectors with 4-bit byproducts (no quantizer
    involved): entry indices uniform [*lead, d/sub] u8, s2 ~ U(0.6, 1.0) fp32
    [*lead], s1 as uniform 4-bit codes packed two per byte [*lead[:-1],
    ceil(T/2)] with per-block (lo, step) fp32 [*lead[:-1], ceil(T/block), 2],
    lo = exp(N(0.8, 0.2^2)), step ~ U(0.02, 0.06), and the means as uniform
    4-bit codes [*lead[:-1], d/2] with (lo, step) [*lead[:-1], 2], lo ~
    U(-1.2, -0.8), step ~ U(0.1, 0.16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lead = tuple(lead)
    T = lead[-1]
    rows = lead[:-1]
    nb = (T + block - 1) // block
    s1p = np.stack([np.exp(rng.normal(0.8, 0.2, size=rows + (nb,))), rng.uniform(0.02, 0.06, size=rows + (nb,))],
                   axis=-1).astype(np.float32)
    op = np.stack([rng.uniform(-1.2, -0.8, size=rows), rng.uniform(0.1, 0.16, size=rows)], axis=-1).astype(np.float32)
    return dict(codes=rng.integers(0, 256, size=lead + (d // sub,), dtype=np.uint8),
                s1q=rng.integers(0, 256, size=rows + ((T + 1) // 2,), dtype=np.uint8), s1p=s1p,
                s2=rng.uniform(0.6, 1.0, size=lead).astype(np.float32),
                oq=rng.integers(0, 256, size=rows + (d // 2,), dtype=np.uint8), op=op)


def random_gsrq_codes(seed: int, lead, d: int = D):
    """Stand-in GSRQ records (no quantizer involved): 12 uniform bytes per
    vector [*lead, 12] (4 stage-1 and 4 stage-2 shape indices, 4 gain bytes),
    with s1, s2 and the means drawn as random_nsn_codes draws them."""
    e = random_nsn_codes(seed, lead, d)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    e["codes"] = rng.integers(0, 256, size=tuple(lead) + (12,), dtype=np.uint8)
    return e


def random_orthogonal(seed: int, d: int = D):
    """A Haar-random orthogonal d x d matrix (float64): QR of a seeded N(0,1)
    matrix with the signs of R's diagonal moved into Q."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))[None, :]
