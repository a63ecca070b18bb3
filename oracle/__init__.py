"""CPU oracle for the rotate-then-quantize KV-cache path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  It wraps ``kvq_oracle.c`` (plain C, IEEE double) through ctypes and
shares no code with the GPU library.  See the header of ``kvq_oracle.c`` for the
page sections each routine follows.  The seeded sign generator (SplitMix64) is
written here in Python integers.

Array conventions: fp16 inputs are widened exactly to float64 here; codes are
packed LSB-first per vector (coordinate i in bits [b*i, b*i+b)).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

BAND = 1e-5  # decision-boundary band inside which code mismatches are allowed


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fast; no GPU needed)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        _setup(_lib)
    return _lib


_D = C.POINTER(C.c_double)
_F = C.POINTER(C.c_float)
_U8 = C.POINTER(C.c_uint8)
_I8 = C.POINTER(C.c_int8)
_I32 = C.POINTER(C.c_int32)
_I64 = C.POINTER(C.c_int64)
i64 = C.c_int64


def _setup(L):
    L.kvqo_lloyd_max.argtypes = [C.c_int, _D, C.c_int, C.c_double, _D, C.POINTER(C.c_int)]
    L.kvqo_gauss_mse.argtypes = [C.c_int, _D, _D]
    L.kvqo_gauss_mse.restype = C.c_double
    L.kvqo_tables_f32.argtypes = [C.c_int, _F, _F]
    L.kvqo_beta_mass.argtypes = [C.c_int, C.c_double, C.c_double]
    L.kvqo_beta_mass.restype = C.c_double
    L.kvqo_lloyd_max_beta.argtypes = [C.c_int, C.c_int, C.c_int, C.c_double, _D, C.POINTER(C.c_int)]
    L.kvqo_beta_mse.argtypes = [C.c_int, C.c_int, _D, _D]
    L.kvqo_beta_mse.restype = C.c_double
    L.kvqo_tables_f32_beta.argtypes = [C.c_int, C.c_int, _F, _F]
    L.kvqo_hadamard_entry.argtypes = [C.c_int, C.c_int]
    L.kvqo_hadamard_dense.argtypes = [_D, _D, C.c_int]
    L.kvqo_fwht.argtypes = [_D, C.c_int]
    L.kvqo_pack.argtypes = [_I32, C.c_int, C.c_int, _U8]
    L.kvqo_unpack.argtypes = [_U8, C.c_int, C.c_int, _I32]
    L.kvqo_scalar_quantize.argtypes = [_D, i64, C.c_int, _F, _F, _I32, _D]
    L.kvqo_quantize.argtypes = [C.c_int, C.c_int, i64, i64, i64, _D, _I8, _F, C.c_double,
                                _U8, _D, _D, _I32, _U8]
    L.kvqo_dequant.argtypes = [C.c_int, C.c_int, _U8, C.c_double, _I8, _F, _D]
    L.kvqo_logits.argtypes = [C.c_int, C.c_int, C.c_int, i64, i64, i64, i64, _D, _U8, _D, _I8,
                              _F, _U8, _D, _D, C.c_int, _D]
    L.kvqo_attention.argtypes = [C.c_int, C.c_int, i64, i64, i64, i64, _D, _U8, _D, _U8, _D,
                                 _I8, _I8, _F, C.c_double, _D]
    L.kvqo_attention_stream.argtypes = [C.c_int, C.c_int, i64, i64, i64, i64, i64, _D, _U8, _D, _U8, _D, _D,
                                        _D, _I8, _I8, _F, C.c_double, _D]
    L.kvqo_quantize_dense.argtypes = [C.c_int, C.c_int, i64, i64, i64, _D, _D, _F, C.c_double, _U8, _D, _D, _I32,
                                      _U8]
    L.kvqo_dequant_dense.argtypes = [C.c_int, C.c_int, _U8, C.c_double, _D, _F, _D]
    L.kvqo_logits_dense.argtypes = [C.c_int, C.c_int, C.c_int, i64, i64, i64, i64, _D, _U8, _D, _D, _F, _U8, _D,
                                    _D, C.c_int, _D]
    L.kvqo_attention_dense.argtypes = [C.c_int, C.c_int, i64, i64, i64, i64, _D, _U8, _D, _U8, _D, _D, _F,
                                       C.c_double, _D]
    L.kvqo_qjl.argtypes = [C.c_int, C.c_int, i64, _D, _I32, _F, _D, C.c_double, _U8, _D, _U8]
    L.kvqo_nsn_vq.argtypes = [C.c_int, C.c_int, C.c_int, i64, i64, _D, _D, C.c_double, _U8, _D,
                              _D, _D, _D, _U8, _D, C.c_int]
    L.kvqo_nsn_reconstruct.argtypes = [C.c_int, _D, C.c_double, C.c_double, _D, _D]
    L.kvqo_nsn_logits.argtypes = [C.c_int, C.c_int, C.c_int, i64, i64, i64, i64, _D, _U8, _D, _D, _D,
                                  _D, _D]
    L.kvqo_nsn_attention.argtypes = [C.c_int, C.c_int, i64, i64, i64, i64, _D, _U8, _D, _D, _D, _U8,
                                     _D, _D, _D, _D, C.c_double, _D]
    L.kvqo_nsn_attention_stream.argtypes = [C.c_int, C.c_int, i64, i64, i64, i64, i64, i64, _D, _U8, _D, _D, _D,
                                            _U8, _D, _D, _D, _D, _D, _D, C.c_double, _D]
    L.kvqo_kmeans.argtypes = [i64, C.c_int, C.c_int, _D, _I64, C.c_int, _D, _D]
    L.kvqo_kmeans.restype = C.c_int
    L.kvqo_dq4.argtypes = [i64, _D, C.c_double, _U8, _D, _D, _U8]
    L.kvqo_nsn_front.argtypes = [C.c_int, i64, i64, _D, _D, _D, _D, _D, _D]
    L.kvqo_gskm.argtypes = [i64, C.c_int, C.c_int, _D, _I64, C.c_int, _D, _D]
    L.kvqo_lloyd_1d.argtypes = [i64, _D, C.c_int, C.c_int, _D]
    L.kvqo_gsrq_encode.argtypes = [i64, C.c_int, C.c_int, C.c_int, _D, _D, _D, _D, _D, C.c_double, _U8, _D, _U8]
    L.kvqo_gsrq_logits.argtypes = [C.c_int, C.c_int, C.c_int, i64, i64, i64, i64, _D, _U8, _D, _D, _D, _D, _D, _D,
                                   _D, _D]
    L.kvqo_gsrq_attention.argtypes = [C.c_int, C.c_int, i64, i64, i64, i64, _D, _U8, _D, _D, _D, _U8, _D, _D, _D,
                                      _D, _D, _D, _D, C.c_double, _D]
    L.kvqo_cosine_refine.argtypes = [i64, C.c_int, C.c_int, _D, _D, C.c_int, _D]
    L.kvqo_cosine_refine.restype = C.c_int


def _p(a, ty):
    return a.ctypes.data_as(ty) if a is not None else None


def _f64(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _chk(rc):
    if rc != 0:
        raise ValueError("oracle routine rejected its arguments (rc=%d)" % rc)


# --------------------------------------------------------------------------- tables
def lloyd_max(bits: int, init=None, max_iter: int = 1_000_000, tol: float = 1e-13):
    """Fixed point of Lloyd's conditions for N(0,1); returns (centroids, iterations)."""
    L = 1 << bits
    c = np.zeros(L)
    it = C.c_int(0)
    ini = None if init is None else _f64(init)
    _chk(lib().kvqo_lloyd_max(bits, _p(ini, _D), max_iter, tol, _p(c, _D), C.byref(it)))
    return c, it.value


def gauss_mse(bits: int, c, t) -> float:
    return lib().kvqo_gauss_mse(bits, _p(_f64(c), _D), _p(_f64(t), _D))


def _tables(bits: int, codebook: str):
    if codebook == "gauss":
        return tables_f32(bits)
    if codebook == "beta":
        return tables_f32_beta(bits)
    raise ValueError(codebook)


def beta_mass(d: int, a: float, b: float) -> float:
    """int_a^b (1 - y^2/d)^((d-3)/2) dy (unnormalised law of sqrt(d) u_i)."""
    return lib().kvqo_beta_mass(d, a, b)


def lloyd_max_beta(bits: int, d: int = 128, max_iter: int = 1_000_000, tol: float = 1e-13):
    """Lloyd-Max centroids for the coordinate law of a uniform unit vector in
    R^d scaled by sqrt(d); returns (centroids, iterations)."""
    c = np.zeros(1 << bits)
    it = C.c_int(0)
    _chk(lib().kvqo_lloyd_max_beta(bits, d, max_iter, tol, _p(c, _D), C.byref(it)))
    return c, it.value


def beta_mse(bits: int, c, t, d: int = 128) -> float:
    return lib().kvqo_beta_mse(bits, d, _p(_f64(c), _D), _p(_f64(t), _D))


def tables_f32_beta(bits: int, d: int = 128):
    """Canonical fp32 centroids and thresholds of the exact-d law."""
    L = 1 << bits
    c = np.zeros(L, np.float32)
    t = np.zeros(L - 1, np.float32)
    _chk(lib().kvqo_tables_f32_beta(bits, d, _p(c, _F), _p(t, _F)))
    return c, t


def tables_f32(bits: int):
    """Canonical fp32 centroids [2^b] and thresholds [2^b - 1]."""
    L = 1 << bits
    c = np.zeros(L, np.float32)
    t = np.zeros(L - 1, np.float32)
    _chk(lib().kvqo_tables_f32(bits, _p(c, _F), _p(t, _F)))
    return c, t


# --------------------------------------------------------------------------- Hadamard
def hadamard_dense(x):
    x = _f64(x)
    y = np.zeros_like(x)
    lib().kvqo_hadamard_dense(_p(x, _D), _p(y, _D), x.shape[0])
    return y


def hadamard_matrix(n: int):
    return np.array([[lib().kvqo_hadamard_entry(i, j) for j in range(n)] for i in range(n)],
                    dtype=np.int64)


def fwht(x):
    y = _f64(x).copy()
    lib().kvqo_fwht(_p(y, _D), y.shape[0])
    return y


# --------------------------------------------------------------------------- random signs
_M64 = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> int:
    """Output n (from 0) of SplitMix64 seeded with `seed` (Steele, Lea and Flood,
    "Fast splittable pseudorandom number generators", OOPSLA 2014): the state
    after n + 1 steps of the golden-gamma increment, passed through the
    variant-13 64-bit finaliser.  Python integers, reduced mod 2^64 by hand."""
    z = (seed + (n + 1) * 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def seeded_signs(seed: int, H: int, kind: int, d: int = 128):
    """Random-sign diagonal D ("PolarQuant", Methodology: the randomized
    Hadamard transform draws a random +-1 diagonal) of tensor `kind` (0 = K,
    1 = V) for H KV heads, drawn from a seed: coordinate i of head h is -1
    when the top bit of SplitMix64 output kind*2^32 + h*d + i is set."""
    out = np.empty((H, d), np.int8)
    for h in range(H):
        for i in range(d):
            out[h, i] = -1 if splitmix64(seed, (kind << 32) + h * d + i) >> 63 else 1
    return out


# --------------------------------------------------------------------------- packing
def pack(idx, bits: int):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    d = idx.shape[-1]
    flat = idx.reshape(-1, d)
    out = np.zeros((flat.shape[0], d * bits // 8), np.uint8)
    for v in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[v])
        rec = np.zeros(d * bits // 8, np.uint8)
        lib().kvqo_pack(_p(row, _I32), d, bits, _p(rec, _U8))
        out[v] = rec
    return out.reshape(idx.shape[:-1] + (d * bits // 8,))


def unpack(codes, d: int, bits: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rec = d * bits // 8
    flat = codes.reshape(-1, rec)
    out = np.zeros((flat.shape[0], d), np.int32)
    for v in range(flat.shape[0]):
        r = np.ascontiguousarray(flat[v])
        o = np.zeros(d, np.int32)
        lib().kvqo_unpack(_p(r, _U8), d, bits, _p(o, _I32))
        out[v] = o
    return out.reshape(codes.shape[:-1] + (d,))


def scalar_quantize(y, bits: int):
    c, t = tables_f32(bits)
    y = _f64(y).ravel()
    idx = np.zeros(y.size, np.int32)
    yh = np.zeros(y.size)
    lib().kvqo_scalar_quantize(_p(y, _D), y.size, bits, _p(c, _F), _p(t, _F), _p(idx, _I32),
                               _p(yh, _D))
    return idx, yh


# --------------------------------------------------------------------------- quantize
def quantize(x, signs, bits: int, band: float = BAND, want_y: bool = False, codebook: str = "gauss"):
    """x [B,H,T,d] (any float dtype; fp16 widened exactly); signs [H,d] (+-1).

    Returns dict(codes [B,H,T,d*b/8] u8, norms [B,H,T] f64, idx [B,H,T,d],
    flags [B,H,T,d] u8, y [B,H,T,d] (rotated coordinates) if want_y)."""
    x = _f64(x)
    B, H, T, d = x.shape
    signs = np.ascontiguousarray(signs, dtype=np.int8)
    assert signs.shape == (H, d)
    _, t = _tables(bits, codebook)
    codes = np.zeros((B, H, T, d * bits // 8), np.uint8)
    norms = np.zeros((B, H, T))
    idx = np.zeros((B, H, T, d), np.int32)
    flags = np.zeros((B, H, T, d), np.uint8)
    y = np.zeros((B, H, T, d)) if want_y else None
    _chk(lib().kvqo_quantize(d, bits, B, H, T, _p(x, _D), _p(signs, _I8), _p(t, _F), band,
                             _p(codes, _U8), _p(norms, _D), _p(y, _D), _p(idx, _I32),
                             _p(flags, _U8)))
    out = dict(codes=codes, norms=norms, idx=idx, flags=flags)
    if want_y:
        out["y"] = y
    return out


def dequant(rec, rho, signs_row, bits: int, d: int = 128):
    c, _ = tables_f32(bits)
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    s = np.ascontiguousarray(signs_row, dtype=np.int8)
    out = np.zeros(d)
    lib().kvqo_dequant(d, bits, _p(rec, _U8), float(rho), _p(s, _I8), _p(c, _F), _p(out, _D))
    return out


def logits(q, codes, norms, signs, bits: int, route: int = 1, qjl_signs=None, gamma=None,
           S=None, codebook: str = "gauss"):
    """q [B,Hq,d]; codes [B,Hkv,T,rec]; norms [B,Hkv,T]; signs [Hkv,d] -> [B,Hq,T]."""
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    _, Hkv, T, _ = codes.shape
    norms = _f64(norms)
    signs = np.ascontiguousarray(signs, dtype=np.int8)
    c, _ = _tables(bits, codebook)
    out = np.zeros((B, Hq, T))
    m = 0
    if qjl_signs is not None:
        qjl_signs = np.ascontiguousarray(qjl_signs, dtype=np.uint8)
        gamma = _f64(gamma)
        S = _f64(S)
        m = S.shape[0]
    _chk(lib().kvqo_logits(route, d, bits, B, Hq, Hkv, T, _p(q, _D), _p(codes, _U8),
                           _p(norms, _D), _p(signs, _I8), _p(c, _F), _p(qjl_signs, _U8),
                           _p(gamma, _D), _p(S, _D), m, _p(out, _D)))
    return out


def attention(q, kc, kn, vc, vn, signs_k, signs_v, bits: int, sm_scale: float | None = None,
              codebook: str = "gauss"):
    q = _f64(q)
    B, Hq, d = q.shape
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    _, Hkv, T, _ = kc.shape
    kn, vn = _f64(kn), _f64(vn)
    sk = np.ascontiguousarray(signs_k, dtype=np.int8)
    sv = np.ascontiguousarray(signs_v, dtype=np.int8)
    c, _ = _tables(bits, codebook)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d))
    _chk(lib().kvqo_attention(d, bits, B, Hq, Hkv, T, _p(q, _D), _p(kc, _U8), _p(kn, _D),
                              _p(vc, _U8), _p(vn, _D), _p(sk, _I8), _p(sv, _I8), _p(c, _F),
                              float(sm_scale), _p(out, _D)))
    return out


def attention_stream(q, kc, kn, vc, vn, k_tail, v_tail, signs_k, signs_v, bits: int,
                     sm_scale: float | None = None):
    """Attention over T quantised tokens (codes [B,Hkv,T,rec], norms [B,Hkv,T])
    followed by R full-precision ones (k_tail, v_tail [B,Hkv,R,d]) -> [B,Hq,d]."""
    q = _f64(q)
    B, Hq, d = q.shape
    kt, vt = _f64(k_tail), _f64(v_tail)
    Hkv, R = kt.shape[1], kt.shape[2]
    kc = np.ascontiguousarray(kc, dtype=np.uint8).reshape(B, Hkv, -1, d * bits // 8)
    vc = np.ascontiguousarray(vc, dtype=np.uint8).reshape(B, Hkv, -1, d * bits // 8)
    T = kc.shape[2]
    kn, vn = _f64(kn), _f64(vn)
    c, _ = tables_f32(bits)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d))
    _chk(lib().kvqo_attention_stream(d, bits, B, Hq, Hkv, T, R, _p(q, _D), _p(kc, _U8), _p(kn, _D), _p(vc, _U8),
                                     _p(vn, _D), _p(kt, _D), _p(vt, _D),
                                     _p(np.ascontiguousarray(signs_k, dtype=np.int8), _I8),
                                     _p(np.ascontiguousarray(signs_v, dtype=np.int8), _I8), _p(c, _F),
                                     float(sm_scale), _p(out, _D)))
    return out


def quantize_dense(x, Q, bits: int, band: float = BAND, want_y: bool = False, codebook: str = "gauss"):
    """As quantize, with the dense rotation y = sqrt(d) Q x / ||x|| (Q [d,d] orthogonal)."""
    x = _f64(x)
    B, H, T, d = x.shape
    Q = _f64(Q)
    _, t = _tables(bits, codebook)
    codes = np.zeros((B, H, T, d * bits // 8), np.uint8)
    norms = np.zeros((B, H, T))
    idx = np.zeros((B, H, T, d), np.int32)
    flags = np.zeros((B, H, T, d), np.uint8)
    y = np.zeros((B, H, T, d)) if want_y else None
    _chk(lib().kvqo_quantize_dense(d, bits, B, H, T, _p(x, _D), _p(Q, _D), _p(t, _F), band, _p(codes, _U8),
                                   _p(norms, _D), _p(y, _D), _p(idx, _I32), _p(flags, _U8)))
    out = dict(codes=codes, norms=norms, idx=idx, flags=flags)
    if want_y:
        out["y"] = y
    return out


def dequant_dense(rec, rho, Q, bits: int, d: int = 128, codebook: str = "gauss"):
    c, _ = _tables(bits, codebook)
    out = np.zeros(d)
    lib().kvqo_dequant_dense(d, bits, _p(np.ascontiguousarray(rec, dtype=np.uint8), _U8), float(rho), _p(_f64(Q), _D),
                             _p(c, _F), _p(out, _D))
    return out


def logits_dense(q, codes, norms, Q, bits: int, route: int = 1, codebook: str = "gauss", qjl_signs=None,
                 gamma=None, S=None):
    """As logits with the dense rotation Q; with qjl_signs/gamma/S, plus the
    QJL term of the residual in the rotated space."""
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    _, Hkv, T, _ = codes.shape
    c, _ = _tables(bits, codebook)
    out = np.zeros((B, Hq, T))
    m = 0
    if qjl_signs is not None:
        qjl_signs = np.ascontiguousarray(qjl_signs, dtype=np.uint8)
        gamma = _f64(gamma)
        S = _f64(S)
        m = S.shape[0]
    _chk(lib().kvqo_logits_dense(route, d, bits, B, Hq, Hkv, T, _p(q, _D), _p(codes, _U8), _p(_f64(norms), _D),
                                 _p(_f64(Q), _D), _p(c, _F), _p(qjl_signs, _U8), _p(gamma, _D), _p(S, _D), m,
                                 _p(out, _D)))
    return out


def attention_dense(q, kc, kn, vc, vn, Q, bits: int, sm_scale: float | None = None, codebook: str = "gauss"):
    q = _f64(q)
    B, Hq, d = q.shape
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    _, Hkv, T, _ = kc.shape
    c, _ = _tables(bits, codebook)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d))
    _chk(lib().kvqo_attention_dense(d, bits, B, Hq, Hkv, T, _p(q, _D), _p(kc, _U8), _p(_f64(kn), _D), _p(vc, _U8),
                                    _p(_f64(vn), _D), _p(_f64(Q), _D), _p(c, _F), float(sm_scale), _p(out, _D)))
    return out


def qjl(y, idx, S, bits: int, band: float = BAND):
    """y, idx [..., d]; S [m, d] -> dict(signs [..., m/8] u8, gamma [...], flags [..., m])."""
    y = _f64(y)
    d = y.shape[-1]
    lead = y.shape[:-1]
    n = int(np.prod(lead))
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    S = _f64(S)
    m = S.shape[0]
    c, _ = tables_f32(bits)
    sg = np.zeros((n, m // 8), np.uint8)
    gm = np.zeros(n)
    fl = np.zeros((n, m), np.uint8)
    _chk(lib().kvqo_qjl(d, m, n, _p(y, _D), _p(idx, _I32), _p(c, _F), _p(S, _D), band,
                        _p(sg, _U8), _p(gm, _D), _p(fl, _U8)))
    return dict(signs=sg.reshape(lead + (m // 8,)), gamma=gm.reshape(lead),
                flags=fl.reshape(lead + (m,)))


def nsn_vq(x, codebook, band: float = BAND, want_z: bool = False, o_given=None, adaptive: bool = False):
    """x [H,T,d]; codebook [K, sub] -> dict(codes [H,T,d/sub], s1, s2 [H,T], o [H,d], flags).
    o_given [H,d]: use this mean instead of the mean of the T tokens passed.
    adaptive: s2 carries the adaptive scale alpha = ||z||^2 / <z, zq>."""
    x = _f64(x)
    H, T, d = x.shape
    cb = _f64(codebook)
    K, sub = cb.shape
    codes = np.zeros((H, T, d // sub), np.uint8)
    s1 = np.zeros((H, T))
    s2 = np.zeros((H, T))
    o = np.zeros((H, d))
    z = np.zeros((H, T, d)) if want_z else None
    fl = np.zeros((H, T, d // sub), np.uint8)
    og = None if o_given is None else _f64(o_given)
    _chk(lib().kvqo_nsn_vq(d, sub, K, H, T, _p(x, _D), _p(cb, _D), band, _p(codes, _U8),
                           _p(s1, _D), _p(s2, _D), _p(o, _D), _p(z, _D), _p(fl, _U8), _p(og, _D),
                           int(adaptive)))
    out = dict(codes=codes, s1=s1, s2=s2, o=o, flags=fl)
    if want_z:
        out["z"] = z
    return out


BAND_DQ = 1e-4  # band of the 4-bit rounding decisions, in units of one step
DQ_BLOCK = 32   # tokens per block of s1 double quantisation


def dq4(v, band: float = BAND_DQ):
    """4-bit min-max quantisation of one block v [n] -> (codes u8 [n], lo, step,
    flags u8 [n]); the stored values are lo + codes * step."""
    v = _f64(v).ravel()
    code = np.zeros(v.shape[0], np.uint8)
    fl = np.zeros(v.shape[0], np.uint8)
    lo, step = C.c_double(), C.c_double()
    _chk(lib().kvqo_dq4(v.shape[0], _p(v, _D), band, _p(code, _U8), C.byref(lo), C.byref(step), _p(fl, _U8)))
    return code, lo.value, step.value, fl


def pack_nibbles(codes):
    """4-bit codes [..., n] -> bytes [..., ceil(n/2)]: code i in byte i // 2,
    the low nibble for even i."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    n = c.shape[-1]
    out = np.zeros(c.shape[:-1] + ((n + 1) // 2,), np.uint8)
    for i in range(n):
        out[..., i // 2] |= (c[..., i] & 15) << (4 * (i % 2))
    return out


def unpack_nibbles(packed, n: int):
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    return np.stack([(p[..., i // 2] >> (4 * (i % 2))) & 15 for i in range(n)], axis=-1).astype(np.uint8)


def nsn_mean(x):
    """Per-head channel mean o of a_t = sqrt(d) x_t / ||x_t|| (0 for a zero
    token) over the T tokens of x [H,T,d] (NSNQuant, Metodologia sec. 1)."""
    x = _f64(x)
    nx = np.linalg.norm(x, axis=-1, keepdims=True)
    a = np.where(nx > 0, np.sqrt(x.shape[-1]) * x / np.where(nx > 0, nx, 1.0), 0.0)
    return a.mean(axis=1)


def nsn_vq_dq(x, codebook, band: float = BAND, band_dq: float = BAND_DQ, block: int = DQ_BLOCK,
              want_z: bool = False, adaptive: bool = False, o_hat=None):
    """NSN-VQ with the byproducts double-quantised to 4 bits (NSNQuant,
    Metodologia sec. 3, "Double Quantization").  The steps in order: the mean o
    of the T tokens, its 4-bit form o_hat (one block of d channels per head),
    the shift and second normalisation with o_hat (so that x_hat = s1 (s2 H zq
    / sqrt(d) + o_hat) undoes the encoding), the codes, then s1 in 4-bit blocks
    of `block` tokens.  o_hat [H,d]: use this quantised mean instead (one of
    the admissible alternatives at flagged channels).  Returns nsn_vq's dict
    plus o_codes [H,d], o_lo, o_step [H], o_hat, o_flags, s1_codes [H,T],
    s1_lo, s1_step [H,ceil(T/block)], s1_hat [H,T], s1_flags, and the packed
    nibbles oq [H,d/2], s1q [H,ceil(T/2)]."""
    x = _f64(x)
    H, T, d = x.shape
    o = nsn_mean(x)
    oc = np.zeros((H, d), np.uint8)
    ofl = np.zeros((H, d), np.uint8)
    olo, ost = np.zeros(H), np.zeros(H)
    for h in range(H):
        oc[h], olo[h], ost[h], ofl[h] = dq4(o[h], band_dq)
    if o_hat is None:
        o_hat = olo[:, None] + oc * ost[:, None]
    r = nsn_vq(x, codebook, band=band, want_z=want_z, o_given=o_hat, adaptive=adaptive)
    nb = (T + block - 1) // block
    sc = np.zeros((H, T), np.uint8)
    sfl = np.zeros((H, T), np.uint8)
    slo, sst = np.zeros((H, nb)), np.zeros((H, nb))
    for h in range(H):
        for b in range(nb):
            sl = slice(b * block, min(T, (b + 1) * block))
            sc[h, sl], slo[h, b], sst[h, b], sfl[h, sl] = dq4(r["s1"][h, sl], band_dq)
    s1_hat = slo[:, np.arange(T) // block] + sc * sst[:, np.arange(T) // block]
    r.update(o=o, o_codes=oc, o_lo=olo, o_step=ost, o_hat=o_hat, o_flags=ofl, s1_codes=sc, s1_lo=slo,
             s1_step=sst, s1_hat=s1_hat, s1_flags=sfl, oq=pack_nibbles(oc), s1q=pack_nibbles(sc))
    return r


def dq_codebook(codebook, band: float = BAND_DQ):
    """The codebook's entries in 4 bits, one block over all of them -> (codes
    [K,sub], lo, step, flags, dequantised codebook [K,sub])."""
    cb = _f64(codebook)
    c, lo, step, fl = dq4(cb.ravel(), band)
    return c.reshape(cb.shape), lo, step, fl.reshape(cb.shape), (lo + c * step).reshape(cb.shape)


def nsn_reconstruct(zq, s1, s2, o):
    zq = _f64(zq)
    o = _f64(o)
    d = zq.shape[0]
    out = np.zeros(d)
    lib().kvqo_nsn_reconstruct(d, _p(zq, _D), float(s1), float(s2), _p(o, _D), _p(out, _D))
    return out


def nsn_logits(q, codes, s1, s2, o, codebook, route: int = 1):
    """q [B,Hq,d]; codes [B,Hkv,T,d/sub] u8; s1, s2 [B,Hkv,T]; o [B,Hkv,d];
    codebook [K,sub] -> logits [B,Hq,T] (route 1: reconstruct then dot;
    route 2: rotated query against the entries)."""
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    _, Hkv, T, _ = codes.shape
    cb = _f64(codebook)
    out = np.zeros((B, Hq, T))
    _chk(lib().kvqo_nsn_logits(route, d, cb.shape[1], B, Hq, Hkv, T, _p(q, _D), _p(codes, _U8),
                               _p(_f64(s1), _D), _p(_f64(s2), _D), _p(_f64(o), _D), _p(cb, _D),
                               _p(out, _D)))
    return out


def nsn_attention(q, kc, ks1, ks2, ko, vc, vs1, vs2, vo, codebook, sm_scale: float | None = None):
    """Decode attention over NSN-VQ keys and values (layouts as nsn_logits)
    -> out [B,Hq,d]."""
    q = _f64(q)
    B, Hq, d = q.shape
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    _, Hkv, T, _ = kc.shape
    cb = _f64(codebook)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d))
    args = [_f64(a) for a in (ks1, ks2, ko, vs1, vs2, vo)]
    _chk(lib().kvqo_nsn_attention(d, cb.shape[1], B, Hq, Hkv, T, _p(q, _D), _p(kc, _U8),
                                  _p(args[0], _D), _p(args[1], _D), _p(args[2], _D), _p(vc, _U8),
                                  _p(args[3], _D), _p(args[4], _D), _p(args[5], _D), _p(cb, _D),
                                  float(sm_scale), _p(out, _D)))
    return out


def nsn_attention_stream(q, kc, ks1, ks2, ko, vc, vs1, vs2, vo, k_tail, v_tail, codebook, Gs: int,
                         sm_scale: float | None = None):
    """Decode over an NSN-VQ streaming cache: T packed tokens (codes [B,Hkv,T,d/sub],
    s1/s2 [B,Hkv,T]) encoded in groups of Gs tokens with per-group means
    [B,Hkv,T/Gs,d], then R full-precision window tokens [B,Hkv,R,d] -> [B,Hq,d]."""
    q = _f64(q)
    B, Hq, d = q.shape
    kt, vt = _f64(k_tail), _f64(v_tail)
    Hkv, R = kt.shape[1], kt.shape[2]
    cb = _f64(codebook)
    sub = cb.shape[1]
    kc = np.ascontiguousarray(kc, dtype=np.uint8).reshape(B, Hkv, -1, d // sub)
    vc = np.ascontiguousarray(vc, dtype=np.uint8).reshape(B, Hkv, -1, d // sub)
    T = kc.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d))
    args = [_f64(a) for a in (ks1, ks2, ko, vs1, vs2, vo)]
    _chk(lib().kvqo_nsn_attention_stream(d, sub, B, Hq, Hkv, T, Gs, R, _p(q, _D), _p(kc, _U8), _p(args[0], _D),
                                         _p(args[1], _D), _p(args[2], _D), _p(vc, _U8), _p(args[3], _D),
                                         _p(args[4], _D), _p(args[5], _D), _p(kt, _D), _p(vt, _D), _p(cb, _D),
                                         float(sm_scale), _p(out, _D)))
    return out


def kmeans(samples, init_idx, max_iter: int = 100):
    """Lloyd's k-means; returns (codebook [K, dim], distortion per pass, passes)."""
    s = _f64(samples)
    n, dim = s.shape
    init_idx = np.ascontiguousarray(init_idx, dtype=np.int64)
    K = init_idx.shape[0]
    cb = np.zeros((K, dim))
    dist = np.zeros(max_iter)
    it = lib().kvqo_kmeans(n, dim, K, _p(s, _D), _p(init_idx, _I64), max_iter, _p(cb, _D),
                           _p(dist, _D))
    return cb, dist[:it], it


def cosine_refine(samples, codebook, passes: int = 10):
    """Cosine refinement of a codebook; returns (codebook, mean cosine per pass)."""
    s = _f64(samples)
    n, dim = s.shape
    cb = _f64(codebook).copy()
    mc = np.zeros(passes)
    it = lib().kvqo_cosine_refine(n, dim, cb.shape[0], _p(s, _D), _p(cb, _D), passes, _p(mc, _D))
    return cb, mc[:it]


# ---------------------------------------------------------------- GSRQ
GSRQ_M = 32  # sub-vector dimension of the GSRQ reading (4 sub-vectors per 128-dim vector)


def nsn_front(x, o_given=None):
    """NSN front end of x [H,T,d] -> dict(s1, s2 [H,T], o [H,d], z [H,T,d])."""
    x = _f64(x)
    H, T, d = x.shape
    s1, s2 = np.zeros((H, T)), np.zeros((H, T))
    o, z = np.zeros((H, d)), np.zeros((H, T, d))
    og = None if o_given is None else _f64(o_given)
    _chk(lib().kvqo_nsn_front(d, H, T, _p(x, _D), _p(og, _D), _p(s1, _D), _p(s2, _D), _p(o, _D), _p(z, _D)))
    return dict(s1=s1, s2=s2, o=o, z=z)


def gskm(samples, init_idx, passes: int = 20):
    """Gain-shape k-means: (unit shapes [K, m], mean best projection per pass)."""
    x = _f64(samples)
    n, m = x.shape
    init_idx = np.ascontiguousarray(init_idx, dtype=np.int64)
    K = init_idx.shape[0]
    shapes = np.zeros((K, m))
    obj = np.zeros(passes)
    it = lib().kvqo_gskm(n, m, K, _p(x, _D), _p(init_idx, _I64), passes, _p(shapes, _D), _p(obj, _D))
    return shapes, obj[:it]


def lloyd_1d(values, L: int, passes: int = 50):
    v = _f64(values).ravel()
    levels = np.zeros(L)
    _chk(lib().kvqo_lloyd_1d(v.shape[0], _p(v, _D), L, passes, _p(levels, _D)))
    return levels


def gsrq_train(samples, inits, L: int = 16, passes: int = 20):
    """Two GSRQ stages trained on samples [n, m]: per stage GSKM shapes (from
    the initial sample indices inits[k], K of them), then the gain levels from
    the best projections, then the residuals feed the next stage."""
    x = _f64(samples)
    out = {}
    r = x.copy()
    for k in (1, 2):
        S, obj = gskm(r, inits[k - 1], passes)
        p = r @ S.T
        j = np.argmax(p, axis=1)
        G = lloyd_1d(p[np.arange(r.shape[0]), j], L)
        codes, zhat, _ = gsrq_encode_stage_only(r, S, G)
        r = r - zhat
        out["S%d" % k], out["G%d" % k], out["objective%d" % k] = S, G, obj
    return out


def gsrq_encode_stage_only(z, S, G):
    """One stage (the second with zero gains) -> (codes, reproductions, flags)."""
    zero = np.zeros_like(G)
    return gsrq_encode(z, dict(S1=S, G1=G, S2=S, G2=zero))


def gsrq_encode(z, tab, band: float = BAND):
    """Sub-vectors z [n, m] -> (codes [n, 3] = (j1, j2, c1 | c2 << 4),
    reproductions [n, m], flags [n])."""
    z = _f64(z)
    n, m = z.shape
    S1, G1, S2, G2 = (_f64(tab[k]) for k in ("S1", "G1", "S2", "G2"))
    codes = np.zeros((n, 3), np.uint8)
    zhat = np.zeros((n, m))
    fl = np.zeros(n, np.uint8)
    _chk(lib().kvqo_gsrq_encode(n, m, S1.shape[0], G1.shape[0], _p(z, _D), _p(S1, _D), _p(G1, _D), _p(S2, _D),
                                _p(G2, _D), band, _p(codes, _U8), _p(zhat, _D), _p(fl, _U8)))
    return codes, zhat, fl


def gsrq_records(codes, P: int):
    """Per-sub-vector codes [..., P, 3] -> records [..., 3P]: the P stage-1
    shapes, the P stage-2 shapes, the P gain bytes."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return np.concatenate([c[..., 0], c[..., 1], c[..., 2]], axis=-1)


def gsrq_vq(x, tab, band: float = BAND, o_given=None):
    """GSRQ of x [H,T,d] on the NSN front end -> dict(codes [H,T,3P] records,
    s1, s2 [H,T], o [H,d], z, zhat [H,T,d], flags [H,T,P])."""
    f = nsn_front(x, o_given)
    H, T, d = f["z"].shape
    m = _f64(tab["S1"]).shape[1]
    P = d // m
    codes, zhat, fl = gsrq_encode(f["z"].reshape(-1, m), tab, band)
    f.update(codes=gsrq_records(codes.reshape(H, T, P, 3), P), zhat=zhat.reshape(H, T, d), flags=fl.reshape(H, T, P))
    return f


def _gsrq_tabs(tab):
    return [_f64(tab[k]) for k in ("S1", "G1", "S2", "G2")]


def gsrq_logits(q, codes, s1, s2, o, tab, route: int = 2):
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    _, Hkv, T, _ = codes.shape
    S1, G1, S2, G2 = _gsrq_tabs(tab)
    out = np.zeros((B, Hq, T))
    _chk(lib().kvqo_gsrq_logits(route, d, S1.shape[1], B, Hq, Hkv, T, _p(q, _D), _p(codes, _U8), _p(_f64(s1), _D),
                                _p(_f64(s2), _D), _p(_f64(o), _D), _p(S1, _D), _p(G1, _D), _p(S2, _D), _p(G2, _D),
                                _p(out, _D)))
    return out


def gsrq_attention(q, kc, ks1, ks2, ko, vc, vs1, vs2, vo, tab, sm_scale: float | None = None):
    q = _f64(q)
    B, Hq, d = q.shape
    kc = np.ascontiguousarray(kc, dtype=np.uint8)
    vc = np.ascontiguousarray(vc, dtype=np.uint8)
    _, Hkv, T, _ = kc.shape
    S1, G1, S2, G2 = _gsrq_tabs(tab)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d))
    a = [_f64(t) for t in (ks1, ks2, ko, vs1, vs2, vo)]
    _chk(lib().kvqo_gsrq_attention(d, S1.shape[1], B, Hq, Hkv, T, _p(q, _D), _p(kc, _U8), _p(a[0], _D),
                                   _p(a[1], _D), _p(a[2], _D), _p(vc, _U8), _p(a[3], _D), _p(a[4], _D),
                                   _p(a[5], _D), _p(S1, _D), _p(G1, _D), _p(S2, _D), _p(G2, _D), float(sm_scale),
                                   _p(out, _D)))
    return out
