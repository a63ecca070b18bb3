"""Thin Python binding of libkvq (C ABI in include/kvq.h).

Every function here only checks tensor placement/dtype/shape, allocates
outputs with torch on the tensors' device and forwards plain pointers to the
library; all computation happens in the HIP kernels of libkvq.so.  There is no
CPU fallback: if the library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB selects another build of the library for the process; KVQ_DEBUG
# (set, and not "0") selects the bounds-checked libkvq_debug.so beside it
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(
    _PKG, "libkvq_debug.so" if os.environ.get("KVQ_DEBUG", "0") not in ("", "0") else "libkvq.so")

KVQ_OK, KVQ_E_INVAL, KVQ_E_UNSUPPORTED, KVQ_E_DEVICE, KVQ_E_NOMEM, KVQ_E_WORKSPACE = range(6)
KVQ_MODE_MSE, KVQ_MODE_MSE_QJL, KVQ_MODE_NSN_VQ = 0, 1, 2
KVQ_KIND_K, KVQ_KIND_V = 0, 1
KVQ_CODEBOOK_GAUSS, KVQ_CODEBOOK_BETA = 0, 1
KVQ_ROTATION_HADAMARD, KVQ_ROTATION_DENSE = 0, 1
KVQ_NSN_ADAPTIVE_SCALE = 1
KVQ_NSN_DQ_CODEBOOK = 2
KVQ_MODE_GSRQ = 3
D = 128

EXPORTS = [
    "kvq_create", "kvq_destroy", "kvq_get_tables", "kvq_codebook", "kvq_code_bytes_per_vec", "kvq_strerror",
    "kvq_quantize", "kvq_quantize_kv", "kvq_logits", "kvq_attn_decode_ws_bytes", "kvq_attn_decode",
    "kvq_attn_decode_splits", "kvq_nsn_vq_ws_bytes", "kvq_nsn_vq_quantize", "kvq_nsn_logits",
    "kvq_nsn_attn_decode_ws_bytes", "kvq_nsn_attn_decode", "kvq_nsn_attn_decode_splits",
    "kvq_attn_decode_stream_ws_bytes", "kvq_attn_decode_stream", "kvq_flush", "kvq_attn_decode_noalloc",
    "kvq_nsn_flush_ws_bytes", "kvq_nsn_flush", "kvq_nsn_attn_decode_stream_ws_bytes", "kvq_nsn_attn_decode_stream",
    "kvq_nsn_vq_dq_ws_bytes", "kvq_nsn_vq_quantize_dq", "kvq_nsn_logits_dq", "kvq_nsn_attn_decode_dq",
    "kvq_gsrq_ws_bytes", "kvq_gsrq_quantize", "kvq_gsrq_logits", "kvq_gsrq_attn_decode",
    "kvq_debug_build", "kvq_debug_take",
]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, strerror(status), status))


class kvq_config(C.Structure):
    _fields_ = [
        ("d", C.c_int32), ("bits", C.c_int32), ("mode", C.c_int32), ("n_kv_heads", C.c_int32),
        ("seed", C.c_uint64), ("signs_k", C.POINTER(C.c_int8)), ("signs_v", C.POINTER(C.c_int8)),
        ("qjl_S", C.POINTER(C.c_float)), ("vq_codebook", C.POINTER(C.c_float)),
        ("device", C.c_int32), ("codebook", C.c_int32), ("rotation", C.c_int32),
        ("rot_Q", C.POINTER(C.c_float)), ("nsn_options", C.c_int32), ("gsrq_tables", C.POINTER(C.c_float)),
    ]


_lib = None


def lib():
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so not found at %s; build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        vp, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        L.kvq_create.argtypes = [C.POINTER(kvq_config), C.POINTER(vp)]
        L.kvq_destroy.argtypes = [vp]
        L.kvq_get_tables.argtypes = [vp, vp, vp, vp, vp]
        L.kvq_codebook.argtypes = [i32, vp, vp]
        L.kvq_code_bytes_per_vec.argtypes = [vp]
        L.kvq_code_bytes_per_vec.restype = i64
        L.kvq_strerror.argtypes = [C.c_int]
        L.kvq_strerror.restype = C.c_char_p
        L.kvq_debug_build.argtypes = []
        L.kvq_debug_build.restype = i32
        L.kvq_debug_take.argtypes = []
        L.kvq_debug_take.restype = C.c_uint32
        L.kvq_quantize.argtypes = [vp, i32, vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.kvq_quantize_kv.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.kvq_logits.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.kvq_attn_decode_ws_bytes.argtypes = [vp, i64, i64, i64]
        L.kvq_attn_decode_ws_bytes.restype = sz
        L.kvq_attn_decode.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, C.c_float, vp, vp, sz, vp]
        L.kvq_attn_decode_splits.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, C.c_float, vp, vp,
                                             sz, i32, vp]
        L.kvq_attn_decode_noalloc.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, C.c_float, vp, vp]
        L.kvq_nsn_vq_ws_bytes.argtypes = [vp, i64, i64]
        L.kvq_nsn_vq_ws_bytes.restype = sz
        L.kvq_nsn_vq_quantize.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, vp, sz, vp]
        L.kvq_attn_decode_stream_ws_bytes.argtypes = [vp, i64, i64, i64]
        L.kvq_attn_decode_stream_ws_bytes.restype = sz
        L.kvq_attn_decode_stream.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, i64, i64, vp, vp,
                                             C.c_float, vp, vp, sz, vp]
        L.kvq_flush.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, i64, i64, vp]
        L.kvq_nsn_logits.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.kvq_nsn_attn_decode_ws_bytes.argtypes = [vp, i64, i64, i64]
        L.kvq_nsn_attn_decode_ws_bytes.restype = sz
        L.kvq_nsn_attn_decode.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, C.c_float, vp,
                                          vp, sz, vp]
        L.kvq_nsn_attn_decode_splits.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                                 C.c_float, vp, vp, sz, i32, vp]
        L.kvq_nsn_flush_ws_bytes.argtypes = [vp, i64, i64]
        L.kvq_nsn_flush_ws_bytes.restype = sz
        L.kvq_nsn_flush.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, sz,
                                    vp]
        L.kvq_nsn_attn_decode_stream_ws_bytes.argtypes = [vp, i64, i64, i64]
        L.kvq_nsn_attn_decode_stream_ws_bytes.restype = sz
        L.kvq_nsn_attn_decode_stream.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                                 i64, i64, vp, vp, C.c_float, vp, vp, sz, i32, vp]
        L.kvq_nsn_vq_dq_ws_bytes.argtypes = [vp, i64, i64]
        L.kvq_nsn_vq_dq_ws_bytes.restype = sz
        L.kvq_nsn_vq_quantize_dq.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.kvq_nsn_logits_dq.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp]
        L.kvq_nsn_attn_decode_dq.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             C.c_float, vp, vp, sz, i32, vp]
        L.kvq_gsrq_ws_bytes.argtypes = [vp, i64, i64]
        L.kvq_gsrq_ws_bytes.restype = sz
        L.kvq_gsrq_quantize.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, vp, sz, vp]
        L.kvq_gsrq_logits.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.kvq_gsrq_attn_decode.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, C.c_float, vp, vp,
                                           sz, i32, vp]
        _lib = L
    return _lib


def kvq_codebook(bits: int):
    """fp32 (centroids, thresholds) of the b-bit N(0,1) Lloyd-Max quantiser (no device needed)."""
    c = np.zeros(1 << bits, np.float32)
    t = np.zeros((1 << bits) - 1, np.float32)
    _check(lib().kvq_codebook(bits, c.ctypes.data_as(C.c_void_p), t.ctypes.data_as(C.c_void_p)),
           "kvq_codebook")
    return c, t


def strerror(status: int) -> str:
    return lib().kvq_strerror(status).decode()


def debug_build() -> bool:
    """True for the bounds-checked build (KVQ_DEBUG)."""
    return bool(lib().kvq_debug_build())


def debug_take() -> int:
    """First failed bounds check on the current device since the last call
    (file id << 16 | line; 0 if none), clearing the records (debug build;
    0 in others).  Call it after a device synchronisation."""
    return int(lib().kvq_debug_take())


def _check(status: int, what: str):
    if status != KVQ_OK:
        raise KvqError(status, what)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev_tensor(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


class Context:
    """A libkvq context (kvq_create/kvq_destroy) holding the b-bit tables, the
    random-sign diagonals of K and V per KV head, the QJL projection and the
    NSN codebook, resident on one GPU.  A diagonal left as None is generated
    by the library from `seed` (SplitMix64, as kvq.h specifies)."""

    def __init__(self, n_kv_heads: int, bits: int = 3, signs_k=None, signs_v=None, mode: int = KVQ_MODE_MSE,
                 qjl_S=None, vq_codebook=None, device: int = 0, seed: int = 0, codebook: int = KVQ_CODEBOOK_GAUSS,
                 rot_Q=None, nsn_options: int = 0, gsrq_tables=None):
        self.n_kv_heads, self.bits, self.mode, self.device = n_kv_heads, bits, mode, device
        cfg = kvq_config()
        cfg.d, cfg.bits, cfg.mode, cfg.n_kv_heads, cfg.device = D, bits, mode, n_kv_heads, device
        cfg.seed, cfg.codebook = seed, codebook
        keep = []

        def arr(a, dt, cty):
            if a is None:
                return None
            a = np.ascontiguousarray(np.asarray(a), dtype=dt)
            keep.append(a)
            return a.ctypes.data_as(C.POINTER(cty))

        cfg.signs_k = arr(signs_k, np.int8, C.c_int8)
        cfg.signs_v = arr(signs_v, np.int8, C.c_int8)
        cfg.qjl_S = arr(qjl_S, np.float32, C.c_float)
        cfg.vq_codebook = arr(vq_codebook, np.float32, C.c_float)
        cfg.rotation = KVQ_ROTATION_DENSE if rot_Q is not None else KVQ_ROTATION_HADAMARD
        cfg.rot_Q = arr(rot_Q, np.float32, C.c_float)
        cfg.nsn_options = nsn_options
        if gsrq_tables is not None:  # dict S1 [256,32], G1 [16], S2, G2 -> the flat host layout
            gsrq_tables = np.concatenate([np.asarray(gsrq_tables[k], np.float32).ravel()
                                          for k in ("S1", "G1", "S2", "G2")])
        cfg.gsrq_tables = arr(gsrq_tables, np.float32, C.c_float)
        h = C.c_void_p()
        _check(lib().kvq_create(C.byref(cfg), C.byref(h)), "kvq_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            lib().kvq_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def dev(self):
        return torch.device("cuda", self.device)

    def tables(self):
        L = 1 << self.bits
        c = np.zeros(L, np.float32)
        t = np.zeros(L - 1, np.float32)
        _check(lib().kvq_get_tables(self.handle, c.ctypes.data_as(C.c_void_p), t.ctypes.data_as(C.c_void_p),
                                    None, None), "kvq_get_tables")
        return c, t

    def signs(self):
        """The int8 +-1 diagonals (signs_k, signs_v) [H_kv, 128] the context uses."""
        sk = np.zeros((self.n_kv_heads, D), np.int8)
        sv = np.zeros((self.n_kv_heads, D), np.int8)
        _check(lib().kvq_get_tables(self.handle, None, None, sk.ctypes.data_as(C.c_void_p),
                                    sv.ctypes.data_as(C.c_void_p)), "kvq_get_tables")
        return sk, sv

    def code_bytes(self) -> int:
        return int(lib().kvq_code_bytes_per_vec(self.handle))

    # ------------------------------------------------------------------ quantize
    def quantize(self, kind: int, x, out=None):
        """x [B,H_kv,T,128] fp16 -> dict(codes, norms[, qjl_signs, qjl_gamma])."""
        _dev_tensor(x, torch.float16, "x")
        B, H, T, d = x.shape
        if d != D:
            raise ValueError("last dimension must be 128")
        qjl = self.mode == KVQ_MODE_MSE_QJL and kind == KVQ_KIND_K
        if out is None:
            out = dict(codes=torch.empty((B, H, T, self.code_bytes()), dtype=torch.uint8, device=x.device),
                       norms=torch.empty((B, H, T), dtype=torch.float32, device=x.device))
            if qjl:
                out["qjl_signs"] = torch.empty((B, H, T, 16), dtype=torch.uint8, device=x.device)
                out["qjl_gamma"] = torch.empty((B, H, T), dtype=torch.float32, device=x.device)
        kvq_quantize(self, kind, x, B, H, T, out["codes"], out["norms"], out.get("qjl_signs"),
                     out.get("qjl_gamma"))
        return out

    def quantize_kv(self, k, v):
        """K and V [B,H_kv,T,128] fp16 in one launch -> (K outputs, V outputs)."""
        _dev_tensor(k, torch.float16, "k")
        B, H, T, _ = k.shape
        mk = lambda: dict(codes=torch.empty((B, H, T, self.code_bytes()), dtype=torch.uint8, device=k.device),  # noqa: E731
                          norms=torch.empty((B, H, T), dtype=torch.float32, device=k.device))
        ko, vo = mk(), mk()
        kvq_quantize_kv(self, k, v, B, H, T, ko["codes"], ko["norms"], vo["codes"], vo["norms"])
        return ko, vo

    def logits(self, q, codes, norms, qjl_signs=None, qjl_gamma=None, out=None):
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = codes.shape[2]
        if out is None:
            out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
        kvq_logits(self, q, B, Hq, T, codes, norms, qjl_signs, qjl_gamma, out)
        return out

    def decode_ws(self, B, Hq, T):
        n = int(lib().kvq_attn_decode_ws_bytes(self.handle, B, Hq, T))
        return torch.zeros(n, dtype=torch.uint8, device=self.dev)

    def attn_decode(self, q, k_codes, k_norms, v_codes, v_norms, sm_scale: float = 0.0, ws=None, out=None,
                    n_split: int = 0):
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = k_codes.shape[2]
        if ws is None:
            ws = self.decode_ws(B, Hq, T)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        kvq_attn_decode_splits(self, q, B, Hq, T, k_codes, k_norms, v_codes, v_norms, sm_scale, out, ws,
                               n_split)
        return out

    def attn_decode_noalloc(self, q, k_codes, k_norms, v_codes, v_norms, sm_scale: float = 0.0, out=None):
        """As attn_decode, on the library's fixed per-device scratch (no workspace)."""
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = k_codes.shape[2]
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        kvq_attn_decode_noalloc(self, q, B, Hq, T, k_codes, k_norms, v_codes, v_norms, sm_scale, out)
        return out

    def nsn_vq_quantize(self, x, out=None, ws=None):
        _dev_tensor(x, torch.float16, "x")
        H, T, _ = x.shape
        if ws is None:
            ws = torch.empty(int(lib().kvq_nsn_vq_ws_bytes(self.handle, H, T)), dtype=torch.uint8,
                             device=x.device)
        if out is None:
            out = dict(codes=torch.empty((H, T, 16), dtype=torch.uint8, device=x.device),
                       s1=torch.empty((H, T), dtype=torch.float32, device=x.device),
                       s2=torch.empty((H, T), dtype=torch.float32, device=x.device),
                       o=torch.empty((H, D), dtype=torch.float32, device=x.device))
        kvq_nsn_vq_quantize(self, x, H, T, out["codes"], out["s1"], out["s2"], out["o"], ws)
        return out

    def stream_ws(self, B, Hq, T_cap):
        n = int(lib().kvq_attn_decode_stream_ws_bytes(self.handle, B, Hq, T_cap))
        return torch.zeros(n, dtype=torch.uint8, device=self.dev)

    def attn_decode_stream(self, q, k_codes, k_norms, v_codes, v_norms, T, k_tail, v_tail, R, sm_scale: float = 0.0,
                           ws=None, out=None):
        """Decode over the first T tokens of packed arrays [B,Hkv,T_cap,...] followed by
        the first R tokens of fp16 windows [B,Hkv,R_cap,128]."""
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T_cap, R_cap = k_codes.shape[2], k_tail.shape[2]
        if ws is None:
            ws = self.stream_ws(B, Hq, T_cap)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        kvq_attn_decode_stream(self, q, B, Hq, T, T_cap, k_codes, k_norms, v_codes, v_norms, R, R_cap, k_tail,
                               v_tail, sm_scale, out, ws)
        return out

    def flush(self, k_tail, v_tail, R, k_codes, k_norms, v_codes, v_norms, T0):
        """Quantise the first R window tokens into positions T0.. of the packed arrays."""
        B, Hkv, R_cap, _ = k_tail.shape
        kvq_flush(self, k_tail, v_tail, B, Hkv, R, R_cap, k_codes, k_norms, v_codes, v_norms, T0, k_codes.shape[2])

    def nsn_logits(self, q, codes, s1, s2, o, out=None):
        """q [B,Hq,128] fp16; codes [B,Hkv,T,16] u8; s1, s2 [B,Hkv,T]; o [B,Hkv,128] -> [B,Hq,T]."""
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = codes.shape[2]
        if out is None:
            out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
        kvq_nsn_logits(self, q, B, Hq, T, codes, s1, s2, o, out)
        return out

    def nsn_decode_ws(self, B, Hq, T):
        n = int(lib().kvq_nsn_attn_decode_ws_bytes(self.handle, B, Hq, T))
        return torch.empty(n, dtype=torch.uint8, device=self.dev)

    def nsn_attn_decode(self, q, k, v, sm_scale: float = 0.0, ws=None, out=None, n_split: int = 0):
        """k, v: dicts of codes, s1, s2, o as nsn_logits takes them -> out [B,Hq,128] fp32."""
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = k["codes"].shape[2]
        if ws is None:
            ws = self.nsn_decode_ws(B, Hq, T)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        kvq_nsn_attn_decode_splits(self, q, B, Hq, T, k["codes"], k["s1"], k["s2"], k["o"], v["codes"], v["s1"],
                                   v["s2"], v["o"], sm_scale, out, ws, n_split)
        return out

    def nsn_vq_quantize_dq(self, x, out=None, ws=None):
        """NSN-VQ with 4-bit s1 and means: x [H,T,128] fp16 -> dict(codes [H,T,16],
        s1q [H,ceil(T/2)] u8, s1p [H,ceil(T/32),2], s2 [H,T], oq [H,64] u8, op [H,2])."""
        _dev_tensor(x, torch.float16, "x")
        H, T, _ = x.shape
        dev = x.device
        if ws is None:
            ws = torch.empty(int(lib().kvq_nsn_vq_dq_ws_bytes(self.handle, H, T)), dtype=torch.uint8, device=dev)
        if out is None:
            out = dict(codes=torch.empty((H, T, 16), dtype=torch.uint8, device=dev),
                       s1q=torch.empty((H, (T + 1) // 2), dtype=torch.uint8, device=dev),
                       s1p=torch.empty((H, (T + 31) // 32, 2), dtype=torch.float32, device=dev),
                       s2=torch.empty((H, T), dtype=torch.float32, device=dev),
                       oq=torch.empty((H, D // 2), dtype=torch.uint8, device=dev),
                       op=torch.empty((H, 2), dtype=torch.float32, device=dev))
        kvq_nsn_vq_quantize_dq(self, x, H, T, out, ws)
        return out

    def nsn_logits_dq(self, q, e, out=None):
        """q [B,Hq,128] fp16; e: dict as nsn_vq_quantize_dq returns it with heads
        [B,Hkv] leading (codes [B,Hkv,T,16], s1q [B,Hkv,ceil(T/2)], ...) -> [B,Hq,T]."""
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = e["codes"].shape[2]
        if out is None:
            out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
        kvq_nsn_logits_dq(self, q, B, Hq, T, e, out)
        return out

    def nsn_attn_decode_dq(self, q, k, v, sm_scale: float = 0.0, ws=None, out=None, n_split: int = 0):
        """Decode over double-quantised keys and values (dicts as nsn_logits_dq takes)."""
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = k["codes"].shape[2]
        if ws is None:
            ws = self.nsn_decode_ws(B, Hq, T)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        kvq_nsn_attn_decode_dq(self, q, B, Hq, T, k, v, sm_scale, out, ws, n_split)
        return out

    def gsrq_quantize(self, x, out=None, ws=None):
        """GSRQ on the NSN front end: x [H,T,128] fp16 -> dict(codes [H,T,12] u8, s1, s2 [H,T],
        o [H,128])."""
        _dev_tensor(x, torch.float16, "x")
        H, T, _ = x.shape
        if ws is None:
            ws = torch.empty(int(lib().kvq_gsrq_ws_bytes(self.handle, H, T)), dtype=torch.uint8, device=x.device)
        if out is None:
            out = dict(codes=torch.empty((H, T, 12), dtype=torch.uint8, device=x.device),
                       s1=torch.empty((H, T), dtype=torch.float32, device=x.device),
                       s2=torch.empty((H, T), dtype=torch.float32, device=x.device),
                       o=torch.empty((H, D), dtype=torch.float32, device=x.device))
        kvq_gsrq_quantize(self, x, H, T, out["codes"], out["s1"], out["s2"], out["o"], ws)
        return out

    def gsrq_logits(self, q, codes, s1, s2, o, out=None):
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = codes.shape[2]
        if out is None:
            out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
        kvq_gsrq_logits(self, q, B, Hq, T, codes, s1, s2, o, out)
        return out

    def gsrq_attn_decode(self, q, k, v, sm_scale: float = 0.0, ws=None, out=None, n_split: int = 0):
        """k, v: dicts of codes [B,Hkv,T,12], s1, s2 [B,Hkv,T], o [B,Hkv,128] -> out [B,Hq,128]."""
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T = k["codes"].shape[2]
        if ws is None:
            ws = self.nsn_decode_ws(B, Hq, T)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        kvq_gsrq_attn_decode(self, q, B, Hq, T, k["codes"], k["s1"], k["s2"], k["o"], v["codes"], v["s1"], v["s2"],
                             v["o"], sm_scale, out, ws, n_split)
        return out

    def nsn_stream_alloc(self, B, T_cap, Gs):
        """Packed arrays of a streaming NSN-VQ cache: codes [B,Hkv,T_cap,16], s1/s2
        [B,Hkv,T_cap], means o [B,Hkv,T_cap/Gs,128], for K and V."""
        dev, H = self.dev, self.n_kv_heads

        def one():
            return dict(codes=torch.zeros((B, H, T_cap, 16), dtype=torch.uint8, device=dev),
                        s1=torch.zeros((B, H, T_cap), dtype=torch.float32, device=dev),
                        s2=torch.zeros((B, H, T_cap), dtype=torch.float32, device=dev),
                        o=torch.zeros((B, H, T_cap // Gs, D), dtype=torch.float32, device=dev))
        return one(), one()

    def nsn_flush(self, k_tail, v_tail, Gs, k, v, T0, ws=None):
        """Encode the first Gs tokens of the fp16 windows [B,Hkv,R_cap,128] as flush
        group T0 / Gs of the packed dicts k, v (layout of nsn_stream_alloc)."""
        B, Hkv, R_cap, _ = k_tail.shape
        if ws is None:
            ws = torch.empty(int(lib().kvq_nsn_flush_ws_bytes(self.handle, B, Gs)), dtype=torch.uint8,
                             device=k_tail.device)
        kvq_nsn_flush(self, k_tail, v_tail, B, Hkv, Gs, R_cap, k["codes"], k["s1"], k["s2"], k["o"], v["codes"],
                      v["s1"], v["s2"], v["o"], T0, k["codes"].shape[2], ws)

    def nsn_stream_ws(self, B, Hq, T_cap):
        n = int(lib().kvq_nsn_attn_decode_stream_ws_bytes(self.handle, B, Hq, T_cap))
        return torch.empty(n, dtype=torch.uint8, device=self.dev)

    def nsn_attn_decode_stream(self, q, k, v, T, Gs, k_tail, v_tail, R, sm_scale: float = 0.0, ws=None, out=None,
                               n_split: int = 0):
        """Decode over the first T packed tokens (dicts of nsn_stream_alloc) followed by the
        first R tokens of the fp16 windows [B,Hkv,R_cap,128] -> out [B,Hq,128] fp32."""
        _dev_tensor(q, torch.float16, "q")
        B, Hq, _ = q.shape
        T_cap, R_cap = k["codes"].shape[2], k_tail.shape[2]
        if ws is None:
            ws = self.nsn_stream_ws(B, Hq, T_cap)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        kvq_nsn_attn_decode_stream(self, q, B, Hq, T, T_cap, Gs, k["codes"], k["s1"], k["s2"], k["o"], v["codes"],
                                   v["s1"], v["s2"], v["o"], R, R_cap, k_tail, v_tail, sm_scale, out, ws, n_split)
        return out


# ---------------------------------------------------------------------- C-ABI mirrors
def kvq_quantize(ctx: Context, kind, x, B, H_kv, T, codes, norms, qjl_signs=None, qjl_gamma=None):
    _dev_tensor(codes, torch.uint8, "codes")
    _dev_tensor(norms, torch.float32, "norms")
    _check(lib().kvq_quantize(ctx.handle, kind, _ptr(x), B, H_kv, T, _ptr(codes), _ptr(norms),
                              _ptr(qjl_signs), _ptr(qjl_gamma), _stream(x.device)), "kvq_quantize")


def kvq_quantize_kv(ctx: Context, k, v, B, H_kv, T, k_codes, k_norms, v_codes, v_norms):
    for t, dt, n in ((k, torch.float16, "k"), (v, torch.float16, "v"), (k_codes, torch.uint8, "k_codes"),
                     (v_codes, torch.uint8, "v_codes"), (k_norms, torch.float32, "k_norms"),
                     (v_norms, torch.float32, "v_norms")):
        _dev_tensor(t, dt, n)
    _check(lib().kvq_quantize_kv(ctx.handle, _ptr(k), _ptr(v), B, H_kv, T, _ptr(k_codes), _ptr(k_norms),
                                 _ptr(v_codes), _ptr(v_norms), _stream(k.device)), "kvq_quantize_kv")


def kvq_logits(ctx: Context, q, B, H_q, T, codes, norms, qjl_signs, qjl_gamma, logits):
    _dev_tensor(logits, torch.float32, "logits")
    _check(lib().kvq_logits(ctx.handle, _ptr(q), B, H_q, T, _ptr(codes), _ptr(norms), _ptr(qjl_signs),
                            _ptr(qjl_gamma), _ptr(logits), _stream(q.device)), "kvq_logits")


def kvq_attn_decode(ctx: Context, q, B, H_q, T, k_codes, k_norms, v_codes, v_norms, sm_scale, out, ws):
    kvq_attn_decode_splits(ctx, q, B, H_q, T, k_codes, k_norms, v_codes, v_norms, sm_scale, out, ws, 0)


def kvq_attn_decode_splits(ctx: Context, q, B, H_q, T, k_codes, k_norms, v_codes, v_norms, sm_scale, out,
                           ws, n_split):
    _dev_tensor(out, torch.float32, "out")
    _check(lib().kvq_attn_decode_splits(ctx.handle, _ptr(q), B, H_q, T, _ptr(k_codes), _ptr(k_norms),
                                        _ptr(v_codes), _ptr(v_norms), float(sm_scale), _ptr(out), _ptr(ws),
                                        ws.numel() * ws.element_size(), int(n_split), _stream(q.device)),
           "kvq_attn_decode")


def kvq_attn_decode_noalloc(ctx: Context, q, B, H_q, T, k_codes, k_norms, v_codes, v_norms, sm_scale, out):
    _dev_tensor(out, torch.float32, "out")
    _check(lib().kvq_attn_decode_noalloc(ctx.handle, _ptr(q), B, H_q, T, _ptr(k_codes), _ptr(k_norms),
                                         _ptr(v_codes), _ptr(v_norms), float(sm_scale), _ptr(out),
                                         _stream(q.device)), "kvq_attn_decode_noalloc")


def kvq_nsn_vq_quantize(ctx: Context, x, H, T, codes, s1, s2, o, ws):
    _check(lib().kvq_nsn_vq_quantize(ctx.handle, _ptr(x), H, T, _ptr(codes), _ptr(s1), _ptr(s2), _ptr(o),
                                     _ptr(ws), ws.numel() * ws.element_size(), _stream(x.device)),
           "kvq_nsn_vq_quantize")


def _nsn_inputs(codes, s1, s2, o, tag):
    _dev_tensor(codes, torch.uint8, tag + "codes")
    for t, n in ((s1, "s1"), (s2, "s2"), (o, "o")):
        _dev_tensor(t, torch.float32, tag + n)


def kvq_nsn_logits(ctx: Context, q, B, H_q, T, codes, s1, s2, o, logits):
    _nsn_inputs(codes, s1, s2, o, "")
    _dev_tensor(logits, torch.float32, "logits")
    _check(lib().kvq_nsn_logits(ctx.handle, _ptr(q), B, H_q, T, _ptr(codes), _ptr(s1), _ptr(s2), _ptr(o),
                                _ptr(logits), _stream(q.device)), "kvq_nsn_logits")


def kvq_nsn_attn_decode_splits(ctx: Context, q, B, H_q, T, kc, ks1, ks2, ko, vc, vs1, vs2, vo, sm_scale, out, ws,
                               n_split):
    _nsn_inputs(kc, ks1, ks2, ko, "k_")
    _nsn_inputs(vc, vs1, vs2, vo, "v_")
    _dev_tensor(out, torch.float32, "out")
    _check(lib().kvq_nsn_attn_decode_splits(ctx.handle, _ptr(q), B, H_q, T, _ptr(kc), _ptr(ks1), _ptr(ks2),
                                            _ptr(ko), _ptr(vc), _ptr(vs1), _ptr(vs2), _ptr(vo), float(sm_scale),
                                            _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), int(n_split),
                                            _stream(q.device)), "kvq_nsn_attn_decode")


def kvq_attn_decode_stream(ctx: Context, q, B, H_q, T, T_cap, k_codes, k_norms, v_codes, v_norms, R, R_cap, k_tail,
                           v_tail, sm_scale, out, ws):
    for t, dt, n in ((k_codes, torch.uint8, "k_codes"), (v_codes, torch.uint8, "v_codes"),
                     (k_norms, torch.float32, "k_norms"), (v_norms, torch.float32, "v_norms"),
                     (k_tail, torch.float16, "k_tail"), (v_tail, torch.float16, "v_tail"), (out, torch.float32, "out")):
        _dev_tensor(t, dt, n)
    _check(lib().kvq_attn_decode_stream(ctx.handle, _ptr(q), B, H_q, T, T_cap, _ptr(k_codes), _ptr(k_norms),
                                        _ptr(v_codes), _ptr(v_norms), R, R_cap, _ptr(k_tail), _ptr(v_tail),
                                        float(sm_scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(q.device)), "kvq_attn_decode_stream")


def kvq_flush(ctx: Context, k_tail, v_tail, B, H_kv, R, R_cap, k_codes, k_norms, v_codes, v_norms, T0, T_cap):
    for t, dt, n in ((k_codes, torch.uint8, "k_codes"), (v_codes, torch.uint8, "v_codes"),
                     (k_norms, torch.float32, "k_norms"), (v_norms, torch.float32, "v_norms"),
                     (k_tail, torch.float16, "k_tail"), (v_tail, torch.float16, "v_tail")):
        _dev_tensor(t, dt, n)
    _check(lib().kvq_flush(ctx.handle, _ptr(k_tail), _ptr(v_tail), B, H_kv, R, R_cap, _ptr(k_codes), _ptr(k_norms),
                           _ptr(v_codes), _ptr(v_norms), T0, T_cap, _stream(k_tail.device)), "kvq_flush")


def kvq_nsn_flush(ctx: Context, k_tail, v_tail, B, H_kv, Gs, R_cap, kc, ks1, ks2, ko, vc, vs1, vs2, vo, T0, T_cap,
                  ws):
    _nsn_inputs(kc, ks1, ks2, ko, "k_")
    _nsn_inputs(vc, vs1, vs2, vo, "v_")
    _dev_tensor(k_tail, torch.float16, "k_tail")
    _dev_tensor(v_tail, torch.float16, "v_tail")
    _check(lib().kvq_nsn_flush(ctx.handle, _ptr(k_tail), _ptr(v_tail), B, H_kv, Gs, R_cap, _ptr(kc), _ptr(ks1),
                               _ptr(ks2), _ptr(ko), _ptr(vc), _ptr(vs1), _ptr(vs2), _ptr(vo), T0, T_cap, _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(k_tail.device)), "kvq_nsn_flush")


def kvq_nsn_attn_decode_stream(ctx: Context, q, B, H_q, T, T_cap, Gs, kc, ks1, ks2, ko, vc, vs1, vs2, vo, R, R_cap,
                               k_tail, v_tail, sm_scale, out, ws, n_split=0):
    _nsn_inputs(kc, ks1, ks2, ko, "k_")
    _nsn_inputs(vc, vs1, vs2, vo, "v_")
    _dev_tensor(k_tail, torch.float16, "k_tail")
    _dev_tensor(v_tail, torch.float16, "v_tail")
    _dev_tensor(out, torch.float32, "out")
    _check(lib().kvq_nsn_attn_decode_stream(ctx.handle, _ptr(q), B, H_q, T, T_cap, Gs, _ptr(kc), _ptr(ks1),
                                            _ptr(ks2), _ptr(ko), _ptr(vc), _ptr(vs1), _ptr(vs2), _ptr(vo), R, R_cap,
                                            _ptr(k_tail), _ptr(v_tail), float(sm_scale), _ptr(out), _ptr(ws),
                                            ws.numel() * ws.element_size(), int(n_split), _stream(q.device)),
           "kvq_nsn_attn_decode_stream")


_DQ_KEYS = (("codes", torch.uint8), ("s1q", torch.uint8), ("s1p", torch.float32), ("s2", torch.float32),
            ("oq", torch.uint8), ("op", torch.float32))


def _dq_args(e, tag):
    for n, dt in _DQ_KEYS:
        _dev_tensor(e[n], dt, tag + n)
    return [_ptr(e[n]) for n, _ in _DQ_KEYS]


def kvq_nsn_vq_quantize_dq(ctx: Context, x, H, T, out, ws):
    c, s1q, s1p, s2, oq, op = _dq_args(out, "")
    _check(lib().kvq_nsn_vq_quantize_dq(ctx.handle, _ptr(x), H, T, c, s1q, s1p, s2, oq, op, _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(x.device)), "kvq_nsn_vq_quantize_dq")


def kvq_nsn_logits_dq(ctx: Context, q, B, H_q, T, e, logits):
    _dev_tensor(logits, torch.float32, "logits")
    _check(lib().kvq_nsn_logits_dq(ctx.handle, _ptr(q), B, H_q, T, *_dq_args(e, ""), _ptr(logits),
                                   _stream(q.device)), "kvq_nsn_logits_dq")


def kvq_nsn_attn_decode_dq(ctx: Context, q, B, H_q, T, k, v, sm_scale, out, ws, n_split=0):
    _dev_tensor(out, torch.float32, "out")
    _check(lib().kvq_nsn_attn_decode_dq(ctx.handle, _ptr(q), B, H_q, T, *_dq_args(k, "k_"), *_dq_args(v, "v_"),
                                        float(sm_scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                        int(n_split), _stream(q.device)), "kvq_nsn_attn_decode_dq")


def kvq_gsrq_quantize(ctx: Context, x, H, T, codes, s1, s2, o, ws):
    _dev_tensor(x, torch.float16, "x")
    _nsn_inputs(codes, s1, s2, o, "")
    _check(lib().kvq_gsrq_quantize(ctx.handle, _ptr(x), H, T, _ptr(codes), _ptr(s1), _ptr(s2), _ptr(o), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(x.device)), "kvq_gsrq_quantize")


def kvq_gsrq_logits(ctx: Context, q, B, H_q, T, codes, s1, s2, o, logits):
    _nsn_inputs(codes, s1, s2, o, "")
    _dev_tensor(logits, torch.float32, "logits")
    _check(lib().kvq_gsrq_logits(ctx.handle, _ptr(q), B, H_q, T, _ptr(codes), _ptr(s1), _ptr(s2), _ptr(o),
                                 _ptr(logits), _stream(q.device)), "kvq_gsrq_logits")


def kvq_gsrq_attn_decode(ctx: Context, q, B, H_q, T, kc, ks1, ks2, ko, vc, vs1, vs2, vo, sm_scale, out, ws, n_split=0):
    _nsn_inputs(kc, ks1, ks2, ko, "k_")
    _nsn_inputs(vc, vs1, vs2, vo, "v_")
    _dev_tensor(out, torch.float32, "out")
    _check(lib().kvq_gsrq_attn_decode(ctx.handle, _ptr(q), B, H_q, T, _ptr(kc), _ptr(ks1), _ptr(ks2), _ptr(ko),
                                      _ptr(vc), _ptr(vs1), _ptr(vs2), _ptr(vo), float(sm_scale), _ptr(out), _ptr(ws),
                                      ws.numel() * ws.element_size(), int(n_split), _stream(q.device)),
           "kvq_gsrq_attn_decode")
