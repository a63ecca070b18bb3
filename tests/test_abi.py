"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/kvq.h declares, validates arguments on the host and builds the same
fp32 Lloyd-Max tables as the oracle."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
from calibration_free_kv_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = kvq.lib()
    names = declared_symbols()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert sorted(kvq.EXPORTS) == names


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_library_tables_equal_oracle_tables(bits):
    c, t = kvq.kvq_codebook(bits)
    co, to = O.tables_f32(bits)
    assert np.array_equal(c, co) and np.array_equal(t, to)


def test_codebook_rejects_bad_bits():
    buf = np.zeros(32, np.float32)
    for b in (0, 5, -1):
        assert kvq.lib().kvq_codebook(b, buf.ctypes.data_as(C.c_void_p), buf.ctypes.data_as(C.c_void_p)) == kvq.KVQ_E_INVAL


def _cfg(**kw):
    cfg = kvq.kvq_config()
    cfg.d, cfg.bits, cfg.mode, cfg.n_kv_heads, cfg.device = 128, 3, 0, 2, 0
    s = np.ones((2, 128), np.int8)
    cfg.signs_k = s.ctypes.data_as(C.POINTER(C.c_int8))
    cfg.signs_v = s.ctypes.data_as(C.POINTER(C.c_int8))
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg, s


def test_create_validation():
    L = kvq.lib()
    h = C.c_void_p()
    assert L.kvq_create(None, C.byref(h)) == kvq.KVQ_E_INVAL
    for bad in (dict(d=64), dict(bits=0), dict(bits=5), dict(n_kv_heads=0), dict(mode=7)):
        cfg, keep = _cfg(**bad)
        assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_INVAL, bad
        assert not h.value
    cfg, keep = _cfg()
    bad_signs = np.zeros((2, 128), np.int8)  # 0 is not a sign
    cfg.signs_k = bad_signs.ctypes.data_as(C.POINTER(C.c_int8))
    assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_INVAL
    cfg, keep = _cfg(mode=1)  # QJL mode needs S
    assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_INVAL
    cfg, keep = _cfg(mode=2)  # NSN mode needs a codebook
    assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_INVAL
    for bad in (dict(codebook=2), dict(codebook=-1)):  # not a KVQ_CODEBOOK_*
        cfg, keep = _cfg(**bad)
        assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_INVAL, bad
    # dense rotation: the configuration is checked before any device is touched,
    # so a valid one reaches the device check
    eye = np.eye(128, dtype=np.float32)
    qp = lambda a: a.ctypes.data_as(C.POINTER(C.c_float))  # noqa: E731
    cfg, keep = _cfg(rotation=1, rot_Q=qp(eye), device=999)
    assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_DEVICE
    half = 0.5 * eye  # entries in range, not orthogonal
    nan = eye.copy()
    nan[3, 4] = np.nan
    big = eye.copy()
    big[0, 0] = 1.5
    near = eye.copy()
    near[5, 6] = 2e-3  # Q Q^T off by 2e-3 in two entries
    for Q in (half, nan, big, near):
        cfg, keep = _cfg(rotation=1, rot_Q=qp(Q), device=999)
        assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_INVAL
    cfg, keep = _cfg(rotation=1, device=999)  # no Q
    assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_INVAL
    cfg, keep = _cfg(rotation=2, rot_Q=qp(eye), device=999)  # not a KVQ_ROTATION_*
    assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_INVAL
    cb = np.ones((256, 8), np.float32)
    cfg, keep = _cfg(mode=2, vq_codebook=qp(cb), rotation=1, rot_Q=qp(eye), device=999)  # NSN keeps its transform
    assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_UNSUPPORTED
    assert not h.value
    cfg, keep = _cfg(device=999)  # no such device (no device at all on a CPU host)
    assert L.kvq_create(C.byref(cfg), C.byref(h)) == kvq.KVQ_E_DEVICE
    assert not h.value


def test_null_context_calls():
    L = kvq.lib()
    assert L.kvq_destroy(None) == kvq.KVQ_OK
    assert L.kvq_code_bytes_per_vec(None) == 0
    assert L.kvq_get_tables(None, None, None, None, None) == kvq.KVQ_E_INVAL
    assert L.kvq_quantize(None, 0, None, 1, 1, 1, None, None, None, None, None) == kvq.KVQ_E_INVAL
    assert L.kvq_logits(None, None, 1, 1, 1, None, None, None, None, None, None) == kvq.KVQ_E_INVAL
    assert L.kvq_attn_decode(None, None, 1, 1, 1, None, None, None, None, 0.0, None, None, 0, None) == kvq.KVQ_E_INVAL
    assert L.kvq_attn_decode_ws_bytes(None, 1, 1, 1) == 0
    assert L.kvq_nsn_vq_ws_bytes(None, 1, 1) == 0
    assert L.kvq_nsn_vq_quantize(None, None, 1, 1, None, None, None, None, None, 0, None) == kvq.KVQ_E_INVAL
    assert L.kvq_nsn_logits(None, None, 1, 4, 1, None, None, None, None, None, None) == kvq.KVQ_E_INVAL
    assert L.kvq_nsn_attn_decode_ws_bytes(None, 1, 4, 1) == 0
    assert L.kvq_nsn_attn_decode(None, None, 1, 4, 1, None, None, None, None, None, None, None, None, 0.0, None,
                                 None, 0, None) == kvq.KVQ_E_INVAL
    assert L.kvq_attn_decode_stream_ws_bytes(None, 1, 4, 1) == 0
    assert L.kvq_attn_decode_stream(None, None, 1, 4, 1, 1, None, None, None, None, 0, 0, None, None, 0.0, None,
                                    None, 0, None) == kvq.KVQ_E_INVAL
    assert L.kvq_flush(None, None, None, 1, 1, 1, 1, None, None, None, None, 0, 1, None) == kvq.KVQ_E_INVAL
    assert L.kvq_nsn_flush_ws_bytes(None, 1, 128) == 0
    assert L.kvq_nsn_flush(None, None, None, 1, 1, 128, 128, None, None, None, None, None, None, None, None, 0, 128,
                           None, 0, None) == kvq.KVQ_E_INVAL
    assert L.kvq_nsn_attn_decode_stream_ws_bytes(None, 1, 4, 128) == 0
    assert L.kvq_nsn_attn_decode_stream(None, None, 1, 4, 128, 128, 128, None, None, None, None, None, None, None,
                                        None, 0, 0, None, None, 0.0, None, None, 0, 0, None) == kvq.KVQ_E_INVAL
    assert L.kvq_nsn_vq_dq_ws_bytes(None, 1, 1) == 0
    assert L.kvq_nsn_vq_quantize_dq(None, None, 1, 1, None, None, None, None, None, None, None, 0,
                                    None) == kvq.KVQ_E_INVAL
    assert L.kvq_nsn_logits_dq(None, None, 1, 4, 1, None, None, None, None, None, None, None, None) == kvq.KVQ_E_INVAL
    assert L.kvq_nsn_attn_decode_dq(None, None, 1, 4, 1, None, None, None, None, None, None, None, None, None, None,
                                    None, None, 0.0, None, None, 0, 0, None) == kvq.KVQ_E_INVAL
    assert L.kvq_gsrq_ws_bytes(None, 1, 1) == 0
    assert L.kvq_gsrq_quantize(None, None, 1, 1, None, None, None, None, None, 0, None) == kvq.KVQ_E_INVAL
    assert L.kvq_gsrq_logits(None, None, 1, 4, 1, None, None, None, None, None, None) == kvq.KVQ_E_INVAL
    assert L.kvq_gsrq_attn_decode(None, None, 1, 4, 1, None, None, None, None, None, None, None, None, 0.0, None,
                                  None, 0, 0, None) == kvq.KVQ_E_INVAL
    for s in range(6):
        assert kvq.strerror(s)


def test_debug_build_selection():
    """The release library reports no debug build and no check records (it
    touches no device for them); KVQ_DEBUG selects the bounds-checked
    libkvq_debug.so in a fresh process, KVQ_LIB any given build."""
    import subprocess
    import sys
    assert kvq.debug_build() is False and kvq.debug_take() == 0
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    prog = ("import sys; sys.path.insert(0, %r)\n"
            "from calibration_free_kv_amd import kvq\n"
            "print(kvq.LIB_PATH.rsplit('/', 1)[-1], kvq.debug_build())\n") % root
    for env, want in (({"KVQ_DEBUG": "1"}, "libkvq_debug.so True"), ({"KVQ_DEBUG": "0"}, "libkvq.so False"),
                      ({"KVQ_LIB": kvq.LIB_PATH.replace("libkvq.so", "libkvq_debug.so")},
                       "libkvq_debug.so True")):
        e = {k: v for k, v in os.environ.items() if k not in ("KVQ_DEBUG", "KVQ_LIB")}
        e.update(env)
        r = subprocess.run([sys.executable, "-c", prog], env=e, capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.split() == want.split(), (env, r.stdout, r.stderr[-1000:])
