"""fp64 CPU oracle for MLA speculative-verify decode -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and the oracle never imports the product.

The arithmetic lives in ``mla_oracle.c`` (plain C, fp64, OpenMP over rows);
this module only compiles it with gcc and marshals numpy arrays.  See the C
file's header for the definition it follows and the pages it cites.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DQK = 576
DV = 512
MODE_DIRECT, MODE_FOLDED, MODE_SPLIT = 0, 1, 2
# 1/sqrt(576) rounded to fp32: the scale the device path receives as a float.
SM_SCALE_F32 = float(np.float32(1.0 / 24.0))


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        i32p = ctypes.POINTER(ctypes.c_int32)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_fold_factor.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.oracle_fold_factor.restype = ctypes.c_int
        lib.oracle_split_layout.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_long), i32p]
        lib.oracle_split_layout.restype = None
        lib.oracle_mla_decode.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i32p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_int, i32p, ctypes.c_int, dp, dp]
        lib.oracle_mla_decode.restype = ctypes.c_int
        lib.oracle_mla_decode_rows.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i32p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                               ctypes.c_double, ctypes.c_double, ctypes.c_long,
                                               ctypes.POINTER(ctypes.c_long), dp, dp]
        lib.oracle_mla_decode_rows.restype = ctypes.c_int
        lib.oracle_mla_partial.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i32p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                                           ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_long, ctypes.c_long, dp, dp]
        lib.oracle_mla_partial.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        _lib = lib
        return lib


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _check_inputs(q_bits, kv, kv_is_fp8, q_len, kv_len, H):
    q_bits = np.ascontiguousarray(q_bits)
    kv = np.ascontiguousarray(kv)
    if q_bits.dtype != np.uint16:
        raise TypeError("q_bits must be uint16 bf16 bit patterns")
    want = np.uint8 if kv_is_fp8 else np.uint16
    if kv.dtype != want:
        raise TypeError(f"kv must be {want} for kv_is_fp8={kv_is_fp8}")
    sq, sn = int(np.sum(q_len)), int(np.sum(kv_len))
    if q_bits.size != sq * H * DQK:
        raise ValueError("q_bits has the wrong size")
    if kv.size != sn * DQK:
        raise ValueError("kv has the wrong size")
    return q_bits, kv


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(int(bits))


def e4m3_to_double(code: int) -> float:
    return _load().oracle_e4m3_to_double(int(code))


def fold_factor(H: int, q: int) -> int:
    return _load().oracle_fold_factor(int(H), int(q))


def split_layout(n: int, S: int, granule: int):
    """Returns (L, S_eff) for n keys cut into S requested chunks of whole granules."""
    L = ctypes.c_long(0)
    s = ctypes.c_int32(0)
    _load().oracle_split_layout(int(n), int(S), int(granule), ctypes.byref(L), ctypes.byref(s))
    return int(L.value), int(s.value)


def mla_decode(q_bits, kv, q_len, kv_len, H, *, kv_is_fp8=False, kv_scale=1.0,
               sm_scale=SM_SCALE_F32, mode=MODE_DIRECT, splits=None, granule=64):
    """Full decode.  Returns (O [sum q, H, 512] f64, LSE [sum q, H] f64)."""
    lib = _load()
    q_len_a, q_len_p = _i32(q_len)
    kv_len_a, kv_len_p = _i32(kv_len)
    q_bits, kv = _check_inputs(q_bits, kv, kv_is_fp8, q_len_a, kv_len_a, H)
    rows = int(q_len_a.sum()) * H
    o = np.full((rows, DV), np.nan, dtype=np.float64)
    lse = np.full((rows,), np.nan, dtype=np.float64)
    if splits is None:
        splits_p = None
        sp = None
    else:
        sp, splits_p = _i32(splits)
    rc = lib.oracle_mla_decode(len(q_len_a), H, q_len_p, kv_len_p, q_bits.ctypes.data,
                               kv.ctypes.data, int(bool(kv_is_fp8)), float(kv_scale),
                               float(sm_scale), int(mode), splits_p, int(granule),
                               o.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                               lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    del sp
    if rc != 0:
        raise ValueError("oracle_mla_decode rejected its arguments")
    sq = int(q_len_a.sum())
    return o.reshape(sq, H, DV), lse.reshape(sq, H)


def mla_decode_rows(q_bits, kv, q_len, kv_len, H, rows, *, kv_is_fp8=False, kv_scale=1.0,
                    sm_scale=SM_SCALE_F32):
    """Selected output rows (index = token * H + head).  Returns (O [n, 512], LSE [n])."""
    lib = _load()
    q_len_a, q_len_p = _i32(q_len)
    kv_len_a, kv_len_p = _i32(kv_len)
    q_bits, kv = _check_inputs(q_bits, kv, kv_is_fp8, q_len_a, kv_len_a, H)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.full((len(rows), DV), np.nan, dtype=np.float64)
    lse = np.full((len(rows),), np.nan, dtype=np.float64)
    rc = lib.oracle_mla_decode_rows(len(q_len_a), H, q_len_p, kv_len_p, q_bits.ctypes.data,
                                    kv.ctypes.data, int(bool(kv_is_fp8)), float(kv_scale),
                                    float(sm_scale), len(rows),
                                    rows.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                                    o.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                    lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError("oracle_mla_decode_rows rejected its arguments")
    return o, lse


def mla_partial(q_bits, kv, q_len, kv_len, H, b, i, h, lo, hi, *, kv_is_fp8=False, kv_scale=1.0,
                sm_scale=SM_SCALE_F32):
    """Partial (normalised O over keys [lo, hi) visible to token i, head h of sequence b, lse)."""
    lib = _load()
    q_len_a, q_len_p = _i32(q_len)
    kv_len_a, kv_len_p = _i32(kv_len)
    q_bits, kv = _check_inputs(q_bits, kv, kv_is_fp8, q_len_a, kv_len_a, H)
    o = np.full((DV,), np.nan, dtype=np.float64)
    lse = ctypes.c_double(np.nan)
    rc = lib.oracle_mla_partial(len(q_len_a), H, q_len_p, kv_len_p, q_bits.ctypes.data,
                                kv.ctypes.data, int(bool(kv_is_fp8)), float(kv_scale),
                                float(sm_scale), int(b), int(i), int(h), int(lo), int(hi),
                                o.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                ctypes.byref(lse))
    if rc != 0:
        raise ValueError("oracle_mla_partial rejected its arguments")
    return o, float(lse.value)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of the following oracle calls (timing only)."""
    _load().oracle_set_num_threads(int(n))
