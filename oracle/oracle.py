"""fp64 CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports, links or calls anything under ``oracle/``,
and this module imports nothing from the product package.

The numeric work lives in ``oracle.c`` (plain C, fp64, OpenMP over
(sequence, kv head)); this file builds it with gcc, loads it with ctypes and
passes numpy arrays in and out.  See the header of ``oracle.c`` for the
passages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_quantize_e4m3.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.oracle_quantize_e4m3.restype = ctypes.c_uint8
    lib.oracle_kv_append.argtypes = [P, P, P, i32, i32, i32, i32, i32, ctypes.c_int, P, P, P, P]
    lib.oracle_kv_append.restype = ctypes.c_int
    lib.oracle_paged_attention.argtypes = [P, P, P, P, P, ctypes.c_int, P, P, P, i32, i32, i32, i32, i32, i32,
                                           ctypes.c_double, i32, i32, P, i32]
    lib.oracle_paged_attention.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------- scalars

def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits))


def e4m3_to_f64(code: int) -> float:
    return _load().oracle_e4m3_to_f64(int(code))


def f32_to_e4m3(x: float) -> int:
    return int(_load().oracle_f32_to_e4m3(float(x)))


def quantize_e4m3(x: float, s: float) -> int:
    return int(_load().oracle_quantize_e4m3(float(x), float(s)))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# -------------------------------------------------------- array functions

def kv_cache_shapes(num_pages: int, Hkv: int, d: int, P: int):
    """Shapes of the K and V page pools ([np][Hkv][d/8][P][8] and [np][Hkv][d][P]); K's slots
    within a page follow the oracle's k_slot order, V's tokens are in order."""
    return (num_pages, Hkv, d // 8, P, 8), (num_pages, Hkv, d, P)


def kv_append(k_new: np.ndarray, v_new: np.ndarray, slot_mapping: np.ndarray, k_cache: np.ndarray,
              v_cache: np.ndarray, *, Hkv: int, d: int, P: int, kv_fp8: bool = False,
              k_scale: np.ndarray | None = None, v_scale: np.ndarray | None = None) -> None:
    """Scatter new rows into the page pools in place (bf16 bits as uint16, or fp8 codes as uint8)."""
    T = int(slot_mapping.shape[0])
    k_new = np.ascontiguousarray(k_new.view(np.uint16).reshape(T, Hkv, d))
    v_new = np.ascontiguousarray(v_new.view(np.uint16).reshape(T, Hkv, d))
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    num_pages = int(k_cache.shape[0])
    if kv_fp8:
        assert k_cache.dtype == np.uint8 and v_cache.dtype == np.uint8
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
    else:
        assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16
    rc = _load().oracle_kv_append(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T, Hkv, d, P, num_pages,
                                  int(kv_fp8), _ptr(k_scale), _ptr(v_scale), _ptr(k_cache), _ptr(v_cache))
    if rc != 0:
        raise ValueError("oracle_kv_append failed with code %d" % rc)


def paged_attention(q: np.ndarray, cu_q_lens: np.ndarray, seq_lens: np.ndarray, k_cache: np.ndarray,
                    v_cache: np.ndarray, block_table: np.ndarray, *, Hq: int, Hkv: int, d: int, P: int,
                    scale: float, kv_fp8: bool = False, k_scale: np.ndarray | None = None,
                    v_scale: np.ndarray | None = None, split_tokens: int = 0, window: int = 0,
                    nthreads: int = 0) -> np.ndarray:
    """fp64 attention output [total_q][Hq][d] for packed ragged queries (bf16 bits as uint16).
    window = 0: full causal attention; window = w > 0: position p sees keys p - w < j <= p."""
    q = np.ascontiguousarray(q.view(np.uint16))
    total_q = int(q.shape[0])
    cu_q_lens = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    B = int(seq_lens.shape[0])
    assert cu_q_lens.shape[0] == B + 1 and int(cu_q_lens[-1]) == total_q
    if kv_fp8:
        k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
        v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
    out = np.zeros((total_q, Hq, d), dtype=np.float64)
    rc = _load().oracle_paged_attention(_ptr(q), _ptr(cu_q_lens), _ptr(seq_lens), _ptr(k_cache), _ptr(v_cache),
                                        int(kv_fp8), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                        int(block_table.shape[1]), B, Hq, Hkv, d, P, float(scale),
                                        int(split_tokens), int(window), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_paged_attention failed with code %d" % rc)
    return out
