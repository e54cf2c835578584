"""CPU oracle for causal grouped-query attention over a cached prefix.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The GPU library never
does, and this package never imports the GPU library.

The arithmetic lives in attn_oracle.c (plain C, double sums, OpenMP over
(row, head)); this wrapper only builds it with gcc and marshals numpy arrays.
It computes the three-step definition from "Inference Attention 1: The Full
Score Matrix" (Lesson) with the causal edge, head mapping and exact 1/8 scale
of "Inference Attention 2: Flash Prefill Against a Cached Prefix" (Lesson).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

HQ, HKV, D = 32, 8, 64


def build(force: bool = True) -> str:
    """Compile attn_oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        f = ctypes.POINTER(ctypes.c_float)
        lib.oracle_attn_prefill.argtypes = [f, f, f, f, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_prefill.restype = ctypes.c_int
        ip = ctypes.POINTER(ctypes.c_int)
        lib.oracle_attn_rows.argtypes = [f, f, f, f, ctypes.c_int, ctypes.c_int, ip, ip,
                                         ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_attn_prefill_paged.argtypes = [f, f, f, ip, ctypes.c_int, ctypes.c_int, f, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int]
        lib.oracle_attn_prefill_paged.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a: np.ndarray, ctype=ctypes.c_float):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(q, k, v, P):
    C = q.shape[0]
    if q.shape != (C, HQ, D) or k.shape != (P + C, HKV, D) or v.shape != k.shape:
        raise ValueError("shapes q %s k %s v %s do not match C=%d P=%d"
                         % (q.shape, k.shape, v.shape, C, P))
    return C


def attn_prefill(q, k, v, P: int, nthreads: int = 0) -> np.ndarray:
    """out[C][32][64] float32 for q[C][32][64], k/v[P+C][8][64].

    Values are read as float32 (bfloat16 inputs must be passed widened to
    float32, which is exact).  nthreads=0 uses the OpenMP default."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    C = _check(q, k, v, P)
    out = np.empty((C, HQ, D), dtype=np.float32)
    if C == 0:
        return out
    rc = _load().oracle_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), C, P, nthreads)
    if rc != 0:
        raise RuntimeError("oracle_attn_prefill failed with code %d" % rc)
    return out


def attn_rows(q, k, v, P: int, rows, heads, nthreads: int = 0) -> np.ndarray:
    """out[i][h][:] for the listed (row, head) pairs only: array [n][64]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    C = _check(q, k, v, P)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    if rows.shape != heads.shape or rows.ndim != 1:
        raise ValueError("rows and heads must be 1-D of equal length")
    out = np.empty((rows.shape[0], D), dtype=np.float32)
    if rows.shape[0] == 0:
        return out
    rc = _load().oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(out), C, P,
                                  _ptr(rows, ctypes.c_int), _ptr(heads, ctypes.c_int),
                                  rows.shape[0], nthreads)
    if rc != 0:
        raise RuntimeError("oracle_attn_rows failed with code %d" % rc)
    return out


def attn_prefill_paged(q, k_pages, v_pages, block_table, P: int, nthreads: int = 0) -> np.ndarray:
    """out[C][32][64] for a paged cache: k_pages/v_pages [numBlocks][pageSize][8][64],
    block_table[ceil((P+C)/pageSize)] of physical page indices."""
    q, kp, vp = _f32(q), _f32(k_pages), _f32(v_pages)
    C = q.shape[0]
    if q.shape != (C, HQ, D) or kp.ndim != 4 or kp.shape[2:] != (HKV, D) or vp.shape != kp.shape:
        raise ValueError("bad shapes q %s pages %s %s" % (q.shape, kp.shape, vp.shape))
    nb, ps = kp.shape[0], kp.shape[1]
    table = np.ascontiguousarray(block_table, dtype=np.int32)
    if table.shape[0] < -(-(P + C) // ps):
        raise ValueError("block table too short")
    out = np.empty((C, HQ, D), dtype=np.float32)
    if C == 0:
        return out
    rc = _load().oracle_attn_prefill_paged(_ptr(q), _ptr(kp), _ptr(vp), _ptr(table, ctypes.c_int), nb, ps,
                                           _ptr(out), C, P, nthreads)
    if rc != 0:
        raise RuntimeError("oracle_attn_prefill_paged failed with code %d" % rc)
    return out


def max_threads() -> int:
    """Threads an OpenMP region of the oracle uses by default."""
    return int(_load().oracle_max_threads())
