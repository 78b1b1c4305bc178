"""Seeded synthetic inputs (keys, values, queries, ragged lengths) for wave-index decode.

Only input drawing lives here; the generator holds none of the method's arithmetic.
Both the CPU oracle and the GPU library are fed from these arrays.  The shapes follow
the long-context Llama-3-8B-like layers of the RetroInfer page (section 1, the KV
cache of 1M tokens; section 4, contexts of 120K and 1M): 8 kv heads of 128 dims,
bf16 storage, clustered keys with per-segment drift, queries near a random key.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def compile_lib():
    """Compile libsynth.so (plain C, OpenMP) in place."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _LIB_PATH, os.path.join(_HERE, "synth.c"), "-lm"]
    subprocess.check_call(cmd)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            compile_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.syn_ctx_lengths.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, P]
        lib.syn_kv.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32,
                               P, P, P]
        lib.syn_queries.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    P, P, P, P]
        lib.syn_normals.argtypes = [ctypes.c_uint64, ctypes.c_int64, P]
        lib.syn_student4s.argtypes = [ctypes.c_uint64, ctypes.c_int64, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def ctx_lengths(seed, batch, lo, hi):
    """N_b ~ U{lo..hi} for b < batch (int64)."""
    out = np.empty(batch, dtype=np.int64)
    _load().syn_ctx_lengths(seed, batch, lo, hi, _ptr(out))
    return out


def kv(seed, batch, n_kv_heads, ctx, drift_seg, heavy=False, values=True, comp=False):
    """Keys/values as uint16 bf16 bit patterns, rows [sum_b G*N_b][128] (sequence-major, then kv head).

    Returns (K, V or None, comp or None); comp[row] is the mixture component the token drew.
    """
    ctx = np.ascontiguousarray(ctx, dtype=np.int64)
    rows = int(n_kv_heads * ctx.sum())
    K = np.empty((rows, 128), dtype=np.uint16)
    V = np.empty((rows, 128), dtype=np.uint16) if values else None
    C = np.empty(rows, dtype=np.int32) if comp else None
    _load().syn_kv(seed, len(ctx), n_kv_heads, _ptr(ctx), drift_seg, 1 if heavy else 0, _ptr(K), _ptr(V), _ptr(C))
    return K, V, C


def queries(seed, steps, batch, n_q_heads, n_kv_heads, ctx, K):
    """q[step][b][h][128] (uint16 bf16 bits) near a uniformly drawn key; also returns t* [step][b][h]."""
    ctx = np.ascontiguousarray(ctx, dtype=np.int64)
    q = np.empty((steps, batch, n_q_heads, 128), dtype=np.uint16)
    ts = np.empty((steps, batch, n_q_heads), dtype=np.int64)
    _load().syn_queries(seed, steps, batch, n_q_heads, n_kv_heads, _ptr(ctx), _ptr(np.ascontiguousarray(K)),
                        _ptr(q), _ptr(ts))
    return q, ts


def normals(seed, n):
    out = np.empty(n, dtype=np.float64)
    _load().syn_normals(seed, n, _ptr(out))
    return out


def student4(seed, n):
    out = np.empty(n, dtype=np.float64)
    _load().syn_student4s(seed, n, _ptr(out))
    return out


def bf16_bits_to_f32(a):
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
