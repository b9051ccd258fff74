"""Seeded synthetic inputs for the CSA / HCA hot path (inputs only).

The C core (``gen.c``) draws counter-based normals and encodes them into the
storage formats a caller hands to the library.  This module holds no step of
the method: both the fp64 oracle and the HIP path consume what it returns.

Workload builders mirror the shapes of the pages' setting (DeepSeek-V4 at
context lengths up to one million tokens; m=4, k=1024, window 128, m'=128):
see ``configs.py``.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libcsagen.so")
_lib = None


def build():
    """Compile gen.c with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", _SO, os.path.join(_HERE, "gen.c"), "-lm"]
    subprocess.check_call(cmd)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    u64, i64, i32, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    vp = ctypes.c_void_p
    lib.gen_u64.restype = u64
    lib.gen_u64.argtypes = [u64, u64, u64]
    lib.gen_uniform.restype = f64
    lib.gen_uniform.argtypes = [u64, u64, u64]
    lib.gen_normal.restype = f64
    lib.gen_normal.argtypes = [u64, u64, u64]
    lib.gen_fill_normal_f32.argtypes = [u64, u64, i64, f64, f64, vp]
    lib.gen_fill_normal_bf16.argtypes = [u64, u64, i64, f64, vp]
    lib.gen_fill_pow2_weights.argtypes = [u64, u64, i64, vp]
    lib.gen_fill_mxfp4.argtypes = [u64, u64, i64, i64, i32, f64, f64, vp, vp, vp]
    lib.gen_fill_entries.argtypes = [u64, u64, i64, i64, i32, vp, vp, vp]
    lib.gen_fill_random_idx.argtypes = [u64, u64, i64, vp, i32, vp, vp]
    _lib = lib
    return lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


def normal_f32(seed, stream, shape, mean=0.0, sigma=1.0):
    out = np.empty(shape, dtype=np.float32)
    _load().gen_fill_normal_f32(seed, stream, out.size, mean, sigma, _p(out))
    return out


def normal_bf16(seed, stream, shape, sigma=1.0):
    """N(0, sigma^2) draws as bf16 bit patterns (uint16)."""
    out = np.empty(shape, dtype=np.uint16)
    _load().gen_fill_normal_bf16(seed, stream, out.size, sigma, _p(out))
    return out


def pow2_weights(seed, stream, shape):
    out = np.empty(shape, dtype=np.float32)
    _load().gen_fill_pow2_weights(seed, stream, out.size, _p(out))
    return out


def mxfp4(seed, stream, rows, dim, plant_frac=0.0, plant_sigma=3.0, row0=0):
    """rows x dim MXFP4: (data uint8 [rows, dim/2], scale uint8 [rows, dim/32], planted uint8 [rows])."""
    assert dim % 32 == 0
    data = np.empty((rows, dim // 2), dtype=np.uint8)
    scale = np.empty((rows, dim // 32), dtype=np.uint8)
    planted = np.zeros(rows, dtype=np.uint8)
    _load().gen_fill_mxfp4(seed, stream, row0, rows, dim, plant_frac, plant_sigma, _p(data), _p(scale), _p(planted))
    return data, scale, planted


def entries(seed, stream, rows, d_nope, row0=0):
    """rows cache entries: (nope uint8 [rows, d_nope], rope uint16 [rows, 64], scale float32 [rows])."""
    nope = np.empty((rows, d_nope), dtype=np.uint8)
    rope = np.empty((rows, 64), dtype=np.uint16)
    scale = np.empty(rows, dtype=np.float32)
    _load().gen_fill_entries(seed, stream, row0, rows, d_nope, _p(nope), _p(rope), _p(scale))
    return nope, rope, scale


def random_idx(seed, stream, n_per_row, k):
    """Distinct ascending indices below n_per_row[t] for each row, -1 padded."""
    n = np.ascontiguousarray(n_per_row, dtype=np.int64)
    T = n.size
    idx = np.empty((T, k), dtype=np.int32)
    scratch = np.empty(max(int(n.max()) if T else 1, 1), dtype=np.int32)
    _load().gen_fill_random_idx(seed, stream, T, _p(n), k, _p(idx), _p(scratch))
    return idx


def uniform(seed, stream, i):
    return _load().gen_uniform(seed, stream, i)
