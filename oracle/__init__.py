"""ctypes front end of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, never by the product package.
It shares no code with the HIP path; both sides only receive the same seeded
inputs.

Arrays are numpy arrays on the host.  16-bit floats are passed as their raw
bits (``uint16``) together with an explicit dtype name, because numpy has no
bfloat16; FP8 e4m3 codes are ``uint8``; 4-bit codes ("u4") are packed two
per ``uint8`` (a u4 cache of head dim D has D / 2 bytes per row, and its
scale arrays hold (x_min, range) pairs: [..., 2] float32).  Dtype names:
``"f32"``, ``"f16"``, ``"bf16"``, ``"i8"``, ``"f8"``, ``"u4"``.

What the functions compute, and the pages they follow, is stated in the C
source.  Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (library routines, closed forms, the worked INT8
example of the absmax passage, exact rational arithmetic, invariances).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "f8": 4, "u4": 5}
_NP_OF = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "i8": np.int8, "f8": np.uint8,
          "u4": np.uint8}

GCC_CMD = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", _SRC, "-o", _LIB, "-lm"]


def build() -> str:
    """Compile liboracle.so with gcc (no GPU code involved)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P, I, L64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_float
        L.oracle_paged_decode.argtypes = [P, P, I, P, P, I, P, P, P, I, P, I, I, I, I, I, I, F,
                                          P, L64, I]
        L.oracle_paged_decode_window.argtypes = [P, P, I, P, P, I, P, P, P, I, P, I, I, I, I, I, I,
                                                 F, I, P, L64, I]
        L.oracle_paged_multi.argtypes = [P, P, I, P, P, I, P, P, P, I, P, P, I, I, I, I, I, I, F,
                                         I]
        L.oracle_paged_partials.argtypes = [P, P, P, P, I, P, P, I, P, P, P, I, P, I, I, I, I, I,
                                            I, F, I, I, I]
        L.oracle_merge_partials.argtypes = [P, P, P, P, L64, I, I]
        L.oracle_quantize_rows.argtypes = [P, P, P, I, L64, I]
        L.oracle_quantize_rows_f8.argtypes = [P, P, P, I, L64, I]
        L.oracle_quantize_rows_u4.argtypes = [P, P, P, I, L64, I]
        L.oracle_f8_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_f8_to_f64.restype = ctypes.c_double
        L.oracle_f8_from_f32.argtypes = [ctypes.c_float]
        L.oracle_f8_from_f32.restype = ctypes.c_uint8
        L.oracle_kv_cache_write.argtypes = [P, P, P, P, P, P, P, L64, I, I, I, I, I, I]
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_num_threads.argtypes = [I]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a, dtype, name):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    want = _NP_OF[dtype] if isinstance(dtype, str) else dtype
    if a.dtype != want:
        raise TypeError(f"{name}: expected {np.dtype(want)}, got {a.dtype}")
    return a


def num_threads(n: int = 0) -> int:
    """Set (n > 0) and return the OpenMP thread count the oracle uses."""
    return lib().oracle_num_threads(n)


def f16_to_f64(bits: int) -> float:
    return lib().oracle_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return lib().oracle_bf16_to_f64(bits)


def paged_decode(q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, context_lens, scale,
                 k_scale=None, v_scale=None, block_size=16, rows=None, nthreads=0, window=0):
    """fp64 gather-then-dense attention.  Shapes: q [B][Hq][D]; caches
    [NB][Hkv][block_size][D]; block_tables int32 [B][MBS]; context_lens int32 [B];
    scales float32 [NB][Hkv][block_size] for "i8" and "f8".  Returns float64 [B][Hq][D]
    (rows not requested are NaN).  window > 0: attend to the last `window`
    positions of each sequence only (sliding window)."""
    q = _check(q, q_dtype, "q")
    k_cache = _check(k_cache, cache_dtype, "k_cache")
    v_cache = _check(v_cache, cache_dtype, "v_cache")
    bt = _check(block_tables, np.int32, "block_tables")
    cl = _check(context_lens, np.int32, "context_lens")
    ks = _check(k_scale, np.float32, "k_scale")
    vs = _check(v_scale, np.float32, "v_scale")
    B, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    assert D2 == (D // 2 if cache_dtype == "u4" else D)
    assert bs == block_size and v_cache.shape == k_cache.shape
    if cache_dtype in ("i8", "f8", "u4"):
        assert ks is not None and vs is not None
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    rc = lib().oracle_paged_decode_window(_ptr(out), _ptr(q), DTYPES[q_dtype], _ptr(k_cache),
                                          _ptr(v_cache), DTYPES[cache_dtype], _ptr(ks), _ptr(vs),
                                          _ptr(bt), bt.shape[1], _ptr(cl), B, Hq, Hkv, D,
                                          block_size, NB, float(scale), int(window), _ptr(r),
                                          0 if r is None else len(r), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_paged_decode failed with {rc}")
    return out


def paged_multi(q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, context_lens,
                query_start_loc, scale, k_scale=None, v_scale=None, block_size=16, nthreads=0):
    """Causal attention of several query tokens per sequence (see oracle.c).
    q [T][Hq][D]; query_start_loc int32 [B+1].  Returns float64 [T][Hq][D]."""
    q = _check(q, q_dtype, "q")
    k_cache = _check(k_cache, cache_dtype, "k_cache")
    v_cache = _check(v_cache, cache_dtype, "v_cache")
    bt = _check(block_tables, np.int32, "block_tables")
    cl = _check(context_lens, np.int32, "context_lens")
    qsl = _check(query_start_loc, np.int32, "query_start_loc")
    ks = _check(k_scale, np.float32, "k_scale")
    vs = _check(v_scale, np.float32, "v_scale")
    T, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    B = len(cl)
    assert D2 == D and len(qsl) == B + 1 and qsl[-1] == T
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    rc = lib().oracle_paged_multi(_ptr(out), _ptr(q), DTYPES[q_dtype], _ptr(k_cache),
                                  _ptr(v_cache), DTYPES[cache_dtype], _ptr(ks), _ptr(vs), _ptr(bt),
                                  bt.shape[1], _ptr(cl), _ptr(qsl), B, Hq, Hkv, D, block_size, NB,
                                  float(scale), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_paged_multi failed with {rc}")
    return out


def paged_partials(q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, context_lens, scale,
                   partition_size, num_partitions, k_scale=None, v_scale=None, block_size=16,
                   nthreads=0):
    """Per-partition (m, l, o) in fp64: m [B][Hq][NP], l [B][Hq][NP], o [B][Hq][NP][D]."""
    q = _check(q, q_dtype, "q")
    k_cache = _check(k_cache, cache_dtype, "k_cache")
    v_cache = _check(v_cache, cache_dtype, "v_cache")
    bt = _check(block_tables, np.int32, "block_tables")
    cl = _check(context_lens, np.int32, "context_lens")
    ks = _check(k_scale, np.float32, "k_scale")
    vs = _check(v_scale, np.float32, "v_scale")
    B, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    m = np.empty((B, Hq, num_partitions), np.float64)
    l = np.empty((B, Hq, num_partitions), np.float64)
    o = np.empty((B, Hq, num_partitions, D), np.float64)
    rc = lib().oracle_paged_partials(_ptr(m), _ptr(l), _ptr(o), _ptr(q), DTYPES[q_dtype],
                                     _ptr(k_cache), _ptr(v_cache), DTYPES[cache_dtype], _ptr(ks),
                                     _ptr(vs), _ptr(bt), bt.shape[1], _ptr(cl), B, Hq, Hkv, D,
                                     block_size, NB, float(scale), partition_size,
                                     num_partitions, nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_paged_partials failed with {rc}")
    return m, l, o


def merge_partials(m, l, o):
    """Merge [..][NP] partials into [..][D] (fp64)."""
    m = np.ascontiguousarray(m, np.float64)
    l = np.ascontiguousarray(l, np.float64)
    o = np.ascontiguousarray(o, np.float64)
    NP, D = o.shape[-2], o.shape[-1]
    rows = int(np.prod(o.shape[:-2]))
    out = np.empty(o.shape[:-2] + (D,), np.float64)
    lib().oracle_merge_partials(_ptr(out), _ptr(m), _ptr(l), _ptr(o), rows, NP, D)
    return out


def quantize_rows(x, dtype, target="i8"):
    """Symmetric per-row quantization of the rows of x ([..., D]) to INT8
    (target "i8") or FP8 e4m3 (target "f8").  Returns (codes [..., D] int8 or
    uint8, scales float32 [...])."""
    x = _check(x, dtype, "x")
    D = x.shape[-1]
    rows = int(np.prod(x.shape[:-1]))
    codes = np.empty(x.shape, _NP_OF[target])
    scales = np.empty(x.shape[:-1], np.float32)
    fn = lib().oracle_quantize_rows if target == "i8" else lib().oracle_quantize_rows_f8
    fn(_ptr(codes), _ptr(scales), _ptr(x), DTYPES[dtype], rows, D)
    return codes, scales


def quantize_rows_u4(x, dtype):
    """4-bit rows by the linear b-bit formula (b = 4) over each row's min and
    max.  Returns (codes uint8 [..., D/2], meta float32 [..., 2] = (x_min,
    range))."""
    x = _check(x, dtype, "x")
    D = x.shape[-1]
    rows = int(np.prod(x.shape[:-1]))
    codes = np.empty(x.shape[:-1] + (D // 2,), np.uint8)
    meta = np.empty(x.shape[:-1] + (2,), np.float32)
    rc = lib().oracle_quantize_rows_u4(_ptr(codes), _ptr(meta), _ptr(x), DTYPES[dtype], rows, D)
    if rc != 0:
        raise RuntimeError(f"oracle_quantize_rows_u4 failed with {rc}")
    return codes, meta


def f8_to_f64(code: int) -> float:
    return lib().oracle_f8_to_f64(code)


def f8_from_f32(x: float) -> int:
    """Nearest e4m3 code (ties to even) to x, |x| <= 448."""
    return lib().oracle_f8_from_f32(x)


def kv_cache_write(k, v, k_cache, v_cache, slot_mapping, src_dtype, cache_dtype, k_scale=None,
                   v_scale=None, block_size=16):
    """In-place write of tokens into host pool images (see oracle.c)."""
    k = _check(k, src_dtype, "k")
    v = _check(v, src_dtype, "v")
    sm = _check(slot_mapping, np.int64, "slot_mapping")
    for a in (k_cache, v_cache, k_scale, v_scale):
        if a is not None and not a.flags.c_contiguous:
            raise ValueError("cache images must be C-contiguous (written in place)")
    T, Hkv, D = k.shape
    NB = k_cache.shape[0]
    rc = lib().oracle_kv_cache_write(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                     _ptr(v_scale), _ptr(sm), T, Hkv, D, block_size, NB,
                                     DTYPES[src_dtype], DTYPES[cache_dtype])
    if rc != 0:
        raise RuntimeError(f"oracle_kv_cache_write failed with {rc}")
