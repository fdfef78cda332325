"""The oracle: plain, slow, obviously correct CPU implementations.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this package.  It shares no
code with the HIP path (``bit_exact_sequential_amd``) and never imports it;
the HIP path never imports this.

Functions and the passages they follow (page titles from the project
documentation the method comes from):

* :func:`seq_sum` -- the in-order fp64 loop ``s += x[i]`` (Research-1433
  "Forming the CPU's sequential double sums on a GPU, bit for bit", Question;
  Research-1424 "integer_ssim_cuda and the CPU's frame sum", Findings 1).
  Plain C in ``seq_sum.c``.
* :func:`box_moments`, :func:`ssim_term`, :func:`ssim_frame_sum` -- the
  integer-SSIM int64 window moments and the per-pixel fp64 term added in
  raster order (Research-1424 Findings 1; ADR-1443 "integer_ssim_sycl computes
  the CPU's fp64 term in 64-bit integers and adds in the CPU's order",
  Context).  Plain C in ``ssim_ref.c``.
* :func:`seq_sum_many` -- many independent loops (the pyramid batch).
* :func:`seq_sum_interleaved` -- k loops over records of k doubles, one
  accumulator per field, and each sum's float mean ``(float)(sum / windows)``
  (ADR-1464 "float_ssim_cuda adds its frame sums in the CPU's raster order,
  on the host", Context and Decision).  Plain C in ``seq_sum.c``.

Every function is pinned by ``tests/test_oracle_pins.py`` against values that
the pages and mathematics fix (closed forms, exact rational brute force, the
binade identity, an independent CPython evaluation, two integer moment
methods).  The deterministic tree sum has no oracle value: its parity is
unpinned by design (only determinism and the standard error bound are
checked).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_SOURCES = ("seq_sum.c", "ssim_ref.c")
# No contraction, no fast-math, SSE2 doubles (no x87 excess precision).
CFLAGS = ("-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-fPIC", "-shared", "-std=c11")

_lib = None


def build(out_path: str = _LIB_PATH, sources=None, extra_flags=()) -> str:
    """Compile the oracle with gcc into ``out_path`` and return the path."""
    srcs = [os.path.join(_HERE, s) for s in (sources or _SOURCES)]
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, *srcs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def load(path: str | None = None):
    """Load a compiled oracle library (building the default one if absent)."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        path = _LIB_PATH
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_seq_sum_f64.restype = ctypes.c_double
    lib.oracle_seq_sum_f64.argtypes = [dp, ctypes.c_size_t, ctypes.c_double]
    lib.oracle_seq_sum_f64_many.restype = None
    lib.oracle_seq_sum_f64_many.argtypes = [dp, i64p, i64p, ctypes.c_int64,
                                            dp, dp]
    lib.oracle_seq_sum_f64_interleaved.restype = None
    lib.oracle_seq_sum_f64_interleaved.argtypes = [dp, ctypes.c_size_t, ctypes.c_int64, dp, dp,
                                                   ctypes.POINTER(ctypes.c_float)]
    lib.oracle_box_moments.restype = None
    lib.oracle_box_moments.argtypes = [u8p, u8p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_ssize_t, ctypes.c_int,
                                       i64p, i64p, i64p, i64p, i64p, i64p]
    lib.oracle_ssim_term.restype = ctypes.c_double
    lib.oracle_ssim_term.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_double,
                                                            ctypes.c_double]
    lib.oracle_ssim_frame_sum.restype = ctypes.c_double
    lib.oracle_ssim_frame_sum.argtypes = [u8p, u8p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_ssize_t,
                                          ctypes.c_int, ctypes.c_double,
                                          ctypes.c_double, dp, i64p]
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _i64ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _u8ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def seq_sum(x, init: float = 0.0, lib=None) -> float:
    """``s = init; for i in range(n): s += x[i]`` in IEEE fp64, in C."""
    lib = lib or load()
    a = np.ascontiguousarray(x, dtype=np.float64)
    return lib.oracle_seq_sum_f64(_dptr(a), a.size, float(init))


def seq_sum_many(arrays, inits=None, lib=None) -> np.ndarray:
    """Independent in-order sums of each array (one loop per array)."""
    lib = lib or load()
    arrays = [np.ascontiguousarray(a, dtype=np.float64) for a in arrays]
    ns = np.array([a.size for a in arrays], dtype=np.int64)
    offs = np.zeros(len(arrays), dtype=np.int64)
    if len(arrays) > 1:
        offs[1:] = np.cumsum(ns)[:-1]
    flat = np.concatenate(arrays) if arrays else np.zeros(0)
    flat = np.ascontiguousarray(flat, dtype=np.float64)
    ini = np.zeros(len(arrays)) if inits is None else np.asarray(inits, dtype=np.float64)
    out = np.zeros(len(arrays), dtype=np.float64)
    lib.oracle_seq_sum_f64_many(_dptr(flat), _i64ptr(offs), _i64ptr(ns),
                                len(arrays), _dptr(ini), _dptr(out))
    return out


def seq_sum_interleaved(x, k: int, inits=None, lib=None):
    """k in-order sums over records of k doubles (``x`` flat, record-major,
    ``k * windows`` values) and their float means -> (float64[k], float32[k])."""
    lib = lib or load()
    a = np.ascontiguousarray(x, dtype=np.float64).reshape(-1)
    assert a.size % k == 0
    windows = a.size // k
    ini = np.zeros(k) if inits is None else np.ascontiguousarray(inits, dtype=np.float64)
    out = np.zeros(k, dtype=np.float64)
    means = np.zeros(k, dtype=np.float32)
    lib.oracle_seq_sum_f64_interleaved(_dptr(a), windows, k, _dptr(ini), _dptr(out),
                                       means.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return out, means


def box_moments(ref, dis, radius: int = 3, lib=None):
    """Brute-force edge-truncated box sums (x, y, x2, y2, xy, w), int64."""
    lib = lib or load()
    r = np.ascontiguousarray(ref, dtype=np.uint8)
    d = np.ascontiguousarray(dis, dtype=np.uint8)
    h, w = r.shape
    outs = [np.zeros((h, w), dtype=np.int64) for _ in range(6)]
    lib.oracle_box_moments(_u8ptr(r), _u8ptr(d), w, h, w, radius,
                           *[_i64ptr(o) for o in outs])
    return tuple(outs)


def ssim_term(x, y, x2, y2, xy, w, c1, c2, lib=None) -> float:
    """The per-pixel fp64 term for one window (scalar, C, no contraction)."""
    lib = lib or load()
    return lib.oracle_ssim_term(int(x), int(y), int(x2), int(y2), int(xy),
                                int(w), float(c1), float(c2))


def ssim_frame_sum(ref, dis, radius: int = 3, c1: float = None,
                   c2: float = None, want_terms: bool = False, lib=None):
    """Raster-order fp64 sum of every pixel's term.

    Returns ``(sum, weight_sum, terms_or_None)``.
    """
    lib = lib or load()
    if c1 is None:
        c1 = SSIM_C1
    if c2 is None:
        c2 = SSIM_C2
    r = np.ascontiguousarray(ref, dtype=np.uint8)
    d = np.ascontiguousarray(dis, dtype=np.uint8)
    h, w = r.shape
    terms = np.zeros((h, w), dtype=np.float64) if want_terms else None
    ws = np.zeros(1, dtype=np.int64)
    s = lib.oracle_ssim_frame_sum(_u8ptr(r), _u8ptr(d), w, h, w, radius,
                                  float(c1), float(c2),
                                  _dptr(terms) if terms is not None else None,
                                  _i64ptr(ws))
    return s, int(ws[0]), terms


# The stabilisers of the fused workload: c1 = (0.01*255)^2 and
# c2 = (0.03*255)^2, each evaluated in fp64 in that order (k = 0.01*255.0,
# then k*k).  Research-1424 Findings 1 notes that such constants are the
# doubles their expressions evaluate to, so the order of evaluation is part
# of the definition.
_K1 = 0.01 * 255.0
_K2 = 0.03 * 255.0
SSIM_C1 = _K1 * _K1
SSIM_C2 = _K2 * _K2
