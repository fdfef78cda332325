"""Bit-exact sequential fp64 sums on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libexseq.so`` (C ABI in ``include/exseq.h``).  It
only marshals arguments: every step of every sum runs in the library's HIP
kernels.  PyTorch supplies device memory and the stream.  There is no CPU
fallback: if the library or a GPU is missing, these functions raise.

``exact_seq_sum(x)`` returns a device tensor holding exactly the bits of
``s = 0.0; for v in x: s += v`` in IEEE fp64 (round to nearest, ties to even).
"""

from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libexseq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "exseq.h")

EXSEQ_OK, EXSEQ_EINVAL, EXSEQ_EWORKSPACE, EXSEQ_EHIP, EXSEQ_ESCRATCH = 0, -1, -2, -3, -4

PLAN_AUTO = 0
PLAN_ALL_FALLBACK = 1
PLAN_PLUS_ONE = 2
PLAN_MINUS_ONE = 3
PLAN_FIXED = 4
PLAN_ALL_ZERO = 5


def plan_fixed(key: int) -> int:
    """Flags that plan every chunk for ``key`` = sign << 11 | biased exponent."""
    return PLAN_FIXED | ((key & 0xFFF) << 8)


WALK_ONLY = 1 << 6
CHAIN_CUT = 1 << 7
PLAN_REUSE = 1 << 20
CHAIN_PATH = 1 << 21
PASS_PATH = 1 << 22
SSIM_IN_TILES = 1 << 23  # ssim_term_and_sum: the sum's tiles form the terms


def tile_flag(chunks_per_tile: int) -> int:
    """Flags that choose the chunks per tile of the single pass (1, 2 or 4)."""
    return {1: 1, 2: 2, 4: 3}[chunks_per_tile] << 4


MUT_TIE_UP = 1
MUT_NO_BINADE_CHECK = 2
MUT_NO_UPPER_CHECK = 4
MUT_IGNORE_PARITY = 8
MUT_NO_RUN_TOP = 16

CHUNK_TERMS = 1024
STAT_NONFINITE = 1


class Stats(ctypes.Structure):
    _fields_ = [("chunks", ctypes.c_uint64), ("fast_chunks", ctypes.c_uint64),
                ("fallback_chunks", ctypes.c_uint64), ("fallback_terms", ctypes.c_uint64),
                ("first_fallback", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("plan_misses", ctypes.c_uint32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


STATS_BYTES = ctypes.sizeof(Stats)

_lib = None


class ExseqError(RuntimeError):
    pass


def lib():
    """Load libexseq.so (built in-tree by ``python -m bit_exact_sequential_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ExseqError("libexseq.so is not built: run "
                         "`python -m bit_exact_sequential_amd.build`")
    # torch's ROCm wheel carries its own HIP runtime under the same soname as
    # /opt/rocm's.  Loading torch first makes libexseq.so bind to that one
    # runtime, so torch's streams and events are valid handles for the
    # library; loading the library first would map a second runtime.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    sz, vp, u32, i32 = ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
    L.exact_seq_sum_f64_workspace_size.restype = sz
    L.exact_seq_sum_f64_workspace_size.argtypes = [sz]
    L.exact_seq_sum_f64.restype = i32
    L.exact_seq_sum_f64.argtypes = [vp, sz, ctypes.c_double, vp, vp, sz, vp, u32, vp]
    L.exact_seq_sum_f64_noalloc_max_terms.restype = sz
    L.exact_seq_sum_f64_noalloc_max_terms.argtypes = []
    L.exact_seq_sum_f64_noalloc.restype = i32
    L.exact_seq_sum_f64_noalloc.argtypes = [vp, sz, ctypes.c_double, vp, vp, u32, vp]
    L.exact_seq_sum_f64_batch_workspace_size.restype = sz
    L.exact_seq_sum_f64_batch_workspace_size.argtypes = [ctypes.POINTER(sz), sz]
    L.exact_seq_sum_f64_batch.restype = i32
    L.exact_seq_sum_f64_batch.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(sz),
                                          ctypes.POINTER(ctypes.c_double), sz, vp, vp, sz,
                                          vp, u32, vp]
    L.exact_seq_sum_f64_interleaved_workspace_size.restype = sz
    L.exact_seq_sum_f64_interleaved_workspace_size.argtypes = [sz, i32]
    L.exact_seq_sum_f64_interleaved.restype = i32
    L.exact_seq_sum_f64_interleaved.argtypes = [vp, sz, i32, ctypes.POINTER(ctypes.c_double), vp,
                                                vp, vp, sz, vp, u32, vp]
    L.ssim_term_and_sum_workspace_size.restype = sz
    L.ssim_term_and_sum_workspace_size.argtypes = [i32, i32]
    L.ssim_term_and_sum.restype = i32
    L.ssim_term_and_sum.argtypes = [vp, vp, i32, i32, ctypes.c_ssize_t, i32,
                                    ctypes.c_double, ctypes.c_double, vp, vp, vp, vp, sz,
                                    vp, u32, vp]
    L.tree_sum_f64_workspace_size.restype = sz
    L.tree_sum_f64_workspace_size.argtypes = [sz]
    L.tree_sum_f64.restype = i32
    L.tree_sum_f64.argtypes = [vp, sz, vp, vp, sz, vp]
    L.exseq_strerror.restype = ctypes.c_char_p
    L.exseq_strerror.argtypes = [i32]
    L.exseq_version.restype = ctypes.c_char_p
    L.exseq_version.argtypes = []
    L.exseq_profile_kernel_count.restype = i32
    L.exseq_profile_kernel_count.argtypes = []
    L.exseq_profile_kernel_name.restype = ctypes.c_char_p
    L.exseq_profile_kernel_name.argtypes = [i32]
    L.exact_seq_sum_f64_profiled.restype = i32
    L.exact_seq_sum_f64_profiled.argtypes = [vp, sz, ctypes.c_double, vp, vp, sz, vp, u32, vp,
                                             ctypes.POINTER(vp), i32]
    L.exseq_stream_read_f64.restype = i32
    L.exseq_stream_read_f64.argtypes = [vp, sz, vp, vp]
    L.exseq_div_f64.restype = i32
    L.exseq_div_f64.argtypes = [vp, vp, vp, sz, vp]
    L.exseq_twin_seq_sum_f64.restype = ctypes.c_double
    L.exseq_twin_seq_sum_f64.argtypes = [vp, sz, ctypes.c_double, u32, u32, vp]
    L.exseq_twin_chain_sum_f64.restype = ctypes.c_double
    L.exseq_twin_chain_sum_f64.argtypes = [vp, sz, ctypes.c_double, u32, u32, ctypes.c_int64, vp, vp]
    L.exseq_model_seq_sum_f64.restype = ctypes.c_double
    L.exseq_model_seq_sum_f64.argtypes = [vp, sz, ctypes.c_double, sz, u32, u32,
                                          ctypes.POINTER(Stats)]
    _lib = L
    return L


def hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process (expect one)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                paths.add(parts[-1])
    return sorted(paths)


def declared_functions(header: str = HEADER):
    """Names of the functions ``include/exseq.h`` declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def _check(rc: int, what: str):
    if rc != EXSEQ_OK:
        raise ExseqError("%s: %s (%d)" % (what, lib().exseq_strerror(rc).decode(), rc))


# ---------------------------------------------------------------------------
# Device entry points (torch tensors on a ROCm device)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _side_stream(stream, device):
    """The caller's stream when it is not the device's current one, else None."""
    torch = _torch()
    if stream is None or stream == torch.cuda.current_stream(device):
        return None
    return stream


def _keep_for(stream, device, *tensors):
    """Tensors allocated here on the current stream but written by kernels on
    another stream: tell the caching allocator, so that their memory is not
    handed out again before that stream has finished with it."""
    s = _side_stream(stream, device)
    if s is not None:
        for t in tensors:
            if t is not None:
                t.record_stream(s)


def _sync_for_stats(stream, device):
    s = _side_stream(stream, device)
    if s is not None:
        s.synchronize()


def _check_device_f64(x):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ExseqError("expected a ROCm device tensor")
    if x.dtype != torch.float64:
        raise ExseqError("expected float64 terms")
    if not x.is_contiguous():
        raise ExseqError("expected contiguous terms")


def workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def exact_seq_sum(x, init: float = 0.0, *, flags: int = 0, out=None, ws=None,
                  stats: bool = False, stream=None):
    """Exact in-order fp64 sum of a device tensor (flattened, raster order).

    Returns a 1-element float64 device tensor (and a stats dict when
    ``stats=True``, which synchronises)."""
    torch = _torch()
    _check_device_f64(x)
    L = lib()
    n = x.numel()
    dev = x.device
    new_out = out is None
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=dev)
    need = L.exact_seq_sum_f64_workspace_size(n)
    new_ws = ws is None
    if ws is None:
        ws = workspace(need, dev)
    st = torch.empty(STATS_BYTES, dtype=torch.uint8, device=dev) if stats else None
    rc = L.exact_seq_sum_f64(x.data_ptr() if n else None, n, float(init), out.data_ptr(),
                             ws.data_ptr(), ws.numel(), _stream_handle(stream, dev),
                             int(flags), st.data_ptr() if st is not None else None)
    _check(rc, "exact_seq_sum_f64")
    _keep_for(stream, dev, out if new_out else None, ws if new_ws else None, st)
    if stats:
        _sync_for_stats(stream, dev)
        return out, _read_stats(st)
    return out


def exact_seq_sum_noalloc(x, init: float = 0.0, *, flags: int = 0, out=None,
                          stats: bool = False, stream=None):
    """``exact_seq_sum`` through ``exact_seq_sum_f64_noalloc``: the library
    takes no workspace from the caller (its static per-GPU array stands in).
    Only ``out`` (and the stats buffer) are allocated here, by torch, when not
    given."""
    torch = _torch()
    _check_device_f64(x)
    L = lib()
    n = x.numel()
    dev = x.device
    new_out = out is None
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=dev)
    st = torch.empty(STATS_BYTES, dtype=torch.uint8, device=dev) if stats else None
    with torch.cuda.device(dev):
        rc = L.exact_seq_sum_f64_noalloc(x.data_ptr() if n else None, n, float(init),
                                         out.data_ptr(), _stream_handle(stream, dev),
                                         int(flags), st.data_ptr() if st is not None else None)
    _check(rc, "exact_seq_sum_f64_noalloc")
    _keep_for(stream, dev, out if new_out else None, st)
    if stats:
        _sync_for_stats(stream, dev)
        return out, _read_stats(st)
    return out


def exact_seq_sum_interleaved(x, k: int, inits=None, *, means: bool = True, flags: int = 0,
                              out=None, ws=None, stats: bool = False, stream=None):
    """k independent in-order sums over records of k doubles (``x``: device
    float64, ``k * windows`` values, record-major) and, with ``means``, each
    sum's float mean ``(float)(sum / windows)``.

    Returns (sums tensor[k] f64, means tensor[k] f32 or None[, stats list])."""
    torch = _torch()
    _check_device_f64(x)
    n = x.numel()
    if k < 1 or n % k:
        raise ExseqError("x must hold k * windows doubles")
    windows = n // k
    L = lib()
    dev = x.device
    new_out = out is None
    if out is None:
        out = torch.empty(k, dtype=torch.float64, device=dev)
    mt = torch.empty(k, dtype=torch.float32, device=dev) if means else None
    ini = None
    if inits is not None:
        ini = (ctypes.c_double * k)(*[float(v) for v in inits])
    need = L.exact_seq_sum_f64_interleaved_workspace_size(windows, k)
    new_ws = ws is None
    if ws is None:
        ws = workspace(need, dev)
    st = torch.empty(STATS_BYTES * k, dtype=torch.uint8, device=dev) if stats else None
    rc = L.exact_seq_sum_f64_interleaved(x.data_ptr() if n else None, windows, k, ini,
                                         out.data_ptr(), mt.data_ptr() if mt is not None else None,
                                         ws.data_ptr(), ws.numel(), _stream_handle(stream, dev),
                                         int(flags), st.data_ptr() if st is not None else None)
    _check(rc, "exact_seq_sum_f64_interleaved")
    _keep_for(stream, dev, out if new_out else None, mt, ws if new_ws else None, st)
    if stats:
        _sync_for_stats(stream, dev)
        return out, mt, _read_stats_many(st, k)
    return out, mt


def _read_stats(st):
    raw = bytes(st.cpu().numpy().tobytes())
    return Stats.from_buffer_copy(raw).as_dict()


def _read_stats_many(st, count):
    raw = bytes(st.cpu().numpy().tobytes())
    return [Stats.from_buffer_copy(raw[k * STATS_BYTES:(k + 1) * STATS_BYTES]).as_dict()
            for k in range(count)]


def exact_seq_sum_batch(xs, inits=None, *, flags: int = 0, out=None, ws=None,
                        stats: bool = False, stream=None):
    """Independent exact sums of a list of device tensors -> device tensor."""
    torch = _torch()
    count = len(xs)
    for x in xs:
        _check_device_f64(x)
    L = lib()
    dev = xs[0].device if count else torch.device("cuda")
    ns = (ctypes.c_size_t * max(count, 1))(*[x.numel() for x in xs])
    ptrs = (ctypes.c_void_p * max(count, 1))(*[x.data_ptr() if x.numel() else None for x in xs])
    ini = None
    if inits is not None:
        ini = (ctypes.c_double * max(count, 1))(*[float(v) for v in inits])
    new_out = out is None
    if out is None:
        out = torch.empty(max(count, 1), dtype=torch.float64, device=dev)
    need = L.exact_seq_sum_f64_batch_workspace_size(ns, count)
    new_ws = ws is None
    if ws is None:
        ws = workspace(need, dev)
    st = torch.empty(STATS_BYTES * max(count, 1), dtype=torch.uint8, device=dev) if stats else None
    rc = L.exact_seq_sum_f64_batch(ptrs, ns, ini, count, out.data_ptr(), ws.data_ptr(),
                                   ws.numel(), _stream_handle(stream, dev), int(flags),
                                   st.data_ptr() if st is not None else None)
    _check(rc, "exact_seq_sum_f64_batch")
    _keep_for(stream, dev, out if new_out else None, ws if new_ws else None, st)
    if stats:
        _sync_for_stats(stream, dev)
        return out[:count], _read_stats_many(st, count)
    return out[:count]


def ssim_term_and_sum(ref, dis, radius: int = 3, c1: float = None, c2: float = None, *,
                      flags: int = 0, want_terms: bool = False, ws=None, stats: bool = False,
                      stream=None):
    """Integer-SSIM frame sum of two uint8 planes (H x W, row-major): every
    pixel's term formed on the device, then added in raster order.  By default
    a producer launch writes the terms (into ``terms`` with ``want_terms``,
    else into the workspace) and the exact sum adds them; with
    ``flags | SSIM_IN_TILES`` the sum's tiles form the terms themselves.

    Returns (sum tensor[1] f64, weight-sum tensor[1] i64, terms or None[, stats])."""
    torch = _torch()
    for p in (ref, dis):
        if not isinstance(p, torch.Tensor) or p.device.type != "cuda" or p.dtype != torch.uint8:
            raise ExseqError("expected uint8 device planes")
        if p.dim() != 2:
            raise ExseqError("expected 2-D planes")
    if ref.shape != dis.shape or ref.stride() != dis.stride() or ref.stride(1) != 1:
        raise ExseqError("planes must share a row-major layout")
    if c1 is None:
        c1 = (0.01 * 255.0) * (0.01 * 255.0)
    if c2 is None:
        c2 = (0.03 * 255.0) * (0.03 * 255.0)
    L = lib()
    h, w = ref.shape
    dev = ref.device
    out = torch.empty(1, dtype=torch.float64, device=dev)
    wsum = torch.empty(1, dtype=torch.int64, device=dev)
    terms = torch.empty((h, w), dtype=torch.float64, device=dev) if want_terms else None
    need = L.ssim_term_and_sum_workspace_size(w, h)
    new_ws = ws is None
    if ws is None:
        ws = workspace(need, dev)
    st = torch.empty(STATS_BYTES, dtype=torch.uint8, device=dev) if stats else None
    rc = L.ssim_term_and_sum(ref.data_ptr(), dis.data_ptr(), w, h, ref.stride(0), radius,
                             float(c1), float(c2), out.data_ptr(), wsum.data_ptr(),
                             terms.data_ptr() if terms is not None else None, ws.data_ptr(),
                             ws.numel(), _stream_handle(stream, dev), int(flags),
                             st.data_ptr() if st is not None else None)
    _check(rc, "ssim_term_and_sum")
    _keep_for(stream, dev, out, wsum, terms, ws if new_ws else None, st)
    if stats:
        _sync_for_stats(stream, dev)
        return out, wsum, terms, _read_stats(st)
    return out, wsum, terms


def tree_sum(x, *, out=None, ws=None, stream=None):
    """Deterministic fixed-tree fp64 sum (NOT the loop's bits)."""
    torch = _torch()
    _check_device_f64(x)
    L = lib()
    n = x.numel()
    new_out = out is None
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=x.device)
    new_ws = ws is None
    if ws is None:
        ws = workspace(L.tree_sum_f64_workspace_size(n), x.device)
    rc = L.tree_sum_f64(x.data_ptr() if n else None, n, out.data_ptr(), ws.data_ptr(),
                        ws.numel(), _stream_handle(stream, x.device))
    _check(rc, "tree_sum_f64")
    _keep_for(stream, x.device, out if new_out else None, ws if new_ws else None)
    return out


# ---------------------------------------------------------------------------
# Host model of the method (CPU; test infrastructure for the rules)
# ---------------------------------------------------------------------------

def device_div(a, b, *, stream=None):
    """a / b elementwise (float64 device tensors) with the fused SSIM term's
    device division."""
    torch = _torch()
    _check_device_f64(a)
    _check_device_f64(b)
    if a.numel() != b.numel():
        raise ExseqError("a and b must have the same size")
    q = torch.empty_like(a)
    rc = lib().exseq_div_f64(a.data_ptr(), b.data_ptr(), q.data_ptr(), a.numel(),
                             _stream_handle(stream, a.device))
    _check(rc, "exseq_div_f64")
    _keep_for(stream, a.device, q)
    return q


def twin_seq_sum(x, init: float = 0.0, flags: int = 0, mutations: int = 0):
    """The single pass replayed on the host in the kernels' grouping of the
    terms (lanes, waves, tiles, finisher windows); returns (sum, stats)."""
    import numpy as np
    a = np.ascontiguousarray(x, dtype=np.float64)
    st = Stats()
    s = lib().exseq_twin_seq_sum_f64(a.ctypes.data if a.size else None, a.size, float(init),
                                     int(flags), int(mutations), ctypes.byref(st))
    return s, st.as_dict()


def twin_chain_sum(x, init: float = 0.0, flags: int = 0, mutations: int = 0, skew: int = 0):
    """The tile chain (four chunks per tile) replayed on the host in the
    kernels' grouping: the tiles' runs, the chain look-back's composition of
    the regular tiles, the irregular tiles' chunks from the exact sum and the
    walk's resume.  skew moves every planned prefix by skew * 2^-30 of itself.
    Returns (sum, stats, paths): paths counts the look-back's waves composed
    as integer sums, falling sums, pairs alone and full runs, the composed
    runs applied, and the stops of the chain."""
    import numpy as np
    a = np.ascontiguousarray(x, dtype=np.float64)
    st = Stats()
    paths = (ctypes.c_uint64 * 6)()
    s = lib().exseq_twin_chain_sum_f64(a.ctypes.data if a.size else None, a.size, float(init),
                                       int(flags), int(mutations), int(skew), ctypes.byref(st),
                                       paths)
    return s, st.as_dict(), dict(zip(("plain", "falling", "pairs", "runs", "applied", "stops"),
                                     (int(v) for v in paths)))


def model_seq_sum(x, init: float = 0.0, chunk_terms: int = CHUNK_TERMS, flags: int = 0,
                  mutations: int = 0):
    """The kernels' rules walked on the host; returns (sum, stats dict)."""
    import numpy as np
    a = np.ascontiguousarray(x, dtype=np.float64)
    st = Stats()
    s = lib().exseq_model_seq_sum_f64(a.ctypes.data if a.size else None, a.size, float(init),
                                      int(chunk_terms), int(flags), int(mutations),
                                      ctypes.byref(st))
    return s, st.as_dict()
