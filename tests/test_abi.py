"""The C-ABI library loads and exports every symbol include/exseq.h declares;
argument checks reject bad calls before anything reaches a GPU (CPU only)."""

import ctypes
import os

import bit_exact_sequential_amd as ex


def test_library_exports_every_declared_function():
    L = ex.lib()
    names = ex.declared_functions()
    assert "exact_seq_sum_f64" in names and "ssim_term_and_sum" in names
    for n in names:
        assert hasattr(L, n), n


def test_strerror_and_version():
    L = ex.lib()
    for code in (0, -1, -2, -3, -4, -99):
        assert L.exseq_strerror(code)
    assert b"gfx950" in L.exseq_version()


def test_workspace_sizes():
    L = ex.lib()
    assert L.exact_seq_sum_f64_workspace_size(0) >= 0
    w = L.exact_seq_sum_f64_workspace_size(8294400)
    # per 1024 terms: a plan status word, a 28-byte descriptor and 408 bytes
    # of chain words: under 6 % of the 66 MB of terms
    assert 8100 * 32 <= w <= 8100 * 444 + 8192
    assert w < 8294400 * 8 * 6 // 100
    assert L.tree_sum_f64_workspace_size(1000) > 0
    # the SSIM sum's workspace holds the producer's terms (8 bytes a pixel)
    # beside the exact sum's
    assert L.ssim_term_and_sum_workspace_size(3840, 2160) >= (
        3840 * 2160 * 8 + L.exact_seq_sum_f64_workspace_size(3840 * 2160))
    ns = (ctypes.c_size_t * 3)(10, 100000, 0)
    assert L.exact_seq_sum_f64_batch_workspace_size(ns, 3) >= L.exact_seq_sum_f64_workspace_size(100000)


def test_argument_errors_return_before_any_launch():
    L = ex.lib()
    # null terms with n > 0
    assert L.exact_seq_sum_f64(None, 10, 0.0, 8, 64, 1 << 20, None, 0, None) == ex.EXSEQ_EINVAL
    # misaligned output
    assert L.exact_seq_sum_f64(64, 10, 0.0, 9, 64, 1 << 20, None, 0, None) == ex.EXSEQ_EINVAL
    # workspace too small
    assert L.exact_seq_sum_f64(64, 100000, 0.0, 8, 64, 16, None, 0, None) == ex.EXSEQ_EWORKSPACE
    # bad geometry
    assert L.ssim_term_and_sum(64, 64, 0, 5, 5, 3, 1.0, 1.0, 8, None, None, 64, 1 << 20, None,
                               0, None) == ex.EXSEQ_EINVAL
    assert L.ssim_term_and_sum(64, 64, 5, 5, 4, 3, 1.0, 1.0, 8, None, None, 64, 1 << 20, None,
                               0, None) == ex.EXSEQ_EINVAL
    assert L.tree_sum_f64(None, 5, 8, 64, 1 << 20, None) == ex.EXSEQ_EINVAL


def test_noalloc_limits_checked_before_any_launch():
    L = ex.lib()
    mx = L.exact_seq_sum_f64_noalloc_max_terms()
    # the static array holds the workspace of the largest accepted input
    assert L.exact_seq_sum_f64_workspace_size(mx) <= 8 << 20 < L.exact_seq_sum_f64_workspace_size(mx + 1)
    assert mx >= 8294400
    # beyond it: an error before anything touches the GPU
    assert L.exact_seq_sum_f64_noalloc(64, mx + 1, 0.0, 8, None, 0, None) == ex.EXSEQ_ESCRATCH
    assert L.exact_seq_sum_f64_noalloc(None, 10, 0.0, 8, None, 0, None) == ex.EXSEQ_EINVAL
    assert L.exact_seq_sum_f64_noalloc(64, 10, 0.0, 9, None, 0, None) == ex.EXSEQ_EINVAL
    assert b"scratch" in L.exseq_strerror(ex.EXSEQ_ESCRATCH)


def test_built_for_gfx950():
    data = open(ex.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_single_hip_runtime():
    """torch and libexseq.so share one HIP runtime (stream handles are valid
    across them)."""
    ex.lib()
    maps = ex.hip_runtimes_mapped()
    assert len(maps) == 1, maps
