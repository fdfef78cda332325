// The integer-SSIM per-pixel fp64 term, formed on the device inside the
// exact sum's tiles (the terms are never stored unless asked for).
//
// Term (Research-1424 "integer_ssim_cuda and the CPU's frame sum", Findings 1;
// ADR-1443 "integer_ssim_sycl computes the CPU's fp64 term in 64-bit integers
// and adds in the CPU's order", Context and Decision):
//     w*(2*mxy + c1)*(c2 + 2*(xy*w - mxy))
//       / ((mx2 + my2 + c1)*(x2*w - mx2 + y2*w - my2 + c2))
// with x, y, x2, y2, xy the integer sums of the edge-truncated window, w its
// pixel count, mx2 = x*x, my2 = y*y, mxy = x*y in fp64.  The expression is
// evaluated left to right, one rounding per operation: the library is built
// with -ffp-contract=off, so no multiply is fused into an add, and the fp64
// divide is the compiler's correctly rounded sequence.
//
// For 8-bit planes and windows of at most 31 x 31 pixels every moment is
// below 961 * 255^2 < 2^26, so the window sums are exact in 32-bit integers
// (they equal the 64-bit sums the term is defined on), and every product of
// two moments is below 2^53 and converts to fp64 without rounding (ADR-1443
// Decision, "three shortcuts, each exact", second item).
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "exseq_internal.h"

namespace exseq {

__device__ __forceinline__ double ssim_term_dev(int64_t x, int64_t y, int64_t x2, int64_t y2,
                                                int64_t xy, int64_t w, double c1, double c2)
{
    const double w_d = (double)w;
    const double mx2 = (double)x * (double)x;
    const double my2 = (double)y * (double)y;
    const double mxy = (double)x * (double)y;
    const double num = w_d * (2.0 * mxy + c1) * (c2 + 2.0 * ((double)xy * w_d - mxy));
    const double den = (mx2 + my2 + c1) *
                       ((double)x2 * w_d - mx2 + (double)y2 * w_d - my2 + c2);
    return num / den;
}

// Terms of a chunk (1024 consecutive pixels in raster order) for the 256
// lanes of a workgroup, 4 consecutive pixels per lane.  Block-level: every
// lane calls it with the same chunk (two barriers).
//   1. for every raster position from r before the chunk to r after it, the
//      column sums of x, y, x^2, y^2, xy over the rows of the window at that
//      row (edge-truncated), into LDS;
//   2. for every pixel, the sums of its row's window from those column sums
//      (the window's columns of a pixel's row are raster positions within r
//      of it, on the same row), and the term.
struct SsimTerms {
    SsimParams p;
    static constexpr int kMaxRadius = 15;
    static constexpr int kSpan = 1024 + 2 * kMaxRadius;  // raster positions per chunk
    static constexpr int kLdsInts = 5 * kSpan;

    __device__ __forceinline__ Four chunk(const BatchArgs &, int, size_t c, int *lds) const
    {
        const int t = threadIdx.x;
        const int w = p.width, h = p.height, r = p.radius;
        const int n = w * h;
        const int p0 = (int)(c * 1024);
        const int plast = (p0 + 1024 < n ? p0 + 1024 : n) - 1;
        const int q0 = p0 - r;
        const int nq = plast + r - q0 + 1;
        __syncthreads();  // earlier reads of lds are done
        for (int k = t; k < nq; k += 256) {
            const int q = q0 + k;
            int sx = 0, sy = 0, sxx = 0, syy = 0, sxy = 0;
            if (q >= 0 && q < n) {
                const int i = q / w, j = q - (q / w) * w;
                const int a0 = i - r < 0 ? 0 : i - r;
                const int a1 = i + r >= h ? h - 1 : i + r;
                for (int row = a0; row <= a1; row++) {
                    const int x = p.ref[(ptrdiff_t)row * p.stride + j];
                    const int y = p.dis[(ptrdiff_t)row * p.stride + j];
                    sx += x;
                    sy += y;
                    sxx += x * x;
                    syy += y * y;
                    sxy += x * y;
                }
            }
            lds[k] = sx;
            lds[kSpan + k] = sy;
            lds[2 * kSpan + k] = sxx;
            lds[3 * kSpan + k] = syy;
            lds[4 * kSpan + k] = sxy;
        }
        __syncthreads();
        Four f;
        const int first = p0 + 4 * t;
        f.cnt = first < n ? (n - first < 4 ? n - first : 4) : 0;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int pix = first + u;
            double v = 0.0;
            if (u < f.cnt) {
                const int i = pix / w, j = pix - (pix / w) * w;
                const int a0 = i - r < 0 ? 0 : i - r;
                const int a1 = i + r >= h ? h - 1 : i + r;
                const int b0 = j - r < 0 ? 0 : j - r;
                const int b1 = j + r >= w ? w - 1 : j + r;
                int sx = 0, sy = 0, sxx = 0, syy = 0, sxy = 0;
                for (int jj = b0; jj <= b1; jj++) {
                    const int k = pix - q0 + (jj - j);
                    sx += lds[k];
                    sy += lds[kSpan + k];
                    sxx += lds[2 * kSpan + k];
                    syy += lds[3 * kSpan + k];
                    sxy += lds[4 * kSpan + k];
                }
                const int64_t wc = (int64_t)(a1 - a0 + 1) * (int64_t)(b1 - b0 + 1);
                v = ssim_term_dev(sx, sy, sxx, syy, sxy, wc, p.c1, p.c2);
            }
            f.v[u] = v;
        }
        return f;
    }

    // The terms of chunk c, also written to the caller's plane if asked for.
    __device__ __forceinline__ void keep(size_t c, const Four &f) const
    {
        if (!p.out_terms)
            return;
        const size_t first = c * 1024 + 4 * (size_t)threadIdx.x;
#pragma unroll
        for (int u = 0; u < 4; u++)
            if (u < f.cnt)
                p.out_terms[first + u] = f.v[u];
    }
};

}  // namespace exseq
