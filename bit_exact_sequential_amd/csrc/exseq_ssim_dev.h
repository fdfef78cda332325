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

// The term's one division (also run alone by exseq_div_f64, so that tests
// can compare it with the host's division on many operands).
__device__ __forceinline__ double ssim_div(double num, double den) { return num / den; }

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
    return ssim_div(num, den);
}

// Terms of a chunk (1024 consecutive pixels in raster order) for the 256
// lanes of a workgroup, 4 consecutive pixels per lane.  Block-level: every
// lane calls it with the same chunk (two barriers).
//   1. for every raster position from r before the chunk to r after it, the
//      column sums of x, y, x^2, y^2, xy over the rows of the window at that
//      row (edge-truncated), into LDS;
//   2. for every pixel, the sums of its row's window from those column sums
//      (the window's columns of a pixel's row are raster positions within r
//      of it, on the same row), and the term.  The window sums are exact
//      integers, so sliding them along a row (adding the column that enters,
//      subtracting the one that leaves) gives the same sums in any order.
// Four words w[u] of four bytes b(u, e) -> t[e] holding b(0, e) .. b(3, e)
// (byte e of every word, in word order), by byte permutes.
__device__ __forceinline__ void transpose4(const uint32_t *w, uint32_t *t)
{
    const uint32_t lo01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // b00 b10 b01 b11
    const uint32_t hi01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // b02 b12 b03 b13
    const uint32_t lo23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    t[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    t[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    t[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    t[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

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
        // Rows at least as wide as the span: the span crosses at most one row
        // end, so one division per chunk gives every position's row and column
        // (q0 may be negative, in the row before the first).
        const bool wide = w >= kSpan;
        const int iq0 = q0 >= 0 ? q0 / w : -1;
        const int jq0 = q0 - iq0 * w;
        // Column sums with 4-byte loads: rows a multiple of four pixels wide
        // in planes whose rows and bases are 4-byte aligned put every group
        // of four raster positions 4m .. 4m + 3 on one row, in one word per
        // plane row; each lane loads its group's window rows at once.
        const bool quad = wide && (w & 3) == 0 && (p.stride & 3) == 0 &&
                          (((uintptr_t)p.ref | (uintptr_t)p.dis) & 3u) == 0;
        __syncthreads();  // earlier reads of lds are done
        if (quad) {
            const int m0 = (q0 >= 0 ? q0 : q0 - 3) / 4;  // floor(q0 / 4)
            const int m1 = (q0 + nq - 1) / 4;
            for (int m = m0 + t; m <= m1; m += 256) {
                const int q = 4 * m;  // first position of the group
                uint32_t acc[5][4];
#pragma unroll
                for (int e = 0; e < 4; e++)
                    acc[0][e] = acc[1][e] = acc[2][e] = acc[3][e] = acc[4][e] = 0u;
                if (q >= 0 && q < n) {
                    // (the first group may start up to 3 positions before q0)
                    int i = iq0;
                    int j = jq0 + (q - q0);
                    if (j < 0) {
                        j += w;
                        i--;
                    } else if (j >= w) {
                        j -= w;
                        i++;
                    }
                    const int a0 = i - r < 0 ? 0 : i - r;
                    const int a1 = i + r >= h ? h - 1 : i + r;
                    const uint32_t *pr = reinterpret_cast<const uint32_t *>(p.ref + (ptrdiff_t)a0 * p.stride + j);
                    const uint32_t *pd = reinterpret_cast<const uint32_t *>(p.dis + (ptrdiff_t)a0 * p.stride + j);
                    const ptrdiff_t sw = p.stride / 4;
                    for (int row0 = a0; row0 <= a1; row0 += 4) {
                        uint32_t vr[4], vd[4];
#pragma unroll
                        for (int u = 0; u < 4; u++) {
                            const bool in = row0 + u <= a1;
                            vr[u] = in ? pr[(ptrdiff_t)(row0 - a0 + u) * sw] : 0u;
                            vd[u] = in ? pd[(ptrdiff_t)(row0 - a0 + u) * sw] : 0u;
                        }
                        // each position's four row bytes in one word (a
                        // 4 x 4 byte transpose), then its moments by 4-way
                        // byte dot products: every sum is an exact integer
                        // below 961 * 255^2 < 2^32, in any order
                        uint32_t tx[4], ty[4];
                        transpose4(vr, tx);
                        transpose4(vd, ty);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            acc[0][e] = __builtin_amdgcn_udot4(tx[e], 0x01010101u, acc[0][e], false);
                            acc[1][e] = __builtin_amdgcn_udot4(ty[e], 0x01010101u, acc[1][e], false);
                            acc[2][e] = __builtin_amdgcn_udot4(tx[e], tx[e], acc[2][e], false);
                            acc[3][e] = __builtin_amdgcn_udot4(ty[e], ty[e], acc[3][e], false);
                            acc[4][e] = __builtin_amdgcn_udot4(tx[e], ty[e], acc[4][e], false);
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int k = q + e - q0;
                    if (k >= 0 && k < nq) {
                        lds[k] = (int)acc[0][e];
                        lds[kSpan + k] = (int)acc[1][e];
                        lds[2 * kSpan + k] = (int)acc[2][e];
                        lds[3 * kSpan + k] = (int)acc[3][e];
                        lds[4 * kSpan + k] = (int)acc[4][e];
                    }
                }
            }
        } else {
            for (int k = t; k < nq; k += 256) {
                const int q = q0 + k;
                int sx = 0, sy = 0, sxx = 0, syy = 0, sxy = 0;
                if (q >= 0 && q < n) {
                    int i, j;
                    if (wide) {
                        i = iq0;
                        j = jq0 + k;
                        if (j >= w) {
                            j -= w;
                            i++;
                        }
                    } else {
                        i = q / w;
                        j = q - i * w;
                    }
                    const int a0 = i - r < 0 ? 0 : i - r;
                    const int a1 = i + r >= h ? h - 1 : i + r;
                    const uint8_t *pr = p.ref + (ptrdiff_t)a0 * p.stride + j;
                    const uint8_t *pd = p.dis + (ptrdiff_t)a0 * p.stride + j;
                    for (int row = a0; row <= a1; row++) {
                        const int x = *pr;
                        const int y = *pd;
                        sx += x;
                        sy += y;
                        sxx += x * x;
                        syy += y * y;
                        sxy += x * y;
                        pr += p.stride;
                        pd += p.stride;
                    }
                }
                lds[k] = sx;
                lds[kSpan + k] = sy;
                lds[2 * kSpan + k] = sxx;
                lds[3 * kSpan + k] = syy;
                lds[4 * kSpan + k] = sxy;
            }
        }
        __syncthreads();
        Four f;
        const int first = p0 + 4 * t;
        f.cnt = first < n ? (n - first < 4 ? n - first : 4) : 0;
        // The window sums of a lane's four pixels: the first from the column
        // sums of its window, each next one on the same row by adding the
        // column entering the window and taking out the one leaving it.
        int sx = 0, sy = 0, sxx = 0, syy = 0, sxy = 0;
        int pj = -2;  // column of the previous pixel (-2: none)
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int pix = first + u;
            double v = 0.0;
            if (u < f.cnt) {
                const int k = pix - q0;
                int i, j;
                if (wide) {
                    i = iq0;
                    j = jq0 + k;
                    if (j >= w) {
                        j -= w;
                        i++;
                    }
                } else {
                    i = pix / w;
                    j = pix - i * w;
                }
                const int a0 = i - r < 0 ? 0 : i - r;
                const int a1 = i + r >= h ? h - 1 : i + r;
                const int b0 = j - r < 0 ? 0 : j - r;
                const int b1 = j + r >= w ? w - 1 : j + r;
                if (j == pj + 1) {
                    if (j + r <= w - 1) {
                        const int ka = k + r;
                        sx += lds[ka];
                        sy += lds[kSpan + ka];
                        sxx += lds[2 * kSpan + ka];
                        syy += lds[3 * kSpan + ka];
                        sxy += lds[4 * kSpan + ka];
                    }
                    if (j - r - 1 >= 0) {
                        const int kd = k - r - 1;
                        sx -= lds[kd];
                        sy -= lds[kSpan + kd];
                        sxx -= lds[2 * kSpan + kd];
                        syy -= lds[3 * kSpan + kd];
                        sxy -= lds[4 * kSpan + kd];
                    }
                } else {
                    sx = sy = sxx = syy = sxy = 0;
                    for (int jj = b0; jj <= b1; jj++) {
                        const int kk = k + (jj - j);
                        sx += lds[kk];
                        sy += lds[kSpan + kk];
                        sxx += lds[2 * kSpan + kk];
                        syy += lds[3 * kSpan + kk];
                        sxy += lds[4 * kSpan + kk];
                    }
                }
                pj = j;
                const int64_t wc = (int64_t)(a1 - a0 + 1) * (int64_t)(b1 - b0 + 1);
                v = ssim_term_dev(sx, sy, sxx, syy, sxy, wc, p.c1, p.c2);
            }
            f.v[u] = v;
        }
        return f;
    }

    // Beside the sum: the frame's weight sum, if asked for.
    __device__ __forceinline__ void done() const
    {
        if (p.out_weight_sum)
            *p.out_weight_sum = p.weight_sum;
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
