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

// Four rows of a group of four positions (word u: row u's four bytes, one
// per position) added to the group's column sums: each position's four row
// bytes in one word (a 4 x 4 byte transpose), then its moments by 4-way byte
// dot products.  Every sum is an exact integer below 961 * 255^2 < 2^32, in
// any order.
__device__ __forceinline__ void add_rows4(const uint32_t *vr, const uint32_t *vd, uint32_t acc[5][4])
{
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

// The window sums of a lane's four consecutive pixels on one row, none of
// them within R columns of a row end: from the column sums of positions
// kb .. kb + 11 of each plane (the lane's pixels are kb + 4 .. kb + 7), read
// with three 16-byte loads per plane.  The first pixel's window is added
// up, each next one slides by the column entering it and the one leaving it
// (exact integers: any order gives the same sums).
template <int R>
__device__ __forceinline__ void window_sums4(const int *lds, int plane, int kb, int s[5][4])
{
    static_assert(R >= 0 && R <= 4, "the lane's twelve positions hold windows of radius 4 at most");
#pragma unroll
    for (int m = 0; m < 5; m++) {
        const int4 *q = reinterpret_cast<const int4 *>(__builtin_assume_aligned(lds + m * plane + kb, 16));
        const int4 a = q[0], b = q[1], c = q[2];
        const int v[12] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c.x, c.y, c.z, c.w};
        int acc = v[4];
#pragma unroll
        for (int d = 1; d <= R; d++)
            acc += v[4 - d] + v[4 + d];
        s[m][0] = acc;
#pragma unroll
        for (int u = 1; u < 4; u++) {
            acc += v[4 + u + R] - v[4 + u - 1 - R];
            s[m][u] = acc;
        }
    }
}

struct SsimTerms {
    SsimParams p;
    // dword 3 of a raw buffer resource on this chip (no stride, no swizzle,
    // 32-bit data format), and an offset past any plane's end
    static constexpr int kBufWord3 = 0x00020000;
    static constexpr int kBufPastEnd = (int)0x80000000;
    static constexpr int kMaxRadius = 15;
    static constexpr int kSpan = 1024 + 2 * kMaxRadius;  // raster positions a chunk needs at most
    // LDS holds the column sums of five planes; position q of chunk c (first
    // pixel p0 = 1024 c) sits at index q - p0 + kLead of its plane, so that
    // every group of four positions 4m .. 4m + 3 starts on a 16-byte boundary.
    static constexpr int kLead = 16;  // kMaxRadius rounded up to a multiple of 4
    static constexpr int kPlane = kLead + 1024 + kMaxRadius + 1;  // 1056, a multiple of 4
    static constexpr int kLdsInts = 5 * kPlane;
    static_assert(kPlane % 4 == 0 && kLead % 4 == 0 && kLead >= kMaxRadius, "aligned planes");

    __device__ __forceinline__ Four chunk(const BatchArgs &, int, size_t c, int *lds_in) const
    {
        return chunk_at(c, lds_in);
    }

    // The terms of chunk c (pixels 1024 c .. 1024 c + 1023 in raster order),
    // lane t holding pixels 4t .. 4t + 3.  Block-level: every lane calls it
    // with the same chunk (two barriers).
    __device__ __forceinline__ Four chunk_at(size_t c, int *lds_in) const
    {
        int *lds = static_cast<int *>(__builtin_assume_aligned(lds_in, 16));
        const int t = threadIdx.x;
        const int w = p.width, h = p.height, r = p.radius;
        const int n = w * h;
        const int p0 = (int)(c * 1024);
        const int plast = (p0 + 1024 < n ? p0 + 1024 : n) - 1;
        const int q0 = p0 - r;
        const int nq = plast + r - q0 + 1;
        const int kd = kLead - r;  // LDS index of position q0 + k is k + kd
        // Rows at least as wide as the span: the span crosses at most one row
        // end, so one division per chunk gives every position's row and column
        // (q0 may be negative, in the row before the first).
        const bool wide = w >= kSpan;
        const int iq0 = q0 >= 0 ? q0 / w : -1;
        const int jq0 = q0 - iq0 * w;
        // Column sums with 4-byte loads: rows a multiple of four pixels wide
        // in planes whose rows and bases are 4-byte aligned put every group
        // of four raster positions 4m .. 4m + 3 on one row, in one word per
        // plane row; each lane loads its group's window rows at once.  Planes
        // below 2 GiB are read through buffer resources: the lane's offset of
        // its group's first window row, each row's offset from it in a
        // scalar register, rows outside the frame at an offset past the
        // buffer's end (which reads as zero).
        const bool quad = wide && (w & 3) == 0 && (p.stride & 3) == 0 &&
                          (((uintptr_t)p.ref | (uintptr_t)p.dis) & 3u) == 0;
        const bool viabuf = quad && (uint64_t)p.stride * (uint64_t)h <= (uint64_t)0x7FFFFFFF;
        __syncthreads();  // earlier reads of lds are done
        if (quad) {
            const int m0 = (q0 >= 0 ? q0 : q0 - 3) / 4;  // floor(q0 / 4)
            const int m1 = (q0 + nq - 1) / 4;
            const int span_rows = 2 * r + 1;  // window rows of a pixel away from the top and bottom
            const int bytes = viabuf ? (int)(p.stride * h) : 0;
            const __amdgpu_buffer_rsrc_t rr =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.ref), (short)0, bytes, kBufWord3);
            const __amdgpu_buffer_rsrc_t rd =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.dis), (short)0, bytes, kBufWord3);
            for (int m = m0 + t; m <= m1; m += 256) {
                const int q = 4 * m;  // first position of the group
                uint32_t acc[5][4];
#pragma unroll
                for (int e = 0; e < 4; e++)
                    acc[0][e] = acc[1][e] = acc[2][e] = acc[3][e] = acc[4][e] = 0u;
                int a0 = 0, rows = 0, j = 0;
                if (q >= 0 && q < n) {
                    // (the first group may start up to 3 positions before q0)
                    int i = iq0;
                    j = jq0 + (q - q0);
                    if (j < 0) {
                        j += w;
                        i--;
                    } else if (j >= w) {
                        j -= w;
                        i++;
                    }
                    a0 = i - r < 0 ? 0 : i - r;
                    const int a1 = i + r >= h ? h - 1 : i + r;
                    rows = a1 - a0 + 1;
                }
                if (viabuf) {
                    // every lane the same number of loads, none in a branch
                    const int o0 = a0 * (int)p.stride + j;
#pragma unroll 2
                    for (int rq = 0; rq < span_rows; rq += 4) {
                        uint32_t vr[4], vd[4];
#pragma unroll
                        for (int u = 0; u < 4; u++) {
                            const int row = rq + u;
                            const int vo = row < rows ? o0 : kBufPastEnd;
                            const int so = row * (int)p.stride;
                            vr[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rr, vo, so, 0);
                            vd[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rd, vo, so, 0);
                        }
                        add_rows4(vr, vd, acc);
                    }
                } else {
                    const uint8_t *pr = p.ref + (ptrdiff_t)a0 * p.stride + j;
                    const uint8_t *pd = p.dis + (ptrdiff_t)a0 * p.stride + j;
                    for (int rq = 0; rq < rows; rq += 4) {
                        uint32_t vr[4], vd[4];
#pragma unroll
                        for (int u = 0; u < 4; u++) {
                            const bool in = rq + u < rows;
                            vr[u] = in ? *reinterpret_cast<const uint32_t *>(pr + (ptrdiff_t)(rq + u) * p.stride) : 0u;
                            vd[u] = in ? *reinterpret_cast<const uint32_t *>(pd + (ptrdiff_t)(rq + u) * p.stride) : 0u;
                        }
                        add_rows4(vr, vd, acc);
                    }
                }
                // the group's four positions at once (positions outside the
                // chunk's span are stored too, and never read)
                const int kk = q - p0 + kLead;
#pragma unroll
                for (int pl = 0; pl < 5; pl++)
                    *reinterpret_cast<int4 *>(lds + pl * kPlane + kk) =
                        int4{(int)acc[pl][0], (int)acc[pl][1], (int)acc[pl][2], (int)acc[pl][3]};
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
                lds[k + kd] = sx;
                lds[kPlane + k + kd] = sy;
                lds[2 * kPlane + k + kd] = sxx;
                lds[3 * kPlane + k + kd] = syy;
                lds[4 * kPlane + k + kd] = sxy;
            }
        }
        __syncthreads();
        Four f;
        const int first = p0 + 4 * t;
        f.cnt = first < n ? (n - first < 4 ? n - first : 4) : 0;
        // The lane's first pixel: its row and column.
        int i0 = 0, j0 = 0;
        if (f.cnt > 0) {
            const int k = first - q0;
            if (wide) {
                i0 = iq0;
                j0 = jq0 + k;
                if (j0 >= w) {
                    j0 -= w;
                    i0++;
                }
            } else {
                i0 = first / w;
                j0 = first - i0 * w;
            }
        }
        // Four whole pixels on one row, none within r columns of its ends
        // (nearly every lane of a wide frame): the register windows.
        if (r <= 4 && f.cnt == 4 && j0 >= r && j0 + 3 + r <= w - 1) {
            int s[5][4];
            const int kb = 4 * t + kLead - 4;  // a multiple of 4
            switch (r) {
            case 0: window_sums4<0>(lds, kPlane, kb, s); break;
            case 1: window_sums4<1>(lds, kPlane, kb, s); break;
            case 2: window_sums4<2>(lds, kPlane, kb, s); break;
            case 3: window_sums4<3>(lds, kPlane, kb, s); break;
            default: window_sums4<4>(lds, kPlane, kb, s); break;
            }
            const int a0 = i0 - r < 0 ? 0 : i0 - r;
            const int a1 = i0 + r >= h ? h - 1 : i0 + r;
            const int64_t wc = (int64_t)((a1 - a0 + 1) * (2 * r + 1));
#pragma unroll
            for (int u = 0; u < 4; u++)
                f.v[u] = ssim_term_dev(s[0][u], s[1][u], s[2][u], s[3][u], s[4][u], wc, p.c1, p.c2);
            return f;
        }
        // Any other lane: the window sums of its pixels from the column sums
        // of their windows, the first added up, each next one on the same
        // row by adding the column entering the window and taking out the
        // one leaving it.
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
                        const int ka = k + r + kd;
                        sx += lds[ka];
                        sy += lds[kPlane + ka];
                        sxx += lds[2 * kPlane + ka];
                        syy += lds[3 * kPlane + ka];
                        sxy += lds[4 * kPlane + ka];
                    }
                    if (j - r - 1 >= 0) {
                        const int kl = k - r - 1 + kd;
                        sx -= lds[kl];
                        sy -= lds[kPlane + kl];
                        sxx -= lds[2 * kPlane + kl];
                        syy -= lds[3 * kPlane + kl];
                        sxy -= lds[4 * kPlane + kl];
                    }
                } else {
                    sx = sy = sxx = syy = sxy = 0;
                    for (int jj = b0; jj <= b1; jj++) {
                        const int kk = k + (jj - j) + kd;
                        sx += lds[kk];
                        sy += lds[kPlane + kk];
                        sxx += lds[2 * kPlane + kk];
                        syy += lds[3 * kPlane + kk];
                        sxy += lds[4 * kPlane + kk];
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
