/*
 * Oracle: integer SSIM window moments and the per-pixel fp64 term, summed in
 * raster order.  TEST INFRASTRUCTURE ONLY (same rules as seq_sum.c: only
 * tests/, smoke() and bench.py's cpu_baseline leg use it; no code shared with
 * the HIP path).
 *
 * Definitions followed:
 *  - Research-1424 "integer_ssim_cuda and the CPU's frame sum", Findings 1:
 *    every pixel's term is added into one double, row after row; the term is
 *        w * (2*mxy + c1) * (c2 + 2*(xy*w_d - mxy))
 *        / ((mx2 + my2 + c1) * (x2*w_d - mx2 + y2*w_d - my2 + c2))
 *    evaluated left to right as C evaluates it, with no contraction.
 *  - ADR-1443 "integer_ssim_sycl computes the CPU's fp64 term ...", Context:
 *    the moments are int64 sums; mx2, my2, mxy are the three products of two
 *    moments (x*x, y*y, x*y) formed in fp64 from the converted moments.
 *  - The window is the edge-truncated (2r+1)x(2r+1) box (r = 3 gives 7x7)
 *    and w is the number of pixels it covers: the pages name the box and w
 *    but not its edges, and a window cut by the frame keeps the pixels inside.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (no FMA may form).
 */
#include <stddef.h>
#include <stdint.h>

/* Brute force: every window summed pixel by pixel. */
void oracle_box_moments(const uint8_t *ref, const uint8_t *dis, int width,
                        int height, ptrdiff_t stride, int radius, int64_t *mx,
                        int64_t *my, int64_t *mx2, int64_t *my2, int64_t *mxy,
                        int64_t *mw)
{
    for (int i = 0; i < height; i++) {
        for (int j = 0; j < width; j++) {
            int64_t sx = 0, sy = 0, sxx = 0, syy = 0, sxy = 0, sw = 0;
            for (int a = i - radius; a <= i + radius; a++) {
                if (a < 0 || a >= height)
                    continue;
                for (int b = j - radius; b <= j + radius; b++) {
                    if (b < 0 || b >= width)
                        continue;
                    int64_t p = ref[(ptrdiff_t)a * stride + b];
                    int64_t q = dis[(ptrdiff_t)a * stride + b];
                    sx += p;
                    sy += q;
                    sxx += p * p;
                    syy += q * q;
                    sxy += p * q;
                    sw += 1;
                }
            }
            size_t k = (size_t)i * (size_t)width + (size_t)j;
            mx[k] = sx;
            my[k] = sy;
            mx2[k] = sxx;
            my2[k] = syy;
            mxy[k] = sxy;
            mw[k] = sw;
        }
    }
}

double oracle_ssim_term(int64_t x, int64_t y, int64_t x2, int64_t y2,
                        int64_t xy, int64_t w, double c1, double c2)
{
    double w_d = (double)w;
    double mx2 = (double)x * (double)x;
    double my2 = (double)y * (double)y;
    double mxy = (double)x * (double)y;
    return w * (2 * mxy + c1) * (c2 + 2 * (xy * w_d - mxy)) /
           ((mx2 + my2 + c1) * (x2 * w_d - mx2 + y2 * w_d - my2 + c2));
}

/* The whole frame: moments by brute force, the term per pixel, one running
 * double in raster order.  `terms` (nullable) receives every term at its
 * raster index.  `wsum` (nullable) receives the sum of the window counts. */
double oracle_ssim_frame_sum(const uint8_t *ref, const uint8_t *dis, int width,
                             int height, ptrdiff_t stride, int radius,
                             double c1, double c2, double *terms,
                             int64_t *wsum)
{
    double s = 0.0;
    int64_t ws = 0;
    for (int i = 0; i < height; i++) {
        for (int j = 0; j < width; j++) {
            int64_t sx = 0, sy = 0, sxx = 0, syy = 0, sxy = 0, sw = 0;
            for (int a = i - radius; a <= i + radius; a++) {
                if (a < 0 || a >= height)
                    continue;
                for (int b = j - radius; b <= j + radius; b++) {
                    if (b < 0 || b >= width)
                        continue;
                    int64_t p = ref[(ptrdiff_t)a * stride + b];
                    int64_t q = dis[(ptrdiff_t)a * stride + b];
                    sx += p;
                    sy += q;
                    sxx += p * p;
                    syy += q * q;
                    sxy += p * q;
                    sw += 1;
                }
            }
            double t = oracle_ssim_term(sx, sy, sxx, syy, sxy, sw, c1, c2);
            if (terms)
                terms[(size_t)i * (size_t)width + (size_t)j] = t;
            s += t;
            ws += sw;
        }
    }
    if (wsum)
        *wsum = ws;
    return s;
}
