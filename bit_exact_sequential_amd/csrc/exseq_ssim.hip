// gfx950 producer of the integer-SSIM per-pixel fp64 term.
//
// Term (Research-1424 "integer_ssim_cuda and the CPU's frame sum", Findings 1;
// ADR-1443 "integer_ssim_sycl computes the CPU's fp64 term in 64-bit integers
// and adds in the CPU's order", Context and Decision):
//     w*(2*mxy + c1)*(c2 + 2*(xy*w - mxy))
//       / ((mx2 + my2 + c1)*(x2*w - mx2 + y2*w - my2 + c2))
// with x, y, x2, y2, xy the int64 sums of the edge-truncated window, w its
// pixel count, mx2 = x*x, my2 = y*y, mxy = x*y in fp64.  The expression is
// evaluated left to right, one rounding per operation: this file is built
// with -ffp-contract=off, so no multiply is fused into an add, and the fp64
// divide is the compiler's correctly rounded sequence.
//
// For 8-bit planes every moment is below 49 * 255^2 < 2^22, so the window
// sums are formed exactly in 32-bit integers; every product of two moments
// is below 2^53 and converts to fp64 without rounding (ADR-1443 Decision,
// "three shortcuts, each exact", second item).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "exseq.h"
#include "exseq_internal.h"
#include "exseq_rules.h"

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

// One thread per pixel; the window is summed directly (the planes stay in
// L2/MALL between neighbouring pixels).
__global__ __launch_bounds__(256) void ssim_terms_kernel(
    const uint8_t *__restrict__ ref, const uint8_t *__restrict__ dis, int width, int height,
    ptrdiff_t stride, int radius, double c1, double c2, double *__restrict__ terms)
{
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    const int i = blockIdx.y;
    if (j >= width)
        return;
    const int a0 = i - radius < 0 ? 0 : i - radius;
    const int a1 = i + radius >= height ? height - 1 : i + radius;
    const int b0 = j - radius < 0 ? 0 : j - radius;
    const int b1 = j + radius >= width ? width - 1 : j + radius;
    int32_t sx = 0, sy = 0, sxx = 0, syy = 0, sxy = 0;
    for (int a = a0; a <= a1; a++) {
        const uint8_t *pr = ref + (ptrdiff_t)a * stride;
        const uint8_t *pd = dis + (ptrdiff_t)a * stride;
        for (int b = b0; b <= b1; b++) {
            int32_t p = pr[b], q = pd[b];
            sx += p;
            sy += q;
            sxx += p * p;
            syy += q * q;
            sxy += p * q;
        }
    }
    const int64_t w = (int64_t)(a1 - a0 + 1) * (int64_t)(b1 - b0 + 1);
    terms[(size_t)i * (size_t)width + (size_t)j] = ssim_term_dev(sx, sy, sxx, syy, sxy, w, c1, c2);
}

__global__ void write_i64_kernel(int64_t *out, int64_t v) { out[0] = v; }

static int64_t line_sum(int len, int radius)
{
    int64_t s = 0;
    for (int j = 0; j < len; j++) {
        int lo = j - radius < 0 ? 0 : j - radius;
        int hi = j + radius >= len ? len - 1 : j + radius;
        s += hi - lo + 1;
    }
    return s;
}

SsimLayout ssim_layout(int width, int height)
{
    SsimLayout L;
    const size_t n = (size_t)width * (size_t)height;
    L.plane_off = 0;
    L.sum_off = (n * sizeof(double) + 255) & ~(size_t)255;
    L.total = L.sum_off + sum_ws_bytes(padded_chunks(n));
    return L;
}

int launch_ssim_sum(const uint8_t *ref, const uint8_t *dis, int width, int height,
                    ptrdiff_t stride, int radius, double c1, double c2, double *out_sum,
                    int64_t *out_weight_sum, double *out_terms, void *ws, hipStream_t stream,
                    uint32_t flags, exseq_stats *stats)
{
    SsimLayout L = ssim_layout(width, height);
    char *w = static_cast<char *>(ws);
    double *plane = out_terms ? out_terms : reinterpret_cast<double *>(w + L.plane_off);
    dim3 grid((unsigned)((width + 255) / 256), (unsigned)height);
    hipLaunchKernelGGL(ssim_terms_kernel, grid, dim3(256), 0, stream, ref, dis, width, height,
                       stride, radius, c1, c2, plane);
    if (hipGetLastError() != hipSuccess)
        return EXSEQ_EHIP;
    if (out_weight_sum) {
        const int64_t wsum = line_sum(height, radius) * line_sum(width, radius);
        hipLaunchKernelGGL(write_i64_kernel, dim3(1), dim3(1), 0, stream, out_weight_sum, wsum);
    }
    const size_t n = (size_t)width * (size_t)height;
    return launch_exact_sum(plane, n, 0.0, out_sum, w + L.sum_off, stream, flags, stats);
}

}  // namespace exseq
