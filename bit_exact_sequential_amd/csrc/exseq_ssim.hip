// Host side of the fused integer-SSIM frame sum: the weight sum of the
// frame (a product of two line sums) and the launch of the exact sum over the
// fused term source, whose tiles form every pixel's term from the two planes
// as they need it (exseq_ssim_dev.h); the terms are never stored unless the
// caller asks for them.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "exseq.h"
#include "exseq_internal.h"
#include "exseq_rules.h"
#include "exseq_ssim_dev.h"

namespace exseq {


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

__global__ void div_kernel(const double *a, const double *b, double *q, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        q[i] = ssim_div(a[i], b[i]);
}

int launch_div(const double *a, const double *b, double *q, size_t n, hipStream_t stream)
{
    if (n == 0)
        return EXSEQ_OK;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(div_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, b, q, n);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
}

size_t ssim_ws_bytes(int width, int height)
{
    return sum_ws_bytes(padded_chunks((size_t)width * (size_t)height));
}

int launch_ssim_sum(const uint8_t *ref, const uint8_t *dis, int width, int height,
                    ptrdiff_t stride, int radius, double c1, double c2, double *out_sum,
                    int64_t *out_weight_sum, double *out_terms, void *ws, hipStream_t stream,
                    uint32_t flags, exseq_stats *stats)
{
    SsimParams sp;
    // the frame's weight sum, a product of line sums, written by the walk
    sp.out_weight_sum = out_weight_sum;
    sp.weight_sum = line_sum(height, radius) * line_sum(width, radius);
    sp.ref = ref;
    sp.dis = dis;
    sp.width = width;
    sp.height = height;
    sp.stride = stride;
    sp.radius = radius;
    sp.c1 = c1;
    sp.c2 = c2;
    sp.out_terms = out_terms;
    return launch_ssim_exact(sp, out_sum, ws, stream, flags, stats);
}

}  // namespace exseq
