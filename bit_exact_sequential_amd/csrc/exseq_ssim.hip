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
#include "exseq_dev.h"

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

// The producer for any frame: every pixel's term in raster order into
// `terms`, one workgroup per chunk of 1024 pixels (the column sums, windows
// and term of the tiles' own source), and the frame's weight sum.
__global__ __launch_bounds__(256) void ssim_terms_kernel(SsimParams sp, double *terms, ChainArea ch,
                                                         uint32_t tiles)
{
    zero_chain_words(ch, tiles);
    __shared__ __attribute__((aligned(16))) int lds[SsimTerms::kLdsInts];
    const SsimTerms src{sp};
    const size_t c = blockIdx.x;
    const Four f = src.chunk_at(c, lds);
    const size_t first = c * 1024 + 4 * (size_t)threadIdx.x;
#pragma unroll
    for (int u = 0; u < 4; u++)
        if (u < f.cnt)
            terms[first + u] = f.v[u];
    if (c == 0 && threadIdx.x == 0 && sp.out_weight_sum)
        *sp.out_weight_sum = sp.weight_sum;
}

// The producer for planes whose rows are a multiple of four pixels,
// 4-byte aligned and under 2 GiB, and windows of radius 4 at most (every
// frame of the usual shapes).  Each wave works alone (no LDS, no barrier):
// it takes kRowBlock rows of a strip of kWaveCols columns, lane l keeping the
// column sums (x, y, x^2, y^2, xy over the window's rows) of four columns,
// the strip's first column minus 4 plus 4l, and sliding them down the rows:
// the row entering the window added, the row leaving it taken out (exact
// integers, any order; all the rows' words are requested at once).  A pixel's
// window adds the column sums of its row's window columns: its own lane's and,
// across the lane edges, its neighbours' (whole-wave DPP shifts by one lane),
// so lanes 1 .. 62 give terms and lanes 0 and 63 hold the columns on either
// side.  Columns outside the frame read as zero, so a window cut by the
// frame's left or right edge adds up the right columns, and its pixel count
// says how many.
constexpr int kRowBlock = 4;
constexpr int kWaveCols = 4 * 62;
constexpr int kDppWaveShl1 = 0x130;  // lane l takes lane l + 1's value (lane 63: 0)

__device__ __forceinline__ uint32_t plane_word(const __amdgpu_buffer_rsrc_t &rs, int vo, int so)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, vo, so, 0);
}

// The window sums of a lane's four pixels from one plane's column sums: its
// own four columns c[0..3] and its neighbours' (R of each side needed).
template <int R>
__device__ __forceinline__ void lane_windows(const int c[4], int s[4])
{
    int v[12];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        v[e] = __builtin_amdgcn_update_dpp(0, c[e], kDppWaveShr1, 0xf, 0xf, false);
        v[4 + e] = c[e];
        v[8 + e] = __builtin_amdgcn_update_dpp(0, c[e], kDppWaveShl1, 0xf, 0xf, false);
    }
    int acc = v[4];
#pragma unroll
    for (int d = 1; d <= R; d++)
        acc += v[4 - d] + v[4 + d];
    s[0] = acc;
#pragma unroll
    for (int u = 1; u < 4; u++) {
        acc += v[4 + u + R] - v[4 + u - 1 - R];
        s[u] = acc;
    }
}

template <int R>
__device__ __forceinline__ void wave_strip(const SsimParams &sp, double *terms)
{
    constexpr int kRows = kRowBlock + 2 * R;  // the rows the block's windows span
    const int lane = (int)(threadIdx.x & 63u);
    const int w = sp.width, h = sp.height;
    const int j0 = ((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * kWaveCols;  // first output column
    if (j0 >= w)
        return;  // the whole wave: nothing of the frame in its strip
    const int i0 = (int)blockIdx.y * kRowBlock;
    const int col = j0 - 4 + 4 * lane;  // this lane's first column
    const int stride = (int)sp.stride;
    const int bytes = stride * h;
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(sp.ref), (short)0, bytes, SsimTerms::kBufWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(sp.dis), (short)0, bytes, SsimTerms::kBufWord3);
    const int vo = col >= 0 && col < w ? col : SsimTerms::kBufPastEnd;
    // every row word the block needs, requested at once (rows and columns
    // outside the frame read as zero)
    uint32_t wx[kRows], wy[kRows];
#pragma unroll
    for (int k = 0; k < kRows; k++) {
        const int row = i0 - R + k;
        const bool in = row >= 0 && row < h;
        const int so = in ? row * stride : 0;
        wx[k] = plane_word(rr, in ? vo : SsimTerms::kBufPastEnd, so);
        wy[k] = plane_word(rd, in ? vo : SsimTerms::kBufPastEnd, so);
    }
    int cs[5][4];
#pragma unroll
    for (int e = 0; e < 4; e++)
        cs[0][e] = cs[1][e] = cs[2][e] = cs[3][e] = cs[4][e] = 0;
#pragma unroll
    for (int k = 0; k <= 2 * R; k++) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int x = (int)((wx[k] >> (8 * e)) & 0xFFu), y = (int)((wy[k] >> (8 * e)) & 0xFFu);
            cs[0][e] += x;
            cs[1][e] += y;
            cs[2][e] += x * x;
            cs[3][e] += y * y;
            cs[4][e] += x * y;
        }
    }
    const double c1 = sp.c1, c2 = sp.c2;
    const bool out = lane >= 1 && lane <= 62 && col < w;
#pragma unroll
    for (int q = 0; q < kRowBlock; q++) {
        const int i = i0 + q;
        if (i >= h)
            break;
        if (q > 0) {
            // slide: row i + R enters, row i - R - 1 leaves
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int x = (int)((wx[q + 2 * R] >> (8 * e)) & 0xFFu);
                const int y = (int)((wy[q + 2 * R] >> (8 * e)) & 0xFFu);
                const int u = (int)((wx[q - 1] >> (8 * e)) & 0xFFu);
                const int z = (int)((wy[q - 1] >> (8 * e)) & 0xFFu);
                cs[0][e] += x - u;
                cs[1][e] += y - z;
                cs[2][e] += x * x - u * u;
                cs[3][e] += y * y - z * z;
                cs[4][e] += x * y - u * z;
            }
        }
        // the windows (every lane takes part in the shifts)
        int s[5][4];
#pragma unroll
        for (int m = 0; m < 5; m++)
            lane_windows<R>(cs[m], s[m]);
        if (out) {
            const int ra0 = i - R < 0 ? 0 : i - R;
            const int ra1 = i + R >= h ? h - 1 : i + R;
            const int rows = ra1 - ra0 + 1;
            double v[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int j = col + e;
                const int b0 = j - R < 0 ? 0 : j - R;
                const int b1 = j + R >= w ? w - 1 : j + R;
                v[e] = ssim_term_dev(s[0][e], s[1][e], s[2][e], s[3][e], s[4][e],
                                     (int64_t)(rows * (b1 - b0 + 1)), c1, c2);
            }
            double *o = terms + (size_t)i * (size_t)w + (size_t)col;
#pragma unroll
            for (int e = 0; e < 4; e++)
                o[e] = v[e];
        }
    }
}

__global__ __launch_bounds__(256) void ssim_terms_rows_kernel(SsimParams sp, double *terms, ChainArea ch,
                                                              uint32_t tiles)
{
    zero_chain_words(ch, tiles);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && sp.out_weight_sum)
        *sp.out_weight_sum = sp.weight_sum;
    switch (sp.radius) {
    case 0: wave_strip<0>(sp, terms); break;
    case 1: wave_strip<1>(sp, terms); break;
    case 2: wave_strip<2>(sp, terms); break;
    case 3: wave_strip<3>(sp, terms); break;
    default: wave_strip<4>(sp, terms); break;
    }
}

static bool rows_producer_ok(const SsimParams &sp)
{
    return sp.radius <= 4 && (sp.width & 3) == 0 && (sp.stride & 3) == 0 &&
           (((uintptr_t)sp.ref | (uintptr_t)sp.dis) & 3u) == 0 &&
           (uint64_t)sp.stride * (uint64_t)sp.height <= (uint64_t)0x7FFFFFFF;
}

// The workspace: the exact sum's, then (without a caller's plane and without
// EXSEQ_SSIM_IN_TILES) the terms, 256-byte aligned.
static size_t ssim_sum_ws(size_t n) { return (sum_ws_bytes(padded_chunks(n)) + 255) & ~(size_t)255; }

size_t ssim_ws_bytes(int width, int height)
{
    const size_t n = (size_t)width * (size_t)height;
    return ssim_sum_ws(n) + n * sizeof(double);
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
    if (flags & EXSEQ_SSIM_IN_TILES)
        return launch_ssim_exact(sp, out_sum, ws, stream, flags & ~EXSEQ_SSIM_IN_TILES, stats);
    // the terms into the caller's plane or the workspace, then the exact sum
    // over them
    const size_t n = (size_t)width * (size_t)height;
    double *terms = out_terms ? out_terms
                              : reinterpret_cast<double *>(static_cast<char *>(ws) + ssim_sum_ws(n));
    sp.out_terms = nullptr;
    // the producer also zeroes the exact sum's chain words, one launch fewer
    ChainArea ch{};
    uint32_t tiles = 0;
    const bool fold = chain_words_of(n, flags, ws, &ch, &tiles);
    if (!fold)
        tiles = 0;
    if (rows_producer_ok(sp))
        hipLaunchKernelGGL(ssim_terms_rows_kernel,
                           dim3((unsigned)((width + 4 * kWaveCols - 1) / (4 * kWaveCols)),
                                (unsigned)((height + kRowBlock - 1) / kRowBlock)),
                           dim3(256), 0, stream, sp, terms, ch, tiles);
    else
        hipLaunchKernelGGL(ssim_terms_kernel, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, stream,
                           sp, terms, ch, tiles);
    if (hipGetLastError() != hipSuccess)
        return EXSEQ_EHIP;
    if (fold)
        return launch_exact_sum_cleared(terms, n, 0.0, out_sum, ws, stream, flags, stats);
    return launch_exact_sum(terms, n, 0.0, out_sum, ws, stream, flags, stats, nullptr, 0);
}

}  // namespace exseq
