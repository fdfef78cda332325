// Internal layout shared by the library's translation units (not part of the
// C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "exseq.h"

namespace exseq {

constexpr int kChunk = EXSEQ_CHUNK_TERMS;  // terms per chunk
constexpr int kChunkThreads = 256;         // 4 waves x 64 lanes x 4 terms
constexpr int kPlanThreads = 1024;
constexpr int kWalkThreads = 256;

static_assert(kChunk == kChunkThreads * 4, "a lane holds 4 consecutive terms");

// One chunk's descriptor (32 bytes): the increment for an even start count
// (the odd one differs by -1, 0 or +1, kept in meta), the prefix bounds, and
// meta = plan key | (r1 - r0 + 1) << 12 | flags.
struct alignas(16) DescRec {
    int64_t r0;
    int64_t lo;
    int64_t hi;
    uint32_t meta;
    uint32_t aux;
};
static_assert(sizeof(DescRec) == 32, "descriptor is 32 bytes");

struct SumLayout {
    size_t nch;
    size_t tsum_off, key_off, desc_off;
    size_t total;
};

SumLayout sum_layout(size_t n);
int launch_exact_sum(const double *x, size_t n, double init, double *out, void *ws,
                     hipStream_t stream, uint32_t flags, exseq_stats *stats,
                     void *const *events = nullptr, int n_events = 0);
extern const char *const kPathKernels[];
extern const int kPathKernelCount;
int launch_tree_sum(const double *x, size_t n, double *out, void *ws, hipStream_t stream);

struct SsimLayout {
    size_t plane_off, sum_off, total;
};
SsimLayout ssim_layout(int width, int height);
int launch_ssim_sum(const uint8_t *ref, const uint8_t *dis, int width, int height,
                    ptrdiff_t stride, int radius, double c1, double c2, double *out_sum,
                    int64_t *out_weight_sum, double *out_terms, void *ws, hipStream_t stream,
                    uint32_t flags, exseq_stats *stats);

}  // namespace exseq
