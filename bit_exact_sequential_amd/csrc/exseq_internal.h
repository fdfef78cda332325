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
constexpr int kWalkThreads = 256;          // one walk workgroup: 4 waves x 4 items
constexpr int kMaxBatch = 64;              // sums per launch (kernel arguments)
constexpr int kPassMax = 128;              // sums per launch of the single pass

static_assert(kChunk == kChunkThreads * 4, "a lane holds 4 consecutive terms");

// Chunks per workgroup of the chunk pass (a tile); each sum's chunk range is
// padded to a multiple of the largest tile.  Bits 4..5 of `flags` choose the
// tile (0 = default 4, 1, 2 or 3 = 4 chunks), a tuning knob.
constexpr int kTileMax = 4;
constexpr uint32_t kTileShift = 4;

inline size_t padded_chunks(size_t n)
{
    const size_t c = (n + kChunk - 1) / kChunk;
    return (c + kTileMax - 1) / kTileMax * kTileMax;
}

// A lane's four consecutive terms of a chunk (cnt of them exist).
struct Four {
    double v[4];
    int cnt;
};

// The fused integer-SSIM term source: two 8-bit planes, the window radius
// and the stabilisers; out_terms (nullable) receives every term.
struct SsimParams {
    const uint8_t *ref;
    const uint8_t *dis;
    int width, height;
    ptrdiff_t stride;
    int radius;
    double c1, c2;
    double *out_terms;
    int64_t *out_weight_sum;  // nullable: written with the sum
    int64_t weight_sum;
};

// Up to kMaxBatch independent sums, passed to the kernels by value.  Sum k
// owns the global chunks [chunk_base[k], chunk_base[k + 1]) (its chunks,
// padded to a multiple of kTileMax).
struct BatchArgs {
    int count;
    uint32_t flags;
    uint32_t epoch;  // tags this launch's look-back status words
    uint32_t tile;   // chunks per tile (1, 2 or 4)
    const double *x[kMaxBatch];
    uint64_t n[kMaxBatch];
    double init[kMaxBatch];
    uint32_t chunk_base[kMaxBatch + 1];
    // Dispatch order of the tiles with the exact chain: each sum's last tile
    // first (last_tile: its index in the launch, ~0u for an empty sum), then
    // the others in order (rest_base: prefix count of them per sum).
    uint32_t last_tile[kMaxBatch];
    uint32_t rest_base[kMaxBatch + 1];
    // With EXSEQ_PLAN_REUSE: the tag of this launch's shape, which the plan
    // left in the workspace by an earlier launch must carry to be used (0:
    // no reuse, and no plan is written).
    uint64_t plan_sig;
    // Sums of one length over interleaved terms (sum s reads every k-th
    // double from x[s]): the tiles of all sums for one range of terms are
    // dispatched together, on one XCD, so that they share cache lines.
    uint32_t interleave;
    // Nullable: means[s] = (float)(sum / n[s]) is written with the sum.
    float *means;
    // A launch of at most a few chunks: the walk alone adds them in order.
    uint32_t tiny;
    // Nullable: where this launch keeps its plan (EXSEQ_PLAN_REUSE) when it is
    // one group of a larger batch: per sum a tag, per tile of kTileMax chunks
    // a prefix, at places of the batch's own that do not depend on the
    // group's size (else they follow the launch's other arrays).
    uint64_t *plan_hdr_ext;
    double *plan_ext;
    // Nonzero: a launch before this one on the stream zeroed the chain words
    // (the SSIM term producer), so the launch sequence skips its clear.
    uint32_t chain_cleared;
};

// Descriptors live in four arrays (structure of arrays, so that the walk
// reads what it needs with coalesced loads): r0, lo, hi (int64) and meta =
// key | (r1 - r0 + 1) << 12 | flags.  For a chunk with kFlagExact, lo holds
// the bits of the exact running sum after it instead.
struct DescArrays {
    int64_t *r0;
    int64_t *lo;
    int64_t *hi;
    uint32_t *meta;
};

// The exact chain between the tiles of a sum (zeroed before every launch;
// a published word is never zero).  Per tile: four words describing it (agg:
// meta, r0, lo, hi of the composition of its chunks, or "irregular") and the
// exact running sum after it (incl, irregular tiles only); per sum, the exact
// sum after its first chunk (head).
struct ChainArea {
    uint64_t *agg;
    uint64_t *incl;
    uint64_t *head;  // per sum: the exact sum after its first chunk
    // The plan kept for the next launch (EXSEQ_PLAN_REUSE): per sum the tag
    // of the launch that wrote it, and the planned prefix before every tile
    // of kTileMax chunks (index: the tile's first chunk in the launch / kTileMax).
    uint64_t *plan_hdr;
    double *plan;
    // Per tile: the irregular tile's O(1) step from the exact sum before it
    // (16 words, each nonzero once written), for the tiles after it.
    uint64_t *rec;
};

// Workspace of a launch over `total_chunks` chunks: plan status words, the
// descriptor arrays, the chain words.
size_t sum_ws_bytes(size_t total_chunks);
int launch_batch(const BatchArgs &a, void *ws, double *outs, hipStream_t stream,
                 exseq_stats *stats, void *const *events = nullptr, int n_events = 0);
int launch_interleaved(const double *x, size_t windows, int k, const double *inits, double *outs,
                       float *means, void *ws, hipStream_t stream, uint32_t flags,
                       exseq_stats *stats);
int launch_exact_sum(const double *x, size_t n, double init, double *out, void *ws,
                     hipStream_t stream, uint32_t flags, exseq_stats *stats,
                     void *const *events = nullptr, int n_events = 0);
// The chain words a launch of launch_exact_sum(n, flags) on workspace ws
// zeroes before its tiles: false if it takes no tile chain (a few chunks, the
// single pass, a mode without the chain).  A launch earlier on the same
// stream may zero them instead (zero_chain_words), and launch_exact_sum with
// chain_cleared then skips its clear.
bool chain_words_of(size_t n, uint32_t flags, void *ws, ChainArea *ch, uint32_t *tiles);
int launch_exact_sum_cleared(const double *x, size_t n, double init, double *out, void *ws,
                             hipStream_t stream, uint32_t flags, exseq_stats *stats);
// The single pass (exseq_pass.hip): whether a launch can take it, its
// workspace, and its launch (one kernel; events[0] and events[1] around it).
bool pass_flags_ok(uint32_t flags);
bool pass_eligible(const BatchArgs &a);
size_t pass_blocks(const size_t *ns, size_t count);
size_t pass_blocks_bound(size_t total_chunks, size_t sums);
size_t pass_ws_bytes(size_t blocks, size_t sums);
int launch_pass(const double *const *xs, const size_t *ns, const double *inits, int count,
                uint32_t flags, void *ws, double *outs, hipStream_t stream, exseq_stats *stats,
                void *const *events, int n_events);
size_t pass_inter_blocks(size_t windows, int k);
bool pass_inter_ok(size_t windows, int k, uint32_t flags);
int launch_pass_interleaved(const double *x, size_t windows, int k, const double *inits, double *outs,
                            float *means, void *ws, hipStream_t stream, uint32_t flags, exseq_stats *stats);
extern const char *const kPathKernels[];
extern const int kPathKernelCount;
int launch_tree_sum(const double *x, size_t n, double *out, void *ws, hipStream_t stream);
int launch_stream_read(const double *x, size_t n, uint64_t *out, hipStream_t stream);

// Workspace of the fused SSIM sum: the exact sum's, over width * height terms.
size_t ssim_ws_bytes(int width, int height);
int launch_div(const double *a, const double *b, double *q, size_t n, hipStream_t stream);
int launch_ssim_sum(const uint8_t *ref, const uint8_t *dis, int width, int height,
                    ptrdiff_t stride, int radius, double c1, double c2, double *out_sum,
                    int64_t *out_weight_sum, double *out_terms, void *ws, hipStream_t stream,
                    uint32_t flags, exseq_stats *stats);
// The exact sum of the fused term source (exseq_sum.hip).
int launch_ssim_exact(const SsimParams &sp, double *out, void *ws, hipStream_t stream,
                      uint32_t flags, exseq_stats *stats);

}  // namespace exseq
