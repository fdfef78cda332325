// The C ABI of libexseq.so: argument checks, workspace carving, launches.
// Declarations and their contracts are in include/exseq.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "exseq.h"
#include "exseq_internal.h"

using namespace exseq;

namespace {

bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0u; }

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

// The workspace of exact_seq_sum_f64_noalloc: a static device array, one copy
// per GPU.  Host code never uses the name `scratch` as an address (on the
// host it only names the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[EXSEQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's array, or null (the runtime failed).
void *scratch_for_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q)
            return nullptr;
        p = q;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

const char *exseq_version(void) { return "exseq 0.1 (gfx950)"; }

const char *exseq_strerror(int code)
{
    switch (code) {
    case EXSEQ_OK:
        return "ok";
    case EXSEQ_EINVAL:
        return "invalid argument (null pointer, misalignment or bad size)";
    case EXSEQ_EWORKSPACE:
        return "workspace too small";
    case EXSEQ_EHIP:
        return "HIP runtime error at launch";
    case EXSEQ_ESCRATCH:
        return "input too large for the static scratch array (exact_seq_sum_f64_noalloc)";
    default:
        return "unknown exseq error";
    }
}

size_t chunks_of(size_t n) { return (n + kChunk - 1) / kChunk; }

size_t exact_seq_sum_f64_workspace_size(size_t n) { return sum_ws_bytes(padded_chunks(n)); }

int exact_seq_sum_f64(const double *x, size_t n, double init, double *out, void *ws,
                      size_t ws_bytes, exseq_stream_t stream, uint32_t flags,
                      exseq_stats *stats)
{
    if (!out || !aligned8(out) || (n && (!x || !aligned8(x))))
        return EXSEQ_EINVAL;
    if (n && !ws)
        return EXSEQ_EINVAL;
    if (n && ws_bytes < exact_seq_sum_f64_workspace_size(n))
        return EXSEQ_EWORKSPACE;
    if (chunks_of(n) > 0xFFFFFFFFull)
        return EXSEQ_EINVAL;
    return launch_exact_sum(x, n, init, out, ws, reinterpret_cast<hipStream_t>(stream), flags,
                            stats);
}

size_t exact_seq_sum_f64_noalloc_max_terms(void)
{
    // the workspace grows with n: the largest n whose workspace fits
    size_t lo = 0, hi = (size_t)1 << 40;
    while (lo < hi) {
        const size_t mid = lo + (hi - lo + 1) / 2;
        if (exact_seq_sum_f64_workspace_size(mid) <= EXSEQ_NOALLOC_SCRATCH_BYTES)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

int exact_seq_sum_f64_noalloc(const double *x, size_t n, double init, double *out,
                              exseq_stream_t stream, uint32_t flags, exseq_stats *stats)
{
    if (!out || !aligned8(out) || (n && (!x || !aligned8(x))))
        return EXSEQ_EINVAL;
    if (chunks_of(n) > 0xFFFFFFFFull)
        return EXSEQ_EINVAL;
    if (exact_seq_sum_f64_workspace_size(n) > EXSEQ_NOALLOC_SCRATCH_BYTES)
        return EXSEQ_ESCRATCH;
    void *ws = scratch_for_current_device();
    if (!ws)
        return EXSEQ_EHIP;
    return launch_exact_sum(x, n, init, out, ws, reinterpret_cast<hipStream_t>(stream), flags,
                            stats);
}

int exseq_profile_kernel_count(void) { return kPathKernelCount; }

const char *exseq_profile_kernel_name(int i)
{
    return (i >= 0 && i < kPathKernelCount) ? kPathKernels[i] : "";
}

int exact_seq_sum_f64_profiled(const double *x, size_t n, double init, double *out, void *ws,
                               size_t ws_bytes, exseq_stream_t stream, uint32_t flags,
                               exseq_stats *stats, void *const *events, int n_events)
{
    if (!out || !aligned8(out) || (n && (!x || !aligned8(x))) || n == 0)
        return EXSEQ_EINVAL;
    if (!ws || ws_bytes < exact_seq_sum_f64_workspace_size(n))
        return ws ? EXSEQ_EWORKSPACE : EXSEQ_EINVAL;
    if (n_events < 0 || (n_events && !events))
        return EXSEQ_EINVAL;
    return launch_exact_sum(x, n, init, out, ws, reinterpret_cast<hipStream_t>(stream), flags,
                            stats, events, n_events);
}

// Sums go to the kernels in groups: up to kPassMax sums in one launch of
// the single pass (the default for several sums), else groups of kMaxBatch
// through the tile chain.  The groups run one after the other on the stream
// and reuse one workspace region, sized for either grouping.
namespace {

bool batch_takes_pass(size_t count, uint32_t flags)
{
    return exseq::pass_flags_ok(flags) && (count > 1 || (flags & EXSEQ_PASS_PATH));
}

// A group of sums of at most a few chunks, with default flags: the walk
// alone adds them in order (one launch).
bool group_is_tiny(const size_t *ns, size_t count, uint32_t flags)
{
    size_t chunks = 0;
    for (size_t k = 0; k < count; k++)
        chunks += padded_chunks(ns[k]);
    return chunks <= 2u * kTileMax && (flags & ~EXSEQ_PASS_PATH) == 0u;
}

// A batch of more than kMaxBatch sums through the tile chain: the groups'
// kept plans (EXSEQ_PLAN_REUSE) at the start of the workspace, each group at
// a place of its own that does not depend on the group's size, and the
// groups' working arrays after them.
size_t batch_plan_bytes(const size_t *ns, size_t count)
{
    if (count <= (size_t)kMaxBatch)
        return 0;
    size_t tiles = 0;
    for (size_t g = 0; g < count; g += kMaxBatch) {
        size_t chunks = 0;
        for (size_t k = g; k < count && k < g + kMaxBatch; k++)
            chunks += padded_chunks(ns[k]);
        tiles += chunks / kTileMax + 1;
    }
    return round256(count * sizeof(uint64_t)) + round256(tiles * sizeof(double));
}

int batch_chain(const double *const *xs, const size_t *ns, const double *inits, size_t count,
                double *outs, void *ws, hipStream_t stream, uint32_t flags, exseq_stats *stats)
{
    const size_t plan_bytes = batch_plan_bytes(ns, count);
    char *work = static_cast<char *>(ws) + plan_bytes;
    size_t tile_off = 0;
    for (size_t g = 0; g < count; g += kMaxBatch) {
        BatchArgs a{};
        a.count = (int)(count - g < (size_t)kMaxBatch ? count - g : (size_t)kMaxBatch);
        a.flags = flags;
        uint64_t chunks = 0;
        for (int k = 0; k < a.count; k++) {
            a.x[k] = xs[g + k];
            a.n[k] = ns[g + k];
            a.init[k] = inits ? inits[g + k] : 0.0;
            a.chunk_base[k] = (uint32_t)chunks;
            chunks += padded_chunks(ns[g + k]);
        }
        if (chunks > 0xFFFFFFFFull)
            return EXSEQ_EINVAL;
        a.chunk_base[a.count] = (uint32_t)chunks;
        if (plan_bytes) {
            a.plan_hdr_ext = static_cast<uint64_t *>(ws) + g;
            a.plan_ext = reinterpret_cast<double *>(static_cast<char *>(ws) + round256(count * sizeof(uint64_t))) +
                         tile_off;
            tile_off += chunks / kTileMax + 1;
        }
        const int rc = launch_batch(a, plan_bytes ? work : ws, outs + g, stream, stats ? stats + g : nullptr);
        if (rc != EXSEQ_OK)
            return rc;
    }
    return EXSEQ_OK;
}

}  // namespace

size_t exact_seq_sum_f64_batch_workspace_size(const size_t *ns, size_t count)
{
    size_t mx = 0;
    for (size_t g = 0; ns && g < count; g += kMaxBatch) {
        size_t chunks = 0;
        for (size_t k = g; k < count && k < g + kMaxBatch; k++)
            chunks += padded_chunks(ns[k]);
        mx = chunks > mx ? chunks : mx;
    }
    size_t bytes = (ns ? batch_plan_bytes(ns, count) : 0) + sum_ws_bytes(mx);
    for (size_t g = 0; ns && g < count; g += kPassMax) {
        const size_t m = count - g < (size_t)kPassMax ? count - g : (size_t)kPassMax;
        const size_t pb = exseq::pass_ws_bytes(exseq::pass_blocks(ns + g, m), m);
        bytes = pb > bytes ? pb : bytes;
    }
    return round256(bytes);
}

int exact_seq_sum_f64_batch(const double *const *xs, const size_t *ns, const double *inits,
                            size_t count, double *outs, void *ws, size_t ws_bytes,
                            exseq_stream_t stream, uint32_t flags, exseq_stats *stats)
{
    if (count == 0)
        return EXSEQ_OK;
    if (!xs || !ns || !outs || !aligned8(outs))
        return EXSEQ_EINVAL;
    for (size_t k = 0; k < count; k++) {
        if (ns[k] && (!xs[k] || !aligned8(xs[k])))
            return EXSEQ_EINVAL;
        if (chunks_of(ns[k]) > 0xFFFFFFFFull)
            return EXSEQ_EINVAL;
    }
    if (!ws || ws_bytes < exact_seq_sum_f64_batch_workspace_size(ns, count))
        return ws ? EXSEQ_EWORKSPACE : EXSEQ_EINVAL;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (!batch_takes_pass(count, flags))
        return batch_chain(xs, ns, inits, count, outs, ws, st, flags, stats);
    for (size_t g = 0; g < count; g += kPassMax) {
        const size_t m = count - g < (size_t)kPassMax ? count - g : (size_t)kPassMax;
        size_t chunks = 0;
        for (size_t k = g; k < g + m; k++)
            chunks += padded_chunks(ns[k]);
        if (exseq::pass_blocks(ns + g, m) > 0xFFFFFFFFull / 8u)  // chunk indices: 8 per workgroup
            return EXSEQ_EINVAL;
        const int rc = chunks == 0 || group_is_tiny(ns + g, m, flags)
                           ? batch_chain(xs + g, ns + g, inits ? inits + g : nullptr, m, outs + g, ws, st,
                                         flags, stats ? stats + g : nullptr)
                           : exseq::launch_pass(xs + g, ns + g, inits ? inits + g : nullptr, (int)m, flags,
                                                ws, outs + g, st, stats ? stats + g : nullptr, nullptr, 0);
        if (rc != EXSEQ_OK)
            return rc;
    }
    return EXSEQ_OK;
}

size_t exact_seq_sum_f64_interleaved_workspace_size(size_t windows, int k)
{
    if (k < 1 || k > EXSEQ_INTERLEAVE_MAX)
        return 256;
    const size_t chain = sum_ws_bytes((size_t)k * padded_chunks(windows));
    const size_t pass = (k == 2 || k == 4) ? exseq::pass_ws_bytes(exseq::pass_inter_blocks(windows, k), (size_t)k) : 0;
    return round256(chain > pass ? chain : pass);
}

int exact_seq_sum_f64_interleaved(const double *x, size_t windows, int k, const double *inits,
                                  double *outs, float *means, void *ws, size_t ws_bytes,
                                  exseq_stream_t stream, uint32_t flags, exseq_stats *stats)
{
    if (k < 1 || k > EXSEQ_INTERLEAVE_MAX || !outs || !aligned8(outs) ||
        (means && (reinterpret_cast<uintptr_t>(means) & 3u)) ||
        (windows && (!x || !aligned8(x))))
        return EXSEQ_EINVAL;
    if ((uint64_t)k * padded_chunks(windows) > 0xFFFFFFFFull)
        return EXSEQ_EINVAL;
    if (!ws || ws_bytes < exact_seq_sum_f64_interleaved_workspace_size(windows, k))
        return ws ? EXSEQ_EWORKSPACE : EXSEQ_EINVAL;
    return launch_interleaved(x, windows, k, inits, outs, means, ws,
                              reinterpret_cast<hipStream_t>(stream), flags, stats);
}

size_t ssim_term_and_sum_workspace_size(int width, int height)
{
    if (width < 1 || height < 1)
        return 256;
    return ssim_ws_bytes(width, height);
}

int ssim_term_and_sum(const uint8_t *ref, const uint8_t *dis, int width, int height,
                      ptrdiff_t stride, int radius, double c1, double c2, double *out_sum,
                      int64_t *out_weight_sum, double *out_terms, void *ws, size_t ws_bytes,
                      exseq_stream_t stream, uint32_t flags, exseq_stats *stats)
{
    if (!ref || !dis || !out_sum || !aligned8(out_sum) || width < 1 || height < 1 ||
        stride < width || radius < 0 || radius > 15)
        return EXSEQ_EINVAL;
    if ((size_t)width * (size_t)height >= ((size_t)1 << 31))
        return EXSEQ_EINVAL;
    if ((out_weight_sum && !aligned8(out_weight_sum)) || (out_terms && !aligned8(out_terms)))
        return EXSEQ_EINVAL;
    if (!ws)
        return EXSEQ_EINVAL;
    if (ws_bytes < ssim_term_and_sum_workspace_size(width, height))
        return EXSEQ_EWORKSPACE;
    return launch_ssim_sum(ref, dis, width, height, stride, radius, c1, c2, out_sum,
                           out_weight_sum, out_terms, ws, reinterpret_cast<hipStream_t>(stream),
                           flags, stats);
}

int exseq_stream_read_f64(const double *x, size_t n, uint64_t *out, exseq_stream_t stream)
{
    if (!out || !aligned8(out) || (n && (!x || (reinterpret_cast<uintptr_t>(x) & 15u))))
        return EXSEQ_EINVAL;
    return launch_stream_read(x, n, out, reinterpret_cast<hipStream_t>(stream));
}

int exseq_div_f64(const double *a, const double *b, double *q, size_t n, exseq_stream_t stream)
{
    if (n && (!a || !b || !q || !aligned8(a) || !aligned8(b) || !aligned8(q)))
        return EXSEQ_EINVAL;
    if ((n + 255) / 256 > 0x7FFFFFFFull)
        return EXSEQ_EINVAL;
    return launch_div(a, b, q, n, reinterpret_cast<hipStream_t>(stream));
}

size_t tree_sum_f64_workspace_size(size_t n) { return round256(chunks_of(n) * sizeof(double)) + 256; }

int tree_sum_f64(const double *x, size_t n, double *out, void *ws, size_t ws_bytes,
                 exseq_stream_t stream)
{
    if (!out || !aligned8(out) || (n && (!x || !aligned8(x))))
        return EXSEQ_EINVAL;
    if (n && (!ws || ws_bytes < tree_sum_f64_workspace_size(n)))
        return ws ? EXSEQ_EWORKSPACE : EXSEQ_EINVAL;
    return launch_tree_sum(x, n, out, ws, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
