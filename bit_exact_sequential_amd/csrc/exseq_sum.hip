// gfx950 kernels of the exact sequential fp64 sum and the fixed-tree sum.
//
// Path (Research-1433 "Forming the CPU's sequential double sums on a GPU,
// bit for bit", Findings 4-6; Research-1424 "integer_ssim_cuda and the CPU's
// frame sum", Findings 3), one chunk = 1024 terms = one workgroup of 256
// lanes (4 waves of 64) with 4 consecutive terms per lane:
//   1. chunk_tsum:   fixed-tree fp64 sum of every chunk (the plan's input).
//   2. plan:         prefix of the chunk sums from init -> each chunk's
//                    planned binade (sign and biased exponent, "key").
//   3. chunk_desc:   every term's increment pair under its chunk's key,
//                    composed in order (lane, then an ordered lane tree, then
//                    the waves in order) into a descriptor: the pair, the
//                    prefix bounds and flags.
//   4. walk:         one workgroup follows the chunks in order with the
//                    exact running sum; a window of 256 descriptors is
//                    scanned at once (composition is associative), every
//                    chunk is checked at its exact start count, and the
//                    first chunk that fails is added term by term.
// Kernels 1-3 stream the terms from HBM; 4 reads descriptors and, for
// fallback chunks only, their terms again.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "exseq.h"
#include "exseq_rules.h"
#include "exseq_internal.h"

using namespace exseq;

namespace exseq {

// ---------------------------------------------------------------------------
// Loads: lane l of a chunk takes terms 4l .. 4l+3; past n a term is absent.
// ---------------------------------------------------------------------------
struct Four {
    double v[4];
    int cnt;  // how many of the four exist (0..4)
};

__device__ __forceinline__ Four load_four(const double *__restrict__ x, size_t n, size_t first)
{
    Four f;
    if (first + 4 <= n) {
        if ((((uintptr_t)(x + first)) & 15u) == 0u) {
            const double2 *p = reinterpret_cast<const double2 *>(x + first);
            double2 a = p[0];
            double2 b = p[1];
            f.v[0] = a.x; f.v[1] = a.y; f.v[2] = b.x; f.v[3] = b.y;
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
                f.v[i] = x[first + i];
        }
        f.cnt = 4;
    } else {
        f.cnt = first < n ? (int)(n - first) : 0;
#pragma unroll
        for (int i = 0; i < 4; i++)
            f.v[i] = (i < f.cnt) ? x[first + i] : 0.0;
    }
    return f;
}

// ---------------------------------------------------------------------------
// Fixed-shape tree sum of a chunk (deterministic: depends on nothing but the
// values and their positions).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double chunk_tree(const Four &f, double *lds4)
{
    double s = (f.v[0] + f.v[1]) + (f.v[2] + f.v[3]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        s += __shfl_down(s, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        lds4[wave] = s;
    __syncthreads();
    double t = (lds4[0] + lds4[1]) + (lds4[2] + lds4[3]);
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(kChunkThreads) void chunk_tsum_kernel(
    const double *__restrict__ x, size_t n, double *__restrict__ tsum)
{
    __shared__ double lds4[4];
    const size_t c = blockIdx.x;
    Four f = load_four(x, n, c * kChunk + (size_t)threadIdx.x * 4);
    double t = chunk_tree(f, lds4);
    if (threadIdx.x == 0)
        tsum[c] = t;
}

// ---------------------------------------------------------------------------
// The plan.  One workgroup per sum: exclusive prefix of the chunk sums,
// starting at init, in any association (it only names binades).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t plan_key(double p, uint32_t flags)
{
    uint32_t mode = flags & EXSEQ_PLAN_MASK;
    if (mode == EXSEQ_PLAN_ALL_FALLBACK)
        return 0u;
    if (mode == EXSEQ_PLAN_FIXED)
        return (flags >> 8) & kKeyMask;
    uint32_t k = key_of(p);
    if (!key_has_fast_path(k))
        return 0u;
    if (mode == EXSEQ_PLAN_PLUS_ONE)
        k += 1u;
    else if (mode == EXSEQ_PLAN_MINUS_ONE)
        k -= 1u;
    return key_has_fast_path(k) ? k : 0u;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const double *__restrict__ tsum, size_t nch, double init, uint32_t flags,
    uint32_t *__restrict__ key)
{
    __shared__ double part[kPlanThreads];
    const int t = threadIdx.x;
    const size_t per = (nch + kPlanThreads - 1) / kPlanThreads;
    const size_t b = (size_t)t * per;
    const size_t e = b + per < nch ? b + per : nch;
    double s = 0.0;
    for (size_t i = b; i < e; i++)
        s += tsum[i];
    part[t] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan of the lane partials.
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        double v = t >= off ? part[t - off] : 0.0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    double p = init + (t > 0 ? part[t - 1] : 0.0);
    for (size_t i = b; i < e; i++) {
        key[i] = plan_key(p, flags);
        p += tsum[i];
    }
}

// ---------------------------------------------------------------------------
// Descriptors.
// ---------------------------------------------------------------------------
__device__ __forceinline__ Run shfl_down_run(const Run &r, int off)
{
    Run o;
    o.p.r0 = __shfl_down(r.p.r0, off, 64);
    o.p.r1 = __shfl_down(r.p.r1, off, 64);
    o.lo = __shfl_down(r.lo, off, 64);
    o.hi = __shfl_down(r.hi, off, 64);
    o.flags = __shfl_down(r.flags, off, 64);
    return o;
}

// Ordered composition of the chunk's 1024 terms under `key`; the result is
// valid in thread 0.
__device__ __forceinline__ Run chunk_run(const Four &f, uint32_t key, Run *lds_runs)
{
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool sgn = (key >> 11) & 1u;
    Run acc = run_identity();
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (i < f.cnt) {
            TermInc ti = term_inc(f.v[i], scale, sgn);
            acc = run_compose(acc, run_of_term(ti, is_nonfinite(f.v[i])));
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // Ordered lane tree: lane i takes lane i + off.
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        Run o = shfl_down_run(acc, off);
        if ((lane & (2 * off - 1)) == 0)
            acc = run_compose(acc, o);
    }
    if (lane == 0)
        lds_runs[wave] = acc;
    __syncthreads();
    Run r = lds_runs[0];
    r = run_compose(r, lds_runs[1]);
    r = run_compose(r, lds_runs[2]);
    r = run_compose(r, lds_runs[3]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ void store_desc(DescRec *d, uint32_t key, const Run &r)
{
    int64_t dr = r.p.r1 - r.p.r0;  // always -1, 0 or +1 (the run's map is monotone)
    DescRec o;
    o.r0 = r.p.r0;
    o.lo = r.lo;
    o.hi = r.hi;
    o.meta = (key & kKeyMask) | ((uint32_t)(dr + 1) << kDrShift) | r.flags;
    o.aux = 0u;
    *d = o;
}

__global__ __launch_bounds__(kChunkThreads) void chunk_desc_kernel(
    const double *__restrict__ x, size_t n, const uint32_t *__restrict__ key,
    DescRec *__restrict__ desc)
{
    __shared__ Run lds_runs[4];
    const size_t c = blockIdx.x;
    const uint32_t k = key[c];
    Four f = load_four(x, n, c * kChunk + (size_t)threadIdx.x * 4);
    Run r;
    if (key_has_fast_path(k)) {
        r = chunk_run(f, k, lds_runs);
    } else {
        // no fast path planned: only the non-finite flag matters
        bool nf = false;
        for (int i = 0; i < f.cnt; i++)
            nf |= is_nonfinite(f.v[i]);
        r = run_identity();
        r.flags = __any(nf) ? kFlagNonFinite : 0u;
        __shared__ uint32_t nfl[4];
        if ((threadIdx.x & 63) == 0)
            nfl[threadIdx.x >> 6] = r.flags;
        __syncthreads();
        r.flags = nfl[0] | nfl[1] | nfl[2] | nfl[3];
    }
    if (threadIdx.x == 0)
        store_desc(desc + c, k, r);
}

// ---------------------------------------------------------------------------
// The walk.
// ---------------------------------------------------------------------------
struct WalkShared {
    int64_t sr0[kWalkThreads], sr1[kWalkThreads];  // scan buffers
    double terms[kChunk];                          // a fallback chunk's terms
    double s;                                      // the exact running sum
    int first;
    int ok2;
    uint32_t misses;
};

__device__ __forceinline__ Pair block_exclusive_scan(Pair v, WalkShared &sh)
{
    const int t = threadIdx.x;
    sh.sr0[t] = v.r0;
    sh.sr1[t] = v.r1;
    __syncthreads();
    Pair incl = v;
    for (int off = 1; off < kWalkThreads; off <<= 1) {
        Pair prev = pair_identity();
        if (t >= off) {
            prev.r0 = sh.sr0[t - off];
            prev.r1 = sh.sr1[t - off];
        }
        __syncthreads();
        incl = compose(prev, incl);
        sh.sr0[t] = incl.r0;
        sh.sr1[t] = incl.r1;
        __syncthreads();
    }
    Pair ex = pair_identity();
    if (t > 0) {
        ex.r0 = sh.sr0[t - 1];
        ex.r1 = sh.sr1[t - 1];
    }
    __syncthreads();
    return ex;
}

// Add a chunk's terms one by one to the exact sum (the fallback).  The terms
// go through LDS with one coalesced load; lane 0 adds them in order.
__device__ __forceinline__ double fallback_chunk(const double *__restrict__ x, size_t n,
                                                 size_t c, double s, WalkShared &sh)
{
    const size_t b = c * kChunk;
    const size_t len = n - b < (size_t)kChunk ? n - b : (size_t)kChunk;
    for (int i = threadIdx.x; i < (int)len; i += kWalkThreads)
        sh.terms[i] = x[b + i];
    __syncthreads();
    if (threadIdx.x == 0) {
        double acc = s;
        for (size_t i = 0; i < len; i++)
            acc = acc + sh.terms[i];
        sh.s = acc;
    }
    __syncthreads();
    double r = sh.s;
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kWalkThreads) void walk_kernel(
    const double *__restrict__ x, size_t n, double init,
    const DescRec *__restrict__ desc, size_t nch, double *__restrict__ out,
    exseq_stats *__restrict__ stats)
{
    __shared__ WalkShared sh;
    const int t = threadIdx.x;
    double s = init;
    uint64_t n_fast = 0, n_fb = 0, fb_terms = 0;
    if (t == 0)
        sh.misses = 0;
    int64_t first_fb = -1;
    uint32_t sflags = 0;

    for (size_t base = 0; base < nch; base += kWalkThreads) {
        const int cnt = (int)(nch - base < (size_t)kWalkThreads ? nch - base : kWalkThreads);
        const bool have = t < cnt;
        DescRec d = have ? desc[base + t] : DescRec{0, 0, 0, 0u, 0u};
        const uint32_t dkey = d.meta & kKeyMask;
        const Pair mine{d.r0, d.r0 + (int64_t)((d.meta >> kDrShift) & 3u) - 1};
        const uint32_t dflags = d.meta & (kFlagNeg | kFlagBad | kFlagNonFinite);
        if (__syncthreads_or(have && (dflags & kFlagNonFinite)))
            sflags |= EXSEQ_STAT_NONFINITE;
        int cur = 0;
        while (cur < cnt) {
            const uint32_t ks = key_of(s);
            const bool fs = key_has_fast_path(ks);
            const int64_t m = count_of(s);
            const bool active = have && t >= cur;
            Pair elem = active ? mine : pair_identity();
            Pair ex = block_exclusive_scan(elem, sh);
            const int64_t mt = m + pair_at(ex, m);
            bool ok = active && fs && dkey == ks && mt >= kCountLo && mt < kCountHi &&
                      run_applies(mt, mine, d.lo, d.hi, dflags);
            if (t == 0)
                sh.first = cnt;
            __syncthreads();
            if (active && !ok)
                atomicMin(&sh.first, t);
            __syncthreads();
            const int first = sh.first;
            // Apply every chunk before `first`: the count after them is the
            // exclusive prefix at `first` (or the inclusive total).
            if (first > cur) {
                if (first < cnt) {
                    if (t == first)
                        sh.s = assemble(ks, mt);
                } else if (t == cnt - 1) {
                    sh.s = assemble(ks, mt + pair_at(mine, mt));
                }
                __syncthreads();
                s = sh.s;
                __syncthreads();
                n_fast += (uint64_t)(first - cur);
            }
            if (first >= cnt)
                break;
            // Chunk `first` does not apply at its start.  If the run before it
            // ended exactly on 2^(e+1) the state is now in the next binade and
            // the chunk may apply there; otherwise add it term by term.
            const uint32_t ks2 = key_of(s);
            const int64_t m2 = count_of(s);
            if (t == first) {
                bool ok2 = key_has_fast_path(ks2) && dkey == ks2 &&
                           run_applies(m2, mine, d.lo, d.hi, dflags);
                sh.ok2 = ok2;
                if (ok2)
                    sh.s = assemble(ks2, m2 + pair_at(mine, m2));
                if (dkey != ks2)
                    sh.misses++;
            }
            __syncthreads();
            if (sh.ok2) {
                s = sh.s;
                n_fast++;
            } else {
                const size_t c = base + (size_t)first;
                s = fallback_chunk(x, n, c, s, sh);
                n_fb++;
                fb_terms += (n - c * kChunk < (size_t)kChunk) ? n - c * kChunk : (size_t)kChunk;
                if (first_fb < 0)
                    first_fb = (int64_t)c;
            }
            __syncthreads();
            cur = first + 1;
        }
    }
    if (t == 0) {
        out[0] = s;
        if (stats) {
            exseq_stats st;
            st.chunks = nch;
            st.fast_chunks = n_fast;
            st.fallback_chunks = n_fb;
            st.fallback_terms = fb_terms;
            st.first_fallback = first_fb;
            st.flags = sflags;
            st.plan_misses = sh.misses;
            *stats = st;
        }
    }
}

// ---------------------------------------------------------------------------
// Fixed-tree total of the chunk sums (tree_sum_f64).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void tree_total_kernel(
    const double *__restrict__ tsum, size_t nch, double *__restrict__ out)
{
    __shared__ double part[kPlanThreads];
    const int t = threadIdx.x;
    // lane t takes chunks t, t + 1024, ... in a fixed order
    double s = 0.0;
    for (size_t i = t; i < nch; i += kPlanThreads)
        s += tsum[i];
    part[t] = s;
    __syncthreads();
    for (int h = kPlanThreads / 2; h >= 1; h >>= 1) {
        if (t < h)
            part[t] = part[t] + part[t + h];
        __syncthreads();
    }
    if (t == 0)
        out[0] = part[0];
}

__global__ void write_value_kernel(double *out, double v) { out[0] = v; }

__global__ void write_stats_empty_kernel(exseq_stats *stats)
{
    exseq_stats st;
    st.chunks = st.fast_chunks = st.fallback_chunks = st.fallback_terms = 0;
    st.first_fallback = -1;
    st.flags = 0;
    st.plan_misses = 0;
    *stats = st;
}

// ---------------------------------------------------------------------------
// Host-side launch sequences.
// ---------------------------------------------------------------------------
SumLayout sum_layout(size_t n)
{
    SumLayout L;
    L.nch = (n + kChunk - 1) / kChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    L.tsum_off = take(L.nch * sizeof(double));
    L.key_off = take(L.nch * sizeof(uint32_t));
    L.desc_off = take(L.nch * sizeof(DescRec));
    L.total = off;
    return L;
}

const char *const kPathKernels[] = {"chunk_tsum_kernel", "plan_kernel", "chunk_desc_kernel",
                                     "walk_kernel"};
const int kPathKernelCount = 4;

int launch_exact_sum(const double *x, size_t n, double init, double *out, void *ws,
                     hipStream_t stream, uint32_t flags, exseq_stats *stats,
                     void *const *events, int n_events)
{
    // events[2i] / events[2i+1] bracket kernel i when profiling.
    auto mark = [&](int i) {
        if (events && i < n_events && events[i])
            hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
    };
    if (n == 0) {
        hipLaunchKernelGGL(write_value_kernel, dim3(1), dim3(1), 0, stream, out, init);
        if (stats)
            hipLaunchKernelGGL(write_stats_empty_kernel, dim3(1), dim3(1), 0, stream, stats);
        return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
    }
    SumLayout L = sum_layout(n);
    char *w = static_cast<char *>(ws);
    double *tsum = reinterpret_cast<double *>(w + L.tsum_off);
    uint32_t *key = reinterpret_cast<uint32_t *>(w + L.key_off);
    DescRec *desc = reinterpret_cast<DescRec *>(w + L.desc_off);
    mark(0);
    hipLaunchKernelGGL(chunk_tsum_kernel, dim3((unsigned)L.nch), dim3(kChunkThreads), 0,
                       stream, x, n, tsum);
    mark(1);
    mark(2);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, tsum, L.nch,
                       init, flags, key);
    mark(3);
    mark(4);
    hipLaunchKernelGGL(chunk_desc_kernel, dim3((unsigned)L.nch), dim3(kChunkThreads), 0,
                       stream, x, n, key, desc);
    mark(5);
    mark(6);
    hipLaunchKernelGGL(walk_kernel, dim3(1), dim3(kWalkThreads), 0, stream, x, n, init,
                       desc, L.nch, out, stats);
    mark(7);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
}

int launch_tree_sum(const double *x, size_t n, double *out, void *ws, hipStream_t stream)
{
    if (n == 0) {
        hipLaunchKernelGGL(write_value_kernel, dim3(1), dim3(1), 0, stream, out, 0.0);
        return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
    }
    SumLayout L = sum_layout(n);
    double *tsum = reinterpret_cast<double *>(static_cast<char *>(ws) + L.tsum_off);
    hipLaunchKernelGGL(chunk_tsum_kernel, dim3((unsigned)L.nch), dim3(kChunkThreads), 0,
                       stream, x, n, tsum);
    hipLaunchKernelGGL(tree_total_kernel, dim3(1), dim3(kPlanThreads), 0, stream, tsum,
                       L.nch, out);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
}

}  // namespace exseq
