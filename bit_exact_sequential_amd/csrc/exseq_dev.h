// Device building blocks of the exact sequential sum on gfx950, shared by the
// kernels of the tile chain (exseq_sum.hip) and of the single pass
// (exseq_pass.hip): term loads and sources, the fixed-tree chunk sum, the
// plan's look-back, the runs of a chunk under a binade, the term-by-term
// resolution from an exact sum, located crossings and the O(1) step of a
// tile (Research-1433 "Forming the CPU's sequential double sums on a GPU,
// bit for bit", Findings 2-6; Research-1424 "integer_ssim_cuda and the CPU's
// frame sum", Findings 3).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "exseq.h"
#include "exseq_internal.h"
#include "exseq_rules.h"
#include "exseq_ssim_dev.h"
#include "exseq_wave.h"

namespace exseq {

// ---------------------------------------------------------------------------
// Loads: lane l of a chunk takes terms 4l .. 4l+3; past n a term is absent.
// ---------------------------------------------------------------------------
// A value the compiler must treat as opaque.  Picking one of several
// register values by a run-time index (unrolled selects) is otherwise turned
// back into an indexed load from a stack copy, i.e. scratch memory.
__device__ __forceinline__ double opaque(double x)
{
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ int64_t opaque(int64_t x)
{
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ uint32_t opaque(uint32_t x)
{
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ Four opaque(Four f)
{
#pragma unroll
    for (int i = 0; i < 4; i++)
        f.v[i] = opaque(f.v[i]);
    return f;
}

typedef double v2f64 __attribute__((ext_vector_type(2)));

// The tiles read their terms once: 16-byte non-temporal loads.
__device__ __forceinline__ Four load_four(const double *__restrict__ x, size_t n, size_t first,
                                          bool nt)
{
    Four f;
    if (first + 4 <= n) {
        if ((((uintptr_t)(x + first)) & 15u) == 0u) {
            const v2f64 *p = reinterpret_cast<const v2f64 *>(x + first);
            v2f64 a, b;
            if (nt) {
                a = __builtin_nontemporal_load(p);
                b = __builtin_nontemporal_load(p + 1);
            } else {
                a = p[0];
                b = p[1];
            }
            f.v[0] = a.x;
            f.v[1] = a.y;
            f.v[2] = b.x;
            f.v[3] = b.y;
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

// Term sources of the exact sum.  chunk() gives lane t its terms 4t .. 4t+3
// of chunk c of sum s; it is called by every lane of the workgroup with the
// same chunk.  keep() hands the terms to the caller where it asked for them.
// One sum's terms as the single pass sees them: its pointer, length and
// start, and where its chunks begin in the launch.
struct SumView {
    const double *x;
    size_t n;
    double init;
    uint32_t cb;   // the sum's first chunk in the launch
    uint32_t nch;  // its chunks
};

struct PlainTerms {
    static constexpr int kLdsInts = 1;
    static constexpr bool kInter = false;  // the single pass: one sum per tile
    static constexpr int kPassWaves = 4;   // the single pass: waves per SIMD it is built for
    __device__ __forceinline__ Four chunk_v(const SumView &v, size_t c, int *) const
    {
        return load_four(v.x, v.n, c * kChunk + 4 * (size_t)threadIdx.x, true);
    }
    __device__ __forceinline__ Four chunk(const BatchArgs &a, int s, size_t c, int *) const
    {
        return load_four(a.x[s], a.n[s], c * kChunk + 4 * (size_t)threadIdx.x, true);
    }
    __device__ __forceinline__ void keep(size_t, const Four &) const {}
    __device__ __forceinline__ void done() const {}
};

// Every k-th double from x[s]: one field of records of k doubles, such as the
// four doubles per window (l*c*s, l, c, s) of an SSIM pass that keeps the
// factors (ADR-1464 "float_ssim_cuda adds its frame sums in the CPU's raster
// order, on the host", Decision).  Cached loads: the k sums' tiles of one
// range run together and read the same lines.
struct StridedTerms {
    static constexpr int kLdsInts = 1;
    uint32_t k;
    __device__ __forceinline__ Four chunk(const BatchArgs &a, int s, size_t c, int *) const
    {
        const size_t n = a.n[s];
        const size_t first = c * kChunk + 4 * (size_t)threadIdx.x;
        const double *__restrict__ x = a.x[s] + first * k;
        Four f;
        f.cnt = first < n ? (int)(n - first < 4 ? n - first : 4) : 0;
#pragma unroll
        for (int i = 0; i < 4; i++)
            f.v[i] = i < f.cnt ? x[(size_t)i * k] : 0.0;
        return f;
    }
    __device__ __forceinline__ void keep(size_t, const Four &) const {}
    __device__ __forceinline__ void done() const {}
};

// Fixed-shape tree sum of a chunk: ((v0+v1)+(v2+v3)) per lane, the wave in a
// fixed order, then the four waves as ((w0+w1)+(w2+w3)).
__device__ __forceinline__ double chunk_tree(const Four &f, double *lds4)
{
    const double s = wave_sum_f64((f.v[0] + f.v[1]) + (f.v[2] + f.v[3]));
    if (lane_id() == 0)
        lds4[wave_id()] = s;
    __syncthreads();
    const double t = (lds4[0] + lds4[1]) + (lds4[2] + lds4[3]);
    __syncthreads();
    return t;
}


// ---------------------------------------------------------------------------
// The plan
// ---------------------------------------------------------------------------
EXSEQ_HD uint32_t plan_key(double p, uint32_t flags)
{
    const uint32_t mode = flags & EXSEQ_PLAN_MASK;
    if (mode == EXSEQ_PLAN_ALL_FALLBACK)
        return 0u;
    if (mode == EXSEQ_PLAN_FIXED)
        return (flags >> 8) & kKeyMask;
    if (mode == EXSEQ_PLAN_ALL_ZERO)
        return key_of(0.0);
    uint32_t k = key_of(p);
    if (!key_has_fast_path(k))
        return 0u;
    if (mode == EXSEQ_PLAN_PLUS_ONE)
        k += 1u;
    else if (mode == EXSEQ_PLAN_MINUS_ONE)
        k -= 1u;
    return key_has_fast_path(k) ? k : 0u;
}

// Status word of a tile: epoch (16 bits) | flag (2 bits) | value (46 bits:
// the top of the double, rounded).  One 64-bit word, written and read with
// relaxed agent-scope atomics: it is self-contained, so nothing else needs
// ordering with it.
constexpr uint64_t kStAgg = 1, kStIncl = 2;
constexpr uint64_t kStValMask = (1ULL << 46) - 1;
constexpr int kSpinLimit = 200000;

__device__ __forceinline__ uint64_t st_pack(uint32_t epoch, uint64_t flag, double v)
{
    const uint64_t r = (dbits(v) + (1ULL << 17)) >> 18;
    return ((uint64_t)(epoch & 0xFFFFu) << 48) | (flag << 46) | (r & kStValMask);
}
__device__ __forceinline__ double st_value(uint64_t w) { return bitsd((w & kStValMask) << 18); }
__device__ __forceinline__ uint64_t st_flag(uint64_t w, uint32_t epoch)
{
    return ((w >> 48) == (uint64_t)(epoch & 0xFFFFu)) ? ((w >> 46) & 3u) : 0u;
}

// Decoupled look-back (one wave): init plus every tile sum before tile c of
// this sum.  Returns NaN if a predecessor never shows up (no plan then).
// The wave waits on the nearest 64 predecessors; once they are all there
// and none is inclusive, it reads up to kLbDeep further windows in one round
// trip (the tiles before them have usually published by then).  Windows are
// summed nearest first, one wave sum each, whichever round trip read them.
constexpr int kLbDeep = 8;
__device__ double lookback(const uint64_t *st0, uint32_t c, double init, uint32_t epoch)
{
    const int lane = lane_id();
    double acc = 0.0;
    int64_t j = (int64_t)c - 1;  // the nearest predecessor not summed yet
    int spins = 0;
    while (true) {
        const int64_t idx = j - lane;
        uint64_t fl;
        double v;
        if (idx >= 0) {
            const uint64_t w = load_relaxed_u64(st0 + idx);
            fl = st_flag(w, epoch);
            v = st_value(w);
        } else {
            fl = kStIncl;
            v = (idx == -1) ? init : 0.0;
        }
        if (__ballot(fl == 0)) {
            if (++spins > kSpinLimit)
                return __builtin_nan("");
            __builtin_amdgcn_s_sleep(2);
            continue;
        }
        uint64_t incl = __ballot(fl == kStIncl);
        int stop = incl ? __builtin_ctzll(incl) : 64;
        acc += wave_sum_f64(lane <= stop ? v : 0.0);
        if (incl)
            return acc;
        j -= 64;
        // the windows further back, all in one round trip
        uint64_t w[kLbDeep];
#pragma unroll
        for (int k = 0; k < kLbDeep; k++) {
            const int64_t ik = j - 64 * k - lane;
            w[k] = ik >= 0 ? load_relaxed_u64(st0 + ik) : 0;
        }
#pragma unroll
        for (int k = 0; k < kLbDeep; k++) {
            const int64_t ik = j - lane;
            if (ik >= 0) {
                fl = st_flag(w[k], epoch);
                v = st_value(w[k]);
            } else {
                fl = kStIncl;
                v = (ik == -1) ? init : 0.0;
            }
            if (__ballot(fl == 0))
                break;  // wait on this window
            incl = __ballot(fl == kStIncl);
            stop = incl ? __builtin_ctzll(incl) : 64;
            acc += wave_sum_f64(lane <= stop ? v : 0.0);
            if (incl)
                return acc;
            j -= 64;
        }
    }
}

// A composed run over many tiles: the components stay bounded (a run that
// large never applies, so it is only marked bad).
EXSEQ_HD Run run_compose_sat(const Run &a, const Run &b)
{
    Run c = run_compose(a, b);
    const int64_t lim = (int64_t)1 << 56;
    if (c.p.r0 > lim || c.p.r0 < -lim || c.p.r1 > lim || c.p.r1 < -lim || c.lo < -lim ||
        c.hi > lim) {
        c.flags |= kFlagBad;
        c.p = Pair{0, 0};
        c.lo = c.hi = 0;
    }
    return c;
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ Run dpp_run(const Run &v)
{
    Run r;
    r.p = dpp_pair<Ctrl, RowMask>(v.p);
    r.lo = dpp_i64<Ctrl, RowMask>(v.lo, 0);
    r.hi = dpp_i64<Ctrl, RowMask>(v.hi, 0);
    r.flags = dpp_u32<Ctrl, RowMask>(v.flags, 0u);
    return r;
}

// Ordered composition of the wave's runs (lane 0 first), in every lane.
__device__ __forceinline__ Run wave_reduce_run(Run v)
{
    v = run_compose_sat(dpp_run<kDppRowShr1>(v), v);
    v = run_compose_sat(dpp_run<kDppRowShr2>(v), v);
    v = run_compose_sat(dpp_run<kDppRowShr4>(v), v);
    v = run_compose_sat(dpp_run<kDppRowShr8>(v), v);
    v = run_compose_sat(dpp_run<kDppRowBcast15, 0xA>(v), v);
    v = run_compose_sat(dpp_run<kDppRowBcast31, 0xC>(v), v);
    Run r;
    r.p = readlane_pair(v.p, 63);
    r.lo = readlane_i64(v.lo, 63);
    r.hi = readlane_i64(v.hi, 63);
    r.flags = (uint32_t)__builtin_amdgcn_readlane((int)v.flags, 63);
    return r;
}

// ---------------------------------------------------------------------------
// A chunk's run under a key
// ---------------------------------------------------------------------------
struct WaveRun {
    Pair p;
    int64_t lo, hi;
    uint32_t flags;
};

// One wave's part of a chunk's run under `key`: the ordered composition of
// the wave's 256 terms.  Uses the order-free integer sum where no term of the
// wave ties (the pair is then (R, R)), and forms prefix bounds only where a
// scaled term is negative.  The same result in every lane.
__device__ __forceinline__ WaveRun wave_run(const Four &f, uint32_t key)
{
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool sgn = (key >> 11) & 1u;
    int64_t r0[4], r1[4];
    bool neg = false, bad = false, nonfin = false, tie = false;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (i < f.cnt) {
            const TermInc ti = term_inc(f.v[i], scale, sgn);
            r0[i] = ti.r0;
            r1[i] = ti.r1;
            neg |= ti.neg;
            bad |= ti.bad;
            nonfin |= is_nonfinite(f.v[i]);
            tie |= ti.r0 != ti.r1;
        } else {
            r0[i] = r1[i] = 0;
        }
    }
    const bool wtie = __ballot(tie) != 0;
    const bool wneg = __ballot(neg) != 0;
    const bool wbad = __ballot(bad) != 0;
    const bool wnf = __ballot(nonfin) != 0;
    WaveRun w;
    if (!wtie) {
        const int64_t r = wave_sum_i64((r0[0] + r0[1]) + (r0[2] + r0[3]));
        w.p = Pair{r, r};
    } else {
        Pair a = Pair{r0[0], r1[0]};
#pragma unroll
        for (int i = 1; i < 4; i++)
            a = compose(a, Pair{r0[i], r1[i]});
        w.p = wave_reduce_pair(a);
    }
    w.lo = 0;
    w.hi = 0;
    if (wneg) {
        // Bounds of every prefix: the smallest and largest prefix of the
        // even-start increments (a scan over the wave), widened by the
        // number of ties -- along either start parity each term adds its r0
        // or its r1, which differ by one exactly where the term ties.
        int64_t a = 0, mn = 0, mx = 0, nt = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a += r0[i];
            mn = a < mn ? a : mn;
            mx = a > mx ? a : mx;
            nt += r0[i] != r1[i];
        }
        const int64_t excl = wave_incl_scan_i64(a) - a;
        int64_t lo = wave_min_i64(excl + mn), hi = wave_max_i64(excl + mx);
        if (wtie) {
            const int64_t ties = wave_sum_i64(nt);
            lo -= ties;
            hi += ties;
        }
        w.lo = lo < 0 ? lo : 0;
        w.hi = hi > 0 ? hi : 0;
    }
    w.flags = (wneg ? kFlagNeg : 0u) | (wbad ? kFlagBad : 0u) | (wnf ? kFlagNonFinite : 0u);
    return w;
}

// The runs of CPB chunks at once (one wave's part of each, as wave_run).
// Where no term of the wave ties and every increment of a chunk's part has
// one sign -- nearly always -- the CPB order-free integer sums are taken
// together so that their reduction chains overlap; otherwise chunk by chunk.
// Missing terms are +0.0 (the sources pad with it), which changes no run.
//
// Per term: y = x * (+-2^scale) (one multiply while the factor is a normal
// double, i.e. for sums from 2^-971 up; ldexp and a sign flip below), the
// two magic adds, and three bit operations on the results: a0 = M0 + y lies
// in [2^52, 2^53) exactly when y rounds to an integer there (high word
// 0x433xxxxx: checked through the AND and the OR of the high words), its
// mantissa bit 51 says whether the increment is >= 0, and a tie shows as a
// difference other than one between the low words of a1 = M0 + 1 + y and a0.
template <int CPB>
__device__ __forceinline__ void wave_runs(const Four *f, const uint32_t *key,
                                          WaveRun (*lds)[kChunkThreads / 64])
{
    uint64_t v[CPB];
    bool easy = true;
    uint32_t negs = 0u;  // chunk k's increments are all < 0 (bit k)
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        const int scale = 1075 - (int)(key[k] & 0x7FFu);
        const bool flip = (key[k] & 0x800u) != 0u;  // mirror a negative plan
        uint32_t tacc = 0u, hand = ~0u, hor = 0u;
        uint64_t sum = 0;
        auto term = [&](double y) {
            const double a0 = kMagic0 + y;
            const double a1 = kMagic1 + y;
            const uint32_t h = (uint32_t)(dbits(a0) >> 32);
            tacc |= ((uint32_t)dbits(a1) - (uint32_t)dbits(a0)) ^ 1u;
            hand &= h;
            hor |= h;
            sum += dbits(a0);
        };
        if (scale <= 1023) {
            const double fac = flip ? -ldexp(1.0, scale) : ldexp(1.0, scale);
#pragma unroll
            for (int i = 0; i < 4; i++)
                term(f[k].v[i] * fac);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const double y = ldexp(f[k].v[i], scale);
                term(flip ? -y : y);
            }
        }
        v[k] = sum - 4 * (uint64_t)kMagic0Bits;
        const bool ok = tacc == 0u && (((hand ^ kMagic0Hi) | (hor ^ kMagic0Hi)) >> 20) == 0u;
        const bool pos = __ballot(!((hand >> 19) & 1u)) == 0;  // every a0 >= M0
        const bool neg = __ballot((hor >> 19) & 1u) == 0;      // every a0 < M0
        easy &= __ballot(!ok) == 0 && (pos || neg);
        negs |= (!pos && neg) ? 1u << k : 0u;
    }
    if (easy) {
        int64_t w[CPB];
#pragma unroll
        for (int k = 0; k < CPB; k++)
            w[k] = (int64_t)v[k];
        wave_sum_i64_n<CPB>(w);
        if (lane_id() == 0) {
#pragma unroll
            for (int k = 0; k < CPB; k++) {
                WaveRun r;
                r.p = Pair{w[k], w[k]};
                const bool n = (negs >> k) & 1u;
                r.lo = n && w[k] < 0 ? w[k] : 0;
                r.hi = 0;
                r.flags = n ? kFlagNeg : 0u;
                lds[k][wave_id()] = r;
            }
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        const WaveRun w = wave_run(f[k], key[k]);
        if (lane_id() == 0)
            lds[k][wave_id()] = w;
    }
}

// The four waves' parts composed in order.
EXSEQ_HD WaveRun join_waves(const WaveRun *w)
{
    WaveRun r = w[0];
#pragma unroll
    for (int k = 1; k < kChunkThreads / 64; k++) {
        const Run c = run_compose(Run{r.p, r.lo, r.hi, r.flags},
                                  Run{w[k].p, w[k].lo, w[k].hi, w[k].flags});
        r.p = c.p;
        r.lo = c.lo;
        r.hi = c.hi;
        r.flags = c.flags;
    }
    if (!(r.flags & kFlagNeg))
        r.hi = r.p.r0 > r.p.r1 ? r.p.r0 : r.p.r1;
    return r;
}

// A run whose increment exceeds the width of a binade can never apply;
// clearing it keeps every sum of runs far from int64 overflow.
EXSEQ_HD WaveRun clamp_run(WaveRun r)
{
    const int64_t lim = kCountLo + 1;
    if (r.p.r0 > lim || r.p.r0 < -lim || r.p.r1 > lim || r.p.r1 < -lim || r.hi > lim ||
        r.lo < -lim) {
        r.flags |= kFlagBad;
        r.p = Pair{0, 0};
        r.lo = r.hi = 0;
    }
    return r;
}

// r must be clamped.
__device__ __forceinline__ void store_desc(const DescArrays &d, size_t c, uint32_t key,
                                           const WaveRun &r, uint32_t extra)
{
    const int64_t dr = r.p.r1 - r.p.r0;  // -1, 0 or +1: the run's map is monotone
    d.r0[c] = r.p.r0;
    d.lo[c] = r.lo;
    d.hi[c] = r.hi;
    d.meta[c] = (key & kKeyMask) | ((uint32_t)(dr + 1) << kDrShift) | r.flags | extra;
}

// acc + t[lo] + t[lo+1] + ... + t[hi-1], one add at a time in that order (the
// loop itself), on one lane.  16-byte LDS reads, three batches of kB pairs
// in flight: a batch's reads have the adds of the two batches before it to
// arrive in (a dependent fp64 add takes a few cycles, an LDS read far more),
// so that mostly the chain of dependent adds is serial.
__device__ __forceinline__ double add_in_order(double acc, const double *t, int lo, int hi)
{
    constexpr int kB = 4;
    int i = lo;
    if ((i & 1) && i < hi)
        acc = acc + t[i++];
    const v2f64 *p = reinterpret_cast<const v2f64 *>(t + i);
    const int nv = (hi - i) >> 1;
    int v = 0;
    if (nv >= 3 * kB) {
        v2f64 a[kB], b[kB], c[kB];
#pragma unroll
        for (int j = 0; j < kB; j++) {
            a[j] = p[j];
            b[j] = p[kB + j];
            c[j] = p[2 * kB + j];
        }
        v = 3 * kB;
        while (nv - v >= 3 * kB) {
#pragma unroll
            for (int j = 0; j < kB; j++) {
                acc = acc + a[j].x;
                acc = acc + a[j].y;
            }
#pragma unroll
            for (int j = 0; j < kB; j++)
                a[j] = p[v + j];
#pragma unroll
            for (int j = 0; j < kB; j++) {
                acc = acc + b[j].x;
                acc = acc + b[j].y;
            }
#pragma unroll
            for (int j = 0; j < kB; j++)
                b[j] = p[v + kB + j];
#pragma unroll
            for (int j = 0; j < kB; j++) {
                acc = acc + c[j].x;
                acc = acc + c[j].y;
            }
#pragma unroll
            for (int j = 0; j < kB; j++)
                c[j] = p[v + 2 * kB + j];
            v += 3 * kB;
        }
#pragma unroll
        for (int j = 0; j < kB; j++) {
            acc = acc + a[j].x;
            acc = acc + a[j].y;
        }
#pragma unroll
        for (int j = 0; j < kB; j++) {
            acc = acc + b[j].x;
            acc = acc + b[j].y;
        }
#pragma unroll
        for (int j = 0; j < kB; j++) {
            acc = acc + c[j].x;
            acc = acc + c[j].y;
        }
    }
    for (; v < nv; v++) {
        const v2f64 q = p[v];
        acc = acc + q.x;
        acc = acc + q.y;
    }
    i += 2 * nv;
    if (i < hi)
        acc = acc + t[i];
    return acc;
}

// ---------------------------------------------------------------------------
// Workgroup building blocks of the chain and the walk: 256 lanes, lane t
// holds 4 consecutive items (the chunks of a window of 1024, or the 1024
// terms of a chunk being resolved).
// ---------------------------------------------------------------------------
constexpr int kPer = 4;
constexpr int kWaves = kWalkThreads / 64;
constexpr int kWindow = kWalkThreads * kPer;  // 1024 chunks or terms
constexpr int kNone = 0x7FFFFFFF;
// A resolve round that adds fewer terms than this counts as short; after two
// short rounds the rest of the chunk goes through one lane in order.
constexpr int kShortRound = 128;

static_assert(kWindow == kChunk, "a window of chunks and a chunk of terms share the layout");
static_assert(kWalkThreads == kChunkThreads, "the tiles and the walk share the resolve");

// One wave's candidate for "the first item that needs attention", with what
// the owning lane computed for it.
struct Cand {
    int idx;
    int ok2;        // chunk applies after renormalising (1), misplanned (2)
    double s_at;    // exact sum at the item (or after the item's plain add)
    double s_next;  // exact sum after the chunk when ok2 == 1
    Pair ex_after;  // window prefix through the chunk
};

// Scan and candidate scratch of the workgroup building blocks (double-
// buffered by `buf`).
struct WalkCore {
    Pair tot[2][kWaves];   // per-wave totals of a scan (double-buffered)
    Cand cand[2][kWaves];  // per-wave candidates (double-buffered)
    double endv[2];        // a round's end state, from the lane holding the last item
    int flag[2][kWaves];
};

// The same with a chunk's terms, for the one-lane path of the resolution.
struct WalkLds : WalkCore {
    double terms[kChunk];
};

// Exclusive workgroup scan of the lanes' pairs; one barrier.  Waves without
// a tie scan plain integers (the pair is (v, v)).  `buf` alternates between
// calls so that a call's writes never race with the previous call's reads.
__device__ __forceinline__ Pair block_excl_scan(Pair v, bool lane_tie, WalkCore &sh, int buf)
{
    const int lane = lane_id(), wave = wave_id();
    Pair inc;
    if (__ballot(lane_tie) == 0) {
        const int64_t s = wave_incl_scan_i64(v.r0);
        inc = Pair{s, s};
    } else {
        inc = wave_incl_scan_pair(v);
    }
    if (lane == 63)
        sh.tot[buf][wave] = inc;
    __syncthreads();
    Pair pre = pair_identity();
#pragma unroll
    for (int w = 0; w < kWaves; w++)
        if (w < wave)
            pre = compose(pre, sh.tot[buf][w]);
    return compose(pre, wave_shift_pair(inc));
}

// Workgroup OR; one barrier.
__device__ __forceinline__ bool block_any(bool p, WalkCore &sh, int buf)
{
    const bool w = __ballot(p) != 0;
    if (lane_id() == 0)
        sh.flag[buf][wave_id()] = w;
    __syncthreads();
    bool r = false;
#pragma unroll
    for (int k = 0; k < kWaves; k++)
        r |= sh.flag[buf][k] != 0;
    return r;
}

// One barrier: whether every lane is clean, whether any lane saw a
// non-finite term, and the sum of the lanes' integers.
struct CleanSum {
    bool clean, nonfinite;
    int64_t sum;
};
__device__ __forceinline__ CleanSum block_clean_sum(bool clean, bool nf, int64_t v, WalkCore &sh,
                                                    int buf)
{
    const bool wclean = __ballot(!clean) == 0;
    const bool wnf = __ballot(nf) != 0;
    const int64_t wsum = wave_sum_i64(v);
    if (lane_id() == 0) {
        sh.flag[buf][wave_id()] = (wclean ? 1 : 0) | (wnf ? 2 : 0);
        sh.tot[buf][wave_id()].r0 = wsum;
    }
    __syncthreads();
    CleanSum r{true, false, 0};
#pragma unroll
    for (int k = 0; k < kWaves; k++) {
        r.clean &= (sh.flag[buf][k] & 1) != 0;
        r.nonfinite |= (sh.flag[buf][k] & 2) != 0;
        r.sum += sh.tot[buf][k].r0;
    }
    return r;
}

// Publish each wave's lowest-lane candidate; the smallest over the workgroup
// (idx = kNone if none).  One barrier.
__device__ __forceinline__ Cand block_first(bool has, const Cand &mine, WalkCore &sh, int buf)
{
    const uint64_t b = __ballot(has);
    const int lane = lane_id(), wave = wave_id();
    if (b == 0) {
        if (lane == 0)
            sh.cand[buf][wave].idx = kNone;
    } else if (lane == __builtin_ctzll(b)) {
        sh.cand[buf][wave] = mine;
    }
    __syncthreads();
    int bw = 0, bi = sh.cand[buf][0].idx;
#pragma unroll
    for (int k = 1; k < kWaves; k++) {
        const int i = sh.cand[buf][k].idx;
        if (i < bi) {
            bi = i;
            bw = k;
        }
    }
    return sh.cand[buf][bw];
}

__device__ __forceinline__ Cand cand_none()
{
    Cand c;
    c.idx = kNone;
    c.ok2 = 0;
    c.s_at = 0.0;
    c.s_next = 0.0;
    c.ex_after = pair_identity();
    return c;
}

// Exact resolution of the len terms of a chunk (lane t holds terms 4t ..
// 4t+3 in f) from the exact running sum S before term pos.
__device__ __forceinline__ double resolve_terms(const Four &f, int len, double S, int pos,
                                                WalkCore &sh, double *terms, int &buf)
{
    const int t = threadIdx.x;
    double xv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        xv[k] = f.v[k];
        terms[kPer * t + k] = xv[k];  // visible after the next barrier
    }
    // A round costs about as much as 300 one-lane adds.  Rounds pay where a
    // binade holds more terms than that; after a crossing (or the first
    // non-zero term) that leaves |S| below 512 times the term just added, the
    // next binades are short and the rest goes through one lane in order.
    int shorts = 0;
    bool small = false;
    while (pos < len) {
        const uint64_t sb = dbits(S);
        const uint32_t E = (uint32_t)(sb >> 52) & 0x7FFu;
        if ((sb << 1) == 0) {
            // S is +-0: zeros keep a zero (-0 only while every term is -0);
            // the first non-zero term becomes S exactly.
            Cand mine = cand_none();
#pragma unroll
            for (int k = kPer - 1; k >= 0; k--) {
                const int i = kPer * t + k;
                if (i >= pos && i < len && (dbits(xv[k]) << 1) != 0) {
                    mine.idx = i;
                    mine.s_at = xv[k];
                }
            }
            const Cand fz = block_first(mine.idx != kNone, mine, sh, buf);
            buf ^= 1;
            if (sb >> 63) {
                bool lane_pz = false;
#pragma unroll
                for (int k = 0; k < kPer; k++) {
                    const int i = kPer * t + k;
                    lane_pz |= i >= pos && i < len && i < fz.idx && dbits(xv[k]) == 0;
                }
                if (block_any(lane_pz, sh, buf))
                    S = 0.0;
                buf ^= 1;
            }
            if (fz.idx >= len)
                break;
            S = fz.s_at;
            pos = fz.idx + 1;
            small = true;  // S is now one term
            continue;
        }
        if (E == 0x7FFu) {
            // S is +-inf or NaN: it stays so, unless an opposite infinity or
            // a NaN term turns it into NaN.
            if (S == S) {
                bool kills = false;
#pragma unroll
                for (int k = 0; k < kPer; k++) {
                    const int i = kPer * t + k;
                    kills |= i >= pos && i < len &&
                             (xv[k] != xv[k] ||
                              (is_nonfinite(xv[k]) && ((dbits(xv[k]) ^ sb) >> 63)));
                }
                if (block_any(kills, sh, buf))
                    S = __builtin_nan("");
                buf ^= 1;
            }
            break;
        }
        if (E == 0u || small || shorts >= 2) {
            // subnormal S, or the binade keeps changing: the remaining terms
            // one by one on lane 0, in order
            __syncthreads();
            Cand mine = cand_none();
            if (t == 0) {
                mine.idx = 0;
                mine.s_at = add_in_order(S, terms, pos, len);
            }
            const Cand fs = block_first(t == 0, mine, sh, buf);
            buf ^= 1;
            S = fs.s_at;
            break;
        }
        // S normal: one round in its binade.
        const uint32_t key = (uint32_t)(sb >> 52);
        const int64_t m = count_of(S);
        const int scale = 1075 - (int)E;
        const bool sgn = (sb >> 63) != 0;
        Pair pr[kPer];
        bool bad[kPer];
        bool tie = false;
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const int i = kPer * t + k;
            if (i >= pos && i < len) {
                const TermInc ti = term_inc(xv[k], scale, sgn);
                pr[k] = Pair{ti.r0, ti.r1};
                bad[k] = ti.bad;
                tie |= ti.r0 != ti.r1;
            } else {
                pr[k] = pair_identity();
                bad[k] = false;
            }
        }
        // lane-local inclusive prefixes, then the workgroup scan
        Pair acc[kPer];
        acc[0] = pr[0];
#pragma unroll
        for (int k = 1; k < kPer; k++)
            acc[k] = tie ? compose(acc[k - 1], pr[k])
                         : Pair{acc[k - 1].r0 + pr[k].r0, acc[k - 1].r0 + pr[k].r0};
        const Pair X = block_excl_scan(acc[kPer - 1], tie, sh, buf);
        buf ^= 1;
        // the count before this lane's items, and after each of them
        const int64_t cnt0 = m + pair_at(X, m);
        int64_t cnt[kPer];
#pragma unroll
        for (int k = 0; k < kPer; k++)
            cnt[k] = cnt0 + pair_at(acc[k], cnt0);
        int firstk = -1;
#pragma unroll
        for (int k = kPer - 1; k >= 0; k--) {
            const int i = kPer * t + k;
            if (i >= pos && i < len && (bad[k] || cnt[k] < kCountLo + 1 || cnt[k] > kCountHi - 1))
                firstk = k;
        }
        Cand mine = cand_none();
        if (firstk >= 0) {
            int64_t cb = cnt0;
            double xf = opaque(xv[0]);
#pragma unroll
            for (int k = 1; k < kPer; k++)
                if (k == firstk) {
                    cb = opaque(cnt[k - 1]);
                    xf = opaque(xv[k]);
                }
            const int i = kPer * t + firstk;
            mine.idx = i;
            mine.s_at = ((i == pos) ? S : assemble(key, cb)) + xf;  // the one plain add
            mine.s_next = xf;
        }
        // the lane holding the last term reports the round's end state
        if ((len - 1) / kPer == t) {
            const int kl = (len - 1) - kPer * t;
            double e = 0.0;
#pragma unroll
            for (int k = 0; k < kPer; k++)
                if (k == kl)
                    e = assemble(key, cnt[k]);
            sh.endv[buf] = e;
        }
        const Cand fr = block_first(firstk >= 0, mine, sh, buf);
        const double endv = sh.endv[buf];
        buf ^= 1;
        if (fr.idx == kNone) {
            S = endv;  // no term left the binade
            break;
        }
        shorts += (fr.idx + 1 - pos) < kShortRound;
        small = fabs(fr.s_at) < 512.0 * fabs(fr.s_next);
        S = fr.s_at;
        pos = fr.idx + 1;
    }
    return S;
}

__device__ __forceinline__ double resolve_terms(const Four &f, int len, double S, int pos, WalkLds &sh,
                                                int &buf)
{
    return resolve_terms(f, len, S, pos, sh, sh.terms, buf);
}

// The same for chunk c of sum s, its terms formed again by the source.
template <class Src>
__device__ __forceinline__ double resolve_chunk(const Src &src, const BatchArgs &a, int s,
                                                size_t c, double S, int pos, WalkLds &sh,
                                                int &buf, int *lds_src)
{
    const size_t n = a.n[s];
    const size_t b = c * kChunk;
    const int len = (int)(n - b < (size_t)kChunk ? n - b : (size_t)kChunk);
    const Four f = src.chunk(a, s, c, lds_src);
    return resolve_terms(f, len, S, pos, sh, buf);
}

// ---------------------------------------------------------------------------
// The exact chain between the tiles of a sum.
//
// Chain words start at zero (chain_clear_kernel runs before the tiles) and a
// published word is never zero, so a word is there exactly when it is not
// zero.  Each word is self-contained and written once with a relaxed
// agent-scope atomic store, so no other memory has to be ordered with it.
//   agg[4 t + 0]: kAggPresent | kAggRegular (regular tiles) | the descriptor
//                 meta bits of the tile's composed run (key, r1 - r0, flags)
//   agg[4 t + 1..3]: r0, lo, hi of that run, each xor kIntTag (regular only)
//   incl[t]:      bits of the exact sum after tile t, xor kInclXor, or
//                 kInclFailed (irregular tiles only)
// A published sum is never the NaN whose bits are kInclXor or kInclXor ^ 1:
// NaNs are published as the default quiet NaN.
// ---------------------------------------------------------------------------
constexpr uint64_t kAggPresent = 1ULL << 63;
constexpr uint64_t kAggRegular = 1ULL << 62;
constexpr uint64_t kIntTag = 1ULL << 62;  // v ^ kIntTag != 0 for |v| < 2^61
constexpr uint64_t kInclXor = 0xFFF8000000000001ULL;
constexpr uint64_t kInclFailed = 1;
constexpr uint64_t kQuietNaN = 0x7FF8000000000000ULL;

EXSEQ_HD uint64_t enc_i64(int64_t v) { return (uint64_t)v ^ kIntTag; }
EXSEQ_HD int64_t dec_i64(uint64_t w) { return (int64_t)(w ^ kIntTag); }
__device__ __forceinline__ uint64_t enc_sum(double s)
{
    return (s == s ? dbits(s) : kQuietNaN) ^ kInclXor;
}

// Composition of the wave's runs with the HIGHER lanes first (lane 63's run,
// then lane 62's, ..., then lane 0's), complete in lane 63: the same ordered
// scan as wave_incl_scan_pair with the operands swapped.
__device__ __forceinline__ Run wave_reduce_run_rev(Run v)
{
    v = run_compose_sat(v, dpp_run<kDppRowShr1>(v));
    v = run_compose_sat(v, dpp_run<kDppRowShr2>(v));
    v = run_compose_sat(v, dpp_run<kDppRowShr4>(v));
    v = run_compose_sat(v, dpp_run<kDppRowShr8>(v));
    v = run_compose_sat(v, dpp_run<kDppRowBcast15, 0xA>(v));
    v = run_compose_sat(v, dpp_run<kDppRowBcast31, 0xC>(v));
    return v;
}

// Pairs of runs without a negative term composed in order, each result held
// within +-2^57 (such pairs only grow, so a total past 2^56 shows at the end).
__device__ __forceinline__ Pair compose_clamped(Pair a, Pair b)
{
    const int64_t lim = (int64_t)1 << 57;
    Pair c = compose(a, b);
    c.r0 = c.r0 > lim ? lim : c.r0;
    c.r1 = c.r1 > lim ? lim : c.r1;
    return c;
}

// The same order as wave_reduce_run_rev (the higher lanes first, complete in
// lane 63) for such pairs.
__device__ __forceinline__ Pair wave_reduce_pair_rev(Pair v)
{
    v = compose_clamped(v, dpp_pair<kDppRowShr1>(v));
    v = compose_clamped(v, dpp_pair<kDppRowShr2>(v));
    v = compose_clamped(v, dpp_pair<kDppRowShr4>(v));
    v = compose_clamped(v, dpp_pair<kDppRowShr8>(v));
    v = compose_clamped(v, dpp_pair<kDppRowBcast15, 0xA>(v));
    v = compose_clamped(v, dpp_pair<kDppRowBcast31, 0xC>(v));
    return v;
}

// Runs that compose by a plain sum of their increments: tie-free and
// monotone, every one non-decreasing (no flag, the bounds unused) or every
// one non-increasing (kFlagNeg, bounds (total, 0)).
EXSEQ_HD bool rising_run(const Pair &p, uint32_t flags)
{
    return p.r0 == p.r1 && flags == 0u && p.r0 >= 0;
}
EXSEQ_HD bool falling_run(const Pair &p, int64_t lo, int64_t hi, uint32_t flags)
{
    return p.r0 == p.r1 && flags == kFlagNeg && p.r0 <= 0 && lo == p.r0 && hi == 0;
}

struct ChainLds {
    Run wrun[2][kWaves];
    uint32_t key0;
    uint64_t incl;
};

// Looks back from tile tl of a sum (whose tile 0 is tile tb of the launch)
// for the nearest irregular tile xp, 1024 tiles at a time (4 per lane, all
// their words requested at once), and composes the regular tiles in between
// in order into acc (they must all be planned for one binade, key0).
// Returns kBackOk, kBackBad (xp found, but the regular tiles in between
// changed binade) or kBackLost (a word never showed up).
constexpr int kBackOk = 0, kBackBad = 1, kBackLost = 2;
constexpr int kBackPer = 4;  // tiles per lane per round

__device__ __forceinline__ int chain_back(const ChainArea &ch, uint32_t tb, uint32_t tl,
                                          WalkLds &sh, ChainLds &cl, int &buf, Run &acc,
                                          uint32_t &key0, int64_t &xp)
{
    constexpr int kRound = kBackPer * kChunkThreads;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    acc = run_identity();  // the tiles after the irregular one, in order
    key0 = 0u;
    xp = -1;
    bool keys_ok = true;
    for (int64_t j0 = (int64_t)tl - 1; j0 >= 0; j0 -= kRound) {
        // lane t holds tiles j0 - 4t - i, i = 0..3 (i = 0 the latest)
        uint64_t w[kBackPer][4];
#pragma unroll
        for (int i = 0; i < kBackPer; i++) {
            const int64_t j = j0 - kBackPer * t - i;
            const uint64_t *p = ch.agg + 4 * ((size_t)tb + (size_t)(j < 0 ? 0 : j));
#pragma unroll
            for (int q = 0; q < 4; q++)
                w[i][q] = j >= 0 ? load_relaxed_u64(p + q) : 0;
        }
        bool miss = false;
        for (int spin = 0;; spin++) {
            bool need = false;
#pragma unroll
            for (int i = 0; i < kBackPer; i++) {
                const int64_t j = j0 - kBackPer * t - i;
                const uint64_t *p = ch.agg + 4 * ((size_t)tb + (size_t)(j < 0 ? 0 : j));
                if (j < 0)
                    continue;
                // the meta word is written last: until it is there, all
                // four are read again (one round trip once they arrive)
                if (w[i][0] == 0) {
                    need = true;
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        w[i][q] = load_relaxed_u64(p + q);
                } else if (w[i][0] & kAggRegular) {
#pragma unroll
                    for (int q = 1; q < 4; q++)
                        if (w[i][q] == 0) {
                            need = true;
                            w[i][q] = load_relaxed_u64(p + q);
                        }
                }
            }
            if (!need)
                break;
            if (spin > kSpinLimit) {
                miss = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        // the nearest irregular tile: the smallest local index 4t + i
        int mine = kRound;
#pragma unroll
        for (int i = kBackPer - 1; i >= 0; i--)
            if (j0 - kBackPer * t - i >= 0 && !(w[i][0] & kAggRegular))
                mine = kBackPer * t + i;
        const uint64_t bi = __ballot(mine < kRound), bm = __ballot(miss);
        if (lane == 0) {
            int wf = kRound;
            if (bi)
                wf = __builtin_amdgcn_readlane(mine, (int)__builtin_ctzll(bi));
            sh.flag[buf][wave] = wf | (bm ? 0x10000 : 0);
        }
        if (t == 0 && j0 == (int64_t)tl - 1)
            cl.key0 = (uint32_t)(w[0][0] & kKeyMask);
        __syncthreads();
        int first = kRound;
        bool anymiss = false;
#pragma unroll
        for (int k = 0; k < kWaves; k++) {
            const int v = sh.flag[buf][k];
            first = (v & 0xFFFF) < first ? (v & 0xFFFF) : first;
            anymiss |= (v >> 16) != 0;
        }
        key0 = cl.key0;
        buf ^= 1;
        if (anymiss)
            return kBackLost;
        // the regular tiles after it, the earlier ones first; a wave whose
        // tiles all have a tie-free run without a negative term (nearly
        // always) composes them as one integer sum, and one whose tiles have
        // no negative term (ties allowed) composes their pairs alone: such a
        // run's prefixes are bounded by its total (run_top), so its bounds
        // need no composing
        bool bad = false, plain = true, fall = true, nonneg = true;
        int64_t tot = 0;
#pragma unroll
        for (int i = kBackPer - 1; i >= 0; i--) {
            if (j0 - kBackPer * t - i >= 0 && kBackPer * t + i < first) {
                const int64_t r0 = dec_i64(w[i][1]);
                const Run ti{Pair{r0, r0 + (int64_t)((w[i][0] >> kDrShift) & 3u) - 1},
                             dec_i64(w[i][2]), dec_i64(w[i][3]),
                             (uint32_t)w[i][0] & (kFlagNeg | kFlagBad | kFlagNonFinite)};
                plain &= rising_run(ti.p, ti.flags);
                fall &= falling_run(ti.p, ti.lo, ti.hi, ti.flags);
                nonneg &= ti.flags == 0u && ti.p.r0 >= 0 && ti.p.r1 >= 0;
                tot += r0;
                bad |= ((uint32_t)w[i][0] & kKeyMask) != key0;
            }
        }
        Run r;
        if (__ballot(!plain) == 0) {
            tot = wave_sum_i64(tot);
            r = Run{Pair{tot, tot}, 0, tot, 0u};
            if (tot > ((int64_t)1 << 56))
                r = Run{Pair{0, 0}, 0, 0, kFlagBad};
        } else if (__ballot(!fall) == 0) {
            tot = wave_sum_i64(tot);
            r = Run{Pair{tot, tot}, tot, 0, kFlagNeg};
            if (tot < -((int64_t)1 << 56))
                r = Run{Pair{0, 0}, 0, 0, kFlagBad};
        } else if (__ballot(!nonneg) == 0) {
            Pair pp = pair_identity();
#pragma unroll
            for (int i = kBackPer - 1; i >= 0; i--) {
                if (j0 - kBackPer * t - i >= 0 && kBackPer * t + i < first) {
                    const int64_t r0 = dec_i64(w[i][1]);
                    pp = compose_clamped(pp, Pair{r0, r0 + (int64_t)((w[i][0] >> kDrShift) & 3u) - 1});
                }
            }
            pp = wave_reduce_pair_rev(pp);
            const int64_t lim = (int64_t)1 << 56;
            r = Run{pp, 0, 0, 0u};
            if (pp.r0 > lim || pp.r1 > lim)
                r = Run{Pair{0, 0}, 0, 0, kFlagBad};
        } else {
            r = run_identity();
#pragma unroll
            for (int i = kBackPer - 1; i >= 0; i--) {
                if (j0 - kBackPer * t - i >= 0 && kBackPer * t + i < first) {
                    const int64_t r0 = dec_i64(w[i][1]);
                    const Run ti{Pair{r0, r0 + (int64_t)((w[i][0] >> kDrShift) & 3u) - 1},
                                 dec_i64(w[i][2]), dec_i64(w[i][3]),
                                 (uint32_t)w[i][0] & (kFlagNeg | kFlagBad | kFlagNonFinite)};
                    r = run_compose_sat(r, ti);
                }
            }
            r = wave_reduce_run_rev(r);
        }
        const uint64_t bb = __ballot(bad);
        if (lane == 63)
            cl.wrun[buf][wave] = r;
        if (lane == 0)
            sh.flag[buf][wave] = bb != 0;
        __syncthreads();
        Run R = cl.wrun[buf][kWaves - 1];
        bool anybad = sh.flag[buf][kWaves - 1] != 0;
#pragma unroll
        for (int k = kWaves - 2; k >= 0; k--) {
            R = run_compose_sat(R, cl.wrun[buf][k]);
            anybad |= sh.flag[buf][k] != 0;
        }
        buf ^= 1;
        keys_ok &= !anybad;
        acc = run_compose_sat(R, acc);
        if (first < kRound) {
            xp = j0 - first;
            break;
        }
    }
    if (xp < 0)
        return kBackLost;  // no irregular tile before (the first tile always is one)
    return keys_ok ? kBackOk : kBackBad;
}

// ---------------------------------------------------------------------------
// Crossings, located by the tile.  For a chunk whose plan expects the running
// sum to cross from its binade into the next one up, the tile forms the
// increment pair of every prefix of the chunk under the planned binade and
// finds, from the planned start count, the term that crosses.  It publishes
// that term, the prefix pairs just before it and through it, and under the
// next binade the pair of the terms after it and of the whole chunk (pairs
// packed as r0 << 2 | (r1 - r0 + 1)).  Given the exact start count m, the
// chain checks in O(1) that the crossing is still at that term -- the count
// before it below 2^53, the count through it at least 2^53; the plan is off
// by far fewer counts than one term moves the count, so it nearly always is
// -- adds the term with one fp64 add and applies the pair of the rest from
// the count the add gave (Research-1433 Findings 4: non-negative increments
// keep every intermediate count below the final one, so the final count
// alone shows that no second crossing happened).  Only chunks with no
// negative scaled term and nothing bad under either binade get a crossing.
// ---------------------------------------------------------------------------
EXSEQ_HD int64_t rec_pack(Pair p)
{
    return p.r0 * 4 + (p.r1 - p.r0 + 1);
}
EXSEQ_HD Pair rec_unpack(int64_t v)
{
    const int64_t r0 = v >> 2;
    return Pair{r0, r0 + (v & 3) - 1};
}

// The lane's inclusive prefixes under `key` (acc) and whether any term was
// negative or bad under it.
__device__ __forceinline__ bool lane_prefixes(const Four &f, uint32_t key, Pair *acc)
{
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool sgn = (key >> 11) & 1u;
    bool bad = false;
    Pair a = pair_identity();
#pragma unroll
    for (int i = 0; i < kPer; i++) {
        if (i < f.cnt) {
            const TermInc ti = term_inc(f.v[i], scale, sgn);
            bad |= ti.bad || ti.neg;
            a = compose(a, Pair{ti.r0, ti.r1});
        }
        acc[i] = a;
    }
    return bad;
}

// Ordered exclusive workgroup scan and the workgroup's total; one barrier.
__device__ __forceinline__ Pair block_scan_total(Pair v, WalkCore &sh, int buf, Pair &total)
{
    const int lane = lane_id(), wave = wave_id();
    const Pair inc = wave_incl_scan_pair(v);
    if (lane == 63)
        sh.tot[buf][wave] = inc;
    __syncthreads();
    Pair pre = pair_identity();
    total = pair_identity();
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        if (w < wave)
            pre = compose(pre, sh.tot[buf][w]);
        total = compose(total, sh.tot[buf][w]);
    }
    return compose(pre, wave_shift_pair(inc));
}

// A crossing as published (kCrossWords words): the crossing term's index j;
// under the planned binade the packed prefix pairs through j - 1 and
// through j, and bounds of every prefix before j; under the next binade the
// packed pair of the terms after j and of the whole chunk, and bounds of
// every prefix of the terms after j; the term itself.
constexpr int kCrossWords = 10;
constexpr int kXj = 0, kXpj1 = 1, kXpj = 2, kXsuf = 3, kXwhole = 4, kXterm = 5, kXpreLo = 6,
              kXpreHi = 7, kXsufLo = 8, kXsufHi = 9;
struct CrossCand {
    int j;
    int64_t pj1, pj;
    double xj;
};
struct CrossLds {
    CrossCand c[kWaves];
    int bad[kWaves];
    Run suf2[kWaves];
    Pair tot2[kWaves];
    int64_t plo[kWaves], phi[kWaves];
};

// Locates the crossing of a chunk (terms f, len of them, planned binade
// key, planned start count m_est); false (uniformly) if the chunk has none
// from m_est or cannot have one.  On success out[] holds the published
// words in every lane.  Three barriers.
__device__ __forceinline__ bool crossing_find(const Four &f, int len, uint32_t key, int64_t m_est,
                                              bool down, WalkCore &sh, CrossLds &xl, int &buf,
                                              uint64_t *out)
{
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool sgn = (key >> 11) & 1u;
    Pair acc[kPer], tot;
    bool bad1 = false;
    {
        Pair a = pair_identity();
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            if (i < f.cnt) {
                const TermInc ti = term_inc(f.v[i], scale, sgn);
                bad1 |= ti.bad;
                a = compose(a, Pair{ti.r0, ti.r1});
            }
            acc[i] = a;
        }
    }
    const Pair pre = block_scan_total(acc[kPer - 1], sh, buf, tot);
    buf ^= 1;
    // the first term whose count from m_est reaches 2^53 (or, downwards,
    // falls below 2^52)
    int firstk = -1;
#pragma unroll
    for (int i = kPer - 1; i >= 0; i--) {
        const Pair pe = compose(pre, acc[i]);
        const int64_t ce = m_est + pair_at(pe, m_est);
        if (kPer * t + i < len && (down ? ce < kCountLo : ce >= kCountHi))
            firstk = i;
    }
    const uint64_t b = __ballot(firstk >= 0), bb = __ballot(bad1);
    if (lane == (b ? (int)__builtin_ctzll(b) : 0)) {
        CrossCand c;
        c.j = kNone;
        c.pj1 = c.pj = 0;
        c.xj = 0.0;
        if (b) {
            Pair before = pre, at = acc[0];
            double x = opaque(f.v[0]);
#pragma unroll
            for (int i = 1; i < kPer; i++)
                if (i == firstk) {
                    before = Pair{opaque(acc[i - 1].r0), opaque(acc[i - 1].r1)};
                    at = Pair{opaque(acc[i].r0), opaque(acc[i].r1)};
                    x = opaque(f.v[i]);
                }
            c.j = kPer * t + firstk;
            c.pj1 = rec_pack(firstk == 0 ? pre : compose(pre, before));
            c.pj = rec_pack(compose(pre, at));
            c.xj = x;
        }
        xl.c[wave] = c;
        xl.bad[wave] = bb != 0;
    }
    __syncthreads();
    int bw = 0;
    bool bad = xl.bad[0] != 0;
#pragma unroll
    for (int k = 1; k < kWaves; k++) {
        bad |= xl.bad[k] != 0;
        if (xl.c[k].j < xl.c[bw].j)
            bw = k;
    }
    const CrossCand c = xl.c[bw];
    if (bad || c.j == kNone)
        return false;
    // Bounds of every prefix before j under the planned binade (either start
    // parity: the smaller and the larger component of each prefix pair).
    int64_t plo = 0, phi = 0;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
        if (kPer * t + i < c.j) {
            const Pair pe = compose(pre, acc[i]);
            const int64_t mn = pe.r0 < pe.r1 ? pe.r0 : pe.r1;
            const int64_t mx = pe.r0 < pe.r1 ? pe.r1 : pe.r0;
            plo = mn < plo ? mn : plo;
            phi = mx > phi ? mx : phi;
        }
    }
    // Under the next binade (up, or down): the whole chunk, and the terms
    // after j as a run with its prefix bounds.
    const uint32_t key2 = down ? key - 1u : key + 1u;
    const int scale2 = 1075 - (int)(key2 & 0x7FFu);
    const bool sgn2 = (key2 >> 11) & 1u;
    bool bad2 = false;
    Pair whole = pair_identity();
    Run suf = run_identity();
#pragma unroll
    for (int i = 0; i < kPer; i++) {
        if (i < f.cnt) {
            const TermInc ti = term_inc(f.v[i], scale2, sgn2);
            bad2 |= ti.bad;
            const Pair q{ti.r0, ti.r1};
            whole = compose(whole, q);
            if (kPer * t + i > c.j) {
                const int64_t mn = ti.r0 < ti.r1 ? ti.r0 : ti.r1;
                const int64_t mx = ti.r0 < ti.r1 ? ti.r1 : ti.r0;
                suf = run_compose(suf, Run{q, mn < 0 ? mn : 0, mx > 0 ? mx : 0, 0u});
            }
        }
    }
    whole = wave_reduce_pair(whole);
    suf = wave_reduce_run(suf);
    plo = wave_min_i64(plo);
    phi = wave_max_i64(phi);
    const uint64_t bb2 = __ballot(bad2);
    if (lane == 0) {
        xl.tot2[wave] = whole;
        xl.suf2[wave] = suf;
        xl.plo[wave] = plo;
        xl.phi[wave] = phi;
        xl.bad[wave] = bb2 != 0;
    }
    __syncthreads();
    Pair tot2 = pair_identity();
    Run suf2 = run_identity();
#pragma unroll
    for (int k = 0; k < kWaves; k++) {
        bad2 |= xl.bad[k] != 0;
        tot2 = compose(tot2, xl.tot2[k]);
        suf2 = run_compose_sat(suf2, xl.suf2[k]);
        plo = xl.plo[k] < plo ? xl.plo[k] : plo;
        phi = xl.phi[k] > phi ? xl.phi[k] : phi;
    }
    if (bad2 || (suf2.flags & kFlagBad))
        return false;
    out[kXj] = enc_i64(c.j);
    out[kXpj1] = enc_i64(c.pj1);
    out[kXpj] = enc_i64(c.pj);
    out[kXsuf] = enc_i64(rec_pack(suf2.p));
    out[kXwhole] = enc_i64(rec_pack(tot2));
    out[kXterm] = dbits(c.xj) ^ kInclXor;  // a crossing term is finite: never kInclXor
    out[kXpreLo] = enc_i64(plo);
    out[kXpreHi] = enc_i64(phi);
    out[kXsufLo] = enc_i64(suf2.lo);
    out[kXsufHi] = enc_i64(suf2.hi);
    return true;
}

// The chain's side: from the exact sum S before a chunk (len terms, planned
// binade key, descriptor flags fl) with a located crossing w[].  Returns 1
// with S the sum after the chunk, 2 with S the exact sum after the crossing
// term and pos the next term (the rest term by term), or 0 if the crossing
// does not hold for this S (the whole chunk term by term).  For a chunk with
// a negative scaled term every prefix is checked against the binade it is
// in, through the published bounds (Research-1424 Findings 3).  The pairs
// w[kXsuf] and w[kXwhole] of a chunk without one may also take in runs that
// follow the chunk in the next binade: every success applies one of them.
EXSEQ_HD int crossing_apply(const uint64_t *w, int len, uint32_t key, uint32_t fl,
                                              bool down, double &S, int &pos)
{
    // a downward crossing has falling counts: every bound is checked
    const bool neg = (fl & kFlagNeg) != 0 || down;
    const uint32_t key2 = down ? key - 1u : key + 1u;
    const uint32_t ks = key_of(S);
    const int64_t m = count_of(S);
    if (ks == key2) {
        // the crossing came before the chunk: all of it in the next binade
        if (neg || !key_has_fast_path(ks))
            return 0;
        const int64_t e = m + pair_at(rec_unpack(dec_i64(w[kXwhole])), m);
        if (e > kCountHi)
            return 0;
        S = assemble(ks, e);
        return 1;
    }
    if (ks != key || !key_has_fast_path(ks))
        return 0;
    const int j = (int)dec_i64(w[kXj]);
    const int64_t cb = j == 0 ? m : m + pair_at(rec_unpack(dec_i64(w[kXpj1])), m);
    const int64_t cj = m + pair_at(rec_unpack(dec_i64(w[kXpj])), m);
    if (j >= len || (down ? cb < kCountLo || cj >= kCountLo : cb > kCountHi - 1 || cj < kCountHi))
        return 0;  // the crossing is elsewhere for this start
    if (neg && (m + dec_i64(w[kXpreLo]) < kCountLo + 1 || m + dec_i64(w[kXpreHi]) > kCountHi - 1))
        return 0;  // some prefix before it leaves the binade
    const double sb = j == 0 ? S : assemble(key, cb);
    S = sb + bitsd(w[kXterm] ^ kInclXor);  // the one plain add
    pos = j + 1;
    const uint32_t k2 = key_of(S);
    const int64_t m2 = count_of(S);
    if (k2 != key2 || !key_has_fast_path(k2))
        return 2;
    const Pair sp = rec_unpack(dec_i64(w[kXsuf]));
    if (!run_applies(m2, sp, dec_i64(w[kXsufLo]), dec_i64(w[kXsufHi]), neg ? kFlagNeg : 0u))
        return 2;  // a second crossing
    S = assemble(k2, m2 + pair_at(sp, m2));
    return 1;
}

// ---------------------------------------------------------------------------
// tile_kernel
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_sum(const BatchArgs &a, uint32_t g)
{
    int lo = 0, hi = a.count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.chunk_base[mid] <= g)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

__host__ __device__ __forceinline__ bool chain_on(uint32_t flags)
{
    return (flags & EXSEQ_PLAN_MASK) != EXSEQ_PLAN_ALL_FALLBACK && !(flags & EXSEQ_WALK_ONLY);
}

// How close (in counts of the binade) a chunk's planned start or end may come
// to an edge of its planned binade before the tile stops trusting the plan
// there: 4096 + 64 sqrt(terms up to the chunk's end).  The planned prefix and
// the exact running sum add the same terms in different orders; each add
// rounds by at most half a count, and rounding errors of either sum grow like
// a random walk, so this is far beyond their usual distance.  The margin only
// decides which chunks the chain adds term by term, never a result.
EXSEQ_HD int64_t plan_margin(uint32_t chunks_to_end)
{
    return 4096 + (int64_t)(64.0 * __builtin_sqrt((double)chunks_to_end * (double)kChunk));
}

// The binade a kept plan gives a tile (EXSEQ_PLAN_REUSE): pa and pb are the
// previous launch's planned prefixes before and after the tile.  Both,
// widened by 1/64 of their magnitude on either side, must lie in one binade
// with a fast path; 0 otherwise.  The widening absorbs how far the prefixes of
// consecutive frames drift apart; a plan that is still wrong costs term by
// term adds where the chain's checks fail, never a wrong result.
__device__ __forceinline__ uint32_t reuse_key(double pa, double pb)
{
    const bool neg = pa < 0.0;
    if (!(pa != 0.0 && pb != 0.0 && (pb < 0.0) == neg))
        return 0u;  // a zero, a NaN, or a sign change
    const double a = fabs(pa), b = fabs(pb);
    const double lo = (a < b ? a : b) * (1.0 - 1.0 / 64.0);
    const double hi = (a < b ? b : a) * (1.0 + 1.0 / 64.0);
    if (!(hi < __builtin_inf()))
        return 0u;
    const uint32_t k = key_of(neg ? -lo : lo);
    return k == key_of(neg ? -hi : hi) && key_has_fast_path(k) ? k : 0u;
}

// A value known to be the same in every lane, moved to scalar registers so
// that the chain's arithmetic on it runs on the scalar unit.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

constexpr int kIrrPer = 4 + kCrossWords;       // bank words per chunk
constexpr uint64_t kIrrCross = 1ULL << 40;     // bank meta: a crossing is located
constexpr uint64_t kIrrDown = 1ULL << 41;      // ... into the binade below
static_assert(4 + kIrrPer * kTileMax <= 64, "the bank fits one wave");

// One irregular tile's O(1) step from the exact sum S before it: the run A
// (the regular tiles since the irregular tile before it, then its chunks
// before the crossing; binade akey, none if 0), then the crossing (w, in a
// chunk of len terms, binade xkey, kFlagNeg in xfl, into the binade above or,
// with xdown, below), whose rest-of-chunk run takes in the chunks after it.
// False, with S unchanged, where a check fails for this S; the tile then adds
// chunk by chunk.
__device__ __forceinline__ bool tile_step(uint32_t akey, const Run &A, bool hasx,
                                          const uint64_t *w, int len, uint32_t xkey, uint32_t xfl,
                                          bool xdown, double &S)
{
    double T = S;
    if (akey != 0u) {
        const uint32_t ks = key_of(T);
        const int64_t mm = count_of(T);
        if (!(ks == akey && key_has_fast_path(ks) && run_applies(mm, A.p, A.lo, A.hi, A.flags)))
            return false;
        T = assemble(ks, mm + pair_at(A.p, mm));
    }
    if (hasx) {
        int pos = 0;
        const bool good = crossing_apply(w, len, xkey, xfl, xdown, T, pos) == 1;
        T = bitsd(uniform_u64(dbits(T)));
        if (!good)
            return false;
    }
    S = T;
    return true;
}

// A published step (kRecWords words per tile, all nonzero once written):
//   0: kRecPresent | akey | xkey << 12 | has crossing << 24 |
//      A's flags >> 14 << 32 | crossing kFlagNeg << 35 | (r1 - r0 + 1) << 36 |
//      crossing downwards << 38
//   1..3: A's r0, lo, hi;  4: the irregular tile before it;  5: the crossing
//   chunk's length;  6..15: the crossing's words  (integers xor kIntTag)
constexpr int kRecWords = 16;
constexpr uint64_t kRecPresent = 1ULL << 63;
constexpr int kCatch = 4;  // records a wave holds while it waits (16 lanes each)

// Zeroes the chain words of a launch of `tiles` tiles (none if 0): every
// tile's agg, incl and record words and the heads (a published chain word is
// never zero, so zero means "not yet").  Called by every thread of a grid of
// any shape, each taking words by its linear index.
__device__ __forceinline__ void zero_chain_words(const ChainArea &ch, uint32_t tiles)
{
    if (tiles == 0)
        return;
    const size_t blocks = (size_t)gridDim.x * gridDim.y;
    const size_t i = ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t stride = blocks * blockDim.x;
    for (size_t k = i; k < 4 * (size_t)tiles; k += stride)
        ch.agg[k] = 0;
    for (size_t k = i; k < (size_t)kRecWords * tiles; k += stride)
        ch.rec[k] = 0;
    for (size_t k = i; k < (size_t)tiles; k += stride)
        ch.incl[k] = 0;
    if (i < (size_t)kMaxBatch)
        ch.head[i] = 0;
}

// The word of the record a lane i < kRecWords of the publishing wave writes.
__device__ __forceinline__ uint64_t rec_word(int i, uint32_t akey, const Run &A, bool hasx,
                                             const uint64_t *w, int len, uint32_t xkey,
                                             uint32_t xfl, bool xdown, int64_t xp)
{
    uint64_t v = enc_i64(0);
    if (i == 0)
        v = kRecPresent | (uint64_t)(akey & kKeyMask) | ((uint64_t)(xkey & kKeyMask) << 12) |
            ((uint64_t)hasx << 24) |
            ((uint64_t)((A.flags >> 14) & 7u) << 32) | ((uint64_t)((xfl & kFlagNeg) != 0) << 35) |
            ((uint64_t)(A.p.r1 - A.p.r0 + 1) << 36) | ((uint64_t)xdown << 38);
    else if (i == 1)
        v = enc_i64(A.p.r0);
    else if (i == 2)
        v = enc_i64(A.lo);
    else if (i == 3)
        v = enc_i64(A.hi);
    else if (i == 4)
        v = enc_i64(xp);
    else if (i == 5)
        v = enc_i64(len);
#pragma unroll
    for (int k = 0; k < kCrossWords; k++)
        if (i == 6 + k && hasx)
            v = w[k];
    return v;
}

// The step of the record held in lanes 16 d .. 16 d + 15 of rw, from S.
__device__ __forceinline__ bool rec_step(uint64_t rw, int d, double &S)
{
    const int b = 16 * d;
    const uint64_t m = (uint64_t)readlane_i64((int64_t)rw, b);
    const int64_t r0 = dec_i64((uint64_t)readlane_i64((int64_t)rw, b + 1));
    const Run A{Pair{r0, r0 + (int64_t)((m >> 36) & 3u) - 1},
                dec_i64((uint64_t)readlane_i64((int64_t)rw, b + 2)),
                dec_i64((uint64_t)readlane_i64((int64_t)rw, b + 3)),
                (uint32_t)((m >> 32) & 7u) << 14};
    const bool hasx = (m >> 24) & 1u;
    uint64_t w[kCrossWords];
#pragma unroll
    for (int k = 0; k < kCrossWords; k++)
        w[k] = (uint64_t)readlane_i64((int64_t)rw, b + 6 + k);
    const int len = (int)dec_i64((uint64_t)readlane_i64((int64_t)rw, b + 5));
    return tile_step((uint32_t)m & kKeyMask, A, hasx, w, len, (uint32_t)(m >> 12) & kKeyMask,
                     ((m >> 35) & 1u) ? kFlagNeg : 0u, ((m >> 38) & 1u) != 0, S);
}

// The exact sum after irregular tile xp of a sum (whose first tile is tile tb
// of the launch), as its published word (0: the wait timed out; kInclFailed:
// the chain failed there).  The wave waits on xp's word and, at the same
// time, collects the records of xp, of the irregular tile before it, and so
// on (kCatch of them), polling the words of all of them: when an earlier one
// arrives first, the records take the sum forward to xp in O(1) steps each,
// so that a run of short links in the chain costs one wait (Research-1433
// Findings 6: the walk composes in order; any exact route gives the same
// bits).  The sums formed on the way are published for the tiles waiting on
// them (when `publish`; the same value a tile computes for itself).
__device__ __forceinline__ uint64_t catch_up(const ChainArea &ch, uint32_t tb, int64_t xp, bool publish)
{
    const int lane = lane_id();
    int64_t cl = lane == 0 ? xp : 0;  // lane d < known: c_d (c_0 = xp)
    int known = 1;
    bool chase = true;
    uint64_t rw = 0;  // lanes 16 d .. 16 d + 15: the record of c_d
    for (int spin = 0; spin <= kSpinLimit; spin++) {
        const int slot = known - 1;  // the record chased: c_slot's
        const bool want_rec = chase && slot < kCatch;
        const int64_t cs = readlane_i64(cl, slot);
        uint64_t wi = 0, wr = 0;
        if (lane < known)
            wi = load_relaxed_u64(ch.incl + tb + (size_t)cl);
        if (want_rec && (lane >> 4) == slot)
            wr = load_relaxed_u64(ch.rec + kRecWords * ((size_t)tb + (size_t)cs) + (lane & 15));
        const uint64_t w0 = (uint64_t)readlane_i64((int64_t)wi, 0);
        if (w0 != 0)
            return w0;  // xp's own word (or its failure)
        const uint64_t bi = __ballot(wi > kInclFailed);
        if (bi) {
            // the nearest member with a word: forward through the records
            int d = (int)__builtin_ctzll(bi);
            double T = bitsd((uint64_t)readlane_i64((int64_t)wi, d) ^ kInclXor);
            while (d > 0 && rec_step(rw, d - 1, T)) {
                d--;
                if (publish && lane == 0)
                    store_relaxed_u64(ch.incl + tb + (size_t)readlane_i64(cl, d), enc_sum(T));
            }
            if (d == 0)
                return enc_sum(T);
            // c_{d-1}'s step does not hold from this sum: wait on the
            // members from c_{d-1} on only
            known = d;
            chase = false;
            continue;
        }
        if (want_rec) {
            const uint64_t mask = 0xFFFFULL << (16 * slot);
            if ((__ballot(wr != 0) & mask) == mask) {
                if ((lane >> 4) == slot)
                    rw = wr;
                const int64_t nx = dec_i64((uint64_t)readlane_i64((int64_t)wr, 16 * slot + 4));
                if (lane == known)
                    cl = nx;
                known++;
            }
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return 0;
}

// The head of a sum's chain: its first chunk added to init term by term,
// published as the exact sum after that chunk.
template <class Src>
__device__ __forceinline__ void chain_head(const Src &src, const BatchArgs &a, int s,
                                           const ChainArea &ch, const DescArrays &d, WalkLds &sh,
                                           int *lds_src)
{
    const size_t n = a.n[s];
    if (n == 0)
        return;
    __builtin_amdgcn_s_setprio(3);  // the chain starts here
    const int len = (int)(n < (size_t)kChunk ? n : (size_t)kChunk);
    int buf = 0;
    const double S = resolve_terms(src.chunk(a, s, 0, lds_src), len, a.init[s], 0, sh, buf);
    if (threadIdx.x == 0)
        store_relaxed_u64(ch.head + s, enc_sum(S));
}


// What a walk over descriptors added, for the statistics.
struct WalkTally {
    uint64_t n_fast, n_fb, fb_terms;
    uint32_t misses;
    int64_t first_fb;
    bool nonfinite;
};

// The ordered walk over the descriptors of chunks [start, end) of sum s from
// the exact sum S before chunk `start` (dr0 .. dmeta point at the sum's first
// chunk); returns the exact sum after chunk end - 1.  A window of up to 1024
// chunks at a time: a clean window (every chunk in the running sum's binade,
// no tie, nothing negative or bad) is applied from the sum of its
// increments; otherwise one scan gives every chunk's start count, every chunk
// is checked at its exact start, and the first one that fails is added term
// by term from the exact sum, its terms formed again by the source.  Called
// by all 256 lanes of the workgroup, with uniform arguments.
template <class Src>
__device__ double walk_descs(const Src &src, const BatchArgs &a, int s,
                             const int64_t *__restrict__ dr0, const int64_t *__restrict__ dlo_a,
                             const int64_t *__restrict__ dhi_a,
                             const uint32_t *__restrict__ dmeta, size_t start, size_t end,
                             double S, WalkTally &wt, WalkLds &sh, int &buf, int *lds_src)
{
    const int t = threadIdx.x;
    const size_t n = a.n[s];
    // r0 and meta of the first window; each window prefetches the next one
    int64_t nr0[kPer];
    uint32_t nmeta[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const size_t i = start + (size_t)(kPer * t + k);
        nr0[k] = i < end ? dr0[i] : 0;
        nmeta[k] = i < end ? dmeta[i] : kFlagBad;
    }
    for (size_t base = start; base < end; base += kWindow) {
        const int cnt = (int)(end - base < (size_t)kWindow ? end - base : kWindow);
        int64_t r0[kPer];
        uint32_t meta[kPer];
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            r0[k] = nr0[k];
            meta[k] = nmeta[k];
            const size_t i = base + kWindow + (size_t)(kPer * t + k);
            nr0[k] = i < end ? dr0[i] : 0;
            nmeta[k] = i < end ? dmeta[i] : kFlagBad;
        }
        uint32_t dkey[kPer], dfl[kPer];
        Pair mine[kPer];
        bool lane_tie = false, lane_nf = false, lane_clean = true;
        int64_t lane_sum = 0;
        const uint32_t ks0 = key_of(S);
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const bool have = kPer * t + k < cnt;
            dkey[k] = have ? (meta[k] & kKeyMask) : 0u;
            dfl[k] = have ? (meta[k] & (kFlagNeg | kFlagBad | kFlagNonFinite)) : kFlagBad;
            const int64_t d1 = (int64_t)((meta[k] >> kDrShift) & 3u) - 1;
            mine[k] = have ? Pair{r0[k], r0[k] + d1} : pair_identity();
            if (have) {
                lane_tie |= d1 != 0;
                lane_nf |= (dfl[k] & kFlagNonFinite) != 0;
                lane_clean &= dkey[k] == ks0 && dfl[k] == 0u && d1 == 0;
                lane_sum += r0[k];
            }
        }
        // A clean window: every chunk planned for S's binade, no tie, no
        // negative scaled term, nothing bad.  Then the counts only grow,
        // every chunk applies iff the count after the last one is at most
        // 2^53, and the window needs only the sum of its increments.
        const CleanSum cs = block_clean_sum(lane_clean, lane_nf, lane_sum, sh, buf);
        buf ^= 1;
        wt.nonfinite |= cs.nonfinite;
        if (cs.clean && key_has_fast_path(ks0)) {
            const int64_t cnt_end = count_of(S) + cs.sum;
            if (cnt_end <= kCountHi) {
                S = assemble(ks0, cnt_end);
                wt.n_fast += (uint64_t)cnt;
                continue;
            }
        }
        int64_t dlo[kPer], dhi[kPer];
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            dlo[k] = dhi[k] = 0;
            if (dfl[k] & kFlagNeg) {
                dlo[k] = dlo_a[base + kPer * t + k];
                dhi[k] = dhi_a[base + kPer * t + k];
            }
        }
        // window prefixes: ex[k] = composition of the window's chunks before
        // this lane's chunk k
        Pair ex[kPer];
        {
            Pair acc = pair_identity();
#pragma unroll
            for (int k = 0; k < kPer; k++) {
                ex[k] = acc;
                acc = compose(acc, mine[k]);
            }
            const Pair X = block_excl_scan(acc, lane_tie, sh, buf);
            buf ^= 1;
#pragma unroll
            for (int k = 0; k < kPer; k++)
                ex[k] = compose(X, ex[k]);
        }

        int cur = 0;
        Pair excur = pair_identity();
        while (cur < cnt) {
            const uint32_t ks = key_of(S);
            const bool fs = key_has_fast_path(ks);
            const int64_t m = count_of(S);
            // The scan's two chains start at the window start with either
            // parity; take the one that has S's parity at `cur`.
            const int64_t want = m & 1;
            int p;
            if ((excur.r0 & 1) == want) {
                p = 0;
            } else if (((1 + excur.r1) & 1) == want) {
                p = 1;
            } else {
                // both chains merged on the other parity: scan again from cur
                Pair a2 = pair_identity();
#pragma unroll
                for (int k = 0; k < kPer; k++) {
                    ex[k] = a2;
                    if (kPer * t + k >= cur)
                        a2 = compose(a2, mine[k]);
                }
                const Pair X2 = block_excl_scan(a2, true, sh, buf);
                buf ^= 1;
#pragma unroll
                for (int k = 0; k < kPer; k++)
                    ex[k] = compose(X2, ex[k]);
                excur = pair_identity();
                p = (int)want;
            }
            const int64_t base_p = p ? excur.r1 : excur.r0;
            // this lane's first chunk (at or after cur) that does not apply,
            // its fields copied out by unrolled selects
            Cand mc = cand_none();
            int fk = -1;
            int64_t fmt = 0, flo = 0, fhi = 0;
            uint32_t fkey = 0, ffl = 0;
            Pair fmine = pair_identity(), fex = pair_identity();
#pragma unroll
            for (int k = kPer - 1; k >= 0; k--) {
                const int i = kPer * t + k;
                if (i >= cur && i < cnt) {
                    const int64_t mt = m + ((p ? ex[k].r1 : ex[k].r0) - base_p);
                    const bool ok = fs && dkey[k] == ks && mt >= count_floor(ks) && mt < kCountHi &&
                                    run_applies(mt, mine[k], dlo[k], dhi[k], dfl[k]);
                    if (!ok) {
                        fk = k;
                        fmt = mt;
                        flo = dlo[k];
                        fhi = dhi[k];
                        fkey = dkey[k];
                        ffl = dfl[k];
                        fmine = mine[k];
                        fex = ex[k];
                    }
                }
            }
            if (fk >= 0) {
                // exact sum before the chunk; if the runs before it ended on
                // 2^(e+1) the chunk may still apply in the next binade.
                const int i = kPer * t + fk;
                const double sat = (i == cur) ? S : assemble(ks, fmt);
                const uint32_t k2 = key_of(sat);
                const int64_t m2 = count_of(sat);
                const bool ok2 = key_has_fast_path(k2) && fkey == k2 &&
                                 run_applies(m2, fmine, flo, fhi, ffl);
                mc.idx = i;
                mc.ok2 = ok2 ? 1 : ((fkey != k2) ? 2 : 0);
                mc.s_at = sat;
                mc.s_next = ok2 ? assemble(k2, m2 + pair_at(fmine, m2)) : 0.0;
                mc.ex_after = compose(fex, fmine);
            }
            // the lane holding the window's last chunk reports the end state
            const int lastk = (cnt - 1) - kPer * t;
            if (fk < 0 && lastk >= 0 && lastk < kPer) {
#pragma unroll
                for (int k = 0; k < kPer; k++) {
                    if (k == lastk) {
                        const int64_t mt = m + ((p ? ex[k].r1 : ex[k].r0) - base_p);
                        mc.idx = cnt;  // "no failure": the sum after the window
                        mc.s_at = assemble(ks, mt + pair_at(mine[k], mt));
                    }
                }
            }
            const Cand fc = block_first(mc.idx != kNone, mc, sh, buf);
            buf ^= 1;
            if (fc.idx >= cnt) {
                wt.n_fast += (uint64_t)(cnt - cur);
                S = fc.s_at;
                break;
            }
            wt.n_fast += (uint64_t)(fc.idx - cur);
            excur = fc.ex_after;
            if (fc.ok2 == 1) {
                S = fc.s_next;
                wt.n_fast++;
            } else {
                wt.misses += fc.ok2 == 2;
                const size_t c = base + (size_t)fc.idx;
                S = resolve_chunk(src, a, s, c, fc.s_at, 0, sh, buf, lds_src);
                wt.n_fb++;
                wt.fb_terms += (n - c * kChunk < (size_t)kChunk) ? n - c * kChunk : (size_t)kChunk;
                if (wt.first_fb < 0)
                    wt.first_fb = (int64_t)c;
            }
            cur = fc.idx + 1;
        }
    }
    return S;
}

}  // namespace exseq
