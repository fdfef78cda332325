// gfx950 kernels of the exact sequential fp64 sum and of the fixed-tree sum.
//
// The path (Research-1433 "Forming the CPU's sequential double sums on a GPU,
// bit for bit", Findings 2-6; Research-1424 "integer_ssim_cuda and the CPU's
// frame sum", Findings 3).  A chunk is 1024 consecutive terms, held by 256
// lanes (4 waves of 64) with 4 consecutive terms per lane.
//
//  tile_kernel (one workgroup per tile of CPB consecutive chunks of one sum;
//  every tile of every sum of a batch in one launch; reads each term once):
//    1. load the tile's terms (16-byte non-temporal loads), fixed-tree fp64
//       sum of every chunk;
//    2. the plan: publish the tile's sum, find the prefix of the chunk sums
//       before the tile by a decoupled look-back over the predecessors'
//       status words, publish the inclusive prefix; a chunk's planned binade
//       is that of the prefix before it;
//    3. every term's increment pair under its chunk's planned binade,
//       composed in order (lane, ordered wave scan, waves in order) into the
//       chunk's descriptor: the pair, prefix bounds, flags;
//    4. the tile holding a sum's first chunk knows its exact start state
//       (init): one lane adds its terms in order and records the exact sum
//       after it, off the walk's critical path.
//  walk_kernel (one workgroup of 256 lanes per sum, after the tiles):
//    5. follows the chunks in order with the exact running sum, a window of
//       1024 chunks at a time.  A clean window (every chunk in the running
//       sum's binade, no tie, nothing negative or bad) is applied from the
//       sum of its increments; otherwise one scan gives every chunk's start
//       count, every chunk is checked at its exact start, and the first one
//       that fails is added term by term from the exact sum;
//    6. term by term means: every lane forms its terms' increments in the
//       current binade, a workgroup scan gives every prefix count, the first
//       term that leaves the binade is added with one fp64 add, and the next
//       round starts after it; when rounds keep resolving only a few terms,
//       one lane adds the rest in order.
//
// The look-back waits are bounded: a workgroup that waits too long gives up
// its plan (no fast path for its chunks).  A plan never changes a result,
// only how much is added term by term.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "exseq.h"
#include "exseq_internal.h"
#include "exseq_rules.h"
#include "exseq_wave.h"

namespace exseq {

// ---------------------------------------------------------------------------
// Loads: lane l of a chunk takes terms 4l .. 4l+3; past n a term is absent.
// ---------------------------------------------------------------------------
struct Four {
    double v[4];
    int cnt;  // how many of the four exist (0..4)
};

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

__global__ __launch_bounds__(kChunkThreads) void chunk_tsum_kernel(
    const double *__restrict__ x, size_t n, double *__restrict__ tsum)
{
    __shared__ double lds4[4];
    const size_t c = blockIdx.x;
    const Four f = load_four(x, n, c * kChunk + (size_t)threadIdx.x * 4, true);
    const double t = chunk_tree(f, lds4);
    if (threadIdx.x == 0)
        tsum[c] = t;
}

// ---------------------------------------------------------------------------
// The plan
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t plan_key(double p, uint32_t flags)
{
    const uint32_t mode = flags & EXSEQ_PLAN_MASK;
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
__device__ double lookback(const uint64_t *st0, uint32_t c, double init, uint32_t epoch)
{
    const int lane = lane_id();
    double acc = 0.0;
    int64_t j = (int64_t)c - 1;
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
        const uint64_t incl = __ballot(fl == kStIncl);
        const int stop = incl ? __builtin_ctzll(incl) : 64;
        acc += wave_sum_f64(lane <= stop ? v : 0.0);
        if (incl)
            return acc;
        j -= 64;
    }
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
        int64_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int64_t mn = r0[i] < r1[i] ? r0[i] : r1[i];
            const int64_t mx = r0[i] < r1[i] ? r1[i] : r0[i];
            lo += mn < 0 ? mn : 0;
            hi += mx > 0 ? mx : 0;
        }
        w.lo = wave_sum_i64(lo);
        w.hi = wave_sum_i64(hi);
    }
    w.flags = (wneg ? kFlagNeg : 0u) | (wbad ? kFlagBad : 0u) | (wnf ? kFlagNonFinite : 0u);
    return w;
}

// The four waves' parts composed in order.
__device__ __forceinline__ WaveRun join_waves(const WaveRun *w)
{
    WaveRun r = w[0];
#pragma unroll
    for (int k = 1; k < kChunkThreads / 64; k++) {
        r.p = compose(r.p, w[k].p);
        r.lo += w[k].lo;
        r.hi += w[k].hi;
        r.flags |= w[k].flags;
    }
    if (!(r.flags & kFlagNeg))
        r.hi = r.p.r0 > r.p.r1 ? r.p.r0 : r.p.r1;
    return r;
}

__device__ __forceinline__ void store_desc(const DescArrays &d, size_t c, uint32_t key, WaveRun r,
                                           bool cross)
{
    // A run whose increment exceeds the width of a binade can never apply;
    // clearing it keeps every sum of descriptors far from int64 overflow.
    const int64_t lim = kCountLo + 1;
    if (r.p.r0 > lim || r.p.r0 < -lim || r.p.r1 > lim || r.p.r1 < -lim || r.hi > lim ||
        r.lo < -lim) {
        r.flags |= kFlagBad;
        r.p = Pair{0, 0};
        r.lo = r.hi = 0;
    }
    const int64_t dr = r.p.r1 - r.p.r0;  // -1, 0 or +1: the run's map is monotone
    d.r0[c] = r.p.r0;
    d.lo[c] = r.lo;
    d.hi[c] = r.hi;
    d.meta[c] = (key & kKeyMask) | ((uint32_t)(dr + 1) << kDrShift) | r.flags |
                (cross ? kFlagCross : 0u);
}

// ---------------------------------------------------------------------------
// Crossing records.  For a chunk whose plan expects the running sum to cross
// into the next binade, the tile also stores, for every term position, the
// increment pair of the prefix ending there under the planned binade and
// under the next one (packed as r0 << 2 | (r1 - r0 + 1)).  Given the exact
// start count, the walk then finds the term that crosses, adds it with one
// fp64 add, and takes the rest of the chunk from the second prefix.
// Records exist only for chunks with no negative scaled term and nothing bad
// under either binade.
// ---------------------------------------------------------------------------
constexpr int64_t kRecMax = (int64_t)1 << 56;  // larger prefixes are clamped (never apply)

__device__ __forceinline__ int64_t rec_pack(Pair p)
{
    const int64_t r0 = p.r0 < kRecMax ? p.r0 : kRecMax;
    return (r0 << 2) | (p.r1 - p.r0 + 1);
}
__device__ __forceinline__ Pair rec_unpack(int64_t v)
{
    const int64_t r0 = v >> 2;
    return Pair{r0, r0 + (v & 3) - 1};
}

// Inclusive prefix pairs of the workgroup's 1024 terms under `key`, written
// to out[0 .. 1023]; returns (uniformly) whether any term was bad or
// negative under that key.  One barrier.
__device__ __forceinline__ bool record_prefix(const Four &f, uint32_t key, int64_t *out,
                                              Pair *lds_wtot, bool *lds_flag)
{
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool sgn = (key >> 11) & 1u;
    Pair acc[4];
    bool bad = false;
    Pair a = pair_identity();
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (i < f.cnt) {
            const TermInc ti = term_inc(f.v[i], scale, sgn);
            bad |= ti.bad || ti.neg;
            a = compose(a, Pair{ti.r0, ti.r1});
        }
        acc[i] = a;
    }
    const Pair inc = wave_incl_scan_pair(a);
    const bool wbad = __ballot(bad) != 0;
    const int lane = lane_id(), wave = wave_id();
    if (lane == 63)
        lds_wtot[wave] = inc;
    if (lane == 0)
        lds_flag[wave] = wbad;
    __syncthreads();
    Pair pre = pair_identity();
    bool any = false;
#pragma unroll
    for (int w = 0; w < kChunkThreads / 64; w++) {
        if (w < wave)
            pre = compose(pre, lds_wtot[w]);
        any |= lds_flag[w];
    }
    pre = compose(pre, wave_shift_pair(inc));
#pragma unroll
    for (int i = 0; i < 4; i++)
        out[threadIdx.x * 4 + i] = rec_pack(compose(pre, acc[i]));
    return any;
}

// acc + t[lo] + t[lo+1] + ... + t[hi-1], one add at a time in that order (the
// loop itself), on one lane.  The LDS reads go out eight at a time so that
// only the chain of adds is serial.
__device__ __forceinline__ double add_in_order(double acc, const double *t, int lo, int hi)
{
    int i = lo;
    for (; i + 8 <= hi; i += 8) {
        double v[8];
#pragma unroll
        for (int j = 0; j < 8; j++)
            v[j] = t[i + j];
#pragma unroll
        for (int j = 0; j < 8; j++)
            acc = acc + v[j];
    }
    for (; i < hi; i++)
        acc = acc + t[i];
    return acc;
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

template <int CPB>
__global__ __launch_bounds__(kChunkThreads) void tile_kernel(BatchArgs a,
                                                             uint64_t *__restrict__ status,
                                                             DescArrays d, RecArea rec)
{
    constexpr int kW = kChunkThreads / 64;
    __shared__ double lds_t[CPB][kW];
    __shared__ WaveRun lds_runs[CPB][kW];
    __shared__ double lds_p;
    __shared__ double lds_terms[kChunk];
    __shared__ Pair lds_wtot[2][kW];
    __shared__ bool lds_flag[2][kW];
    __shared__ int lds_slot;
    const uint32_t g0 = blockIdx.x * CPB;  // first global chunk of the tile
    const int s = find_sum(a, g0);
    const double *__restrict__ x = a.x[s];
    const size_t n = a.n[s];
    const uint32_t c0 = g0 - a.chunk_base[s];  // first local chunk
    const double init = a.init[s];
    const uint32_t mode = a.flags & EXSEQ_PLAN_MASK;
    const int lane = lane_id(), wave = wave_id();
    const uint32_t nch = (uint32_t)((n + kChunk - 1) / kChunk);

    Four f[CPB];
#pragma unroll
    for (int k = 0; k < CPB; k++)
        f[k] = load_four(x, n, (size_t)(c0 + k) * kChunk + (size_t)threadIdx.x * 4, true);
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        const double ws = wave_sum_f64((f[k].v[0] + f[k].v[1]) + (f[k].v[2] + f[k].v[3]));
        if (lane == 0)
            lds_t[k][wave] = ws;
    }
    __syncthreads();
    double T[CPB];
    double Ttile = 0.0;
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        T[k] = (lds_t[k][0] + lds_t[k][1]) + (lds_t[k][2] + lds_t[k][3]);
        Ttile += T[k];
    }

    double P;
    if (mode == EXSEQ_PLAN_ALL_FALLBACK || mode == EXSEQ_PLAN_FIXED) {
        P = 0.0;  // these modes do not look at the prefix
    } else {
        const uint32_t tl = c0 / CPB;  // tile index within the sum
        uint64_t *st0 = status + a.chunk_base[s] / CPB;
        if (tl == 0) {
            P = init;
        } else {
            if (threadIdx.x == 0)
                store_relaxed_u64(st0 + tl, st_pack(a.epoch, kStAgg, Ttile));
            if (wave == 0) {
                const double p = lookback(st0, tl, init, a.epoch);
                if (lane == 0)
                    lds_p = p;
            }
            __syncthreads();
            P = lds_p;
        }
        if (threadIdx.x == 0)
            store_relaxed_u64(st0 + tl, st_pack(a.epoch, kStIncl, P + Ttile));
    }

    uint32_t key[CPB], key2[CPB];
    bool cross[CPB];
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        key[k] = plan_key(P, a.flags);
        key2[k] = key_of(P + T[k]);
        cross[k] = key2[k] != key_of(P);
        P += T[k];
    }
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        WaveRun w;
        if (key_has_fast_path(key[k])) {
            w = wave_run(f[k], key[k]);
        } else {
            bool nf = false;
#pragma unroll
            for (int i = 0; i < 4; i++)
                nf |= i < f[k].cnt && is_nonfinite(f[k].v[i]);
            w.p = pair_identity();
            w.lo = w.hi = 0;
            w.flags = __ballot(nf) ? kFlagNonFinite : 0u;
        }
        if (lane == 0)
            lds_runs[k][wave] = w;
    }
    __syncthreads();
    if ((int)threadIdx.x < CPB) {
        const int k = threadIdx.x;
        if (c0 + k < nch) {
            uint32_t kk = 0;
            bool cc = false;
#pragma unroll
            for (int j = 0; j < CPB; j++)
                if (j == k) {
                    kk = key[j];
                    cc = cross[j];
                }
            store_desc(d, (size_t)(g0 + k), kk, join_waves(lds_runs[k]), cc);
        }
    }

    // crossing records (see record_prefix)
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        if (!cross[k] || c0 + k >= nch || c0 + k == 0 || !key_has_fast_path(key[k]) ||
            !key_has_fast_path(key2[k]) || ((key[k] ^ key2[k]) & 0x800u) ||
            (join_waves(lds_runs[k]).flags & (kFlagNeg | kFlagBad | kFlagNonFinite)))
            continue;
        if (threadIdx.x == 0)
            lds_slot = (int)atomicAdd(rec.counter, 1u);
        __syncthreads();
        const int slot = lds_slot;
        __syncthreads();  // every lane has read the slot before it is reused
        if (slot < 0 || slot >= (int)a.rec_slots)
            continue;
        int64_t *r = rec.data + (size_t)slot * 2 * kChunk;
        const bool bad1 = record_prefix(f[k], key[k], r, lds_wtot[0], lds_flag[0]);
        const bool bad2 = record_prefix(f[k], key2[k], r + kChunk, lds_wtot[1], lds_flag[1]);
        if (threadIdx.x == 0 && !bad1 && !bad2) {
            const size_t c = (size_t)(g0 + k);
            d.lo[c] = (int64_t)key2[k];
            d.hi[c] = slot;
            d.meta[c] |= kFlagRecord;
        }
    }

    // A sum's first chunk starts from init exactly.  There the running sum
    // is small next to the terms and crosses many binades, which is the
    // worst case of the walk's rounds, so its tile adds it in order on one
    // lane (about 10 ns a term, hidden under the stream of the other tiles)
    // and records the exact sum after it.
    if (c0 == 0) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; i++)
            lds_terms[threadIdx.x * 4 + i] = f[0].v[i];
        __syncthreads();
        if (threadIdx.x == 0) {
            const int len = (int)(n < (size_t)kChunk ? n : (size_t)kChunk);
            d.lo[g0] = (int64_t)dbits(add_in_order(init, lds_terms, 0, len));
            d.meta[g0] |= kFlagExact;
        }
    }
}

// ---------------------------------------------------------------------------
// The walk: one workgroup of 256 lanes per sum; lane t holds 4 consecutive
// items (the chunks of a window of 1024, or the 1024 terms of a chunk being
// resolved).
// ---------------------------------------------------------------------------
constexpr int kPer = 4;
constexpr int kWaves = kWalkThreads / 64;
constexpr int kWindow = kWalkThreads * kPer;  // 1024 chunks or terms
constexpr int kNone = 0x7FFFFFFF;
// A resolve round that adds fewer terms than this counts as short; after two
// short rounds the rest of the chunk goes through one lane in order.
constexpr int kShortRound = 128;

static_assert(kWindow == kChunk, "a window of chunks and a chunk of terms share the layout");

// One wave's candidate for "the first item that needs attention", with what
// the owning lane computed for it.
struct Cand {
    int idx;
    int ok2;        // chunk applies after renormalising (1), misplanned (2)
    double s_at;    // exact sum at the item (or after the item's plain add)
    double s_next;  // exact sum after the chunk when ok2 == 1
    Pair ex_after;  // window prefix through the chunk (a record's second prefix)
    int rec;        // the chunk's crossing record, or -1
    uint32_t key, key2;  // the chunk's planned binade and the record's next one
};

struct WalkLds {
    Pair tot[2][kWaves];   // per-wave totals of a scan (double-buffered)
    Cand cand[2][kWaves];  // per-wave candidates (double-buffered)
    double endv[2];        // a round's end state, from the lane holding the last item
    Pair lastp[2];         // a record's last second-binade prefix
    int flag[2][kWaves];
    double terms[kChunk];  // a chunk's terms, for the one-lane path
};

// Exclusive workgroup scan of the lanes' pairs; one barrier.  Waves without
// a tie scan plain integers (the pair is (v, v)).  `buf` alternates between
// calls so that a call's writes never race with the previous call's reads.
__device__ __forceinline__ Pair block_excl_scan(Pair v, bool lane_tie, WalkLds &sh, int buf)
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
__device__ __forceinline__ bool block_any(bool p, WalkLds &sh, int buf)
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
__device__ __forceinline__ CleanSum block_clean_sum(bool clean, bool nf, int64_t v, WalkLds &sh,
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
__device__ __forceinline__ Cand block_first(bool has, const Cand &mine, WalkLds &sh, int buf)
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
    c.rec = -1;
    c.key = c.key2 = 0u;
    return c;
}

// Exact resolution of one chunk from the exact running sum S.
__device__ double resolve_chunk(const double *__restrict__ x, size_t n, size_t c, double S,
                                int pos, WalkLds &sh, int &buf)
{
    const int t = threadIdx.x;
    const size_t b = c * kChunk;
    const int len = (int)(n - b < (size_t)kChunk ? n - b : (size_t)kChunk);
    const Four f = load_four(x, n, b + (size_t)kPer * t, false);
    double xv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        xv[k] = f.v[k];
        sh.terms[kPer * t + k] = xv[k];  // visible after the next barrier
    }
    int shorts = 0;
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
        if (E == 0u || shorts >= 2) {
            // subnormal S, or the binade keeps changing: the remaining terms
            // one by one on lane 0, in order
            __syncthreads();
            Cand mine = cand_none();
            if (t == 0) {
                mine.idx = 0;
                mine.s_at = add_in_order(S, sh.terms, pos, len);
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
            double xf = xv[0];
#pragma unroll
            for (int k = 1; k < kPer; k++)
                if (k == firstk) {
                    cb = cnt[k - 1];
                    xf = xv[k];
                }
            const int i = kPer * t + firstk;
            mine.idx = i;
            mine.s_at = ((i == pos) ? S : assemble(key, cb)) + xf;  // the one plain add
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
        S = fr.s_at;
        pos = fr.idx + 1;
    }
    return S;
}

// A crossing chunk from its record, given the exact sum S at its start (in
// the chunk's planned binade).  One barrier.  Returns done with the sum
// after the chunk, or not done with the state after the crossing term and
// the position to continue term by term from.
struct RecOut {
    bool done;
    double S;
    int pos;
};

// This lane's share of a record chunk: its terms and packed prefixes (loaded
// ahead of need, so that the resolve does not wait for memory).
struct RecPre {
    Four f;
    int64_t pe[kPer], pe2[kPer], prev;
    int len;
};

__device__ __forceinline__ RecPre rec_load(const double *__restrict__ x, size_t n, size_t c,
                                           const int64_t *__restrict__ rec)
{
    RecPre r;
    const int t = threadIdx.x;
    const size_t b = c * kChunk;
    r.len = (int)(n - b < (size_t)kChunk ? n - b : (size_t)kChunk);
    r.f = load_four(x, n, b + (size_t)kPer * t, false);
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = kPer * t + k;
        r.pe[k] = i < r.len ? rec[i] : 1;
        r.pe2[k] = i < r.len ? rec[kChunk + i] : 1;
    }
    r.prev = t > 0 && kPer * t - 1 < r.len ? rec[kPer * t - 1] : 1;  // 1: packed identity
    return r;
}

__device__ RecOut resolve_with_record(const RecPre &R, double S, uint32_t key2, WalkLds &sh,
                                      int &buf)
{
    const int t = threadIdx.x;
    const int len = R.len;
    const Four &f = R.f;
    const uint32_t key = key_of(S);
    const int64_t m = count_of(S);
    int64_t pe[kPer], pe2[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        pe[k] = R.pe[k];
        pe2[k] = R.pe2[k];
    }
    const int64_t prev = R.prev;
    int64_t cnt[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++)
        cnt[k] = m + pair_at(rec_unpack(pe[k]), m);
    Cand mine = cand_none();
    int firstk = -1;
#pragma unroll
    for (int k = kPer - 1; k >= 0; k--) {
        const int i = kPer * t + k;
        if (i < len && (cnt[k] < kCountLo + 1 || cnt[k] > kCountHi - 1))
            firstk = k;
    }
    if (firstk >= 0) {
        int64_t cb = m + pair_at(rec_unpack(prev), m);
        double xf = f.v[0];
        int64_t p2 = pe2[0];
#pragma unroll
        for (int k = 1; k < kPer; k++)
            if (k == firstk) {
                cb = cnt[k - 1];
                xf = f.v[k];
                p2 = pe2[k];
            }
        const int i = kPer * t + firstk;
        mine.idx = i;
        mine.s_at = ((i == 0) ? S : assemble(key, cb)) + xf;  // the one plain add
        mine.ex_after = rec_unpack(p2);
    }
    if ((len - 1) / kPer == t) {
        const int kl = (len - 1) - kPer * t;
#pragma unroll
        for (int k = 0; k < kPer; k++)
            if (k == kl) {
                sh.endv[buf] = assemble(key, cnt[k]);
                sh.lastp[buf] = rec_unpack(pe2[k]);
            }
    }
    const Cand fr = block_first(firstk >= 0, mine, sh, buf);
    const double endv = sh.endv[buf];
    const Pair lastp = sh.lastp[buf];
    buf ^= 1;
    if (fr.idx == kNone)
        return RecOut{true, endv, len};
    const double s2 = fr.s_at;
    if (fr.idx == len - 1)
        return RecOut{true, s2, len};
    const uint32_t k2 = key_of(s2);
    const int64_t m2 = count_of(s2);
    const Pair at = fr.ex_after;
    int p = -1;
    if ((at.r0 & 1) == (m2 & 1))
        p = 0;
    else if (((1 + at.r1) & 1) == (m2 & 1))
        p = 1;
    if (k2 != key2 || !key_has_fast_path(k2) || p < 0)
        return RecOut{false, s2, fr.idx + 1};
    const int64_t cnt_end = m2 + ((p ? lastp.r1 : lastp.r0) - (p ? at.r1 : at.r0));
    if (cnt_end > kCountHi)
        return RecOut{false, s2, fr.idx + 1};  // a second crossing
    return RecOut{true, assemble(k2, cnt_end), len};
}

__global__ __launch_bounds__(kWalkThreads) void walk_kernel(BatchArgs a, DescArrays dall,
                                                            RecArea rec,
                                                            double *__restrict__ outs,
                                                            exseq_stats *__restrict__ stats)
{
    __shared__ WalkLds sh;
    const int s = blockIdx.x;
    const double *__restrict__ x = a.x[s];
    const size_t n = a.n[s];
    const size_t nch = (n + kChunk - 1) / kChunk;
    const size_t cb = a.chunk_base[s];
    const int64_t *__restrict__ dr0 = dall.r0 + cb;
    const int64_t *__restrict__ dlo_a = dall.lo + cb;
    const int64_t *__restrict__ dhi_a = dall.hi + cb;
    const uint32_t *__restrict__ dmeta = dall.meta + cb;
    const int t = threadIdx.x;
    uint64_t n_fast = 0, n_fb = 0, fb_terms = 0;
    uint32_t misses = 0;
    int64_t first_fb = -1;
    bool nonfinite = false;
    int buf = 0;

    // The first tile left the exact sum after the first chunk.
    double S = a.init[s];
    size_t start = 0;
    if (nch && (dmeta[0] & kFlagExact)) {
        S = bitsd((uint64_t)dlo_a[0]);
        nonfinite |= (dmeta[0] & kFlagNonFinite) != 0;
        start = 1;
        n_fb = 1;
        fb_terms = n < (size_t)kChunk ? n : (size_t)kChunk;
        first_fb = 0;
    }

    // r0 and meta of the first window; each window prefetches the next one
    int64_t nr0[kPer];
    uint32_t nmeta[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const size_t i = start + (size_t)(kPer * t + k);
        nr0[k] = i < nch ? dr0[i] : 0;
        nmeta[k] = i < nch ? dmeta[i] : kFlagBad;
    }
    for (size_t base = start; base < nch; base += kWindow) {
        const int cnt = (int)(nch - base < (size_t)kWindow ? nch - base : kWindow);
        int64_t r0[kPer];
        uint32_t meta[kPer];
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            r0[k] = nr0[k];
            meta[k] = nmeta[k];
            const size_t i = base + kWindow + (size_t)(kPer * t + k);
            nr0[k] = i < nch ? dr0[i] : 0;
            nmeta[k] = i < nch ? dmeta[i] : kFlagBad;
        }
        uint32_t dkey[kPer], dfl[kPer];
        bool drec[kPer];
        Pair mine[kPer];
        bool lane_tie = false, lane_nf = false, lane_clean = true;
        int64_t lane_sum = 0;
        const uint32_t ks0 = key_of(S);
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const bool have = kPer * t + k < cnt;
            dkey[k] = have ? (meta[k] & kKeyMask) : 0u;
            dfl[k] = have ? (meta[k] & (kFlagNeg | kFlagBad | kFlagNonFinite)) : kFlagBad;
            drec[k] = have && (meta[k] & kFlagRecord) != 0;
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
        nonfinite |= cs.nonfinite;
        if (cs.clean && key_has_fast_path(ks0)) {
            const int64_t cnt_end = count_of(S) + cs.sum;
            if (cnt_end <= kCountHi) {
                S = assemble(ks0, cnt_end);
                n_fast += (uint64_t)cnt;
                continue;
            }
        }
        int64_t dlo[kPer], dhi[kPer];
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            dlo[k] = dhi[k] = 0;
            if ((dfl[k] & kFlagNeg) || drec[k]) {
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
            bool frec = false;
            Pair fmine = pair_identity(), fex = pair_identity();
#pragma unroll
            for (int k = kPer - 1; k >= 0; k--) {
                const int i = kPer * t + k;
                if (i >= cur && i < cnt) {
                    const int64_t mt = m + ((p ? ex[k].r1 : ex[k].r0) - base_p);
                    const bool ok = fs && dkey[k] == ks && mt >= kCountLo && mt < kCountHi &&
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
                        frec = drec[k];
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
                mc.key = fkey;
                if (frec) {
                    mc.rec = (int)fhi;
                    mc.key2 = (uint32_t)flo;
                }
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
                n_fast += (uint64_t)(cnt - cur);
                S = fc.s_at;
                break;
            }
            n_fast += (uint64_t)(fc.idx - cur);
            excur = fc.ex_after;
            if (fc.ok2 == 1) {
                S = fc.s_next;
                n_fast++;
            } else {
                misses += fc.ok2 == 2;
                const size_t c = base + (size_t)fc.idx;
                if (fc.rec >= 0 && key_of(fc.s_at) == fc.key) {
                    const RecPre R = rec_load(x, n, c, rec.data + (size_t)fc.rec * 2 * kChunk);
                    const RecOut r = resolve_with_record(R, fc.s_at, fc.key2, sh, buf);
                    S = r.done ? r.S : resolve_chunk(x, n, c, r.S, r.pos, sh, buf);
                } else {
                    S = resolve_chunk(x, n, c, fc.s_at, 0, sh, buf);
                }
                n_fb++;
                fb_terms += (n - c * kChunk < (size_t)kChunk) ? n - c * kChunk : (size_t)kChunk;
                if (first_fb < 0)
                    first_fb = (int64_t)c;
            }
            cur = fc.idx + 1;
        }
    }
    if (t == 0) {
        // the next launch (after this one, in stream order) numbers records from 0
        if (s == 0)
            *rec.counter = 0u;
        outs[s] = S;
        if (stats) {
            exseq_stats st;
            st.chunks = nch;
            st.fast_chunks = n_fast;
            st.fallback_chunks = n_fb;
            st.fallback_terms = fb_terms;
            st.first_fallback = first_fb;
            st.flags = nonfinite ? EXSEQ_STAT_NONFINITE : 0u;
            st.plan_misses = misses;
            stats[s] = st;
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

// ---------------------------------------------------------------------------
// Host-side launch sequences.
// ---------------------------------------------------------------------------
namespace {
std::atomic<uint32_t> g_epoch{0};

// A tag per launch for the look-back status words (16 bits used, never 0,
// so zero-filled memory never matches).
uint32_t next_epoch()
{
    uint32_t e;
    do {
        e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    } while ((e & 0xFFFFu) == 0);
    return e;
}

struct WsParts {
    uint64_t *status;
    DescArrays d;
    RecArea rec;
};

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

WsParts carve(void *ws, size_t total)
{
    char *w = static_cast<char *>(ws);
    WsParts p;
    p.rec.counter = reinterpret_cast<uint32_t *>(w);
    w += 256;
    p.status = reinterpret_cast<uint64_t *>(w);
    w += round256(total * sizeof(uint64_t));
    p.d.r0 = reinterpret_cast<int64_t *>(w);
    w += round256(total * sizeof(int64_t));
    p.d.lo = reinterpret_cast<int64_t *>(w);
    w += round256(total * sizeof(int64_t));
    p.d.hi = reinterpret_cast<int64_t *>(w);
    w += round256(total * sizeof(int64_t));
    p.d.meta = reinterpret_cast<uint32_t *>(w);
    w += round256(total * sizeof(uint32_t));
    p.rec.data = reinterpret_cast<int64_t *>(w);
    return p;
}
}  // namespace

const char *const kPathKernels[] = {"tile_kernel", "walk_kernel"};
const int kPathKernelCount = 2;

// Records a launch may make: about one per binade a sum crosses is needed;
// one slot per 8 chunks (16 to 512) leaves room for mis-planned ones.
size_t rec_slots(size_t total_chunks)
{
    const size_t s = total_chunks / 8;
    return s < 16 ? 16 : (s > 512 ? 512 : s);
}

size_t sum_ws_bytes(size_t total_chunks)
{
    return 256 + 4 * round256(total_chunks * sizeof(int64_t)) +
           round256(total_chunks * sizeof(uint32_t)) +
           rec_slots(total_chunks) * 2 * kChunk * sizeof(int64_t) + 256;
}

template <int CPB>
static void launch_tiles(const BatchArgs &args, uint32_t total, const WsParts &p,
                         hipStream_t stream)
{
    const unsigned tiles = total / CPB;
    if (tiles)
        hipLaunchKernelGGL(tile_kernel<CPB>, dim3(tiles), dim3(kChunkThreads), 0, stream, args,
                           p.status, p.d, p.rec);
}

int launch_batch(const BatchArgs &a, void *ws, double *outs, hipStream_t stream,
                 exseq_stats *stats, void *const *events, int n_events)
{
    auto mark = [&](int i) {
        if (events && i < n_events && events[i])
            hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
    };
    const uint32_t total = a.chunk_base[a.count];  // a multiple of kTileMax
    const WsParts p = carve(ws, total);
    BatchArgs args = a;
    args.epoch = next_epoch();
    args.rec_slots = (uint32_t)rec_slots(total);
    const uint32_t tile = (a.flags >> kTileShift) & 3u;  // 0: default
    mark(0);
    if (tile == 1)
        launch_tiles<1>(args, total, p, stream);
    else if (tile == 2)
        launch_tiles<2>(args, total, p, stream);
    else
        launch_tiles<4>(args, total, p, stream);
    mark(1);
    mark(2);
    hipLaunchKernelGGL(walk_kernel, dim3((unsigned)a.count), dim3(kWalkThreads), 0, stream, args,
                       p.d, p.rec, outs, stats);
    mark(3);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
}

int launch_exact_sum(const double *x, size_t n, double init, double *out, void *ws,
                     hipStream_t stream, uint32_t flags, exseq_stats *stats, void *const *events,
                     int n_events)
{
    BatchArgs a{};
    a.count = 1;
    a.flags = flags;
    a.x[0] = x;
    a.n[0] = n;
    a.init[0] = init;
    a.chunk_base[0] = 0;
    a.chunk_base[1] = (uint32_t)padded_chunks(n);
    return launch_batch(a, ws, out, stream, stats, events, n_events);
}

int launch_tree_sum(const double *x, size_t n, double *out, void *ws, hipStream_t stream)
{
    if (n == 0) {
        hipLaunchKernelGGL(write_value_kernel, dim3(1), dim3(1), 0, stream, out, 0.0);
        return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
    }
    const size_t nch = (n + kChunk - 1) / kChunk;
    double *tsum = static_cast<double *>(ws);
    hipLaunchKernelGGL(chunk_tsum_kernel, dim3((unsigned)nch), dim3(kChunkThreads), 0, stream, x,
                       n, tsum);
    hipLaunchKernelGGL(tree_total_kernel, dim3(1), dim3(kPlanThreads), 0, stream, tsum, nch, out);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
}

}  // namespace exseq
