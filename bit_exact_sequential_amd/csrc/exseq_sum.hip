// gfx950 kernels of the exact sequential fp64 sum and of the fixed-tree sum.
//
// The path (Research-1433 "Forming the CPU's sequential double sums on a GPU,
// bit for bit", Findings 2-6; Research-1424 "integer_ssim_cuda and the CPU's
// frame sum", Findings 3).  A chunk is 1024 consecutive terms, held by 256
// lanes (4 waves of 64) with 4 consecutive terms per lane.
//
//  A launch of at most 8 chunks runs walk_kernel alone (every chunk term by
//  term from init, in order).  Otherwise:
//  chain_clear_kernel: zeroes the chain words and step records of the
//  launch's tiles.
//  tile_kernel (one launch for every tile of every sum of a batch; reads
//  each term once).  Blocks: each sum's last tile, each sum's head (its
//  first chunk added to init term by term), then the other tiles in order
//  (the tiles of interleaved sums for one range together), one workgroup
//  per tile of CPB consecutive chunks of one sum (1, 2 or 4, by the
//  launch's size):
//    1. load the tile's terms (contiguous: 16-byte non-temporal loads;
//       interleaved: every k-th double; SSIM: formed from the two planes),
//       fixed-tree fp64 sum of every chunk;
//    2. the plan: publish the tile's sum, find the prefix of the chunk sums
//       before the tile by a decoupled look-back over the predecessors'
//       status words, publish the inclusive prefix; a chunk's planned binade
//       is that of the prefix before it (or, with a plan kept from the
//       previous call and far from a binade edge, that plan's binade, with
//       no look-back);
//    3. every term's increment pair under its chunk's planned binade,
//       composed in order (lane, ordered wave scan, waves in order) into the
//       chunk's run: the pair, prefix bounds, flags;
//    4. the exact chain.  A tile whose chunks all share one planned binade
//       and stay clear of its edges (with a margin for the plan's error) is
//       regular: it publishes the composition of its runs and is done.  Any
//       other tile (a sum's first and last tile among them) locates the
//       crossing of every chunk planned to cross into the next binade up or
//       down, composes the regular tiles back to the nearest irregular one,
//       publishes its own O(1) step as a record, waits for that tile's exact
//       sum (the first tile: the head's) or catches up to it through the
//       records of the irregular tiles before, applies the composed runs and
//       its own chunks in order -- a run where it applies, a crossing where
//       it holds, term by term from the exact sum where neither does -- and
//       publishes the exact sum after itself.  The last tile's value is the
//       result.
//  walk_kernel (one workgroup of 256 lanes per sum, after the tiles):
//    5. takes the last tile's exact sum.  Where the chain could not finish
//       (a wait that timed out, a composed run that did not apply), it
//       resumes from the last exact sum the chain published and follows the
//       remaining chunks in order, a window of 1024 chunks at a time: a
//       clean window (every chunk in the running sum's binade, no tie,
//       nothing negative or bad) is applied from the sum of its increments;
//       otherwise one scan gives every chunk's start count, every chunk is
//       checked at its exact start, and the first one that fails is added
//       term by term from the exact sum;
//    6. term by term means: every lane forms its terms' increments in the
//       current binade, a workgroup scan gives every prefix count, the first
//       term that leaves the binade is added with one fp64 add, and the next
//       round starts after it; when rounds keep resolving only a few terms,
//       one lane adds the rest in order;
//    7. writes each sum (and the float means of interleaved sums, the SSIM
//       weight sum) and, when asked, keeps the plan for the next call.
//
// Every wait is bounded: a plan wait that times out gives up the tile's
// plan (no fast path for its chunks), a chain wait that times out reports
// failure to the tiles after it and leaves the rest to the walk.  Neither a
// plan nor the chain ever changes a result, only where and how much is added
// term by term.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <stdint.h>

#include "exseq.h"
#include "exseq_internal.h"
#include "exseq_rules.h"
#include "exseq_ssim_dev.h"
#include "exseq_wave.h"
#include "exseq_dev.h"

// The diagnostic build (-DEXSEQ_TIMELINE, libexseq_timeline.so) records the
// 100 MHz real-time counter at the steps of the exact chain's tiles, for the
// host to read back (exseq_timeline_read): per tile, words 0-9 of its 12 are
// its start, its plan, its runs, its record (regular) or its look-back
// (irregular), 1 for an irregular tile, the look-back's end, the exact sum's
// arrival, its own exact sum, and its last crossing search's start and end;
// then two words per sum for its head.  Tiles past the array are not
// recorded.  The product build compiles every stamp away.
#ifdef EXSEQ_TIMELINE
namespace exseq {
constexpr uint32_t kTlTiles = 16384;
constexpr uint32_t kTlPer = 12;
constexpr uint32_t kTlWords = kTlPer * kTlTiles + 2 * kMaxBatch;
__device__ uint64_t exseq_timeline[kTlWords];
}  // namespace exseq
#define EXSEQ_TL(tile, slot, v)                                                   \
    do {                                                                           \
        if (threadIdx.x == 0 && (uint32_t)(tile) < kTlTiles)                       \
            exseq_timeline[kTlPer * (uint32_t)(tile) + (slot)] = (v);              \
    } while (0)
#define EXSEQ_TL_HEAD(s, slot)                                                    \
    do {                                                                           \
        if (threadIdx.x == 0 && (uint32_t)(s) < (uint32_t)kMaxBatch)               \
            exseq_timeline[kTlPer * kTlTiles + 2 * (uint32_t)(s) + (slot)] =       \
                __builtin_amdgcn_s_memrealtime();                                  \
    } while (0)
#define EXSEQ_TL_NOW() __builtin_amdgcn_s_memrealtime()
#else
#define EXSEQ_TL(tile, slot, v) \
    do {                        \
    } while (0)
#define EXSEQ_TL_HEAD(s, slot) \
    do {                       \
    } while (0)
#endif

namespace exseq {


// Fixed-tree sum of every chunk (the tree sum beside the exact one).
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

// What the waves of a tile hand each other.
template <int CPB>
struct TileLds {
    double wsum[CPB][kWaves];    // per-wave fixed-tree chunk sums
    WaveRun wrun[CPB][kWaves];   // per-wave parts of the chunk runs
    WaveRun join[CPB];           // the chunk runs
    double pk[CPB];              // planned prefix before each chunk
    uint32_t key[CPB];           // planned binade of each chunk (0: none)
    uint32_t cross[CPB];         // the plan does not keep the chunk in its binade
    uint32_t down[CPB];          // ... and takes it into the binade below (same sign)
    uint64_t xw[CPB][kCrossWords];  // located crossings
    uint64_t word;               // a word read by one lane for all
    uint32_t reused;             // the tile took its binade from a kept plan
};

// One workgroup per tile of CPB consecutive chunks of one sum.  With the
// chain on, each sum's last tile comes first (blocks 0 .. count-1): started
// early, it has composed the tiles before it by the time they are done, and
// nothing waits on it.  Then one head block per sum (count .. 2 count - 1)
// adds the sum's first chunk to init term by term -- there the running sum
// is small next to the terms and crosses binade after binade, the slowest
// part of any chain -- while the tiles stream.  The other tiles follow in
// order.
template <int CPB, class Src>
__global__ __launch_bounds__(kChunkThreads) void tile_kernel(BatchArgs a, Src src,
                                                             uint64_t *__restrict__ status,
                                                             DescArrays d, ChainArea ch)
{
    __shared__ TileLds<CPB> L;
    __shared__ WalkLds sh;
    __shared__ ChainLds cl;
    __shared__ CrossLds xl;
    __shared__ __attribute__((aligned(16))) int lds_src[Src::kLdsInts];
    const bool chain = chain_on(a.flags);
    uint32_t gt = blockIdx.x;  // this block's tile
    if (chain) {
        if (gt < (uint32_t)a.count) {
            gt = a.last_tile[gt];
            if (gt == ~0u)
                return;
        } else if (gt < 2u * (uint32_t)a.count) {
            EXSEQ_TL_HEAD(gt - (uint32_t)a.count, 0);
            chain_head(src, a, (int)(gt - (uint32_t)a.count), ch, d, sh, lds_src);
            EXSEQ_TL_HEAD(gt - (uint32_t)a.count, 1);
            return;
        } else {
            const uint32_t r = gt - 2u * (uint32_t)a.count;
            int lo = 0;
            uint32_t q;
            if (a.interleave) {
                // sums of one length: groups of 8 tiles of every sum in
                // turn, so that tile q of each sum lands on the same XCD
                // (blocks go round robin over the 8) close in time
                const uint32_t per = a.rest_base[1];  // other tiles per sum
                const uint32_t g = 8u * (uint32_t)a.count;
                const uint32_t Q = r / g, rem = r - Q * g, full = per / 8u;
                const uint32_t G = Q < full ? 8u : per - 8u * full;
                lo = (int)(rem / G);
                q = 8u * Q + rem % G;
            } else {
                int hi = a.count - 1;  // the first sum with rest_base[s + 1] > r
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (a.rest_base[mid + 1] > r)
                        hi = mid;
                    else
                        lo = mid + 1;
                }
                q = r - a.rest_base[lo];
            }
            const uint32_t first = a.chunk_base[lo] / CPB;
            gt = first + (q < a.last_tile[lo] - first ? q : q + 1);
        }
    }
    const uint32_t g0 = gt * CPB;  // first global chunk of the tile
    const int s = find_sum(a, g0);
    const size_t n = a.n[s];
    const uint32_t c0 = g0 - a.chunk_base[s];  // first local chunk
    const uint32_t nch = (uint32_t)((n + kChunk - 1) / kChunk);
    if (c0 >= nch)
        return;  // padding after the sum's last chunk
    const uint32_t mode = a.flags & EXSEQ_PLAN_MASK;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    const uint32_t tl = c0 / CPB;               // tile index within the sum
    EXSEQ_TL(gt, 0, EXSEQ_TL_NOW());
    const uint32_t tb = a.chunk_base[s] / CPB;  // the sum's first tile in the launch
    // A sum's first tile heads the exact chain: its waves go first in the
    // instruction arbitration of their SIMDs, ahead of streaming tiles.
    if (c0 == 0 && chain)
        __builtin_amdgcn_s_setprio(3);
    // A kept plan (EXSEQ_PLAN_REUSE) for a tile between the sum's first and
    // last: its tag and the prefixes around the tile, read with the terms.
    const bool try_reuse = CPB == kTileMax && a.plan_sig != 0 && tl != 0 && c0 + CPB < nch;
    uint64_t phdr = 0;
    double pa = 0.0, pb = 0.0;
    if (try_reuse && wave == 0) {
        phdr = ch.plan_hdr[s];
        pa = ch.plan[gt];
        pb = ch.plan[gt + 1];
    }

    // ---- the terms, and the fixed-tree sum of each chunk
    Four f[CPB];
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        f[k] = src.chunk(a, s, c0 + k, lds_src);
        src.keep(c0 + k, f[k]);
    }
    {
        double ws[CPB];
#pragma unroll
        for (int k = 0; k < CPB; k++)
            ws[k] = (f[k].v[0] + f[k].v[1]) + (f[k].v[2] + f[k].v[3]);
        wave_sum_f64_n<CPB>(ws);
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < CPB; k++)
                L.wsum[k][wave] = ws[k];
        }
    }
    __syncthreads();

    // ---- the plan (wave 0): the prefix before the tile by look-back, then
    // lane k < CPB plans chunk k
    if (wave == 0) {
        double T[CPB];
        double Ttile = 0.0;
#pragma unroll
        for (int k = 0; k < CPB; k++) {
            T[k] = (L.wsum[k][0] + L.wsum[k][1]) + (L.wsum[k][2] + L.wsum[k][3]);
            Ttile += T[k];
        }
        double P = 0.0;  // the fallback and fixed-binade modes do not look at it
        uint32_t rkey = 0u;  // the binade a kept plan gives every chunk (0: none)
        if (mode != EXSEQ_PLAN_ALL_FALLBACK && mode != EXSEQ_PLAN_FIXED) {
            uint64_t *st0 = status + tb;
            if (try_reuse && phdr == a.plan_sig)
                rkey = reuse_key(pa, pb);
            if (tl == 0) {
                P = a.init[s];
            } else {
                if (lane == 0)
                    store_relaxed_u64(st0 + tl, st_pack(a.epoch, kStAgg, Ttile));
                // with a kept binade, the tiles after this one look back past
                // it to the nearest inclusive prefix
                P = rkey ? pa : lookback(st0, tl, a.init[s], a.epoch);
            }
            if (lane == 0 && !rkey)
                store_relaxed_u64(st0 + tl, st_pack(a.epoch, kStIncl, P + Ttile));
        }
        if (lane == 0)
            L.reused = rkey;
        if (lane < CPB) {
            double pk = P, tk = T[0];
#pragma unroll
            for (int k = 0; k < CPB - 1; k++) {
                if (k < lane)
                    pk += T[k];
                if (k + 1 == lane)
                    tk = T[k + 1];
            }
            L.pk[lane] = pk;
            L.key[lane] = rkey ? rkey : plan_key(pk, a.flags);
            L.cross[lane] = !rkey && key_of(pk + tk) != key_of(pk);
            L.down[lane] = ((key_of(pk + tk) ^ key_of(pk)) & 0x800u) == 0u &&
                           (key_of(pk + tk) & 0x7FFu) < (key_of(pk) & 0x7FFu);
        }
    }
    __syncthreads();

    EXSEQ_TL(gt, 1, EXSEQ_TL_NOW());
    // ---- every chunk's run under its planned binade
    uint32_t key[CPB];
    bool allfast = true;
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        key[k] = L.key[k];
        allfast &= key_has_fast_path(key[k]);
    }
    if (allfast) {
        wave_runs<CPB>(f, key, L.wrun);
    } else {
#pragma unroll
        for (int k = 0; k < CPB; k++) {
            WaveRun w;
            if (key_has_fast_path(key[k])) {
                w = wave_run(f[k], key[k]);
            } else {
                bool nf = false;
#pragma unroll
                for (int i = 0; i < 4; i++)
                    nf |= is_nonfinite(f[k].v[i]);
                w.p = pair_identity();
                w.lo = w.hi = 0;
                w.flags = __ballot(nf) ? kFlagNonFinite : 0u;
            }
            if (lane == 0)
                L.wrun[k][wave] = w;
        }
    }
    __syncthreads();
    // Each chunk's run is joined, clamped and checked against the edges of
    // its binade once, by lane k for chunk k, which also stores the chunk's
    // descriptor; the rest of the tile reads the result from LDS.
    if (t < CPB) {
        const uint32_t kk = L.key[t];
        const double pk = L.pk[t];
        bool cc = L.cross[t] != 0;
        // the waves' parts in order; parts that are all tie-free and
        // without a negative term (nearly always) just add up
        bool plain = true, fall = true;
        int64_t sum = 0;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const WaveRun &q = L.wrun[t][w];
            plain &= rising_run(q.p, q.flags);
            fall &= falling_run(q.p, q.lo, q.hi, q.flags);
            sum += q.p.r0;
        }
        const WaveRun r =
            clamp_run(plain ? WaveRun{Pair{sum, sum}, 0, sum, 0u}
                            : fall ? WaveRun{Pair{sum, sum}, sum, 0, kFlagNeg} : join_waves(L.wrun[t]));
        // near an edge of the planned binade: the plan is not trusted there
        if (key_has_fast_path(kk) && kk == key_of(pk)) {
            const int64_t m = count_of(pk);
            const int64_t mg = plan_margin(c0 + t + 1);
            bool near = m < count_floor(kk) + mg;
            if (r.flags & kFlagNeg)
                near |= m + r.lo - mg < kCountLo + 1 || m + r.hi + mg > kCountHi - 1;
            else
                near |= m + r.hi + mg > kCountHi;
            cc |= near;
        }
        L.join[t] = r;
        L.cross[t] = cc;
        if (c0 + t < nch)
            store_desc(d, (size_t)(g0 + t), kk, r, cc ? kFlagCross : 0u);
    }
    __syncthreads();

    if (!chain) {
        // A sum's first chunk starts from init exactly.  There the running
        // sum is small next to the terms and crosses many binades, the worst
        // case of the walk's rounds, so its tile adds it in order and records
        // the exact sum after it.
        if (c0 == 0) {
            const int len = (int)(n < (size_t)kChunk ? n : (size_t)kChunk);
            int buf = 0;
            const double e = resolve_terms(f[0], len, a.init[s], 0, sh, buf);
            if (t == 0) {
                d.lo[g0] = (int64_t)dbits(e);
                d.meta[g0] |= kFlagExact;
            }
        }
        return;
    }

    EXSEQ_TL(gt, 2, EXSEQ_TL_NOW());
    // ---- the exact chain ----------------------------------------------------
    uint64_t *agg = ch.agg + 4 * (size_t)(tb + tl);
    bool regular = c0 != 0 && c0 + CPB < nch;
#pragma unroll
    for (int k = 0; k < CPB; k++)
        regular &= key_has_fast_path(key[k]) && key[k] == key[0] && !L.cross[k] &&
                   !(L.join[k].flags & (kFlagBad | kFlagNonFinite));
    if (regular) {
        if (t == 0) {
            // the chunks' runs in order (plain ones add up)
            bool plain = true, fall = true;
            int64_t sum = 0;
#pragma unroll
            for (int k = 0; k < CPB; k++) {
                const WaveRun &q = L.join[k];
                plain &= rising_run(q.p, q.flags);
                fall &= falling_run(q.p, q.lo, q.hi, q.flags);
                sum += q.p.r0;
            }
            Run tr = run_identity();
            if (plain) {
                tr = Run{Pair{sum, sum}, 0, sum, 0u};
            } else if (fall) {
                tr = Run{Pair{sum, sum}, sum, 0, kFlagNeg};
            } else {
#pragma unroll
                for (int k = 0; k < CPB; k++) {
                    const WaveRun r = L.join[k];
                    tr = run_compose_sat(tr, Run{r.p, r.lo, r.hi, r.flags});
                }
            }
            const int64_t dr = tr.p.r1 - tr.p.r0;
            store_relaxed_u64(agg + 1, enc_i64(tr.p.r0));
            store_relaxed_u64(agg + 2, enc_i64(tr.lo));
            store_relaxed_u64(agg + 3, enc_i64(tr.hi));
            store_relaxed_u64(agg + 0, kAggPresent | kAggRegular | (uint64_t)(key[0] & kKeyMask) |
                                           ((uint64_t)(dr + 1) << kDrShift) |
                                           (uint64_t)(tr.flags & kFlagNeg));
        }
        EXSEQ_TL(gt, 3, EXSEQ_TL_NOW());
        return;
    }
    EXSEQ_TL(gt, 4, 1);
    // An irregular tile: located crossings, the composed run of the regular
    // tiles back to the nearest irregular one, that tile's exact sum, then
    // this tile's chunks in order from it.
    if (t == 0)
        store_relaxed_u64(agg, kAggPresent);
    // The chain is the critical path: this tile's waves go first in the
    // instruction arbitration of their SIMDs, ahead of streaming tiles.
    __builtin_amdgcn_s_setprio(3);
    int buf = 0;
    const int nk = (int)(nch - c0 < (uint32_t)CPB ? nch - c0 : (uint32_t)CPB);
    // Crossings: every chunk expected to cross into the next binade up in
    // magnitude, with a plan for its binade and no non-finite term, gets one
    // located -- except in a sum's first tile, which has the exact sum before
    // its chunks early (the head's) and adds such chunks by the rounds of the
    // resolve instead.  (A run clamped for spanning more than its binade is
    // no obstacle: the crossing's own checks cover each binade.)  A negative
    // running sum is the mirror image: round to nearest even is symmetric in
    // sign, the plan's sign bit mirrors every term (term_inc), and key + 1 is
    // the next binade of the same sign.
    uint32_t want = 0u;
#pragma unroll
    for (int k = 0; k < CPB; k++) {
        const uint32_t fl = L.join[k].flags;
        if (k < nk && c0 != 0 && !L.reused && L.cross[k] && key_has_fast_path(key[k]) &&
            key[k] == key_of(L.pk[k]) &&
            key_has_fast_path(L.down[k] ? key[k] - 1u : key[k] + 1u) &&
            !(fl & kFlagNonFinite))
            want |= 1u << k;
    }
    uint32_t found = 0u;
#pragma unroll 1
    for (int k = 0; k < CPB; k++) {
        if (!((want >> k) & 1u))
            continue;
        // the terms again (from cache, most likely): irregular tiles are few,
        // and not keeping every chunk's terms in registers this far keeps
        // the register count of all tiles down
        EXSEQ_TL(gt, 8, EXSEQ_TL_NOW());
        const Four fr = src.chunk(a, s, c0 + k, lds_src);
        const size_t b = (size_t)(c0 + k) * kChunk;
        const int len = (int)(n - b < (size_t)kChunk ? n - b : (size_t)kChunk);
        uint64_t w[kCrossWords];
        if (crossing_find(fr, len, L.key[k], count_of(L.pk[k]), L.down[k] != 0u, sh, xl, buf, w)) {
            found |= 1u << k;
            EXSEQ_TL(gt, 9, EXSEQ_TL_NOW());
            if (t == 0) {
#pragma unroll
                for (int i = 0; i < kCrossWords; i++)
                    L.xw[k][i] = w[i];
            }
        }
    }

    __syncthreads();  // L.xw is complete
    // Everything the chain applies, one 64-bit word per lane (the bank):
    // lane 4 + 10k + i holds word i of chunk k -- meta (key, r1 - r0 + 1,
    // flags, crossing located), r0, lo, hi, then the crossing's words -- so
    // that from the exact sum on every step reads its operands with
    // readlane straight into scalar registers, with no LDS round trip.
    uint64_t bank = 0;
    {
        const int k = (lane - 4) / kIrrPer, i = (lane - 4) - kIrrPer * ((lane - 4) / kIrrPer);
        if (lane >= 4 && k < CPB) {
            const WaveRun r = L.join[k];
            if (i == 0)
                bank = (uint64_t)(L.key[k] & kKeyMask) |
                       ((uint64_t)(r.p.r1 - r.p.r0 + 1) << kDrShift) |
                       (uint64_t)(r.flags & (kFlagNeg | kFlagBad | kFlagNonFinite)) |
                       (((found >> k) & 1u) ? kIrrCross : 0ULL) |
                       (((found >> k) & 1u) && L.down[k] ? kIrrDown : 0ULL);
            else if (i == 1)
                bank = (uint64_t)r.p.r0;
            else if (i == 2)
                bank = (uint64_t)r.lo;
            else if (i == 3)
                bank = (uint64_t)r.hi;
            else
                bank = L.xw[k][i - 4];
        }
    }

    // The exact sum before the tile's first chunk that it adds itself: after
    // the nearest irregular tile before it and the regular tiles in between
    // (R), or, in a sum's first tile, after the first chunk (the head's).
    double S = a.init[s];
    bool ok = true;
    bool done = false;  // the tile's chunks are applied too
    const int kfirst = c0 == 0 ? 1 : 0;
    {
        Run acc = run_identity();
        uint32_t key0 = 0u;
        int64_t xp = -1;
        int st = kBackOk;
        if (c0 != 0) {
            EXSEQ_TL(gt, 3, EXSEQ_TL_NOW());
            st = chain_back(ch, tb, tl, sh, cl, buf, acc, key0, xp);
            EXSEQ_TL(gt, 5, EXSEQ_TL_NOW());
            if ((a.flags & EXSEQ_CHAIN_CUT) && tl >= ((nch + CPB - 1) / CPB) / 2 && st == kBackOk)
                st = kBackBad;  // a test hook: the chain stops here
        }
        ok = st == kBackOk;
        // R as scalars
        const bool rnone = c0 == 0 || xp == (int64_t)tl - 1;
        const Run R{Pair{readlane_i64(acc.p.r0, 0), readlane_i64(acc.p.r1, 0)},
                    readlane_i64(acc.lo, 0), readlane_i64(acc.hi, 0),
                    (uint32_t)__builtin_amdgcn_readfirstlane(
                        (int)(acc.flags & (kFlagNeg | kFlagBad | kFlagNonFinite)))};
        const uint32_t rkey = (uint32_t)__builtin_amdgcn_readfirstlane((int)key0);
        // While the exact sum is on its way: the whole tile as few steps as
        // its shape allows -- R and the chunks before the located crossing
        // (all in one binade) composed into one run A, then the crossing,
        // whose rest-of-chunk run takes in the chunks after it (all in the
        // next binade; under negative terms with its prefix bounds).  Any
        // other shape, or any step that does not hold for the exact sum,
        // goes chunk by chunk below.
        bool fast = ok;
        Run A = R;
        uint32_t akey = rnone ? 0u : rkey;
        int kx = nk;  // the crossing chunk (nk: none)
        uint64_t xw[kCrossWords];
#pragma unroll
        for (int i = 0; i < kCrossWords; i++)
            xw[i] = 0;
        for (int k = kfirst; fast && k < nk; k++) {
            const int base = 4 + kIrrPer * k;
            const uint64_t cm = (uint64_t)readlane_i64((int64_t)bank, base);
            const uint32_t kk = (uint32_t)cm & kKeyMask;
            if (cm & kIrrCross) {
                kx = k;
                break;
            }
            const int64_t r0 = readlane_i64((int64_t)bank, base + 1);
            const Run rk{Pair{r0, r0 + (int64_t)((cm >> kDrShift) & 3u) - 1},
                         readlane_i64((int64_t)bank, base + 2), readlane_i64((int64_t)bank, base + 3),
                         (uint32_t)cm & (kFlagNeg | kFlagBad | kFlagNonFinite)};
            fast = key_has_fast_path(kk) && !(rk.flags & (kFlagBad | kFlagNonFinite)) &&
                   (akey == 0u || akey == kk);
            A = run_compose_sat(A, rk);
            akey = kk;
        }
        uint32_t xkey = 0u;
        uint32_t xfl = 0u;  // kFlagNeg: a negative term in the crossing or after it
        bool xdown = false;  // the crossing goes into the binade below
        if (fast && kx < nk) {
            const int base = 4 + kIrrPer * kx;
            const uint64_t xm = (uint64_t)readlane_i64((int64_t)bank, base);
            xkey = (uint32_t)xm & kKeyMask;
#pragma unroll
            for (int i = 0; i < kCrossWords; i++)
                xw[i] = (uint64_t)readlane_i64((int64_t)bank, base + 4 + i);
            xfl = (uint32_t)xm & kFlagNeg;
            xdown = (xm & kIrrDown) != 0;
            fast = akey == 0u || akey == xkey;
            // the chunks after the crossing (all in the next binade) folded
            // into its rest-of-chunk run, bounds and all, so that a negative
            // term anywhere is checked as the crossing's own are
            Run suf{rec_unpack(dec_i64(xw[kXsuf])), dec_i64(xw[kXsufLo]), dec_i64(xw[kXsufHi]), xfl};
            Pair whole = rec_unpack(dec_i64(xw[kXwhole]));
            for (int k = kx + 1; fast && k < nk; k++) {
                const int b2 = 4 + kIrrPer * k;
                const uint64_t cm = (uint64_t)readlane_i64((int64_t)bank, b2);
                const int64_t r0 = readlane_i64((int64_t)bank, b2 + 1);
                fast = ((uint32_t)cm & kKeyMask) == (xdown ? xkey - 1u : xkey + 1u) &&
                       !(cm & kIrrCross) &&
                       !((uint32_t)cm & (kFlagBad | kFlagNonFinite));
                const Run q{Pair{r0, r0 + (int64_t)((cm >> kDrShift) & 3u) - 1},
                            readlane_i64((int64_t)bank, b2 + 2), readlane_i64((int64_t)bank, b2 + 3),
                            (uint32_t)cm & kFlagNeg};
                suf = run_compose_sat(suf, q);
                whole = compose(whole, q.p);
                xfl |= (uint32_t)cm & kFlagNeg;
            }
            const int64_t lim = (int64_t)1 << 56;
            fast = fast && !(suf.flags & kFlagBad) && whole.r0 < lim && whole.r1 < lim &&
                   whole.r0 > -lim && whole.r1 > -lim;
            xw[kXsuf] = enc_i64(rec_pack(suf.p));
            xw[kXsufLo] = enc_i64(suf.lo);
            xw[kXsufHi] = enc_i64(suf.hi);
            xw[kXwhole] = enc_i64(rec_pack(whole));
        }
        const int xlen = kx < nk ? (int)(n - (size_t)(c0 + kx) * kChunk < (size_t)kChunk
                                             ? n - (size_t)(c0 + kx) * kChunk
                                             : (size_t)kChunk)
                                 : 0;
        // the tile's step, for the tiles after it that catch up through it
        if (ok && fast && c0 != 0 && wave == 0 && lane < kRecWords)
            store_relaxed_u64(ch.rec + kRecWords * (size_t)(tb + tl) + lane,
                              rec_word(lane, akey, A, kx < nk, xw, xlen, xkey, xfl, xdown, xp));
        if (ok) {
            // every wave waits on its own (no barrier between the word
            // arriving and the steps that use it)
            uint64_t w = 0;
            if (c0 == 0) {
                if (lane == 0) {
                    const uint64_t *p = ch.head + s;
                    w = load_relaxed_u64(p);
                    for (int spin = 0; w == 0 && spin <= kSpinLimit; spin++)
                        w = load_relaxed_u64(p);
                }
                w = uniform_u64(w);
            } else {
                // one wave waits and catches up (its loop is not cheap, and
                // more waves of it would take issue slots from the streaming
                // tiles on the same compute unit); the rest wait at a barrier
                w = uniform_u64(catch_up(ch, tb, xp, wave == 0));
            }
            ok = w > kInclFailed;  // 0: the wait timed out
            EXSEQ_TL(gt, 6, EXSEQ_TL_NOW());
            if (ok)
                S = bitsd(w ^ kInclXor);
            if (ok && fast && tile_step(akey, A, kx < nk, xw, xlen, xkey, xfl, xdown, S))
                done = true;
            if (ok && !done && !rnone) {
                const uint32_t ks = key_of(S);
                const int64_t mm = count_of(S);
                ok = ks == rkey && key_has_fast_path(ks) &&
                     run_applies(mm, R.p, R.lo, R.hi, R.flags);
                if (ok)
                    S = assemble(ks, mm + pair_at(R.p, mm));
            }
        }
    }
    // This tile's chunks in order: each chunk's run where it applies from
    // the exact sum, else its crossing, else term by term.
    uint32_t resolved = c0 == 0 ? 1u : 0u;  // the head adds the first chunk term by term
    if (ok && !done) {
#pragma unroll 1
        for (int k = kfirst; k < nk; k++) {
            const size_t b = (size_t)(c0 + k) * kChunk;
            const int len = (int)(n - b < (size_t)kChunk ? n - b : (size_t)kChunk);
            int pos = 0;
            {
                const int base = 4 + kIrrPer * k;
                const uint64_t cm = (uint64_t)readlane_i64((int64_t)bank, base);
                const uint32_t kk = (uint32_t)cm & kKeyMask;
                const int64_t r0 = readlane_i64((int64_t)bank, base + 1);
                const Pair rp{r0, r0 + (int64_t)((cm >> kDrShift) & 3u) - 1};
                const uint32_t ks = key_of(S);
                const int64_t mm = count_of(S);
                if (key_has_fast_path(ks) && ks == kk &&
                    run_applies(mm, rp, readlane_i64((int64_t)bank, base + 2),
                                readlane_i64((int64_t)bank, base + 3),
                                (uint32_t)cm & (kFlagNeg | kFlagBad | kFlagNonFinite))) {
                    S = assemble(ks, mm + pair_at(rp, mm));
                    continue;
                }
                int xr = 0;
                if (cm & kIrrCross) {
                    uint64_t xw[kCrossWords];
#pragma unroll
                    for (int i = 0; i < kCrossWords; i++)
                        xw[i] = (uint64_t)readlane_i64((int64_t)bank, base + 4 + i);
                    xr = crossing_apply(xw, len, kk, (uint32_t)cm, (cm & kIrrDown) != 0, S, pos);
                    S = bitsd(uniform_u64(dbits(S)));
                }
                if (xr == 1)
                    continue;
                if (xr == 0)
                    pos = 0;
            }
            S = resolve_terms(src.chunk(a, s, c0 + k, lds_src), len, S, pos, sh, buf);
            S = bitsd(uniform_u64(dbits(S)));
            resolved |= 1u << k;
        }
    }
    if (t == 0) {
        store_relaxed_u64(ch.incl + tb + tl, ok ? enc_sum(S) : kInclFailed);
        EXSEQ_TL(gt, 7, EXSEQ_TL_NOW());
#pragma unroll
        for (int k = 0; k < CPB; k++)
            if ((resolved >> k) & 1u)
                d.meta[g0 + k] |= kFlagResolved;
    }
}

// The plan kept for the next launch (EXSEQ_PLAN_REUSE): the planned prefix
// before every tile of sum s, from this launch's status words -- the
// inclusive prefix where a tile published one, else the previous prefix plus
// the tile's own sum -- then the launch's tag.  Lane t takes a contiguous
// run of tiles; the runs' (restart, sum) pairs are scanned across the
// workgroup in order.
struct PlanLds {
    double v[kWaves];
    int r[kWaves];
};
constexpr int kPlanGroup = 8;  // status words a lane holds at once
__device__ void keep_plan(const BatchArgs &a, const uint64_t *status, const ChainArea &ch, int s,
                          PlanLds &pl)
{
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    const size_t n = a.n[s];
    const uint32_t nt = (uint32_t)((n + kChunk * kTileMax - 1) / (kChunk * kTileMax));
    const uint32_t tb = a.chunk_base[s] / kTileMax;
    const uint32_t per = (nt + kWalkThreads - 1) / kWalkThreads;
    const uint32_t j0 = (uint32_t)t * per < nt ? (uint32_t)t * per : nt;
    const uint32_t j1 = j0 + per < nt ? j0 + per : nt;
    // this lane's run: r set if it holds an inclusive prefix (v is then the
    // prefix after the run), else v adds to the prefix before it; the status
    // words are read kPlanGroup at a time, all in flight together
    int r = 0;
    double v = 0.0;
    for (uint32_t g = j0; g < j1; g += kPlanGroup) {
        uint64_t w[kPlanGroup];
#pragma unroll
        for (int i = 0; i < kPlanGroup; i++)
            w[i] = g + i < j1 ? status[tb + g + i] : 0;
#pragma unroll
        for (int i = 0; i < kPlanGroup; i++) {
            const uint64_t fl = st_flag(w[i], a.epoch);
            if (fl == kStIncl) {
                r = 1;
                v = st_value(w[i]);
            } else if (fl == kStAgg) {
                v += st_value(w[i]);
            }
        }
    }
    // inclusive scan in order: (r1, v1) then (r2, v2) is r2 ? (1, v2) : (r1, v1 + v2)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double vu = __shfl_up(v, off);
        const int ru = __shfl_up(r, off);
        if (lane >= off && !r) {
            r = ru;
            v += vu;
        }
    }
    if (lane == 63) {
        pl.v[wave] = v;
        pl.r[wave] = r;
    }
    __syncthreads();
    double P = a.init[s];  // the prefix before this wave: init, then the waves before
    for (int k = 0; k < wave; k++)
        P = pl.r[k] ? pl.v[k] : P + pl.v[k];
    const double vu = __shfl_up(v, 1);
    const int ru = __shfl_up(r, 1);
    if (lane > 0)
        P = ru ? vu : P + vu;
    for (uint32_t g = j0; g < j1; g += kPlanGroup) {
        uint64_t w[kPlanGroup];
#pragma unroll
        for (int i = 0; i < kPlanGroup; i++)
            w[i] = g + i < j1 ? status[tb + g + i] : 0;
#pragma unroll
        for (int i = 0; i < kPlanGroup; i++) {
            if (g + i < j1)
                ch.plan[tb + g + i] = P;
            const uint64_t fl = st_flag(w[i], a.epoch);
            if (fl == kStIncl)
                P = st_value(w[i]);
            else if (fl == kStAgg)
                P += st_value(w[i]);
        }
    }
    __syncthreads();
    if (t == 0)
        ch.plan_hdr[s] = a.plan_sig;
}

template <class Src>
__global__ __launch_bounds__(kWalkThreads) void walk_kernel(BatchArgs a, Src src, DescArrays dall,
                                                            ChainArea ch,
                                                            const uint64_t *__restrict__ status,
                                                            double *__restrict__ outs,
                                                            exseq_stats *__restrict__ stats)
{
    __shared__ WalkLds sh;
    __shared__ __attribute__((aligned(16))) int lds_src[Src::kLdsInts];
    __shared__ unsigned long long st_fb, st_terms;
    __shared__ long long st_first;
    __shared__ unsigned st_nf;
    __shared__ long long st_best[kWaves];
    __shared__ PlanLds pl;
    const int s = blockIdx.x;
    if (a.plan_sig != 0)
        keep_plan(a, status, ch, s, pl);
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

    double S = a.init[s];
    size_t start = 0;
    if (a.tiny) {
        // A launch of a few chunks (no tiles ran): every chunk term by term
        // from init, in order.  Three dependent launches would cost more than
        // the adds.
        for (size_t c = 0; c < nch; c++) {
            const size_t b = c * kChunk;
            const int len = (int)(n - b < (size_t)kChunk ? n - b : (size_t)kChunk);
            const Four f = src.chunk(a, s, c, lds_src);
            src.keep(c, f);
            bool nf = false;
#pragma unroll
            for (int i = 0; i < 4; i++)
                nf |= i < f.cnt && is_nonfinite(f.v[i]);
            nonfinite |= __syncthreads_or(nf) != 0;
            S = resolve_terms(f, len, S, 0, sh, buf);
            S = bitsd(uniform_u64(dbits(S)));
            n_fb++;
            fb_terms += (uint64_t)len;
            first_fb = 0;
        }
        start = nch;
    } else if (nch && chain_on(a.flags)) {
        // The chain's exact sum after the last tile, or else the last exact
        // sum it published (the chain fails at one tile and at every
        // irregular tile after it, so that is where it stopped).
        const size_t tile = a.tile;
        const size_t tb = cb / tile;
        const int64_t tlast = (int64_t)((nch - 1) / tile);
        int64_t best = -1;
        if (ch.incl[tb + (size_t)tlast] > kInclFailed) {
            best = tlast;
        } else {
            for (int64_t j = t; j <= tlast; j += kWalkThreads)
                if (ch.incl[tb + (size_t)j] > kInclFailed)
                    best = j;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const long long o = __shfl_xor((long long)best, off);
                best = o > best ? o : best;
            }
            if (lane_id() == 0)
                st_best[wave_id()] = best;
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kWaves; k++)
                best = st_best[k] > best ? st_best[k] : best;
        }
        if (best >= 0) {
            S = bitsd(ch.incl[tb + (size_t)best] ^ kInclXor);
            start = (size_t)(best + 1) * tile;
            start = start < nch ? start : nch;
        }
        if (stats && start > 0) {
            // what the tiles did before that point
            if (t == 0) {
                st_fb = 0;
                st_terms = 0;
                st_first = 0x7FFFFFFFFFFFFFFFLL;
                st_nf = 0;
            }
            __syncthreads();
            unsigned long long my_fb = 0, my_terms = 0;
            long long my_first = 0x7FFFFFFFFFFFFFFFLL;
            unsigned my_nf = 0;
            for (size_t j = t; j < start; j += kWalkThreads) {
                const uint32_t mt = dmeta[j];
                my_nf |= mt & kFlagNonFinite;
                if (mt & kFlagResolved) {
                    my_fb++;
                    my_terms += n - j * kChunk < (size_t)kChunk ? n - j * kChunk : (size_t)kChunk;
                    my_first = (long long)j < my_first ? (long long)j : my_first;
                }
            }
            atomicAdd(&st_fb, my_fb);
            atomicAdd(&st_terms, my_terms);
            atomicMin(&st_first, my_first);
            atomicOr(&st_nf, my_nf);
            __syncthreads();
            n_fb = st_fb;
            fb_terms = st_terms;
            first_fb = st_first == 0x7FFFFFFFFFFFFFFFLL ? -1 : (int64_t)st_first;
            nonfinite |= st_nf != 0;
            n_fast = start - n_fb;
        }
    } else if (nch && (dmeta[0] & kFlagExact)) {
        // the first tile left the exact sum after the first chunk
        S = bitsd((uint64_t)dlo_a[0]);
        nonfinite |= (dmeta[0] & kFlagNonFinite) != 0;
        start = 1;
        n_fb = 1;
        fb_terms = n < (size_t)kChunk ? n : (size_t)kChunk;
        first_fb = 0;
    }

    WalkTally wt{n_fast, n_fb, fb_terms, misses, first_fb, nonfinite};
    S = walk_descs(src, a, s, dr0, dlo_a, dhi_a, dmeta, start, nch, S, wt, sh, buf, lds_src);
    n_fast = wt.n_fast;
    n_fb = wt.n_fb;
    fb_terms = wt.fb_terms;
    misses = wt.misses;
    first_fb = wt.first_fb;
    nonfinite = wt.nonfinite;
    if (t == 0) {
        outs[s] = S;
        src.done();  // what the source writes beside the sum
        if (a.means)
            a.means[s] = (float)(S / (double)n);  // ADR-1464: (float)(sum / windows)
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

// Zeroes the chain words of `tiles` tiles before a launch's tiles run.
__global__ __launch_bounds__(256) void chain_clear_kernel(ChainArea ch, uint32_t tiles)
{
    zero_chain_words(ch, tiles);  // consecutive lanes on consecutive words
}

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
    ChainArea ch;
};

// The tag of a launch's shape for a kept plan: every sum's length, init and
// first chunk, mixed by splitmix64 steps; never 0.
uint64_t plan_tag(const BatchArgs &a)
{
    auto mix = [](uint64_t h, uint64_t v) {
        uint64_t z = h ^ (v + 0x9E3779B97F4A7C15ULL + (h << 6) + (h >> 2));
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
        return z ^ (z >> 31);
    };
    uint64_t h = mix(0x6578736571706C6EULL, (uint64_t)a.count);
    for (int k = 0; k < a.count; k++) {
        uint64_t ib;
        std::memcpy(&ib, &a.init[k], sizeof ib);
        h = mix(mix(mix(h, a.n[k]), ib), a.chunk_base[k]);
    }
    h = mix(h, a.chunk_base[a.count]);
    return h ? h : 1;
}


size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Chunks per tile of a launch over `total` chunks.
uint32_t tile_chunks(uint32_t total, uint32_t flags)
{
    const uint32_t sel = (flags >> kTileShift) & 3u;  // 0: by size
    if (sel == 0 && !(flags & EXSEQ_PLAN_REUSE))
        return total <= 2u * kTileMax ? 4u : total <= 2048u ? 1u : total <= 4096u ? 2u : 4u;
    return sel == 1 ? 1u : (sel == 2 ? 2u : 4u);
}

WsParts carve(void *ws, size_t total)
{
    char *w = static_cast<char *>(ws);
    WsParts p;
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
    p.ch.agg = reinterpret_cast<uint64_t *>(w);
    w += round256(4 * total * sizeof(uint64_t));
    p.ch.incl = reinterpret_cast<uint64_t *>(w);
    w += round256(total * sizeof(uint64_t));
    p.ch.head = reinterpret_cast<uint64_t *>(w);
    w += round256(kMaxBatch * sizeof(uint64_t));
    p.ch.plan_hdr = reinterpret_cast<uint64_t *>(w);
    w += round256(kMaxBatch * sizeof(uint64_t));
    p.ch.plan = reinterpret_cast<double *>(w);
    w += round256((total / kTileMax + 1) * sizeof(double));
    p.ch.rec = reinterpret_cast<uint64_t *>(w);
    return p;
}
}  // namespace

// The kernels of the default path of one plain sum (the tile chain), in
// launch order, for the profiled entry point.
const char *const kPathKernels[] = {"chain_clear_kernel", "tile_kernel", "walk_kernel"};
const int kPathKernelCount = 3;

// Per chunk (a tile is at least one chunk): the plan status word, the four
// descriptor arrays, the chain words; per sum a head word and a kept-plan
// tag; per tile of kTileMax chunks a kept planned prefix.
size_t sum_ws_bytes(size_t total_chunks)
{
    const size_t pass = pass_ws_bytes(pass_blocks_bound(total_chunks, kMaxBatch), kMaxBatch);
    const size_t chain = 4 * round256(total_chunks * sizeof(int64_t)) +
           round256(total_chunks * sizeof(uint32_t)) +
           round256(4 * total_chunks * sizeof(uint64_t)) +
           round256(total_chunks * sizeof(uint64_t)) +
           2 * round256(kMaxBatch * sizeof(uint64_t)) +
           round256((total_chunks / kTileMax + 1) * sizeof(double)) +
           round256(kRecWords * total_chunks * sizeof(uint64_t));
    return chain > pass ? chain : pass;
}

template <int CPB, class Src>
static void launch_tiles(const BatchArgs &args, const Src &src, uint32_t total, const WsParts &p,
                         hipStream_t stream)
{
    const unsigned tiles = total / CPB;
    const bool chain = chain_on(args.flags);
    const unsigned blocks = chain ? 2u * (unsigned)args.count + args.rest_base[args.count] : tiles;
    if (tiles)
        hipLaunchKernelGGL(HIP_KERNEL_NAME(tile_kernel<CPB, Src>), dim3(blocks),
                           dim3(kChunkThreads), 0, stream, args, src, p.status, p.d, p.ch);
}

template <class Src>
static int launch_batch_src(const BatchArgs &a, const Src &src, void *ws, double *outs,
                            hipStream_t stream, exseq_stats *stats, void *const *events,
                            int n_events)
{
    auto mark = [&](int i) {
        if (events && i < n_events && events[i])
            hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
    };
    const uint32_t total = a.chunk_base[a.count];  // a multiple of kTileMax
    WsParts p = carve(ws, total);
    if (a.plan_hdr_ext) {
        p.ch.plan_hdr = a.plan_hdr_ext;
        p.ch.plan = a.plan_ext;
    }
    BatchArgs args = a;
    args.epoch = next_epoch();
    // Chunks per tile.  By default as many as keep the launch's tiles within
    // about two generations of workgroups in flight (1024 tiles each on 256
    // compute units): fewer chunks per tile mean shorter residency and more
    // tiles streaming at once, until a third generation costs more than
    // that saves.  A sum of at most two tiles of kTileMax chunks keeps them
    // (more tiles would only add links to its chain), and a kept plan is
    // kept per tile of kTileMax chunks.
    args.tile = tile_chunks(total, a.flags);
    const uint32_t tiles = total / args.tile;
    args.plan_sig = (a.flags & EXSEQ_PLAN_REUSE) && (a.flags & EXSEQ_PLAN_MASK) == EXSEQ_PLAN_AUTO &&
                            chain_on(a.flags) && args.tile == (uint32_t)kTileMax && tiles
                        ? plan_tag(a)
                        : 0;
    args.rest_base[0] = 0;
    for (int k = 0; k < a.count; k++) {
        const uint32_t nch = (uint32_t)((a.n[k] + kChunk - 1) / kChunk);
        const uint32_t tk = (a.chunk_base[k + 1] - a.chunk_base[k]) / args.tile;
        args.last_tile[k] = nch ? a.chunk_base[k] / args.tile + (nch - 1) / args.tile : ~0u;
        args.rest_base[k + 1] = args.rest_base[k] + (nch ? tk - 1 : tk);
    }
    // A launch of at most two tiles of kTileMax chunks, with default flags
    // and no per-kernel events: the walk kernel alone adds every chunk.
    args.tiny = total <= 2u * kTileMax && a.flags == 0u && !(events && n_events) ? 1u : 0u;
    if (args.tiny) {
        hipLaunchKernelGGL(HIP_KERNEL_NAME(walk_kernel<Src>), dim3((unsigned)a.count),
                           dim3(kWalkThreads), 0, stream, args, src, p.d, p.ch, p.status, outs, stats);
        return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
    }
    mark(0);
    if (chain_on(a.flags) && tiles && !a.chain_cleared)
        hipLaunchKernelGGL(chain_clear_kernel,
                           dim3((unsigned)((4 * tiles > (uint32_t)kMaxBatch ? 4 * tiles : (uint32_t)kMaxBatch) + 255) / 256),
                           dim3(256), 0, stream, p.ch, tiles);
    mark(1);
    mark(2);
    if (args.tile == 1)
        launch_tiles<1>(args, src, total, p, stream);
    else if (args.tile == 2)
        launch_tiles<2>(args, src, total, p, stream);
    else
        launch_tiles<4>(args, src, total, p, stream);
    mark(3);
    mark(4);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(walk_kernel<Src>), dim3((unsigned)a.count),
                       dim3(kWalkThreads), 0, stream, args, src, p.d, p.ch, p.status, outs, stats);
    mark(5);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
}

int launch_batch(const BatchArgs &a, void *ws, double *outs, hipStream_t stream,
                 exseq_stats *stats, void *const *events, int n_events)
{
    // the single pass for batches (and on request), except for launches of a
    // few chunks (the walk alone)
    const uint32_t total = a.chunk_base[a.count];
    const bool tiny = total <= 2u * kTileMax && (a.flags & ~EXSEQ_PASS_PATH) == 0u &&
                      !(events && n_events);
    const bool want = a.count > 1 || (a.flags & EXSEQ_PASS_PATH);
    if (want && !tiny && total > 0 && pass_eligible(a)) {
        size_t ns[kMaxBatch];
        for (int k = 0; k < a.count; k++)
            ns[k] = (size_t)a.n[k];
        return launch_pass(a.x, ns, a.init, a.count, a.flags, ws, outs, stream, stats, events, n_events);
    }
    return launch_batch_src(a, PlainTerms{}, ws, outs, stream, stats, events, n_events);
}

int launch_ssim_exact(const SsimParams &sp, double *out, void *ws, hipStream_t stream,
                      uint32_t flags, exseq_stats *stats)
{
    const size_t n = (size_t)sp.width * (size_t)sp.height;
    BatchArgs a{};
    a.count = 1;
    a.flags = flags;
    a.x[0] = nullptr;
    a.n[0] = n;
    a.init[0] = 0.0;
    a.chunk_base[0] = 0;
    a.chunk_base[1] = (uint32_t)padded_chunks(n);
    return launch_batch_src(a, SsimTerms{sp}, ws, out, stream, stats, nullptr, 0);
}

int launch_interleaved(const double *x, size_t windows, int k, const double *inits, double *outs,
                       float *means, void *ws, hipStream_t stream, uint32_t flags,
                       exseq_stats *stats)
{
    // k = 2 or 4 fields: the single pass, each line of the records read once
    if (pass_inter_ok(windows, k, flags))
        return launch_pass_interleaved(x, windows, k, inits, outs, means, ws, stream, flags, stats);
    BatchArgs a{};
    a.count = k;
    a.flags = flags;
    a.interleave = 1;
    a.means = means;
    const uint32_t per = (uint32_t)padded_chunks(windows);
    for (int j = 0; j < k; j++) {
        a.x[j] = x ? x + j : nullptr;
        a.n[j] = windows;
        a.init[j] = inits ? inits[j] : 0.0;
        a.chunk_base[j] = (uint32_t)j * per;
    }
    a.chunk_base[k] = (uint32_t)k * per;
    return launch_batch_src(a, StridedTerms{(uint32_t)k}, ws, outs, stream, stats, nullptr, 0);
}

bool chain_words_of(size_t n, uint32_t flags, void *ws, ChainArea *ch, uint32_t *tiles)
{
    const uint32_t total = (uint32_t)padded_chunks(n);
    // the decisions of launch_batch and launch_batch_src for one sum
    const bool tiny = total <= 2u * kTileMax && (flags & ~EXSEQ_PASS_PATH) == 0u;
    if (total == 0 || tiny || (flags & EXSEQ_PASS_PATH) || !chain_on(flags))
        return false;
    *tiles = total / tile_chunks(total, flags);
    *ch = carve(ws, total).ch;
    return *tiles > 0;
}

int launch_exact_sum_cleared(const double *x, size_t n, double init, double *out, void *ws,
                             hipStream_t stream, uint32_t flags, exseq_stats *stats)
{
    BatchArgs a{};
    a.count = 1;
    a.flags = flags;
    a.x[0] = x;
    a.n[0] = n;
    a.init[0] = init;
    a.chunk_base[0] = 0;
    a.chunk_base[1] = (uint32_t)padded_chunks(n);
    a.chain_cleared = 1;
    return launch_batch_src(a, PlainTerms{}, ws, out, stream, stats, nullptr, 0);
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

// A plain streaming read of n doubles: 16-byte non-temporal loads over a
// grid-stride loop, each block folding the bits it read with xor into one
// word out[block] (so that no load can be dropped).  The achievable read
// rate over a buffer, measured beside the exact sum.
__global__ __launch_bounds__(256) void stream_read_kernel(const double *x, size_t n, uint64_t *out)
{
    typedef double v2d __attribute__((ext_vector_type(2)));
    const size_t pairs = n / 2;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint64_t acc = 0;
    const v2d *p = reinterpret_cast<const v2d *>(x);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < pairs; i += stride) {
        const v2d v = __builtin_nontemporal_load(p + i);
        acc ^= dbits(v.x) ^ (dbits(v.y) * 3u);
    }
    if ((n & 1) && blockIdx.x == 0 && threadIdx.x == 0)
        acc ^= dbits(x[n - 1]);
    __shared__ uint64_t part[4];
    for (int o = 32; o > 0; o >>= 1)
        acc ^= (uint64_t)__shfl_xor((unsigned long long)acc, o);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
        out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

int launch_stream_read(const double *x, size_t n, uint64_t *out, hipStream_t stream)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3(EXSEQ_STREAM_READ_BLOCKS), dim3(256), 0, stream, x, n, out);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
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

#ifdef EXSEQ_TIMELINE
// The diagnostic build's read-back of the stamps (words: how many to copy,
// at most the array's size) and their reset; both synchronous.
extern "C" int exseq_timeline_read(uint64_t *host, size_t words)
{
    if (!host || words > exseq::kTlWords)
        return EXSEQ_EINVAL;
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(exseq::exseq_timeline), words * 8, 0,
                               hipMemcpyDeviceToHost) == hipSuccess
               ? EXSEQ_OK
               : EXSEQ_EHIP;
}
extern "C" int exseq_timeline_clear(void)
{
    static uint64_t zeros[exseq::kTlWords];
    return hipMemcpyToSymbol(HIP_SYMBOL(exseq::exseq_timeline), zeros, sizeof zeros, 0,
                             hipMemcpyHostToDevice) == hipSuccess
               ? EXSEQ_OK
               : EXSEQ_EHIP;
}
extern "C" size_t exseq_timeline_words(void) { return exseq::kTlWords; }
#endif
