// The single pass of the exact sequential sum: one launch per call.
//
// Research-1433 "Forming the CPU's sequential double sums on a GPU, bit for
// bit" (Findings 2-6, Open questions) describes four kernels: chunk tree
// sums, a one-lane plan, the increment pairs, and a one-lane walk over the
// chunks.  Here all of it is one launch.  A sum of n terms is cut into
// chunks of 1024 and into tiles: the sum's first tile is its first four
// chunks, every later tile eight.  Each sum gets, in this order of
// dispatch, three kinds of workgroup:
//
//  * the head: the first tile from init, exactly.  It publishes the tile's
//    inclusive plan prefix at once, adds the first chunk to init term by
//    term (there the running sum crosses binade after binade), then each
//    further chunk by its run under the exact sum's binade where that run
//    applies, else term by term, and publishes the exact sum after the tile.
//  * the finisher: it takes the head's exact sum and then follows the tiles'
//    records in order, a window of 1024 tiles at a time as they appear: the
//    regular tiles between irregular ones are composed with one segmented
//    scan (Research-1433 Open questions: compose runs that share a binade so
//    that the walk steps over many chunks at once), and the segments and the
//    irregular tiles' steps are applied in order from the exact sum.  A
//    segment or a step that does not hold for the exact sum is walked chunk
//    by chunk from its descriptors, and a chunk that fails there is added
//    term by term (Research-1433 Findings 4-5: a plan only decides where that
//    happens).  It writes the result and the statistics.
//  * one workgroup per later tile:
//     1. its 8192 terms requested at once: the first four chunks into
//        registers (16-byte non-temporal loads), the last four straight into
//        LDS (16-byte global-to-LDS loads), so that a frame's tiles are all
//        in flight together; the fixed-tree sum of every chunk;
//     2. the plan: the approximate prefix before the tile by a two-level
//        look-back, polled by two waves at once -- the tile words of its group
//        of 64 tiles, and the group words before that group.  Every tile
//        publishes its sum at once and its inclusive prefix when known; the
//        last tile of a group publishes the group's sum, then its inclusive
//        prefix;
//     3. every term's increment pair under its chunk's planned binade,
//        composed in order into each chunk's run (pair, prefix bounds,
//        flags), half a tile at a time; the descriptors are stored;
//     4. a tile that stays inside one planned binade away from its edges is
//        regular and publishes its composed run.  Any other tile locates the
//        crossing of every chunk planned to cross a binade edge (the term at
//        which the running sum leaves its binade, from the planned start
//        count) and publishes its O(1) step: the run before the crossing, the
//        crossing term, and the run after it in the next binade.  Nothing
//        waits for an exact sum.
//
// Cross-workgroup words carry a tag of the launch (42 bits, never zero and
// never reused within a process), so no word needs clearing between launches
// and stale words never match.  Plan words are self-contained.  Every word
// another workgroup reads is written and read with device-coherent
// (agent-scope) accesses, and a record's data words are acknowledged before
// its tagged first word is written.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstring>
#include <stdint.h>

#include "exseq.h"
#include "exseq_dev.h"
#include "exseq_internal.h"
#include "exseq_rules.h"
#include "exseq_wave.h"

namespace exseq {

constexpr int kHalf = 4;             // chunks per half tile (one Four each in registers)
constexpr int kTileCh = 8;           // chunks of every tile after a sum's first
constexpr int kHeadCh = 4;           // chunks of a sum's first tile
constexpr int kGroupShift = 6;
constexpr uint32_t kGroup = 1u << kGroupShift;  // tiles per look-back group
constexpr int kFinLane = 4;          // tiles per lane in a finisher window
constexpr int kFinTiles = kFinLane * kChunkThreads;  // tiles per finisher window
constexpr int kStepCap = 16;         // step records a finisher window holds
constexpr int kOpCap = 128;          // walk ops a finisher window holds
// A finisher tile word: key | kind << kKkKind | step shape (A present, the
// number of crossings) << kKkShape | (step record slot + 1) << kKkSlot.
constexpr int kKkKind = 12, kKkShape = 15, kKkSlot = 18;
constexpr int kTagShift = 22;       // record words: tag << 22 | ...; tags have 42 bits
// An irregular tile's step (kStepWords words): word 0 holds A's key (12
// bits), whether A is present (bit 12), the number of crossings (bits
// 13..14), A's neg and bad flags (bits 15..16) and r1 - r0 + 1 (bits
// 17..18); words 1..3 A's r0, lo, hi; then per crossing j a word with its
// chunk's key (12 bits), direction (bit 12: down), negative-term flag (bit
// 13) and length (bits 16..26), and the crossing's kCrossWords words.
constexpr int kMaxCross = 2;
constexpr int kXrecW = 1 + kCrossWords;
constexpr int kStepWords = 4 + kMaxCross * kXrecW;
static_assert(kStepCap * kStepWords <= 2 * kChunkThreads, "a window's step records: two words per thread");
constexpr uint32_t kKindReg = 1, kKindStep = 2, kKindSlow = 3;
constexpr uint32_t kKindLost = 4;    // finisher only: the record never came

static_assert(kHeadCh == kTileMax, "a sum's first tile is one padding unit of chunks");

// Tiles of a sum of nch chunks, and the first chunk of tile i.
// (tch: chunks of a later tile of the sum; kTileCh except in a launch of
// interleaved sums, whose tiles take 8 / k chunks of each of k sums)
__host__ __device__ __forceinline__ uint32_t tiles_of(uint32_t nch, uint32_t tch = kTileCh)
{
    return nch == 0 ? 0u : nch <= (uint32_t)kHeadCh ? 1u : 1u + (nch - kHeadCh + tch - 1) / tch;
}
__host__ __device__ __forceinline__ uint32_t tile_c0(uint32_t i, uint32_t tch = kTileCh)
{
    return i == 0 ? 0u : (uint32_t)kHeadCh + tch * (i - 1);
}

// First word of a tile record: tag | ext << 19 | kind << 17 | flags (neg,
// bad, non-finite at their descriptor positions) | r1 - r0 + 1 | key.  For
// an irregular tile, ext holds its step's shape (run A present: bit 0; the
// number of crossings: bits 1..2) and key, dr and neg its last run's.
__device__ __forceinline__ uint64_t rec_w0(uint64_t tag, uint32_t kind, uint32_t flags, int64_t dr,
                                           uint32_t key, uint32_t ext = 0u)
{
    return (tag << kTagShift) | ((uint64_t)(ext & 7u) << 19) | ((uint64_t)kind << 17) |
           (uint64_t)(flags & (kFlagNeg | kFlagBad | kFlagNonFinite)) |
           ((uint64_t)(dr + 1) << kDrShift) | (uint64_t)(key & kKeyMask);
}

// Second word of a regular tile's record: r0 + 2^53 in the low 54 bits and
// the launch tag's low 10 bits above (|r0| <= 2^52 + 1 for a record).  The
// finisher reads the first two words with one 16-byte load; the tag bits
// let it see that this word belongs to the same launch as the first.
__device__ __forceinline__ uint64_t rec_w1(uint64_t tag, int64_t r0)
{
    return ((uint64_t)(r0 + ((int64_t)1 << 53)) & (((uint64_t)1 << 54) - 1)) | ((tag & 0x3FFu) << 54);
}
__device__ __forceinline__ bool rec_w1_ok(uint64_t tag, uint64_t w1) { return (w1 >> 54) == (tag & 0x3FFu); }
__device__ __forceinline__ int64_t rec_w1_r0(uint64_t w1)
{
    return (int64_t)(w1 & (((uint64_t)1 << 54) - 1)) - ((int64_t)1 << 53);
}

// 16 bytes of device-coherent memory in one load.
typedef uint64_t v2u64 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2u64 load_coherent_16(const uint64_t *p)
{
    typedef const volatile __attribute__((address_space(1))) v2u64 *gptr;
    return *(gptr)(p);
}

// 16 bytes to device-coherent memory in one store (written through).
__device__ __forceinline__ void store_coherent_16(uint64_t *p, uint64_t a, uint64_t b)
{
    typedef volatile __attribute__((address_space(1))) v2u64 *gptr;
    v2u64 v;
    v.x = a;
    v.y = b;
    *(gptr)(p) = v;
}

// Workspace of a pass launch (see pass_carve).
struct PassWs {
    uint64_t *st;    // per tile: plan status word
    uint64_t *gst;   // per group: plan status word
    DescArrays d;    // per chunk: descriptor
    uint64_t *trec;  // per tile: 4 words (w0, then r0, lo, hi each with tag bits;
                     // lo and hi only for a run with a negative term)
    uint64_t *xrec;  // per tile: kStepWords words (an irregular tile's step)
    uint64_t *hrec;  // per sum: 2 words (w0, exact sum after the first tile)
};

// Up to kPassMax sums, by value.  Sum s has the workgroups block_base[s] ..
// block_base[s + 1] - 1 (its head, its finisher, its later tiles), and the
// workspace is laid out by the same index: the tile words of sum s start at
// block_base[s], its look-back group words at block_base[s] / kGroup + s, its
// chunk descriptors at 8 * block_base[s] (a sum of nt tiles has nt + 1
// workgroups, at most 8 nt - 4 chunks and at most nt / kGroup + 1 groups).
struct PassArgs {
    int count;
    uint32_t flags;
    uint32_t tch;    // chunks of a sum's later tiles (kTileCh, or 8 / inter)
    uint32_t inter;  // interleaved sums: k fields per record (x[s] = x[0] + s), else 0
    float *means;    // nullable: means[s] = (float)(sum / n[s])
    uint32_t epoch;  // tags this launch's look-back status words
    uint64_t tag;    // this launch's record tag (42 bits, nonzero)
    double *outs;
    exseq_stats *stats;
    const double *x[kPassMax];
    uint64_t n[kPassMax];
    double init[kPassMax];
    uint32_t block_base[kPassMax + 1];
    __device__ __forceinline__ uint32_t tile_base(int s) const { return block_base[s]; }
    __device__ __forceinline__ uint32_t group_base(int s) const { return (block_base[s] >> kGroupShift) + (uint32_t)s; }
    __device__ __forceinline__ uint32_t chunk_base(int s) const { return (uint32_t)kTileCh * block_base[s]; }
};
static_assert(sizeof(PassArgs) <= 4096, "kernel arguments of the single pass");

// ---------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------
struct PassTileLds {
    double tsum[kTileCh];
    double wsum[kHeadCh][kWaves];  // the head's chunk sums per wave
    WaveRun wrun[kWaves];          // the head's block_run scratch
    WaveRun join[kTileCh];
    double pk[kTileCh];
    uint32_t key[kTileCh];
    uint32_t cross[kTileCh];
    uint32_t down[kTileCh];
    uint32_t locate[kTileCh];
    uint64_t xw[kTileCh][kCrossWords];
    uint64_t rec[kStepWords];
    uint64_t xexit[4];  // an irregular tile's last run: key etc., r0, lo, hi
    // the look-back's results, one slot per sum of the workgroup (the
    // interleaved tiles take up to four sums)
    double lb1[4], lb2[4];
    int lb_found[4], lb_ok1[4], lb_ok2[4];
    volatile int lb_stop[4];
};

// The finisher composes the runs of a segment's tiles with an ordered
// segmented scan: values carry whether they start a segment (head) and that
// segment's first tile (start).
struct SegRun {
    Run r;
    int32_t start;
    int32_t head;
};

// What the walks over descriptors added (the fallback), for the statistics.
struct FinTally {
    unsigned long long fast, fb, terms;
    long long first;
    unsigned misses, nonfinite;
};

// The finisher's ordered walk runs a list of ops compiled from the window's
// events, one lane per event, before the walk starts: REG applies a run in
// the binade it names (S's count m must lie in [L, H(m's parity)], then m
// grows by r(parity)), CROSS adds a located crossing term with one fp64 add
// after checking that the crossing is where the tile found it for this S,
// FAIL stands for a tile whose records give no O(1) step.  An event (a
// regular segment, or an irregular tile's step: run A, then per crossing a
// CROSS and the REG of the rest in the next binade) is one to five ops;
// where one fails, the event's chunks are walked from the sum before it.
constexpr int kOpWords = 9;
constexpr uint32_t kOpReg = 1, kOpCross = 2, kOpFail = 3;
// word 0: kind | key << 2 | first << 14 | last << 15 | down << 16 |
// j0 << 17 | nodesc << 18 | ops after this one in its event << 19
// REG: L, H0, H1, r0, r1.  CROSS: L of the prefix check, the pairs before
// and through the crossing term (r0, r1 each), H of the prefix check, the
// term's bits.  Word 8: the event's chunks, c_lo | c_hi << 32.  Words 1,
// 2 + parity and 4 + parity are read for either kind.
constexpr uint32_t kOpFirst = 1u << 14, kOpLast = 1u << 15, kOpDown = 1u << 16, kOpJ0 = 1u << 17,
                   kOpNoDesc = 1u << 18;
constexpr int kOpRestShift = 19;

struct FinLds {
    uint32_t kk[kFinTiles];      // per tile of the window (see kKkKind)
    uint16_t opoff[kFinTiles];   // a segment's first op, at its first tile
    uint64_t rec[kStepCap][kStepWords];
    uint64_t ops[kOpCap][kOpWords];
    int32_t cut, nops_cut;
    int32_t nslots;  // step record slots taken in this window
    uint32_t stile[kStepCap];  // the tile (in the launch) of each slot
    struct {
        uint64_t sbits;
        int32_t i;
        uint32_t fast, fb_lo, fb_hi, fb_desc;
    } wk;  // where wave 0's walk stopped
    SegRun wr[kWaves];
    int32_t cnt[kWaves];
    uint32_t nf[kWaves];
    FinTally tally;
};

// The workgroup's 32 KB of role-dependent LDS: a tile's last four chunks, the
// head's chunk terms, or the finisher's window and chunk terms.
constexpr int kUnionDoubles = kHalf * kChunk + 16;
constexpr int kFinTermsOff = (int)((sizeof(FinLds) + 15) / 16 * 2);  // in doubles
static_assert(kFinTermsOff + kChunk <= kUnionDoubles, "the finisher's LDS fits the union");

// ---------------------------------------------------------------------------
// Device-coherent words
// ---------------------------------------------------------------------------
// A record's data words are acknowledged before its tagged first word is
// written: each storing wave waits for its stores to complete (a
// workgroup-scope release, which is only that wait), then the workgroup
// meets at a barrier, then one lane writes the tagged word.
__device__ __forceinline__ void stores_complete()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
}
__device__ __forceinline__ uint32_t load_relaxed_u32(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed_u32(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int64_t load_relaxed_i64(const int64_t *p)
{
    return (int64_t)load_relaxed_u64(reinterpret_cast<const uint64_t *>(p));
}

// A chunk's descriptor (as store_desc), with device-coherent stores.
__device__ __forceinline__ void store_desc_coherent(const DescArrays &d, size_t c, uint32_t key,
                                                    const WaveRun &r, uint32_t extra)
{
    const int64_t dr = r.p.r1 - r.p.r0;
    store_relaxed_u64(reinterpret_cast<uint64_t *>(d.r0 + c), (uint64_t)r.p.r0);
    store_relaxed_u64(reinterpret_cast<uint64_t *>(d.lo + c), (uint64_t)r.lo);
    store_relaxed_u64(reinterpret_cast<uint64_t *>(d.hi + c), (uint64_t)r.hi);
    store_relaxed_u32(d.meta + c,
                      (key & kKeyMask) | ((uint32_t)(dr + 1) << kDrShift) | r.flags | extra);
}

__device__ __forceinline__ uint32_t chunks_of_n(size_t n) { return (uint32_t)((n + kChunk - 1) / kChunk); }
__device__ __forceinline__ int chunk_len(size_t n, size_t c)
{
    const size_t b = c * kChunk;
    return (int)(n - b < (size_t)kChunk ? n - b : (size_t)kChunk);
}

// ---------------------------------------------------------------------------
// A tile's last four chunks in LDS.  Lane l of wave w keeps terms 4l, 4l+1 of
// slot k at stage[k*1024 + w*256 + 2l] and terms 4l+2, 4l+3 at 128 doubles
// further (the layout of a 16-byte global-to-LDS load: lane l's 16 bytes at
// 16 l from the wave's base).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double *stage_at(double *stage, int k, int half)
{
    return stage + k * kChunk + wave_id() * 256 + half * 128;
}

// Requests lane t's terms of chunk c into slot k: directly into LDS where
// the chunk's terms all exist and are 16-byte aligned, else through
// registers (missing terms are +0.0).
__device__ __forceinline__ void stage_chunk(double *stage, int k, const SumView &v, size_t c, bool direct)
{
    const size_t first = c * kChunk + 4 * (size_t)threadIdx.x;
    const int lane = lane_id();
    if (direct) {
        const double *p = v.x + first;
        __builtin_amdgcn_global_load_lds((const void *)p,
                                         (__attribute__((address_space(3))) void *)stage_at(stage, k, 0),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(p + 2),
                                         (__attribute__((address_space(3))) void *)stage_at(stage, k, 1),
                                         16, 0, 0);
    } else {
        const Four f = load_four(v.x, v.n, first, true);
        double *a = stage_at(stage, k, 0) + 2 * lane;
        double *b = stage_at(stage, k, 1) + 2 * lane;
        a[0] = f.v[0];
        a[1] = f.v[1];
        b[0] = f.v[2];
        b[1] = f.v[3];
    }
}

// Lane t's four terms of chunk c from slot k.
__device__ __forceinline__ Four staged_chunk(double *stage, int k, size_t n, size_t c)
{
    const int lane = lane_id();
    const double *a = stage_at(stage, k, 0) + 2 * lane;
    const double *b = stage_at(stage, k, 1) + 2 * lane;
    Four f;
    f.v[0] = a[0];
    f.v[1] = a[1];
    f.v[2] = b[0];
    f.v[3] = b[1];
    const size_t first = c * kChunk + 4 * (size_t)threadIdx.x;
    f.cnt = first < n ? (int)(n - first < 4 ? n - first : 4) : 0;
    return f;
}

// ---------------------------------------------------------------------------
// The plan: two-level look-back
// ---------------------------------------------------------------------------
// Level 1 (one wave): the p tile words before this tile in its group (at
// st).  Returns whether an inclusive prefix was among them; val is that
// prefix plus the sums of the tiles after it, else the sum of all p tiles.
// False in ok on a timeout.
__device__ __forceinline__ bool lb_level1(const uint64_t *st, int p, uint32_t epoch, double &val,
                                          bool &ok)
{
    const int lane = lane_id();
    ok = true;
    val = 0.0;
    if (p == 0)
        return false;
    const uint64_t need = (p >= 64) ? ~0ULL : ((1ULL << p) - 1);
    for (int spin = 0;; spin++) {
        const uint64_t w = lane < p ? load_relaxed_u64(st + lane) : 0;
        const uint64_t fl = lane < p ? st_flag(w, epoch) : 0;
        const uint64_t present = __ballot(fl != 0) & need;
        const uint64_t incl = __ballot(fl == kStIncl) & need;
        if (incl) {
            const int j = 63 - __builtin_clzll(incl);
            const uint64_t above = need & ~((j == 63) ? ~0ULL : ((2ULL << j) - 1));
            if ((present & above) == above) {
                val = wave_sum_f64(lane >= j && lane < p ? st_value(w) : 0.0);
                return true;
            }
        }
        if (present == need) {
            val = wave_sum_f64(lane < p ? st_value(w) : 0.0);
            return false;
        }
        if (spin >= kSpinLimit) {
            ok = false;
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Level 2 (one wave): the prefix before group lg from the group words before
// it (decoupled look-back: the nearest inclusive prefix plus the group sums
// after it).  Gives up when `stop` is set (level 1 found an inclusive
// prefix) or on a timeout (ok false).
__device__ __forceinline__ double lb_level2(const uint64_t *gst, uint32_t lg, uint32_t epoch,
                                            volatile int *stop, bool &ok)
{
    const int lane = lane_id();
    ok = true;
    double acc = 0.0;
    int64_t j = (int64_t)lg - 1;
    for (int spin = 0;; spin++) {
        if (*stop)
            return 0.0;
        const int64_t idx = j - lane;
        uint64_t fl;
        double v;
        if (idx >= 0) {
            const uint64_t w = load_relaxed_u64(gst + idx);
            fl = st_flag(w, epoch);
            v = st_value(w);
        } else {
            fl = kStIncl;  // before the sum's first group: nothing
            v = 0.0;
        }
        const uint64_t missing = __ballot(fl == 0);
        const uint64_t incl = __ballot(fl == kStIncl);
        const int first_missing = missing ? __builtin_ctzll(missing) : 64;
        const int first_incl = incl ? __builtin_ctzll(incl) : 64;
        if (first_incl < first_missing) {
            acc += wave_sum_f64(lane <= first_incl ? v : 0.0);
            return acc;
        }
        if (!missing) {
            acc += wave_sum_f64(v);
            j -= 64;
            continue;
        }
        if (spin >= kSpinLimit) {
            ok = false;
            return 0.0;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// ---------------------------------------------------------------------------
// Building blocks of the head and the finisher
// ---------------------------------------------------------------------------
// Chunk f's run under `key` (all 256 lanes; the same result everywhere).
__device__ __forceinline__ WaveRun block_run(const Four &f, uint32_t key, WaveRun *part)
{
    const WaveRun w = wave_run(f, key);
    if (lane_id() == 0)
        part[wave_id()] = w;
    __syncthreads();
    const WaveRun r = clamp_run(join_waves(part));
    __syncthreads();
    return r;
}

// The finisher composes the regular tiles of a segment with two segmented
// scans instead of one of whole runs, which needs far fewer registers.
// First the pairs (the parity-dependent increments), ordered; then the
// prefix bounds, which compose as a prefix minimum and maximum: a segment's
// lowest prefix is the least over its tiles of (the smaller component of
// the pair before the tile + the tile's lowest prefix), its highest the
// greatest of (the larger component + the tile's largest prefix), exactly as
// run_compose folds them one at a time.


// The ordered segmented composition of runs: r starts a segment, or the
// segment continues with r (run_compose_sat: a composed run too wide for a
// binade is only marked bad).
__device__ __forceinline__ SegRun segr_op(const SegRun &l, const SegRun &r)
{
    if (r.head)
        return r;
    return SegRun{run_compose_sat(l.r, r.r), l.start, l.head};
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ SegRun dpp_segr(const SegRun &v)
{
    // lanes without a source take the identity
    return SegRun{dpp_run<Ctrl, RowMask>(v.r),
                  (int32_t)dpp_u32<Ctrl, RowMask>((uint32_t)v.start, 0xFFFFFFFFu),
                  (int32_t)dpp_u32<Ctrl, RowMask>((uint32_t)v.head, 0u)};
}

// Exclusive ordered segmented scan over the workgroup's lanes (one
// barrier): lane t gets the composition of lanes 0 .. t-1.
__device__ __forceinline__ SegRun block_excl_segr(const SegRun &v, FinLds &F)
{
    const int lane = lane_id(), wave = wave_id();
    SegRun inc = v;
    inc = segr_op(dpp_segr<kDppRowShr1>(inc), inc);
    inc = segr_op(dpp_segr<kDppRowShr2>(inc), inc);
    inc = segr_op(dpp_segr<kDppRowShr4>(inc), inc);
    inc = segr_op(dpp_segr<kDppRowShr8>(inc), inc);
    inc = segr_op(dpp_segr<kDppRowBcast15, 0xA>(inc), inc);
    inc = segr_op(dpp_segr<kDppRowBcast31, 0xC>(inc), inc);
    if (lane == 63)
        F.wr[wave] = inc;
    const SegRun before = dpp_segr<kDppWaveShr1>(inc);  // lane 0: the identity
    __syncthreads();
    SegRun carry{run_identity(), -1, 0};
    for (int k = 0; k < kWaves; k++)
        if (k < wave)
            carry = segr_op(carry, F.wr[k]);
    return segr_op(carry, before);
}

// The finisher's fallback: the ordered walk over the descriptors of chunks
// [c_lo, c_hi) of the sum from the exact sum S before c_lo, one chunk per
// lane, 256 at a time.  A scan of the pairs from the first chunk not yet
// applied gives every chunk's start count in the running sum's binade,
// every chunk is checked there, the first that fails is applied in the next
// binade if the runs before it ended exactly on 2^(e+1), else added term by
// term from the exact sum, and the next scan starts after it.  With
// use_desc false (a record or the head's sum never came) every chunk is added
// term by term.  Counts go to `tally` (lane 0).  Inlined: as a call, every
// value of the finisher live across it would be spilled to scratch memory and
// reloaded in the event loop.
template <class Src>
__device__ __forceinline__ double walk_lean(const Src &src, const SumView v, const DescArrays d,
                                         uint32_t c_lo, uint32_t c_hi, double S, WalkCore &sh,
                                         double *terms, int *lds_src, bool use_desc,
                                         FinTally &tally)
{
    const int t = threadIdx.x;
    const size_t n = v.n;
    const size_t cb = v.cb;
    int buf = 0;
    uint64_t n_fast = 0, n_fb = 0, fb_terms = 0;
    uint32_t misses = 0;
    int64_t first = -1;
    bool nonfinite = false;
    __syncthreads();  // the caller's last reads of the scratch are done
    for (uint32_t base = c_lo; base < c_hi; base += kChunkThreads) {
        const int cnt = (int)(c_hi - base < (uint32_t)kChunkThreads ? c_hi - base : (uint32_t)kChunkThreads);
        Pair mine = pair_identity();
        int64_t dlo = 0, dhi = 0;
        uint32_t dkey = 0u, dfl = kFlagBad;
        if (t < cnt && use_desc) {
            const size_t c = cb + base + (size_t)t;
            const uint32_t mt = load_relaxed_u32(d.meta + c);
            const int64_t r0 = load_relaxed_i64(d.r0 + c);
            mine = Pair{r0, r0 + (int64_t)((mt >> kDrShift) & 3u) - 1};
            dkey = mt & kKeyMask;
            dfl = mt & (kFlagNeg | kFlagBad | kFlagNonFinite);
            if (dfl & kFlagNeg) {
                dlo = load_relaxed_i64(d.lo + c);
                dhi = load_relaxed_i64(d.hi + c);
            }
        }
        nonfinite |= __syncthreads_or(t < cnt && (dfl & kFlagNonFinite)) != 0;
        int cur = 0;
        while (cur < cnt) {
            const bool in = t >= cur && t < cnt;
            const Pair pv = in ? mine : pair_identity();
            const Pair X = block_excl_scan(pv, in && mine.r0 != mine.r1, sh, buf);
            buf ^= 1;
            const uint32_t ks = key_of(S);
            const bool fs = key_has_fast_path(ks);
            const int64_t m = count_of(S);
            const int64_t mt = m + pair_at(X, m);
            const bool ok = fs && dkey == ks && mt >= count_floor(ks) && mt < kCountHi &&
                            run_applies(mt, mine, dlo, dhi, dfl);
            Cand mc = cand_none();
            if (in && !ok) {
                mc.idx = t;
                mc.s_at = t == cur ? S : assemble(ks, mt);
            }
            if (t == cnt - 1)
                sh.endv[buf] = ok ? assemble(ks, mt + pair_at(mine, mt)) : 0.0;
            const Cand fc = block_first(in && !ok, mc, sh, buf);
            const double endv = sh.endv[buf];
            buf ^= 1;
            if (fc.idx == kNone) {
                n_fast += (uint64_t)(cnt - cur);
                S = bitsd(uniform_u64(dbits(endv)));
                break;
            }
            const int f = __builtin_amdgcn_readfirstlane(fc.idx);
            n_fast += (uint64_t)(f - cur);
            const double sat = bitsd(uniform_u64(dbits(fc.s_at)));
            const size_t c = cb + base + (size_t)f;
            const uint32_t fmt = use_desc ? load_relaxed_u32(d.meta + c) : kFlagBad;
            const int64_t fr0 = use_desc ? load_relaxed_i64(d.r0 + c) : 0;
            const Pair fp{fr0, fr0 + (int64_t)((fmt >> kDrShift) & 3u) - 1};
            const uint32_t ffl = fmt & (kFlagNeg | kFlagBad | kFlagNonFinite);
            const int64_t flo = use_desc && (ffl & kFlagNeg) ? load_relaxed_i64(d.lo + c) : 0;
            const int64_t fhi = use_desc && (ffl & kFlagNeg) ? load_relaxed_i64(d.hi + c) : 0;
            const uint32_t k2 = key_of(sat);
            const int64_t m2 = count_of(sat);
            if (key_has_fast_path(k2) && (fmt & kKeyMask) == k2 && run_applies(m2, fp, flo, fhi, ffl)) {
                S = assemble(k2, m2 + pair_at(fp, m2));
                n_fast++;
            } else {
                misses += (fmt & kKeyMask) != k2;
                const uint32_t cc = base + (uint32_t)f;
                const Four fr = src.chunk_v(v, cc, lds_src);
                if (!use_desc) {
                    bool nf = false;
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        nf |= i < fr.cnt && is_nonfinite(fr.v[i]);
                    nonfinite |= __syncthreads_or(nf) != 0;
                }
                S = resolve_terms(fr, chunk_len(n, cc), sat, 0, sh, terms, buf);
                S = bitsd(uniform_u64(dbits(S)));
                n_fb++;
                fb_terms += (uint64_t)chunk_len(n, cc);
                if (first < 0)
                    first = (int64_t)cc;
            }
            cur = f + 1;
        }
    }
    __syncthreads();
    if (t == 0) {
        tally.fast += n_fast;
        tally.fb += n_fb;
        tally.terms += fb_terms;
        if (tally.first < 0 && first >= 0)
            tally.first = first;
        tally.misses += misses;
        tally.nonfinite |= nonfinite ? 1u : 0u;
    }
    __syncthreads();
    return S;
}

// ---------------------------------------------------------------------------
// The head: a sum's first tile (its first four chunks) from init, exactly.
// A sum without terms is its init.
// ---------------------------------------------------------------------------
template <class Src>
__device__ __forceinline__ void head_block(const PassArgs &pa, const Src &src, const PassWs &w,
                                           int s, PassTileLds &L, WalkCore &sc, double *terms,
                                           int *lds_src)
{
    const PassArgs &a = pa;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    const size_t n = a.n[s];
    exseq_stats *stats = pa.stats ? pa.stats + s : nullptr;
    if (n == 0) {
        if (t == 0) {
            pa.outs[s] = a.init[s];
            if (stats) {
                exseq_stats st;
                st.chunks = st.fast_chunks = st.fallback_chunks = st.fallback_terms = 0;
                st.first_fallback = -1;
                st.flags = 0u;
                st.plan_misses = 0u;
                stats[0] = st;
            }
        }
        return;
    }
    const uint32_t nch = chunks_of_n(n);
    const uint32_t nt = tiles_of(nch, pa.tch);
    const int nk = (int)(nch < (uint32_t)kHeadCh ? nch : (uint32_t)kHeadCh);
    const SumView v{a.x[s], n, a.init[s], a.chunk_base(s), nch};
    Four f[kHeadCh];
#pragma unroll
    for (int k = 0; k < kHeadCh; k++)
        f[k] = src.chunk_v(v, (size_t)k, lds_src);
    bool nf = false;
#pragma unroll
    for (int k = 0; k < kHeadCh; k++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            nf |= i < f[k].cnt && is_nonfinite(f[k].v[i]);
    // the tile's inclusive plan prefix (fixed-tree chunk sums)
    if (nt > 1 && (a.flags & EXSEQ_PLAN_MASK) != EXSEQ_PLAN_FIXED) {
        double ws[kHeadCh];
#pragma unroll
        for (int k = 0; k < kHeadCh; k++)
            ws[k] = (f[k].v[0] + f[k].v[1]) + (f[k].v[2] + f[k].v[3]);
        wave_sum_f64_n<kHeadCh>(ws);
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < kHeadCh; k++)
                L.wsum[k][wave] = ws[k];
        }
        __syncthreads();
        if (t == 0) {
            double Ttile = 0.0;
#pragma unroll
            for (int k = 0; k < kHeadCh; k++)
                Ttile += (L.wsum[k][0] + L.wsum[k][1]) + (L.wsum[k][2] + L.wsum[k][3]);
            store_relaxed_u64(w.st + pa.tile_base(s), st_pack(a.epoch, kStIncl, a.init[s] + Ttile));
        }
    }
    nf = __syncthreads_or(nf) != 0;
    int buf = 0;
    double S = a.init[s];
    uint32_t resolved = 0u;
#pragma unroll 1
    for (int k = 0; k < nk; k++) {
        // chunk k's terms, by unrolled selects (no indexed register array)
        Four fk = f[0];
#pragma unroll
        for (int j = 1; j < kHeadCh; j++)
            if (j == k)
                fk = opaque(f[j]);
        const uint32_t ks = key_of(S);
        bool applied = false;
        if (k > 0 && key_has_fast_path(ks)) {
            const WaveRun r = block_run(fk, ks, L.wrun);
            const int64_t m = count_of(S);
            if (run_applies(m, r.p, r.lo, r.hi, r.flags)) {
                S = assemble(ks, m + pair_at(r.p, m));
                applied = true;
            }
        }
        if (!applied) {
            S = resolve_terms(fk, chunk_len(n, (size_t)k), S, 0, sc, terms, buf);
            S = bitsd(uniform_u64(dbits(S)));
            resolved |= 1u << k;
        }
    }
    if (t != 0)
        return;
    if (nt == 1) {
        pa.outs[s] = S;
        if (stats) {
            exseq_stats st;
            st.chunks = nch;
            st.fallback_chunks = (uint64_t)__builtin_popcount(resolved);
            st.fast_chunks = nch - st.fallback_chunks;
            uint64_t ft = 0;
            for (int k = 0; k < nk; k++)
                if ((resolved >> k) & 1u)
                    ft += (uint64_t)chunk_len(n, (size_t)k);
            st.fallback_terms = ft;
            st.first_fallback = 0;
            st.flags = nf ? EXSEQ_STAT_NONFINITE : 0u;
            st.plan_misses = 0u;
            stats[0] = st;
        }
        return;
    }
    uint64_t *hrec = w.hrec + 2 * (size_t)s;
    store_relaxed_u64(hrec + 1, dbits(S));
    stores_complete();
    store_relaxed_u64(hrec, (pa.tag << kTagShift) | (nf ? 16u : 0u) | (uint64_t)resolved);
}

// Writes a REG op for a run (pair p, prefix bounds lo/hi, flags) in binade
// key; a run that cannot apply becomes FAIL.
__device__ __forceinline__ void op_reg(uint64_t *o, uint32_t key, Pair p, int64_t lo, int64_t hi,
                                       uint32_t flags, uint64_t head, uint64_t range)
{
    if ((flags & (kFlagBad | kFlagNonFinite)) || !key_has_fast_path(key)) {
        o[0] = kOpFail | head;
        o[8] = range;
        return;
    }
    const bool neg = (flags & kFlagNeg) != 0;
    o[0] = kOpReg | ((uint64_t)(key & kKeyMask) << 2) | head;
    o[1] = (uint64_t)(neg ? kCountLo + 1 - lo : (int64_t)0);
    o[2] = (uint64_t)(neg ? kCountHi - 1 - hi : kCountHi - p.r0);
    o[3] = (uint64_t)(neg ? kCountHi - 1 - hi : kCountHi - p.r1);
    o[4] = (uint64_t)p.r0;
    o[5] = (uint64_t)p.r1;
    o[8] = range;
}


// A finisher tile word's fields.
__device__ __forceinline__ uint32_t kk_kind(uint32_t w) { return (w >> kKkKind) & 7u; }
// The walk ops of the segment a tile starts: an irregular tile with a
// record slot takes run A (when it has crossings), and per crossing CROSS
// and the REG of the rest (the last one: the segment's run); any other
// tile one op.
__device__ __forceinline__ int kk_ops(uint32_t w)
{
    const uint32_t kind = kk_kind(w);
    if (kind == 0u)
        return 0;
    if (kind != kKindStep || (w >> kKkSlot) == 0u)
        return 1;
    const uint32_t shape = (w >> kKkShape) & 7u;
    const int nx = (int)(shape >> 1);
    return nx == 0 ? 1 : (int)(shape & 1u) + 2 * nx;
}

// Writes the leading ops of an irregular tile's step (all but the last of
// its n_op ops, which is the segment's run): run A, then per crossing CROSS
// and, for all but the last crossing, the REG of its rest.
__device__ __forceinline__ void op_step_lead(uint64_t (*o)[kOpWords], const uint64_t *rw, int n_op,
                                             uint64_t range)
{
    const uint64_t m0 = rw[0];
    const int nx = (int)((m0 >> 13) & 3u);
    int k = 0;
    auto head = [&](int k) {
        return (k == 0 ? (uint64_t)kOpFirst : 0u) | (k == n_op - 1 ? (uint64_t)kOpLast : 0u) |
               ((uint64_t)(n_op - 1 - k) << kOpRestShift);
    };
    if (nx == 0)
        return;  // A alone: the segment's run starts with it
    if ((m0 >> 12) & 1u) {
        const int64_t r0 = dec_i64(rw[1]);
        op_reg(o[k], (uint32_t)m0 & kKeyMask, Pair{r0, r0 + (int64_t)((m0 >> 17) & 3u) - 1},
               dec_i64(rw[2]), dec_i64(rw[3]), (uint32_t)((m0 >> 15) & 3u) << 14, head(k), range);
        k++;
    }
    for (int j = 0; j < nx; j++) {
        const uint64_t *x = rw + 4 + kXrecW * j;
        const uint64_t xm = x[0];
        const uint32_t key = (uint32_t)xm & kKeyMask;
        const bool down = ((xm >> 12) & 1u) != 0;
        const bool neg = ((xm >> 13) & 1u) != 0 || down;
        const int len = (int)((xm >> 16) & 0x7FFu);
        const int64_t jj = dec_i64(x[1 + kXj]);
        const uint32_t key2 = down ? key - 1u : key + 1u;
        uint64_t *c = o[k];
        if (jj >= len || !key_has_fast_path(key) || !key_has_fast_path(key2)) {
            c[0] = kOpFail | head(k);
        } else {
            const Pair pj1 = rec_unpack(dec_i64(x[1 + kXpj1]));
            const Pair pj = rec_unpack(dec_i64(x[1 + kXpj]));
            c[0] = kOpCross | ((uint64_t)key << 2) | head(k) | (down ? (uint64_t)kOpDown : 0u) |
                   (jj == 0 ? (uint64_t)kOpJ0 : 0u);
            c[1] = (uint64_t)(neg ? kCountLo + 1 - dec_i64(x[1 + kXpreLo]) : (int64_t)0);
            c[2] = (uint64_t)pj1.r0;
            c[3] = (uint64_t)pj1.r1;
            c[4] = (uint64_t)pj.r0;
            c[5] = (uint64_t)pj.r1;
            c[6] = (uint64_t)(neg ? kCountHi - 1 - dec_i64(x[1 + kXpreHi]) : kCountHi);
            c[7] = x[1 + kXterm] ^ kInclXor;
        }
        c[8] = range;
        k++;
        if (j < nx - 1) {
            op_reg(o[k], key2, rec_unpack(dec_i64(x[1 + kXsuf])), dec_i64(x[1 + kXsufLo]),
                   dec_i64(x[1 + kXsufHi]), neg ? kFlagNeg : 0u, head(k), range);
            k++;
        }
    }
}

// ---------------------------------------------------------------------------
// The finisher of sum s
// ---------------------------------------------------------------------------
template <class Src>
__device__ __forceinline__ void finisher_block(const PassArgs &pa, const Src &src, const PassWs &w,
                                               int s, FinLds &F, WalkCore &sc, double *terms,
                                               int *lds_src)
{
    const PassArgs &a = pa;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    const size_t n = a.n[s];
    const uint32_t nch = chunks_of_n(n);
    const uint32_t nt = tiles_of(nch, pa.tch);
    if (nt <= 1)
        return;  // the head wrote the result
    const SumView v{a.x[s], n, a.init[s], a.chunk_base(s), nch};
    const uint32_t tb = pa.tile_base(s);
    const uint64_t tag = pa.tag;
    uint64_t n_fast = 0, n_fb = 0, fb_terms = 0;
    int64_t first_fb = -1;
    bool nonfinite = false;
    if (t == 0) {
        F.tally.fast = F.tally.fb = F.tally.terms = 0;
        F.tally.first = -1;
        F.tally.misses = F.tally.nonfinite = 0;
    }
    // a chunk range the finisher walks from its descriptors (fb_desc) or
    // term by term: [fb_lo, fb_hi)
    uint32_t fb_lo = 0, fb_hi = 0;
    bool fb_desc = false;

    // the head's exact sum after the first tile
    double S = a.init[s];
    {
        uint64_t h0 = 0;
        for (int spin = 0; spin <= kSpinLimit; spin++) {
            h0 = uniform_u64(load_relaxed_u64(w.hrec + 2 * (size_t)s));
            if ((h0 >> kTagShift) == tag)
                break;
            __builtin_amdgcn_s_sleep(2);
        }
        const uint32_t nk0 = nch < (uint32_t)kHeadCh ? nch : (uint32_t)kHeadCh;
        if ((h0 >> kTagShift) == tag) {
            S = bitsd(uniform_u64(load_relaxed_u64(w.hrec + 2 * (size_t)s + 1)));
            const uint32_t res = (uint32_t)h0 & 0xFu;
            nonfinite |= ((h0 >> 4) & 1u) != 0;
            for (uint32_t k = 0; k < nk0; k++) {
                if ((res >> k) & 1u) {
                    n_fb++;
                    fb_terms += (uint64_t)chunk_len(n, k);
                    if (first_fb < 0)
                        first_fb = (int64_t)k;
                } else {
                    n_fast++;
                }
            }
        } else {
            fb_hi = nk0;  // the head's sum never came: its chunks term by term
        }
    }

    if (t == 0)
        F.nslots = 0;
    __syncthreads();
    uint32_t base = 1;
    while (base < nt) {
        uint32_t cnt = nt - base < (uint32_t)kFinTiles ? nt - base : (uint32_t)kFinTiles;
        // ---- this lane's tiles (q = kFinLane t + j in the window): their
        // records, polled until their tags show
        const uint32_t q0 = (uint32_t)(kFinLane * t);
        const size_t g0 = (size_t)(tb + base) + q0;
        // (the bounds words of a run with a negative term are polled with
        // the first two: all four words of a record in one round trip)
        uint64_t w0[kFinLane], w1[kFinLane], w2[kFinLane], w3[kFinLane];
        bool got[kFinLane];
#pragma unroll
        for (int j = 0; j < kFinLane; j++) {
            w0[j] = w1[j] = w2[j] = w3[j] = 0;
            got[j] = q0 + (uint32_t)j >= cnt;
        }
        for (int spin = 0; spin <= kSpinLimit; spin++) {
            bool all = true;
#pragma unroll
            for (int j = 0; j < kFinLane; j++) {
                if (!got[j]) {
                    const v2u64 r = load_coherent_16(w.trec + 4 * (g0 + j));
                    const v2u64 b = load_coherent_16(w.trec + 4 * (g0 + j) + 2);
                    w0[j] = r.x;
                    w1[j] = r.y;
                    w2[j] = b.x;
                    w3[j] = b.y;
                    const uint32_t kd = (uint32_t)(r.x >> 17) & 3u;
                    const bool runs = kd == kKindReg || kd == kKindStep;
                    got[j] = (r.x >> kTagShift) == tag && (!runs || rec_w1_ok(tag, r.y)) &&
                             (!runs || !(r.x & kFlagNeg) || (rec_w1_ok(tag, b.x) && rec_w1_ok(tag, b.y)));
                    all &= got[j];
                }
            }
            if (all)
                break;
            __builtin_amdgcn_s_sleep(2);
        }
        // per tile: kk = key | kind << 12 | step shape << 15 | (slot + 1) << 18,
        // its run (a regular tile's, or the run an irregular one ends with),
        // and its number of walk ops (counted at a segment's first tile)
        uint32_t kk[kFinLane];
        Run rr[kFinLane];
        bool lane_nf = false;
        int nop_lane = 0;
#pragma unroll
        for (int j = 0; j < kFinLane; j++) {
            const bool in = q0 + (uint32_t)j < cnt;
            const uint32_t kind = !in ? 0u : got[j] ? (uint32_t)(w0[j] >> 17) & 3u : kKindLost;
            const uint32_t shape = (uint32_t)(w0[j] >> 19) & 7u;
            kk[j] = (in && got[j] ? (uint32_t)w0[j] & kKeyMask : 0u) | kind << kKkKind;
            lane_nf |= in && got[j] && ((uint32_t)w0[j] & kFlagNonFinite);
            rr[j] = run_identity();
            if (kind == kKindReg || kind == kKindStep) {
                const int64_t r0 = rec_w1_r0(w1[j]);
                rr[j].p = Pair{r0, r0 + (int64_t)((w0[j] >> kDrShift) & 3u) - 1};
                rr[j].flags = (uint32_t)w0[j] & (kFlagNeg | kFlagBad);
                if (rr[j].flags & kFlagNeg) {
                    // a run with a negative term: its prefix bounds
                    rr[j].lo = rec_w1_r0(w2[j]);
                    rr[j].hi = rec_w1_r0(w3[j]);
                } else {
                    // rising along either start parity: the largest prefix is
                    // the total
                    rr[j].hi = rr[j].p.r0 > rr[j].p.r1 ? rr[j].p.r0 : rr[j].p.r1;
                }
            }
            if (kind == kKindStep) {
                // a slot for its step record (the words are fetched below)
                const int sl = atomicAdd(&F.nslots, 1);
                if (sl < kStepCap) {
                    F.stile[sl] = (uint32_t)(g0 + j);
                    kk[j] |= shape << kKkShape | (uint32_t)(sl + 1) << kKkSlot;
                }
            }
        }
        // ---- walk ops per tile (at a segment's first tile), their offsets
        // in the window by a workgroup count
        int nop[kFinLane];
#pragma unroll
        for (int j = 0; j < kFinLane; j++) {
            if (q0 + (uint32_t)j < cnt)
                F.kk[q0 + j] = kk[j];
        }
        __syncthreads();
        // the step records' words, one or two per thread, requested now and
        // written to their slots after the scan
        const int nsl = F.nslots < kStepCap ? F.nslots : kStepCap;
        uint64_t recw[2] = {0, 0};
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int qq = t + h * kChunkThreads;
            if (qq < nsl * kStepWords)
                recw[h] = load_relaxed_u64(w.xrec + kStepWords * (size_t)F.stile[qq / kStepWords] +
                                           (qq % kStepWords));
        }
        // segments: a regular tile continues the segment of a regular tile or
        // of an irregular one's last run in its binade; every other tile is a
        // segment of its own
        uint32_t heads = 0u, ends = 0u;
        {
            const uint32_t prev0 = q0 == 0 ? 0u : F.kk[q0 - 1];
            const uint32_t next3 = q0 + kFinLane < cnt ? F.kk[q0 + kFinLane] : 0u;
#pragma unroll
            for (int j = 0; j < kFinLane; j++) {
                const uint32_t q = q0 + (uint32_t)j;
                if (q >= cnt)
                    continue;
                const uint32_t me = kk[j];
                const uint32_t kme = kk_kind(me);
                const bool runs = kme == kKindReg || kme == kKindStep;
                const uint32_t prev = j == 0 ? prev0 : kk[j - 1];
                const uint32_t kpv = kk_kind(prev);
                const uint32_t nx = j + 1 < kFinLane ? kk[j + 1] : next3;
                const bool head = kme != kKindReg || q == 0 || (kpv != kKindReg && kpv != kKindStep) ||
                                  ((prev ^ me) & kKeyMask) != 0u;
                const bool end = !runs || q + 1 >= cnt || kk_kind(nx) != kKindReg ||
                                 ((nx ^ me) & kKeyMask) != 0u;
                heads |= (head ? 1u : 0u) << j;
                ends |= (end ? 1u : 0u) << j;
            }
        }
#pragma unroll
        for (int j = 0; j < kFinLane; j++) {
            nop[j] = 0;
            if (((heads >> j) & 1u) && q0 + (uint32_t)j < cnt)
                nop[j] = kk_ops(kk[j]);
            nop_lane += nop[j];
        }
        const int64_t incn = wave_incl_scan_i64(nop_lane);
        if (lane == 63)
            F.cnt[wave] = (int32_t)incn;
        const uint32_t wnf = __ballot(lane_nf) != 0;
        if (lane == 0)
            F.nf[wave] = wnf;
        if (t == 0)
            F.cut = (int32_t)cnt;
        __syncthreads();
        int off_lane = (int)(incn - nop_lane), nops_tot = 0;
        for (int k = 0; k < kWaves; k++) {
            if (k < wave)
                off_lane += F.cnt[k];
            nops_tot += F.cnt[k];
            nonfinite |= F.nf[k] != 0;
        }
        // the window ends before the first segment whose ops do not fit
        if (nops_tot > kOpCap) {
            int o = off_lane;
#pragma unroll
            for (int j = 0; j < kFinLane; j++) {
                if (nop[j] && o + nop[j] > kOpCap) {
                    atomicMin(&F.cut, (int32_t)(q0 + j));
                    break;
                }
                o += nop[j];
            }
            __syncthreads();
            const uint32_t cut = (uint32_t)F.cut;
            if (cut < cnt) {
                // the ops before the first segment left out
                int oc = off_lane;
#pragma unroll
                for (int j = 0; j < kFinLane; j++) {
                    if (q0 + (uint32_t)j == cut)
                        F.nops_cut = oc;
                    oc += nop[j];
                }
                cnt = cut;
#pragma unroll
                for (int j = 0; j < kFinLane; j++) {
                    const uint32_t q = q0 + (uint32_t)j;
                    if (q >= cnt) {
                        heads &= ~(1u << j);
                        ends &= ~(1u << j);
                        nop[j] = 0;
                    } else if (q + 1 == cnt) {
                        ends |= 1u << j;
                    }
                }
            }
        }
        // ---- the segments' runs: this lane's fold, then an ordered segmented
        // scan over the lanes
        SegRun sr{run_identity(), -1, 0};
#pragma unroll
        for (int j = 0; j < kFinLane; j++) {
            if (q0 + (uint32_t)j >= cnt)
                continue;
            const bool h = (heads >> j) & 1u;
            sr = segr_op(sr, SegRun{rr[j], h ? (int32_t)(q0 + j) : -1, h ? 1 : 0});
        }
        const SegRun rexc = block_excl_segr(sr, F);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int qq = t + h * kChunkThreads;
            if (qq < nsl * kStepWords)
                F.rec[qq / kStepWords][qq % kStepWords] = recw[h];
        }
        // each head's first op in the window, for the lane that ends its segment
        {
            int o = off_lane;
#pragma unroll
            for (int j = 0; j < kFinLane; j++) {
                if (nop[j])
                    F.opoff[q0 + j] = (uint16_t)o;
                o += nop[j];
            }
        }
        __syncthreads();
        const int nops = nops_tot <= kOpCap ? nops_tot : F.nops_cut;
        // ---- the ops: a segment's last tile writes its final op (the run of
        // the segment) and, for an irregular first tile, that tile's other ops
        {
            SegRun run = rexc;
#pragma unroll
            for (int j = 0; j < kFinLane; j++) {
                const uint32_t q = q0 + (uint32_t)j;
                if (q >= cnt)
                    continue;
                const bool h = (heads >> j) & 1u;
                run = segr_op(run, SegRun{rr[j], h ? (int32_t)q : -1, h ? 1 : 0});
                if (!((ends >> j) & 1u))
                    continue;
                const uint32_t qs = (uint32_t)run.start;
                const uint32_t hw = h ? kk[j] : F.kk[qs];
                const uint32_t kind = kk_kind(hw);
                const int o0 = F.opoff[qs];
                const int n_op = kk_ops(hw);
                const uint32_t c_lo = tile_c0(base + qs, pa.tch);
                const uint32_t c_end = tile_c0(base + q + 1, pa.tch);
                const uint64_t range = (uint64_t)c_lo | (uint64_t)(c_end < nch ? c_end : nch) << 32;
                const int slot = (int)(hw >> kKkSlot) - 1;
                if (kind == kKindReg || (kind == kKindStep && slot >= 0)) {
                    auto head_of = [&](int k) {
                        return (k == 0 ? (uint64_t)kOpFirst : 0u) | (k == n_op - 1 ? (uint64_t)kOpLast : 0u) |
                               ((uint64_t)(n_op - 1 - k) << kOpRestShift);
                    };
                    // the segment's run, in the binade of its last tile
                    op_reg(F.ops[o0 + n_op - 1], kk[j] & kKeyMask, run.r.p, run.r.lo, run.r.hi,
                           run.r.flags, head_of(n_op - 1), range);
                    if (kind == kKindStep)
                        op_step_lead(F.ops + o0, F.rec[slot], n_op, range);
                } else {
                    // no O(1) step: the tile's chunks are walked
                    F.ops[o0][0] = kOpFail | kOpFirst | kOpLast | (kind == kKindLost ? (uint64_t)kOpNoDesc : 0u);
                    F.ops[o0][8] = range;
                }
            }
        }
        __syncthreads();
        // ---- the ordered walk over the ops: lane k holds word k of the
        // current op and of the next; S as its bit pattern.  (One call site
        // of the fallback walk: the first window's walk also takes the
        // head's chunks when its sum never came.)
        const uint32_t next = base + cnt;
        {
            auto op_word = [&](int i) { return lane < kOpWords && i < nops ? F.ops[i][lane] : (uint64_t)0; };
            auto W = [&](uint64_t v, int k) { return (uint64_t)readlane_i64((int64_t)v, k); };
            int i = 0;
            for (;;) {
                if (fb_hi > fb_lo) {
                    S = walk_lean(src, v, w.d, fb_lo, fb_hi, S, sc, terms, lds_src, fb_desc, F.tally);
                    S = bitsd(uniform_u64(dbits(S)));
                    fb_lo = fb_hi = 0;
                }
                if (i >= nops)
                    break;
                // ops until one fails (which leaves fb_lo/fb_hi set), on wave 0
                // alone: the waves of a workgroup share one scalar unit
                if (wave == 0) {
                uint64_t sbits = uniform_u64(dbits(S));
                uint64_t sev = sbits;
                uint64_t cur = op_word(i);
                uint32_t fast = 0;
                while (i < nops) {
                    const uint64_t nxt = op_word(i + 1);
                    const uint32_t meta = (uint32_t)W(cur, 0);
                    sev = (meta & kOpFirst) ? sbits : sev;
                    const int64_t m = count_of(bitsd(sbits));
                    const int par = (int)(m & 1);
                    const int64_t a = (int64_t)W(cur, 1), b = (int64_t)W(cur, 2 + par),
                                  c = (int64_t)W(cur, 4 + par);
                    // REG: m in [a, b], then m + c.  CROSS: m in [a, word 6], the
                    // counts before (cb) and through (cj) the crossing term on
                    // either side of the binade's edge, then the one plain add
                    // from the exact sum before the term.
                    const bool reg = (meta & 3u) == kOpReg;
                    const int64_t cb = (meta & kOpJ0) ? m : m + b;
                    const int64_t cj = m + c;
                    const bool edge = (meta & kOpDown) ? (cb >= kCountLo) & (cj < kCountLo)
                                                       : (cb <= kCountHi - 1) & (cj >= kCountHi);
                    const bool okc = (m <= (int64_t)W(cur, 6)) & edge;
                    const bool ok = (key_of(bitsd(sbits)) == ((meta >> 2) & kKeyMask)) &
                                    ((meta & 3u) != kOpFail) & (m >= a) & (reg ? m <= b : okc);
                    const uint64_t crossed =
                        uniform_u64(dbits(bitsd(sbits + (uint64_t)(cb - m)) + bitsd(W(cur, 7))));
                    const uint64_t after = reg ? sbits + (uint64_t)c : crossed;
                    const uint64_t range = W(cur, 8);
                    if (!ok) {
                        // the event's chunks, from the sum before it
                        fb_lo = (uint32_t)range;
                        fb_hi = (uint32_t)(range >> 32);
                        fb_desc = !(meta & kOpNoDesc);
                        sbits = sev;
                        i += 1 + (int)(meta >> kOpRestShift);
                        break;
                    }
                    sbits = after;
                    if (meta & kOpLast)
                        fast += (uint32_t)(range >> 32) - (uint32_t)range;
                    i++;
                    cur = nxt;
                }
                if (lane == 0) {
                    F.wk.sbits = sbits;
                    F.wk.i = i;
                    F.wk.fast = fast;
                    F.wk.fb_lo = fb_lo;
                    F.wk.fb_hi = fb_hi;
                    F.wk.fb_desc = fb_desc;
                }
                }
                __syncthreads();
                S = bitsd(F.wk.sbits);
                i = F.wk.i;
                n_fast += F.wk.fast;
                fb_lo = F.wk.fb_lo;
                fb_hi = F.wk.fb_hi;
                fb_desc = F.wk.fb_desc != 0;
                __syncthreads();
            }
        }
        if (t == 0)
            F.nslots = 0;
        __syncthreads();  // the window's LDS is reused by the next one
        base = next;
    }
    if (t == 0) {
        pa.outs[s] = S;
        if (pa.means)
            pa.means[s] = (float)(S / (double)n);  // ADR-1464: (float)(sum / windows)
        if (pa.stats) {
            const FinTally &ft = F.tally;
            exseq_stats st;
            st.chunks = nch;
            st.fast_chunks = n_fast + ft.fast;
            st.fallback_chunks = n_fb + ft.fb;
            st.fallback_terms = fb_terms + ft.terms;
            st.first_fallback = first_fb >= 0 ? first_fb : ft.first;
            st.flags = (nonfinite || ft.nonfinite) ? EXSEQ_STAT_NONFINITE : 0u;
            st.plan_misses = ft.misses;
            pa.stats[s] = st;
        }
    }
}

// ---------------------------------------------------------------------------
// A tile after a sum's first: eight chunks
// ---------------------------------------------------------------------------
// Each wave forms two chunks of the tile on its own: chunk 2w from
// registers, chunk 2w + 1 staged in LDS slot w.  Lane l holds terms
// 256 j + 4 l .. 256 j + 4 l + 3 of its chunk for j = 0 .. 3 (group j is the
// part a wave of the workgroup layout holds), so one reduction over the wave
// forms a chunk and nothing is joined across waves.

// Lane l's group-j terms of chunk c of a sum (+0.0 past its end).
__device__ __forceinline__ Four wave_four(const SumView &v, size_t c, int j)
{
    return load_four(v.x, v.n, c * kChunk + 256 * (size_t)j + 4 * (size_t)lane_id(), true);
}

// Chunk c into LDS slot k by this wave alone, in the workgroup layout's
// arrangement (group j where wave j would put it), so that staged_chunk reads
// lane t's four terms for a block-wide step and staged_four this lane's.
__device__ __forceinline__ void stage_wave_chunk(double *stage, int k, const SumView &v, size_t c, bool direct)
{
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < 4; j++) {
        double *base = stage + k * kChunk + j * 256;
        const size_t first = c * kChunk + 256 * (size_t)j + 4 * (size_t)lane;
        if (direct) {
            const double *p = v.x + first;
            __builtin_amdgcn_global_load_lds((const void *)p, (__attribute__((address_space(3))) void *)base,
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(p + 2),
                                             (__attribute__((address_space(3))) void *)(base + 128), 16, 0, 0);
        } else {
            const Four f = load_four(v.x, v.n, first, true);
            base[2 * lane] = f.v[0];
            base[2 * lane + 1] = f.v[1];
            base[128 + 2 * lane] = f.v[2];
            base[128 + 2 * lane + 1] = f.v[3];
        }
    }
}

__device__ __forceinline__ Four staged_four(const double *stage, int k, int j)
{
    const int lane = lane_id();
    const double *base = stage + k * kChunk + j * 256;
    Four f;
    f.v[0] = base[2 * lane];
    f.v[1] = base[2 * lane + 1];
    f.v[2] = base[128 + 2 * lane];
    f.v[3] = base[128 + 2 * lane + 1];
    f.cnt = 4;
    return f;
}

// The fixed-tree sum of a chunk held as four groups per lane.
__device__ __forceinline__ double lane_tree(const Four *g)
{
    double q[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
        q[j] = (g[j].v[0] + g[j].v[1]) + (g[j].v[2] + g[j].v[3]);
    return (q[0] + q[1]) + (q[2] + q[3]);
}

// A chunk's run under `key`, formed by one wave from its four groups, the
// same in every lane.  Where no term ties and every increment has one sign
// (the bit tests of wave_runs on all 1024 terms), one integer reduction;
// otherwise each group's ordered run (wave_run) and the four composed in
// order.  A key with no fast path gives only the non-finite flag.  Clamped.
__device__ __forceinline__ WaveRun chunk_run(const Four *g, uint32_t key)
{
    if (!key_has_fast_path(key)) {
        bool nf = false;
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                nf |= is_nonfinite(g[j].v[i]);
        return WaveRun{pair_identity(), 0, 0, __ballot(nf) ? kFlagNonFinite : 0u};
    }
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool flip = (key & 0x800u) != 0u;
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
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                term(g[j].v[i] * fac);
    } else {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const double y = ldexp(g[j].v[i], scale);
                term(flip ? -y : y);
            }
    }
    const bool ok = tacc == 0u && (((hand ^ kMagic0Hi) | (hor ^ kMagic0Hi)) >> 20) == 0u;
    const bool pos = __ballot(!((hand >> 19) & 1u)) == 0;  // every a0 >= M0
    const bool neg = __ballot((hor >> 19) & 1u) == 0;      // every a0 < M0
    if (__ballot(!ok) == 0 && (pos || neg)) {
        const int64_t r = wave_sum_i64((int64_t)(sum - 16 * (uint64_t)kMagic0Bits));
        return clamp_run(pos ? WaveRun{Pair{r, r}, 0, r, 0u} : WaveRun{Pair{r, r}, r, 0, kFlagNeg});
    }
    // the groups' runs composed in order as they come (join_waves)
    WaveRun acc{};
    bool plain = true, fall = true;
    int64_t tot = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const WaveRun q = wave_run(g[j], key);
        plain &= rising_run(q.p, q.flags);
        fall &= falling_run(q.p, q.lo, q.hi, q.flags);
        tot += q.p.r0;
        if (j == 0) {
            acc = q;
        } else {
            const Run c = run_compose(Run{acc.p, acc.lo, acc.hi, acc.flags}, Run{q.p, q.lo, q.hi, q.flags});
            acc = WaveRun{c.p, c.lo, c.hi, c.flags};
        }
    }
    if (!(acc.flags & kFlagNeg))
        acc.hi = acc.p.r0 > acc.p.r1 ? acc.p.r0 : acc.p.r1;
    return clamp_run(plain  ? WaveRun{Pair{tot, tot}, 0, tot, 0u}
                     : fall ? WaveRun{Pair{tot, tot}, tot, 0, kFlagNeg}
                            : acc);
}

// The look-back's first level, by one wave: the plan prefix before the
// tile from the tile words of its group (into L); the group's last tile
// publishes the group's sum (or its inclusive prefix) as soon as known.
__device__ __forceinline__ void level1(PassTileLds &L, const uint64_t *st, int pg, uint32_t lg, uint32_t epoch,
                                       uint64_t *gs0, double Ttile, int slot = 0)
{
    double v1;
    bool ok1;
    const bool found = lb_level1(st, pg, epoch, v1, ok1);
    if (lane_id() == 0) {
        L.lb1[slot] = v1;
        L.lb_found[slot] = found;
        L.lb_ok1[slot] = ok1;
        if (found || lg == 0)
            L.lb_stop[slot] = 1;
        if (pg == (int)kGroup - 1 && ok1)
            store_relaxed_u64(gs0 + lg, st_pack(epoch, found ? kStIncl : kStAgg, v1 + Ttile));
    }
}

// The record of one sum's tile, whose chunks c0 .. c0 + nk - 1 have their
// runs, keys and crossings in L at q0 .. q0 + nk - 1 (g: the tile in the
// launch).  Every thread of the workgroup calls it; the tile's descriptor
// stores are complete before any tagged word of its record.
// A regular tile's record, by one lane, once the tile's descriptor stores
// are complete: the chunks' runs in order (plain ones add up), then the
// bounds of a run with a negative term, and once they are complete its
// first two words in one 16-byte store (every word carries bits of the
// launch tag).
__device__ __forceinline__ void reg_record(const PassWs &w, uint64_t tag, uint32_t g, const PassTileLds &L,
                                       int q0, int nk)
{
    uint64_t *trec = w.trec + 4 * (size_t)g;
    Run tr = run_identity();
    bool plain = true, fall = true;
    int64_t sum = 0;
    for (int k = 0; k < nk; k++) {
        const WaveRun &q = L.join[q0 + k];
        plain &= rising_run(q.p, q.flags);
        fall &= falling_run(q.p, q.lo, q.hi, q.flags);
        sum += q.p.r0;
    }
    if (plain) {
        tr = Run{Pair{sum, sum}, 0, sum, 0u};
    } else if (fall) {
        tr = Run{Pair{sum, sum}, sum, 0, kFlagNeg};
    } else {
        for (int k = 0; k < nk; k++) {
            const WaveRun r = L.join[q0 + k];
            tr = run_compose_sat(tr, Run{r.p, r.lo, r.hi, r.flags});
        }
        if (!(tr.flags & kFlagNeg))
            tr.hi = run_top(tr);
    }
    // a run past the width of a binade never applies; bounded runs
    // keep the finisher's sums over a window far from overflow
    const int64_t lim = kCountLo + 1;
    if (tr.p.r0 > lim || tr.p.r0 < -lim || tr.lo < -lim || tr.hi > lim) {
        tr.flags |= kFlagBad;
        tr.p = pair_identity();
        tr.lo = tr.hi = 0;
    }
    if (tr.flags & kFlagNeg) {
        store_coherent_16(trec + 2, rec_w1(tag, tr.lo), rec_w1(tag, tr.hi));
        stores_complete();
    }
    store_coherent_16(trec, rec_w0(tag, kKindReg, tr.flags, tr.p.r1 - tr.p.r0, L.key[q0]),
                      rec_w1(tag, tr.p.r0));
}

__device__ __forceinline__ void publish_tile(const PassWs &w, uint64_t tag, uint32_t g, PassTileLds &L, int q0,
                                             int nk, bool regular, uint32_t found, size_t n, uint32_t c0)
{
    const int t = threadIdx.x;
    uint64_t *trec = w.trec + 4 * (size_t)g;
    if (regular) {
        // once every wave's descriptor stores are complete
        stores_complete();
        __syncthreads();
        if (t == 0)
            reg_record(w, tag, g, L, q0, nk);
        return;
    }
    // An irregular tile: its O(1) step -- the chunks before the first located
    // crossing as one run A, then up to kMaxCross crossings, each with the
    // chunks after it (in the next binade) folded into its rest-of-chunk
    // run.  Built in LDS by lane 0.  Any other shape is walked by the
    // finisher chunk by chunk.
    bool fast = true;
    uint32_t nfl = 0u;
    if (t == 0) {
        Run A = run_identity();
        uint32_t akey = 0u;
        int nx = 0;
        uint32_t next_key = 0u;  // the binade the chunks after the last crossing are in
        Run suf = run_identity();
        Pair whole = pair_identity();
        uint64_t *xr = nullptr;  // the current crossing's words in L.rec
        for (int k = 0; k < nk; k++)
            nfl |= L.join[q0 + k].flags & kFlagNonFinite;
        auto close_crossing = [&]() {
            const int64_t lim = (int64_t)1 << 56;
            fast = fast && !(suf.flags & kFlagBad) && whole.r0 < lim && whole.r1 < lim &&
                   whole.r0 > -lim && whole.r1 > -lim;
            xr[1 + kXsuf] = enc_i64(rec_pack(suf.p));
            xr[1 + kXsufLo] = enc_i64(suf.lo);
            xr[1 + kXsufHi] = enc_i64(suf.hi);
            xr[1 + kXwhole] = enc_i64(rec_pack(whole));
            xr[0] |= (uint64_t)((suf.flags & kFlagNeg) ? 1u : 0u) << 13;
        };
        for (int k = 0; fast && k < nk; k++) {
            const WaveRun &q = L.join[q0 + k];
            const uint32_t kk = L.key[q0 + k];
            if ((found >> k) & 1u) {
                if (nx == kMaxCross || (nx == 0 ? (akey != 0u && akey != kk) : kk != next_key)) {
                    fast = false;
                    break;
                }
                if (nx > 0)
                    close_crossing();
                xr = L.rec + 4 + kXrecW * nx;
                const bool down = L.down[q0 + k] != 0u;
#pragma unroll
                for (int c = 0; c < kCrossWords; c++)
                    xr[1 + c] = L.xw[q0 + k][c];
                xr[0] = (uint64_t)(kk & kKeyMask) | ((uint64_t)down << 12) |
                        ((uint64_t)chunk_len(n, c0 + k) << 16);
                suf = Run{rec_unpack(dec_i64(xr[1 + kXsuf])), dec_i64(xr[1 + kXsufLo]),
                          dec_i64(xr[1 + kXsufHi]), q.flags & kFlagNeg};
                whole = rec_unpack(dec_i64(xr[1 + kXwhole]));
                next_key = down ? kk - 1u : kk + 1u;
                nx++;
                continue;
            }
            fast = key_has_fast_path(kk) && !(q.flags & (kFlagBad | kFlagNonFinite));
            if (nx == 0) {
                fast = fast && (akey == 0u || akey == kk);
                A = run_compose_sat(A, Run{q.p, q.lo, q.hi, q.flags});
                akey = kk;
            } else {
                fast = fast && kk == next_key;
                suf = run_compose_sat(suf, Run{q.p, q.lo, q.hi, q.flags & kFlagNeg});
                whole = compose(whole, q.p);
            }
        }
        if (fast && nx > 0)
            close_crossing();
        fast = fast && (akey != 0u || nx > 0) && !(A.flags & kFlagBad);
        // the run the tile ends with (the rest after its last crossing, or A
        // without one) and its binade: published in the tile's record words
        // so that the finisher composes the regular tiles after it with it
        {
            const bool lastdown = nx > 0 && ((L.rec[4 + kXrecW * (nx - 1)] >> 12) & 1u);
            const Run ex = nx > 0 ? suf : A;
            const bool neg = (ex.flags & kFlagNeg) || lastdown;
            const int64_t lim = kCountLo + 1;
            fast = fast && ex.p.r0 <= lim && ex.p.r0 >= -lim && ex.p.r1 <= lim && ex.p.r1 >= -lim &&
                   (!neg || (ex.lo >= -lim && ex.hi <= lim));
            L.xexit[0] = (uint64_t)(nx > 0 ? next_key : akey) | ((uint64_t)neg << 14) |
                         ((uint64_t)(ex.p.r1 - ex.p.r0 + 1) << 32);
            L.xexit[1] = rec_w1(tag, ex.p.r0);
            L.xexit[2] = rec_w1(tag, ex.lo);
            L.xexit[3] = rec_w1(tag, ex.hi);
        }
        L.rec[0] = (uint64_t)(akey & kKeyMask) | ((uint64_t)(akey != 0u) << 12) |
                   ((uint64_t)nx << 13) | ((uint64_t)((A.flags >> 14) & 3u) << 15) |
                   ((uint64_t)(A.p.r1 - A.p.r0 + 1) << 17);
        L.rec[1] = enc_i64(A.p.r0);
        L.rec[2] = enc_i64(A.lo);
        L.rec[3] = enc_i64(A.hi);
        L.lb_found[0] = fast ? 1 : 0;  // reused: tells the other lanes
    }
    __syncthreads();
    fast = L.lb_found[0] != 0;
    const bool xneg = ((L.xexit[0] >> 14) & 1u) != 0;
    if (fast && t < kStepWords)
        store_relaxed_u64(w.xrec + kStepWords * (size_t)g + t, L.rec[t]);
    if (fast && t >= 64 && t < 64 + (xneg ? 3 : 1))
        store_relaxed_u64(trec + (t - 63), L.xexit[t - 63]);
    stores_complete();
    __syncthreads();
    if (t == 0) {
        const uint64_t x0 = L.xexit[0];
        const uint32_t shape = (uint32_t)(L.rec[0] >> 12) & 7u;  // A present, crossings
        store_relaxed_u64(trec, fast ? rec_w0(tag, kKindStep, nfl | (xneg ? kFlagNeg : 0u),
                                              (int64_t)(x0 >> 32) - 1, (uint32_t)x0 & kKeyMask, shape)
                                     : rec_w0(tag, kKindSlow, nfl, 0, 0u));
    }
}

// ---------------------------------------------------------------------------
// Interleaved sums: k fields per record, field s of record r at x[r k + s]
// (ADR-1464 "float_ssim_cuda adds its frame sums in the CPU's raster order,
// on the host", Decision: the l*c*s, l, c, s sums of a pass), k = 2 or 4.
// One workgroup takes the same tile of all k sums, 8 / k chunks of each, so
// that every cache line of the records is read once, with 16-byte loads:
// the tile's records go through LDS in two halves, written field by field,
// and each wave takes two chunks of one sum (the first from registers, the
// second from the LDS image).
// ---------------------------------------------------------------------------
struct PassStrided {
    static constexpr int kLdsInts = 1;
    static constexpr bool kInter = true;
    // Three waves per SIMD: the interleaved tile's 16-byte record loads and
    // field images need more registers than four waves leave, and spilling
    // them costs more than the fourth wave gains.
    static constexpr int kPassWaves = 3;
    uint32_t k;
    // lane t's terms 4t .. 4t + 3 of chunk c of the sum viewed by v (+0.0
    // past its end), for the head, the walks and a located crossing
    __device__ __forceinline__ Four chunk_v(const SumView &v, size_t c, int *) const
    {
        const size_t first = c * kChunk + 4 * (size_t)threadIdx.x;
        Four f;
        f.cnt = first < v.n ? (int)(v.n - first < 4 ? v.n - first : 4) : 0;
#pragma unroll
        for (int i = 0; i < 4; i++)
            f.v[i] = i < f.cnt ? v.x[(first + (size_t)i) * k] : 0.0;
        return f;
    }
};

// Lane l's group-g terms of chunk c of a sum of interleaved terms (x: its
// first term; stride k), read again from memory.
__device__ __forceinline__ Four strided_wave_four(const double *x, size_t n, uint32_t k, size_t c, int g)
{
    const size_t first = c * kChunk + 256 * (size_t)g + 4 * (size_t)lane_id();
    Four f;
    f.cnt = 4;
#pragma unroll
    for (int i = 0; i < 4; i++)
        f.v[i] = first + (size_t)i < n ? x[(first + (size_t)i) * k] : 0.0;
    return f;
}

// Four consecutive terms of an LDS image in natural order: this lane's
// group g of a chunk (wave layout), or lane t's four (workgroup layout).
__device__ __forceinline__ Four image_four(const double *base, size_t at)
{
    const double *p = base + at;
    Four f;
    f.v[0] = p[0];
    f.v[1] = p[1];
    f.v[2] = p[2];
    f.v[3] = p[3];
    f.cnt = 4;
    return f;
}

template <class Src>
__device__ __forceinline__ void inter_tile_block(const PassArgs &pa, const Src &src, const PassWs &w, uint32_t i,
                                                 PassTileLds &L, WalkCore &sc, CrossLds &xl, double *stage,
                                                 int *lds_src)
{
    const int K = (int)pa.inter, tch = (int)pa.tch, half = tch / 2;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    const size_t n = pa.n[0];  // every sum's length
    const uint32_t nch = chunks_of_n(n);
    const uint32_t c0 = tile_c0(i, (uint32_t)tch);
    const int nk = (int)(nch - c0 < (uint32_t)tch ? nch - c0 : (uint32_t)tch);
    const uint32_t mode = pa.flags & EXSEQ_PLAN_MASK;
    const uint64_t tag = pa.tag;
    const double *xb = pa.x[0];  // record 0, field 0
    const int sw = wave / half;                 // this wave's sum
    const int jr = wave % half, js = half + jr; // its chunks in the sum's tile
    const int qr = sw * tch + jr, qs = sw * tch + js;  // their places in L
    const int Fs = half * kChunk + 2;           // doubles per field of an LDS image
    const bool lead = jr == 0;                  // the sum's first wave
    // With four sums each wave holds all of its sum's chunks in the tile, and
    // everything up to the records is the wave's own: its barriers are
    // wave barriers.  With two, two waves share a sum and meet at the
    // workgroup's.
    const bool solo = half == 1;
    auto sync = [&]() {
        if (solo) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        } else {
            __syncthreads();
        }
    };

    if (t < 4)
        L.lb_stop[t] = 0;
    // ---- the terms: the tile's records in two halves, each read once with
    // 16-byte loads and written to LDS field by field
    const bool vec = ((reinterpret_cast<uintptr_t>(xb) & 15u) == 0u);
    // all sixteen 16-byte loads of the thread requested at once (both
    // halves), then each half through LDS
    v2f64 ld[16];
#pragma unroll
    for (int m = 0; m < 16; m++) {
        const size_t r0 = ((size_t)c0 + (size_t)(m >> 3) * (size_t)half) * kChunk;
        const size_t d = 2 * (256 * (size_t)(m & 7) + (size_t)t);  // double of the half
        const size_t rec = r0 + d / (size_t)K;
        ld[m].x = 0.0;
        ld[m].y = 0.0;
        if (rec < n) {
            const double *p = xb + r0 * (size_t)K + d;
            if (vec) {
                ld[m] = __builtin_nontemporal_load(reinterpret_cast<const v2f64 *>(p));
            } else {
                ld[m].x = p[0];
                ld[m].y = p[1];
            }
        }
    }
    Four f[4];
#pragma unroll
    for (int ph = 0; ph < 2; ph++) {
        if (ph)
            __syncthreads();  // the first half's image has been read
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const size_t d = 2 * (256 * (size_t)m + (size_t)t);
            const int rr = (int)(d / (size_t)K), fld = (int)(d % (size_t)K);
            stage[fld * Fs + rr] = ld[8 * ph + m].x;
            stage[(fld + 1) * Fs + rr] = ld[8 * ph + m].y;
        }
        __syncthreads();
        if (ph == 0) {
#pragma unroll
            for (int g = 0; g < 4; g++)
                f[g] = image_four(stage + sw * Fs + jr * kChunk, 256 * (size_t)g + 4 * (size_t)lane);
        }
    }
    const double *img = stage + sw * Fs + jr * kChunk;  // this wave's second chunk
    // ---- the chunk sums (fixed tree)
    {
        double ws[2];
        ws[0] = jr < nk ? lane_tree(f) : 0.0;
        Four q[4];
#pragma unroll
        for (int g = 0; g < 4; g++)
            q[g] = image_four(img, 256 * (size_t)g + 4 * (size_t)lane);
        ws[1] = js < nk ? lane_tree(q) : 0.0;
        wave_sum_f64_n<2>(ws);
        if (lane == 0) {
            L.tsum[qr] = ws[0];
            L.tsum[qs] = ws[1];
        }
    }
    sync();
    double Ttile = 0.0;
    for (int j = 0; j < nk; j++)
        Ttile += L.tsum[sw * tch + j];

    // ---- the plan of this wave's sum, and its runs formed meanwhile
    uint64_t *st0 = w.st + pa.tile_base(sw);
    uint64_t *gs0 = w.gst + pa.group_base(sw);
    const uint32_t lg = i / kGroup, pg = i % kGroup;
    const bool lookback = mode != EXSEQ_PLAN_FIXED;
    if (lookback && lead && lane == 0)
        store_relaxed_u64(st0 + i, st_pack(pa.epoch, kStAgg, Ttile));
    const bool last_in_group = lookback && pg == kGroup - 1;
    if (last_in_group && lead)
        level1(L, st0 + kGroup * lg, (int)pg, lg, pa.epoch, gs0, Ttile, sw);
    const bool spec = lookback;
    uint32_t gk[2] = {0u, 0u};
    WaveRun run[2];
    if (spec) {
        const double mean = Ttile / (double)nk;
        double pk = pa.init[sw] + (double)c0 * mean;
        for (int j = 0; j < tch; j++) {
            const uint32_t kk = (uint32_t)__builtin_amdgcn_readfirstlane((int)plan_key(pk, pa.flags));
            if (j == jr)
                gk[0] = kk;
            if (j == js)
                gk[1] = kk;
            pk += L.tsum[sw * tch + j];
        }
        if (jr < nk)
            run[0] = chunk_run(f, gk[0]);
        if (js < nk) {
            Four q[4];
#pragma unroll
            for (int g = 0; g < 4; g++)
                q[g] = image_four(img, 256 * (size_t)g + 4 * (size_t)lane);
            run[1] = chunk_run(q, gk[1]);
        }
    }
    double P = pa.init[sw];
    if (lookback) {
        // the first level by the sum's first wave, the second by its second
        // (the same wave where a sum has one)
        if (lead && !last_in_group)
            level1(L, st0 + kGroup * lg, (int)pg, lg, pa.epoch, gs0, Ttile, sw);
        if (jr == (half > 1 ? 1 : 0)) {
            bool ok2 = true;
            double v2 = 0.0;
            if (lg > 0)
                v2 = lb_level2(gs0, lg, pa.epoch, &L.lb_stop[sw], ok2);
            if (lane == 0) {
                L.lb2[sw] = v2;
                L.lb_ok2[sw] = ok2;
            }
        }
        sync();
        const bool found = L.lb_found[sw] != 0;
        const bool ok = L.lb_ok1[sw] && (found || (lg > 0 && L.lb_ok2[sw]));
        P = !ok ? __builtin_nan("") : (found ? L.lb1[sw] : L.lb2[sw] + L.lb1[sw]);
        if (lead && lane == 0 && ok) {
            store_relaxed_u64(st0 + i, st_pack(pa.epoch, kStIncl, P + Ttile));
            if (pg == kGroup - 1)
                store_relaxed_u64(gs0 + lg, st_pack(pa.epoch, kStIncl, P + Ttile));
        }
    }
    // ---- the planned prefix and binade of this wave's chunks
    uint32_t kc[2] = {0u, 0u};
    {
        double pk = P;
        for (int j = 0; j < tch; j++) {
            const double tk = L.tsum[sw * tch + j];
            if (j == jr || j == js) {
                const int h = j == js ? 1 : 0;
                const int q = sw * tch + j;
                const uint32_t ka = key_of(pk), kb = key_of(pk + tk);
                const uint32_t kp = plan_key(pk, pa.flags);
                if (h)
                    kc[1] = kp;
                else
                    kc[0] = kp;
                if (lane == 0) {
                    L.pk[q] = pk;
                    L.key[q] = kp;
                    L.cross[q] = kb != ka;
                    L.down[q] = ((kb ^ ka) & 0x800u) == 0u && (kb & 0x7FFu) < (ka & 0x7FFu);
                }
            }
            pk += tk;
        }
    }
    // ---- the runs not formed under the guess (the register chunk read
    // again from memory)
#pragma unroll 1
    for (int h = 0; h < 2; h++) {
        const int j = h ? js : jr;
        const uint32_t kh = h ? kc[1] : kc[0];
        if (j >= nk || (spec && (h ? gk[1] : gk[0]) == kh))
            continue;
        Four q[4];
#pragma unroll
        for (int g = 0; g < 4; g++)
            q[g] = h ? image_four(img, 256 * (size_t)g + 4 * (size_t)lane)
                     : strided_wave_four(xb + sw, n, (uint32_t)K, c0 + (uint32_t)jr, g);
        const WaveRun r = chunk_run(q, kh);
        if (h)
            run[1] = r;
        else
            run[0] = r;
    }
    // ---- the binade edges and the descriptors (lane h: this wave's chunk h)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (lane < 2 && (lane ? js : jr) < nk) {
        const int h = lane, j = h ? js : jr, q = sw * tch + j;
        const WaveRun r = h ? run[1] : run[0];
        const uint32_t kk = L.key[q];
        const double pk = L.pk[q];
        const bool dn = L.down[q] != 0u;
        bool cc = L.cross[q] != 0u;
        if (key_has_fast_path(kk) && kk == key_of(pk)) {
            const int64_t m = count_of(pk);
            const int64_t mg = plan_margin(c0 + (uint32_t)j + 1);
            bool near = m < count_floor(kk) + mg;
            if (r.flags & kFlagNeg)
                near |= m + r.lo - mg < kCountLo + 1 || m + r.hi + mg > kCountHi - 1;
            else
                near |= m + r.hi + mg > kCountHi;
            cc |= near;
        }
        L.join[q] = r;
        L.cross[q] = cc;
        store_desc_coherent(w.d, (size_t)pa.chunk_base(sw) + c0 + (size_t)j, kk, r, cc ? kFlagCross : 0u);
        L.locate[q] = cc && key_has_fast_path(kk) && kk == key_of(pk) &&
                      key_has_fast_path(dn ? kk - 1u : kk + 1u) && !(r.flags & kFlagNonFinite);
    }
    // ---- a sum alone in its wave: its record at once when it is regular
    // (its descriptors are this wave's stores)
    uint32_t regmask = 0u;
    bool done = false;
    if (solo) {
        sync();
        bool reg = true;
        for (int j = 0; j < nk; j++) {
            const int q = sw * tch + j;
            reg &= key_has_fast_path(L.key[q]) && L.key[q] == L.key[sw * tch] && !L.cross[q] &&
                   !(L.join[q].flags & (kFlagBad | kFlagNonFinite));
        }
        if (reg) {
            stores_complete();
            if (lane == 0)
                reg_record(w, tag, pa.tile_base(sw) + i, L, sw * tch, nk);
        }
        // the irregular sums, if any, by the whole workgroup
        done = __syncthreads_or(reg ? 0 : 1) == 0;
    } else {
        __syncthreads();
    }
    if (done)
        return;
    // ---- per sum: its crossings located by the whole workgroup, and an
    // irregular sum's record
#pragma unroll 1
    for (int s = 0; s < K; s++) {
        const int q0 = s * tch;
        uint32_t xmask = 0u;
        bool regular = true;
        for (int j = 0; j < nk; j++) {
            const int q = q0 + j;
            xmask |= L.locate[q] ? 1u << j : 0u;
            regular &= key_has_fast_path(L.key[q]) && L.key[q] == L.key[q0] && !L.cross[q] &&
                       !(L.join[q].flags & (kFlagBad | kFlagNonFinite));
        }
        xmask = (uint32_t)__builtin_amdgcn_readfirstlane((int)xmask);
        regular = __builtin_amdgcn_readfirstlane((int)regular) != 0;
        const SumView vs{xb + s, n, pa.init[s], pa.chunk_base(s), nch};
        uint32_t found = 0u;
        int buf = 0;
#pragma unroll 1
        for (int j = 0; j < nk; j++) {
            if (!((xmask >> j) & 1u))
                continue;
            // the chunk's terms in the workgroup layout: from the LDS image
            // (the tile's second half), else read again from memory
            const int len = chunk_len(n, c0 + (size_t)j);
            Four q;
            if (j >= half) {
                q = image_four(stage + s * Fs + (j - half) * kChunk, 4 * (size_t)t);
                q.cnt = len - 4 * t >= 4 ? 4 : (len - 4 * t > 0 ? len - 4 * t : 0);
            } else {
                q = src.chunk_v(vs, c0 + (size_t)j, lds_src);
            }
            uint64_t xw[kCrossWords];
            if (crossing_find(q, len, L.key[q0 + j], count_of(L.pk[q0 + j]), L.down[q0 + j] != 0u, sc, xl,
                              buf, xw)) {
                found |= 1u << j;
                if (t == 0) {
#pragma unroll
                    for (int q2 = 0; q2 < kCrossWords; q2++)
                        L.xw[q0 + j][q2] = xw[q2];
                }
            }
        }
        if (xmask)
            __syncthreads();
        if (!regular) {
            publish_tile(w, tag, pa.tile_base(s) + i, L, q0, nk, false, found, n, c0);
            __syncthreads();  // the next sum's record reuses L.rec
        }
        regmask |= regular ? 1u << s : 0u;
    }
    if (solo)
        return;  // (the regular sums' records are out)
    // the regular sums' records together: lane 0 of wave s for sum s, once
    // the tile's descriptor stores are complete
    stores_complete();
    __syncthreads();
    if (lane == 0 && wave < K && ((regmask >> wave) & 1u))
        reg_record(w, tag, pa.tile_base(wave) + i, L, wave * tch, nk);
}

template <class Src>
__device__ __forceinline__ void tile_block(const PassArgs &pa, const Src &src, const PassWs &w,
                                           int s, uint32_t i, PassTileLds &L, WalkCore &sc,
                                           CrossLds &xl, double *stage, int *lds_src)
{
    const PassArgs &a = pa;
    const int t = threadIdx.x, lane = lane_id(), wave = wave_id();
    const size_t n = a.n[s];
    const uint32_t nch = chunks_of_n(n);
    const uint32_t c0 = tile_c0(i, pa.tch);
    const int nk = (int)(nch - c0 < (uint32_t)kTileCh ? nch - c0 : (uint32_t)kTileCh);
    const uint32_t mode = a.flags & EXSEQ_PLAN_MASK;
    const uint64_t tag = pa.tag;
    const uint32_t g = pa.tile_base(s) + i;           // the tile in the launch
    const size_t gc0 = (size_t)a.chunk_base(s) + c0;  // its first chunk in the launch
    const SumView v{a.x[s], n, a.init[s], a.chunk_base(s), nch};
    const int cr = 2 * wave, cs = 2 * wave + 1;       // this wave's chunks

    if (t == 0)
        L.lb_stop[0] = 0;
    // ---- the terms: chunk cr into registers, chunk cs into LDS slot `wave`
    Four f[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if (cr < nk) {
            f[j] = wave_four(v, c0 + cr, j);
        } else {
#pragma unroll
            for (int q = 0; q < 4; q++)
                f[j].v[q] = 0.0;
            f[j].cnt = 0;
        }
    }
    if (cs < nk) {
        const bool direct = ((reinterpret_cast<uintptr_t>(v.x) & 15u) == 0u) &&
                            (size_t)(c0 + cs + 1) * kChunk <= n;
        stage_wave_chunk(stage, wave, v, c0 + cs, direct);
    }
    // ---- the fixed-tree sum of both chunks
    {
        double ws[2];
        ws[0] = lane_tree(f);
        ws[1] = 0.0;
        if (cs < nk) {
            // the wave reads back only what its own loads put in LDS
            __builtin_amdgcn_s_waitcnt(0);
            Four q[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                q[j] = staged_four(stage, wave, j);
            ws[1] = lane_tree(q);
        }
        wave_sum_f64_n<2>(ws);
        if (lane == 0) {
            L.tsum[cr] = ws[0];
            L.tsum[cs] = ws[1];
        }
    }
    __syncthreads();
    // (the chunk sums are read from LDS where needed, not held in registers)
    double Ttile = 0.0;
#pragma unroll
    for (int k = 0; k < kTileCh; k++)
        Ttile += L.tsum[k];

    // ---- the plan, and the runs formed while it is looked up
    uint64_t *st0 = w.st + pa.tile_base(s);
    uint64_t *gs0 = w.gst + pa.group_base(s);
    const uint32_t lg = i / kGroup, pg = i % kGroup;
    const bool lookback = mode != EXSEQ_PLAN_FIXED;
    if (lookback && t == 0)
        store_relaxed_u64(st0 + i, st_pack(a.epoch, kStAgg, Ttile));
    // A group's last tile publishes the group's sum from its look-back over
    // the group: its first wave does that first.
    const bool last_in_group = lookback && pg == kGroup - 1;
    if (last_in_group && wave == 0)
        level1(L, st0 + kGroup * lg, (int)pg, lg, a.epoch, gs0, Ttile);
    // A guess of every chunk's planned binade, from the prefix before the
    // tile taken as its first chunk's index times the tile's mean chunk sum:
    // the runs are formed under it while the look-back waits for the tiles
    // before (the plan decides speed only; a chunk whose guess differs from
    // its planned binade is formed again).
    const bool spec = lookback;
    uint32_t gk[2] = {0u, 0u};
    WaveRun run[2];
    if (spec) {
        const double mean = Ttile / (double)nk;
        double pk = a.init[s] + (double)c0 * mean;
#pragma unroll
        for (int k = 0; k < kTileCh; k++) {
            const uint32_t kk = (uint32_t)__builtin_amdgcn_readfirstlane((int)plan_key(pk, a.flags));
            if (k == cr)
                gk[0] = kk;
            if (k == cs)
                gk[1] = kk;
            pk += L.tsum[k];
        }
        // the register chunk first: its registers are free after it
        if (cr < nk)
            run[0] = chunk_run(f, gk[0]);
        if (cs < nk) {
            Four q[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                q[j] = staged_four(stage, wave, j);
            run[1] = chunk_run(q, gk[1]);
        }
    }
    double P = a.init[s];
    if (lookback) {
        if (wave == 0) {
            if (!last_in_group)
                level1(L, st0 + kGroup * lg, (int)pg, lg, a.epoch, gs0, Ttile);
        } else if (wave == 1) {
            bool ok2 = true;
            double v2 = 0.0;
            if (lg > 0)
                v2 = lb_level2(gs0, lg, a.epoch, &L.lb_stop[0], ok2);
            if (lane == 0) {
                L.lb2[0] = v2;
                L.lb_ok2[0] = ok2;
            }
        }
        __syncthreads();
        const bool found = L.lb_found[0] != 0;
        const bool ok = L.lb_ok1[0] && (found || (lg > 0 && L.lb_ok2[0]));
        P = !ok ? __builtin_nan("") : (found ? L.lb1[0] : L.lb2[0] + L.lb1[0]);
        if (t == 0 && ok) {
            store_relaxed_u64(st0 + i, st_pack(a.epoch, kStIncl, P + Ttile));
            if (pg == kGroup - 1)
                store_relaxed_u64(gs0 + lg, st_pack(a.epoch, kStIncl, P + Ttile));
        }
    }
    // ---- every chunk's planned prefix and binade (each wave its own two,
    // from the same sums in the same order), kept in LDS by the wave
    uint32_t kc[2];
    {
        double pk = P;
#pragma unroll
        for (int k = 0; k < kTileCh; k++) {
            const double tk = L.tsum[k];
            if ((k >> 1) == wave) {
                const uint32_t ka = key_of(pk), kb = key_of(pk + tk);
                const uint32_t kp = plan_key(pk, a.flags);
                kc[k & 1] = kp;
                if (lane == 0) {
                    L.pk[k] = pk;
                    L.key[k] = kp;
                    L.cross[k] = kb != ka;
                    L.down[k] = ((kb ^ ka) & 0x800u) == 0u && (kb & 0x7FFu) < (ka & 0x7FFu);
                }
            }
            pk += tk;
        }
    }
    // ---- the runs not formed under the guess: every chunk without one, else
    // a chunk whose guess missed (its terms read again: the register chunk
    // from memory, the other from its LDS slot)
#pragma unroll 1
    for (int h = 0; h < 2; h++) {
        const int c = cr + h;
        const uint32_t kh = h ? kc[1] : kc[0];
        if (c >= nk || (spec && (h ? gk[1] : gk[0]) == kh))
            continue;
        Four q[4];
#pragma unroll
        for (int j = 0; j < 4; j++)
            q[j] = h ? staged_four(stage, wave, j) : wave_four(v, c0 + cr, j);
        const WaveRun r = chunk_run(q, kh);
        if (h)
            run[1] = r;
        else
            run[0] = r;
    }
    // ---- the binade edges checked and the descriptors stored (lane h for
    // the wave's chunk cr + h; lane 0 wrote their plan words above)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (lane < 2 && cr + lane < nk) {
        const int h = lane, c = cr + h;
        const WaveRun r = h ? run[1] : run[0];
        const uint32_t kk = L.key[c];
        const double pk = L.pk[c];
        const bool dn = L.down[c] != 0u;
        bool cc = L.cross[c] != 0u;
        if (key_has_fast_path(kk) && kk == key_of(pk)) {
            const int64_t m = count_of(pk);
            const int64_t mg = plan_margin(c0 + c + 1);
            bool near = m < count_floor(kk) + mg;
            if (r.flags & kFlagNeg)
                near |= m + r.lo - mg < kCountLo + 1 || m + r.hi + mg > kCountHi - 1;
            else
                near |= m + r.hi + mg > kCountHi;
            cc |= near;
        }
        L.join[c] = r;
        L.cross[c] = cc;
        store_desc_coherent(w.d, gc0 + (size_t)c, kk, r, cc ? kFlagCross : 0u);
        // a crossing to locate
        L.locate[c] = cc && key_has_fast_path(kk) && kk == key_of(pk) &&
                      key_has_fast_path(dn ? kk - 1u : kk + 1u) && !(r.flags & kFlagNonFinite);
    }
    __syncthreads();
    uint32_t xmask = 0u;
    bool regular = true;
#pragma unroll
    for (int k = 0; k < kTileCh; k++) {
        if (k < nk) {
            xmask |= L.locate[k] ? 1u << k : 0u;
            regular &= key_has_fast_path(L.key[k]) && L.key[k] == L.key[0] && !L.cross[k] &&
                       !(L.join[k].flags & (kFlagBad | kFlagNonFinite));
        }
    }
    xmask = (uint32_t)__builtin_amdgcn_readfirstlane((int)xmask);
    // ---- the crossing of every chunk planned to cross, located by the
    // whole workgroup (a register chunk read again from memory)
    uint32_t found = 0u;
    int buf = 0;
#pragma unroll 1
    for (int c = 0; c < nk; c++) {
        if (!((xmask >> c) & 1u))
            continue;
        const Four q = (c & 1) ? staged_chunk(stage, c >> 1, n, c0 + c) : src.chunk_v(v, c0 + c, lds_src);
        uint64_t xw[kCrossWords];
        if (crossing_find(q, chunk_len(n, c0 + c), L.key[c], count_of(L.pk[c]), L.down[c] != 0u, sc, xl,
                          buf, xw)) {
            found |= 1u << c;
            if (t == 0) {
#pragma unroll
                for (int q2 = 0; q2 < kCrossWords; q2++)
                    L.xw[c][q2] = xw[q2];
            }
        }
    }
    if (xmask)
        __syncthreads();

    // ---- the tile's record
    publish_tile(w, tag, g, L, 0, nk, regular, found, n, c0);
}

// ---------------------------------------------------------------------------
// The kernel: per sum, its head, its finisher, then its later tiles
// ---------------------------------------------------------------------------
template <class Src>
__global__ __launch_bounds__(kChunkThreads, Src::kPassWaves) void pass_kernel(PassArgs pa, Src src, PassWs w)
{
    __shared__ PassTileLds L;
    __shared__ WalkCore sc;
    __shared__ CrossLds xl;
    __shared__ __align__(16) double U[kUnionDoubles];
    __shared__ __attribute__((aligned(16))) int lds_src[Src::kLdsInts];
    const PassArgs &a = pa;
    int s;
    uint32_t b;
    if constexpr (Src::kInter) {
        // interleaved sums: every sum's head and finisher, then the tiles,
        // each the same tile of all sums
        const uint32_t k2 = 2u * a.inter;
        if (blockIdx.x >= k2) {
            inter_tile_block(pa, src, w, blockIdx.x - k2 + 1u, L, sc, xl, U, lds_src);
            return;
        }
        s = (int)(blockIdx.x >> 1);
        b = blockIdx.x & 1u;
    } else {
        // this block's sum: the last with block_base <= blockIdx.x
        int lo = 0, hi = a.count - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pa.block_base[mid] <= blockIdx.x)
                lo = mid;
            else
                hi = mid - 1;
        }
        s = lo;
        b = blockIdx.x - pa.block_base[s];
    }
    // The head and the finisher are the sum's serial path; their waves go
    // first in issue on the SIMDs they share with streaming tiles.
    if (b <= 1)
        __builtin_amdgcn_s_setprio(3);
    if (b == 0)
        head_block(pa, src, w, s, L, sc, U, lds_src);
    else if (b == 1)
        finisher_block(pa, src, w, s, *reinterpret_cast<FinLds *>(U), sc, U + kFinTermsOff, lds_src);
    else if constexpr (!Src::kInter)
        tile_block(pa, src, w, s, b - 1, L, sc, xl, U, lds_src);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

// Launch tags: 42 bits, never zero, never repeated within a process; the
// start is drawn from the clock and the process so that words a previous
// process left in reused memory are unlikely to match.
std::atomic<uint64_t> g_tag{0};

uint64_t next_tag()
{
    uint64_t cur = g_tag.load(std::memory_order_relaxed);
    if (cur == 0) {
        uint64_t seed = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        seed ^= (uint64_t)(uintptr_t)&g_tag * 0x9E3779B97F4A7C15ULL;
        seed = (seed ^ (seed >> 31)) * 0xBF58476D1CE4E5B9ULL;
        uint64_t expect = 0;
        g_tag.compare_exchange_strong(expect, seed | 1u, std::memory_order_relaxed);
    }
    uint64_t tg;
    do {
        tg = g_tag.fetch_add(1, std::memory_order_relaxed) & ((1ULL << 42) - 1);
    } while (tg == 0);
    return tg;
}

size_t r256(size_t b) { return (b + 255) & ~(size_t)255; }

PassWs pass_carve(void *ws, size_t blocks, size_t sums)
{
    char *p = static_cast<char *>(ws);
    const size_t groups = (blocks >> kGroupShift) + sums + 1, chunks = (size_t)kTileCh * blocks;
    PassWs w;
    w.st = reinterpret_cast<uint64_t *>(p);
    p += r256(blocks * 8);
    w.gst = reinterpret_cast<uint64_t *>(p);
    p += r256(groups * 8);
    w.d.r0 = reinterpret_cast<int64_t *>(p);
    p += r256(chunks * 8);
    w.d.lo = reinterpret_cast<int64_t *>(p);
    p += r256(chunks * 8);
    w.d.hi = reinterpret_cast<int64_t *>(p);
    p += r256(chunks * 8);
    w.d.meta = reinterpret_cast<uint32_t *>(p);
    p += r256(chunks * 4);
    w.trec = reinterpret_cast<uint64_t *>(p);
    p += r256(blocks * 4 * 8);
    w.xrec = reinterpret_cast<uint64_t *>(p);
    p += r256(blocks * kStepWords * 8);
    w.hrec = reinterpret_cast<uint64_t *>(p);
    return w;
}

}  // namespace

// Workgroups of a launch over sums of ns[0 .. count - 1] terms.
size_t pass_blocks(const size_t *ns, size_t count)
{
    size_t blocks = 0;
    for (size_t k = 0; k < count; k++)
        blocks += 1 + tiles_of((uint32_t)((ns[k] + kChunk - 1) / kChunk));
    return blocks;
}

size_t pass_ws_bytes(size_t blocks, size_t sums)
{
    const size_t groups = (blocks >> kGroupShift) + sums + 1, chunks = (size_t)kTileCh * blocks;
    return r256(blocks * 8) + r256(groups * 8) + 3 * r256(chunks * 8) + r256(chunks * 4) +
           r256(blocks * 32) + r256(blocks * kStepWords * 8) + r256(sums * 16 + 16);
}

// An upper bound of the workgroups of sums of `total_chunks` padded chunks:
// per sum at most one tile per eight chunks plus three.
size_t pass_blocks_bound(size_t total_chunks, size_t sums) { return total_chunks / kTileCh + 3 * sums + 1; }

bool pass_flags_ok(uint32_t flags)
{
    const uint32_t mode = flags & EXSEQ_PLAN_MASK;
    if (mode == EXSEQ_PLAN_ALL_FALLBACK)
        return false;
    if (flags & (EXSEQ_WALK_ONLY | EXSEQ_CHAIN_CUT | EXSEQ_PLAN_REUSE | EXSEQ_CHAIN_PATH))
        return false;
    return ((flags >> kTileShift) & 3u) == 0u;
}

bool pass_eligible(const BatchArgs &a) { return pass_flags_ok(a.flags) && !a.interleave; }

int launch_pass(const double *const *xs, const size_t *ns, const double *inits, int count,
                uint32_t flags, void *ws, double *outs, hipStream_t stream, exseq_stats *stats,
                void *const *events, int n_events)
{
    if (count < 1 || count > kPassMax)
        return EXSEQ_EINVAL;
    PassArgs pa{};
    pa.count = count;
    pa.flags = flags;
    pa.tch = kTileCh;
    pa.outs = outs;
    pa.stats = stats;
    uint32_t blocks = 0;
    for (int s = 0; s < count; s++) {
        pa.x[s] = xs[s];
        pa.n[s] = ns[s];
        pa.init[s] = inits ? inits[s] : 0.0;
        pa.block_base[s] = blocks;
        blocks += 1 + tiles_of((uint32_t)((ns[s] + kChunk - 1) / kChunk));
    }
    pa.block_base[count] = blocks;
    pa.tag = next_tag();
    pa.epoch = (uint32_t)(pa.tag & 0xFFFFu) ? (uint32_t)pa.tag : (uint32_t)pa.tag + 1u;
    const PassWs w = pass_carve(ws, blocks, (size_t)count);
    if (events && n_events > 0 && events[0])
        hipEventRecord(static_cast<hipEvent_t>(events[0]), stream);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(pass_kernel<PlainTerms>), dim3(blocks), dim3(kChunkThreads), 0,
                       stream, pa, PlainTerms{}, w);
    if (events && n_events > 1 && events[1])
        hipEventRecord(static_cast<hipEvent_t>(events[1]), stream);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
}

// Interleaved sums (k = 2 or 4 fields per record) in one launch: the k
// heads and finishers, then one workgroup per tile of all k sums.
size_t pass_inter_blocks(size_t windows, int k)
{
    const uint32_t nch = (uint32_t)((windows + kChunk - 1) / kChunk);
    return (size_t)k * (1 + tiles_of(nch, (uint32_t)(kTileCh / k)));
}

bool pass_inter_ok(size_t windows, int k, uint32_t flags)
{
    return (k == 2 || k == 4) && pass_flags_ok(flags) && windows > 0 &&
           (uint64_t)windows * (uint64_t)k > (uint64_t)2 * kTileMax * kChunk;
}

int launch_pass_interleaved(const double *x, size_t windows, int k, const double *inits, double *outs,
                            float *means, void *ws, hipStream_t stream, uint32_t flags, exseq_stats *stats)
{
    if (!(k == 2 || k == 4) || windows == 0)
        return EXSEQ_EINVAL;
    PassArgs pa{};
    pa.count = k;
    pa.flags = flags;
    pa.tch = (uint32_t)(kTileCh / k);
    pa.inter = (uint32_t)k;
    pa.means = means;
    pa.outs = outs;
    pa.stats = stats;
    const uint32_t nch = (uint32_t)((windows + kChunk - 1) / kChunk);
    const uint32_t nt = tiles_of(nch, pa.tch);
    for (int s = 0; s < k; s++) {
        pa.x[s] = x + s;
        pa.n[s] = windows;
        pa.init[s] = inits ? inits[s] : 0.0;
        pa.block_base[s] = (uint32_t)s * (nt + 1);  // the workspace layout of each sum
    }
    pa.block_base[k] = (uint32_t)k * (nt + 1);
    pa.tag = next_tag();
    pa.epoch = (uint32_t)(pa.tag & 0xFFFFu) ? (uint32_t)pa.tag : (uint32_t)pa.tag + 1u;
    const PassWs w = pass_carve(ws, pa.block_base[k], (size_t)k);
    const unsigned grid = 2u * (unsigned)k + (nt > 1 ? nt - 1 : 0u);
    hipLaunchKernelGGL(HIP_KERNEL_NAME(pass_kernel<PassStrided>), dim3(grid), dim3(kChunkThreads), 0, stream,
                       pa, PassStrided{(uint32_t)k}, w);
    return hipGetLastError() == hipSuccess ? EXSEQ_OK : EXSEQ_EHIP;
}

}  // namespace exseq
