/*
 * exseq -- bit-exact sequential fp64 sums on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libexseq.so.  Every result equals, bit for bit, the CPU loop
 *
 *     double s = init; for (i = 0; i < n; i++) s += x[i];
 *
 * in IEEE-754 binary64 with round to nearest, ties to even (Research-1433
 * "Forming the CPU's sequential double sums on a GPU, bit for bit", Question
 * and Findings 1; Research-1424 "integer_ssim_cuda and the CPU's frame sum",
 * Findings 1 and 3).  The terms stay on the device and are not added on one
 * thread: inside one binade the running sum is an integer count of units,
 * each term an increment pair formed from its own bits (ties to even make it
 * a pair), runs compose in order, prefix bounds prove a run stayed in its
 * binade, and chunks that leave it are added term by term from the exact sum.
 *
 * Conventions for every call below:
 *  - Data pointers (`x`, `xs[k]`, `ref`, `dis`, `out*`, `means`, `ws`, `stats`) are
 *    DEVICE pointers on the current HIP device; `ns`, `inits`, `xs` (the array of
 *    pointers itself) and `shapes` are HOST arrays.  The caller owns every
 *    buffer; the library allocates nothing and never frees.
 *  - Every call is stream-ordered and non-blocking on `stream` (0 = the null
 *    stream): no host synchronisation, no device-to-host copy.  A return of
 *    EXSEQ_OK means the work was enqueued; the result appears in device
 *    memory when the stream reaches it.
 *  - `ws` is a caller-provided device workspace of at least the size the
 *    matching *_workspace_size() call returns.  Its contents need no
 *    initialisation and are clobbered (with EXSEQ_PLAN_REUSE a call leaves a
 *    plan in it for the next call; see there).  Calls that share a workspace
 *    must be ordered (same stream); calls on different streams need
 *    different workspaces.
 *  - Terms are fp64 in native (little-endian) layout, contiguous, 8-byte
 *    aligned.  n == 0 is valid and writes `init`.
 *  - Non-finite terms are allowed: the result is what the loop gives (NaN
 *    payloads are not specified); `stats->flags` then has EXSEQ_STAT_NONFINITE.
 *  - Return value: EXSEQ_OK (0) or a negative EXSEQ_E* code.  Argument errors
 *    are found before anything is enqueued; EXSEQ_EHIP reports a launch
 *    error from the HIP runtime.
 */
#ifndef EXSEQ_H
#define EXSEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *exseq_stream_t; /* a hipStream_t */

enum {
    EXSEQ_OK = 0,
    EXSEQ_EINVAL = -1,     /* null pointer with work to do, misalignment, bad size */
    EXSEQ_EWORKSPACE = -2, /* ws_bytes below the required size */
    EXSEQ_EHIP = -3,       /* the HIP runtime rejected a launch */
    EXSEQ_ESCRATCH = -4    /* the input needs more than the static scratch array */
};

/* Plan modes (low 4 bits of `flags`).  The plan names the binade each chunk's
 * increments are formed for.  It is an approximation and can never change a
 * result, only how many chunks are added term by term (Research-1433
 * Findings 5).  The overrides exist to test that statement.
 *   AUTO          binade of the prefix of the chunks' tree sums (default)
 *   ALL_FALLBACK  no chunk gets a fast path: every chunk term by term
 *   PLUS_ONE      one binade too high on every chunk
 *   MINUS_ONE     one binade too low on every chunk
 *   FIXED         every chunk planned for the key in bits 8..19 of `flags`
 *                 (sign bit << 11 | biased exponent; 1023 is [1, 2))
 *   ALL_ZERO      every chunk planned as if the sum before it were +0 (the
 *                 binade of the subnormals) */
#define EXSEQ_PLAN_AUTO 0u
#define EXSEQ_PLAN_ALL_FALLBACK 1u
#define EXSEQ_PLAN_PLUS_ONE 2u
#define EXSEQ_PLAN_MINUS_ONE 3u
#define EXSEQ_PLAN_FIXED 4u
#define EXSEQ_PLAN_ALL_ZERO 5u
#define EXSEQ_PLAN_MASK 0xFu
#define EXSEQ_PLAN_FIXED_KEY(key) (EXSEQ_PLAN_FIXED | (((uint32_t)(key) & 0xFFFu) << 8))

/* Further bits of `flags` (testing and tuning; 0 for production use).
 *   bits 4..5     chunks per tile of the single pass: 0 (default) = by the
 *                 launch's chunk count (4 up to 8 chunks, 1 up to 2048, 2 up
 *                 to 4096, else 4; always 4 with EXSEQ_PLAN_REUSE), 1 = 1,
 *                 2 = 2, 3 = 4
 *   WALK_ONLY     the tiles only plan and describe; the ordered walk after
 *                 them follows every chunk (no exact chain between tiles)
 *   CHAIN_CUT     the exact chain stops half way through every sum (the tiles
 *                 of the second half report failure), so that the walk must
 *                 resume from the last exact value the chain published
 * ALL_FALLBACK implies WALK_ONLY. */
#define EXSEQ_TILE_SHIFT 4
#define EXSEQ_WALK_ONLY (1u << 6)
#define EXSEQ_CHAIN_CUT (1u << 7)
/* EXSEQ_CHAIN_PATH and EXSEQ_PASS_PATH choose between the two launch plans
 * of a plain sum or batch (the same results): the tile chain and walk of
 * three launches, and the single pass (one launch for all the sums of a
 * batch: streaming tiles, a head block and a finisher block per sum).  By
 * default a batch of two or more sums takes the single pass and one sum the
 * chain.  Only the AUTO, PLUS_ONE, MINUS_ONE and FIXED plans with the
 * default tile take the single pass; every other mode (ALL_FALLBACK,
 * WALK_ONLY, CHAIN_CUT, PLAN_REUSE, a tile size) and the interleaved and
 * fused SSIM sums take the chain. */
#define EXSEQ_CHAIN_PATH (1u << 21)
#define EXSEQ_PASS_PATH (1u << 22)

/* EXSEQ_PLAN_REUSE (with EXSEQ_PLAN_AUTO and the default tile): the plan of
 * the previous call on the same workspace stands in for this call's where it
 * leaves no doubt (Research-1433 "Forming the CPU's sequential double sums
 * on a GPU, bit for bit", Open questions, first throughput candidate: keep a
 * frame's plan for the next frame of a video, form the increments under it
 * in the pass that forms the tree sums, and plan again only where the plan
 * may have changed).
 *   - Every call with the flag writes, after its sums, the planned prefix
 *     before each tile of 4096 terms into the workspace, tagged with the
 *     call's shape (count, every n and init, the chunk layout).
 *   - A later call with the flag and the same shape on the same workspace
 *     reads it.  A tile whose prefix range there, widened by 1/64 of its
 *     magnitude on both sides, stays inside one binade takes that binade
 *     for all its chunks and does not wait for the look-back over the tiles
 *     before it.  Other tiles, a sum's first and last tile, and every tile
 *     of a call without a matching tagged plan plan as without the flag.
 *   - Results do not depend on the flag or on the stored plan (Research-1433
 *     Findings 5: a plan only decides which chunks go term by term).  A
 *     frame unlike the one before it (a scene cut) is still exact, and may
 *     be slower: chunks whose reused binade is wrong go term by term.
 * The flag is ignored with other plan modes, WALK_ONLY or a tile size other
 * than the default. */
#define EXSEQ_PLAN_REUSE (1u << 20)

/* EXSEQ_SSIM_IN_TILES (ssim_term_and_sum only): the exact sum's tiles form
 * the terms as they need them (no term is stored unless asked for).  Without
 * it the terms are formed by a producer launch into device memory (the
 * caller's out_terms plane, else the workspace: 8 bytes per pixel), then
 * added by the exact sum of exact_seq_sum_f64 (every other flag applies to
 * that sum).  Both give the same bits; the producer's windows slide down the
 * rows, which the tiles' raster chunks cannot. */
#define EXSEQ_SSIM_IN_TILES (1u << 23)

/* Device-side statistics of one sum (written when the walk finishes). */
typedef struct exseq_stats {
    uint64_t chunks;          /* chunks walked */
    uint64_t fast_chunks;     /* chunks applied from their increment pairs */
    uint64_t fallback_chunks; /* chunks added term by term */
    uint64_t fallback_terms;  /* terms added one by one */
    int64_t first_fallback;   /* index of the first fallback chunk, -1 if none */
    uint32_t flags;           /* EXSEQ_STAT_* */
    uint32_t plan_misses;     /* chunks whose planned binade was not the exact one */
} exseq_stats;

#define EXSEQ_STAT_NONFINITE 1u

/* Terms per chunk: the unit of descriptors and of the term-by-term fallback. */
#define EXSEQ_CHUNK_TERMS 1024

/* ---------------------------------------------------------------------------
 * exact_seq_sum_f64
 *   out[0] = ((init + x[0]) + x[1]) + ... + x[n-1], in fp64 RNE, bit exact.
 *   x: n device doubles.  out: one device double.  stats: nullable device
 *   pointer.  flags: EXSEQ_PLAN_* (0 for production use).
 *   Research-1433 Findings 2-6 (method and layout); Research-1424 Findings 3.
 * ------------------------------------------------------------------------- */
size_t exact_seq_sum_f64_workspace_size(size_t n);
int exact_seq_sum_f64(const double *x, size_t n, double init, double *out,
                      void *ws, size_t ws_bytes, exseq_stream_t stream,
                      uint32_t flags, exseq_stats *stats);

/* ---------------------------------------------------------------------------
 * exact_seq_sum_f64_noalloc
 *   For callers that cannot allocate device memory (code under HIP graph
 *   capture, tight serving loops, harnesses that forbid hipMalloc): the same
 *   sum and launches as exact_seq_sum_f64, with its workspace in a static
 *   device array of the library, EXSEQ_NOALLOC_SCRATCH_BYTES per GPU, held
 *   until the process ends.  It calls no allocating routine.  The array of
 *   the current device is used: `stream` must belong to it.  Sizes whose
 *   workspace (exact_seq_sum_f64_workspace_size(n)) exceeds the array return
 *   EXSEQ_ESCRATCH before anything is enqueued; that is n up to
 *   exact_seq_sum_f64_noalloc_max_terms().  Every call on a GPU shares that
 *   GPU's array: calls that overlap in time on one GPU (other streams, other
 *   threads) race and give undefined results; calls in one stream are
 *   ordered and safe.  The array needs no clearing (launch words are tagged
 *   per launch; EXSEQ_PLAN_REUSE reuses the plan of the last call on that
 *   GPU, which affects speed only).  Other arguments and errors as
 *   exact_seq_sum_f64; EXSEQ_EHIP also when the array's address cannot be
 *   obtained.
 * ------------------------------------------------------------------------- */
#define EXSEQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
size_t exact_seq_sum_f64_noalloc_max_terms(void);
int exact_seq_sum_f64_noalloc(const double *x, size_t n, double init, double *out,
                              exseq_stream_t stream, uint32_t flags, exseq_stats *stats);

/* ---------------------------------------------------------------------------
 * exact_seq_sum_f64_batch
 *   count independent sums: outs[k] = the loop over xs[k][0 .. ns[k]) started
 *   at inits[k] (inits: host array, or NULL for +0.0 everywhere).  One launch
 *   sequence covers every sum (the per-scale sums of a frame pyramid; ADR-1391
 *   "The CUDA ssimulacra2 twin is device-resident", Decision step 2-3).
 *   xs, ns, inits: HOST arrays of length count (xs holds device pointers).
 *   outs: count device doubles.  stats: nullable device array of count.
 * ------------------------------------------------------------------------- */
size_t exact_seq_sum_f64_batch_workspace_size(const size_t *ns, size_t count);
int exact_seq_sum_f64_batch(const double *const *xs, const size_t *ns,
                            const double *inits, size_t count, double *outs,
                            void *ws, size_t ws_bytes, exseq_stream_t stream,
                            uint32_t flags, exseq_stats *stats);

/* ---------------------------------------------------------------------------
 * exact_seq_sum_f64_interleaved
 *   k independent sums over records of k doubles: for j < k,
 *   outs[j] = ((inits[j] + x[j]) + x[j + k]) + ... + x[j + (windows-1) k],
 *   each in fp64 RNE, bit exact, and, if `means` is not NULL,
 *   means[j] = (float)(outs[j] / (double)windows) (IEEE division, then
 *   round to nearest float).  ADR-1464 "float_ssim_cuda adds its frame sums
 *   in the CPU's raster order, on the host", Context and Decision: a window
 *   keeps four doubles (l*c*s, l, c, s), the four sums are independent, each
 *   in index order, and the score is the float of the mean.
 *   x: k * windows device doubles, record-major (record w holds x[w k] ..
 *   x[w k + k - 1]).  inits: HOST array of k, or NULL for +0.0.  outs: k
 *   device doubles.  means: nullable, k device floats (4-byte aligned).
 *   stats: nullable device array of k.  1 <= k <= EXSEQ_INTERLEAVE_MAX.
 *   windows == 0 writes inits (and their means, init / 0.0).
 * ------------------------------------------------------------------------- */
#define EXSEQ_INTERLEAVE_MAX 8
size_t exact_seq_sum_f64_interleaved_workspace_size(size_t windows, int k);
int exact_seq_sum_f64_interleaved(const double *x, size_t windows, int k,
                                  const double *inits, double *outs, float *means,
                                  void *ws, size_t ws_bytes, exseq_stream_t stream,
                                  uint32_t flags, exseq_stats *stats);

/* ---------------------------------------------------------------------------
 * ssim_term_and_sum
 *   Integer-SSIM frame sum, the terms formed on the device from the planes
 *   (by a producer launch, or with EXSEQ_SSIM_IN_TILES inside the sum's
 *   tiles).  For every pixel (i, j) of two 8-bit planes
 *   (row-major, `stride` bytes between rows) the edge-truncated
 *   (2r+1) x (2r+1) window gives int64 sums x, y, x2, y2, xy and the pixel
 *   count w; the fp64 term
 *     w*(2*mxy + c1)*(c2 + 2*(xy*w - mxy))
 *       / ((mx2 + my2 + c1)*(x2*w - mx2 + y2*w - my2 + c2)),
 *   mx2 = x*x, my2 = y*y, mxy = x*y in fp64, evaluated left to right with no
 *   contraction (Research-1424 Findings 1; ADR-1443 "integer_ssim_sycl
 *   computes the CPU's fp64 term in 64-bit integers and adds in the CPU's
 *   order", Context and Decision), is added into one double in raster order
 *   starting from +0.0.  out_sum: one device double.  out_weight_sum:
 *   nullable device int64, the sum of w over the frame.  out_terms: nullable
 *   device plane of width*height doubles receiving every term (debugging);
 *   without it the producer writes the terms into the workspace, whose size
 *   (ssim_term_and_sum_workspace_size) includes 8 bytes per pixel for them.
 *   ws must not overlap the planes or out_terms.  width, height >= 1;
 *   stride >= width; 0 <= radius <= 15.  Errors: EXSEQ_EINVAL for a null
 *   plane or out_sum, misaligned outputs, a bad geometry or width*height
 *   >= 2^31; EXSEQ_EWORKSPACE for a workspace below the size; EXSEQ_EHIP for
 *   a launch that failed.
 * ------------------------------------------------------------------------- */
size_t ssim_term_and_sum_workspace_size(int width, int height);
int ssim_term_and_sum(const uint8_t *ref, const uint8_t *dis, int width,
                      int height, ptrdiff_t stride, int radius, double c1,
                      double c2, double *out_sum, int64_t *out_weight_sum,
                      double *out_terms, void *ws, size_t ws_bytes,
                      exseq_stream_t stream, uint32_t flags, exseq_stats *stats);

/* ---------------------------------------------------------------------------
 * tree_sum_f64
 *   Deterministic fixed-shape tree sum of x (NOT the loop's bits): chunks of
 *   1024 terms reduced in a fixed tree, then the chunk sums in a fixed tree.
 *   Its result depends only on n and the values, and is reported beside the
 *   exact sum to show the gap a tree leaves (ADR-1391 Decision, Numerics).
 *   out: one device double.
 * ------------------------------------------------------------------------- */
size_t tree_sum_f64_workspace_size(size_t n);
int tree_sum_f64(const double *x, size_t n, double *out, void *ws,
                 size_t ws_bytes, exseq_stream_t stream);

/* ---------------------------------------------------------------------------
 * Profiling of the exact-sum path (used by the benchmark for per-kernel
 * device time).  exseq_profile_kernel_count() kernels run, in order, for
 * every n > 0; exseq_profile_kernel_name(i) names kernel i (static storage;
 * "" out of range).  exact_seq_sum_f64_profiled() is exact_seq_sum_f64 (n > 0)
 * that also records events[2i] just before and events[2i+1] just after
 * kernel i on `stream`; `events` is a HOST array of n_events hipEvent_t
 * handles created by the caller (NULL entries are skipped).
 * ------------------------------------------------------------------------- */
int exseq_profile_kernel_count(void);
const char *exseq_profile_kernel_name(int i);
int exact_seq_sum_f64_profiled(const double *x, size_t n, double init, double *out,
                               void *ws, size_t ws_bytes, exseq_stream_t stream,
                               uint32_t flags, exseq_stats *stats,
                               void *const *events, int n_events);

/* ---------------------------------------------------------------------------
 * exseq_stream_read_f64
 *   A plain streaming read of x[0 .. n) (16-byte loads): the achievable HBM
 *   read rate over the buffer the exact sum reads, measured beside it (a
 *   measurement reference, not part of the method).  Each of the
 *   EXSEQ_STREAM_READ_BLOCKS workgroups writes the xor of the bit patterns it
 *   read to out[block].  x: device, 16-byte aligned; out: device array of
 *   EXSEQ_STREAM_READ_BLOCKS words.  EXSEQ_EINVAL for null or misaligned
 *   pointers.
 * ------------------------------------------------------------------------- */
#define EXSEQ_STREAM_READ_BLOCKS 2048
int exseq_stream_read_f64(const double *x, size_t n, uint64_t *out, exseq_stream_t stream);

/* ---------------------------------------------------------------------------
 * exseq_div_f64
 *   q[i] = a[i] / b[i] for i < n: the device fp64 division that the fused
 *   SSIM term performs (Research-1424 Findings 1: the term's one divide), run
 *   alone so that tests can compare it with the host's correctly rounded
 *   division on many operands.  a, b, q: device arrays of n doubles (8-byte
 *   aligned); stream-ordered; EXSEQ_EINVAL for null or misaligned pointers.
 * ------------------------------------------------------------------------- */
int exseq_div_f64(const double *a, const double *b, double *q, size_t n, exseq_stream_t stream);

/* Text for an EXSEQ_* return code (static storage). */
const char *exseq_strerror(int code);

/* Library version string (static storage). */
const char *exseq_version(void);

/* ---------------------------------------------------------------------------
 * Host model of the method (test infrastructure; runs on the CPU, no GPU).
 *   The same rules as the kernels, walked chunk by chunk on the host, with
 *   the plan overrides and four deliberate mutations of the rules that the
 *   method's own tests must catch (Research-1433 Findings 1 "Tests": always
 *   round a tie up, drop the binade check, drop the upper bound check,
 *   ignore the parity when composing).  x: HOST array.  chunk_terms >= 1.
 *   stats: nullable HOST pointer.  Returns the sum.
 * ------------------------------------------------------------------------- */
#define EXSEQ_MUT_TIE_UP 1u
#define EXSEQ_MUT_NO_BINADE_CHECK 2u
#define EXSEQ_MUT_NO_UPPER_CHECK 4u
#define EXSEQ_MUT_IGNORE_PARITY 8u
#define EXSEQ_MUT_NO_RUN_TOP 16u
double exseq_model_seq_sum_f64(const double *x, size_t n, double init,
                               size_t chunk_terms, uint32_t flags,
                               uint32_t mutations, exseq_stats *stats);

/* ---------------------------------------------------------------------------
 * CPU twins of the kernels' composition (test infrastructure; no GPU).
 *   The same rule helpers as the kernels, replayed in the kernels' grouping
 *   of the terms -- four per lane, 64-lane waves with their shortcuts and
 *   scan trees, four waves per chunk -- so that the grouping's shortcuts are
 *   checked against the sequential loop on the host (Research-1433 "Forming
 *   the CPU's sequential double sums on a GPU, bit for bit", Findings
 *   "Tests").  x: HOST array of n doubles; flags: a plan mode; mutations:
 *   EXSEQ_MUT_* planted in the replay; stats: nullable HOST pointer.
 *   exseq_twin_seq_sum_f64: the single pass (tiles of eight chunks, the
 *   finisher's windows).  exseq_twin_chain_sum_f64: the tile chain (tiles of
 *   four chunks, the chain look-back, the irregular tiles, the walk's
 *   resume), every planned prefix moved by skew * 2^-30 of itself; paths:
 *   nullable HOST array of 6 counts (look-back waves composed as integer
 *   sums, falling sums, pairs alone, full runs; composed runs applied; chain
 *   stops).  Both return the sum.
 * ------------------------------------------------------------------------- */
double exseq_twin_seq_sum_f64(const double *x, size_t n, double init, uint32_t flags,
                              uint32_t mutations, exseq_stats *stats);
double exseq_twin_chain_sum_f64(const double *x, size_t n, double init, uint32_t flags,
                                uint32_t mutations, int64_t skew, exseq_stats *stats,
                                uint64_t *paths);

#ifdef __cplusplus
}
#endif

#endif /* EXSEQ_H */
