// Host replay of the single pass, in the kernels' grouping of the terms: the
// CPU twin of how pass_kernel composes runs.  A chunk's 1024 terms sit four
// to a lane on 256 lanes in four waves of 64; each wave's part of a chunk is
// formed as wave_runs / wave_run form it (the tie-free single-sign shortcut
// with hi = 0, the order-free sums, the prefix bounds of the even-start sums
// widened by the wave's ties), the four parts are joined in order
// (join_waves, or the rising/falling shortcut of the tile), a tile composes
// its eight chunks in order, an irregular tile locates its crossings
// (crossing_find's steps, up and down) and folds the chunks after them, the
// head adds a sum's first four chunks from init, and the finisher composes
// each window's tiles as pass_kernel does -- four per lane in order, then the
// wave scan tree of row shifts and row broadcasts, then the carry over the
// waves -- before it walks the ops.  A check that fails sends the event's
// chunks through the descriptor walk and term-by-term adds, as on the GPU.
// A second replay, of the tile chain (tile_kernel with four chunks per tile
// and the chain after it), forms the tiles' runs in the same way, composes
// the regular tiles before each irregular one in chain_back's grouping, adds
// the irregular tiles' chunks from the exact sum and resumes with the walk
// where a composed run does not apply.
//
// The rule helpers (term_inc, compose, run_compose, run_top, run_applies,
// run_compose_sat, join_waves, clamp_run, crossing_apply, plan_key,
// plan_margin) are the kernels' own, from exseq_rules.h and exseq_dev.h.  The
// mutations of Research-1433 "Forming the CPU's sequential double sums on a
// GPU, bit for bit", Findings "Tests" (a tie always rounding up, no binade
// check, no upper check, parity ignored) and one more (a rising part's
// largest prefix taken from its stored hi instead of run_top) can be planted
// in the twin's calls, so that a test sees them fail.  It is test
// infrastructure: the GPU entry points never call it.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "exseq.h"
#include "exseq_dev.h"
#include "exseq_rules.h"

using namespace exseq;

namespace {

constexpr int kLanes = 256, kWaveLanes = 64, kPerLane = 4;
constexpr int kTwinTile = 8, kTwinHead = 4, kTwinWindow = 1024;

// ---------------------------------------------------------------------------
// The rules, with the mutations
// ---------------------------------------------------------------------------
struct Rules {
    uint32_t mut;

    TermInc inc(double x, int scale, bool sgn) const
    {
        TermInc t = term_inc(x, scale, sgn);
        if (mut & EXSEQ_MUT_TIE_UP)
            t.r0 = t.r1 = std::max(t.r0, t.r1);
        return t;
    }
    Pair comp(Pair a, Pair b) const
    {
        if (mut & EXSEQ_MUT_IGNORE_PARITY)
            return Pair{a.r0 + b.r0, a.r1 + b.r1};
        return compose(a, b);
    }
    Run rcomp(const Run &a, const Run &b) const
    {
        if (!(mut & (EXSEQ_MUT_IGNORE_PARITY | EXSEQ_MUT_NO_RUN_TOP)))
            return run_compose(a, b);
        Run c;
        c.p = comp(a.p, b.p);
        const int64_t amin = std::min(a.p.r0, a.p.r1), amax = std::max(a.p.r0, a.p.r1);
        const int64_t ahi = (mut & EXSEQ_MUT_NO_RUN_TOP) ? a.hi : run_top(a);
        const int64_t bhi = (mut & EXSEQ_MUT_NO_RUN_TOP) ? b.hi : run_top(b);
        c.lo = std::min(a.lo, amin + b.lo);
        c.hi = std::max(ahi, amax + bhi);
        c.flags = a.flags | b.flags;
        return c;
    }
    Run rcomp_sat(const Run &a, const Run &b) const
    {
        if (!(mut & (EXSEQ_MUT_IGNORE_PARITY | EXSEQ_MUT_NO_RUN_TOP)))
            return run_compose_sat(a, b);
        Run c = rcomp(a, b);
        const int64_t lim = (int64_t)1 << 56;
        if (c.p.r0 > lim || c.p.r0 < -lim || c.p.r1 > lim || c.p.r1 < -lim || c.lo < -lim ||
            c.hi > lim) {
            c.flags |= kFlagBad;
            c.p = Pair{0, 0};
            c.lo = c.hi = 0;
        }
        return c;
    }
    WaveRun join(const WaveRun *w) const
    {
        if (!(mut & (EXSEQ_MUT_IGNORE_PARITY | EXSEQ_MUT_NO_RUN_TOP)))
            return join_waves(w);
        WaveRun r = w[0];
        for (int k = 1; k < 4; k++) {
            const Run c = rcomp(Run{r.p, r.lo, r.hi, r.flags}, Run{w[k].p, w[k].lo, w[k].hi, w[k].flags});
            r.p = c.p;
            r.lo = c.lo;
            r.hi = c.hi;
            r.flags = c.flags;
        }
        if (!(r.flags & kFlagNeg))
            r.hi = std::max(r.p.r0, r.p.r1);
        return r;
    }
    bool applies(int64_t m, Pair p, int64_t lo, int64_t hi, uint32_t flags) const
    {
        if (mut & EXSEQ_MUT_NO_UPPER_CHECK) {
            if (flags & (kFlagBad | kFlagNonFinite))
                return false;
            return !(flags & kFlagNeg) || m + lo >= kCountLo + 1;
        }
        return run_applies(m, p, lo, hi, flags);
    }
    bool key_ok(uint32_t ks, uint32_t key) const
    {
        return key_has_fast_path(ks) && key_has_fast_path(key) &&
               (ks == key || (mut & EXSEQ_MUT_NO_BINADE_CHECK));
    }
    // S advanced by a run's increment from count m (a count past the binade,
    // only reachable under a mutation, is clipped to its edge)
    double advance(double S, int64_t m, Pair p) const
    {
        int64_t c = m + pair_at(p, m);
        c = std::min(std::max(c, count_floor(key_of(S))), kCountHi);
        return assemble(key_of(S), c);
    }
};

// ---------------------------------------------------------------------------
// The wave scan tree of the kernels' DPP scans: an inclusive scan by row
// shifts 1, 2, 4 and 8 inside rows of 16 lanes, then row 15's value into
// rows 1 and 3, then lane 31's into rows 2 and 3.  Every step computes
// op(source, v) in every lane, op(l, r) with l the earlier part; a lane
// without a source (or outside the step's rows) takes the identity as its
// source, as the DPP moves' bound values give it.
// ---------------------------------------------------------------------------
template <class T, class Op>
void wave_scan_tree(T *v, Op op, const T &id)
{
    for (int sh : {1, 2, 4, 8}) {
        T nv[kWaveLanes];
        for (int l = 0; l < kWaveLanes; l++)
            nv[l] = op((l % 16) >= sh ? v[l - sh] : id, v[l]);
        std::copy(nv, nv + kWaveLanes, v);
    }
    {
        T nv[kWaveLanes];
        for (int l = 0; l < kWaveLanes; l++) {
            const int row = l / 16;
            nv[l] = op((row == 1 || row == 3) ? v[16 * row - 1] : id, v[l]);
        }
        std::copy(nv, nv + kWaveLanes, v);
    }
    {
        T nv[kWaveLanes];
        for (int l = 0; l < kWaveLanes; l++) {
            const int row = l / 16;
            nv[l] = op(row >= 2 ? v[31] : id, v[l]);
        }
        std::copy(nv, nv + kWaveLanes, v);
    }
}

// ---------------------------------------------------------------------------
// A chunk's terms (1024, missing ones +0.0) and its run under a key
// ---------------------------------------------------------------------------
struct Chunk {
    double v[kLanes * kPerLane];
    int len;
    int cnt(int lane) const { return std::max(0, std::min(kPerLane, len - kPerLane * lane)); }
};

// wave_run: one wave's part of a chunk under key
WaveRun twin_wave_run(const Rules &R, const Chunk &c, int wave, uint32_t key)
{
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool sgn = (key >> 11) & 1u;
    int64_t r0[kWaveLanes][4], r1[kWaveLanes][4];
    bool wneg = false, wbad = false, wnf = false, wtie = false;
    for (int l = 0; l < kWaveLanes; l++) {
        const int lane = kWaveLanes * wave + l;
        for (int i = 0; i < 4; i++) {
            if (i < c.cnt(lane)) {
                const double x = c.v[kPerLane * lane + i];
                const TermInc t = R.inc(x, scale, sgn);
                r0[l][i] = t.r0;
                r1[l][i] = t.r1;
                wneg |= t.neg;
                wbad |= t.bad;
                wnf |= is_nonfinite(x);
                wtie |= t.r0 != t.r1;
            } else {
                r0[l][i] = r1[l][i] = 0;
            }
        }
    }
    WaveRun w;
    if (!wtie) {
        int64_t r = 0;
        for (int l = 0; l < kWaveLanes; l++)
            r += (r0[l][0] + r0[l][1]) + (r0[l][2] + r0[l][3]);
        w.p = Pair{r, r};
    } else {
        Pair a[kWaveLanes];
        for (int l = 0; l < kWaveLanes; l++) {
            a[l] = Pair{r0[l][0], r1[l][0]};
            for (int i = 1; i < 4; i++)
                a[l] = R.comp(a[l], Pair{r0[l][i], r1[l][i]});
        }
        wave_scan_tree(a, [&](Pair x, Pair y) { return R.comp(x, y); }, pair_identity());
        w.p = a[kWaveLanes - 1];
    }
    w.lo = w.hi = 0;
    if (wneg) {
        int64_t lo = 0, hi = 0, excl = 0, ties = 0;
        bool first = true;
        for (int l = 0; l < kWaveLanes; l++) {
            int64_t s = 0, mn = 0, mx = 0;
            for (int i = 0; i < 4; i++) {
                s += r0[l][i];
                mn = std::min(s, mn);
                mx = std::max(s, mx);
                ties += r0[l][i] != r1[l][i];
            }
            lo = first ? excl + mn : std::min(lo, excl + mn);
            hi = first ? excl + mx : std::max(hi, excl + mx);
            first = false;
            excl += s;
        }
        if (wtie) {
            lo -= ties;
            hi += ties;
        }
        w.lo = lo < 0 ? lo : 0;
        w.hi = hi > 0 ? hi : 0;
    }
    w.flags = (wneg ? kFlagNeg : 0u) | (wbad ? kFlagBad : 0u) | (wnf ? kFlagNonFinite : 0u);
    return w;
}

// The tile's join of a chunk's four wave parts (the lane < 4 code of
// tile_block), clamped
WaveRun twin_join(const Rules &R, const WaveRun *w)
{
    bool plain = true, fall = true;
    int64_t sum = 0;
    for (int k = 0; k < 4; k++) {
        plain &= rising_run(w[k].p, w[k].flags);
        fall &= falling_run(w[k].p, w[k].lo, w[k].hi, w[k].flags);
        sum += w[k].p.r0;
    }
    return clamp_run(plain ? WaveRun{Pair{sum, sum}, 0, sum, 0u}
                     : fall ? WaveRun{Pair{sum, sum}, sum, 0, kFlagNeg}
                            : R.join(w));
}

// chunk_run: one wave forms a whole chunk of a tile (lane l holds terms
// 256 j + 4 l .. + 3 of group j).  The shortcut where no term of the chunk
// ties and its increments are all >= 0 or all < 0, with the kernel's tests on
// the magic sums' bit patterns (AND and OR over the terms, in any grouping);
// otherwise each group's run (wave_run over the 256 terms a wave of the
// workgroup layout holds) and the four composed in order.  Clamped.
WaveRun twin_chunk_run(const Rules &R, const Chunk &c, uint32_t key)
{
    if (!key_has_fast_path(key)) {
        bool nf = false;
        for (int q = 0; q < kLanes * kPerLane; q++)
            nf |= is_nonfinite(c.v[q]);
        return WaveRun{pair_identity(), 0, 0, nf ? kFlagNonFinite : 0u};
    }
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool flip = (key & 0x800u) != 0u;
    const double fac = flip ? -std::ldexp(1.0, scale) : std::ldexp(1.0, scale);
    uint32_t tacc = 0u, hand = ~0u, hor = 0u;
    uint64_t sum = 0;
    for (int q = 0; q < kLanes * kPerLane; q++) {
        const double x = c.v[q];  // +0.0 past the end
        double y;
        if (scale <= 1023) {
            y = x * fac;
        } else {
            y = std::ldexp(x, scale);
            y = flip ? -y : y;
        }
        const double a0 = kMagic0 + y, a1 = kMagic1 + y;
        const uint32_t h = (uint32_t)(dbits(a0) >> 32);
        tacc |= ((uint32_t)dbits(a1) - (uint32_t)dbits(a0)) ^ 1u;
        hand &= h;
        hor |= h;
        sum += dbits(a0);
    }
    const bool ok = tacc == 0u && (((hand ^ kMagic0Hi) | (hor ^ kMagic0Hi)) >> 20) == 0u;
    const bool pos = (hand >> 19) & 1u, neg = !((hor >> 19) & 1u);
    // (a tie that the mutation rounds up is no tie: the shortcut then sees
    // exactly what wave_run sees)
    if (ok && (pos || neg) && !(R.mut & EXSEQ_MUT_TIE_UP)) {
        const int64_t r = (int64_t)(sum - (uint64_t)(kLanes * kPerLane) * (uint64_t)kMagic0Bits);
        return clamp_run(pos ? WaveRun{Pair{r, r}, 0, r, 0u} : WaveRun{Pair{r, r}, r, 0, kFlagNeg});
    }
    WaveRun w[4];
    for (int j = 0; j < 4; j++)
        w[j] = twin_wave_run(R, c, j, key);
    return twin_join(R, w);
}

// block_run (the head): wave_run per wave, joined, clamped
WaveRun twin_block_run(const Rules &R, const Chunk &c, uint32_t key)
{
    WaveRun w[4];
    for (int k = 0; k < 4; k++)
        w[k] = twin_wave_run(R, c, k, key);
    return clamp_run(R.join(w));
}

// The fixed-tree sum of a tile's chunk (one wave): per lane and group j
// (v0 + v1) + (v2 + v3), the lane's four groups (g0 + g1) + (g2 + g3), then
// the row tree of wave_sum_f64 over the lanes
double twin_tree_sum(const Chunk &c)
{
    double v[kWaveLanes];
    for (int l = 0; l < kWaveLanes; l++) {
        double g[4];
        for (int j = 0; j < 4; j++) {
            const double *q = c.v + 256 * j + kPerLane * l;
            g[j] = (q[0] + q[1]) + (q[2] + q[3]);
        }
        v[l] = (g[0] + g[1]) + (g[2] + g[3]);
    }
    wave_scan_tree(v, [](double a, double b) { return a + b; }, 0.0);
    return v[kWaveLanes - 1];
}

// crossing_find: the crossing of a chunk from the planned count m_est under
// key (upward, or downward)
bool twin_crossing_find(const Rules &R, const Chunk &c, uint32_t key, int64_t m_est, bool down,
                        uint64_t *out)
{
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool sgn = (key >> 11) & 1u;
    // lanes' inclusive prefixes, the exclusive prefix before each lane
    std::vector<Pair> acc(kLanes * kPerLane);
    std::vector<Pair> pre(kLanes);
    bool bad1 = false;
    for (int lane = 0; lane < kLanes; lane++) {
        Pair a = pair_identity();
        for (int i = 0; i < kPerLane; i++) {
            if (i < c.cnt(lane)) {
                const TermInc t = R.inc(c.v[kPerLane * lane + i], scale, sgn);
                bad1 |= t.bad;
                a = R.comp(a, Pair{t.r0, t.r1});
            }
            acc[kPerLane * lane + i] = a;
        }
    }
    {
        Pair run = pair_identity();
        for (int lane = 0; lane < kLanes; lane++) {
            pre[lane] = run;
            run = R.comp(run, acc[kPerLane * lane + kPerLane - 1]);
        }
    }
    int j = -1;
    for (int lane = 0; lane < kLanes && j < 0; lane++) {
        for (int i = 0; i < kPerLane; i++) {
            const int idx = kPerLane * lane + i;
            if (idx >= c.len)
                break;
            const Pair pe = R.comp(pre[lane], acc[idx]);
            const int64_t ce = m_est + pair_at(pe, m_est);
            if (down ? ce < kCountLo : ce >= kCountHi) {
                j = idx;
                break;
            }
        }
    }
    if (bad1 || j < 0)
        return false;
    const int jl = j / kPerLane, ji = j % kPerLane;
    const Pair before = ji == 0 ? pre[jl] : R.comp(pre[jl], acc[j - 1]);
    const Pair at = R.comp(pre[jl], acc[j]);
    int64_t plo = 0, phi = 0;
    for (int idx = 0; idx < j; idx++) {
        const Pair pe = R.comp(pre[idx / kPerLane], acc[idx]);
        plo = std::min(plo, std::min(pe.r0, pe.r1));
        phi = std::max(phi, std::max(pe.r0, pe.r1));
    }
    // under the next binade: the whole chunk, and the terms after j as a run
    // (per lane in order, the wave scan tree, the four waves in order)
    const uint32_t key2 = down ? key - 1u : key + 1u;
    const int scale2 = 1075 - (int)(key2 & 0x7FFu);
    const bool sgn2 = (key2 >> 11) & 1u;
    bool bad2 = false;
    Pair tot2 = pair_identity();
    Run suf2 = run_identity();
    for (int wave = 0; wave < 4; wave++) {
        Pair whole[kWaveLanes];
        Run suf[kWaveLanes];
        for (int l = 0; l < kWaveLanes; l++) {
            const int lane = kWaveLanes * wave + l;
            whole[l] = pair_identity();
            suf[l] = run_identity();
            for (int i = 0; i < kPerLane; i++) {
                if (i < c.cnt(lane)) {
                    const int idx = kPerLane * lane + i;
                    const TermInc t = R.inc(c.v[idx], scale2, sgn2);
                    bad2 |= t.bad;
                    const Pair q{t.r0, t.r1};
                    whole[l] = R.comp(whole[l], q);
                    if (idx > j) {
                        const int64_t mn = std::min(t.r0, t.r1), mx = std::max(t.r0, t.r1);
                        suf[l] = R.rcomp(suf[l], Run{q, mn < 0 ? mn : 0, mx > 0 ? mx : 0, 0u});
                    }
                }
            }
        }
        wave_scan_tree(whole, [&](Pair a, Pair b) { return R.comp(a, b); }, pair_identity());
        wave_scan_tree(suf, [&](const Run &a, const Run &b) { return R.rcomp_sat(a, b); }, run_identity());
        tot2 = R.comp(tot2, whole[kWaveLanes - 1]);
        suf2 = R.rcomp_sat(suf2, suf[kWaveLanes - 1]);
    }
    if (bad2 || (suf2.flags & kFlagBad))
        return false;
    out[kXj] = enc_i64(j);
    out[kXpj1] = enc_i64(rec_pack(before));
    out[kXpj] = enc_i64(rec_pack(at));
    out[kXsuf] = enc_i64(rec_pack(suf2.p));
    out[kXwhole] = enc_i64(rec_pack(tot2));
    out[kXterm] = dbits(c.v[j]) ^ kInclXor;
    out[kXpreLo] = enc_i64(plo);
    out[kXpreHi] = enc_i64(phi);
    out[kXsufLo] = enc_i64(suf2.lo);
    out[kXsufHi] = enc_i64(suf2.hi);
    return true;
}

// ---------------------------------------------------------------------------
// The sum
// ---------------------------------------------------------------------------
struct Desc {
    uint32_t key;
    WaveRun r;
};

// A located crossing, as a tile keeps it
struct Cross {
    uint64_t w[kCrossWords];
    uint32_t key;
    bool down, neg;
    int len;
};

// A tile's record: a regular run, an irregular tile's step, or nothing
struct Tile {
    int kind;  // 1 regular, 2 step, 3 slow
    uint32_t key;
    Run run;   // regular: the tile's run; step: the run it ends with
    bool hasA;
    uint32_t akey;
    Run A;
    int nx;
    Cross x[2];
    uint32_t c0, c1;
};

struct Twin {
    Rules R;
    const double *x;
    size_t n;
    double init;
    uint32_t flags;
    exseq_stats st;
    uint32_t nch;
    std::vector<Desc> desc;
    std::vector<double> tsum;

    Chunk chunk(uint32_t c) const
    {
        Chunk k;
        const size_t b = (size_t)c * kLanes * kPerLane;
        k.len = (int)std::min<size_t>(kLanes * kPerLane, n - b);
        for (int i = 0; i < kLanes * kPerLane; i++)
            k.v[i] = i < k.len ? x[b + i] : 0.0;
        return k;
    }

    void note_fallback(uint32_t c)
    {
        const Chunk k = chunk(c);
        st.fallback_chunks++;
        st.fallback_terms += (uint64_t)k.len;
        if (st.first_fallback < 0)
            st.first_fallback = (int64_t)c;
    }

    // term by term
    double add_terms(double S, uint32_t c)
    {
        const size_t b = (size_t)c * kLanes * kPerLane;
        const size_t e = std::min(n, b + kLanes * kPerLane);
        for (size_t i = b; i < e; i++)
            S = S + x[i];
        note_fallback(c);
        return S;
    }

    // walk_lean: chunks [c_lo, c_hi) from their descriptors where they apply
    double walk_chunks(double S, uint32_t c_lo, uint32_t c_hi, bool use_desc)
    {
        for (uint32_t c = c_lo; c < c_hi; c++) {
            const uint32_t ks = key_of(S);
            if (use_desc && R.key_ok(ks, desc[c].key)) {
                const WaveRun &r = desc[c].r;
                const int64_t m = count_of(S);
                if (R.applies(m, r.p, r.lo, r.hi, r.flags)) {
                    S = R.advance(S, m, r.p);
                    st.fast_chunks++;
                    continue;
                }
            }
            S = add_terms(S, c);
        }
        return S;
    }

    // a run applied from S (a REG op), or false
    bool apply_run(double &S, uint32_t key, const Run &r) const
    {
        if ((r.flags & (kFlagBad | kFlagNonFinite)) || !R.key_ok(key_of(S), key))
            return false;
        const int64_t m = count_of(S);
        if (!R.applies(m, r.p, r.lo, r.hi, r.flags))
            return false;
        S = R.advance(S, m, r.p);
        return true;
    }

    // a CROSS op: the crossing term added where the tile found it
    bool apply_cross(double &S, const Cross &x) const
    {
        const uint32_t ks = key_of(S);
        const uint32_t key2 = x.down ? x.key - 1u : x.key + 1u;
        if (!R.key_ok(ks, x.key) || !key_has_fast_path(key2))
            return false;
        const int64_t j = dec_i64(x.w[kXj]);
        if (j >= x.len)
            return false;
        const int64_t m = count_of(S);
        const int64_t cb = j == 0 ? m : m + pair_at(rec_unpack(dec_i64(x.w[kXpj1])), m);
        const int64_t cj = m + pair_at(rec_unpack(dec_i64(x.w[kXpj])), m);
        const bool edge = x.down ? (cb >= kCountLo && cj < kCountLo) : (cb <= kCountHi - 1 && cj >= kCountHi);
        if (!edge)
            return false;
        if (x.neg && (m + dec_i64(x.w[kXpreLo]) < kCountLo + 1 || m + dec_i64(x.w[kXpreHi]) > kCountHi - 1))
            return false;
        const double sb = j == 0 ? S : assemble(ks, cb);
        S = sb + bitsd(x.w[kXterm] ^ kInclXor);
        return true;
    }

    // the head: chunks 0 .. 3 from init
    double head(uint32_t nk)
    {
        double S = init;
        for (uint32_t k = 0; k < nk; k++) {
            const uint32_t ks = key_of(S);
            if (k > 0 && key_has_fast_path(ks)) {
                const Chunk c = chunk(k);
                const WaveRun r = twin_block_run(R, c, ks);
                const int64_t m = count_of(S);
                if (R.applies(m, r.p, r.lo, r.hi, r.flags)) {
                    S = R.advance(S, m, r.p);
                    st.fast_chunks++;
                    continue;
                }
            }
            S = add_terms(S, k);
        }
        return S;
    }

    // a tile (chunks c0 .. c0 + 7) under its plan prefix P
    Tile tile(uint32_t c0, double P)
    {
        const uint32_t nk = std::min<uint32_t>(kTwinTile, nch - c0);
        Tile T;
        std::memset(&T, 0, sizeof(T));
        T.c0 = c0;
        T.c1 = c0 + nk;
        std::vector<Chunk> ch(kTwinTile);
        double pk[kTwinTile], tk[kTwinTile];
        uint32_t key[kTwinTile];
        bool cross[kTwinTile], down[kTwinTile];
        for (uint32_t k = 0; k < kTwinTile; k++) {
            if (k < nk)
                ch[k] = chunk(c0 + k);
            else {
                ch[k].len = 0;
                std::fill(ch[k].v, ch[k].v + kLanes * kPerLane, 0.0);
            }
            tk[k] = k < nk ? tsum[c0 + k] : 0.0;
        }
        double p = P;
        for (uint32_t k = 0; k < kTwinTile; k++) {
            pk[k] = p;
            key[k] = plan_key(p, flags);
            cross[k] = key_of(p + tk[k]) != key_of(p);
            down[k] = ((key_of(p + tk[k]) ^ key_of(p)) & 0x800u) == 0u &&
                      (key_of(p + tk[k]) & 0x7FFu) < (key_of(p) & 0x7FFu);
            p += tk[k];
        }
        WaveRun join[kTwinTile];
        for (uint32_t c = 0; c < kTwinTile; c++) {
            join[c] = twin_chunk_run(R, ch[c], key[c]);
            if (key_has_fast_path(key[c]) && key[c] == key_of(pk[c])) {
                const int64_t m = count_of(pk[c]);
                const int64_t mg = plan_margin(c0 + c + 1);
                bool near = m < count_floor(key[c]) + mg;
                if (join[c].flags & kFlagNeg)
                    near |= m + join[c].lo - mg < kCountLo + 1 || m + join[c].hi + mg > kCountHi - 1;
                else
                    near |= m + join[c].hi + mg > kCountHi;
                cross[c] |= near;
            }
            if (c < nk)
                desc[c0 + c] = Desc{key[c], join[c]};
        }
        // the crossings it locates
        uint32_t found = 0u;
        Cross xs[kTwinTile];
        for (uint32_t c = 0; c < nk; c++) {
            const uint32_t fl = join[c].flags;
            if (!(cross[c] && key_has_fast_path(key[c]) && key[c] == key_of(pk[c]) &&
                  key_has_fast_path(down[c] ? key[c] - 1u : key[c] + 1u) && !(fl & kFlagNonFinite)))
                continue;
            if (twin_crossing_find(R, ch[c], key[c], count_of(pk[c]), down[c], xs[c].w)) {
                found |= 1u << c;
                xs[c].key = key[c];
                xs[c].down = down[c];
                xs[c].len = ch[c].len;
                xs[c].neg = false;
            }
        }
        // a regular tile: one run
        bool regular = true;
        for (uint32_t k = 0; k < nk; k++)
            regular &= key_has_fast_path(key[k]) && key[k] == key[0] && !cross[k] &&
                       !(join[k].flags & (kFlagBad | kFlagNonFinite));
        if (regular) {
            bool plain = true, fall = true;
            int64_t sum = 0;
            for (uint32_t k = 0; k < nk; k++) {
                plain &= rising_run(join[k].p, join[k].flags);
                fall &= falling_run(join[k].p, join[k].lo, join[k].hi, join[k].flags);
                sum += join[k].p.r0;
            }
            Run tr = run_identity();
            if (plain) {
                tr = Run{Pair{sum, sum}, 0, sum, 0u};
            } else if (fall) {
                tr = Run{Pair{sum, sum}, sum, 0, kFlagNeg};
            } else {
                for (uint32_t k = 0; k < nk; k++)
                    tr = R.rcomp_sat(tr, Run{join[k].p, join[k].lo, join[k].hi, join[k].flags});
                if (!(tr.flags & kFlagNeg))
                    tr.hi = run_top(tr);
            }
            const int64_t lim = kCountLo + 1;
            if (tr.p.r0 > lim || tr.p.r0 < -lim || tr.lo < -lim || tr.hi > lim) {
                tr.flags |= kFlagBad;
                tr.p = pair_identity();
                tr.lo = tr.hi = 0;
            }
            // as the finisher reads it
            T.kind = 1;
            T.key = key[0];
            T.run.p = tr.p;
            T.run.flags = tr.flags & (kFlagNeg | kFlagBad);
            if (T.run.flags & kFlagNeg) {
                T.run.lo = tr.lo;
                T.run.hi = tr.hi;
            } else {
                T.run.lo = 0;
                T.run.hi = std::max(tr.p.r0, tr.p.r1);
            }
            return T;
        }
        // an irregular tile: run A, then up to two crossings with the chunks
        // after each folded into its rest
        bool fast = true;
        Run A = run_identity(), suf = run_identity();
        Pair whole = pair_identity();
        uint32_t akey = 0u, next_key = 0u;
        int nx = 0;
        auto close = [&](Cross &cx) {
            const int64_t lim = (int64_t)1 << 56;
            fast = fast && !(suf.flags & kFlagBad) && whole.r0 < lim && whole.r1 < lim &&
                   whole.r0 > -lim && whole.r1 > -lim;
            cx.w[kXsuf] = enc_i64(rec_pack(suf.p));
            cx.w[kXsufLo] = enc_i64(suf.lo);
            cx.w[kXsufHi] = enc_i64(suf.hi);
            cx.w[kXwhole] = enc_i64(rec_pack(whole));
            cx.neg = (suf.flags & kFlagNeg) != 0;
        };
        for (uint32_t k = 0; fast && k < nk; k++) {
            const WaveRun &q = join[k];
            const uint32_t kk = key[k];
            if ((found >> k) & 1u) {
                if (nx == 2 || (nx == 0 ? (akey != 0u && akey != kk) : kk != next_key)) {
                    fast = false;
                    break;
                }
                if (nx > 0)
                    close(T.x[nx - 1]);
                T.x[nx] = xs[k];
                suf = Run{rec_unpack(dec_i64(xs[k].w[kXsuf])), dec_i64(xs[k].w[kXsufLo]),
                          dec_i64(xs[k].w[kXsufHi]), q.flags & kFlagNeg};
                whole = rec_unpack(dec_i64(xs[k].w[kXwhole]));
                next_key = xs[k].down ? kk - 1u : kk + 1u;
                nx++;
                continue;
            }
            fast = key_has_fast_path(kk) && !(q.flags & (kFlagBad | kFlagNonFinite));
            if (nx == 0) {
                fast = fast && (akey == 0u || akey == kk);
                A = R.rcomp_sat(A, Run{q.p, q.lo, q.hi, q.flags});
                akey = kk;
            } else {
                fast = fast && kk == next_key;
                suf = R.rcomp_sat(suf, Run{q.p, q.lo, q.hi, q.flags & kFlagNeg});
                whole = R.comp(whole, q.p);
            }
        }
        if (fast && nx > 0)
            close(T.x[nx - 1]);
        fast = fast && (akey != 0u || nx > 0) && !(A.flags & kFlagBad);
        const bool lastdown = nx > 0 && T.x[nx - 1].down;
        const Run ex = nx > 0 ? suf : A;
        const bool neg = (ex.flags & kFlagNeg) || lastdown;
        const int64_t lim = kCountLo + 1;
        fast = fast && ex.p.r0 <= lim && ex.p.r0 >= -lim && ex.p.r1 <= lim && ex.p.r1 >= -lim &&
               (!neg || (ex.lo >= -lim && ex.hi <= lim));
        if (!fast) {
            T.kind = 3;
            return T;
        }
        T.kind = 2;
        T.nx = nx;
        T.hasA = akey != 0u;
        T.akey = akey;
        T.A = A;
        T.key = nx > 0 ? next_key : akey;
        T.run.p = ex.p;
        T.run.flags = neg ? kFlagNeg : 0u;
        if (neg) {
            T.run.lo = ex.lo;
            T.run.hi = ex.hi;
        } else {
            T.run.lo = 0;
            T.run.hi = std::max(ex.p.r0, ex.p.r1);
        }
        return T;
    }

    double run_sum()
    {
        std::memset(&st, 0, sizeof(st));
        st.first_fallback = -1;
        nch = (uint32_t)((n + kLanes * kPerLane - 1) / (kLanes * kPerLane));
        st.chunks = nch;
        if (n == 0)
            return init;
        for (size_t i = 0; i < n; i++)
            if (is_nonfinite(x[i]))
                st.flags |= EXSEQ_STAT_NONFINITE;
        desc.assign(nch, Desc{0u, WaveRun{pair_identity(), 0, 0, kFlagBad}});
        tsum.resize(nch);
        for (uint32_t c = 0; c < nch; c++)
            tsum[c] = twin_tree_sum(chunk(c));
        const uint32_t nk0 = std::min<uint32_t>(kTwinHead, nch);
        double S = head(nk0);
        if (nch <= (uint32_t)kTwinHead)
            return S;
        // the tiles, each under the plan prefix before it
        std::vector<Tile> tiles;
        double P = init;
        for (uint32_t k = 0; k < nk0; k++)
            P += tsum[k];
        for (uint32_t c0 = nk0; c0 < nch; c0 += kTwinTile) {
            tiles.push_back(tile(c0, P));
            for (uint32_t k = c0; k < std::min<uint32_t>(c0 + kTwinTile, nch); k++)
                P += tsum[k];
        }
        // the finisher, window by window
        for (size_t b = 0; b < tiles.size(); b += kTwinWindow)
            S = window(S, tiles, b, std::min(tiles.size(), b + kTwinWindow));
        return S;
    }

    // one finisher window: segments composed in pass_kernel's grouping, then
    // the ordered walk
    double window(double S, const std::vector<Tile> &tl, size_t b, size_t e)
    {
        const int cnt = (int)(e - b);
        auto runs = [&](int q) { return tl[b + q].kind == 1 || tl[b + q].kind == 2; };
        std::vector<char> head(cnt), end(cnt);
        for (int q = 0; q < cnt; q++) {
            const Tile &me = tl[b + q];
            head[q] = me.kind != 1 || q == 0 || !runs(q - 1) || tl[b + q - 1].key != me.key;
            end[q] = !runs(q) || q + 1 >= cnt || tl[b + q + 1].kind != 1 || tl[b + q + 1].key != me.key;
        }
        struct SR {
            Run r;
            int start, head;
        };
        auto op = [&](const SR &l, const SR &r) {
            if (r.head)
                return r;
            return SR{R.rcomp_sat(l.r, r.r), l.start, l.head};
        };
        auto val = [&](int q) {
            const Run rr = runs(q) ? tl[b + q].run : run_identity();
            return SR{rr, head[q] ? q : -1, head[q] ? 1 : 0};
        };
        // four tiles per lane in order, the wave scan tree, the carry over
        // the waves: the exclusive value before each lane
        std::vector<SR> lane(kLanes), excl(kLanes);
        for (int t = 0; t < kLanes; t++) {
            SR v{run_identity(), -1, 0};
            for (int j = 0; j < 4; j++)
                if (4 * t + j < cnt)
                    v = op(v, val(4 * t + j));
            lane[t] = v;
        }
        SR carry{run_identity(), -1, 0};
        for (int w = 0; w < 4; w++) {
            SR inc[kWaveLanes];
            for (int l = 0; l < kWaveLanes; l++)
                inc[l] = lane[kWaveLanes * w + l];
            wave_scan_tree(inc, op, SR{run_identity(), -1, 0});
            for (int l = 0; l < kWaveLanes; l++)
                excl[kWaveLanes * w + l] = op(carry, l == 0 ? SR{run_identity(), -1, 0} : inc[l - 1]);
            carry = op(carry, inc[kWaveLanes - 1]);
        }
        // each tile's inclusive segment run; events at segment ends, walked
        // in order
        std::vector<SR> incl(cnt);
        for (int t = 0; t < kLanes; t++) {
            SR run = excl[t];
            for (int j = 0; j < 4; j++) {
                const int q = 4 * t + j;
                if (q >= cnt)
                    break;
                run = op(run, val(q));
                incl[q] = run;
            }
        }
        for (int q = 0; q < cnt; q++) {
            if (!end[q])
                continue;
            const int qs = incl[q].start >= 0 && runs(q) ? incl[q].start : q;
            const Tile &h = tl[b + qs];
            const uint32_t c_lo = h.c0, c_hi = tl[b + q].c1;
            const double S0 = S;
            bool ok = false;
            if (h.kind == 1) {
                ok = apply_run(S, tl[b + q].key, incl[q].r);
            } else if (h.kind == 2) {
                ok = true;
                if (h.nx > 0 && h.hasA)
                    ok = apply_run(S, h.akey, h.A);
                for (int j = 0; ok && j < h.nx; j++) {
                    ok = apply_cross(S, h.x[j]);
                    const uint32_t k2 = h.x[j].down ? h.x[j].key - 1u : h.x[j].key + 1u;
                    if (ok && j < h.nx - 1)
                        ok = apply_run(S, k2, Run{rec_unpack(dec_i64(h.x[j].w[kXsuf])),
                                                  dec_i64(h.x[j].w[kXsufLo]), dec_i64(h.x[j].w[kXsufHi]),
                                                  (h.x[j].neg || h.x[j].down) ? kFlagNeg : 0u});
                }
                if (ok)
                    ok = apply_run(S, tl[b + q].key, incl[q].r);
            }
            if (ok) {
                st.fast_chunks += c_hi - c_lo;
            } else {
                S = walk_chunks(S0, c_lo, c_hi, true);
            }
        }
        return S;
    }

    // -----------------------------------------------------------------------
    // The tile chain (tile_kernel with four chunks per tile, then the chain):
    // each chunk's four wave parts in the workgroup layout, joined; a regular
    // tile's one run as its look-back words hold it; chain_back's grouping
    // of the regular tiles before an irregular one (four per lane, earlier
    // tiles first; per wave the integer sum, the falling sum, the pairs alone
    // or the full runs, then the reversed wave tree; the waves in reverse;
    // the rounds of 1024 tiles); the irregular tiles' chunk loop from the
    // exact sum (a chunk's run where it applies, else its located crossing,
    // else its terms in order); and walk_kernel's resume from the last exact
    // sum where the chain stops.  The plan prefix before a tile is init plus
    // the earlier tiles' sums in order, moved by skew * 2^-30 of itself: the
    // plan never decides the bits, so no skew may change them.
    // -----------------------------------------------------------------------
    static constexpr int kCT = 4;
    struct CTile {
        bool regular;
        uint64_t w[4];  // a regular tile's look-back words
        uint32_t key[kCT];
        WaveRun join[kCT];
        bool hasx[kCT];
        Cross x[kCT];
    };
    int64_t skew = 0;
    uint64_t paths[6] = {0, 0, 0, 0, 0, 0};  // waves composed: plain, falling, pairs, runs; applied; stops

    CTile chain_tile(uint32_t c0, double P)
    {
        CTile T;
        std::memset(&T, 0, sizeof(T));
        const uint32_t nk = std::min<uint32_t>(kCT, nch - c0);
        std::vector<Chunk> ch(kCT);
        double pk[kCT], tk[kCT];
        bool cross[kCT], down[kCT];
        for (uint32_t k = 0; k < kCT; k++) {
            if (k < nk) {
                ch[k] = chunk(c0 + k);
            } else {
                ch[k].len = 0;
                std::fill(ch[k].v, ch[k].v + kLanes * kPerLane, 0.0);
            }
            tk[k] = k < nk ? tsum[c0 + k] : 0.0;
        }
        double p = P;
        for (uint32_t k = 0; k < kCT; k++) {
            pk[k] = p;
            T.key[k] = plan_key(p, flags);
            cross[k] = key_of(p + tk[k]) != key_of(p);
            down[k] = ((key_of(p + tk[k]) ^ key_of(p)) & 0x800u) == 0u &&
                      (key_of(p + tk[k]) & 0x7FFu) < (key_of(p) & 0x7FFu);
            p += tk[k];
        }
        for (uint32_t k = 0; k < kCT; k++) {
            const uint32_t kk = T.key[k];
            WaveRun w[4];
            for (int wv = 0; wv < 4; wv++) {
                if (key_has_fast_path(kk)) {
                    w[wv] = twin_wave_run(R, ch[k], wv, kk);
                } else {
                    bool nf = false;
                    for (int q = kWaveLanes * kPerLane * wv; q < kWaveLanes * kPerLane * (wv + 1); q++)
                        nf |= is_nonfinite(ch[k].v[q]);
                    w[wv] = WaveRun{pair_identity(), 0, 0, nf ? kFlagNonFinite : 0u};
                }
            }
            const WaveRun r = twin_join(R, w);
            bool cc = cross[k];
            if (key_has_fast_path(kk) && kk == key_of(pk[k])) {
                const int64_t m = count_of(pk[k]);
                const int64_t mg = plan_margin(c0 + k + 1);
                bool near = m < count_floor(kk) + mg;
                if (r.flags & kFlagNeg)
                    near |= m + r.lo - mg < kCountLo + 1 || m + r.hi + mg > kCountHi - 1;
                else
                    near |= m + r.hi + mg > kCountHi;
                cc |= near;
            }
            T.join[k] = r;
            cross[k] = cc;
            if (k < nk)
                desc[c0 + k] = Desc{kk, r};
        }
        bool regular = c0 != 0 && c0 + kCT < nch;
        for (uint32_t k = 0; k < kCT; k++)
            regular &= key_has_fast_path(T.key[k]) && T.key[k] == T.key[0] && !cross[k] &&
                       !(T.join[k].flags & (kFlagBad | kFlagNonFinite));
        if (regular) {
            bool plain = true, fall = true;
            int64_t sum = 0;
            for (uint32_t k = 0; k < kCT; k++) {
                const WaveRun &q = T.join[k];
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
                for (uint32_t k = 0; k < kCT; k++)
                    tr = R.rcomp_sat(tr, Run{T.join[k].p, T.join[k].lo, T.join[k].hi, T.join[k].flags});
            }
            const int64_t dr = tr.p.r1 - tr.p.r0;
            T.regular = true;
            T.w[0] = kAggPresent | kAggRegular | (uint64_t)(T.key[0] & kKeyMask) |
                     ((uint64_t)(dr + 1) << kDrShift) | (uint64_t)(tr.flags & kFlagNeg);
            T.w[1] = enc_i64(tr.p.r0);
            T.w[2] = enc_i64(tr.lo);
            T.w[3] = enc_i64(tr.hi);
            return T;
        }
        for (uint32_t k = 0; k < nk; k++) {
            const uint32_t kk = T.key[k];
            if (!(c0 != 0 && cross[k] && key_has_fast_path(kk) && kk == key_of(pk[k]) &&
                  key_has_fast_path(down[k] ? kk - 1u : kk + 1u) &&
                  !(T.join[k].flags & kFlagNonFinite)))
                continue;
            if (twin_crossing_find(R, ch[k], kk, count_of(pk[k]), down[k], T.x[k].w)) {
                T.hasx[k] = true;
                T.x[k].key = kk;
                T.x[k].down = down[k];
                T.x[k].len = ch[k].len;
            }
        }
        return T;
    }

    // A regular tile's run as chain_back decodes its words
    static Run agg_run(const uint64_t *w)
    {
        const int64_t r0 = dec_i64(w[1]);
        return Run{Pair{r0, r0 + (int64_t)((w[0] >> kDrShift) & 3u) - 1}, dec_i64(w[2]), dec_i64(w[3]),
                   (uint32_t)w[0] & (kFlagNeg | kFlagBad | kFlagNonFinite)};
    }

    Pair pair_clamped(Pair a, Pair b) const
    {
        const int64_t lim = (int64_t)1 << 57;
        Pair c = R.comp(a, b);
        c.r0 = c.r0 > lim ? lim : c.r0;
        c.r1 = c.r1 > lim ? lim : c.r1;
        return c;
    }

    // chain_back from irregular tile tl: 0 ok, 1 the keys differ, 2 lost
    int chain_back_twin(const std::vector<CTile> &tiles, uint32_t tl, Run &acc, uint32_t &key0,
                        int64_t &xp)
    {
        constexpr int kPer = 4, kRound = kPer * kLanes;
        const int64_t big = (int64_t)1 << 56;
        acc = run_identity();
        key0 = 0u;
        xp = -1;
        bool keys_ok = true;
        for (int64_t j0 = (int64_t)tl - 1; j0 >= 0; j0 -= kRound) {
            if (j0 == (int64_t)tl - 1)
                key0 = tiles[j0].regular ? (uint32_t)(tiles[j0].w[0] & kKeyMask) : 0u;
            int first = kRound;
            for (int q = 0; q < kRound; q++)
                if (j0 - q >= 0 && !tiles[j0 - q].regular) {
                    first = q;
                    break;
                }
            auto in = [&](int t, int i) { return j0 - kPer * t - i >= 0 && kPer * t + i < first; };
            Run wr[4];
            bool anybad = false;
            for (int wv = 0; wv < 4; wv++) {
                bool plain = true, fall = true, nonneg = true, any = false;
                int64_t tot = 0;
                for (int l = 0; l < kWaveLanes; l++) {
                    const int t = kWaveLanes * wv + l;
                    for (int i = kPer - 1; i >= 0; i--) {
                        if (!in(t, i))
                            continue;
                        const uint64_t *w = tiles[j0 - kPer * t - i].w;
                        const Run ti = agg_run(w);
                        plain &= rising_run(ti.p, ti.flags);
                        fall &= falling_run(ti.p, ti.lo, ti.hi, ti.flags);
                        nonneg &= ti.flags == 0u && ti.p.r0 >= 0 && ti.p.r1 >= 0;
                        tot += ti.p.r0;
                        anybad |= ((uint32_t)w[0] & kKeyMask) != key0;
                        any = true;
                    }
                }
                Run r;
                if (plain) {
                    r = Run{Pair{tot, tot}, 0, tot, 0u};
                    if (tot > big)
                        r = Run{Pair{0, 0}, 0, 0, kFlagBad};
                    paths[0] += any;
                } else if (fall) {
                    r = Run{Pair{tot, tot}, tot, 0, kFlagNeg};
                    if (tot < -big)
                        r = Run{Pair{0, 0}, 0, 0, kFlagBad};
                    paths[1] += any;
                } else if (nonneg) {
                    Pair pp[kWaveLanes];
                    for (int l = 0; l < kWaveLanes; l++) {
                        const int t = kWaveLanes * wv + l;
                        pp[l] = pair_identity();
                        for (int i = kPer - 1; i >= 0; i--)
                            if (in(t, i))
                                pp[l] = pair_clamped(pp[l], agg_run(tiles[j0 - kPer * t - i].w).p);
                    }
                    wave_scan_tree(pp, [&](Pair s, Pair v) { return pair_clamped(v, s); }, pair_identity());
                    const Pair q = pp[kWaveLanes - 1];
                    r = Run{q, 0, 0, 0u};
                    if (q.r0 > big || q.r1 > big)
                        r = Run{Pair{0, 0}, 0, 0, kFlagBad};
                    paths[2] += any;
                } else {
                    Run rr[kWaveLanes];
                    for (int l = 0; l < kWaveLanes; l++) {
                        const int t = kWaveLanes * wv + l;
                        rr[l] = run_identity();
                        for (int i = kPer - 1; i >= 0; i--)
                            if (in(t, i))
                                rr[l] = R.rcomp_sat(rr[l], agg_run(tiles[j0 - kPer * t - i].w));
                    }
                    wave_scan_tree(rr, [&](Run s, Run v) { return R.rcomp_sat(v, s); }, run_identity());
                    r = rr[kWaveLanes - 1];
                    paths[3] += any;
                }
                wr[wv] = r;
            }
            Run Rr = wr[3];
            for (int k = 2; k >= 0; k--)
                Rr = R.rcomp_sat(Rr, wr[k]);
            keys_ok &= !anybad;
            acc = R.rcomp_sat(Rr, acc);
            if (first < kRound) {
                xp = j0 - first;
                break;
            }
        }
        if (xp < 0)
            return 2;
        return keys_ok ? 0 : 1;
    }

    // chunk c's terms from position pos on, in order
    double add_terms_from(double S, uint32_t c, int pos)
    {
        const size_t b = (size_t)c * kLanes * kPerLane;
        const size_t e = std::min(n, b + kLanes * kPerLane);
        for (size_t i = b + (size_t)pos; i < e; i++)
            S = S + x[i];
        note_fallback(c);
        return S;
    }

    // an irregular tile's chunks [kfirst, nk) from the exact sum S
    double chain_chunks(double S, const CTile &T, uint32_t c0, uint32_t kfirst, uint32_t nk)
    {
        for (uint32_t k = kfirst; k < nk; k++) {
            const WaveRun &r = T.join[k];
            const uint32_t fl = r.flags & (kFlagNeg | kFlagBad | kFlagNonFinite);
            const int64_t m = count_of(S);
            if (R.key_ok(key_of(S), T.key[k]) && R.applies(m, r.p, r.lo, r.hi, fl)) {
                S = R.advance(S, m, r.p);
                st.fast_chunks++;
                continue;
            }
            int pos = 0, xr = 0;
            if (T.hasx[k])
                xr = crossing_apply(T.x[k].w, T.x[k].len, T.key[k], fl, T.x[k].down, S, pos);
            if (xr == 1) {
                st.fast_chunks++;
                continue;
            }
            if (xr == 0)
                pos = 0;
            S = add_terms_from(S, c0 + k, pos);
        }
        return S;
    }

    double run_chain()
    {
        std::memset(&st, 0, sizeof(st));
        st.first_fallback = -1;
        nch = (uint32_t)((n + kLanes * kPerLane - 1) / (kLanes * kPerLane));
        st.chunks = nch;
        if (n == 0)
            return init;
        for (size_t i = 0; i < n; i++)
            if (is_nonfinite(x[i]))
                st.flags |= EXSEQ_STAT_NONFINITE;
        desc.assign(nch, Desc{0u, WaveRun{pair_identity(), 0, 0, kFlagBad}});
        tsum.resize(nch);
        for (uint32_t c = 0; c < nch; c++)
            tsum[c] = twin_tree_sum(chunk(c));
        const uint32_t mode = flags & EXSEQ_PLAN_MASK;
        const bool looks = mode != EXSEQ_PLAN_ALL_FALLBACK && mode != EXSEQ_PLAN_FIXED;
        const uint32_t ntl = (nch + kCT - 1) / kCT;
        std::vector<CTile> tiles;
        tiles.reserve(ntl);
        double P = init;
        for (uint32_t tl = 0; tl < ntl; tl++) {
            const double Pk = P + std::ldexp((double)skew, -30) * P;
            tiles.push_back(chain_tile(tl * kCT, looks ? Pk : 0.0));
            for (uint32_t c = tl * kCT; c < std::min<uint32_t>(tl * kCT + kCT, nch); c++)
                P += tsum[c];
        }
        if (!chain_on(flags))
            return walk_chunks(init, 0, nch, true);
        // the head, then the first tile's other chunks
        double S = add_terms(init, 0);
        S = chain_chunks(S, tiles[0], 0, 1, std::min<uint32_t>(kCT, nch));
        for (uint32_t tl = 1; tl < ntl; tl++) {
            if (tiles[tl].regular)
                continue;
            Run acc;
            uint32_t key0;
            int64_t xp;
            bool ok = chain_back_twin(tiles, tl, acc, key0, xp) == 0;
            if (ok && xp != (int64_t)tl - 1) {
                const int64_t m = count_of(S);
                ok = R.key_ok(key_of(S), key0) &&
                     R.applies(m, acc.p, acc.lo, acc.hi, acc.flags & (kFlagNeg | kFlagBad | kFlagNonFinite));
                if (ok) {
                    S = R.advance(S, m, acc.p);
                    st.fast_chunks += (uint64_t)kCT * (tl - 1 - (uint32_t)xp);
                    paths[4]++;
                }
            }
            if (!ok) {
                // the walk resumes after the last tile that published its sum
                paths[5]++;
                uint32_t j = tl - 1;
                while (tiles[j].regular)
                    j--;
                return walk_chunks(S, (j + 1) * kCT, nch, true);
            }
            S = chain_chunks(S, tiles[tl], tl * kCT, 0, std::min<uint32_t>(kCT, nch - tl * kCT));
        }
        return S;
    }
};

}  // namespace

// The twin's sum of x[0 .. n) from init (flags: a plan mode; mut: planted
// mutations, EXSEQ_MUT_*).  stats: nullable host pointer.
extern "C" double exseq_twin_seq_sum_f64(const double *x, size_t n, double init, uint32_t flags,
                                         uint32_t mut, exseq_stats *stats)
{
    Twin tw;
    tw.R = Rules{mut};
    tw.x = x;
    tw.n = n;
    tw.init = init;
    tw.flags = flags;
    const double S = tw.run_sum();
    if (stats)
        *stats = tw.st;
    return S;
}

// The twin of the tile chain (four chunks per tile): the sum of x[0 .. n)
// from init, its plan prefixes moved by skew * 2^-30 of themselves (flags: a
// plan mode; mut: planted mutations).  paths: nullable host array of 6 counts
// (waves of regular tiles composed as integer sums, falling sums, pairs
// alone, full runs; composed runs applied; stops of the chain).
extern "C" double exseq_twin_chain_sum_f64(const double *x, size_t n, double init, uint32_t flags,
                                           uint32_t mut, int64_t skew, exseq_stats *stats,
                                           uint64_t *paths)
{
    Twin tw;
    tw.R = Rules{mut};
    tw.x = x;
    tw.n = n;
    tw.init = init;
    tw.flags = flags;
    tw.skew = skew;
    const double S = tw.run_chain();
    if (stats)
        *stats = tw.st;
    if (paths)
        for (int k = 0; k < 6; k++)
            paths[k] = tw.paths[k];
    return S;
}
