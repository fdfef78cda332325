// Host model of the exact sequential sum: the rules of exseq_rules.h applied
// chunk by chunk on the CPU, each chunk's run composed term by term (a left
// fold), with the plan overrides and the four rule mutations of Research-1433
// "Forming the CPU's sequential double sums on a GPU, bit for bit", Findings
// "Tests".  It checks the rules themselves, not the kernels' grouping of the
// terms into lanes, waves and tiles (the composition twin replays that).  The
// GPU entry points never call it.
#include <algorithm>
#include <cstring>
#include <vector>

#include "exseq.h"
#include "exseq_rules.h"

using namespace exseq;

namespace {

// The plan key for a chunk from the estimate p of the running sum at its
// start; key 0 means "no fast path" (the chunk is added term by term).
uint32_t plan_key(double p, uint32_t flags)
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

// Fixed-shape tree sum of one chunk (the plan's input; any fixed shape works
// because the plan never changes a result).
double chunk_tree_sum(const double *x, size_t len)
{
    std::vector<double> v(x, x + len);
    size_t m = len;
    while (m > 1) {
        size_t h = (m + 1) / 2;
        for (size_t i = 0; i + h < m; i++)
            v[i] = v[i] + v[i + h];
        m = h;
    }
    return len ? v[0] : 0.0;
}

Run describe_chunk(const double *x, size_t len, uint32_t key, uint32_t mut)
{
    Run acc = run_identity();
    const int scale = 1075 - (int)(key & 0x7FFu);
    const bool sgn = (key >> 11) & 1u;
    for (size_t i = 0; i < len; i++) {
        TermInc t = term_inc(x[i], scale, sgn);
        if (mut & EXSEQ_MUT_TIE_UP) {
            int64_t up = std::max(t.r0, t.r1);
            t.r0 = t.r1 = up;
        }
        Run r = run_of_term(t, is_nonfinite(x[i]));
        if (mut & EXSEQ_MUT_IGNORE_PARITY) {
            Run c;
            c.p.r0 = acc.p.r0 + r.p.r0;
            c.p.r1 = acc.p.r1 + r.p.r1;
            c.lo = acc.lo + r.lo;
            c.hi = acc.hi + r.hi;
            c.flags = acc.flags | r.flags;
            acc = c;
        } else {
            acc = run_compose(acc, r);
        }
    }
    return acc;
}

}  // namespace

extern "C" double exseq_model_seq_sum_f64(const double *x, size_t n, double init,
                                          size_t chunk_terms, uint32_t flags,
                                          uint32_t mut, exseq_stats *stats)
{
    exseq_stats st;
    std::memset(&st, 0, sizeof(st));
    st.first_fallback = -1;
    const size_t C = chunk_terms ? chunk_terms : 1;
    const size_t nch = (n + C - 1) / C;

    // a2: the plan -- prefix of the chunks' tree sums from init.
    std::vector<uint32_t> key(nch);
    double p = init;
    for (size_t c = 0; c < nch; c++) {
        size_t len = std::min(C, n - c * C);
        key[c] = plan_key(p, flags);
        p += chunk_tree_sum(x + c * C, len);
    }

    // a3-a6: descriptors under the plan, then the ordered walk.
    double s = init;
    for (size_t c = 0; c < nch; c++) {
        const double *xc = x + c * C;
        size_t len = std::min(C, n - c * C);
        Run run = describe_chunk(xc, len, key[c], mut);
        if (run.flags & kFlagNonFinite)
            st.flags |= EXSEQ_STAT_NONFINITE;
        uint32_t ks = key_of(s);
        if (ks != key[c])
            st.plan_misses++;
        bool fast = false;
        if (key_has_fast_path(key[c]) && key_has_fast_path(ks) &&
            (ks == key[c] || (mut & EXSEQ_MUT_NO_BINADE_CHECK))) {
            int64_t m = count_of(s);
            bool ok;
            if (mut & EXSEQ_MUT_NO_UPPER_CHECK) {
                ok = !(run.flags & (kFlagBad | kFlagNonFinite)) &&
                     (!(run.flags & kFlagNeg) || m + run.lo >= kCountLo + 1);
            } else {
                ok = run_applies(m, run.p, run.lo, run.hi, run.flags);
            }
            if (ok) {
                int64_t cnt = m + pair_at(run.p, m);
                if (cnt > kCountHi)   // only reachable under a mutation
                    cnt = kCountHi;
                if (cnt < count_floor(ks))
                    cnt = count_floor(ks);
                s = assemble(ks, cnt);
                fast = true;
            }
        }
        if (!fast) {
            for (size_t i = 0; i < len; i++)
                s += xc[i];
            st.fallback_chunks++;
            st.fallback_terms += len;
            if (st.first_fallback < 0)
                st.first_fallback = (int64_t)c;
        } else {
            st.fast_chunks++;
        }
        st.chunks++;
    }
    if (stats)
        *stats = st;
    return s;
}
