// The rules of the exact sequential sum, shared by the gfx950 kernels and the
// host model of the method.  Everything here is integer or exactly-rounded
// fp64 arithmetic with a stated result; nothing depends on association order.
//
// The method (Research-1433 "Forming the CPU's sequential double sums on a
// GPU, bit for bit", Findings 2-4; Research-1424 "integer_ssim_cuda and the
// CPU's frame sum", Findings 3):
//
//  * Within one binade [2^e, 2^(e+1)) every double is an integer multiple
//    of the binade's unit u = 2^(e-52), with a multiplier (the count)
//    between 2^52 and 2^53.  So while the running sum stays inside the
//    binade, adding a term moves the count by that term measured in units
//    and rounded to a whole number; the sum is an integer sum of those
//    increments, and integer sums may be grouped in any way.
//  * A term exactly half way between two counts rounds to the even count, so
//    r depends on the parity of m: every term, and every run, is a pair of
//    increments (start count even, start count odd).  Two runs compose by
//    taking the second run's increment for the parity the first run leaves.
//    This composition is associative but not commutative.
//  * A run may be applied to an exact S only if S is in the binade the run
//    was formed for and every prefix of the run keeps the count inside the
//    binade (the smallest/largest prefix check).  Otherwise its terms are
//    added one by one.
//
// How an increment pair is formed here (this library's own construction, not
// the pages' bit-shift form): y = x * 2^(52 - e) is exact (a power-of-two
// scaling).  For |y| < 2^51 the fp64 add t = fl(M + y) with M = 1.5 * 2^52
// lands in [2^52, 2^53], where doubles are exactly the integers; so t - M is
// y rounded to an integer, and a tie goes to the even t.  With M even that
// is the increment for an even start count; with M + 1 (odd) a tie makes
// M + 1 + r even, i.e. m + r even for an odd m.  The increment is read from
// the bit patterns: bits(t) - bits(M) = t - M for t in [2^52, 2^53].  A
// negative running sum is mirrored (-S is in a positive binade, and RNE is
// sign-symmetric), so the terms are negated.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#define EXSEQ_HD __host__ __device__ __forceinline__

namespace exseq {

constexpr double kMagic0 = 6755399441055744.0;          // 1.5 * 2^52, even
constexpr double kMagic1 = 6755399441055745.0;          // 1.5 * 2^52 + 1, odd
constexpr int64_t kMagic0Bits = 0x4338000000000000LL;
constexpr int64_t kMagic1Bits = 0x4338000000000001LL;
constexpr uint32_t kMagic0Hi = 0x43380000u;              // high word of M0: exponent field 0x433
constexpr double kHugeY = 2251799813685248.0;           // 2^51
constexpr int64_t kCountLo = 1LL << 52;                 // counts of one binade
constexpr int64_t kCountHi = 1LL << 53;
constexpr uint64_t kFracMask = (1ULL << 52) - 1;

// Descriptor flag bits (the low 12 bits of `meta` hold the plan key).
constexpr uint32_t kKeyMask = 0xFFFu;
constexpr uint32_t kDrShift = 12;        // (r1 - r0) + 1 in bits 12..13
constexpr uint32_t kFlagNeg = 1u << 14;  // some term had y < 0
constexpr uint32_t kFlagBad = 1u << 15;  // some term had |y| >= 2^51 or was NaN
constexpr uint32_t kFlagNonFinite = 1u << 16;  // some term was +-inf or NaN
constexpr uint32_t kFlagCross = 1u << 17;      // the plan expects a binade crossing
constexpr uint32_t kFlagExact = 1u << 18;      // the exact sum after the chunk is known
constexpr uint32_t kFlagResolved = 1u << 19;   // the chunk was added term by term

EXSEQ_HD uint64_t dbits(double x) { return __builtin_bit_cast(uint64_t, x); }
EXSEQ_HD double bitsd(uint64_t b) { return __builtin_bit_cast(double, b); }

// Plan key of a value: its sign and biased exponent (the top 12 bits).  A key
// names a binade with a fast path only when the value is finite and not -0.
//
// The subnormal range: below 2^-1022 every double is a multiple of 2^-1074,
// the unit of the lowest normal binade [2^-1022, 2^-1021) too.  So the two
// form one range [0, 2^-1021) with one unit, where a sum is an integer count
// in [0, 2^53) rounded to the nearest count (ties to even) exactly as in a
// binade.  Subnormals and +0 take the key of that lowest binade (biased
// exponent 1), and their count has no implicit bit; -0 keeps its own key
// (no fast path), since adding +0 to it gives +0 and a count cannot say so.
// Runs keep their usual lower bound (every prefix count at least 2^52 + 1
// where a term is negative), so a run is applied below 2^-1022 only when it
// rises (Research-1433 "Forming the CPU's sequential double sums on a GPU,
// bit for bit" is silent on this range; this reading is the build's).
EXSEQ_HD uint32_t key_of(double v)
{
    const uint64_t b = dbits(v);
    const uint32_t k = (uint32_t)(b >> 52);
    return ((k & 0x7FFu) == 0u && b != 0x8000000000000000ULL) ? k | 1u : k;
}
EXSEQ_HD bool key_has_fast_path(uint32_t key)
{
    uint32_t e = key & 0x7FFu;
    return e != 0u && e != 0x7FFu;
}

// Count of S in its binade: the 52 fraction bits plus the implicit bit, m in
// [2^52, 2^53) for a normal S; the fraction bits alone, m in [0, 2^52), for a
// subnormal S or +0 (in the lowest binade's range, see key_of).
EXSEQ_HD int64_t count_of(double s)
{
    const uint64_t b = dbits(s);
    return (int64_t)((b & kFracMask) | ((b & 0x7FF0000000000000ULL) ? (1ULL << 52) : 0ULL));
}

// The lowest count a binade's range holds: 0 for the lowest binade (which
// takes in the subnormals), 2^52 for the others.
EXSEQ_HD int64_t count_floor(uint32_t key) { return (key & 0x7FFu) == 1u ? 0 : kCountLo; }

// S = sign * count * 2^(E - 1075) for count in [2^52, 2^53]; a count of 2^53
// carries into the exponent (2^(e+1)), and past the largest binade it gives
// the correctly signed infinity, which is what the add rounds to there.
EXSEQ_HD double assemble(uint32_t key, int64_t count)
{
    return bitsd(((uint64_t)key << 52) + (uint64_t)(count - kCountLo));
}

// One term under the plan key (sign sgn, biased exponent E of the binade):
// the scaled term y and its increments for an even and an odd start count.
struct TermInc {
    int64_t r0, r1;
    bool neg;  // y < 0
    bool bad;  // |y| >= 2^51 (or NaN): the run cannot be applied
};

// `scale` is 1075 - E; `sgn` is the plan's sign bit (mirror the terms).
EXSEQ_HD TermInc term_inc(double x, int scale, bool sgn)
{
    double y = ldexp(sgn ? -x : x, scale);
    TermInc t;
    t.bad = !(fabs(y) < kHugeY);
    double a0 = kMagic0 + y;
    double a1 = kMagic1 + y;
    t.r0 = t.bad ? 0 : (int64_t)dbits(a0) - kMagic0Bits;
    t.r1 = t.bad ? 0 : (int64_t)dbits(a1) - kMagic1Bits;
    t.neg = y < 0.0;
    return t;
}

// A run of terms as a function of the start count's parity.
struct Pair {
    int64_t r0, r1;
};

EXSEQ_HD Pair pair_identity() { return Pair{0, 0}; }

// a then b: the start parity p picks a's increment, which leaves the parity
// (p + a.r_p) & 1 for b.
EXSEQ_HD Pair compose(Pair a, Pair b)
{
    Pair c;
    c.r0 = a.r0 + ((a.r0 & 1) ? b.r1 : b.r0);
    c.r1 = a.r1 + (((a.r1 + 1) & 1) ? b.r1 : b.r0);
    return c;
}

EXSEQ_HD int64_t pair_at(Pair p, int64_t m) { return (m & 1) ? p.r1 : p.r0; }

// A chunk's descriptor.  lo/hi bound the increment of every prefix of the
// run, for either start parity (lo <= 0 <= hi: the empty prefix counts).
struct Run {
    Pair p;
    int64_t lo, hi;
    uint32_t flags;  // kFlagNeg | kFlagBad | kFlagNonFinite
};

EXSEQ_HD Run run_identity() { return Run{Pair{0, 0}, 0, 0, 0u}; }

EXSEQ_HD Run run_of_term(const TermInc& t, bool nonfinite)
{
    Run r;
    r.p = Pair{t.r0, t.r1};
    int64_t mn = t.r0 < t.r1 ? t.r0 : t.r1;
    int64_t mx = t.r0 < t.r1 ? t.r1 : t.r0;
    r.lo = mn < 0 ? mn : 0;
    r.hi = mx > 0 ? mx : 0;
    r.flags = (t.neg ? kFlagNeg : 0u) | (t.bad ? kFlagBad : 0u) |
              (nonfinite ? kFlagNonFinite : 0u);
    return r;
}

// The largest prefix of a run.  A run without a negative term rises
// monotonically along either start parity, so its largest prefix is its
// larger total; producers of such runs may leave hi at 0 and rely on this.
EXSEQ_HD int64_t run_top(const Run& r)
{
    if (r.flags & kFlagNeg)
        return r.hi;
    const int64_t t = r.p.r0 < r.p.r1 ? r.p.r1 : r.p.r0;
    return t > r.hi ? t : r.hi;
}

// a then b.  A prefix of the composition is a prefix of a, or all of a
// (r0 or r1 of a, by the start parity) followed by a prefix of b, so the
// bounds compose as a minimum and a maximum (sound for either start parity
// and for any grouping of the terms).  A rising part's largest prefix is
// taken as its total, so that a rise after a negative term is bounded too.
EXSEQ_HD Run run_compose(const Run& a, const Run& b)
{
    Run c;
    c.p = compose(a.p, b.p);
    const int64_t amin = a.p.r0 < a.p.r1 ? a.p.r0 : a.p.r1;
    const int64_t amax = a.p.r0 < a.p.r1 ? a.p.r1 : a.p.r0;
    const int64_t ahi = run_top(a), bhi = run_top(b);
    c.lo = a.lo < amin + b.lo ? a.lo : amin + b.lo;
    c.hi = ahi > amax + bhi ? ahi : amax + bhi;
    c.flags = a.flags | b.flags;
    return c;
}

// May a run formed under some key be applied from start count m (with S
// already known to be in that key's binade)?  Research-1424 Findings 3 (every
// prefix count inside [2^52 + 1, 2^53 - 1]) for runs with a negative term;
// Research-1433 Findings 4 (non-negative terms: the result bounds every
// intermediate value and may reach 2^(e+1)) for the others.
EXSEQ_HD bool run_applies(int64_t m, Pair p, int64_t lo, int64_t hi, uint32_t flags)
{
    if (flags & (kFlagBad | kFlagNonFinite))
        return false;
    if (!(flags & kFlagNeg))
        return m + pair_at(p, m) <= kCountHi;
    return m + lo >= kCountLo + 1 && m + hi <= kCountHi - 1;
}

EXSEQ_HD bool is_nonfinite(double x) { return (dbits(x) & 0x7FF0000000000000ULL) == 0x7FF0000000000000ULL; }

}  // namespace exseq
