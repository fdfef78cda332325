"""Pins of the oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load(path)``)
and raises ``AssertionError`` when the oracle disagrees with the pinned fact.
``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutations.py`` runs them on copies of the oracle with a
planted mistake and requires at least one pin to fail for every mistake.

Sources of truth (none of them is the oracle itself):

* the exact integer model of IEEE-754 addition in ``ieee_model.py``
  (brute force over every short sequence of tie-building alphabets);
* closed forms of sequential sums that the pages describe (Research-1433
  "Forming the CPU's sequential double sums on a GPU, bit for bit",
  Findings 2 and 3: a run that stays in one binade is an integer sum of
  rounded increments; a half-way increment rounds to the even count);
* the binade identity fl(S + t) = (m + round(t / u)) * u (same Findings 2)
  evaluated with Python integers;
* an independent sequential evaluation by CPython's float add over whole
  workloads (``functools.reduce``, never numpy's pairwise sum);
* for the SSIM term: the textbook SSIM index (Wang et al., 2004) computed from
  the window's pixels with exact rational statistics, scaled by the window
  count with the stabilisers divided by w^2 (the algebraic identity of the
  term on Research-1424 "integer_ssim_cuda and the CPU's frame sum",
  Findings 1), and the special case ref == dis;
* for the window moments: a summed-area table (a second integer method);
* for the weight sum: the product of the two line sums (ADR-1443
  "integer_ssim_sycl computes the CPU's fp64 term ...", Decision, the weight
  is not a plane);
* for the interleaved sums and their float means (ADR-1464 "float_ssim_cuda
  adds its frame sums in the CPU's raster order, on the host", Decision):
  the integer IEEE model per field, the exact quotient rounded to binary64
  and then to binary32 with Python integers, and float roundings that are
  IEEE facts (midpoints, 1/3, division by zero).
"""

from __future__ import annotations

import functools
import math
import operator
import struct
from fractions import Fraction

import numpy as np

import oracle
import seeded_inputs as si
from tests import ieee_model as ieee


def bits(x: float) -> int:
    return struct.unpack("<Q", struct.pack("<d", x))[0]


def same(a: float, b: float) -> bool:
    """Bit equality (NaNs compare by NaN-ness only)."""
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return bits(a) == bits(b)


# --------------------------------------------------------------------------
# The loop
# --------------------------------------------------------------------------

def _all_sequences(alphabet, max_len):
    """Every sequence over a 2-symbol alphabet of length 0..max_len, as a flat
    array plus (offsets, lengths), and the tree of prefixes for the exact
    model (node i's parent sequence is its prefix)."""
    seqs_flat, offs, lens = [], [], []
    pos = 0
    for L in range(max_len + 1):
        if L == 0:
            offs.append(pos)
            lens.append(0)
            continue
        codes = np.arange(2 ** L, dtype=np.int64)
        bitsm = (codes[:, None] >> np.arange(L - 1, -1, -1)) & 1
        vals = np.where(bitsm == 0, alphabet[0], alphabet[1]).astype(np.float64)
        seqs_flat.append(vals.ravel())
        offs.extend(pos + L * np.arange(2 ** L))
        lens.extend([L] * (2 ** L))
        pos += L * 2 ** L
    flat = np.concatenate(seqs_flat) if seqs_flat else np.zeros(0)
    return flat, np.array(offs, dtype=np.int64), np.array(lens, dtype=np.int64)


def _exact_tree(alphabet, max_len, init):
    """Exact sequential sums of every sequence, in the same enumeration order
    as ``_all_sequences`` (level by level, codes in increasing order)."""
    out = [init]
    level = [init]
    for L in range(1, max_len + 1):
        nxt = []
        for s in level:                       # code c at level L-1 -> 2c, 2c+1
            nxt.append(ieee.add(s, alphabet[0]))
            nxt.append(ieee.add(s, alphabet[1]))
        out.extend(nxt)
        level = nxt
    return out


TIE_ALPHABETS = (
    ((2.0 ** -53, 1.0), 0.0),
    ((2.0 ** -53, 1.0), 1.0),
    ((3 * 2.0 ** -54, 2.0 ** -53), 1.0),
    ((3 * 2.0 ** -54, 2.0 ** -53), 0.0),
    ((1.0, -3 * 2.0 ** -54), 1.0),
    ((2.0 ** -53, -(2.0 ** -53)), 1.0 + 2.0 ** -52),
)


def pin_exhaustive_short(lib, max_len=16, alphabets=TIE_ALPHABETS):
    """Every sequence of length <= max_len over tie-building alphabets equals
    the exact integer model of in-order IEEE adds (brute force)."""
    for alphabet, init in alphabets:
        flat, offs, lens = _all_sequences(alphabet, max_len)
        got = np.zeros(len(offs))
        inits = np.full(len(offs), init)
        dp = oracle._dptr
        lib.oracle_seq_sum_f64_many(dp(flat), oracle._i64ptr(offs),
                                    oracle._i64ptr(lens), len(offs), dp(inits),
                                    dp(got))
        want = _exact_tree(alphabet, max_len, init)
        assert len(want) == len(got)
        for i, (w, g) in enumerate(zip(want, got)):
            if not same(w, float(g)):
                raise AssertionError(
                    "alphabet %r init %r sequence #%d: oracle %r, exact %r"
                    % (alphabet, init, i, float(g), w))


def pin_closed_forms(lib):
    """Sums whose value is fixed in closed form."""
    f = lambda xs, init=0.0: oracle.seq_sum(np.array(xs, dtype=np.float64), init, lib=lib)
    u = 2.0 ** -52
    # A tie from an even count stays (ties to even): 1 + u/2 -> 1, repeatedly.
    for k in (1, 2, 7, 100):
        assert same(f([1.0] + [2.0 ** -53] * k), 1.0), k
    # From an odd count a tie rounds up to the even neighbour.
    assert same(f([1.0 + u, 2.0 ** -53]), 1.0 + 2 * u)
    # 1 + 1.5u: half way between counts 2^52+1 and 2^52+2 -> the even one.
    assert same(f([1.0, 3 * 2.0 ** -53]), 1.0 + 2 * u)
    # 2^53 + 1 is half way between 2^53 and 2^53 + 2 -> 2^53.
    assert same(f([2.0 ** 53, 1.0]), 2.0 ** 53)
    assert same(f([2.0 ** 53, 1.0, 1.0]), 2.0 ** 53)
    assert same(f([2.0 ** 53, 3.0]), 2.0 ** 53 + 4)
    # Order matters: the small terms first add up exactly.
    assert same(f([1.0, 1.0, 2.0 ** 53]), 2.0 ** 53 + 2)
    # Empty sum returns the start; a -0 term from +0 gives +0 (the start).
    assert same(f([]), 0.0)
    assert same(f([], 2.5), 2.5)
    assert same(f([-0.0]), 0.0)
    assert same(f([-0.0], -0.0), -0.0)
    assert same(f([1.0, -1.0]), 0.0)
    # Integer-valued terms with partial sums below 2^53 add exactly.
    rng = np.random.default_rng(7)
    ints = rng.integers(-2 ** 40, 2 ** 40, 5000)
    assert same(f(ints.astype(np.float64)), float(int(ints.sum())))
    # The start value takes part: init is the first operand.
    assert same(f([2.0 ** -53], 1.0), 1.0)
    assert same(f([1.0], 2.0 ** 53), 2.0 ** 53)
    # Overflow and non-finite propagation.
    assert f([1.7e308, 1.7e308]) == math.inf
    assert math.isnan(f([math.inf, -math.inf]))
    assert math.isnan(f([1.0, math.nan, 2.0]))
    assert f([1.0, math.inf, 5.0]) == math.inf
    # Multiples of u = 2^-40 inside one binade [2^12, 2^13): exact.
    m = rng.integers(0, 2 ** 20, 3000)
    xs = [4096.0] + list((m.astype(np.float64) * 2.0 ** -40))
    want = Fraction(4096) + sum(Fraction(int(v), 2 ** 40) for v in m)
    assert want < 8192
    assert same(f(xs), float(want))


def pin_binade_identity(lib, count=20000, seed=3):
    """fl(S + t) = (m + r) * u with u = 2^(e-52), m = S/u, r = t/u rounded to
    the nearest integer and a half-way case rounded so that m + r is even,
    whenever the count stays inside the binade (Research-1433 Findings 2-3).
    Checked on random S, t including constructed ties and negative t."""
    rng = np.random.default_rng(seed)
    pairs = []
    for i in range(count):
        e = int(rng.integers(-30, 60))
        m = int(rng.integers(2 ** 52, 2 ** 53))
        S = math.ldexp(m, e - 52)
        kind = i % 4
        if kind == 0:            # random term below S
            t = math.ldexp(float(rng.random()), e - int(rng.integers(1, 40)))
        elif kind == 1:          # exact tie: (k + 1/2) u
            k = int(rng.integers(0, 2 ** int(rng.integers(1, 40))))
            t = math.ldexp(2 * k + 1, e - 53)
        elif kind == 2:          # tie between a coarser pair of its own bits
            k = int(rng.integers(0, 2 ** 30))
            t = math.ldexp(2 * k + 1, e - 53)
        else:                    # negative term
            t = -math.ldexp(float(rng.random()), e - int(rng.integers(1, 40)))
        if rng.random() < 0.5 and kind in (1, 2):
            t = -t
        pairs.append((S, t, m, e))
    xs = np.array([[p[0], p[1]] for p in pairs], dtype=np.float64).ravel()
    offs = np.arange(0, 2 * len(pairs), 2, dtype=np.int64)
    lens = np.full(len(pairs), 2, dtype=np.int64)
    got = np.zeros(len(pairs))
    inits = np.zeros(len(pairs))
    dp = oracle._dptr
    lib.oracle_seq_sum_f64_many(dp(xs), oracle._i64ptr(offs), oracle._i64ptr(lens),
                                len(pairs), dp(inits), dp(got))
    checked = 0
    for (S, t, m, e), g in zip(pairs, got):
        q = Fraction(t) / Fraction(2) ** (e - 52)       # t / u exactly
        fl = math.floor(q)
        frac = q - fl
        if frac > Fraction(1, 2):
            r = fl + 1
        elif frac < Fraction(1, 2):
            r = fl
        else:
            r = fl if (m + fl) % 2 == 0 else fl + 1
        c = m + r
        if not (2 ** 52 < c < 2 ** 53):
            continue                # left the binade: the identity does not apply
        want = math.ldexp(c, e - 52)
        checked += 1
        if not same(float(g), want):
            raise AssertionError("S=%r t=%r: oracle %r, binade identity %r"
                                 % (S, t, float(g), want))
    assert checked > count // 2


def pin_cpython_reduce(lib, sizes=(4096, 200_000)):
    """The oracle equals CPython's own in-order float adds on whole workloads
    (an independent sequential evaluation; numpy.sum is pairwise and is
    never used for this)."""
    cases = [si.uniform(4096, 0), si.tie_heavy(sizes[1], 1),
             si.signed_terms(sizes[1], 2), si.half_normal(sizes[1], 3)]
    for x in cases:
        want = functools.reduce(operator.add, x.tolist(), 0.0)
        got = oracle.seq_sum(x, 0.0, lib=lib)
        assert same(got, want), (got, want)
    x = si.tie_suite(5000, 4)
    assert same(oracle.seq_sum(x, 1.0, lib=lib),
                functools.reduce(operator.add, x.tolist(), 1.0))


def pin_seq_sum_many(lib):
    arrays = [si.uniform(n, n) for n in (0, 1, 5, 1000)]
    inits = [0.0, 1.5, -2.0, 3.0]
    out = oracle.seq_sum_many(arrays, inits, lib=lib)
    for a, i, o in zip(arrays, inits, out):
        assert same(float(o), functools.reduce(operator.add, a.tolist(), i))


# --------------------------------------------------------------------------
# Window moments, the term, the frame sum
# --------------------------------------------------------------------------

def sat_moments(ref, dis, radius):
    """Edge-truncated box sums by summed-area tables (int64)."""
    r = ref.astype(np.int64)
    d = dis.astype(np.int64)
    h, w = r.shape

    def box(p):
        s = np.zeros((h + 1, w + 1), dtype=np.int64)
        s[1:, 1:] = p.cumsum(0).cumsum(1)
        i = np.arange(h)
        j = np.arange(w)
        i0 = np.clip(i - radius, 0, h)[:, None]
        i1 = np.clip(i + radius + 1, 0, h)[:, None]
        j0 = np.clip(j - radius, 0, w)[None, :]
        j1 = np.clip(j + radius + 1, 0, w)[None, :]
        return s[i1, j1] - s[i0, j1] - s[i1, j0] + s[i0, j0]

    one = np.ones_like(r)
    return box(r), box(d), box(r * r), box(d * d), box(r * d), box(one)


def pin_box_moments(lib, shapes=((1, 1), (2, 2), (3, 4), (7, 5), (9, 9), (17, 33),
                                 (40, 23)), radius=3):
    for k, (h, w) in enumerate(shapes):
        ref, dis = si.frame_pair(h, w, 100 + k)
        got = oracle.box_moments(ref, dis, radius, lib=lib)
        want = sat_moments(ref, dis, radius)
        for name, g, wv in zip(("x", "y", "x2", "y2", "xy", "w"), got, want):
            assert np.array_equal(g, wv), (h, w, name)


def _line_sum(n, radius):
    return sum(min(j + radius, n - 1) - max(j - radius, 0) + 1 for j in range(n))


def textbook_ssim_term(win_ref, win_dis, c1, c2):
    """w * SSIM(ref, dis) with the textbook formula (Wang et al. 2004) on the
    window's pixels in exact rationals, stabilisers c/w^2:
    (2 mu_x mu_y + C1)(2 cov + C2) / ((mu_x^2 + mu_y^2 + C1)(var_x + var_y + C2))."""
    a = [Fraction(int(v)) for v in np.asarray(win_ref).ravel()]
    b = [Fraction(int(v)) for v in np.asarray(win_dis).ravel()]
    w = len(a)
    mx = sum(a) / w
    my = sum(b) / w
    vx = sum((p - mx) ** 2 for p in a) / w
    vy = sum((q - my) ** 2 for q in b) / w
    cov = sum((p - mx) * (q - my) for p, q in zip(a, b)) / w
    C1 = Fraction(c1) / (w * w)
    C2 = Fraction(c2) / (w * w)
    ssim = ((2 * mx * my + C1) * (2 * cov + C2)) / ((mx * mx + my * my + C1) * (vx + vy + C2))
    return w * ssim


def pin_term_textbook(lib, count=400, seed=11, rel_tol=64 * 2.0 ** -52):
    """The fp64 term agrees with the exact textbook value to a few dozen ulps
    (the expression takes ~20 roundings), on windows of 1..49 pixels including
    flat, anti-correlated and identical ones."""
    rng = np.random.default_rng(seed)
    c1, c2 = oracle.SSIM_C1, oracle.SSIM_C2
    for i in range(count):
        w = int(rng.integers(1, 50))
        kind = i % 5
        a = rng.integers(0, 256, w)
        if kind == 0:
            b = np.clip(a + rng.normal(0, 8, w), 0, 255).astype(np.int64)
        elif kind == 1:
            b = 255 - a                         # anti-correlated
        elif kind == 2:
            b = rng.integers(0, 256, w)
        elif kind == 3:
            a = np.full(w, int(rng.integers(0, 256)))
            b = rng.integers(0, 256, w)         # flat reference
        else:
            b = rng.integers(0, 256, w) // 2 + a // 3
        x, y = int(a.sum()), int(b.sum())
        x2, y2, xy = int((a * a).sum()), int((b * b).sum()), int((a * b).sum())
        got = oracle.ssim_term(x, y, x2, y2, xy, w, c1, c2, lib=lib)
        want = textbook_ssim_term(a, b, c1, c2)
        err = abs(Fraction(got) - want)
        assert err <= abs(want) * Fraction(rel_tol) + Fraction(1, 10 ** 300), \
            (i, w, kind, got, float(want))


def pin_term_per_operation(lib, count=20000, seed=13):
    """No contraction and C's left-to-right order: every operation of the
    term rounds once.  CPython evaluates float expressions one IEEE operation
    at a time (it never fuses a multiply into an add), so the same expression
    in the same order must give the same bits.  This pins how the oracle is
    compiled and evaluated; the formula itself is pinned by
    ``pin_term_textbook``."""
    rng = np.random.default_rng(seed)
    c1, c2 = oracle.SSIM_C1, oracle.SSIM_C2
    for i in range(count):
        w = int(rng.integers(1, 50))
        if i % 2:
            # 8-bit windows: every product of moments is exact here
            a = rng.integers(0, 256, w)
            b = np.clip(a + rng.normal(0, 3 + i % 40, w), 0, 255).astype(np.int64)
            x, y = int(a.sum()), int(b.sum())
            x2, y2, xy = int((a * a).sum()), int((b * b).sum()), int((a * b).sum())
        else:
            # wide int64 moments: products round, so contraction would show
            x, y = (int(v) for v in rng.integers(0, 2 ** 31, 2))
            x2, y2, xy = (int(v) for v in rng.integers(0, 2 ** 45, 3))
        wd = float(w)
        mx2 = float(x) * float(x)
        my2 = float(y) * float(y)
        mxy = float(x) * float(y)
        num = wd * (2.0 * mxy + c1) * (c2 + 2.0 * (float(xy) * wd - mxy))
        den = (mx2 + my2 + c1) * (float(x2) * wd - mx2 + float(y2) * wd - my2 + c2)
        want = num / den
        got = oracle.ssim_term(x, y, x2, y2, xy, w, c1, c2, lib=lib)
        assert same(got, want), (i, got, want)


def pin_term_identical_windows(lib, count=300, seed=12):
    """ref == dis: SSIM is 1, so the term is w up to a few roundings."""
    rng = np.random.default_rng(seed)
    for i in range(count):
        w = int(rng.integers(1, 50))
        a = rng.integers(0, 256, w)
        x, x2 = int(a.sum()), int((a * a).sum())
        got = oracle.ssim_term(x, x, x2, x2, x2, w, oracle.SSIM_C1,
                               oracle.SSIM_C2, lib=lib)
        assert abs(got - w) <= 8 * w * 2.0 ** -52, (w, got)


def pin_frame_sum(lib, shapes=((1, 1), (2, 2), (3, 4), (5, 7), (9, 9), (16, 16),
                               (33, 17), (65, 63)), radius=3):
    """The frame sum is the in-order loop over terms formed from pinned
    moments, in raster (row-major) order, and the weight sum is the product
    of the two line sums."""
    c1, c2 = oracle.SSIM_C1, oracle.SSIM_C2
    for k, (h, w) in enumerate(shapes):
        ref, dis = si.frame_pair(h, w, 200 + k)
        s, wsum, terms = oracle.ssim_frame_sum(ref, dis, radius, c1, c2,
                                               want_terms=True, lib=lib)
        mom = sat_moments(ref, dis, radius)
        t2 = np.array([oracle.ssim_term(*(int(m[i, j]) for m in mom), c1, c2, lib=lib)
                       for i in range(h) for j in range(w)])
        assert np.array_equal(terms.ravel().view(np.uint64), t2.view(np.uint64)), (h, w)
        want = functools.reduce(operator.add, t2.tolist(), 0.0)
        assert same(s, want), (h, w, s, want)
        assert wsum == _line_sum(h, radius) * _line_sum(w, radius), (h, w)
        # textbook check on a few pixels of the frame itself
        for (i, j) in ((0, 0), (h - 1, w - 1), (h // 2, w // 2)):
            wr = ref[max(0, i - radius):i + radius + 1, max(0, j - radius):j + radius + 1]
            wd = dis[max(0, i - radius):i + radius + 1, max(0, j - radius):j + radius + 1]
            want_t = textbook_ssim_term(wr, wd, c1, c2)
            assert abs(Fraction(terms[i, j]) - want_t) <= abs(want_t) * Fraction(64 * 2.0 ** -52)


def f32_round(q):
    """A rational rounded to the nearest binary32, ties to even (Python
    integers only; subnormals included, overflow to infinity)."""
    q = Fraction(q)
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    m, r = divmod(a, ulp)
    m = int(m)
    if r > ulp / 2 or (r == ulp / 2 and m % 2 == 1):
        m += 1
    v = m * ulp
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)


def pin_interleaved_brute_force(lib):
    """k loops over records of k doubles (one accumulator per field, each in
    index order) and their float means, against the integer IEEE model per
    field and the exact quotient rounded twice (to binary64, then to
    binary32) -- an evaluation that shares nothing with the C loop.
    Tie-heavy fields make any other order of adds, or a swap of fields, give
    other bits."""
    cases = [(1, 1), (3, 2), (17, 4), (64, 3), (200, 8), (1000, 4)]
    for windows, k in cases:
        x = np.empty(windows * k)
        for j in range(k):
            if j % 2 == 0:
                x[j::k] = si.tie_suite(windows, 11 * j + windows)
            else:
                x[j::k] = si.uniform(windows, 7 * j + windows) * (j + 1)
        x[0] = 1.0
        inits = np.array([0.0, 1.0, -0.5, 2.0, 0.0, 1.0, 0.25, 3.0][:k])
        sums, means = oracle.seq_sum_interleaved(x, k, inits, lib=lib)
        for j in range(k):
            want = ieee.seq_sum(list(x[j::k]), float(inits[j]))
            assert same(sums[j], want), (windows, k, j)
            q = ieee.round_fraction(Fraction(want) / windows)
            assert struct.pack("<f", float(means[j])) == struct.pack("<f", f32_round(q)), \
                (windows, k, j)


def pin_interleaved_mean_textbook(lib):
    """Means whose float is an IEEE fact: 1 + 2^-24 is the midpoint of 1 and
    1 + 2^-23 and rounds to the even 1; 1 + 3 * 2^-24 rounds up to the even
    1 + 2^-22; 1/3 is 0x3EAAAAAB; x / 0 is NaN for x = 0 and inf for x > 0."""
    _, means = oracle.seq_sum_interleaved([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, -1.0], 3, lib=lib)
    assert list(means) == [1.0, 1 + 2.0 ** -22, -1.0]
    sums, means = oracle.seq_sum_interleaved([0.5, 0.25, 0.25], 1, lib=lib)
    assert sums[0] == 1.0
    assert struct.pack(">f", float(means[0])).hex() == "3eaaaaab"
    _, means = oracle.seq_sum_interleaved(np.zeros(0), 2, [0.0, 1.0], lib=lib)
    assert math.isnan(float(means[0])) and float(means[1]) == math.inf


LOOP_PINS = (pin_closed_forms, pin_binade_identity, pin_cpython_reduce,
             pin_seq_sum_many, pin_exhaustive_short)
TERM_PINS = (pin_box_moments, pin_term_textbook, pin_term_identical_windows,
             pin_term_per_operation, pin_frame_sum)
INTERLEAVE_PINS = (pin_interleaved_brute_force, pin_interleaved_mean_textbook)
