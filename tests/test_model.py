"""The method's rules, walked by the host model, against the oracle (CPU).

Research-1433 "Forming the CPU's sequential double sums on a GPU, bit for
bit", Findings "Tests": the method run chunk by chunk on the host and
compared with the loop for several input kinds and plans, and mutations of
the rules (tie always up, no binade check, no upper bound check, parity
ignored when composing) that must each make it fail.  Findings 5: a plan
cannot change a result, only cost term-by-term chunks."""

import math
import struct

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import bit_exact_sequential_amd as ex
from tests import suites


def bits(v):
    return struct.unpack("<Q", struct.pack("<d", v))[0]


def same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return bits(a) == bits(b)


PLANS = [ex.PLAN_AUTO, ex.PLAN_ALL_FALLBACK, ex.PLAN_PLUS_ONE, ex.PLAN_MINUS_ONE, ex.PLAN_ALL_ZERO,
         ex.plan_fixed(1023)]
CHUNKS = [1, 2, 4, 1024]


@pytest.mark.parametrize("case", suites.edge_suite(), ids=lambda c: c[0])
def test_edge_cases(case):
    name, x, init = case
    want = oracle.seq_sum(x, init)
    for plan in PLANS:
        for C in CHUNKS:
            got, _ = ex.model_seq_sum(x, init, C, plan)
            assert same(got, want), (name, plan, C, got, want)


@pytest.mark.parametrize("case", suites.workload_suite(small=True), ids=lambda c: c[0])
def test_workloads_all_plans(case):
    name, x, init = case
    want = oracle.seq_sum(x, init)
    for plan in PLANS:
        for C in (4, 1024):
            got, st = ex.model_seq_sum(x, init, C, plan)
            assert same(got, want), (name, plan, C)


def test_auto_plan_is_mostly_fast():
    """With the automatic plan almost every chunk of the tie-heavy frame-size
    workload is applied from its increments (Research-1433 Findings 4: the
    first chunk with a non-zero term and about one per binade crossed)."""
    x = si.tie_heavy(si.FRAME_N, 0)
    got, st = ex.model_seq_sum(x, 0.0, 1024, ex.PLAN_AUTO)
    assert same(got, oracle.seq_sum(x))
    assert st["chunks"] == 8100
    assert st["fallback_chunks"] <= 40, st
    assert st["fast_chunks"] >= 8060, st


def test_exhaustive_short_at_small_chunks():
    """Every length-10 sequence over tie-building alphabets, with chunks of 1,
    2 and 4 terms so that tiny inputs reach the fast path."""
    for x, init in suites.exhaustive_short(10):
        want = oracle.seq_sum(x, init)
        for C in (1, 2, 4):
            got, _ = ex.model_seq_sum(x, init, C, ex.plan_fixed(1023))
            assert same(got, want), (x, init, C)
            got, _ = ex.model_seq_sum(x, init, C, ex.PLAN_AUTO)
            assert same(got, want), (x, init, C)


def test_resume_with_init():
    """The loop's whole state is S: summing a suffix from the exact prefix sum
    gives the same bits as the whole sum."""
    x = si.signed_terms(50_000, 9)
    whole = oracle.seq_sum(x)
    for k in (0, 1, 1023, 1024, 30_001, 50_000):
        head = oracle.seq_sum(x[:k])
        got, _ = ex.model_seq_sum(x[k:], head, 1024, ex.PLAN_AUTO)
        assert same(got, whole), k


MUTATIONS = {"tie_up": ex.MUT_TIE_UP, "no_binade_check": ex.MUT_NO_BINADE_CHECK,
             "no_upper_check": ex.MUT_NO_UPPER_CHECK, "ignore_parity": ex.MUT_IGNORE_PARITY}


@pytest.mark.parametrize("mut", sorted(MUTATIONS))
def test_mutations_are_caught(mut):
    cases = [(si.tie_heavy(100_000, 1), 0.0), (si.uniform(4096, 0), 0.0),
             (si.tie_suite(20_000, 3), 1.0), (si.signed_terms(100_000, 2), 0.0)]
    failures = 0
    for x, init in cases:
        want = oracle.seq_sum(x, init)
        for plan in (ex.PLAN_AUTO, ex.PLAN_PLUS_ONE, ex.plan_fixed(1023)):
            for C in (4, 1024):
                got, _ = ex.model_seq_sum(x, init, C, plan, MUTATIONS[mut])
                failures += not same(got, want)
    assert failures > 0, "mutation %s was not caught" % mut


def test_single_term_rule_against_the_add():
    """The one-term rule against the fp add on many samples (Research-1433
    Findings 1 "Tests"): a one-term run applied from S equals fl(S + t)
    wherever the model claims it applies."""
    rng = np.random.default_rng(21)
    S = np.ldexp(rng.integers(2 ** 52, 2 ** 53, 200_000).astype(np.float64),
                 rng.integers(-80, 80, 200_000) - 52)
    t = S * np.ldexp(rng.random(200_000), -rng.integers(0, 60, 200_000))
    t[::3] = np.ldexp(2 * rng.integers(0, 2 ** 20, t[::3].size) + 1.0,
                      np.frexp(S[::3])[1] - 54)       # exact half-unit ties
    t[1::5] *= -1
    for s0, tt in zip(S[:20000], t[:20000]):
        want = s0 + tt
        got, _ = ex.model_seq_sum(np.array([tt]), float(s0), 1, ex.PLAN_AUTO)
        assert same(got, want), (s0, tt)
