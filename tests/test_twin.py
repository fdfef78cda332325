"""The CPU twin of the single pass's composition against the oracle (CPU).

The twin (csrc/exseq_twin.cpp) replays pass_kernel's grouping of the terms
on the host -- four per lane, 64-lane waves with their shortcuts and scan
trees, the four waves joined, eight-chunk tiles, crossings located and
folded, the head, the finisher's segment scan and its walk -- with the
kernels' own rule helpers.  Research-1433 "Forming the CPU's sequential
double sums on a GPU, bit for bit", Findings "Tests": such a replay must
match the loop bit for bit over adversarial inputs, and each mutation of the
rules (a tie always rounding up, no binade check, no upper check, parity
ignored) must make it fail.  One more mutation reverts the rule that a
rising part's largest prefix is its total (run_top), whose absence let a
negative term early in a chunk hide a rise past the binade later in it."""

import math
import os
import struct
from concurrent.futures import ProcessPoolExecutor

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


MUTATIONS = {"tie_up": ex.MUT_TIE_UP, "no_binade_check": ex.MUT_NO_BINADE_CHECK,
             "no_upper_check": ex.MUT_NO_UPPER_CHECK, "ignore_parity": ex.MUT_IGNORE_PARITY,
             "no_run_top": ex.MUT_NO_RUN_TOP}


@pytest.mark.parametrize("case", suites.edge_suite(), ids=lambda c: c[0])
def test_edge_cases(case):
    name, x, init = case
    for plan in (ex.PLAN_AUTO, ex.PLAN_PLUS_ONE, ex.PLAN_MINUS_ONE, ex.PLAN_ALL_ZERO):
        got, _ = ex.twin_seq_sum(x, init, flags=plan)
        assert same(got, oracle.seq_sum(x, init)), (name, plan)


@pytest.mark.parametrize("case", suites.workload_suite(small=True), ids=lambda c: c[0])
def test_workloads_take_the_fast_paths(case):
    name, x, init = case
    got, st = ex.twin_seq_sum(x, init)
    assert same(got, oracle.seq_sum(x, init)), name
    assert st["fast_chunks"] + st["fallback_chunks"] == st["chunks"], st
    if st["chunks"] >= 64:
        assert st["fast_chunks"] >= 0.9 * st["chunks"], (name, st)


def test_full_size_frames():
    for x in (si.tie_heavy(si.FRAME_N, 31), -si.tie_heavy(si.FRAME_N, 32),
              si.signed_terms(si.HALF_N, 33)):
        got, st = ex.twin_seq_sum(x)
        assert same(got, oracle.seq_sum(x))
        assert st["fallback_chunks"] <= 8, st


def _campaign(args):
    """Adversarial sums from seed range [lo, hi): (mismatches, chunks, fast)."""
    lo, hi = args
    bad, chunks, fast = [], 0, 0
    for sd in range(lo, hi):
        fam = si.TWIN_FAMILIES[sd % len(si.TWIN_FAMILIES)]
        x, init = si.twin_case(sd, fam)
        plan = (ex.PLAN_AUTO, ex.PLAN_AUTO, ex.PLAN_AUTO, ex.PLAN_PLUS_ONE, ex.PLAN_MINUS_ONE)[sd % 5]
        got, st = ex.twin_seq_sum(x, init, flags=plan)
        if not same(got, oracle.seq_sum(x, init)):
            bad.append((sd, fam, plan))
        chunks += st["chunks"]
        fast += st["fast_chunks"]
    return bad, chunks, fast


def test_adversarial_campaign_million_chunks():
    """At least 10^6 chunks of the seven families under several plans, in
    worker processes: no mismatch, and most chunks through the fast paths."""
    n_sums, step = 120_000, 2_000
    with ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        res = list(pool.map(_campaign, [(a, a + step) for a in range(0, n_sums, step)]))
    bad = [b for r in res for b in r[0]]
    chunks = sum(r[1] for r in res)
    fast = sum(r[2] for r in res)
    assert not bad, bad[:10]
    assert chunks >= 1_000_000, chunks
    assert fast >= 0.5 * chunks, (fast, chunks)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_each_mutation_fails(name):
    m = MUTATIONS[name]
    caught = 0
    for sd in range(600):
        fam = si.TWIN_FAMILIES[sd % len(si.TWIN_FAMILIES)]
        x, init = si.twin_case(sd, fam)
        want = oracle.seq_sum(x, init)
        for plan in (ex.PLAN_AUTO, ex.PLAN_PLUS_ONE):
            got, _ = ex.twin_seq_sum(x, init, flags=plan, mutations=m)
            caught += not same(got, want)
    assert caught > 0, name


def test_run_top_guards_rise_after_negative_term():
    """The neg_rise family: without run_top the mutated twin goes wrong on it
    (where the chunk is one the head applies from the exact sum), with it the
    twin is exact."""
    wrong = 0
    for sd in range(200):
        x, init = si.twin_case(sd, "neg_rise")
        want = oracle.seq_sum(x, init)
        got, _ = ex.twin_seq_sum(x, init)
        assert same(got, want), sd
        got, _ = ex.twin_seq_sum(x, init, mutations=ex.MUT_NO_RUN_TOP)
        wrong += not same(got, want)
    assert wrong >= 10, wrong


# ---------------------------------------------------------------------------
# The tile chain's twin: tiles of four chunks, the chain look-back's grouping
# of the regular tiles (four per lane, per wave an integer sum, a falling sum,
# the pairs alone or the full runs, the reversed wave tree, the waves in
# reverse), the irregular tiles' chunks from the exact sum and the walk's
# resume.  The plan never decides the bits, so the tests also move every
# planned prefix by skew * 2^-30 of itself: far past the plan's margin, the
# composed runs' checks alone must keep the result exact.
# ---------------------------------------------------------------------------
CHAIN_PLANS = (ex.PLAN_AUTO, ex.PLAN_PLUS_ONE, ex.PLAN_MINUS_ONE, ex.PLAN_ALL_ZERO)
SKEWS = (0, -1, 1, -64, 64)


@pytest.mark.parametrize("case", suites.edge_suite(), ids=lambda c: c[0])
def test_chain_edge_cases(case):
    name, x, init = case
    want = oracle.seq_sum(x, init)
    for plan in CHAIN_PLANS:
        got, _, _ = ex.twin_chain_sum(x, init, flags=plan)
        assert same(got, want), (name, plan)


def test_chain_full_size_frames():
    for x in (si.tie_heavy(si.FRAME_N, 41), -si.tie_heavy(si.FRAME_N, 42),
              si.signed_terms(si.HALF_N, 43)):
        got, st, paths = ex.twin_chain_sum(x)
        assert same(got, oracle.seq_sum(x))
        assert st["fallback_chunks"] <= 16, st
        assert paths["stops"] == 0 and paths["applied"] >= 5, paths


def _chain_campaign(args):
    lo, hi = args
    bad, tot, chunks = [], {}, 0
    for sd in range(lo, hi):
        fam = si.TWIN_CHAIN_FAMILIES[sd % len(si.TWIN_CHAIN_FAMILIES)]
        x, init = si.twin_chain_case(sd, fam)
        want = oracle.seq_sum(x, init)
        for plan in CHAIN_PLANS:
            skew = SKEWS[(sd + plan) % len(SKEWS)]
            got, st, paths = ex.twin_chain_sum(x, init, flags=plan, skew=skew)
            if not same(got, want):
                bad.append((sd, fam, plan, skew))
            chunks += st["chunks"]
            for k, v in paths.items():
                tot[k] = tot.get(k, 0) + v
    return bad, tot, chunks


def test_chain_campaign():
    """Sums of whole tiles of every kind, under four plans and skewed plan
    prefixes: no mismatch, and every composition of the look-back used, some
    applied, some refused (the chain stops and the walk resumes)."""
    with ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        res = list(pool.map(_chain_campaign, [(a, a + 150) for a in range(0, 2400, 150)]))
    bad = [b for r in res for b in r[0]]
    tot = {}
    for r in res:
        for k, v in r[1].items():
            tot[k] = tot.get(k, 0) + v
    assert not bad, bad[:10]
    assert sum(r[2] for r in res) >= 1_000_000
    assert all(tot[k] > 0 for k in ("plain", "falling", "pairs", "runs", "applied", "stops")), tot


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_chain_each_mutation_fails(name):
    m = MUTATIONS[name]
    caught = 0
    for sd in range(40):
        x, init = si.twin_chain_case(sd, "chain_mix")
        want = oracle.seq_sum(x, init)
        for skew in (0, -1, 1):
            for plan in (ex.PLAN_AUTO, ex.PLAN_PLUS_ONE):
                got, _, _ = ex.twin_chain_sum(x, init, flags=plan, mutations=m, skew=skew)
                caught += not same(got, want)
    assert caught > 0, name


def test_chain_skewed_plan_stops_at_the_edge():
    """chain_wave_rise under a plan 2^-30 low: every tile but the first and
    the last is regular, the last tile's look-back composes a wave of full
    runs and a wave of pairs alone, the composed run passes the binade's top
    for the exact sum, so the chain stops and the walk gives the exact bits."""
    for sd in range(6):
        x, init = si.twin_chain_case(sd, "chain_wave_rise")
        got, st, paths = ex.twin_chain_sum(x, init, skew=-1)
        assert same(got, oracle.seq_sum(x, init)), sd
        assert paths["stops"] == 1 and paths["pairs"] >= 1 and paths["runs"] >= 1, paths
