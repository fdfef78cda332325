"""The oracle against its pins (CPU only).  See tests/oracle_pins.py."""

import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from tests import ieee_model as ieee
from tests import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


def test_ieee_model_textbook_values():
    """The integer IEEE model itself, on additions whose results are
    textbook facts of binary64 round-to-nearest-even."""
    assert ieee.add(2.0 ** 53, 1.0) == 2.0 ** 53
    assert ieee.add(2.0 ** 53, 3.0) == 2.0 ** 53 + 4
    assert ieee.add(1.0, 2.0 ** -53) == 1.0
    assert ieee.add(1.0 + 2.0 ** -52, 2.0 ** -53) == 1.0 + 2.0 ** -51
    assert ieee.add(1.0, 2.0 ** -52) == 1.0 + 2.0 ** -52
    assert ieee.add(1e308, 1e308) == math.inf
    assert math.copysign(1, ieee.add(5e-324, -5e-324)) == 1
    assert math.copysign(1, ieee.add(-0.0, -0.0)) == -1
    assert ieee.add(5e-324, 5e-324) == 1e-323
    assert ieee.add(2.0 ** -1022, -(2.0 ** -1074)) == 2.0 ** -1022 - 2.0 ** -1074
    from fractions import Fraction
    assert ieee.round_fraction(Fraction(1, 3)) == 1 / 3
    assert ieee.round_fraction(Fraction(1) + Fraction(1, 2 ** 53)) == 1.0
    assert ieee.round_fraction(Fraction(3, 2 ** 1075)) == 2 * 5e-324


def test_closed_forms(lib):
    P.pin_closed_forms(lib)


def test_binade_identity(lib):
    P.pin_binade_identity(lib)


def test_cpython_reduce(lib):
    P.pin_cpython_reduce(lib)


def test_seq_sum_many(lib):
    P.pin_seq_sum_many(lib)


def test_exhaustive_short(lib):
    P.pin_exhaustive_short(lib)


def test_box_moments(lib):
    P.pin_box_moments(lib)


def test_term_textbook(lib):
    P.pin_term_textbook(lib)


def test_term_per_operation(lib):
    P.pin_term_per_operation(lib)


def test_term_identical_windows(lib):
    P.pin_term_identical_windows(lib)


def test_frame_sum(lib):
    P.pin_frame_sum(lib)


def test_page_values():
    g = json.load(open(GOLDEN))
    assert repr(0.01 * 0.01) == g["stabiliser_doubles"]["0.01*0.01"]
    assert repr(0.03 * 0.03) == g["stabiliser_doubles"]["0.03*0.03"]
    b = lambda x: hex(struct.unpack("<Q", struct.pack("<d", x))[0])
    assert b(oracle.SSIM_C1) == g["fused_workload_stabilisers"]["c1_bits"]
    assert b(oracle.SSIM_C2) == g["fused_workload_stabilisers"]["c2_bits"]
    v = float(g["float_rounding_of_a_printed_mean"]["value"])
    fb = hex(struct.unpack("<I", struct.pack("<f", v))[0])
    assert fb == g["float_rounding_of_a_printed_mean"]["float_bits"]
    fa = g["frame_arithmetic"]
    assert fa["width"] * fa["height"] == fa["terms"] == si.FRAME_N
    assert fa["terms"] * 8 == fa["bytes"]
    assert fa["terms"] == fa["chunks"] * fa["chunk_terms"]


def test_tie_rule_count(lib):
    """Research-1433 Findings 3: with terms d = 1 - q (multiples of 2^-53) and
    the sum in [1, 2), a term ties when its last bit is set.  Counted with the
    exact model: every tie leaves the sum's count even, as the oracle does."""
    x = si.tie_heavy(2000, 5)
    x = x[x < 2.0 ** -10]                 # keep the sum inside [1, 2)
    ties = 0
    s = 1.0
    for t in x.tolist():
        k = t / 2.0 ** -53
        assert k == int(k)
        if int(k) % 2 == 1:
            ties += 1
        s = ieee.add(s, t)
        assert 1.0 <= s < 2.0
        assert (int((s - 1.0) * 2.0 ** 52) % 2 == 0) or int(k) % 2 == 0
    assert P.same(oracle.seq_sum(x, 1.0, lib=lib), s)
    assert ties > 0


@pytest.mark.slow
def test_cpython_reduce_full_size(lib):
    """Full-size workloads: the oracle equals CPython's in-order adds."""
    import functools, operator
    for x in (si.tie_heavy(si.FRAME_N, 0), si.signed_terms(si.HALF_N, 0)):
        want = functools.reduce(operator.add, x.tolist(), 0.0)
        assert P.same(oracle.seq_sum(x, lib=lib), want)



def test_interleaved_brute_force(lib):
    P.pin_interleaved_brute_force(lib)


def test_interleaved_mean_textbook(lib):
    P.pin_interleaved_mean_textbook(lib)
