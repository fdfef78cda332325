"""Named input suites shared by the CPU model tests and the GPU parity tests.

Each entry is (name, terms ndarray, init).  Inputs come from
``seeded_inputs`` or are built here from plain constants; no expected value is
stored: every test compares against the oracle run on the same bytes.
"""

from __future__ import annotations

import math

import numpy as np

import seeded_inputs as si


def edge_suite():
    """Degenerate and boundary cases of the loop."""
    tiny = 5e-324
    out = [
        ("empty", np.zeros(0), 0.0),
        ("empty_init", np.zeros(0), -3.25),
        ("one_neg_zero", np.array([-0.0]), 0.0),
        ("neg_zero_from_neg_zero", np.array([-0.0, -0.0]), -0.0),
        ("one_term", np.array([0.1]), 0.0),
        ("zeros", np.zeros(5000), 0.0),
        ("leading_zeros", np.concatenate([np.zeros(3000), si.uniform(3000, 1)]), 0.0),
        ("subnormal_terms", np.full(3000, tiny) * np.arange(1, 3001), 0.0),
        ("subnormal_mix", np.concatenate([np.full(2000, 3 * tiny), si.uniform(2000, 2) * 1e-300]), 0.0),
        ("into_normal", np.full(4000, 2.0 ** -1030), 0.0),
        ("huge_terms", np.array([1e300, 1e300, -1e300, 5.0, 1e-300] * 500), 0.0),
        ("overflow", np.full(2100, 1.7e305), 0.0),
        ("negative_start", si.uniform(5000, 3), -1000.0),
        ("negative_sum", -si.uniform(5000, 4), 0.0),
        ("cancel_to_zero", np.tile(np.array([0.75, -0.75]), 2500), 0.0),
        ("crossing_zero", np.concatenate([-np.ones(1500), np.ones(3000) * 0.5]), 700.5),
        ("power_of_two_hits", np.full(8192, 0.25), 0.0),
        ("exact_2e53", np.full(3000, 1.0), 2.0 ** 53 - 1500),
        ("ties_from_one", si.tie_suite(5000, 5), 1.0),
        ("ties_from_odd", si.tie_suite(5000, 6), 1.0 + 2.0 ** -52),
        ("ties_negative", -si.tie_suite(5000, 7), -1.0),
        ("alternating_ties", np.tile(np.array([2.0 ** -53, -(2.0 ** -53), 3 * 2.0 ** -53]), 1500), 1.0),
        ("big_then_small", np.concatenate([np.array([2.0 ** 60]), si.uniform(5000, 8)]), 0.0),
        ("nan_middle", np.concatenate([si.uniform(3000, 9), [math.nan], si.uniform(1000, 10)]), 0.0),
        ("inf_middle", np.concatenate([si.uniform(3000, 11), [math.inf], si.uniform(1000, 12)]), 0.0),
        ("inf_minus_inf", np.concatenate([si.uniform(2000, 13), [math.inf, -math.inf], si.uniform(100, 1)]), 0.0),
        ("start_nan", si.uniform(2000, 14), math.nan),
        ("start_inf", si.uniform(2000, 15), -math.inf),
        ("max_finite", np.full(1500, 1e307), 1.7e308),
        # the running sum doubles every ~700 terms: crossings in the middle of
        # chunks, sometimes two in one chunk
        ("geometric_growth", 2.0 ** (np.arange(20000) / 700.0) * si.uniform(20000, 16), 0.0),
        # exactly 256 per chunk from 256: every crossing lands on a chunk's
        # last term
        ("crossing_on_last_term", np.full(16384, 0.25), 256.0),
        # a chunk whose sum is three times the running sum (two crossings)
        ("triple_jump", np.concatenate([np.full(4096, 0.5), np.full(1024, 6.0),
                                        np.full(4096, 0.5)]), 0.0),
    ]
    return out


def ragged_sizes():
    return (1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049,
            4095, 4096, 4097, 262143, 262145, 100003)


def workload_suite(small: bool):
    """The workloads at full size (small=False) or at sizes that still span
    many chunks and a ragged tail (small=True)."""
    n2 = 300_001 if small else si.FRAME_N
    n3 = 200_003 if small else si.HALF_N
    return [
        ("uniform_4096_s0", si.uniform(4096, 0), 0.0),
        ("uniform_4096_s1", si.uniform(4096, 1), 0.0),
        ("tie_heavy_s0", si.tie_heavy(n2, 0), 0.0),
        ("tie_heavy_s1", si.tie_heavy(n2, 1), 0.0),
        ("signed_s0", si.signed_terms(n3, 0), 0.0),
        ("signed_s1", si.signed_terms(n3, 1), 0.0),
        ("half_normal", si.half_normal(n3, 2), 0.0),
    ]


def exhaustive_short(max_len=10):
    """Every sequence of length max_len over tie-building 2-symbol alphabets
    (each prefix is itself a sequence of the shorter lengths)."""
    alphabets = (((2.0 ** -53, 1.0), 0.0), ((2.0 ** -53, 1.0), 1.0),
                 ((3 * 2.0 ** -54, 2.0 ** -53), 1.0), ((1.0, -3 * 2.0 ** -54), 1.0))
    out = []
    for (a, b), init in alphabets:
        for code in range(2 ** max_len):
            bits = [(code >> (max_len - 1 - i)) & 1 for i in range(max_len)]
            out.append((np.array([b if v else a for v in bits], dtype=np.float64), init))
    return out
