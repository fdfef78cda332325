"""GPU parity of negative running sums (the fast path mirrored by the plan's
sign bit, crossings of negative binades included): every sum of -x equals the
oracle's bits, and, since round to nearest even is symmetric in sign, the
path treats -x exactly as it treats x -- the same chunks go term by term."""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import bit_exact_sequential_amd as ex
from tests.gpu_util import same, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    say("start", request.node.nodeid)
    yield


def run(torch, x, init=0.0, flags=0):
    out, st = ex.exact_seq_sum(to_dev(torch, x), init, flags=flags, stats=True)
    return float(out.cpu()[0]), st


CASES = [
    ("tie_heavy_600k", lambda: si.tie_heavy(600_000, 3), 0.0),
    ("tie_heavy_init", lambda: si.tie_heavy(300_001, 4), 5.0),
    ("signed_1920x1080", lambda: si.signed_terms(si.HALF_N, 5), 0.0),
    ("uniform_1m", lambda: si.uniform(1_000_000, 6), 0.0),
    ("tie_suite", lambda: si.tie_suite(200_000, 7), 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("flags", [0, ex.PLAN_PLUS_ONE, ex.PLAN_MINUS_ONE, ex.CHAIN_CUT])
def test_negated_workloads(case, flags):
    torch = torch_cuda()
    name, make, init = case
    x = make()
    got_p, st_p = run(torch, x, init, flags)
    got_n, st_n = run(torch, -x, -init, flags)
    assert same(got_p, oracle.seq_sum(x, init)), name
    assert same(got_n, oracle.seq_sum(-x, -init)), name
    assert same(got_n, -got_p), name
    for key in ("chunks", "fast_chunks", "fallback_chunks", "fallback_terms", "first_fallback"):
        assert st_n[key] == st_p[key], (name, key, st_n[key], st_p[key])


def test_negated_full_size_frame():
    torch = torch_cuda()
    x = si.tie_heavy(si.FRAME_N, 0)
    got_p, st_p = run(torch, x)
    got_n, st_n = run(torch, -x)
    assert same(got_n, oracle.seq_sum(-x))
    assert same(got_n, -got_p)
    say("fallback chunks", st_p["fallback_chunks"], st_n["fallback_chunks"])
    assert st_n["fallback_chunks"] == st_p["fallback_chunks"]


def test_sign_change_sequences():
    """Running sums that change sign and cross binades downwards as well."""
    torch = torch_cuda()
    n = 400_000
    base = si.tie_heavy(n, 9)
    for init in (-50_000.0, -1.0e5, 3.0e4):
        got, _ = run(torch, base, init)
        assert same(got, oracle.seq_sum(base, init)), init
    x = np.concatenate([base, -base[::-1]])
    got, _ = run(torch, x)
    assert same(got, oracle.seq_sum(x))
