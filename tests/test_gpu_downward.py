"""GPU parity of running sums whose magnitude falls through binades
(crossings downwards, located by the tiles like upward ones): every sum
equals the oracle's bits, the mirror image (-x from -init) is the exact
negation with the same statistics, and few chunks go term by term."""

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
    # terms in [-0.5, 0): the sum falls by about 0.225 per term
    ("falling_4m_from_2p20", lambda: -si.tie_heavy(4_000_000, 21), 2.0 ** 20 + 0.5),
    ("falling_1m_from_2p18", lambda: -si.tie_heavy(1_000_000, 22), 2.0 ** 18 + 3.0),
    # mostly negative with some positive terms
    ("signed_falling", lambda: -si.signed_terms(si.HALF_N, 23), 2.0 ** 21),
    ("uniform_falling", lambda: -si.uniform(2_000_000, 24), 2.0 ** 20 + 7.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("flags", [0, ex.PLAN_PLUS_ONE, ex.PLAN_MINUS_ONE, ex.CHAIN_CUT])
def test_falling_sums(case, flags):
    torch = torch_cuda()
    name, make, init = case
    x = make()
    got, st = run(torch, x, init, flags)
    assert same(got, oracle.seq_sum(x, init)), name
    got_m, st_m = run(torch, -x, -init, flags)
    assert same(got_m, -got), name
    for key in ("chunks", "fast_chunks", "fallback_chunks", "fallback_terms", "first_fallback"):
        assert st_m[key] == st[key], (name, key, st_m[key], st[key])
    say(name, "flags", flags, "fallback chunks", st["fallback_chunks"], "of", st["chunks"])
    if flags == 0:
        assert st["fallback_chunks"] <= 4, (name, st)


def test_falling_full_size_frame():
    torch = torch_cuda()
    x = -si.tie_heavy(si.FRAME_N, 25)
    got, st = run(torch, x, 2.0 ** 21)
    assert same(got, oracle.seq_sum(x, 2.0 ** 21))
    say("fallback chunks", st["fallback_chunks"])
    assert st["fallback_chunks"] <= 4, st


def test_up_then_down():
    """A sum that climbs through binades and falls back through them."""
    torch = torch_cuda()
    up = si.tie_heavy(1_500_000, 26)
    x = np.concatenate([up, -si.tie_heavy(1_500_000, 27)])
    got, st = run(torch, x)
    assert same(got, oracle.seq_sum(x))
    say("fallback chunks", st["fallback_chunks"], "of", st["chunks"])
