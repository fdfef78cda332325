"""exact_seq_sum_f64_noalloc (the entry point that takes no workspace and
allocates nothing) against exact_seq_sum_f64 with a caller workspace, bit for
bit, on two calls in a row, the second with a smaller input, and against the
oracle."""

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import bit_exact_sequential_amd as ex
from tests.gpu_util import same, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("flags", [0, ex.PASS_PATH])
def test_noalloc_matches_workspace_entry(flags):
    torch = torch_cuda()
    assert ex.lib().exact_seq_sum_f64_noalloc_max_terms() >= si.FRAME_N
    # two calls in a row on the same static array, the second smaller
    cases = (("tie_heavy 3840x2160", si.tie_heavy(si.FRAME_N, 21), 0.0),
             ("signed 300001", si.signed_terms(300_001, 22), 2.5))
    for name, x, init in cases:
        say("noalloc", name, flags)
        xd = to_dev(torch, x)
        ref = ex.exact_seq_sum(xd, init, flags=flags)
        got, st = ex.exact_seq_sum_noalloc(xd, init, flags=flags, stats=True)
        torch.cuda.synchronize()
        r, g = float(ref.cpu()[0]), float(got.cpu()[0])
        assert same(g, r), (name, g, r)
        assert same(g, oracle.seq_sum(x, init)), name
        assert st["fast_chunks"] + st["fallback_chunks"] == st["chunks"], st


def test_noalloc_small_and_empty():
    torch = torch_cuda()
    for n in (0, 1, 1023, 4097):
        x = si.tie_heavy(n, 23) if n else np.zeros(0)
        xd = to_dev(torch, x)
        got = float(ex.exact_seq_sum_noalloc(xd, 1.25).cpu()[0])
        assert same(got, float(ex.exact_seq_sum(xd, 1.25).cpu()[0])), n
        assert same(got, oracle.seq_sum(x, 1.25)), n
