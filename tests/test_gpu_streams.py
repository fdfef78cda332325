"""Calls on a stream other than the current one (a default-priority side
stream): every entry point gives the oracle's bits, the statistics are read
after the side stream's kernels, and many calls in a row with workspaces the
binding allocates (and the caching allocator reuses) keep their bits."""

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


def test_every_entry_point_on_a_side_stream():
    torch = torch_cuda()
    s = torch.cuda.Stream()
    x = si.tie_heavy(200_000, 3)
    xs = [si.signed_terms(50_000 + 1000 * k, 40 + k) for k in range(3)]
    rec = si.lcs_records(30_000, 5)
    ref, dis = si.frame_pair(61, 128, 9)
    want = oracle.seq_sum(x)
    want_b = oracle.seq_sum_many(xs)
    want_i = [oracle.seq_sum(rec[f::4].copy()) for f in range(4)]
    want_s, wsum, _ = oracle.ssim_frame_sum(ref, dis, 3)
    xd, xsd, recd = to_dev(torch, x), [to_dev(torch, a) for a in xs], to_dev(torch, rec)
    rd, dd = torch.from_numpy(ref).cuda(), torch.from_numpy(dis).cuda()
    torch.cuda.synchronize()
    for rep in range(20):
        o, st = ex.exact_seq_sum(xd, stream=s, stats=True)
        assert st["chunks"] == (x.size + 1023) // 1024
        ob = ex.exact_seq_sum_batch(xsd, stream=s)
        oi, _ = ex.exact_seq_sum_interleaved(recd, 4, stream=s)
        gs, gw, _ = ex.ssim_term_and_sum(rd, dd, 3, stream=s)
        s.synchronize()
        assert same(float(o.cpu()[0]), want), rep
        assert all(same(a, b) for a, b in zip(ob.cpu().tolist(), want_b)), rep
        assert all(same(a, b) for a, b in zip(oi.cpu().tolist(), want_i)), rep
        assert same(float(gs.cpu()[0]), want_s) and int(gw.cpu()[0]) == wsum, rep
