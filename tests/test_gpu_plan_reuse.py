"""GPU parity of the kept plan (EXSEQ_PLAN_REUSE): a call that takes its
tiles' binades from the plan the previous call left in the workspace returns
the oracle's bits (0 ULP) for every frame of a sequence, for a kept plan that
is wrong, for a workspace of garbage and for a change of shape; and the plan is
really used (a wrong one shows up as chunks added term by term)."""

import ctypes

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import bit_exact_sequential_amd as ex
from tests.gpu_util import same, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

REUSE = ex.PLAN_REUSE


@pytest.fixture(autouse=True)
def _name(request):
    say("start", request.node.nodeid)
    yield


def run(torch, xd, init, ws, flags=REUSE):
    out, st = ex.exact_seq_sum(xd, init, flags=flags, ws=ws, stats=True)
    return float(out.cpu()[0]), st


def new_ws(torch, n):
    return ex.workspace(ex.lib().exact_seq_sum_f64_workspace_size(n), torch.device("cuda"))


@pytest.mark.parametrize("n,init", [(600_000, 0.0), (1_000_003, 2.5), (40_960, -1.0)])
def test_video_sequence(n, init):
    """Frames of one distribution in sequence on one workspace: each exact,
    and no more chunks term by term than without the kept plan."""
    torch = torch_cuda()
    ws = new_ws(torch, n)
    for f in range(5):
        x = si.tie_heavy(n, 100 + f)
        xd = to_dev(torch, x)
        want = oracle.seq_sum(x, init)
        got, st = run(torch, xd, init, ws)
        assert same(got, want), (n, f, got, want)
        base, st0 = run(torch, xd, init, new_ws(torch, n), flags=0)
        assert same(base, want)
        say("frame", f, "fallback chunks reuse", st["fallback_chunks"], "plain", st0["fallback_chunks"])
        assert st["fallback_chunks"] <= st0["fallback_chunks"] + 2, (st, st0)


def test_wrong_plan_is_exact_and_used():
    """The kept plan of x, reused for 4x (every binade two too low), -x and
    2^-40 x: exact every time.  That the 4x call adds many more chunks term by
    term than the same call without the flag shows the plan was taken; the
    next call (whose kept plan is 4x's own) is back to normal."""
    torch = torch_cuda()
    n = 800_000
    x = si.tie_heavy(n, 7)
    ws = new_ws(torch, n)
    got, _ = run(torch, to_dev(torch, x), 0.0, ws)
    assert same(got, oracle.seq_sum(x))
    y = 4.0 * x
    yd = to_dev(torch, y)
    want = oracle.seq_sum(y)
    got, st = run(torch, yd, 0.0, ws)
    assert same(got, want)
    _, st0 = run(torch, yd, 0.0, new_ws(torch, n), flags=0)
    say("wrong plan: fallback chunks", st["fallback_chunks"], "without reuse", st0["fallback_chunks"])
    assert st["fallback_chunks"] > st0["fallback_chunks"] + 10
    got, st2 = run(torch, yd, 0.0, ws)
    assert same(got, want)
    assert st2["fallback_chunks"] <= st0["fallback_chunks"] + 2
    for z in (-x, x * 2.0 ** -40, x):
        got, _ = run(torch, to_dev(torch, z), 0.0, ws)
        assert same(got, oracle.seq_sum(z))


def test_signed_sequence():
    torch = torch_cuda()
    n = si.HALF_N
    ws = new_ws(torch, n)
    for f in range(3):
        x = si.signed_terms(n, 40 + f)
        got, _ = run(torch, to_dev(torch, x), 0.0, ws)
        assert same(got, oracle.seq_sum(x)), f


def test_shape_change_and_garbage_workspace():
    """A kept plan of another length or init is not taken; neither is random
    workspace content."""
    torch = torch_cuda()
    n1, n2 = 500_000, 500_000 + 4096
    ws = new_ws(torch, n2)
    rng = np.random.default_rng(3)
    ws.copy_(torch.from_numpy(rng.integers(0, 256, ws.numel(), dtype=np.uint8)).cuda())
    for n, init in ((n1, 0.0), (n2, 0.0), (n2, 1.0), (n1, 1.0), (n1, 1.0)):
        x = si.tie_heavy(n, n + int(init))
        got, _ = run(torch, to_dev(torch, x), init, ws)
        assert same(got, oracle.seq_sum(x, init)), (n, init)


def test_batch_sequence():
    torch = torch_cuda()
    sizes = [0, 1, 5000, 70_000, 300_001, 4096 * 9]
    inits = [0.0, 1.0, -2.0, 0.5, 0.0, 3.0]
    need = ex.lib().exact_seq_sum_f64_batch_workspace_size(
        (ctypes.c_size_t * len(sizes))(*sizes), len(sizes))
    ws = ex.workspace(need, torch.device("cuda"))
    for f in range(3):
        arrays = [si.tie_heavy(n, 1000 * f + n) for n in sizes]
        out = ex.exact_seq_sum_batch([to_dev(torch, a) for a in arrays], inits,
                                     flags=REUSE, ws=ws).cpu().tolist()
        for k, (a, i, o) in enumerate(zip(arrays, inits, out)):
            assert same(o, oracle.seq_sum(a, i)), (f, k)


def test_full_size_frames():
    """Three 3840x2160 tie-heavy frames in sequence, as a video would give."""
    torch = torch_cuda()
    ws = new_ws(torch, si.FRAME_N)
    for f in range(3):
        x = si.tie_heavy(si.FRAME_N, f)
        got, st = run(torch, to_dev(torch, x), 0.0, ws)
        want = oracle.seq_sum(x)
        say("frame", f, "fallback chunks", st["fallback_chunks"])
        assert same(got, want), f


@pytest.mark.parametrize("mode", [0, ex.SSIM_IN_TILES], ids=["producer", "in_tiles"])
def test_ssim_sequence(mode):
    """The SSIM sum of consecutive frame pairs with the kept plan."""
    torch = torch_cuda()
    h, w = 270, 480
    need = ex.lib().ssim_term_and_sum_workspace_size(w, h)
    ws = ex.workspace(need, torch.device("cuda"))
    for f in range(3):
        ref, dis = si.frame_pair(h, w, 500 + f)
        s, wsum, _ = oracle.ssim_frame_sum(ref, dis, 3)
        gs, gw, _ = ex.ssim_term_and_sum(torch.from_numpy(ref).cuda(), torch.from_numpy(dis).cuda(),
                                         3, flags=REUSE | mode, ws=ws)
        assert same(float(gs.cpu()[0]), s), f
        assert int(gw.cpu()[0]) == wsum


def test_batch_of_two_groups_keeps_both_plans():
    """A batch of more than 64 sums through the tile chain runs as groups of
    64 that share the workspace.  Each group keeps its plan at a place of its
    own, so both groups take it: the plan of x, reused for 4x (every binade
    two too low), is exact and adds many more chunks term by term in both
    groups than the same call without the flag; the next call (whose kept
    plans are 4x's own) is back to normal."""
    torch = torch_cuda()
    sizes = [150_000 + 1024 * (k % 7) for k in range(100)]
    xs = [si.tie_heavy(n, 700 + k) for k, n in enumerate(sizes)]
    need = ex.lib().exact_seq_sum_f64_batch_workspace_size(
        (ctypes.c_size_t * len(sizes))(*sizes), len(sizes))
    ws = ex.workspace(need, torch.device("cuda"))
    fl = REUSE | ex.CHAIN_PATH
    out = ex.exact_seq_sum_batch([to_dev(torch, a) for a in xs], flags=fl, ws=ws).cpu().tolist()
    for k, (a, o) in enumerate(zip(xs, out)):
        assert same(o, oracle.seq_sum(a)), k
    ys = [4.0 * a for a in xs]
    yd = [to_dev(torch, a) for a in ys]
    want = oracle.seq_sum_many(ys)
    _, st0 = ex.exact_seq_sum_batch(yd, flags=ex.CHAIN_PATH, stats=True)
    for rep in range(2):
        out, st = ex.exact_seq_sum_batch(yd, flags=fl, ws=ws, stats=True)
        out = out.cpu().tolist()
        for k in range(len(ys)):
            assert same(out[k], want[k]), (rep, k)
        for lo, hi in ((0, 64), (64, 100)):
            fb = sum(s["fallback_chunks"] for s in st[lo:hi])
            fb0 = sum(s["fallback_chunks"] for s in st0[lo:hi])
            say("group", lo, "call", rep, "fallback chunks reuse", fb, "plain", fb0)
            if rep == 0:
                assert fb > fb0 + 50, (lo, fb, fb0)
            else:
                assert fb <= fb0 + 2 * (hi - lo), (lo, fb, fb0)
