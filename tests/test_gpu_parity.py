"""GPU parity: every sum from the HIP path equals the oracle bit for bit
(tolerance 0 ULP), through the C ABI.  Inputs are seeded; both sides see the
same bytes."""

import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import bit_exact_sequential_amd as ex
from tests import suites
from tests.gpu_util import same, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

PLANS = [ex.PLAN_AUTO, ex.PLAN_ALL_FALLBACK, ex.PLAN_PLUS_ONE, ex.PLAN_MINUS_ONE, ex.PLAN_ALL_ZERO,
         ex.plan_fixed(1023)]
# both launch plans of a plain sum: the tile chain (default for one sum) and
# the single pass
PATHS = [0, ex.PASS_PATH]


@pytest.fixture(autouse=True)
def _name(request):
    say("start", request.node.nodeid)
    yield


def gpu_sum(torch, x, init=0.0, flags=0, stats=False):
    xd = to_dev(torch, x)
    r = ex.exact_seq_sum(xd, init, flags=flags, stats=stats)
    if stats:
        out, st = r
        return float(out.cpu()[0]), st
    return float(r.cpu()[0])


@pytest.mark.parametrize("case", suites.edge_suite(), ids=lambda c: c[0])
def test_edge_cases(case):
    torch = torch_cuda()
    name, x, init = case
    want = oracle.seq_sum(x, init)
    for plan in (ex.PLAN_AUTO, ex.PLAN_ALL_FALLBACK, ex.PLAN_PLUS_ONE):
        for path in PATHS:
            got = gpu_sum(torch, x, init, plan | path)
            assert same(got, want), (name, plan, path, got, want)


@pytest.mark.parametrize("n", suites.ragged_sizes())
def test_ragged_sizes(n):
    torch = torch_cuda()
    for x in (si.tie_heavy(n, n), si.signed_terms(n, n + 1)):
        for path in PATHS:
            got = gpu_sum(torch, x, 0.0, path)
            assert same(got, oracle.seq_sum(x)), (n, path)


@pytest.mark.parametrize("case", suites.workload_suite(small=True), ids=lambda c: c[0])
def test_workloads_every_plan(case):
    """Research-1433 Findings 5: the plan cannot change a result."""
    torch = torch_cuda()
    name, x, init = case
    want = oracle.seq_sum(x, init)
    for plan in PLANS:
        for path in PATHS:
            got = gpu_sum(torch, x, init, plan | path)
            assert same(got, want), (name, plan, path, got, want)


CHAIN_VARIANTS = [0, ex.PASS_PATH, ex.WALK_ONLY, ex.CHAIN_CUT, ex.tile_flag(1), ex.tile_flag(2),
                  ex.tile_flag(1) | ex.CHAIN_CUT, ex.tile_flag(2) | ex.CHAIN_CUT]


@pytest.mark.parametrize("case", suites.workload_suite(small=True), ids=lambda c: c[0])
def test_workloads_chain_variants(case):
    """The exact chain between tiles, the walk alone, and the walk resuming
    from the chain's last exact value give the same bits at every tile size."""
    torch = torch_cuda()
    name, x, init = case
    want = oracle.seq_sum(x, init)
    for fl in CHAIN_VARIANTS:
        got, st = gpu_sum(torch, x, init, fl, stats=True)
        assert same(got, want), (name, fl, got, want)
        assert st["fast_chunks"] + st["fallback_chunks"] == st["chunks"], (name, fl, st)


def test_full_size_chain_cut():
    """The frame-size sum with the chain stopped half way: the walk resumes
    from the last exact value published before the cut."""
    torch = torch_cuda()
    for name, x in (("tie_heavy", si.tie_heavy(si.FRAME_N, 11)),
                    ("signed", si.signed_terms(si.HALF_N, 12))):
        want = oracle.seq_sum(x)
        for fl in (ex.CHAIN_CUT, ex.WALK_ONLY):
            got, st = gpu_sum(torch, x, 0.0, fl, stats=True)
            say(name, fl, st)
            assert same(got, want), (name, fl, got, want)


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
def test_full_size_workloads(seed):
    """The frame-size tie-heavy sum (8,294,400 terms), the 1920x1080 signed
    sum and the 4096-term uniform sum, five seeds each, at full size."""
    torch = torch_cuda()
    for name, x in (("uniform", si.uniform(4096, seed)),
                    ("tie_heavy", si.tie_heavy(si.FRAME_N, seed)),
                    ("signed", si.signed_terms(si.HALF_N, seed))):
        want = oracle.seq_sum(x)
        for path in PATHS:
            got, st = gpu_sum(torch, x, 0.0, path, stats=True)
            say(name, seed, path, st)
            assert same(got, want), (name, seed, path, got, want)


def test_full_size_stats_ranges():
    """Fallback counts in the range the method predicts (Research-1433
    Findings 4; Research-1424 Findings 3): both frames add only their first
    chunk term by term, give or take a crossing whose checks fail -- every
    binade crossing after it is located and applied in O(1), under negative
    terms too (their prefixes checked against the bounds)."""
    torch = torch_cuda()
    x = si.tie_heavy(si.FRAME_N, 0)
    _, st = gpu_sum(torch, x, stats=True)
    assert st["chunks"] == 8100
    assert 1 <= st["fallback_chunks"] <= 3, st
    assert st["first_fallback"] == 0, st
    assert st["fast_chunks"] + st["fallback_chunks"] == 8100
    assert st["flags"] == 0
    y = si.signed_terms(si.HALF_N, 0)
    _, st = gpu_sum(torch, y, stats=True)
    assert st["chunks"] == 2025
    assert 1 <= st["fallback_chunks"] <= 4, st
    assert st["fast_chunks"] + st["fallback_chunks"] == 2025


def test_tie_fast_path_suite():
    """init = 1 and terms k * 2^-53: the sum stays in [1, 2) and every odd k
    is a tie on the fast path."""
    torch = torch_cuda()
    for seed in range(3):
        x = si.tie_suite(1 << 20, seed)
        got, st = gpu_sum(torch, x, 1.0, stats=True)
        assert same(got, oracle.seq_sum(x, 1.0))
        # only the first chunk, added in order from init by its tile
        assert st["fallback_chunks"] <= 1, st
        assert st["fast_chunks"] + st["fallback_chunks"] == st["chunks"], st


def test_exhaustive_short_sequences():
    torch = torch_cuda()
    cases = suites.exhaustive_short(8)
    for i, (x, init) in enumerate(cases):
        got = gpu_sum(torch, x, init)
        assert same(got, oracle.seq_sum(x, init)), (i, x, init)


def test_resume_with_init():
    torch = torch_cuda()
    x = si.signed_terms(300_000, 5)
    whole = oracle.seq_sum(x)
    for k in (0, 1, 1024, 150_001, 300_000):
        head = oracle.seq_sum(x[:k])
        assert same(gpu_sum(torch, x[k:], head), whole), k


def test_unaligned_terms():
    """Terms at an 8-byte but not 16-byte aligned address take the scalar
    load path."""
    torch = torch_cuda()
    x = si.tie_heavy(100_001, 3)
    xd = to_dev(torch, np.concatenate([[0.0], x]))[1:]
    assert xd.data_ptr() % 16 == 8
    got = float(ex.exact_seq_sum(xd).cpu()[0])
    assert same(got, oracle.seq_sum(x))


def test_repeat_determinism():
    torch = torch_cuda()
    x = to_dev(torch, si.signed_terms(si.HALF_N, 7))
    first = float(ex.exact_seq_sum(x).cpu()[0])
    outs = torch.empty(50, dtype=torch.float64, device="cuda")
    for i in range(50):
        ex.exact_seq_sum(x, out=outs[i:i + 1])
    assert all(same(v, first) for v in outs.cpu().tolist())


def test_tree_sum_gap_and_determinism():
    """The fixed tree is deterministic and within the standard error bound
    of a depth-d tree (d * 2^-53 * sum|x|); its gap to the exact sum is what
    the exact path removes."""
    torch = torch_cuda()
    x = si.tie_heavy(si.FRAME_N, 1)
    xd = to_dev(torch, x)
    t1 = float(ex.tree_sum(xd).cpu()[0])
    t2 = float(ex.tree_sum(xd).cpu()[0])
    assert same(t1, t2)
    exact = math.fsum(x)
    depth = 2 + 6 + 2 + 3 + 10 + 1
    assert abs(t1 - exact) <= depth * 2.0 ** -53 * float(np.abs(x).sum()) * 1.01
    seq = oracle.seq_sum(x)
    say("tree", t1, "seq", seq, "gap", t1 - seq)


def test_batch_matches_single_sums():
    torch = torch_cuda()
    arrays = [si.tie_heavy(n, n) for n in (0, 1, 1000, 4097, 65_536, 300_001)]
    inits = [0.0, 1.0, -2.0, 0.5, 0.0, 3.0]
    xs = [to_dev(torch, a) for a in arrays]
    out = ex.exact_seq_sum_batch(xs, inits).cpu().tolist()
    for a, i, o in zip(arrays, inits, out):
        assert same(o, oracle.seq_sum(a, i))


def test_pyramid_batch_full():
    """108 sums of the 6-scale pyramid of a 3840x2160 frame."""
    torch = torch_cuda()
    arrays = si.pyramid(0)
    assert len(arrays) == 108
    xs = [to_dev(torch, a) for a in arrays]
    out = ex.exact_seq_sum_batch(xs).cpu().tolist()
    want = oracle.seq_sum_many(arrays)
    for k, (o, w) in enumerate(zip(out, want)):
        assert same(o, w), k


SIZES = [(1, 1), (2, 2), (3, 4), (5, 7), (9, 9), (16, 16), (33, 17), (65, 63), (182, 322),
         (8, 8), (17, 9), (31, 33), (323, 577), (48, 64), (47, 65)]


SSIM_MODES = [0, ex.SSIM_IN_TILES]


@pytest.mark.parametrize("mode", SSIM_MODES, ids=["producer", "in_tiles"])
@pytest.mark.parametrize("hw", SIZES, ids=lambda s: "%dx%d" % s)
def test_ssim_small_frames(hw, mode):
    """Frame sizes from the pages' random-size lists; every term and the sum
    equal the oracle's, with the terms formed by the producer or in the sum's
    tiles."""
    torch = torch_cuda()
    h, w = hw
    ref, dis = si.frame_pair(h, w, h * 1000 + w)
    s, wsum, terms = oracle.ssim_frame_sum(ref, dis, 3, want_terms=True)
    r = torch.from_numpy(ref).cuda()
    d = torch.from_numpy(dis).cuda()
    gs, gw, gt = ex.ssim_term_and_sum(r, d, 3, want_terms=True, flags=mode)
    assert np.array_equal(gt.cpu().numpy().view(np.uint64), terms.view(np.uint64))
    assert same(float(gs.cpu()[0]), s)
    assert int(gw.cpu()[0]) == wsum
    # without the terms asked for (the producer: the workspace holds them)
    gs2, gw2, _ = ex.ssim_term_and_sum(r, d, 3, flags=mode)
    assert same(float(gs2.cpu()[0]), s)
    assert int(gw2.cpu()[0]) == wsum


@pytest.mark.parametrize("hwsr", [(40, 1088, 1088, 3), (33, 1100, 1100, 5), (21, 1057, 1057, 3),
                                  (19, 1088, 1096, 15), (9, 2048, 2052, 0), (64, 1280, 1280, 1),
                                  (24, 1280, 1284, 2), (17, 1104, 1104, 4), (12, 1536, 1540, 6)],
                         ids=lambda v: "%dx%d_s%d_r%d" % v)
@pytest.mark.parametrize("mode", SSIM_MODES, ids=["producer", "in_tiles"])
def test_ssim_wide_rows(hwsr, mode):
    """Rows at least as wide as a chunk's span (the producer's one-division
    row tracking; 4-byte plane loads where rows and strides are multiples of
    four): every term and the sum equal the oracle's, padded strides too."""
    torch = torch_cuda()
    h, w, stride, radius = hwsr
    ref, dis = si.frame_pair(h, w, h * 7 + w)
    s, wsum, terms = oracle.ssim_frame_sum(ref, dis, radius, want_terms=True)
    big_r = np.zeros((h, stride), np.uint8)
    big_d = np.zeros((h, stride), np.uint8)
    big_r[:, :w] = ref
    big_d[:, :w] = dis
    r = torch.from_numpy(big_r).cuda()[:, :w]
    d = torch.from_numpy(big_d).cuda()[:, :w]
    gs, gw, gt = ex.ssim_term_and_sum(r, d, radius, want_terms=True, flags=mode)
    assert np.array_equal(gt.cpu().numpy().view(np.uint64), terms.view(np.uint64))
    assert same(float(gs.cpu()[0]), s)
    assert int(gw.cpu()[0]) == wsum


@pytest.mark.parametrize("mode", SSIM_MODES, ids=["producer", "in_tiles"])
@pytest.mark.parametrize("radius", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("hw", [(37, 203), (16, 64), (9, 13)], ids=lambda s: "%dx%d" % s)
def test_ssim_radius_small_frames(hw, radius, mode):
    """Narrow frames at every window radius up to five (the producer's
    register windows take radii up to four, on pixels away from the row
    ends; the rest add up their windows from LDS): every term and the sum
    equal the oracle's."""
    torch = torch_cuda()
    h, w = hw
    ref, dis = si.frame_pair(h, w, 31 * h + w + radius)
    s, wsum, terms = oracle.ssim_frame_sum(ref, dis, radius, want_terms=True)
    gs, gw, gt = ex.ssim_term_and_sum(torch.from_numpy(ref).cuda(), torch.from_numpy(dis).cuda(),
                                      radius, want_terms=True, flags=mode)
    assert np.array_equal(gt.cpu().numpy().view(np.uint64), terms.view(np.uint64))
    assert same(float(gs.cpu()[0]), s)
    assert int(gw.cpu()[0]) == wsum


@pytest.mark.parametrize("mode", SSIM_MODES, ids=["producer", "in_tiles"])
def test_ssim_full_frame(mode):
    torch = torch_cuda()
    ref, dis = si.frame_pair(si.FRAME_H, si.FRAME_W, 0)
    s, wsum, _ = oracle.ssim_frame_sum(ref, dis, 3)
    r = torch.from_numpy(ref).cuda()
    d = torch.from_numpy(dis).cuda()
    gs, gw, _, st = ex.ssim_term_and_sum(r, d, 3, stats=True, flags=mode)
    say("ssim full", mode, st)
    assert same(float(gs.cpu()[0]), s)
    assert int(gw.cpu()[0]) == wsum


@pytest.mark.parametrize("flags", [ex.SSIM_IN_TILES | ex.WALK_ONLY, ex.SSIM_IN_TILES | ex.CHAIN_CUT,
                                   ex.SSIM_IN_TILES | ex.PLAN_ALL_FALLBACK, ex.SSIM_IN_TILES | ex.tile_flag(1),
                                   ex.SSIM_IN_TILES | ex.tile_flag(2) | ex.CHAIN_CUT,
                                   ex.CHAIN_CUT, ex.PASS_PATH, ex.PLAN_ALL_FALLBACK, ex.WALK_ONLY])
def test_ssim_fused_paths(flags):
    """The terms formed in the tiles under every walk (the terms the tiles
    form and the ones the walk forms again for chunks it adds term by term),
    and the producer's terms under the sum's launch plans, give the oracle's
    sum (radius 5, a frame whose rows are not a multiple of a chunk, plane
    rows padded)."""
    torch = torch_cuda()
    h, w = 211, 373
    ref, dis = si.frame_pair(h, w, 77)
    s, wsum, _ = oracle.ssim_frame_sum(ref, dis, 5)
    big_r = np.zeros((h, 400), np.uint8)
    big_d = np.zeros((h, 400), np.uint8)
    big_r[:, :w] = ref
    big_d[:, :w] = dis
    r = torch.from_numpy(big_r).cuda()[:, :w]
    d = torch.from_numpy(big_d).cuda()[:, :w]
    gs, gw, _, st = ex.ssim_term_and_sum(r, d, 5, flags=flags, stats=True)
    assert same(float(gs.cpu()[0]), s), flags
    assert int(gw.cpu()[0]) == wsum
    assert st["fast_chunks"] + st["fallback_chunks"] == st["chunks"]


def test_ssim_term_divide_against_host():
    """The device divide and term equal the host's on many random windows,
    including wide int64 moments where products round (stride > width)."""
    torch = torch_cuda()
    for radius in (0, 1, 3, 5):
        ref, dis = si.frame_pair(37, 53, 40 + radius)
        s, wsum, terms = oracle.ssim_frame_sum(ref, dis, radius, want_terms=True)
        big_r = np.zeros((37, 64), np.uint8)
        big_d = np.zeros((37, 64), np.uint8)
        big_r[:, :53] = ref
        big_d[:, :53] = dis
        r = torch.from_numpy(big_r).cuda()[:, :53]
        d = torch.from_numpy(big_d).cuda()[:, :53]
        gs, gw, gt = ex.ssim_term_and_sum(r, d, radius, want_terms=True)
        assert np.array_equal(gt.cpu().numpy().view(np.uint64), terms.view(np.uint64)), radius
        assert same(float(gs.cpu()[0]), s)


@pytest.mark.parametrize("n", [1, 1023, 1024, 5000, 8192])
def test_one_launch_small_sums(n):
    """Sums of at most 8 chunks run as one launch that adds every chunk in
    order: exact, every chunk counted as added term by term, and the same
    bits as with the three-launch path (forced by an explicit tile size)."""
    torch = torch_cuda()
    x = si.tie_heavy(n, n)
    got, st = gpu_sum(torch, x, 0.5, stats=True)
    assert same(got, oracle.seq_sum(x, 0.5))
    nch = (n + 1023) // 1024
    assert st["chunks"] == nch and st["fallback_chunks"] == nch and st["fast_chunks"] == 0, st
    assert st["fallback_terms"] == n and st["first_fallback"] == 0, st
    got4 = gpu_sum(torch, x, 0.5, flags=3 << 4)
    assert same(got4, got)


@pytest.mark.parametrize("flags", [1 << 4, 2 << 4, 3 << 4, (3 << 4) | ex.WALK_ONLY, ex.WALK_ONLY])
def test_rise_after_negative_term(flags):
    """A rising sum whose chunk holds a negative term in one wave and its
    upward binade crossing in a later, rising wave (the l*c*s products,
    whose prefixes of 3 chunks show it): the chunk's largest prefix counts
    the later wave's rise, so the chunk is never applied as staying in its
    binade.  Every prefix length, every tile size, with and without the chain."""
    torch = torch_cuda()
    f = np.ascontiguousarray(si.lcs_records(518400, 0)[0::4])
    for n in (3072, 4096, 5000, 40960, 518400):
        x = f[:n]
        assert same(gpu_sum(torch, x, 0.0, flags=flags), oracle.seq_sum(x)), (n, flags)


def test_twin_replays_the_single_pass():
    """The CPU twin of the single pass takes the kernel's paths: the same
    result and the same fast and term-by-term chunk counts on the GPU."""
    torch = torch_cuda()
    cases = (("tie_heavy 100003", si.tie_heavy(100_003, 41), 0.0),
             ("signed 300001", si.signed_terms(300_001, 42), 0.0),
             ("tie suite", si.tie_suite(1 << 20, 43), 1.0),
             ("negated tie_heavy", -si.tie_heavy(200_000, 44), 0.0),
             ("tie_heavy 3840x2160", si.tie_heavy(si.FRAME_N, 45), 0.0))
    for name, x, init in cases:
        got, st = gpu_sum(torch, x, init, ex.PASS_PATH, stats=True)
        tw, tst = ex.twin_seq_sum(x, init)
        say(name, st, tst)
        assert same(got, tw), name
        assert (st["fast_chunks"], st["fallback_chunks"]) == (tst["fast_chunks"], tst["fallback_chunks"]), name
