"""Parity coverage on the GPU beyond the basic suites: more seeds at full
size for the fused SSIM frame and the pyramid batch, every term of a full
frame, the device divide on a million operand pairs, the non-finite flag,
determinism over a thousand calls per launch plan, and the exhaustive
tie-alphabet sequences placed where the tiles' lane and wave composition
adds them, and sums that grow through the subnormal range (Research-1433
"Forming the CPU's sequential double sums on a GPU, bit for bit", Findings 5
and "Tests"; Research-1424 "integer_ssim_cuda and the CPU's frame sum",
Findings 1)."""

import math

import numpy as np
import pytest

import oracle
import seeded_inputs as si
import bit_exact_sequential_amd as ex
from tests import suites
from tests.gpu_util import same, say, to_dev, torch_cuda


def gpu_sum(torch, x, init=0.0, flags=0, stats=False):
    r = ex.exact_seq_sum(to_dev(torch, x), init, flags=flags, stats=stats)
    if stats:
        out, st = r
        return float(out.cpu()[0]), st
    return float(r.cpu()[0])


pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    say("start", request.node.nodeid)
    yield


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_pyramid_batch_more_seeds(seed):
    torch = torch_cuda()
    arrays = si.pyramid(seed)
    want = oracle.seq_sum_many(arrays)
    xs = [to_dev(torch, a) for a in arrays]
    for path in ((0, ex.CHAIN_PATH) if seed == 1 else (0,)):
        got = ex.exact_seq_sum_batch(xs, flags=path).cpu().tolist()
        for k, (o, w) in enumerate(zip(got, want)):
            assert same(o, w), (seed, path, k)


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_ssim_full_frame_more_seeds(seed):
    torch = torch_cuda()
    ref, dis = si.frame_pair(si.FRAME_H, si.FRAME_W, seed)
    s, wsum, _ = oracle.ssim_frame_sum(ref, dis, 3)
    r, d = torch.from_numpy(ref).cuda(), torch.from_numpy(dis).cuda()
    for mode in (0, ex.SSIM_IN_TILES):
        gs, gw, _ = ex.ssim_term_and_sum(r, d, 3, flags=mode)
        assert same(float(gs.cpu()[0]), s), (seed, mode)
        assert int(gw.cpu()[0]) == wsum


@pytest.mark.parametrize("mode", [0, ex.SSIM_IN_TILES], ids=["producer", "in_tiles"])
def test_ssim_full_frame_every_term(mode):
    torch = torch_cuda()
    ref, dis = si.frame_pair(si.FRAME_H, si.FRAME_W, 0)
    s, wsum, terms = oracle.ssim_frame_sum(ref, dis, 3, want_terms=True)
    gs, gw, gt = ex.ssim_term_and_sum(torch.from_numpy(ref).cuda(), torch.from_numpy(dis).cuda(), 3,
                                      want_terms=True, flags=mode)
    g = gt.cpu().numpy()
    assert g.size == si.FRAME_N
    diff = np.nonzero(g.view(np.uint64) != terms.view(np.uint64))[0]
    assert diff.size == 0, diff[:10]
    assert same(float(gs.cpu()[0]), s)


def _divide_operands(seed: int, n: int):
    g = np.random.Generator(np.random.PCG64(seed))
    edge = np.array([0.0, -0.0, 1.0, -1.0, 3.0, 1.0 / 3.0, 2.0 ** -1074, -(2.0 ** -1074),
                     2.0 ** -1022, 2.0 ** -1022 * (1 - 2.0 ** -52), np.finfo(np.float64).max,
                     -np.finfo(np.float64).max, 2.0 ** 52, 2.0 ** 53 + 2, 0.5, 2.0 ** 1023,
                     math.inf, -math.inf, math.nan, 1e-300, 1e300, 7.0, 0.1])
    ea, eb = np.meshgrid(edge, edge)
    # random bit patterns over every exponent (NaNs drawn this way are kept)
    ra = g.integers(0, 2 ** 63, n, dtype=np.int64).view(np.float64) * np.where(g.random(n) < 0.5, -1, 1)
    rb = g.integers(0, 2 ** 63, n, dtype=np.int64).view(np.float64)
    # operands of the term's shape: products of window moments
    w = g.integers(1, 50, n).astype(np.float64)
    x = g.integers(0, 255 * 49, n).astype(np.float64)
    y = g.integers(0, 255 * 49, n).astype(np.float64)
    num = w * (2.0 * (x * y) + 6.5025) * (58.5225 + 2.0 * (g.integers(0, 2 ** 20, n) * w - x * y))
    den = (x * x + y * y + 6.5025) * (g.integers(0, 2 ** 22, n) * w + 58.5225)
    a = np.concatenate([ea.ravel(), ra, num])
    b = np.concatenate([eb.ravel(), rb, den])
    return a, b


def test_device_divide_million_pairs():
    torch = torch_cuda()
    a, b = _divide_operands(77, 600_000)
    assert a.size >= 1_000_000
    with np.errstate(all="ignore"):
        want = a / b
    got = ex.device_div(to_dev(torch, a), to_dev(torch, b)).cpu().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    bad = np.nonzero(got[~nan].view(np.uint64) != want[~nan].view(np.uint64))[0]
    assert bad.size == 0, (a[~nan][bad[:5]], b[~nan][bad[:5]])


@pytest.mark.parametrize("case", suites.edge_suite(), ids=lambda c: c[0])
def test_nonfinite_flag(case):
    """EXSEQ_STAT_NONFINITE is set exactly when a term is +-inf or NaN."""
    torch = torch_cuda()
    name, x, init = case
    want_flag = bool(np.any(~np.isfinite(x)))
    for path in (0, ex.PASS_PATH):
        out, st = ex.exact_seq_sum(to_dev(torch, x), init, flags=path, stats=True)
        assert same(float(out.cpu()[0]), oracle.seq_sum(x, init)), (name, path)
        assert bool(st["flags"] & ex.STAT_NONFINITE) == want_flag, (name, path, st)


def test_thousand_repeats_every_launch_plan():
    torch = torch_cuda()
    x = si.signed_terms(si.HALF_N, 8)
    xd = to_dev(torch, x)
    want = oracle.seq_sum(x)
    for fl in (0, ex.PASS_PATH, ex.tile_flag(1), ex.tile_flag(2), ex.tile_flag(4)):
        outs = torch.empty(1000, dtype=torch.float64, device="cuda")
        for i in range(1000):
            ex.exact_seq_sum(xd, flags=fl, out=outs[i:i + 1])
        vals = outs.cpu().numpy()
        assert np.all(vals.view(np.uint64) == np.float64(want).view(np.uint64)), fl


@pytest.mark.parametrize("offset", [4096, 4096 + 252, 4096 + 1020])
def test_exhaustive_sequences_through_tiles(offset):
    """Every length-10 sequence over the tie-building alphabets, after
    `offset` zeros: at a tile's start, across a wave edge and across a chunk
    edge, so that the tiles' lane, wave and chunk composition adds them."""
    torch = torch_cuda()
    cases = suites.exhaustive_short(10)
    for path in (0, ex.CHAIN_PATH):
        for k in range(0, len(cases), 64):
            group = cases[k:k + 64]
            xs = [np.concatenate([np.zeros(offset), x]) for x, _ in group]
            inits = [i for _, i in group]
            got = ex.exact_seq_sum_batch([to_dev(torch, a) for a in xs], inits, flags=path).cpu().tolist()
            for j, (a, init) in enumerate(zip(xs, inits)):
                assert same(got[j], oracle.seq_sum(a, init)), (offset, path, k + j)


@pytest.mark.parametrize("init", [0.0, -0.0, 3 * 2.0 ** -1074], ids=["zero", "minus_zero", "subnormal"])
def test_subnormal_range_runs(init):
    """Sums that start at zero or a subnormal and grow through the subnormals
    into the normal binades: exact under every launch plan and tile size, and
    the fast paths take them (the subnormal range is one count range with the
    lowest binade's unit)."""
    torch = torch_cuda()
    g = np.random.Generator(np.random.PCG64(91))
    n = 600_001
    rising = g.integers(0, 2 ** 30, n).astype(np.float64) * 2.0 ** -1074
    mixed = rising.copy()
    mixed[g.random(n) < 0.01] *= -1.0
    for name, x in (("rising", rising), ("some negative", mixed)):
        want = oracle.seq_sum(x, init)
        for fl in (0, ex.PASS_PATH, ex.tile_flag(1), ex.tile_flag(2), ex.tile_flag(4), ex.WALK_ONLY):
            got, st = gpu_sum(torch, x, init, fl, stats=True)
            assert same(got, want), (name, fl, got, want)
            if name == "rising" and fl != ex.WALK_ONLY:
                assert st["fast_chunks"] >= 0.9 * st["chunks"], (fl, st)


TILE4 = 3 << 4  # bits 4..5 of flags: four chunks per tile


@pytest.mark.parametrize("family", si.TWIN_CHAIN_FAMILIES)
def test_chain_families(family):
    """The adversarial sums of whole tiles that the tile chain's CPU twin is
    checked on (blocks of tie-free rising, tied rising, falling and mixed
    tiles meeting a binade edge; a wave of tiles with negative terms before
    a wave of tied rising tiles that passes the binade's top), through the
    GPU's tile chain at four chunks per tile under every plan, with the
    chain cut half way, and through the single pass: the oracle's bits."""
    torch = torch_cuda()
    seeds = range(60) if family == "chain_mix" else range(6)
    flag_sets = (0, TILE4, TILE4 | ex.PLAN_PLUS_ONE, TILE4 | ex.PLAN_MINUS_ONE,
                 TILE4 | ex.PLAN_ALL_ZERO, TILE4 | ex.CHAIN_CUT, ex.PASS_PATH)
    for sd in seeds:
        x, init = si.twin_chain_case(sd, family)
        want = oracle.seq_sum(x, init)
        xd = to_dev(torch, x)
        for fl in flag_sets:
            got = float(ex.exact_seq_sum(xd, init, flags=fl).cpu()[0])
            assert same(got, want), (family, sd, fl)
