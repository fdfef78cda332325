"""GPU parity of the interleaved sums (exact_seq_sum_f64_interleaved): k
independent in-order sums over records of k doubles and their float means
equal the oracle's bits (0 ULP, and the same float bits), through the C ABI."""

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


def records(windows, k, seed):
    """Fields of different kinds side by side: tie-heavy, uniform, signed."""
    x = np.empty(windows * k)
    for j in range(k):
        kind = j % 3
        if kind == 0:
            x[j::k] = si.tie_heavy(windows, seed + j)
        elif kind == 1:
            x[j::k] = si.uniform(windows, seed + j)
        else:
            x[j::k] = si.signed_terms(windows, seed + j)
    return x


def check(torch, x, k, inits=None, flags=0, means=True):
    sums, mt = ex.exact_seq_sum_interleaved(to_dev(torch, x), k, inits, means=means, flags=flags)
    want, wmeans = oracle.seq_sum_interleaved(x, k, inits)
    got = sums.cpu().numpy()
    for j in range(k):
        assert same(got[j], want[j]), (k, j, got[j], want[j])
    if means:
        assert np.array_equal(mt.cpu().numpy().view(np.uint32), wmeans.view(np.uint32))


# both launch plans: the default (the single pass for k = 2 and 4, whose
# tiles read every record line once; the tile chain otherwise) and the tile
# chain forced
PATHS = [0, ex.CHAIN_PATH]


@pytest.mark.parametrize("windows", [0, 1, 3, 1023, 1024, 1025, 4096 * 3 + 7, 200_001])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("path", PATHS)
def test_sizes(windows, k, path):
    torch = torch_cuda()
    x = records(windows, k, windows + 10 * k)
    inits = [0.5 * j for j in range(k)] if windows % 2 else None
    check(torch, x, k, inits, flags=path)


@pytest.mark.parametrize("path", PATHS)
def test_lcs_full_size(path):
    """The LCS layout of a 3840x2160 frame: (l*c*s, l, c, s) per window."""
    torch = torch_cuda()
    x = si.lcs_records(si.FRAME_N, 0)
    check(torch, x, 4, flags=path)


@pytest.mark.parametrize("k", [2, 4])
def test_records_not_16_byte_aligned(k):
    """Records that start 8 bytes past a 16-byte boundary (the tiles then
    read them with 8-byte loads)."""
    torch = torch_cuda()
    windows = 300_001
    x = records(windows, k, 77 + k)
    buf = torch.empty(x.size + 1, dtype=torch.float64, device="cuda")
    buf[1:] = torch.from_numpy(x).cuda()
    xd = buf[1:]
    assert xd.data_ptr() % 16 == 8
    sums, mt = ex.exact_seq_sum_interleaved(xd, k, None, means=True)
    want, wmeans = oracle.seq_sum_interleaved(x, k)
    got = sums.cpu().numpy()
    for j in range(k):
        assert same(got[j], want[j]), (k, j)
    assert np.array_equal(mt.cpu().numpy().view(np.uint32), wmeans.view(np.uint32))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_lcs_full_size_more_seeds(seed):
    torch = torch_cuda()
    check(torch, si.lcs_records(si.FRAME_N, seed), 4, inits=[0.0, 1.0, -1.0, 0.25])


@pytest.mark.parametrize("flags", [ex.PLAN_ALL_FALLBACK, ex.PLAN_PLUS_ONE, ex.PLAN_MINUS_ONE, ex.PLAN_ALL_ZERO,
                                   ex.plan_fixed(1023), ex.WALK_ONLY, 1 << 4, 2 << 4, 3 << 4, ex.CHAIN_CUT])
def test_plan_and_chain_variants(flags):
    torch = torch_cuda()
    x = records(300_000, 4, 5)
    check(torch, x, 4, [1.0, 0.0, -1.0, 2.0], flags=flags)


@pytest.mark.parametrize("windows", [32773, 200001, 518400])
@pytest.mark.parametrize("flags", [0, 1 << 4, 2 << 4, 3 << 4, (3 << 4) | ex.WALK_ONLY,
                                   (3 << 4) | ex.CHAIN_CUT])
def test_lcs_tile_sizes(windows, flags):
    """The l*c*s field rises through binades with a rare negative term: a
    chunk whose negative term lies in an earlier wave than its upward
    crossing must not pass as staying in its binade, for every tile size."""
    torch = torch_cuda()
    check(torch, si.lcs_records(windows, 0), 4, flags=flags)


def test_plan_reuse_sequence_and_no_means():
    torch = torch_cuda()
    windows, k = 400_000, 4
    ws = ex.workspace(ex.lib().exact_seq_sum_f64_interleaved_workspace_size(windows, k),
                      torch.device("cuda"))
    for f in range(3):
        x = si.lcs_records(windows, 20 + f)
        sums, mt = ex.exact_seq_sum_interleaved(to_dev(torch, x), k, means=False,
                                                flags=ex.PLAN_REUSE, ws=ws)
        assert mt is None
        want, _ = oracle.seq_sum_interleaved(x, k)
        got = sums.cpu().numpy()
        for j in range(k):
            assert same(got[j], want[j]), (f, j)


def test_rejects_bad_arguments():
    torch = torch_cuda()
    L = ex.lib()
    x = to_dev(torch, np.ones(8))
    out = torch.empty(8, dtype=torch.float64, device="cuda")
    ws = ex.workspace(L.exact_seq_sum_f64_interleaved_workspace_size(2, 4), torch.device("cuda"))
    for k in (0, 9):
        assert L.exact_seq_sum_f64_interleaved(x.data_ptr(), 1, k, None, out.data_ptr(), None,
                                               ws.data_ptr(), ws.numel(), None, 0, None) == -1
    assert L.exact_seq_sum_f64_interleaved(x.data_ptr(), 2, 4, None, out.data_ptr(), None,
                                           ws.data_ptr(), 16, None, 0, None) == -2
