"""Where the exact chain's time goes: a timeline of one call's tiles.

    python -m bit_exact_sequential_amd.build --timeline
    python -m bit_exact_sequential_amd.timeline [--ssim] [--seed S]

Runs the 3840x2160 tie-heavy frame sum (or, with ``--ssim``, the fused SSIM
frame) once through the diagnostic twin of the library, whose tiles record the
GPU's 100 MHz real-time counter at their steps, and prints, in microseconds
from the first stamp:

* the head (the sum's first chunk added term by term);
* when the tiles started, planned (look-back done) and, for regular tiles,
  published their runs: how many ran in the first round of resident
  workgroups and how many waited for a slot;
* for every irregular tile: its plan, its runs, its crossing search, its
  look-back over the regular tiles before it, the arrival of the exact sum
  before it, and its own exact sum -- the links of the serial chain.

The result is compared bit for bit with the product library's.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

from . import build as _build

KTL_TILES = 16384  # tiles the diagnostic build records (kTlTiles)
KTL_PER = 12       # words per tile (kTlPer)
TILE_CHUNKS = 4    # chunks per tile of the single-sum chain (the default tile)


def _pct(a, q):
    return float(np.percentile(a, q)) if len(a) else float("nan")


def run(ssim: bool = False, seed: int = 0, out=sys.stdout) -> dict:
    if not os.path.exists(_build.TIMELINE_LIB):
        raise RuntimeError("libexseq_timeline.so is not built: run "
                           "`python -m bit_exact_sequential_amd.build --timeline`")
    import torch
    import seeded_inputs as si
    import bit_exact_sequential_amd as ex

    dev = torch.device("cuda:0")
    # the product library's result first, then the diagnostic twin's
    if ssim:
        ref, dis = si.frame_pair(si.FRAME_H, si.FRAME_W, seed)
        rd, dd = torch.from_numpy(ref).to(dev), torch.from_numpy(dis).to(dev)
        call = lambda: ex.ssim_term_and_sum(rd, dd, 3)[0]  # noqa: E731
        n = si.FRAME_N
    else:
        x = torch.from_numpy(si.tie_heavy(si.FRAME_N, seed)).to(dev)
        call = lambda: ex.exact_seq_sum(x)  # noqa: E731
        n = si.FRAME_N
    want = call().cpu().numpy().view(np.uint64)[0]
    saved = (ex._lib, ex.LIB_PATH)
    ex._lib = None
    ex.LIB_PATH = _build.TIMELINE_LIB
    try:
        return _timed(ex, torch, call, want, n, ssim, seed, out)
    finally:
        # the process goes on with the product library
        ex._lib, ex.LIB_PATH = saved


def _timed(ex, torch, call, want, n, ssim, seed, out):
    L = ex.lib()
    L.exseq_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.exseq_timeline_words.restype = ctypes.c_size_t
    words = int(L.exseq_timeline_words())
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    if L.exseq_timeline_clear() != 0:
        raise RuntimeError("exseq_timeline_clear failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    got = call()
    e1.record()
    torch.cuda.synchronize()
    same = got.cpu().numpy().view(np.uint64)[0] == want
    buf = np.zeros(words, dtype=np.uint64)
    if L.exseq_timeline_read(buf.ctypes.data, words) != 0:
        raise RuntimeError("exseq_timeline_read failed")

    nt = (n + 1024 * TILE_CHUNKS - 1) // (1024 * TILE_CHUNKS)
    st = buf[:KTL_PER * nt].reshape(nt, KTL_PER).astype(np.int64)
    head = buf[KTL_PER * KTL_TILES: KTL_PER * KTL_TILES + 2].astype(np.int64)
    t0 = min(int(st[st[:, 0] > 0, 0].min()), int(head[0]) if head[0] else 1 << 62)
    us = lambda v: (np.asarray(v, dtype=np.int64) - t0) / 100.0  # noqa: E731
    irr = st[:, 4] == 1
    reg = ~irr & (st[:, 3] > 0)
    s0, s1, s3 = us(st[:, 0]), us(st[:, 1]), us(st[reg, 3])
    late = s0 > 4.0
    res = {"call_us": e0.elapsed_time(e1) * 1e3, "same_bits": bool(same), "tiles": nt,
           "irregular": int(irr.sum()), "head": (float(us(head[0])), float(us(head[1]))),
           "first_round": int((~late).sum()), "late": int(late.sum())}
    p = lambda *a: print(*a, file=out)  # noqa: E731
    p("workload: %s, seed %d, %d tiles of %d chunks" %
      ("fused SSIM 3840x2160 (radius 3)" if ssim else "tie-heavy 3840x2160 frame sum", seed, nt,
       TILE_CHUNKS))
    p("call (events, diagnostic build): %.1f us; same bits as the product library: %s" %
      (res["call_us"], same))
    p("head (first chunk term by term): %.2f -> %.2f" % res["head"])
    p("tiles started within 4 us (the first round of resident workgroups): %d; later: %d "
      "(first late tile %d)" % (res["first_round"], res["late"],
                                int(np.nonzero(late)[0][0]) if late.any() else -1))
    p("                 p10     p50     p90     max")
    for name, v in (("started", s0), ("planned", s1), ("published", s3)):
        p("%-12s %7.2f %7.2f %7.2f %7.2f" % (name, _pct(v, 10), _pct(v, 50), _pct(v, 90),
                                              v.max() if len(v) else float("nan")))
    p("irregular tiles (the serial chain), us:")
    p("  tile   start  planned   runs  x-search  x-found  back-in  back-out  S-arrived  own-S")
    f = lambda v: "%8.2f" % us(v) if v else "       -"  # noqa: E731
    for k in np.nonzero(irr)[0]:
        r = st[k]
        p("  %4d %s %s %s %s %s %s %s %s %s" % (k, f(r[0]), f(r[1]), f(r[2]), f(r[8]), f(r[9]),
                                                f(r[3]), f(r[5]), f(r[6]), f(r[7])))
    last = st[nt - 1]
    res["last_tile_S_us"] = float(us(last[7])) if last[7] else None
    p("the sum's last tile has its exact sum at %.2f us" % (res["last_tile_S_us"] or float("nan")))
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--ssim", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    a = ap.parse_args(argv)
    r = run(ssim=a.ssim, seed=a.seed)
    return 0 if r["same_bits"] else 1


if __name__ == "__main__":
    sys.exit(main())
