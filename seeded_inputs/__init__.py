"""Seeded synthetic inputs shared by the tests, the bench and the oracle side.

This module only draws random numbers into arrays of the workloads' shapes
and distributions; it holds none of the summation method's arithmetic and
imports neither the oracle nor the HIP path.  numpy ``Generator(PCG64(seed))``
everywhere, so a seed names the same bytes on every machine with the same
numpy version.

Workloads (the pages measure on video fixtures that are not available; these
synthetic inputs stand in for them with the same sizes and the structure that
matters to the method):

* ``uniform(n, seed)`` -- n fp64 terms uniform in [0, 1).
* ``tie_heavy(n, seed)`` -- d = 1 - q with q = k * 2^-53, k uniform in
  [2^52, 2^53), so d is a multiple of 2^-53 in (0, 0.5]; 10 % of the terms are
  exactly 0.  Research-1433 Findings 3 describes this term shape (every second
  such term ties while the running sum is in [1, 2)).
* ``signed_terms(n, seed)`` -- 90 % Beta(20, 2), 10 % uniform in [-1, 0.2]:
  signed SSIM-like terms whose running sum needs prefix bounds.
* ``frame_pair(h, w, seed)`` -- uint8 ref uniform in 0..255 and
  dis = clamp(rint(ref + N(0, 8)), 0, 255).
* ``pyramid(seed)`` -- 6 scales of a 3840x2160 frame (each side halved with
  (s + 1) // 2), 3 channels, 6 sums each: sums 0-2 tie-heavy, sums 3-5
  |N(0, 0.05)|; an independent stream per (scale, channel, sum).
"""

from __future__ import annotations

import numpy as np

FRAME_W, FRAME_H = 3840, 2160
FRAME_N = FRAME_W * FRAME_H            # 8,294,400 terms (66,355,200 bytes)
HALF_W, HALF_H = 1920, 1080
HALF_N = HALF_W * HALF_H               # 2,073,600 terms


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def uniform(n: int = 4096, seed: int = 0) -> np.ndarray:
    return rng(seed).random(n)


def tie_heavy(n: int = FRAME_N, seed: int = 0, zero_frac: float = 0.1) -> np.ndarray:
    g = rng(seed)
    k = g.integers(2 ** 52, 2 ** 53, n, dtype=np.int64)
    q = k.astype(np.float64) * 2.0 ** -53      # exact: k < 2^53
    d = 1.0 - q                                 # exact: q in [0.5, 1)
    d[g.random(n) < zero_frac] = 0.0
    return d


def signed_terms(n: int = HALF_N, seed: int = 0) -> np.ndarray:
    g = rng(seed)
    m = g.random(n) < 0.9
    pos = g.beta(20.0, 2.0, n)
    neg = g.uniform(-1.0, 0.2, n)
    return np.where(m, pos, neg)


def half_normal(n: int, seed: int = 0, sigma: float = 0.05) -> np.ndarray:
    return np.abs(rng(seed).normal(0.0, sigma, n))


def frame_pair(h: int = FRAME_H, w: int = FRAME_W, seed: int = 0, sigma: float = 8.0):
    g = rng(seed)
    ref = g.integers(0, 256, (h, w), dtype=np.uint8)
    noise = g.normal(0.0, sigma, (h, w))
    dis = np.clip(np.rint(ref.astype(np.float64) + noise), 0, 255).astype(np.uint8)
    return ref, dis


def pyramid_shapes(w: int = FRAME_W, h: int = FRAME_H, scales: int = 6):
    """(width, height) per scale; each side halved as (s + 1) // 2 while both
    sides stay >= 8, at most ``scales`` scales."""
    out = []
    for _ in range(scales):
        if w < 8 or h < 8:
            break
        out.append((w, h))
        w, h = (w + 1) // 2, (h + 1) // 2
    return out


def pyramid(seed: int = 0, w: int = FRAME_W, h: int = FRAME_H, scales: int = 6,
            channels: int = 3, sums: int = 6):
    """List of ``scales * channels * sums`` fp64 arrays (scale-major order)."""
    out = []
    ss = np.random.SeedSequence(seed)
    children = ss.spawn(len(pyramid_shapes(w, h, scales)) * channels * sums)
    i = 0
    for (sw, sh) in pyramid_shapes(w, h, scales):
        n = sw * sh
        for _c in range(channels):
            for j in range(sums):
                g = np.random.Generator(np.random.PCG64(children[i]))
                i += 1
                if j < sums // 2:
                    k = g.integers(2 ** 52, 2 ** 53, n, dtype=np.int64)
                    d = 1.0 - k.astype(np.float64) * 2.0 ** -53
                    d[g.random(n) < 0.1] = 0.0
                    out.append(d)
                else:
                    out.append(np.abs(g.normal(0.0, 0.05, n)))
    return out


def tie_suite(n: int = 4096, seed: int = 0) -> np.ndarray:
    """Terms k * 2^-53 with k in [0, 7]: started from 1.0 the running sum
    stays in [1, 2) and every term with odd k is a tie at that scale."""
    k = rng(seed).integers(0, 8, n)
    return k.astype(np.float64) * 2.0 ** -53


def lcs_records(windows: int = FRAME_N, seed: int = 0) -> np.ndarray:
    """Records of four doubles per window, (l*c*s, l, c, s), shaped like an
    SSIM pass that keeps the factors: l = 1 - |N(0, 0.02)|,
    c = 1 - |N(0, 0.1)|, s = 1 - |N(0, 0.3)| clipped to [-1, 1], and their
    fp64 product (l * c) * s.  Returned flat, record-major (4 * windows)."""
    r = rng(seed)
    l = 1.0 - np.abs(r.normal(0.0, 0.02, windows))
    c = 1.0 - np.abs(r.normal(0.0, 0.1, windows))
    s = np.clip(1.0 - np.abs(r.normal(0.0, 0.3, windows)), -1.0, 1.0)
    rec = np.empty((windows, 4), dtype=np.float64)
    rec[:, 0] = (l * c) * s
    rec[:, 1] = l
    rec[:, 2] = c
    rec[:, 3] = s
    return rec.reshape(-1)


# ---------------------------------------------------------------------------
# Adversarial sums for the CPU twin of the kernels' composition: each a few
# chunks of 1024 terms whose running sum, in units u = 2^(e - 52) of the
# binade [2^e, 2^(e+1)) it starts in, comes close to or crosses a binade edge
# in the ways the fast paths must refuse or take exactly.  Families:
#
# * ``rise_fall`` -- a negative term in the chunk's first 256 terms, a rise
#   of ~50,000 units over the next 512 that passes 2^(e+1), a fall over the
#   last 256 that comes back below it (the chunk's own sum stays inside).
# * ``edge_counts`` -- whole-unit terms whose running count lands exactly on
#   2^52, 2^52 + 1, 2^53 - 1 or 2^53 at a chunk's end, then odd terms.
# * ``ties`` -- terms of k + 1/2 units (ties) among whole units, placed on
#   lane, wave and chunk edges.
# * ``falling`` -- a sum starting just above 2^e that falls through it.
# * ``neg_cross`` -- a negative term early, an upward crossing late.
# * ``neg_rise`` -- a negative term in the first 256 terms, a rise over the
#   last 256 that passes 2^(e+1) at the chunk's end (the chunk among a sum's
#   first four, or after them).
# * ``subnormal`` -- a sum from +0, -0 or a subnormal that grows through
#   the subnormals (terms of up to 2^24 units of 2^-1074, a few of them
#   negative) into the lowest normal binades.
# * ``mixed`` -- signed terms spanning a few binades.
#
# A sum's first chunks are zeros or not (the adversarial chunk in a sum's
# first four chunks, or in the tiles after them); regular chunks may follow.
# ---------------------------------------------------------------------------
TWIN_FAMILIES = ("rise_fall", "edge_counts", "ties", "falling", "neg_cross", "neg_rise", "subnormal",
                 "mixed")


TWIN_CHAIN_FAMILIES = ("chain_mix", "chain_wave_rise")


def twin_chain_case(seed: int, family: str):
    """(terms, init) of one sum of whole tiles of 4096 terms, for the tile
    chain's twin.  chain_mix: 3-40 tiles in blocks of one kind (tie-free
    rising, rising with half-unit ties, tie-free falling, rising with a few
    negative terms and ties), placed so that the running count meets an edge
    of its binade along the sum (up or down; sometimes the whole sum
    negated).  chain_wave_rise: about 60 tiles with negative terms, then 258
    rising tiles with ties, the count passing the binade's top among the
    latter: one look-back wave of full runs before one of pairs alone."""
    g = rng(seed)
    C = 4096
    e = int(g.integers(-40, 40))
    u = 2.0 ** (e - 52)

    def tile(kind):
        if kind == 0:
            return g.integers(0, 9, C).astype(np.float64)
        if kind == 1:
            k = g.integers(0, 4, C).astype(np.float64)
            return k + np.where(g.random(C) < 0.3, 0.5, 0.0)
        if kind == 2:
            return -g.integers(0, 9, C).astype(np.float64)
        k = g.integers(0, 6, C).astype(np.float64)
        k[g.random(C) < 0.01] = -3.0
        return k + np.where(g.random(C) < 0.1, 0.5, 0.0)

    if family == "chain_wave_rise":
        kinds = [3] * int(g.integers(58, 66)) + [1] * 258
        x = np.concatenate([tile(k) for k in kinds])
        cum = np.cumsum(x)
        m0 = 2.0 ** 53 - float(cum[-1]) * float(g.uniform(0.3, 0.9))
        return x * u, m0 * u
    T = int(g.integers(3, 40))
    kinds = []
    while len(kinds) < T:
        kinds += [int(g.integers(0, 4))] * int(g.integers(1, 12))
    x = np.concatenate([tile(k) for k in kinds[:T]])
    cum = np.cumsum(x)
    top, bot = float(cum.max()), float(cum.min())
    if g.random() < 0.5:
        m0 = 2.0 ** 53 - max(top, 1.0) * float(g.uniform(0.3, 1.3))
        m0 = max(m0, 2.0 ** 52 - bot + 8.0)
    else:
        m0 = 2.0 ** 52 - min(bot, -1.0) * float(g.uniform(0.3, 1.3))
        m0 = min(m0, 2.0 ** 53 - top - 8.0)
    init = float(np.floor(m0)) * u
    x = x * u
    if g.random() < 0.25:
        return -x, -init
    return x, init


def twin_case(seed: int, family: str):
    """(terms, init) of one adversarial sum."""
    g = rng(seed)
    C = 1024
    e = int(g.integers(-60, 60))
    u = 2.0 ** (e - 52)
    lead = int(g.choice([0, 1, 2, 3, 4, 5]))    # zero chunks before (head or tiles)
    tail = int(g.integers(0, 10))               # quiet chunks after
    parts = [np.zeros(lead * C)]
    if family == "rise_fall":
        rise = g.uniform(50.0, 150.0, 2 * 256)
        fall = -g.uniform(150.0, 250.0, 256)
        w0 = g.uniform(0.0, 2.0, 256)
        w0[int(g.integers(0, 256))] = -g.uniform(1.0, 3.0)
        R = float(rise.sum())
        m0 = 2.0 ** 53 - np.floor(R * g.uniform(0.2, 0.8))
        init = m0 * u
        parts.append(np.concatenate([w0, rise, fall]) * u)
    elif family == "neg_rise":
        w = g.uniform(0.0, 2.0, 768)
        w[int(g.integers(0, 256))] = -g.uniform(1.0, 3.0)
        rise = g.uniform(50.0, 150.0, 256)
        m0 = 2.0 ** 53 - float(w.sum()) - np.floor(float(rise.sum()) * g.uniform(0.2, 0.9))
        init = m0 * u
        parts.append(np.concatenate([w, rise]) * u)
    elif family == "edge_counts":
        up = bool(g.integers(0, 2))
        t = g.integers(1, 20, C).astype(np.float64)
        T = float(t.sum())
        d = float(g.integers(-1, 2))
        if up:
            m0 = 2.0 ** 53 - T - d
            chunk = t
        else:
            m0 = 2.0 ** 52 + T + d
            chunk = -t
        init = m0 * u
        odd = (2.0 * g.integers(0, 8, C) + 1.0) * (1 if up else -1)
        parts += [chunk * u, odd * u]
    elif family == "ties":
        m0 = 2.0 ** 52 + float(g.integers(0, 2 ** 51))
        init = m0 * u
        k = g.integers(0, 6, 2 * C).astype(np.float64)
        half = g.random(2 * C) < 0.3
        for p in (0, 3, 4, 63, 64, 255, 256, 1023, 1024, 1279, 1280):
            half[p] = True
        parts.append((k + np.where(half, 0.5, 0.0)) * u)
    elif family == "falling":
        F = 40000.0
        m0 = 2.0 ** 52 + np.floor(F * g.uniform(0.2, 0.8))
        init = m0 * u
        x = -g.uniform(50.0, 110.0, C)
        x[g.random(C) < 0.05] *= -0.5
        parts.append(x * u)
    elif family == "neg_cross":
        x = g.uniform(10.0, 60.0, C)
        x[int(g.integers(0, 256))] = -g.uniform(1.0, 400.0)
        m0 = 2.0 ** 53 - np.floor(float(x[:768].sum()) + g.uniform(0.0, float(x[768:].sum())))
        init = m0 * u
        parts.append(x * u)
    elif family == "subnormal":
        init = float(g.choice([0.0, -0.0, float(g.integers(1, 2 ** 30)) * 2.0 ** -1074]))
        k = g.integers(0, 2 ** int(g.integers(4, 25)), 2 * C).astype(np.float64)
        k[g.random(2 * C) < 0.02] *= -1.0
        parts = [np.zeros(lead * C), k * 2.0 ** -1074]
    else:  # mixed
        init = float(g.uniform(-4.0, 4.0)) * 2.0 ** e
        x = g.normal(0.0, 1.0, 2 * C) * 2.0 ** (e + g.integers(-12, 2, 2 * C).astype(np.float64))
        parts.append(x)
    parts.append(np.zeros(tail * C) if g.random() < 0.5 else g.uniform(0.0, 1.0, tail * C) * u)
    return np.concatenate(parts).astype(np.float64), float(init)
