"""The timeline build of the library: its reader fails loudly without it
(CPU), and on the GPU, where it is built, its call of the frame sum gives the
product library's bits and stamps every tile (the stamps are diagnostics:
the product build compiles them away)."""

import os

import pytest

from bit_exact_sequential_amd import build, timeline
from tests.gpu_util import say, torch_cuda


def test_reader_needs_the_timeline_build(monkeypatch, tmp_path):
    monkeypatch.setattr(build, "TIMELINE_LIB", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="--timeline"):
        timeline.run()


@pytest.mark.gpu
def test_timeline_of_the_frame_sum():
    say("start", "tests/test_timeline.py::test_timeline_of_the_frame_sum")
    if not os.path.exists(build.TIMELINE_LIB):
        pytest.skip("libexseq_timeline.so not built (python -m bit_exact_sequential_amd.build --timeline)")
    torch_cuda()
    r = timeline.run(out=open(os.devnull, "w"))
    assert r["same_bits"]
    assert r["tiles"] == 2025 and r["irregular"] >= 1
    assert r["first_round"] + r["late"] == r["tiles"]
    assert r["last_tile_S_us"] is not None and r["last_tile_S_us"] > 0
