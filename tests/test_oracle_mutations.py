"""Plant a plausible mistake in a copy of the oracle (on the CPU) and require
at least one pin to catch it.  This shows the pins constrain every part of the
oracle: the loop's bounds, sign, start value, precision and order; the term's
operands, signs, constants and rounding; the moments' window and products;
the frame sum's raster order; the interleaved sums' fields, start values,
record count and the float mean's rounding."""

import os
import shutil

import pytest

import oracle
from tests import oracle_pins as P

HERE = os.path.dirname(oracle.__file__)

LOOP_MUTANTS = {
    "drop_first": ("for (size_t i = 0; i < n; i++)", "for (size_t i = 1; i < n; i++)"),
    "drop_last": ("for (size_t i = 0; i < n; i++)", "for (size_t i = 0; i + 1 < n; i++)"),
    "wrong_sign": ("s += x[i];", "s -= x[i];"),
    "ignore_init": ("double s = init;", "double s = 0.0;"),
    "x87_accumulator": ("double s = init;", "long double s = init;"),
    "float_accumulator": ("double s = init;", "float s = init;"),
    "reversed_order": ("s += x[i];", "s += x[n - 1 - i];"),
    "kahan": (("double s = init;", "double s = init, c = 0.0;"),
              ("        s += x[i];\n",
               "    { double y = x[i] - c; double t = s + y; c = (t - s) - y; s = t; }\n")),
    "pairs": ("        s += x[i];\n",
              "        { if (i + 1 < n) { s += x[i] + x[i + 1]; i++; } else s += x[i]; }\n"),
}

TERM_MUTANTS = {
    "wrong_moment": ("x2 * w_d - mx2 + y2 * w_d - my2 + c2", "x2 * w_d - mx2 + y2 * w_d - mxy + c2"),
    "swapped_constants": ("(2 * mxy + c1)", "(2 * mxy + c2)"),
    "wrong_sign_cov": ("(c2 + 2 * (xy * w_d - mxy))", "(c2 + 2 * (xy * w_d + mxy))"),
    "dropped_c1": ("((mx2 + my2 + c1)", "((mx2 + my2)"),
    "wrong_product": ("double mxy = (double)x * (double)y;", "double mxy = (double)x * (double)x;"),
    "dropped_factor_w": ("return w * (2 * mxy + c1)", "return (2 * mxy + c1)"),
    "window_off_by_one": ("for (int a = i - radius; a <= i + radius; a++) {\n                if (a < 0",
                          "for (int a = i - radius; a < i + radius; a++) {\n                if (a < 0"),
    "cross_product": ("sxy += p * q;", "sxy += p * p;"),
    "untruncated_weight": ("mw[k] = sw;", "mw[k] = (2 * radius + 1) * (2 * radius + 1);"),
    "column_order_sum": ("double s = 0.0;\n    int64_t ws = 0;\n    for (int i = 0; i < height; i++) {",
                         "double s = 0.0;\n    int64_t ws = 0;\n    for (int i = height - 1; i >= 0; i--) {"),
}


INTERLEAVE_MUTANTS = {
    "swapped_fields": ("out[j] += x[w * (size_t)k + (size_t)j];",
                       "out[j] += x[w * (size_t)k + (size_t)(k - 1 - j)];"),
    "float_division": ("means[j] = (float)(out[j] / (double)windows);",
                       "means[j] = (float)out[j] / (float)windows;"),
    "ignore_init": ("out[j] = inits[j];", "out[j] = 0.0;"),
    "drop_last_record": ("for (size_t w = 0; w < windows; w++)",
                         "for (size_t w = 0; w + 1 < windows; w++)"),
    "float_terms": ("out[j] += x[w * (size_t)k + (size_t)j];",
                    "out[j] += (float)x[w * (size_t)k + (size_t)j];"),
    "mean_by_k": ("means[j] = (float)(out[j] / (double)windows);",
                  "means[j] = (float)(out[j] / (double)(windows * (size_t)k));"),
}


def _build_mutant(tmp_path, src_name, edits, extra_flags=()):
    """``edits``: one (old, new) pair or a tuple of them; every occurrence of
    ``old`` is replaced (the window mutation must hit the moments and the
    frame sum alike)."""
    d = tmp_path / "m"
    d.mkdir(exist_ok=True)
    for s in oracle._SOURCES:
        shutil.copy(os.path.join(HERE, s), d / s)
    text = (d / src_name).read_text()
    if isinstance(edits[0], str):
        edits = (edits,)
    for old, new in edits:
        assert text.count(old) >= 1, "mutation site not found: %r" % old
        text = text.replace(old, new)
    (d / src_name).write_text(text)
    out = str(d / "liboracle_mut.so")
    oracle.build(out, sources=[str(d / s) for s in oracle._SOURCES],
                 extra_flags=extra_flags)
    return oracle.load(out)


def _caught(lib, pins):
    for pin in pins:
        try:
            pin(lib)
        except AssertionError:
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(LOOP_MUTANTS))
def test_loop_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, "seq_sum.c", LOOP_MUTANTS[name])
    caught = _caught(lib, P.LOOP_PINS)
    assert caught, "mutant %s passed every loop pin" % name


@pytest.mark.parametrize("name", sorted(TERM_MUTANTS))
def test_term_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, "ssim_ref.c", TERM_MUTANTS[name])
    caught = _caught(lib, P.TERM_PINS)
    assert caught, "mutant %s passed every term pin" % name


def test_contracted_build_is_caught(tmp_path):
    """Built with FMA contraction the term's roundings change; the per-operation
    evaluation pin (CPython floats, one rounding per operation, C's order)
    catches it.  That pin checks evaluation, not the formula: the formula is
    pinned by the textbook value above."""
    lib = _build_mutant(tmp_path, "ssim_ref.c", ("double w_d", "double w_d"),
                        extra_flags=("-ffp-contract=fast", "-mfma", "-O3"))
    assert _caught(lib, (P.pin_term_per_operation,)), "contraction not detected"


@pytest.mark.parametrize("name", sorted(INTERLEAVE_MUTANTS))
def test_interleave_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, "seq_sum.c", INTERLEAVE_MUTANTS[name])
    caught = _caught(lib, P.INTERLEAVE_PINS)
    assert caught, "mutant %s passed every interleave pin" % name
