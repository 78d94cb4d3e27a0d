"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of ``oracle/ddpm_oracle.c`` with one plausible mistake
(a dropped term, a wrong sign or index, a transposed operand, a wrong block or
dilation), compiled into a temporary library on the CPU.  The test passes when
at least one pin from ``oracle_pins.py`` rejects the mutant.  Every mutant is
memory-safe: none of them moves an access outside its buffer.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "ddpm_oracle.c")

# (name, text to replace, replacement, which occurrence (0-based) or None for all)
MUTANTS = [
    ("flipped_taps", "const int64_t hh = h + (int64_t)(ki - r) * D;\n            const int64_t ww",
     "const int64_t hh = h + (int64_t)(r - ki) * D;\n            const int64_t ww", 0),
    ("wrong_dilations", "{1, 3, 5}", "{1, 2, 4}", 0),
    ("swapped_dilation_order", "{1, 3, 5}", "{5, 3, 1}", 0),
    ("channel_major_rows", "return ((int64_t)b * C + c) * (int64_t)(K * K) + t;",
     "return ((int64_t)c * 3 + b) * (int64_t)(K * K) + t;", 0),
    ("tap_column_major", "const int t = ki * K + kj;", "const int t = kj * K + ki;", 0),
    ("dropped_bias", "double acc = bg[o];\n        const double *wrow", "double acc = 0.0;\n        const double *wrow", 0),
    ("transposed_weight", "acc += wrow[ci] * yv[ci];", "acc += Wg[ci * R + o] * yv[ci];", 0),
    ("x_block_last", "out[((n * 4 * C + c) * H + h) * W + w] = x[",
     "out[((n * 4 * C + 3 * C + c) * H + h) * W + w] = x[", None),
    ("dx_missing_passthrough", "dxp[q] = Gx[q];", "dxp[q] = 0.0;", 0),
    ("dx_scatter_wrong_direction", "const int64_t hh = h + (int64_t)(ki - r) * D;\n                                const int64_t ww = w + (int64_t)(kj - r) * D;",
     "const int64_t hh = h - (int64_t)(ki - r) * D;\n                                const int64_t ww = w - (int64_t)(kj - r) * D;", 0),
    ("dx_without_bias", "double acc = bg[o];\n                            for", "double acc = 0.0;\n                            for", 0),
    ("dy_transposed_weight", "acc += Wg[o * C + ci] * dK[o];", "acc += Wg[(o % C) * (R / C) + o / C] * dK[o];", 0),
    ("dy_unshifted_x", "xv = x[((n * C + c) * H + hh) * W + ww];", "xv = x[((n * C + c) * H + h) * W + w];", 0),
    ("dw_shifted_y", "wrow[ci] += dk * y[((n * C + ci) * H + h) * W + w];",
     "wrow[ci] += dk * y[((n * C + ci) * H + hh) * W + ww];", 0),
    ("db_sums_grad", "sb += dk;", "sb += G[((n * 4 * C + (1 + b) * C + c) * H + h) * W + w];", 0),
    ("partials_skip_last", "for (int64_t s = 0; s < S; ++s)", "for (int64_t s = 0; s + 1 < S; ++s)", 0),
    ("filter_bwd_dtaps_unshifted_x", "Gb[h * W + w] * x[((n * C + c) * H + hh) * W + ww]",
     "Gb[h * W + w] * x[((n * C + c) * H + h) * W + w]", 0),
    ("filter_bwd_dx_missing_passthrough", "dxp[q] = Gx[q];", "dxp[q] = 0.0;", 1),
    ("filter_bwd_dx_tap_at_destination", "dxp[hh * W + ww] += tp[h * W + w] * Gb[h * W + w];",
     "dxp[hh * W + ww] += tp[hh * W + ww] * Gb[h * W + w];", 0),
    ("filter_bwd_wrong_grad_block", "const double *Gb = G + (n * 4 * C + (1 + b) * C + c) * HW;",
     "const double *Gb = G + (n * 4 * C + b * C + c) * HW;", 0),
]


def _mutate(text, old, new, which):
    assert old in text, f"mutation anchor not found: {old!r}"
    if which is None:
        return text.replace(old, new)
    parts = text.split(old)
    assert which < len(parts) - 1
    return old.join(parts[:which + 1]) + new + old.join(parts[which + 1:])


@pytest.mark.parametrize("name,old,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, which):
    text = open(SRC).read()
    mutated = _mutate(text, old, new, which)
    assert mutated != text
    src = tmp_path / f"{name}.c"
    src.write_text(mutated)
    lib = oracle.build(src=str(src), out=str(tmp_path / f"{name}.so"))
    orc = oracle.Oracle(oracle.load(lib))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            caught.append((pin.__name__, str(e)[:120]))
            break
    assert caught, f"mutant {name} passed every pin"
