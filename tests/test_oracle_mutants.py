"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake into a temporary copy of the oracle's C source
(on the CPU; the real oracle is untouched), builds it, points the oracle
wrapper at the mutant and runs the pins of test_oracle.py: at least one of
them must fail.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins
from tests import test_oracle_decode as dpins

SRC = os.path.join(os.path.dirname(oracle.__file__), "fa_ref.c")

MUTANTS = {
    "max_shift_sign": ("buf[j] = exp(buf[j] - m);", "buf[j] = exp(m - buf[j]);"),
    "max_shift_dropped_from_lse": ("*lse = m + log(l);", "*lse = log(l);"),
    "scale_dropped": ("buf[j] = scale * acc;", "buf[j] = acc;"),
    "normalisation_dropped": ("double w = buf[j] / l;", "double w = buf[j];"),
    "keys_used_as_values": ("const float *vr = vb + (long)j * vs;",
                            "const float *vr = kb + (long)j * ks;"),
    "transposed_score_operand": ("acc += (double)q[c] * (double)kr[c];",
                                 "acc += (double)q[c] * (double)kb[(long)c * ks + j];"),
    "causal_off_by_one": ("return i + 1 < n ? i + 1 : n;", "return i < n ? i : n;"),
    "causal_ignored": ("    if (!causal)\n        return n;", "    if (1)\n        return n;"),
    "online_rescale_dropped": ("acc[c] *= alpha;", "acc[c] *= 1.0;"),
    "online_sum_not_rescaled": ("l = l * alpha + psum;", "l = l + psum;"),
    "decode_mask_from_the_first_key": ("last = (long)nk - nq + i;", "last = i;"),
    "decode_mask_off_by_one": ("last = (long)nk - nq + i;", "last = (long)nk - nq + i - 1;"),
    "decode_causal_ignored": ("    if (!causal)\n        return nk;", "    if (1)\n        return nk;"),
    "decode_key_stride_of_queries": ("row_three_pass(q + r * d, k + bh * Nk * (long)d, d,",
                                     "row_three_pass(q + r * d, k + bh * Nq * (long)d, d,"),
}

PINS = [
    lambda: pins.test_hand_worked_examples(False),
    lambda: pins.test_hand_worked_examples(True),
    lambda: pins.test_identity_values_give_softmax_rows(False),
    lambda: pins.test_identity_values_give_softmax_rows(True),
    lambda: pins.test_brute_force_4x4_decimal(False),
    lambda: pins.test_brute_force_4x4_decimal(True),
    lambda: pins.test_zero_queries_give_prefix_means(True),
    lambda: pins.test_large_margin_rows_pick_the_argmax_value(),
    lambda: pins.test_online_recurrence_equals_three_pass(True, 37, 8, 11),
    lambda: pins.test_online_recurrence_equals_three_pass(False, 37, 8, 11),
    lambda: dpins.test_decode_square_equals_fwd(True),
    lambda: dpins.test_decode_batch_is_independent_heads(True),
    lambda: dpins.test_decode_is_the_last_rows_of_the_square_problem(3),
    lambda: dpins.test_decode_zero_queries_give_visible_means(True, 4, 9),
    lambda: dpins.test_decode_zero_queries_give_visible_means(True, 12, 9),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                    str(path), "-o", str(so), "-lm"], check=True)
    return oracle._bind(ctypes.CDLL(str(so)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, monkeypatch, name):
    old, new = MUTANTS[name]
    monkeypatch.setattr(oracle, "_lib", _build_mutant(tmp_path, name, old, new))
    caught = []
    for i, pin in enumerate(PINS):
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(i)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    monkeypatch.setattr(oracle, "_lib", _build_mutant(tmp_path, "none", "#include <math.h>", "#include <math.h>"))
    for pin in PINS:
        pin()
