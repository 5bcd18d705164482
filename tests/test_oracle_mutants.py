"""The oracle's pins reject plausible mistakes (CPU only).

Each case copies oracle.c, plants one mistake by text substitution (a dropped
term, a transposed operand, a wrong tie or rounding rule), builds the copy as
a separate library and runs the pins that should catch it with the oracle
module pointed at that library. The case passes when at least one of those
pins fails. The committed oracle source is never modified.
"""
from __future__ import annotations

import inspect
import os
import subprocess

import pytest

from oracle import oracle as orc

import test_oracle_pins as pins

_SRC = os.path.join(os.path.dirname(orc.__file__), "oracle.c")

# (name, original text, planted text, pins expected to catch it)
MUTANTS = [
    # block score keeps only the q'*min term: the min/max bound no longer
    # covers the block's tokens
    ("score_min_only", "s += a > b ? a : b;", "s += b;",
     [pins.test_P5_quest_score_equals_eq12_at_block_size_one]),
    # logits and scores without the 1/sqrt(d) factor
    ("score_unscaled", "sc[noff + l] = s * scale;", "sc[noff + l] = s;",
     [pins.test_P5_quest_score_equals_eq12_at_block_size_one]),
    # top-r ties go to the higher channel instead of the lower
    ("topr_ties_high", "return x->c - y->c;", "return y->c - x->c;",
     [pins.test_P3_worked_example_d4]),
    # storage rounding rounds halves up instead of to even
    ("round_half_up", "if (rem > half || (rem == half && (kept & 1))) kept++;", "if (rem >= half) kept++;",
     [pins.test_round_bf16_is_nearest_even, pins.test_round_f32_matches_ieee_cast]),
    # the rotation multiplies by R^T instead of R
    ("rotation_transposed", "s += R[c * d + j] * x[j];", "s += R[j * d + c] * x[j];",
     [pins.test_P4_full_retention_equals_dense_attention]),
    # the block count rounds down instead of up
    ("keep_floor", "else k = ((int64_t)keep_ppm * n + 999999) / 1000000;",
     "else k = ((int64_t)keep_ppm * n) / 1000000;", [pins.test_block_keep_rule]),
    # top-k ties go to the higher block instead of the lower
    ("topk_ties_high", "return x->l < y->l ? -1 : (x->l > y->l ? 1 : 0);",
     "return x->l > y->l ? -1 : (x->l < y->l ? 1 : 0);", [pins.test_P6_topk_matches_subset_enumeration]),
    # sigma reported as the eigenvalue itself, not its square root
    ("sigma_not_sqrt", "if (sigma) sigma[c] = sqrt(lam > 0.0 ? lam : 0.0);",
     "if (sigma) sigma[c] = lam > 0.0 ? lam : 0.0;", [pins.test_P2_energy_closed_form_and_singular_values]),
    # R stored with the singular vectors as columns instead of rows
    ("rotation_vectors_as_columns", "for (int j = 0; j < d; ++j) R[c * d + j] = sg * V[j * d + col];",
     "for (int j = 0; j < d; ++j) R[j * d + c] = sg * V[j * d + col];",
     [pins.test_P2_energy_closed_form_and_singular_values, pins.test_rotation_matches_library_svd_vectors]),
    # the inverse rotation multiplies by R_v instead of R_v^T
    ("inverse_rotation_transposed", "s += Rvj[c * d + jj] *", "s += Rvj[jj * d + c] *",
     [pins.test_P4_full_retention_equals_dense_attention]),
    # forced selection: every packed segment reads the first segment's columns
    ("forced_offset_dropped", "sh[koff + i] = forced_sel[h * ksum + koff + i];",
     "sh[koff + i] = forced_sel[h * ksum + i];",
     [pins.test_forced_random_selection_equals_dense_reconstruction,
      pins.test_forced_selection_of_own_choice_is_identical]),
    # the threshold reported is the (k+1)-th score instead of the k-th
    ("tau_next_score", "tau[h * npacked + pj] = k > 0 ? tmp[k - 1].s : NAN;",
     "tau[h * npacked + pj] = k > 0 ? tmp[k].s : NAN;", [pins.test_tau_is_kth_largest_score]),
    # incremental appends rebuild block keys from the block after the one the
    # previous call left partly filled
    ("incremental_keys_skip_open_block", "const int64_t from = t_from > t_begin[j] ? (t_from - t_begin[j]) / block : 0;",
     "const int64_t from = t_from > t_begin[j] ? (t_from - t_begin[j]) / block + 1 : 0;",
     [pins.test_incremental_compression_equals_bulk]),
    # a segment with its own rotation is scored and attended with the unit's q'
    ("segment_query_not_rotated", "if (segR && segR[j]) rotate(segR[j], q + (int64_t)h * d, d, qseg + (int64_t)j * d);",
     "if (0) rotate(segR[j], q + (int64_t)h * d, d, qseg + (int64_t)j * d);",
     [pins.test_P4_per_segment_rotations_equal_dense_attention,
      pins.test_per_segment_rotation_matches_unrotated_reconstruction]),
    # a segment's share of the output is rotated back by the unit's R_v
    ("segment_inverse_rotation_unit", "const double *Rvj = (segR && segR[j]) ? segR[j] + (int64_t)d * d : Rv;",
     "const double *Rvj = Rv;",
     [pins.test_P4_per_segment_rotations_equal_dense_attention,
      pins.test_per_segment_rotation_matches_unrotated_reconstruction]),
    # a segment with its own rotation is compressed with the unit's
    ("segment_compressed_with_unit_rotation",
     "const double *R = (segR && segR[j]) ? segR[j] + (int64_t)which * d * d : (which == 0 ? Rk : Rv);",
     "const double *R = which == 0 ? Rk : Rv;",
     [pins.test_P4_per_segment_rotations_equal_dense_attention]),
    # channel-compressed block keys are ignored: every score sums all d channels
    ("key_channels_ignored", "const int m = (key_ch && key_ch[j] > 0 && key_ch[j] < d) ? key_ch[j] : d;",
     "const int m = d;", [pins.test_key_channels_score_equals_full_score_of_masked_query]),
    # the scores sum the trailing channels instead of the leading ones
    ("key_channels_trailing", "for (int c = 0; c < m; ++c) {", "for (int c = d - m; c < d; ++c) {",
     [pins.test_key_channels_score_equals_full_score_of_masked_query]),
    # group energies leave out each group's last channel
    ("group_energy_drops_last", "for (int m = 0; m < g; ++m) {\n            const double v = xr[g * i + m];",
     "for (int m = 0; m < g - 1; ++m) {\n            const double v = xr[g * i + m];",
     [pins.test_group_topr_matches_subset_enumeration, pins.test_group_topr_with_one_channel_per_group_is_per_element_topr]),
    # groups of strided instead of adjacent channels
    ("group_strided", "const double v = xr[g * i + m];", "const double v = xr[i + ng * m];",
     [pins.test_group_topr_matches_subset_enumeration, pins.test_group_topr_with_one_channel_per_group_is_per_element_topr]),
    # the kept groups are the lowest-energy ones
    ("group_lowest_kept", "for (int m = 0; m < g; ++m) idx[n++] = g * tmp[k].c + m;",
     "for (int m = 0; m < g; ++m) idx[n++] = g * tmp[ng - 1 - k].c + m;",
     [pins.test_group_topr_matches_subset_enumeration]),
    # incremental appends skip the first new token
    ("incremental_skips_first_token", "for (int64_t t = t_from; t < len; ++t) {\n        const int j",
     "for (int64_t t = t_from + 1; t < len; ++t) {\n        const int j",
     [pins.test_incremental_compression_equals_bulk]),
]


def _build_mutant(tmp_path, name, old, new):
    with open(_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation site not unique in oracle.c: %r" % old
    path = tmp_path / ("oracle_%s.c" % name)
    path.write_text(src.replace(old, new))
    so = str(tmp_path / ("liboracle_%s.so" % name))
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC",
                           "-shared", "-o", so, str(path), "-lm"])
    return so


def _call(pin):
    """Run a pin against whichever oracle library is current; pins that take
    the rotation case get one computed by that library."""
    if "rot_case" in inspect.signature(pin).parameters:
        K, _ = pins._unit_inputs(3000)
        R, sig = orc.rotation(K)
        pin((K, R, sig))
    else:
        pin()


@pytest.mark.parametrize("name,old,new,catchers", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(tmp_path, name, old, new, catchers):
    so = _build_mutant(tmp_path, name, old, new)
    saved_so, saved_lib = orc._SO, orc._LIB
    caught = []
    try:
        orc._SO, orc._LIB = so, None
        for pin in catchers:
            try:
                _call(pin)
            except AssertionError:
                caught.append(pin.__name__)
    finally:
        orc._SO, orc._LIB = saved_so, saved_lib
    assert caught, "no pin caught the planted mistake %s" % name


def test_unmutated_copy_passes_the_same_pins(tmp_path):
    """The harness itself: a copy built the same way with no change passes every pin used above."""
    so = _build_mutant(tmp_path, "none", "return x->c - y->c;", "return x->c - y->c;")
    saved_so, saved_lib = orc._SO, orc._LIB
    try:
        orc._SO, orc._LIB = so, None
        for pin in {p for m in MUTANTS for p in m[3]}:
            _call(pin)
    finally:
        orc._SO, orc._LIB = saved_so, saved_lib
