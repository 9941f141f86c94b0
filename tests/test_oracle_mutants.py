"""Plant mistakes in copies of the oracle source and check that the pins notice.

Each mutant is a one-line edit of ``oracle/attn_oracle.c`` of the kind that
slips into a hand-written attention routine (a dropped term, a wrong sign,
index or operand).  The copy is built in a temporary directory on the CPU;
every mutant must fail at least one pin.  No GPU is involved.

``PY_MUTANTS`` do the same to the oracle's Python wrapper
(``oracle/__init__.py``), whose batch loop and host-thread split of heads and
rows carry no arithmetic but choose which inputs each call sees: the patched
copy is loaded as a module of its own over the real oracle library.
"""
import importlib.util
import os

import pytest

import oracle
from oracle import _build
import oracle_pins

MUTANTS = {
    "scale_dropped": ("s[p] = dot * scale;", "s[p] = dot;"),
    "scale_without_sqrt": ("1.0 / sqrt((double)D)", "1.0 / (double)D"),
    "k_layout_transposed": ("k[(p * H + h) * D + i]", "k[(h * S + p) * D + i]"),
    "v_always_head0": ("v[(p * H + h) * D + d]", "v[(p * H) * D + d]"),
    "v_positions_reversed": ("v[(p * H + h) * D + d]", "v[((L - 1 - p) * H + h) * D + d]"),
    "q_always_head0": ("q[h * D + i]", "q[i]"),
    "mask_one_past": ("(size_t)current_pos : S - 1) + 1;", "(size_t)current_pos + 1 : S - 1) + 1;"),
    "shift_sign_flipped": ("e[p] = exp(s[p] - m);", "e[p] = exp(m - s[p]);"),
    "min_instead_of_max": ("if (s[p] > m)", "if (s[p] < m)"),
    "not_normalised": ("acc += (e[p] / z) *", "acc += e[p] *"),
    "decoder_bias_off": ("expo - 25", "expo - 24"),
    "decoder_subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "decoder_sign_dropped": ("return sign ? -mag : mag;", "return mag;"),
    "decoder_implicit_bit_dropped": ("(1024 + frac)", "(frac)"),
    "masked_score_zero": ("p < L ? s[p] : -INFINITY", "p < L ? s[p] : 0.0"),
    "pv_scores_transposed": ("oracle_half_to_double(scores[h * S + p])", "oracle_half_to_double(scores[p * H + h])"),
    "pv_max_is_min": ("            if (s > m)\n", "            if (s < m || m == -INFINITY)\n"),
    "pv_neg_inf_not_skipped": ("                if (e[p] != 0.0)\n", ""),
    "half_ties_always_up": ("return fmod(f, 2.0) == 0.0 ? f : f + 1.0;", "return f + 1.0;"),
    "half_subnormal_scale": ("ldexp(a, 24)", "ldexp(a, 23)"),
    "half_overflow_missed": ("int E = ex - 1;\n    if (E > 15)", "int E = ex - 1;\n    if (E > 99)"),
    "half_sign_dropped": ("signbit(x) ? 0x8000u : 0u", "0u"),
    "rope_sin_sign_flipped": ("o[ia] = a * c - b * s;", "o[ia] = a * c + b * s;"),
    "rope_frequency_exponent": ("-(2.0 * i) / (double)dims", "-(1.0 * i) / (double)dims"),
    "rope_pairing_swapped": ("traditional ? ", "!traditional ? "),
    "rope_position_off_by_one": ("(double)pos[r] * theta", "(double)(pos[r] + 1) * theta"),
    "rope_tail_zeroed": ("o[d] = oracle_half_to_double(row[d]);", "o[d] = 0.0;"),
    "rope_partner_wrong": ("(size_t)i + half;", "(size_t)i + half - (i > 0);"),
    "softmax_min_for_max": ("            if ((double)row[c] > m)\n", "            if ((double)row[c] < m)\n"),
    "softmax_no_shift": ("o[c] = exp((double)row[c] - m);", "o[c] = exp((double)row[c]);"),
    "softmax_not_normalised": ("o[c] = o[c] / z;", "o[c] = o[c];"),
    "softmax_column_major": ("const float *row = x + r * C;", "const float *row = x + r;"),
    "softmax_last_column_dropped": ("        for (size_t c = 0; c < C; ++c) {\n            o[c] = exp(", "        for (size_t c = 0; c + 1 < C; ++c) {\n            o[c] = exp("),
}

PY_MUTANTS = {
    "batched_shared_current_pos": ("int(current_pos[b])", "int(current_pos[0])"),
    "batched_query_of_first_sequence": ("self.decode(q[b], k[b], v[b]", "self.decode(q[0], k[b], v[b]"),
    "batched_cache_of_first_sequence": ("self.decode(q[b], k[b], v[b]", "self.decode(q[b], k[0], v[0]"),
    "threads_head_range_short_by_one": (
        "bounds = [(H * i // threads, H * (i + 1) // threads) for i in range(threads)]",
        "bounds = [(H * i // threads, H * (i + 1) // threads - 1) for i in range(threads)]"),
    "threads_last_head_range_dropped": (
        "bounds = [(H * i // threads, H * (i + 1) // threads) for i in range(threads)]",
        "bounds = [(H * i // threads, H * (i + 1) // threads) for i in range(threads - 1)]"),
    "softmax_threads_row_skipped": ("(rows * i // threads, rows * (i + 1) // threads)",
                                    "(rows * i // threads + (i > 0), rows * (i + 1) // threads)"),
}


def _failed_pins(orc):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_wrapper_mutant_fails_a_pin(name, tmp_path):
    old, new = PY_MUTANTS[name]
    src_path = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")
    with open(src_path) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation site missing or ambiguous: %r" % old
    path = os.path.join(tmp_path, "mutant_wrapper.py")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    # a module inside the oracle package, so its relative import resolves
    spec = importlib.util.spec_from_file_location("oracle._mutant_" + name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    oracle.load()   # the real C library, built if missing
    failed = _failed_pins(mod.OracleLib(_build.LIB))
    assert failed, "no pin caught wrapper mutant %s" % name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    with open(_build.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, "mutation site missing: %r" % old
    mutated = src.replace(old, new)
    c_path = os.path.join(tmp_path, "mutant.c")
    with open(c_path, "w") as f:
        f.write(mutated)
    lib = _build.build(src=c_path, lib=os.path.join(tmp_path, "libmutant.so"))
    failed = _failed_pins(oracle.OracleLib(lib))
    assert failed, "no pin caught mutant %s" % name
