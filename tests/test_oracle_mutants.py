"""Plant plausible mistakes in copies of the reference convolution and check
that the pins catch each one (on the CPU, never on the GPU)."""
import os

import pytest

from oracle_pins import ALL_PINS

# (name, text in conv_oracle.c, replacement) -- each a plausible slip
MUTANTS = [
    ("flipped_kernel", "w[w_index(pr, k, c, r, s)]", "w[w_index(pr, k, c, pr->R - 1 - r, pr->S - 1 - s)]"),
    ("pad_sign", "p * pr->stride_h - pr->pad_h", "p * pr->stride_h + pr->pad_h"),
    ("pad_w_uses_pad_h", "q * pr->stride_w - pr->pad_w", "q * pr->stride_w - pr->pad_h"),
    ("filter_r_s_swapped", "((k * pr->C + c) * pr->R + r) * pr->S + s", "((k * pr->C + c) * pr->R + s) * pr->S + r"),
    ("nhwc_filter_c_k_mixed", "((k * pr->R + r) * pr->S + s) * pr->C + c", "((c * pr->R + r) * pr->S + s) * pr->K + k"),
    ("x_h_w_transposed_nhwc", "((n * pr->H + h) * pr->W + w) * pr->C + c", "((n * pr->H + w) * pr->W + h) * pr->C + c"),
    ("bias_dropped", "double acc = b ? b[k] : 0.0;", "double acc = 0.0;"),
    ("dilation_is_stride", "r * pr->dil_h", "r * pr->stride_h"),
    ("last_tap_dropped", "s < pr->S; ++s", "s + 1 < pr->S; ++s"),
    ("first_channel_dropped", "c = 0; c < pr->C; ++c", "c = 1; c < pr->C; ++c"),
    ("out_extent_off_by_one", "*Q = span_w / pr->stride_w + 1;", "*Q = (span_w + 1) / pr->stride_w + 1;"),
    ("bf16_bias_off", "expo - 134", "expo - 133"),
    ("f16_subnormal_scale", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("abs_scale_signed", "mag += fabs(prod);", "mag += prod;"),
    ("nchw_output_p_q_swapped", "((n * pr->K + k) * P + p) * Q + q", "((n * pr->K + k) * Q + q) * P + p"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, oracle_mod, tmp_path):
    src = oracle_mod.source_text()
    assert src.count(old) >= 1, "mutation anchor not found: %r" % old
    mutant = oracle_mod.build_variant(src.replace(old, new), os.path.join(str(tmp_path), "mutant_%s.so" % name))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception as e:  # any failure (assertion, error code) counts as caught
            caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
