"""Strength of the oracle's pins: copies of oracle.c with one plausible
mistake planted each (a dropped term, a wrong sign or index, a transposed
operand) must each fail at least one pin.  Mistakes are planted in the
oracle, on the CPU only.
"""
import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("no_half_pixel_shift", "double x = (double)W * sx - 0.5;", "double x = (double)W * sx;"),
    ("y_scaled_by_width", "double y = (double)H * sy - 0.5;", "double y = (double)W * sy - 0.5;"),
    ("x_corner_weights_swapped", "(i ? fx : 1.0 - fx)", "(i ? 1.0 - fx : fx)"),
    ("y_weight_uses_fx", "(j ? fy : 1.0 - fy)", "(j ? fx : 1.0 - fy)"),
    ("column_zero_dropped", "cx < 0.0 ||", "cx < 1.0 ||"),
    ("flatten_transposed", "(int64_t)cy * W + (int64_t)cx", "(int64_t)cx * H + (int64_t)cy"),
    ("level_start_ignored", "int64_t pixel = start + (int64_t)cy * W", "int64_t pixel = 0 * start + (int64_t)cy * W"),
    ("wrong_head_channels", "(pixel * v->nH + h) * v->Dh + d", "(pixel * v->nH + (v->nH - 1 - h)) * v->Dh + d"),
    ("softmax_not_normalised", "alpha[i] = exp((double)logits[i]) / denom;", "alpha[i] = exp((double)logits[i]);"),
    ("anchor_by_group", "int m = k % D;", "int m = (k / D) % D;"),
    ("x_offset_over_height", "(double)off[0] / (double)W", "(double)off[0] / (double)H"),
    ("y_offset_sign", "(double)off[1] / (double)H", "-(double)off[1] / (double)H"),
    ("mean_over_all_cameras", "double n = hits > 1 ? (double)hits : 1.0;", "double n = (double)Ncam;"),
    ("first_anchor_ignored", "for (int m = 0; m < D; ++m) any |=", "for (int m = 1; m < D; ++m) any |="),
    ("pairs_camera_major",
     "        for (int64_t b = 0; b < B; ++b)\n            for (int64_t c = 0; c < Ncam; ++c) {\n"
     "                if (pair_offsets) pair_offsets[b * Ncam + c] = (int32_t)n;",
     "        for (int64_t c = 0; c < Ncam; ++c)\n            for (int64_t b = 0; b < B; ++b) {\n"
     "                if (pair_offsets) pair_offsets[b * Ncam + c] = (int32_t)n;"),
    ("frames_summed", "o[i] /= (double)F;", "o[i] /= 1.0;"),
    ("frames_share_weights", "head_weights(attention_weights + (bf * Nq + q) * nH * LP",
     "head_weights(attention_weights + (b * F * Nq + q) * nH * LP"),
    ("bf16_truncates", "rint(x / quantum)", "trunc(x / quantum)"),
    ("bf16_decode_shift", "(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    ("linear_weight_transposed", "W[n * K + k]", "W[k * N + n]"),
    ("query_pos_dropped", "if (query_pos) s = s + query_pos[i * K + k];", "(void)0;"),
    ("query_pos_subtracted", "s = s + query_pos[i * K + k];", "s = s - query_pos[i * K + k];"),
    ("offset_bias_dropped", "W_off, b_off, 1, N_off", "W_off, NULL, 1, N_off"),
    ("residual_dropped", "y[n] += (double)residual[i * N + n];", "y[n] += 0.0;"),
    ("norm_unbiased_variance", "var /= (double)N;", "var /= (double)(N - 1);"),
    ("norm_eps_outside_sqrt", "1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)"),
    ("norm_mean_kept", "y[n] = (y[n] - mean) * inv", "y[n] = y[n] * inv"),
    ("norm_gamma_ignored", "* inv * (double)gamma[n]", "* inv * 1.0"),
    ("bwd_dx_sign", "double wx = (i ? 1.0 : -1.0)", "double wx = (i ? -1.0 : 1.0)"),
    ("bwd_dy_uses_fy", "double wy = (i ? fx : 1.0 - fx) * (j ? 1.0 : -1.0);",
     "double wy = (i ? fy : 1.0 - fy) * (j ? 1.0 : -1.0);"),
    ("bwd_location_not_scaled", "grad_locations[at * 2 + 0] = a * (double)W * dx;",
     "grad_locations[at * 2 + 0] = a * dx;"),
    ("bwd_value_weight_dropped", "+= weight * w * g[d];", "+= w * g[d];"),
    ("bwd_softmax_not_centred", "gw[i] = a[i] * (da[i] - dot);", "gw[i] = a[i] * da[i];"),
    ("bwd_sample_from_x_slope", "*dot_s += w * vg;", "*dot_s += wx * vg;"),
    ("bwd_camera_mean_dropped", "(double)grad_slots[bq * C + (int64_t)h * Dh + d] / n;",
     "(double)grad_slots[bq * C + (int64_t)h * Dh + d] / 1.0;"),
    ("bwd_offset_scaled_by_width", "goff[at * 2 + 0] += a * dx;", "goff[at * 2 + 0] += a * dx * (double)W;"),
]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    src = open(SRC).read()
    d = tmp_path_factory.mktemp("mutants")
    libs = {}
    control = [("control_unmutated", "", "")]
    for name, old, new in control + MUTANTS:
        assert old == "" or src.count(old) >= 1, f"mutant {name}: text not found in oracle.c"
        c = d / f"{name}.c"
        c.write_text(src.replace(old, new, 1) if old else src)
        so = d / f"{name}.so"
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", str(c), "-o",
                        str(so), "-lm"], check=True)
        libs[name] = str(so)
    out = subprocess.run([sys.executable, os.path.join(HERE, "mutant_runner.py"), *libs.values()],
                         check=True, capture_output=True, text=True, timeout=600)
    res = json.loads(out.stdout.strip().splitlines()[-1])
    return {name: res[path] for name, path in libs.items()}


def test_unmutated_copy_passes(mutant_results):
    assert mutant_results["control_unmutated"] == []


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_mutant_is_caught(mutant_results, name):
    assert mutant_results[name], f"planted mistake '{name}' passes every pin"
