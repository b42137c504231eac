"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks
that the pin suite catches each one.  The real oracle is never modified."""
import os
import subprocess

import pytest

from oracle import oracle as O
from tests import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attnres_oracle.c")

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("eps_dropped", "sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H)"),
    ("eps_outside_root", "sqrt(ss / (double)H + eps)", "(sqrt(ss / (double)H) + eps)"),
    ("sum_not_mean", "sqrt(ss / (double)H + eps)", "sqrt(ss + eps)"),
    ("norm_weight_dropped", "double normed = xhat[h] * bf16_bits_to_double(rms_w[h]);",
     "double normed = xhat[h];"),
    ("score_weight_dropped", "acc += bf16_bits_to_double(res_w[h]) * normed;", "acc += normed;"),
    ("mix_normalised_rows", "            l[j] = acc;\n",
     "            l[j] = acc;\n            memcpy(src + (int64_t)j * H, xhat, sizeof(double) * (size_t)H);\n"),
    ("strides_transposed", "blocks + t * token_stride + (int64_t)j * slot_stride",
     "blocks + t * slot_stride + (int64_t)j * token_stride"),
    ("softmax_sign", "p[j] = exp(l[j] - m);", "p[j] = exp(m - l[j]);"),
    ("softmax_not_normalised", "        p[j] /= z;\n", "        p[j] /= 1.0;\n"),
    ("cur_not_rounded", "round_to_bf16(pv + bf16_bits_to_double(delta[t * H + h]))",
     "(pv + bf16_bits_to_double(delta[t * H + h]))"),
    ("delta_subtracted", "round_to_bf16(pv + bf16_bits_to_double(delta[t * H + h]))",
     "round_to_bf16(pv - bf16_bits_to_double(delta[t * H + h]))"),
    ("cur_source_missing", "memcpy(src + (int64_t)nb * H, cur, sizeof(double) * (size_t)H);",
     "memset(src + (int64_t)nb * H, 0, sizeof(double) * (size_t)H);"),
    ("output_norm_weight_dropped", "y[h] = xhat[h] * bf16_bits_to_double(onw[h]);", "y[h] = xhat[h];"),
    ("output_norm_skipped", "        if (onw) {\n            rms_normalise(y, H, out_eps, xhat);",
     "        if (0) {\n            rms_normalise(y, H, out_eps, xhat);"),
    ("prefix_not_written", "prefix[t * H + h] = bf16_value_to_bits(cur[h]);", "(void)h;"),
    ("bank_gets_output", "row[h] = bf16_value_to_bits(cur[h]);",
     "row[h] = bf16_value_to_bits(round_to_bf16(y[h]));"),
    ("write_ignores_token", "blocks + t * token_stride + (int64_t)widx * slot_stride",
     "blocks + (int64_t)widx * slot_stride"),
    ("write_before_read", "        /* Gather sources in order (R6), all read before any write (R5). */\n",
     "        if (widx >= 0) for (int64_t h = 0; h < H; ++h)\n"
     "            blocks[t * token_stride + (int64_t)widx * slot_stride + h] = bf16_value_to_bits(cur[h]);\n"),
    ("rounding_ties_away", "ldexp(nearbyint(ldexp(x, -qexp)), qexp)", "ldexp(round(ldexp(x, -qexp)), qexp)"),
    ("rounding_7_bits", "int qexp = e - 8;", "int qexp = e - 7;"),
    ("rounding_via_float", "    double y = ldexp(nearbyint(ldexp(x, -qexp)), qexp);",
     "    x = (double)(float)x;\n    double y = ldexp(nearbyint(ldexp(x, -qexp)), qexp);"),
    ("gather_ignores_token", "blocks + t * token_stride + (int64_t)j * slot_stride",
     "blocks + (int64_t)j * slot_stride"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = src.replace(old, new)
    c = tmp_path / "mutant.c"
    c.write_text(mutant)
    so = tmp_path / f"mutant_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-w", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    lib = O.load_library(str(so))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin detects the planted mistake {name!r}"
