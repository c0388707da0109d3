"""The oracle's pins must bite: plant plausible mistakes in copies of the
oracle (on the CPU) and check that each one makes at least one pin fail."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qgemm_oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_int4.py", "test_oracle_int8.py",
                                                 "test_oracle_w4a8_g32.py", "test_oracle_int4_dq.py",
                                                 "test_oracle_intn.py")]

# (id, original text, planted text): each is a single, plausible slip.
MUTANTS = [
    ("add_then_round", "rintf(v[i] / s) + z", "rintf(v[i] / s + z)"),
    ("range_not_widened_to_zero", "float lo = 0.0f, hi = 0.0f;", "float lo = INFINITY, hi = -INFINITY;"),
    ("scale_one_ulp_small", "sbits = smallest_fp16_covering(r, (double)levels);",
     "sbits = smallest_fp16_covering(r, (double)levels) - 1;"),
    ("zero_point_sign", "rintf(-lo / s)", "rintf(lo / s)"),
    ("half_away_rounding", "float t = rintf(v[i] / s) + z;", "float t = roundf(v[i] / s) + z;"),
    ("nibble_order_linear", "(e & 1) * 4 + (e >> 1)", "e"),
    ("chunk_index_transposed", "(j * T_ROWS + r) * 16", "(r * T_GROUPS + j) * 16"),
    ("scale_bytes_swapped", "(uint8_t)(s & 0xFF);", "(uint8_t)(s >> 8);"),
    ("zero_nibble_swapped", "(uint8_t)((zeros[row * groups + g] & 0xF) << ((j % 2) * 4));",
     "(uint8_t)((zeros[row * groups + g] & 0xF) << ((1 - j % 2) * 4));"),
    ("dequant_sign", "(double)(q - z) * s", "(double)(z - q) * s"),
    ("scale_of_neighbour_group", "double s = orc_fp16_to_double(c->scales[row * groups + g]);",
     "double s = orc_fp16_to_double(c->scales[row * groups + (g ^ 1)]);"),
    ("activation_row_ignored", "acc += orc_bf16_to_double(c->x[mi * c->k + kk]) * wdq;",
     "acc += orc_bf16_to_double(c->x[kk]) * wdq;"),
    ("w8_scale_dropped", "c->y[mi * c->n + row] = acc * orc_bf16_to_double(c->scales[row]);",
     "c->y[mi * c->n + row] = acc;"),
    ("w8_weight_transposed", "(double)c->w[row * c->k + kk]", "(double)c->w[kk * c->n + row]"),
    ("int8_scale_one_ulp_big", "smallest_bf16_covering(amax, 127.0)", "(smallest_bf16_covering(amax, 127.0) + 1)"),
    ("actquant_128_levels", "float inv = 127.0f / a;", "float inv = 128.0f / a;"),
    ("actquant_non_finite_ignored", "if (!isfinite(v)) finite = 0;", "if (0) finite = 0;"),
    ("actquant_tiny_span_kept", "if (isinf(inv)) {", "if (0) {"),
    ("w4a8_zero_point_dropped", "(int64_t)(c->codes[row * c->k + kk] - z)", "(int64_t)(c->codes[row * c->k + kk])"),
    ("w4a8_act_scale_dropped", "c->y[mi * c->n + row] = (double)c->sx[mi] * acc;", "c->y[mi * c->n + row] = acc;"),
    ("g32_first_group_scale_for_all", "(double)c->sx[mi * groups + g] *", "(double)c->sx[mi * groups] *"),
    ("g32_groups_of_the_row_scale", "quant_span(x + mi * k + g * 32, 32, xq + mi * k + g * 32, sx + mi * groups + g);",
     "{ quant_span(x + mi * k + g * 32, 32, xq + mi * k + g * 32, sx + mi * groups + g); "
     "if (g) sx[mi * groups + g] = sx[mi * groups]; }"),
    ("g32_zero_point_of_next_group", "int zg = c->zeros[row * groups + g];",
     "int zg = c->zeros[row * groups + (g + 1) % groups];"),
    ("g32_span_shifted", "quant_span(x + mi * k + g * 32, 32,", "quant_span(x + mi * k + g * 32 + (g > 0), 32,"),
    ("dq_code_rounded_to_nearest", "while (c < 255 && 15.0 * c * ds < r) c++;",
     "while (c < 255 && 15.0 * c * ds < r) c++; "
     "if (c > 1 && r - 15.0 * (c - 1) * ds < 15.0 * c * ds - r) c--;"),
    ("dq_step_without_the_15", "smallest_fp16_covering(rmax, 3825.0)", "smallest_fp16_covering(rmax, 255.0)"),
    ("dq_code_may_be_zero", "int c = 1;", "int c = 0;"),
    ("dq_head_bytes_swapped", "block[2 * r] = (uint8_t)(sstep[row] & 0xFF);",
     "block[2 * r] = (uint8_t)(sstep[row] >> 8);"),
    ("dq_scale_code_transposed", "tile[D_SCODE_OFF + r * 8 + j] = scode[row * groups + g];",
     "tile[D_SCODE_OFF + j * 64 + r] = scode[row * groups + g];"),
    ("intn_levels_off_by_one", "return quantize_group_levels(w32, (1 << bits) - 1, scale, zp, q32);",
     "return quantize_group_levels(w32, (1 << bits), scale, zp, q32);"),
    ("int5_plane_pair_and_dword_swapped", "if (hb == 1) return 16 * odd + 4 * d + p;",
     "if (hb == 1) return 16 * odd + 4 * p + d;"),
    ("int6_plane_bit_and_pair_swapped", "8 * (d % 2) + 2 * p + b;", "8 * (d % 2) + 4 * b + p;"),
    ("intn_zero_bytes_swapped", "tile[z_off + r * 8 + j] = zeros[row * groups + g];",
     "tile[z_off + r * 8 + (j ^ 1)] = zeros[row * groups + g];"),
    ("intn_scales_at_the_v1_offset", "int64_t hi_off = 8192, s_off = 8192 + 2048 * hb, z_off = s_off + 1024;",
     "int64_t hi_off = 8192, s_off = 8192 + 1024 * hb, z_off = s_off + 1024;"),
    ("dq_w4a8_row_scale_dropped", "c->y[mi * c->n + row] = c->per_group ? acc : (double)c->sx[mi] * acc;",
     "c->y[mi * c->n + row] = acc;"),
    ("dq_w4a8_scale_code_of_group_0", "double s = (double)c->scode[row * groups + g] * step;",
     "double s = (double)c->scode[row * groups] * step;"),
    ("dq_gemm_step_of_row_0", "double step = orc_fp16_to_double(c->sstep[row]);",
     "double step = orc_fp16_to_double(c->sstep[0]);"),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("mid,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant_dir, mid, orig, planted):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutation site for {mid} not found"
    bad = src.replace(orig, planted, 1)
    csrc = os.path.join(mutant_dir, f"{mid}.c")
    lib = os.path.join(mutant_dir, f"{mid}.so")
    with open(csrc, "w") as fh:
        fh.write(bad)
    subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    "-I", os.path.join(ROOT, "oracle"), csrc, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, QGEMM_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"no pin failed for planted mistake {mid}:\n{r.stdout[-2000:]}"
