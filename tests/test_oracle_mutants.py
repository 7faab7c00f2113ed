"""Plausible mistakes planted in copies of the oracle must each fail a pin.

Each mutant is the oracle's C source with one textual change (a dropped term,
a wrong order, index or offset, a flushed sign), compiled to a temporary
library on the CPU.  The pins of tests/oracle_pins.py run against it and at
least one must fail; the unmodified oracle passes all of them
(test_oracle.py).  The mutants only ever run on the host.
"""
import os
import subprocess

import pytest

from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "tide_oracle.c")

MUTANTS = [
    ("drop_last_rank",
     "for (int32_t u = 1; u < g->W; ++u) acc = acc +",
     "for (int32_t u = 1; u < g->W - 1; ++u) acc = acc +"),
    ("reverse_rank_order",
     "float acc = bf16_to_f32(j->grads[(int64_t)0 * g->P + p][i]);\n"
     "            for (int32_t u = 1; u < g->W; ++u) acc = acc + bf16_to_f32(j->grads[(int64_t)u * g->P + p][i]);",
     "float acc = bf16_to_f32(j->grads[(int64_t)(g->W - 1) * g->P + p][i]);\n"
     "            for (int32_t u = g->W - 2; u >= 0; --u) acc = acc + bf16_to_f32(j->grads[(int64_t)u * g->P + p][i]);"),
    ("accumulator_starts_at_plus_zero",
     "float acc = bf16_to_f32(j->grads[(int64_t)0 * g->P + p][i]);",
     "float acc = 0.0f + bf16_to_f32(j->grads[(int64_t)0 * g->P + p][i]);"),
    ("double_accumulator",
     "float acc = bf16_to_f32(", "double acc = bf16_to_f32("),
    ("floor_rows_per_rank",
     "int64_t R = (D + W - 1) / W;", "int64_t R = D / W;"),
    ("landing_pitch_uses_row_length",
     "landing_offset[(int64_t)p * W + r] = (int64_t)W * g.o[p] + (int64_t)r * g.n[p];",
     "landing_offset[(int64_t)p * W + r] = (int64_t)W * g.o[p] + (int64_t)r * g.K[p];"),
    ("rank_major_offset_drops_prefix",
     "rank_major_offset[(int64_t)p * W + r] = (int64_t)r * g.S + g.o[p];",
     "rank_major_offset[(int64_t)p * W + r] = (int64_t)r * g.S;"),
    ("copyout_source_drops_prefix",
     "const uint16_t* src = j->rank_major + (int64_t)r * g->S + g->o[p];",
     "const uint16_t* src = j->rank_major + (int64_t)r * g->S;"),
    ("copyout_destination_uses_real_count",
     "uint16_t* dst = j->params[p] + (int64_t)r * g->R[p] * g->K[p];",
     "uint16_t* dst = j->params[p] + (int64_t)r * real;"),
    ("rs_padding_negative_zero",
     "dst[e] = 0.0f;", "dst[e] = -0.0f;"),
    ("pack_padding_not_zero",
     "(e < real) ? src[e] : (uint16_t)0;", "(e < real) ? src[e] : (uint16_t)0x8000;"),
    ("row_length_drops_last_dim",
     "for (int32_t j = 1; j < ndims[p]; ++j) {", "for (int32_t j = 1; j < ndims[p] - 1; ++j) {"),
    ("cast_rounds_half_up",
     "return (uint16_t)((u + 0x7FFFu + keep_odd) >> 16);", "return (uint16_t)((u + 0x8000u) >> 16);"),
    ("cast_truncates",
     "return (uint16_t)((u + 0x7FFFu + keep_odd) >> 16);", "return (uint16_t)((u + 0u * keep_odd) >> 16);"),
    ("cast_nan_not_quieted",
     "if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);",
     "if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(u >> 16);"),
    ("copyin_padding_not_zero",
     "        if (e >= real) {\n            dst[e] = 0;", "        if (e >= real) {\n            dst[e] = 0x8000;"),
    ("copyin_wrong_destination_rank",
     "uint16_t* dst = j->rank_major_out + (int64_t)r * g->S + g->o[p];\n    const void* src = j->shards",
     "uint16_t* dst = j->rank_major_out + (int64_t)(g->W - 1 - r) * g->S + g->o[p];\n    const void* src = j->shards"),
    ("alpha_dropped",
     "float v = j->alpha * sum;", "float v = sum;"),
    ("accumulate_ignored",
     "dst[e] = j->accumulate ? dst[e] + v : v;", "dst[e] = v;"),
    ("fp32_grads_read_as_bf16",
     "if (j->grad_dtype == 1) return ((const float*)t)[i];", "if (j->grad_dtype == 2) return ((const float*)t)[i];"),
    ("chunk_cat_padding_not_zero",
     "dst[e] = (e < real) ? bf16_to_f32(src[e]) : 0.0f;", "dst[e] = (e < real) ? bf16_to_f32(src[e]) : 1.0f;"),
    ("chunk_cat_rows_of_wrong_rank",
     "const uint16_t* src = j->grads_one[p] + (int64_t)r * g->R[p] * g->K[p];",
     "const uint16_t* src = j->grads_one[p] + (int64_t)(r > 0 ? r - 1 : 0) * g->R[p] * g->K[p];"),
    ("rs_source_row_offset_uses_real_count",
     "int64_t first = (int64_t)r * g->R[p] * g->K[p];\n    float* dst = j->out[r] + g->o[p];\n"
     "    for (int64_t e = 0; e < g->n[p]; ++e) {\n        if (e < real) {",
     "int64_t first = (int64_t)r * real;\n    float* dst = j->out[r] + g->o[p];\n"
     "    for (int64_t e = 0; e < g->n[p]; ++e) {\n        if (e < real) {"),
    ("general_source_row_offset_uses_real_count",
     "int64_t first = (int64_t)r * g->R[p] * g->K[p];\n    float* dst = j->out[r] + g->o[p];\n"
     "    for (int64_t e = 0; e < g->n[p]; ++e) {\n        float sum",
     "int64_t first = (int64_t)r * real;\n    float* dst = j->out[r] + g->o[p];\n"
     "    for (int64_t e = 0; e < g->n[p]; ++e) {\n        float sum"),
    ("accumulate_fused",
     "float v = j->alpha * sum;\n        dst[e] = j->accumulate ? dst[e] + v : v;",
     "float v = j->alpha * sum;\n        dst[e] = j->accumulate ? fmaf(j->alpha, sum, dst[e]) : v;"),
    ("padding_sum_not_scaled",
     "float v = j->alpha * sum;", "float v = (sum == 0.0f) ? sum : j->alpha * sum;"),
    ("axpb_fused",
     "volatile float prod = a * x[i]; /* one rounding, kept apart from the sum */\n        y[i] = prod + b;",
     "y[i] = fmaf(a, x[i], b);"),
    ("axpb_flushes_subnormals",
     "unsigned saved = ieee_mode_enter();\n    for (int64_t i = 0; i < n; ++i) {\n        volatile float prod",
     "unsigned saved = _mm_getcsr();\n    _mm_setcsr(saved | 0x8040u);\n    for (int64_t i = 0; i < n; ++i) {\n"
     "        volatile float prod"),
]


def _build(tmp_path, name, old, new):
    src = open(SOURCE).read()
    assert src.count(old) == 1, f"mutant {name}: pattern must occur once in the oracle source"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    "-fno-fast-math", str(path), "-o", str(lib)], check=True)
    return str(lib)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, name, old, new, oracle_mod):
    orc = oracle_mod.Oracle(_build(tmp_path, name, old, new))
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, oracle_mod.OracleError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
