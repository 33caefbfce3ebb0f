"""Plants one plausible mistake at a time in a copy of oracle.c (on the CPU) and
checks that the pins in pins.py catch every one of them."""
import os

import pytest

import oracle
from pins import ALL_CHECKS

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("inner_chain_unfused", "ab[L] = fmaf(d1, (float)s, ab[L]);", "ab[L] = d1 * (float)s + ab[L];"),
    ("first_product_fused_with_zero", "ab[L] = d1 * (float)s;", "ab[L] = d1 * (float)s * 1.0000001f;"),
    ("outer_step_unfused", "acc[L] = fmaf(d0, ab[L], acc[L]);", "acc[L] = d0 * ab[L] + acc[L];"),
    ("tree_left_to_right",
     "return ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));",
     "return acc[0] + acc[1] + acc[2] + acc[3] + acc[4] + acc[5] + acc[6] + acc[7];"),
    ("tree_adjacent_pairs",
     "return ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));",
     "return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));"),
    ("lanes_stride_8", "int k = 32 * j + 4 * L + i; /* weight index inside the block */",
     "int k = 32 * j + 8 * i + L;"),
    ("no_int8_wrap", "return qv == -128 ? -128 : -(int32_t)qv;", "return -(int32_t)qv;"),
    ("bit_order_msb_first", "int bit = (qs[k >> 3] >> (k & 7)) & 1;", "int bit = (qs[k >> 3] >> (7 - (k & 7))) & 1;"),
    ("sign_map_inverted", "int bit = (qs[k >> 3] >> (k & 7)) & 1;", "int bit = !((qs[k >> 3] >> (k & 7)) & 1);"),
    ("act_scale_per_block", "float d1 = d[e0 / qa];", "float d1 = d[b];"),
    ("scale_bytes_swapped", "float d0 = oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));",
     "float d0 = oracle_f16_to_f32((uint16_t)(blk[1] | (blk[0] << 8)));"),
    ("last_block_dropped", "for (int64_t b = 0; b < nb; ++b) {", "for (int64_t b = 0; b + 1 < nb; ++b) {"),
    ("q2_code_map_reversed", "s += (code - 1) * (int32_t)q[e0 + 4 * L + i];", "s += (1 - code) * (int32_t)q[e0 + 4 * L + i];"),
    ("q2_code_offset_wrong", "s += (code - 1) * (int32_t)q[e0 + 4 * L + i];", "s += code * (int32_t)q[e0 + 4 * L + i];"),
    ("q2_code3_decoded_as_zero", "s += (code - 1) * (int32_t)q[e0 + 4 * L + i];",
     "s += (code == 3 ? 0 : code - 1) * (int32_t)q[e0 + 4 * L + i];"),
    ("q2_code_shift_wrong", "int code = (qs[k >> 2] >> (2 * (k & 3))) & 3;", "int code = (qs[k >> 2] >> (k & 3)) & 3;"),
    ("quant_round_half_even", "float r = roundf(xb[i] / db);", "float r = rintf(xb[i] / db);"),
    ("quant_divisor_128", "float db = amax / 127.0f;", "float db = amax / 128.0f;"),
    ("quant_multiply_by_reciprocal", "float r = roundf(xb[i] / db);", "float r = roundf(xb[i] * (1.0f / db));"),
    ("f16_subnormal_wrong", "v = ldexpf((float)m, -24);", "v = ldexpf((float)m, -25);"),
    ("f16_narrow_truncates", "float m = rintf(ldexpf(a, 11 - e));", "float m = floorf(ldexpf(a, 11 - e));"),
    ("f16_narrow_ties_away", "float m = rintf(ldexpf(a, 11 - e));", "float m = roundf(ldexpf(a, 11 - e));"),
    ("f16_narrow_subnormal_grid", "return sign | (uint16_t)rintf(ldexpf(a, 24));",
     "return sign | (uint16_t)rintf(ldexpf(a, 23));"),
    ("f16_narrow_overflow_early", "if (a >= 65520.0f)", "if (a >= 65504.0f)"),
    ("quant_f16_scale_ignored", "db = oracle_f16_to_f32(oracle_f32_to_f16(db)); /* reading R6 */", "db = db;"),
    ("f16_bias_wrong", "v = ldexpf((float)(1024 + m), e - 25);", "v = ldexpf((float)(1024 + m), e - 24);"),
    ("acc_starts_at_minus_zero_sign_flip", "acc[L] = 0.0f;\n    for (int64_t b = 0; b < nb; ++b) {\n        const uint8_t *blk = blocks + b * ORACLE_BLOCK_BYTES;\n        float d0 = oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));\n        const uint8_t *qs = blk + 2;\n        float ab[8];\n        for (int j = 0; j < 4; ++j) {",
     "acc[L] = 0.0f;\n    for (int64_t b = 0; b < nb; ++b) {\n        const uint8_t *blk = blocks + b * ORACLE_BLOCK_BYTES;\n        float d0 = -oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));\n        const uint8_t *qs = blk + 2;\n        float ab[8];\n        for (int j = 0; j < 4; ++j) {"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new, 1))
    lib = oracle.build(str(path), str(tmp_path / f"lib{name}.so"))
    o = oracle.Oracle(lib)
    caught = []
    for check_name, check in ALL_CHECKS:
        try:
            check(o)
        except AssertionError:
            caught.append(check_name)
    assert caught, f"mutant {name} passed every pin"
