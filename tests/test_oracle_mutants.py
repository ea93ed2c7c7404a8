"""Planted mistakes in the CPU oracle must be caught by its pins.

Each mutant is a copy of oracle/lpc_oracle.c with one plausible mistake
(a wrong tie rule, a dropped rank, a wrong index, an FMA, FNUZ's 240 in place
of 448, ...), compiled with gcc into a temporary directory and loaded as a
separate oracle.  The test runs the pins on it and requires at least one to
fail.  Nothing here touches a GPU.
"""
import os
import shutil

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "lpc_oracle.c")

MUTANTS = {
    "tie_away_from_even": ("pick = (k % 2 == 0) ? k : k + 1;", "pick = k + 1;"),
    "tie_toward_zero": ("pick = (k % 2 == 0) ? k : k + 1;", "pick = k;"),
    "sign_by_comparison": ("uint8_t sign = signbit(v) ? 0x80 : 0x00;",
                           "uint8_t sign = (v < 0) ? 0x80 : 0x00;"),
    "fnuz_max_240": ("#define LPO_FP8_MAX 448.0f", "#define LPO_FP8_MAX 240.0f"),
    "exponent_bias_off_by_one": ("v = ldexpf((float)(8 + m), e - 10);",
                                 "v = ldexpf((float)(8 + m), e - 9);"),
    "subnormal_step_wrong": ("v = ldexpf((float)m, -9);", "v = ldexpf((float)m, -10);"),
    "overflow_to_nan": ("    if (a >= LPO_FP8_MAX)\n        return (uint8_t)(sign | 0x7E);",
                        "    if (a >= 464.0f)\n        return (uint8_t)(sign | 0x7F);"),
    "reciprocal_multiply": ("float q = x[i] / s;", "float q = x[i] * (1.0f / s);"),
    "signed_max_not_absmax": ("float a = fabsf(x[i]);\n        if (a > amax)",
                              "float a = x[i];\n        if (a > amax)"),
    "zero_test_on_amax": ("    if (s == 0.0f) {\n        *scale = 0.0f;",
                          "    if (amax == 0.0f) {\n        *scale = 0.0f;"),
    "bf16_widen_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "rs_drops_last_rank": ("            for (p = 1; p < nranks; p++) {\n"
                           "                float d = lpo_e4m3_decode(codes[p][base + i])",
                           "            for (p = 1; p < nranks - 1; p++) {\n"
                           "                float d = lpo_e4m3_decode(codes[p][base + i])"),
    "rs_fused_multiply_add": ("                acc[i] = acc[i] + d;",
                              "                acc[i] = fmaf(lpo_e4m3_decode(codes[p][base + i]), "
                              "scales[p][gblk], acc[i]); (void)d;"),
    "rs_ignores_chunk_offset": ("size_t base = (size_t)rank * C + b * LPO_BLOCK;",
                                "size_t base = b * LPO_BLOCK;"),
    "rs_chunk_local_scale_index": ("size_t gblk = base / LPO_BLOCK;", "size_t gblk = b;"),
    "rs_out_skips_rank0": ("        float acc = lpo_e4m3_decode(codes[0][e]) * scales[0][e / LPO_BLOCK];",
                           "        float acc = 0.0f;"),
    "ag_first_scale_only": ("float v = lpo_e4m3_decode(chunk_codes[p][i]) * chunk_scales[p][i / LPO_BLOCK];",
                            "float v = lpo_e4m3_decode(chunk_codes[p][i]) * chunk_scales[p][0];"),
    "ag_chunk_order_swapped": ("((float *)out)[(size_t)p * C + i] = v;",
                               "((float *)out)[(size_t)(nranks - 1 - p) * C + i] = v;"),
    "bf16_ties_up": ("if (rest > 0x8000 || (rest == 0x8000 && (down & 1)))", "if (rest >= 0x8000)"),
    "bf16_truncates": ("if (rest > 0x8000 || (rest == 0x8000 && (down & 1)))", "if (0)"),
    "dda_skips_rank1": ("        for (p = 1; p < nranks; p++)\n            acc = acc + lpo_bf16_to_f32(bufs[p][i]);",
                        "        for (p = 2; p < nranks; p++)\n            acc = acc + lpo_bf16_to_f32(bufs[p][i]);"),
    "dda_tree_fp32_wrong_start": ("            acc = ((const float *)bufs[0])[e];",
                                  "            acc = ((const float *)bufs[1])[e];"),
    "route_not_stable": ("        for (k = 0; k < rows; k++)\n            if (dest[k] == d)",
                         "        for (k = rows; k-- > 0;)\n            if (dest[k] == d)"),
    "route_inclusive_offsets": ("        offsets[d] = (int32_t)pos;\n        pos += (size_t)counts[d];",
                                "        pos += (size_t)counts[d];\n        offsets[d] = (int32_t)pos;"),
    "rows_not_gathered": ("size_t src = (size_t)perm[k];", "size_t src = k;"),
    "rows_f32_half_stride": ("lpo_quantize_f32((const float *)x + src * row_len, row_len,",
                             "lpo_quantize_f32((const float *)x + src * (row_len / 2), row_len,"),
    "rs_out_bf16_truncates": ("            ((uint16_t *)out)[i] = lpo_bf16_rne(acc);\n        else\n"
                              "            ((float *)out)[i] = acc;",
                              "            { uint32_t u_; memcpy(&u_, &acc, 4); ((uint16_t *)out)[i] = (uint16_t)(u_ >> 16); }\n"
                              "        else\n"
                              "            ((float *)out)[i] = acc;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site for %s not unique in the oracle source" % name
    src = tmp_path / ("lpc_oracle_%s.c" % name)
    src.write_text(text.replace(old, new))
    lib = oracle.build(force=True, src=str(src), lib=str(tmp_path / ("lib_%s.so" % name)))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError) as e:  # noqa: PERF203
            caught.append((pin.__name__, e))
            break
    assert caught, "no pin rejects the planted mistake %r" % name
    shutil.rmtree(tmp_path, ignore_errors=True)
