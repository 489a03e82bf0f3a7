"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one.  Each mutant is a single textual edit of oracle.cpp,
compiled into a temporary library; the real oracle is never modified."""
import os

import pytest

import oracle
import oracle_checks as K

MUTANTS = {
    # layout: wrong expert -> group mapping (divide by the group count)
    "group_index": ("bits |= 1u << (id / experts_per_group);", "bits |= 1u << (id / G);"),
    # layout: a bad id is not reported
    "no_bad_id_status": ("if (id != -1 && !routed(id, E)) st |= ORACLE_ERR_BAD_EXPERT;",
                         "if (id < -1) st |= ORACLE_ERR_BAD_EXPERT;"),
    # layout: repeats within a token are not reported
    "no_dup_status": ("if (topk_idx[(int64_t)t * k + jj] == id) st |= ORACLE_ERR_DUP_EXPERT;",
                      "if (topk_idx[(int64_t)t * k + jj] == id + E) st |= ORACLE_ERR_DUP_EXPERT;"),
    # layout: group count taken from bit g+1
    "group_count_shift": ("c += (int32_t)((is_token_in_group[t] >> g) & 1u);",
                          "c += (int32_t)((is_token_in_group[t] >> (g + 1)) & 1u);"),
    # dispatch: inclusive instead of exclusive offsets reported
    "inclusive_offsets": ("expert_offsets[e] = (int32_t)run;", "expert_offsets[e] = (int32_t)(run + c);"),
    # dispatch: slot-major instead of token-major receive order
    "slot_major_order": ("    for (int t = 0; t < T; ++t) {\n        for (int j = 0; j < k; ++j) {\n            int64_t s",
                         "    for (int j = 0; j < k; ++j) {\n        for (int t = 0; t < T; ++t) {\n            int64_t s"),
    # dispatch: source index off by one
    "src_off_by_one": ("recv_src_idx[r] = t;", "recv_src_idx[r] = t + 1;"),
    # dispatch: weight of the token's first slot for every copy
    "weight_wrong_slot": ("recv_weights[r] = topk_weights[s];", "recv_weights[r] = topk_weights[(int64_t)t * k];"),
    # dispatch: the row copy takes the wrong token
    "row_wrong_token": ("memcpy(recv_x + r * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);",
                        "memcpy(recv_x + r * row_bytes, x + (int64_t)(T - 1 - t) * row_bytes, (size_t)row_bytes);"),
    # combine: last slot dropped
    "drop_last_slot": ("            for (int j = 0; j < k; ++j) {\n                int32_t r = slot_to_row",
                       "            for (int j = 0; j + 1 < k; ++j) {\n                int32_t r = slot_to_row"),
    # combine: sign error on the weight
    "weight_sign": ("acc = fmaf(recv_weights[r], v, acc);", "acc = fmaf(-recv_weights[r], v, acc);"),
    # combine: accumulator dropped (keeps only the last term)
    "no_accumulate": ("acc = fmaf(recv_weights[r], v, acc);", "acc = fmaf(recv_weights[r], v, 0.0f);"),
    # combine: weight ignored
    "weight_ignored": ("acc = fmaf(recv_weights[r], v, acc);", "acc = acc + v;"),
    # bf16 rounding: truncation instead of nearest-even
    "bf16_truncate": ("double r = rint(d / spacing) * spacing;", "double r = floor(d / spacing) * spacing;"),
    # bf16 rounding: one bit too many kept
    "bf16_spacing": ("double spacing = ldexp(1.0, p - 8);", "double spacing = ldexp(1.0, p - 9);"),
    # bf16 rounding: subnormal spacing wrong
    "bf16_subnormal": ("if (p < -125) p = -125;", "if (p < -126) p = -126;"),
    # E4M3: truncation instead of nearest-even
    "e4m3_truncate": ("double r = rint(a / spacing) * spacing;", "double r = floor(a / spacing) * spacing;"),
    # E4M3: ties away from zero instead of to even
    "e4m3_ties_away": ("double r = rint(a / spacing) * spacing;", "double r = round(a / spacing) * spacing;"),
    # E4M3: exponent bias 8 in the decoder
    "e4m3_bias": ("mag = ldexp(1.0 + f / 8.0, e - 7);", "mag = ldexp(1.0 + f / 8.0, e - 8);"),
    # E4M3: two fraction bits kept instead of three
    "e4m3_spacing": ("double spacing = ldexp(1.0, lo - 3);", "double spacing = ldexp(1.0, lo - 2);"),
    # E4M3: subnormal range ends one binade too low
    "e4m3_subnormal": ("if (lo < -6) lo = -6;", "if (lo < -7) lo = -7;"),
    # E4M3: overflow gives NaN instead of saturating
    "e4m3_no_saturation": ("if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
                           "if (a >= 464.0) return (uint8_t)(sign | 0x7F);"),
    # E4M3: sign dropped
    "e4m3_sign": ("uint8_t sign = signbit(v) ? 0x80 : 0x00;", "uint8_t sign = v < 0 ? 0x80 : 0x00;"),
    # FP32 scales: wrong format maximum
    "scale_max_240": ("float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
                      "float scale = amax > 0.0f ? amax / 240.0f : 1.0f;"),
    # FP32 scales: all-zero block gets scale 0
    "scale_zero_block": ("float scale = amax > 0.0f ? amax / 448.0f : 1.0f;",
                         "float scale = amax > 0.0f ? amax / 448.0f : 0.0f;"),
    # amax of signed values instead of magnitudes
    "amax_signed": ("float m = fabsf((float)oracle_bf16_to_double(xb[i]));",
                    "float m = (float)oracle_bf16_to_double(xb[i]);"),
    # FP32 scales: multiply instead of divide
    "scale_multiply": ("float v = (float)oracle_bf16_to_double(xb[i]) / scale;",
                       "float v = (float)oracle_bf16_to_double(xb[i]) * scale;"),
    # UE8M0: one binade too large (<= instead of <)
    "ue8m0_off_by_one": ("while (s < 127 && ldexp(448.0, s) < (double)amax) ++s;",
                         "while (s < 127 && ldexp(448.0, s) <= (double)amax) ++s;"),
    # UE8M0: no clamp at code zero (tiny blocks flushed)
    "ue8m0_no_low_clamp": ("    int s = -127;\n", "    int s = -150;\n"),
    # UE8M0: scaling in the wrong direction
    "ue8m0_direction": ("float v = ldexpf((float)oracle_bf16_to_double(xb[i]), -sx);",
                        "float v = ldexpf((float)oracle_bf16_to_double(xb[i]), sx);"),
    # UE8M0: bias 128 in the scale byte
    "ue8m0_bias": ("scales[(int64_t)t * nb + b] = (uint8_t)(sx + 127);",
                   "scales[(int64_t)t * nb + b] = (uint8_t)(sx + 128);"),
    # quantiser: block offset forgotten (every block reads the first)
    "quant_block_offset": ("const uint16_t* xb = x + (int64_t)t * H + (int64_t)b * B;",
                           "const uint16_t* xb = x + (int64_t)t * H;"),
    # group dispatch: group membership taken from the neighbouring bit
    "group_bit": ("run += (is_token_in_group[t] >> g) & 1u;", "run += (is_token_in_group[t] >> (g + 1)) & 1u;"),
    # group dispatch: restricted slots keep every expert
    "group_no_restrict": ("int here = routed(id, E) && id / experts_per_group == g;", "int here = routed(id, E);"),
    # group dispatch: weights of other groups' slots kept
    "group_weights_kept": ("recv_topk_weights[r * k + j] = here ? topk_weights[(int64_t)t * k + j] : 0.0f;",
                           "recv_topk_weights[r * k + j] = topk_weights[(int64_t)t * k + j];"),
    # group dispatch: row of (t, g) recorded one too high
    "group_row_off_by_one": ("token_group_row[(int64_t)t * G + g] = (int32_t)r;",
                             "token_group_row[(int64_t)t * G + g] = (int32_t)(r + 1);"),
    # group combine: the last group dropped
    "group_combine_drop": ("            for (int g = 0; g < G; ++g) {\n                int32_t r = token_group_row",
                           "            for (int g = 0; g + 1 < G; ++g) {\n                int32_t r = token_group_row"),
    # padded layout: one slot too many kept per expert
    "padded_capacity": ("if (i >= C) {", "if (i > C) {"),
    # padded layout: this source's first row inside the slab ignored
    "padded_no_base": ("int64_t q = (int64_t)id * S + B + i;", "int64_t q = (int64_t)id * S + i;"),
    # padded layout: slabs spaced by the capacity instead of the stride
    "padded_stride": ("int64_t q = (int64_t)id * S + B + i;", "int64_t q = (int64_t)id * C + B + i;"),
    # padded layout: overflow not reported
    "padded_no_status": ("st |= ORACLE_ERR_OVERFLOW;", "st |= 0;"),
    # combine: slots summed in descending order
    "combine_reverse_order": ("            for (int j = 0; j < k; ++j) {\n                int32_t r = slot_to_row",
                              "            for (int j = k - 1; j >= 0; --j) {\n                int32_t r = slot_to_row"),
    # combine: the product rounded to fp32 before the add (no fused multiply-add)
    "combine_no_fma": ("acc = fmaf(recv_weights[r], v, acc);",
                       "{ volatile float p = recv_weights[r] * v; acc = acc + p; }"),
    # group combine: groups summed in descending order
    "group_combine_reverse": ("            for (int g = 0; g < G; ++g) {\n                int32_t r = token_group_row",
                              "            for (int g = G - 1; g >= 0; --g) {\n                int32_t r = token_group_row"),
    # layout: a count set instead of incremented
    "layout_count_assign": ("if (routed(id, E)) tokens_per_expert[id] += 1;",
                            "if (routed(id, E)) tokens_per_expert[id] = 1;"),
    # dispatch: fp8 scales not moved with the rows
    "dispatch_scales_dropped": ("memcpy(recv_x + r * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);\n"
                                "            if (x_scales && recv_scales && scale_row_bytes > 0)",
                                "memcpy(recv_x + r * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);\n"
                                "            if (0)"),
    # group dispatch: the group rows' total one short
    "group_total_off": ("    group_offsets[G] = (int32_t)run;", "    group_offsets[G] = (int32_t)(run - 1);"),
    # group dispatch: wrong source token recorded
    "group_src_idx": ("recv_src_idx[r] = (int32_t)t;", "recv_src_idx[r] = (int32_t)(T - 1 - t);"),
    # padded layout: the token's first weight for every copy
    "padded_weight_slot": ("recv_weights[q] = topk_weights[s];", "recv_weights[q] = topk_weights[(int64_t)t * k];"),
    # quantised dispatch: the scales are not moved with the rows
    "quant_scales_dropped": ("st = oracle_dispatch(T, k, E, H, scale_bytes, q, sc, topk_idx",
                             "st = oracle_dispatch(T, k, E, H, scale_bytes, q, NULL, topk_idx"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} must occur exactly once"
    path = os.path.join(tmp_path, "mutant.cpp")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.compile_oracle(path, os.path.join(tmp_path, f"libmutant_{name}.so"))
    orc = oracle.Oracle(lib)
    with pytest.raises(AssertionError):
        K.run_all(orc)


def test_unmutated_oracle_passes_all_pins(orc):
    K.run_all(orc)
