"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one.  Each mutant is a single textual edit of oracle.c,
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
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} must occur exactly once"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.compile_oracle(path, os.path.join(tmp_path, f"libmutant_{name}.so"))
    orc = oracle.Oracle(lib)
    with pytest.raises(AssertionError):
        K.run_all(orc)


def test_unmutated_oracle_passes_all_pins(orc):
    K.run_all(orc)
