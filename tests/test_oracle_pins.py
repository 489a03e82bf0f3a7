"""Pins of the CPU oracle (no GPU): library cast, brute force, invariants,
closed forms and a hand-worked example."""
import numpy as np
import pytest

from combine_ep_get_dispatch_amd import workloads as W
import oracle_checks as K


def test_bf16_rounding_matches_library_cast(orc):
    K.check_bf16_rounding(orc)


def test_bruteforce_every_tiny_routing(orc):
    K.check_bruteforce(orc)


def test_worked_example(orc):
    K.check_worked_example(orc)


def test_sum_order(orc):
    """Both combines' fp32 summation order (ascending slots by FMA, ascending
    groups), from hand-derived binary32 cases (tests/golden/sum_order.json)."""
    K.check_sum_order(orc)


def test_error_status_bits(orc):
    K.check_error_status(orc)


@pytest.mark.parametrize("i", range(5))
def test_layout_and_dispatch_invariants(orc, i):
    wl = K.small_configs()[i]
    K.check_layout_invariants(orc, wl)
    K.check_dispatch_invariants(orc, wl)


def test_combine_dyadic_weights_exact(orc):
    K.check_combine_exact_dyadic(orc)


def test_combine_k1_is_inverse_permutation(orc):
    K.check_combine_k1_inverse(orc)


def test_combine_round_trip_tiny_config(orc):
    K.check_combine_round_trip(orc, W.config(1))


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_combine_closed_forms(orc, i):
    wl = K.small_configs()[i]
    K.check_combine_closed_form(orc, wl, K.CLOSED_FORM_BOUND[wl.expert_kind])


def test_edge_shapes(orc):
    # T = 0; every slot masked; k = 1; G = 1; G = E; 16-byte rows
    cases = [
        W.make_workload("empty", 0, 8, 4, 2, 2, seed=1),
        W.make_workload("all_masked", 5, 8, 4, 2, 2, seed=2, mask_frac=1.0),
        W.make_workload("k1", 33, 8, 4, 2, 1, seed=3),
        W.make_workload("g1", 40, 8, 16, 1, 4, seed=4),
        W.make_workload("g_eq_e", 40, 8, 16, 16, 4, seed=5),
        W.make_workload("fp8_16B", 20, 128, 8, 2, 2, seed=6, x_dtype=W.X_FP8, scale_block=128),
    ]
    for wl in cases:
        K.check_layout_invariants(orc, wl)
        d = K.check_dispatch_invariants(orc, wl)
        if wl.name == "all_masked":
            assert d["expert_offsets"][-1] == 0
            eo = np.zeros((0, wl.H), np.uint16)
            of, ob = orc.combine(eo, d["recv_weights"][:0], d["slot_to_row"])
            assert np.all(of == 0) and np.all(ob == 0), "an all-masked token sums to +0"


def test_full_size_dispatch_invariants(orc):
    """The DeepSeek-V3-shaped workload at its real size (dispatch only)."""
    wl = W.config(2)
    K.check_layout_invariants(orc, wl)
    K.check_dispatch_invariants(orc, wl)


def test_e4m3_codes_match_library_decoding(orc):
    K.check_e4m3_codes(orc)


def test_e4m3_rounding_ties_and_saturation(orc):
    K.check_e4m3_rounding(orc)


@pytest.mark.parametrize("B", [32, 128])
def test_quant_fp32_scales(orc, B):
    K.check_quant_fp32(orc, B)


def test_quant_ue8m0_scales(orc):
    K.check_quant_ue8m0(orc, 32)


def test_quant_worked_example(orc):
    K.check_quant_example(orc)


@pytest.mark.parametrize("B,fmt", [(32, K.SCALE_FP32), (128, K.SCALE_FP32), (32, K.SCALE_UE8M0)])
def test_dispatch_quant_is_quantise_then_dispatch(orc, B, fmt):
    wl = W.make_workload("quant_mid", 300, 256, 64, 8, 6, seed=26, routing="zipf", mask_frac=0.05)
    K.check_dispatch_quant(orc, wl, B, fmt)


def test_group_dispatch_bruteforce_every_tiny_routing(orc):
    K.check_groups_bruteforce(orc)


def test_group_combine_exact_with_half_weights(orc):
    K.check_groups_combine_exact(orc)


@pytest.mark.parametrize("i", range(4))
def test_group_path_invariants_and_closed_form(orc, i):
    wl = K.group_configs()[i]
    K.check_groups_invariants(orc, wl)
    K.check_groups_combine_closed_form(orc, wl, K.GROUP_BOUND[wl.expert_kind])


def test_padded_worked_example(orc):
    K.check_padded_example(orc)


def test_padded_bruteforce_every_tiny_routing(orc):
    K.check_padded_bruteforce(orc)


@pytest.mark.parametrize("cid", [1, 4])
def test_padded_is_flat_shifted_per_expert(orc, cid):
    K.check_padded_vs_flat(orc, W.config(cid))


def test_padded_is_flat_shifted_per_expert_zipf(orc):
    K.check_padded_vs_flat(orc, W.make_workload("padded_zipf", 300, 64, 64, 8, 8, seed=56, routing="zipf",
                                                mask_frac=0.1))
