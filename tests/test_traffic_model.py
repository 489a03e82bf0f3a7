"""The algorithmic byte model behind the benchmark's bandwidth figures and
roofline entry (no GPU needed).

Each routed copy moves one row each way: the combine returns one expert
output per dispatched copy ("MSCCLPP EP implementation - #852", commit
message on the combine's byte accounting).  The totals below are written out
term by term for the five workloads (rows of H elements plus, for fp8, one
fp32 scale per 128 channels; int32 routing, handle and offsets), and the
model must reproduce them exactly, as must the split into the notify phase,
the scatter and the combine, and into reads and writes.
"""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from combine_ep_get_dispatch_amd.traffic import algorithmic_bytes  # noqa: E402


def terms(T, H, E, G, k, R, x_elt, sb):
    """The same totals as a plain sum of named terms."""
    row = H * x_elt + (H // sb) * 4 if sb else H * x_elt
    out = 2 * H
    dispatch = sum([
        T * row,        # source rows (and scales), read once
        R * row,        # one received row per routed copy
        T * k * 4,      # topk_idx
        T * k * 4,      # topk_weights
        R * 4,          # recv_src_idx
        R * 4,          # recv_weights
        T * k * 4,      # slot_to_row
        (E + 1) * 4,    # expert_offsets
    ])
    combine = sum([R * out, T * out, T * k * 4, R * 4])
    layout = sum([T * k * 4, E * 4, G * 4, T * 4])
    return dispatch, combine, layout


# (T, H, E, G, k, R, bytes per element, scale block): dispatch, combine, layout
CASES = {
    "tiny": ((128, 256, 8, 2, 2, 256, 2, 0), 201_764, 198_656, 1_576),
    "dsv3_prefill": ((4096, 7168, 256, 8, 8, 32_768, 2, 0), 529_138_692, 528_744_448, 148_512),
    "skewed_zipf": ((4096, 7168, 256, 8, 8, 31_130, 2, 0), 505_643_220, 505_255_528, 148_512),
    "decode_fp8": ((128, 7168, 256, 8, 8, 1_024, 1, 128), 8_537_092, 16_523_264, 5_664),
    "mixtral_large": ((16384, 4096, 8, 8, 2, 32_768, 2, 0), 403_308_580, 402_915_328, 196_672),
}


@pytest.mark.parametrize("name", list(CASES))
def test_algorithmic_bytes(name):
    (T, H, E, G, k, R, elt, sb), d, c, lay = CASES[name]
    assert terms(T, H, E, G, k, R, elt, sb) == (d, c, lay)
    B = algorithmic_bytes(T, H, E, G, k, R, elt, sb)
    assert (B["dispatch"], B["combine"], B["layout"]) == (d, c, lay)
    assert B["dispatch_combine"] == d + c and B["step"] == d + c + lay
    assert B["notify"] == T * k * 4 + (E + 1) * 4


@pytest.mark.parametrize("name", list(CASES))
def test_read_write_split(name):
    """The notify phase reads topk_idx and writes expert_offsets; the scatter
    reads the source rows and the weights and writes the rows, the handle and
    slot_to_row; the combine reads the expert outputs, slot_to_row and the
    weights and writes only its output."""
    (T, H, E, G, k, R, elt, sb), d, c, lay = CASES[name]
    B = algorithmic_bytes(T, H, E, G, k, R, elt, sb)
    rw = bench.kernel_rw_bytes(B, T, H, k, R, elt, sb)
    row = H * elt + (H // sb) * 4 if sb else H * elt
    assert rw["scatter"] == (T * row + T * k * 4, R * row + 2 * R * 4 + T * k * 4)
    assert rw["combine"] == (R * 2 * H + T * k * 4 + R * 4, T * 2 * H)
    assert sum(rw["scatter"]) + B["notify"] == d and sum(rw["combine"]) == c


def test_roofline_bytes_of_the_copy():
    """The roofline entry's algorithmic bytes at T = 4096, H = 7168, k = 8:
    the dispatch less its notify phase."""
    B = algorithmic_bytes(4096, 7168, 256, 8, 8, 32_768)
    assert sum(bench.kernel_rw_bytes(B, 4096, 7168, 8, 32_768, 2, 0)["scatter"]) == 529_006_592
