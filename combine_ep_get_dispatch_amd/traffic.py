"""Algorithmic HBM bytes of layout, dispatch and combine.

Every routed copy counts once, in both directions: dispatch writes one
received row per routed slot, and combine reads one expert-output row per
routed slot (the "MSCCLPP EP implementation - #852" page's commit message on
combine byte accounting: each expert sends one copy per dispatched token
back).  Index and weight arrays count once per read or write.  Bytes the
library moves beyond these (the workspace, the combine's check of
recv_src_idx) are overhead and are not counted.
"""
from __future__ import annotations

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak


def algorithmic_bytes(T: int, H: int, E: int, G: int, k: int, R: int, x_elt: int = 2, scale_block: int = 0) -> dict:
    row = H * x_elt + ((H // scale_block) * 4 if scale_block else 0)  # payload + fp32 scales
    out_row = H * 2  # combine reads and writes bf16
    layout = T * k * 4 + E * 4 + G * 4 + T * 4
    dispatch = (T * row            # x (and scales) read once
                + R * row          # one received row per routed copy
                + 2 * T * k * 4    # topk_idx, topk_weights
                + 2 * R * 4        # recv_src_idx, recv_weights
                + T * k * 4        # slot_to_row
                + (E + 1) * 4)     # expert_offsets
    combine = (R * out_row         # one expert-output row per routed copy
               + T * out_row       # output
               + T * k * 4         # slot_to_row
               + R * 4)            # recv_weights
    # the notify phase of dispatch reads topk_idx and writes expert_offsets;
    # the scatter phase moves everything else
    notify = T * k * 4 + (E + 1) * 4
    return dict(layout=layout, dispatch=dispatch, notify=notify, combine=combine,
                dispatch_combine=dispatch + combine, step=layout + dispatch + combine)


def algorithmic_bytes_quant(T: int, H: int, E: int, k: int, R: int, block: int, scale_bytes: int) -> dict:
    """Dispatch with quantisation: bf16 rows read once, E4M3 codes plus one
    scale per block written per routed copy."""
    row_out = H + (H // block) * scale_bytes
    dispatch = (T * H * 2             # x read once
                + R * row_out         # codes and scales per routed copy
                + 2 * T * k * 4       # topk_idx, topk_weights
                + 2 * R * 4           # recv_src_idx, recv_weights
                + T * k * 4           # slot_to_row
                + (E + 1) * 4)        # expert_offsets
    notify = T * k * 4 + (E + 1) * 4
    return dict(dispatch=dispatch, notify=notify, scatter=dispatch - notify)


def algorithmic_bytes_groups(T: int, H: int, E: int, G: int, k: int, R: int, Rg: int, x_elt: int = 2,
                             scale_block: int = 0) -> dict:
    """The group-deduplicated path: group dispatch (one row per (token,
    group)), local expert permutation, local reduce, group combine."""
    row = H * x_elt + ((H // scale_block) * 4 if scale_block else 0)
    out_row = H * 2
    dispatch_groups = (T * row + Rg * row      # rows read once, one group row per (token, group)
                       + 2 * T * k * 4 + T * 4  # topk_idx, topk_weights, bitmap
                       + Rg * 4 + Rg * k * 8    # recv_src_idx, restricted ids and weights
                       + (G + 1) * 4 + T * G * 4)
    permute = (Rg * row + R * row             # group rows in, expert rows out
               + Rg * k * 8                   # restricted ids and weights
               + 2 * R * 4 + Rg * k * 4       # recv_src_idx, recv_weights, slot_to_row
               + (E + 1) * 4)
    reduce = R * out_row + Rg * out_row + Rg * k * 4 + R * 4
    combine_groups = Rg * out_row + T * out_row + T * G * 4
    return dict(dispatch_groups=dispatch_groups, permute=permute, reduce=reduce, combine_groups=combine_groups,
                total=dispatch_groups + permute + reduce + combine_groups)
