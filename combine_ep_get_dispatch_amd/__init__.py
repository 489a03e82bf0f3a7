"""libmoedisp: MoE expert-parallel layout / dispatch / combine for MI355X (gfx950).

The product is the C library libmoedisp.so (include/moedisp.h; plan query
and calibration probes in include/moedisp_tools.h); this package
holds its HIP sources (csrc/), its build script, the Python binding and the
seeded synthetic workloads.
"""
from .binding import (BF16, FP8_E4M3, FP32, SCALE_FP32, SCALE_UE8M0, EpBuffers, EpGroupBuffers, EpPaddedBuffers,
                      MoeDispError, ep_check_status, ep_combine, ep_combine_groups, ep_combine_padded, ep_dispatch, ep_dispatch_groups, ep_dispatch_noalloc,
                      ep_dispatch_notify, ep_dispatch_quant, ep_dispatch_scatter, ep_dispatch_scatter_quant,
                      ep_group_permute, ep_group_reduce, ep_layout_dispatch_small, ep_layout_dispatch_small_padded,
                      ep_get_dispatch_layout, ep_get_dispatch_layout_notify, ep_plan_query, ep_probe_copy, ep_probe_fill, ep_probe_read,
                      ep_status_string,
                      ep_workspace_bytes, ep_workspace_init, load, moedisp_shape)

__all__ = ["BF16", "FP8_E4M3", "FP32", "SCALE_FP32", "SCALE_UE8M0", "EpBuffers", "EpGroupBuffers", "EpPaddedBuffers",
           "MoeDispError", "ep_check_status", "ep_combine", "ep_combine_groups", "ep_combine_padded", "ep_dispatch", "ep_dispatch_groups", "ep_dispatch_noalloc",
           "ep_dispatch_notify", "ep_dispatch_quant", "ep_dispatch_scatter", "ep_dispatch_scatter_quant",
           "ep_group_permute", "ep_group_reduce", "ep_layout_dispatch_small", "ep_layout_dispatch_small_padded",
           "ep_get_dispatch_layout", "ep_get_dispatch_layout_notify", "ep_plan_query", "ep_probe_copy", "ep_probe_fill", "ep_probe_read",
           "ep_status_string",
           "ep_workspace_bytes", "ep_workspace_init", "load", "moedisp_shape"]
