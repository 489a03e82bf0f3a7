"""Python binding of libmoedisp: argument marshalling only.

Every function has the name of the C entry point it calls and takes torch
tensors where the C call takes device pointers; torch provides the device
memory and the stream (the current stream unless one is given).  Every step
of layout, dispatch and combine runs in the library's HIP kernels.  There is
no fallback: if libmoedisp.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoedisp.so")

# element types (moedisp_dtype)
BF16 = 0
FP8_E4M3 = 1
FP32 = 2

# scale formats of quantise-on-dispatch (moedisp_scale_fmt)
SCALE_FP32 = 0
SCALE_UE8M0 = 1

# host return codes
OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_MISALIGNED = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_HIP = -5

# device status bits
DEV_BAD_EXPERT_ID = 1
DEV_DUPLICATE_EXPERT = 2
DEV_BAD_LAYOUT = 4
DEV_BAD_HANDLE = 8
DEV_EXPERT_OVERFLOW = 16

EXPORTS = ("ep_workspace_bytes", "ep_workspace_init", "ep_get_dispatch_layout", "ep_get_dispatch_layout_notify",
           "ep_dispatch", "ep_dispatch_noalloc",
           "ep_dispatch_notify", "ep_dispatch_scatter", "ep_dispatch_quant", "ep_dispatch_scatter_quant",
           "ep_dispatch_groups", "ep_group_permute", "ep_group_reduce", "ep_combine_groups",
           "ep_layout_dispatch_small", "ep_layout_dispatch_small_padded",
           "ep_combine", "ep_combine_padded", "ep_check_status", "ep_status_string")
# tools (include/moedisp_tools.h): plan query and calibration probes, exported
# by the same library
CALIB_EXPORTS = ("ep_plan_query", "ep_probe_read", "ep_probe_copy", "ep_probe_fill")


class MoeDispError(RuntimeError):
    def __init__(self, call: str, code: int, text: str):
        super().__init__(f"{call} failed: {code} ({text})")
        self.code = code


class moedisp_shape(C.Structure):
    _fields_ = [("num_tokens", C.c_int32), ("hidden", C.c_int32), ("num_experts", C.c_int32),
                ("num_groups", C.c_int32), ("topk", C.c_int32), ("x_dtype", C.c_int32),
                ("scale_block", C.c_int32)]

    @classmethod
    def make(cls, T, H, E, G, k, x_dtype=BF16, scale_block=0):
        return cls(T, H, E, G, k, x_dtype, scale_block)

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class moedisp_launch_info(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("blocks", "threads", "lds_bytes", "static_lds_bytes")]


_L, _I = moedisp_launch_info, C.c_int64


class moedisp_plan_info(C.Structure):
    """What the entry points would launch for one shape (moedisp_tools.h)."""
    _fields_ = [("struct_bytes", _I), ("layout", _L), ("layout_reduce", _L), ("layout_tokens_per_block", _I),
                ("layout_notify_fused", _I), ("layout_notify", _L),
                ("tile_tokens", _I), ("tiles", _I), ("tile_stride", _I),
                ("block_tokens", _I), ("block_slots", _I), ("col_splits", _I), ("split_units", _I),
                ("units_per_lane", _I), ("count", _L), ("scatter", _L),
                ("pull", _I), ("pull_tb", _I), ("pull_nblk", _I), ("pull_cap_b", _I), ("pull_cnt_stride", _I),
                ("pull_rows_per_wg", _I), ("pull_units", _I), ("pull_notify", _L), ("pull_copy", _L),
                ("quant_block_slots", _I), ("scatter_quant", _L),
                ("group_rows", _I), ("groups_tile_stride", _I), ("groups_tiles", _I), ("groups_block_slots", _I),
                ("permute_tile_stride", _I), ("permute_tiles", _I), ("permute_block_slots", _I),
                ("groups_count", _L), ("groups_scatter", _L), ("permute_count", _L), ("permute_scatter", _L),
                ("group_reduce", _L), ("combine_groups", _L),
                ("permute_pull", _I), ("permute_pull_tb", _I), ("permute_pull_nblk", _I), ("permute_pull_cap_b", _I),
                ("permute_pull_cnt_stride", _I), ("permute_pull_units", _I), ("permute_pull_wgs_per_xcd", _I),
                ("permute_pull_notify", _L), ("permute_pull_copy", _L),
                ("combine_col_splits", _I), ("combine_units_per_lane", _I), ("combine", _L),
                ("small", _I), ("small_fused", _L),
                ("ws_total", _I), ("ws_partial_offset", _I), ("ws_partial_bytes", _I), ("ws_counts_offset", _I),
                ("ws_counts_bytes", _I), ("ws_counts_needed_flat", _I), ("ws_counts_needed_groups", _I),
                ("ws_counts_needed_rows", _I), ("ws_pull_cnt_offset", _I), ("ws_pull_ls_offset", _I),
                ("ws_pull_n_offset", _I), ("ws_pull_ent_offset", _I), ("ws_pull_end", _I),
                ("ws_permute_pull_cnt_offset", _I), ("ws_permute_pull_ls_offset", _I),
                ("ws_permute_pull_n_offset", _I), ("ws_permute_pull_ent_offset", _I), ("ws_permute_pull_end", _I),
                ("max_block_slots", _I), ("max_tile_slots", _I), ("max_threads", _I),
                ("pull_max_block_slots", _I), ("pull_max_blocks", _I)]


def _as_dict(st):
    out = {}
    for n, t in st._fields_:
        v = getattr(st, n)
        out[n] = _as_dict(v) if isinstance(v, C.Structure) else int(v)
    return out


_lib = None


def load(path: str = LIB_PATH):
    """Load libmoedisp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m combine_ep_get_dispatch_amd.build` "
                           "(there is no fallback path)")
    L = C.CDLL(path)
    P, S = C.c_void_p, C.POINTER(moedisp_shape)
    L.ep_workspace_bytes.argtypes = [S]
    L.ep_workspace_bytes.restype = C.c_size_t
    L.ep_workspace_init.argtypes = [P, C.c_size_t, P]
    L.ep_workspace_init.restype = C.c_int
    L.ep_get_dispatch_layout.argtypes = [S, P, P, P, P, P, C.c_size_t, P]
    L.ep_get_dispatch_layout.restype = C.c_int
    L.ep_get_dispatch_layout_notify.argtypes = [S, P, P, P, P, P, P, C.c_size_t, P]
    L.ep_get_dispatch_layout_notify.restype = C.c_int
    L.ep_dispatch.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.ep_dispatch.restype = C.c_int
    L.ep_dispatch_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P]
    L.ep_dispatch_noalloc.restype = C.c_int
    L.ep_dispatch_notify.argtypes = [S, P, P, P, P, C.c_size_t, P]
    L.ep_dispatch_notify.restype = C.c_int
    L.ep_dispatch_scatter.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.ep_dispatch_scatter.restype = C.c_int
    L.ep_dispatch_quant.argtypes = [S, C.c_int32, C.c_int32, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.ep_dispatch_quant.restype = C.c_int
    L.ep_dispatch_scatter_quant.argtypes = [S, C.c_int32, C.c_int32, P, P, P, P, P, P, P, P, P, P, P,
                                            C.c_size_t, P]
    L.ep_dispatch_scatter_quant.restype = C.c_int
    L.ep_layout_dispatch_small.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.ep_layout_dispatch_small.restype = C.c_int
    L.ep_dispatch_groups.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.ep_dispatch_groups.restype = C.c_int
    L.ep_group_permute.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.ep_group_permute.restype = C.c_int
    L.ep_group_reduce.argtypes = [S, P, P, P, P, P, P, C.c_int32, P, C.c_size_t, P]
    L.ep_group_reduce.restype = C.c_int
    L.ep_combine_groups.argtypes = [S, P, P, P, P, C.c_int32, P, C.c_size_t, P]
    L.ep_combine_groups.restype = C.c_int
    L.ep_combine.argtypes = [S, P, P, P, P, P, C.c_int32, P, C.c_size_t, P]
    L.ep_combine.restype = C.c_int
    L.ep_layout_dispatch_small_padded.argtypes = [S, C.c_int32, C.c_int32, C.c_int32, P, P, P, P, P, P, P, P, P, P,
                                                  P, P, P, C.c_size_t, P]
    L.ep_layout_dispatch_small_padded.restype = C.c_int
    L.ep_combine_padded.argtypes = [S, C.c_int32, P, P, P, P, P, C.c_int32, P, C.c_size_t, P]
    L.ep_combine_padded.restype = C.c_int
    L.ep_check_status.argtypes = [P, C.c_size_t, P, C.POINTER(C.c_int32)]
    L.ep_check_status.restype = C.c_int
    L.ep_status_string.argtypes = [C.c_int]
    L.ep_status_string.restype = C.c_char_p
    L.ep_plan_query.argtypes = [S, C.POINTER(moedisp_plan_info), C.c_size_t]
    L.ep_plan_query.restype = C.c_int
    L.ep_probe_read.argtypes = [P, C.c_size_t, P, P]
    L.ep_probe_read.restype = C.c_int
    L.ep_probe_copy.argtypes = [P, P, C.c_size_t, P]
    L.ep_probe_copy.restype = C.c_int
    L.ep_probe_fill.argtypes = [P, C.c_size_t, C.c_int32, P]
    L.ep_probe_fill.restype = C.c_int
    _lib = L
    return L


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _check(call: str, rc: int):
    if rc != OK:
        raise MoeDispError(call, rc, ep_status_string(rc))


# Element types a row argument may be viewed as: the library reads raw bytes,
# so a row buffer may be handed over as its element type or as bytes.
_U16 = tuple(d for d in (getattr(torch, "uint16", None),) if d is not None)
_I32 = (torch.int32,) + tuple(d for d in (getattr(torch, "uint32", None),) if d is not None)
_ROWS_BF16 = (torch.bfloat16, torch.int16, torch.uint8) + _U16
_ROWS_FP8 = (torch.uint8, torch.int8, torch.float8_e4m3fn)
_F32 = (torch.float32,)
_INT32 = (torch.int32,)
_BYTES = None  # any element type (workspaces, probe buffers)


class _Args:
    """Checks of the tensor arguments of one call, before any pointer crosses
    the C ABI: each tensor must have an accepted element type, be contiguous
    and hold at least the bytes the shape needs (need), and every tensor must
    be a GPU tensor (done, checked after all the others so that a host-memory
    test sees each size and type check).  A failed check raises MoeDispError
    (invalid argument): no kernel is ever handed a buffer smaller than the
    shape says, or an int64 table read as int32."""

    def __init__(self, call: str):
        self.call = call
        self.tensors = []

    def fail(self, msg: str):
        raise MoeDispError(self.call, ERR_INVALID_ARG, msg)

    def need(self, name: str, t, dtypes, nbytes: int, optional: bool = False):
        if t is None:
            if optional or nbytes == 0:
                return
            self.fail(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            self.fail(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if dtypes is not None and t.dtype not in dtypes:
            want = ", ".join(str(d).replace("torch.", "") for d in dtypes)
            self.fail(f"{name} has dtype {str(t.dtype).replace('torch.', '')}, expected one of: {want}")
        if not t.is_contiguous():
            self.fail(f"{name} must be contiguous")
        have = t.numel() * t.element_size()
        if have < nbytes:
            self.fail(f"{name} holds {have} bytes, the shape needs {nbytes}")
        self.tensors.append((name, t))

    def done(self):
        for name, t in self.tensors:
            if t.device.type != "cuda":
                self.fail(f"{name} is on {t.device}, expected a GPU tensor")


def _dims(shape: moedisp_shape):
    """(T, H, E, G, k, row bytes, fp32 scales per row) of a shape."""
    T, H, E, G, k = shape.num_tokens, shape.hidden, shape.num_experts, shape.num_groups, shape.topk
    fp8 = shape.x_dtype == FP8_E4M3
    nsc = H // shape.scale_block if fp8 and shape.scale_block > 0 else 0
    return max(T, 0), max(H, 0), max(E, 0), max(G, 0), max(k, 0), H * (1 if fp8 else 2), nsc


def _rows_dtypes(shape: moedisp_shape):
    return _ROWS_FP8 if shape.x_dtype == FP8_E4M3 else _ROWS_BF16


def _out_dtypes(out_dtype: int):
    return _F32 if out_dtype == FP32 else _ROWS_BF16


def _ws(A: _Args, ws):
    A.need("ws", ws, _BYTES, 1)


def _nb(t) -> int:
    return t.numel() * t.element_size()


def ep_status_string(code: int) -> str:
    return load().ep_status_string(code).decode()


def ep_workspace_bytes(shape: moedisp_shape) -> int:
    return int(load().ep_workspace_bytes(C.byref(shape)))


def ep_workspace_init(ws: torch.Tensor, stream=None):
    A = _Args("ep_workspace_init")
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_workspace_init(_p(ws), _nb(ws), _s(stream)))


def _need_layout(A, shape, topk_idx, tokens_per_expert, tokens_per_group, is_token_in_group, ws):
    T, H, E, G, k, rb, nsc = _dims(shape)
    A.need("topk_idx", topk_idx, _INT32, 4 * T * k)
    A.need("tokens_per_expert", tokens_per_expert, _INT32, 4 * E)
    A.need("tokens_per_group", tokens_per_group, _INT32, 4 * G)
    A.need("is_token_in_group", is_token_in_group, _I32, 4 * T)
    _ws(A, ws)


def ep_get_dispatch_layout(shape, topk_idx, tokens_per_expert, tokens_per_group, is_token_in_group, ws,
                           stream=None):
    A = _Args("ep_get_dispatch_layout")
    _need_layout(A, shape, topk_idx, tokens_per_expert, tokens_per_group, is_token_in_group, ws)
    A.done()
    _check(A.call, load().ep_get_dispatch_layout(
        C.byref(shape), _p(topk_idx), _p(tokens_per_expert), _p(tokens_per_group), _p(is_token_in_group),
        _p(ws), _nb(ws), _s(stream)))


def ep_get_dispatch_layout_notify(shape, topk_idx, tokens_per_expert, tokens_per_group, is_token_in_group,
                                  expert_offsets, ws, stream=None):
    A = _Args("ep_get_dispatch_layout_notify")
    _need_layout(A, shape, topk_idx, tokens_per_expert, tokens_per_group, is_token_in_group, ws)
    A.need("expert_offsets", expert_offsets, _INT32, 4 * (_dims(shape)[2] + 1))
    A.done()
    _check(A.call, load().ep_get_dispatch_layout_notify(
        C.byref(shape), _p(topk_idx), _p(tokens_per_expert), _p(tokens_per_group), _p(is_token_in_group),
        _p(expert_offsets), _p(ws), _nb(ws), _s(stream)))


def _need_dispatch(A, shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                   recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws=None):
    T, H, E, G, k, rb, nsc = _dims(shape)
    cap = T * k
    A.need("x", x, _rows_dtypes(shape), T * rb)
    A.need("x_scales", x_scales, _F32, 4 * T * nsc, optional=nsc == 0)
    A.need("topk_idx", topk_idx, _INT32, 4 * T * k)
    A.need("topk_weights", topk_weights, _F32, 4 * T * k)
    A.need("tokens_per_expert", tokens_per_expert, _INT32, 4 * E)
    A.need("recv_x", recv_x, _rows_dtypes(shape), cap * rb)
    A.need("recv_scales", recv_scales, _F32, 4 * cap * nsc, optional=nsc == 0)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * cap)
    A.need("recv_weights", recv_weights, _F32, 4 * cap)
    A.need("expert_offsets", expert_offsets, _INT32, 4 * (E + 1))
    A.need("slot_to_row", slot_to_row, _INT32, 4 * T * k)
    if ws is not None:
        _ws(A, ws)


def ep_dispatch(shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales, recv_src_idx,
                recv_weights, expert_offsets, slot_to_row, ws, stream=None):
    A = _Args("ep_dispatch")
    _need_dispatch(A, shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                   recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws)
    A.done()
    _check(A.call, load().ep_dispatch(
        C.byref(shape), _p(x), _p(x_scales), _p(topk_idx), _p(topk_weights), _p(tokens_per_expert), _p(recv_x),
        _p(recv_scales), _p(recv_src_idx), _p(recv_weights), _p(expert_offsets), _p(slot_to_row), _p(ws),
        _nb(ws), _s(stream)))


def ep_dispatch_noalloc(shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                        recv_src_idx, recv_weights, expert_offsets, slot_to_row, status, stream=None):
    """ep_dispatch with the library's static per-device workspace; `status`
    (one device int32) receives the call's status bits.  Allocates nothing."""
    A = _Args("ep_dispatch_noalloc")
    _need_dispatch(A, shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                   recv_src_idx, recv_weights, expert_offsets, slot_to_row)
    A.need("status", status, _INT32, 4)
    A.done()
    _check(A.call, load().ep_dispatch_noalloc(
        C.byref(shape), _p(x), _p(x_scales), _p(topk_idx), _p(topk_weights), _p(tokens_per_expert), _p(recv_x),
        _p(recv_scales), _p(recv_src_idx), _p(recv_weights), _p(expert_offsets), _p(slot_to_row), _p(status),
        _s(stream)))


def ep_dispatch_notify(shape, topk_idx, tokens_per_expert, expert_offsets, ws, stream=None):
    A = _Args("ep_dispatch_notify")
    T, H, E, G, k, rb, nsc = _dims(shape)
    A.need("topk_idx", topk_idx, _INT32, 4 * T * k)
    A.need("tokens_per_expert", tokens_per_expert, _INT32, 4 * E)
    A.need("expert_offsets", expert_offsets, _INT32, 4 * (E + 1))
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_dispatch_notify(
        C.byref(shape), _p(topk_idx), _p(tokens_per_expert), _p(expert_offsets), _p(ws), _nb(ws), _s(stream)))


def ep_dispatch_scatter(shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                        recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, stream=None):
    A = _Args("ep_dispatch_scatter")
    _need_dispatch(A, shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                   recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws)
    A.done()
    _check(A.call, load().ep_dispatch_scatter(
        C.byref(shape), _p(x), _p(x_scales), _p(topk_idx), _p(topk_weights), _p(tokens_per_expert), _p(recv_x),
        _p(recv_scales), _p(recv_src_idx), _p(recv_weights), _p(expert_offsets), _p(slot_to_row), _p(ws),
        _nb(ws), _s(stream)))


def _need_quant(A, shape, quant_block, scale_fmt, x, topk_idx, topk_weights, tokens_per_expert, recv_x,
                recv_scales, recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws):
    T, H, E, G, k, rb, nsc = _dims(shape)
    cap = T * k
    blocks = H // int(quant_block) if int(quant_block) > 0 else 0
    A.need("x", x, _ROWS_BF16, T * H * 2)
    A.need("topk_idx", topk_idx, _INT32, 4 * T * k)
    A.need("topk_weights", topk_weights, _F32, 4 * T * k)
    A.need("tokens_per_expert", tokens_per_expert, _INT32, 4 * E)
    A.need("recv_x", recv_x, _ROWS_FP8, cap * H)
    if int(scale_fmt) == SCALE_FP32:
        A.need("recv_scales", recv_scales, _F32, 4 * cap * blocks)
    else:
        A.need("recv_scales", recv_scales, (torch.uint8, torch.int8), cap * blocks)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * cap)
    A.need("recv_weights", recv_weights, _F32, 4 * cap)
    A.need("expert_offsets", expert_offsets, _INT32, 4 * (E + 1))
    A.need("slot_to_row", slot_to_row, _INT32, 4 * T * k)
    _ws(A, ws)


def ep_dispatch_quant(shape, quant_block, scale_fmt, x, topk_idx, topk_weights, tokens_per_expert, recv_x,
                      recv_scales, recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, stream=None):
    A = _Args("ep_dispatch_quant")
    _need_quant(A, shape, quant_block, scale_fmt, x, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws)
    A.done()
    _check(A.call, load().ep_dispatch_quant(
        C.byref(shape), int(quant_block), int(scale_fmt), _p(x), _p(topk_idx), _p(topk_weights),
        _p(tokens_per_expert), _p(recv_x), _p(recv_scales), _p(recv_src_idx), _p(recv_weights), _p(expert_offsets),
        _p(slot_to_row), _p(ws), _nb(ws), _s(stream)))


def ep_dispatch_scatter_quant(shape, quant_block, scale_fmt, x, topk_idx, topk_weights, tokens_per_expert, recv_x,
                              recv_scales, recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws,
                              stream=None):
    A = _Args("ep_dispatch_scatter_quant")
    _need_quant(A, shape, quant_block, scale_fmt, x, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws)
    A.done()
    _check(A.call, load().ep_dispatch_scatter_quant(
        C.byref(shape), int(quant_block), int(scale_fmt), _p(x), _p(topk_idx), _p(topk_weights),
        _p(tokens_per_expert), _p(recv_x), _p(recv_scales), _p(recv_src_idx), _p(recv_weights), _p(expert_offsets),
        _p(slot_to_row), _p(ws), _nb(ws), _s(stream)))


def ep_layout_dispatch_small(shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, tokens_per_group,
                             is_token_in_group, recv_x, recv_scales, recv_src_idx, recv_weights, expert_offsets,
                             slot_to_row, ws, stream=None):
    A = _Args("ep_layout_dispatch_small")
    _need_dispatch(A, shape, x, x_scales, topk_idx, topk_weights, tokens_per_expert, recv_x, recv_scales,
                   recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws)
    T, H, E, G, k, rb, nsc = _dims(shape)
    A.need("tokens_per_group", tokens_per_group, _INT32, 4 * G)
    A.need("is_token_in_group", is_token_in_group, _I32, 4 * T)
    A.done()
    _check(A.call, load().ep_layout_dispatch_small(
        C.byref(shape), _p(x), _p(x_scales), _p(topk_idx), _p(topk_weights), _p(tokens_per_expert),
        _p(tokens_per_group), _p(is_token_in_group), _p(recv_x), _p(recv_scales), _p(recv_src_idx),
        _p(recv_weights), _p(expert_offsets), _p(slot_to_row), _p(ws), _nb(ws), _s(stream)))


def ep_layout_dispatch_small_padded(shape, expert_capacity, expert_stride, row_base, x, x_scales, topk_idx,
                                    topk_weights, tokens_per_expert, tokens_per_group, is_token_in_group, recv_x,
                                    recv_scales, recv_src_idx, recv_weights, slot_to_row, ws, stream=None):
    A = _Args("ep_layout_dispatch_small_padded")
    T, H, E, G, k, rb, nsc = _dims(shape)
    rows = E * max(int(expert_stride), 0)
    A.need("x", x, _rows_dtypes(shape), T * rb)
    A.need("x_scales", x_scales, _F32, 4 * T * nsc, optional=nsc == 0)
    A.need("topk_idx", topk_idx, _INT32, 4 * T * k)
    A.need("topk_weights", topk_weights, _F32, 4 * T * k)
    A.need("tokens_per_expert", tokens_per_expert, _INT32, 4 * E)
    A.need("tokens_per_group", tokens_per_group, _INT32, 4 * G)
    A.need("is_token_in_group", is_token_in_group, _I32, 4 * T)
    A.need("recv_x", recv_x, _rows_dtypes(shape), rows * rb)
    A.need("recv_scales", recv_scales, _F32, 4 * rows * nsc, optional=nsc == 0)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * rows)
    A.need("recv_weights", recv_weights, _F32, 4 * rows)
    A.need("slot_to_row", slot_to_row, _INT32, 4 * T * k)
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_layout_dispatch_small_padded(
        C.byref(shape), int(expert_capacity), int(expert_stride), int(row_base), _p(x), _p(x_scales), _p(topk_idx),
        _p(topk_weights), _p(tokens_per_expert), _p(tokens_per_group), _p(is_token_in_group), _p(recv_x),
        _p(recv_scales), _p(recv_src_idx), _p(recv_weights), _p(slot_to_row), _p(ws), _nb(ws), _s(stream)))


def ep_dispatch_groups(shape, x, x_scales, topk_idx, topk_weights, is_token_in_group, tokens_per_group, recv_x,
                       recv_scales, recv_src_idx, recv_topk_idx, recv_topk_weights, group_offsets, token_group_row, ws,
                       stream=None):
    A = _Args("ep_dispatch_groups")
    T, H, E, G, k, rb, nsc = _dims(shape)
    cap = T * min(G, k)
    A.need("x", x, _rows_dtypes(shape), T * rb)
    A.need("x_scales", x_scales, _F32, 4 * T * nsc, optional=nsc == 0)
    A.need("topk_idx", topk_idx, _INT32, 4 * T * k)
    A.need("topk_weights", topk_weights, _F32, 4 * T * k)
    A.need("is_token_in_group", is_token_in_group, _I32, 4 * T)
    A.need("tokens_per_group", tokens_per_group, _INT32, 4 * G)
    A.need("recv_x", recv_x, _rows_dtypes(shape), cap * rb)
    A.need("recv_scales", recv_scales, _F32, 4 * cap * nsc, optional=nsc == 0)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * cap)
    A.need("recv_topk_idx", recv_topk_idx, _INT32, 4 * cap * k)
    A.need("recv_topk_weights", recv_topk_weights, _F32, 4 * cap * k)
    A.need("group_offsets", group_offsets, _INT32, 4 * (G + 1))
    A.need("token_group_row", token_group_row, _INT32, 4 * T * G)
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_dispatch_groups(
        C.byref(shape), _p(x), _p(x_scales), _p(topk_idx), _p(topk_weights), _p(is_token_in_group),
        _p(tokens_per_group), _p(recv_x), _p(recv_scales), _p(recv_src_idx), _p(recv_topk_idx),
        _p(recv_topk_weights), _p(group_offsets), _p(token_group_row), _p(ws), _nb(ws), _s(stream)))


def ep_group_permute(shape, group_x, group_scales, recv_topk_idx, recv_topk_weights, tokens_per_expert, recv_x,
                     recv_scales, recv_src_idx, recv_weights, expert_offsets, slot_to_row, ws, stream=None):
    A = _Args("ep_group_permute")
    T, H, E, G, k, rb, nsc = _dims(shape)
    gr = T * min(G, k)  # group rows, each seen as a token of k slots
    A.need("group_x", group_x, _rows_dtypes(shape), gr * rb)
    A.need("group_scales", group_scales, _F32, 4 * gr * nsc, optional=nsc == 0)
    A.need("recv_topk_idx", recv_topk_idx, _INT32, 4 * gr * k)
    A.need("recv_topk_weights", recv_topk_weights, _F32, 4 * gr * k)
    A.need("tokens_per_expert", tokens_per_expert, _INT32, 4 * E)
    A.need("recv_x", recv_x, _rows_dtypes(shape), T * k * rb)
    A.need("recv_scales", recv_scales, _F32, 4 * T * k * nsc, optional=nsc == 0)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * T * k)
    A.need("recv_weights", recv_weights, _F32, 4 * T * k)
    A.need("expert_offsets", expert_offsets, _INT32, 4 * (E + 1))
    A.need("slot_to_row", slot_to_row, _INT32, 4 * gr * k)
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_group_permute(
        C.byref(shape), _p(group_x), _p(group_scales), _p(recv_topk_idx), _p(recv_topk_weights),
        _p(tokens_per_expert), _p(recv_x), _p(recv_scales), _p(recv_src_idx), _p(recv_weights), _p(expert_offsets),
        _p(slot_to_row), _p(ws), _nb(ws), _s(stream)))


def _out_bytes(rows: int, H: int, out_dtype: int) -> int:
    return rows * H * (4 if int(out_dtype) == FP32 else 2)


def ep_group_reduce(shape, expert_out, recv_src_idx, recv_weights, slot_to_row, group_offsets, group_out, out_dtype,
                    ws, stream=None):
    A = _Args("ep_group_reduce")
    T, H, E, G, k, rb, nsc = _dims(shape)
    gr = T * min(G, k)
    A.need("expert_out", expert_out, _ROWS_BF16, T * k * H * 2)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * T * k, optional=True)
    A.need("recv_weights", recv_weights, _F32, 4 * T * k)
    A.need("slot_to_row", slot_to_row, _INT32, 4 * gr * k)
    A.need("group_offsets", group_offsets, _INT32, 4 * (G + 1))
    A.need("group_out", group_out, _out_dtypes(int(out_dtype)), _out_bytes(gr, H, out_dtype))
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_group_reduce(
        C.byref(shape), _p(expert_out), _p(recv_src_idx), _p(recv_weights), _p(slot_to_row), _p(group_offsets),
        _p(group_out), int(out_dtype), _p(ws), _nb(ws), _s(stream)))


def ep_combine_groups(shape, group_rows, recv_src_idx, token_group_row, out, out_dtype, ws, stream=None):
    A = _Args("ep_combine_groups")
    T, H, E, G, k, rb, nsc = _dims(shape)
    gr = T * min(G, k)
    A.need("group_rows", group_rows, _ROWS_BF16, gr * H * 2)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * gr, optional=True)
    A.need("token_group_row", token_group_row, _INT32, 4 * T * G)
    A.need("out", out, _out_dtypes(int(out_dtype)), _out_bytes(T, H, out_dtype))
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_combine_groups(
        C.byref(shape), _p(group_rows), _p(recv_src_idx), _p(token_group_row), _p(out), int(out_dtype), _p(ws),
        _nb(ws), _s(stream)))


def ep_combine(shape, expert_out, recv_src_idx, recv_weights, slot_to_row, out, out_dtype, ws, stream=None):
    A = _Args("ep_combine")
    T, H, E, G, k, rb, nsc = _dims(shape)
    A.need("expert_out", expert_out, _ROWS_BF16, T * k * H * 2)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * T * k, optional=True)
    A.need("recv_weights", recv_weights, _F32, 4 * T * k)
    A.need("slot_to_row", slot_to_row, _INT32, 4 * T * k)
    A.need("out", out, _out_dtypes(int(out_dtype)), _out_bytes(T, H, out_dtype))
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_combine(
        C.byref(shape), _p(expert_out), _p(recv_src_idx), _p(recv_weights), _p(slot_to_row), _p(out),
        int(out_dtype), _p(ws), _nb(ws), _s(stream)))


def ep_combine_padded(shape, expert_stride, expert_out, recv_src_idx, recv_weights, slot_to_row, out, out_dtype, ws,
                      stream=None):
    A = _Args("ep_combine_padded")
    T, H, E, G, k, rb, nsc = _dims(shape)
    rows = E * max(int(expert_stride), 0)
    A.need("expert_out", expert_out, _ROWS_BF16, rows * H * 2)
    A.need("recv_src_idx", recv_src_idx, _INT32, 4 * rows, optional=True)
    A.need("recv_weights", recv_weights, _F32, 4 * rows)
    A.need("slot_to_row", slot_to_row, _INT32, 4 * T * k)
    A.need("out", out, _out_dtypes(int(out_dtype)), _out_bytes(T, H, out_dtype))
    _ws(A, ws)
    A.done()
    _check(A.call, load().ep_combine_padded(
        C.byref(shape), int(expert_stride), _p(expert_out), _p(recv_src_idx), _p(recv_weights), _p(slot_to_row),
        _p(out), int(out_dtype), _p(ws), _nb(ws), _s(stream)))


def ep_check_status(ws, stream=None) -> int:
    A = _Args("ep_check_status")
    _ws(A, ws)
    A.done()
    v = C.c_int32(0)
    _check(A.call, load().ep_check_status(_p(ws), _nb(ws), _s(stream), C.byref(v)))
    return int(v.value)


def ep_plan_query(shape) -> dict:
    """The launch geometry, LDS and workspace layout of `shape` as a dict
    (launches as nested dicts); raises for a shape the library rejects."""
    info = moedisp_plan_info()
    _check("ep_plan_query", load().ep_plan_query(C.byref(shape), C.byref(info), C.sizeof(info)))
    return _as_dict(info)


def ep_probe_read(src, nbytes: int, sink, stream=None):
    A = _Args("ep_probe_read")
    A.need("src", src, _BYTES, int(nbytes))
    A.need("sink", sink, _BYTES, 16)
    A.done()
    _check(A.call, load().ep_probe_read(_p(src), int(nbytes), _p(sink), _s(stream)))


def ep_probe_copy(dst, src, nbytes: int, stream=None):
    A = _Args("ep_probe_copy")
    A.need("dst", dst, _BYTES, int(nbytes))
    A.need("src", src, _BYTES, int(nbytes))
    A.done()
    _check(A.call, load().ep_probe_copy(_p(dst), _p(src), int(nbytes), _s(stream)))


def ep_probe_fill(dst, nbytes: int, shuffled: bool = False, stream=None):
    A = _Args("ep_probe_fill")
    A.need("dst", dst, _BYTES, int(nbytes))
    A.done()
    _check(A.call, load().ep_probe_fill(_p(dst), int(nbytes), 1 if shuffled else 0, _s(stream)))


class EpBuffers:
    """Device buffers for one shape (plumbing): workspace, layout outputs,
    receive buffers at capacity T*k rows and the dispatch handle."""

    def __init__(self, shape: moedisp_shape, device="cuda"):
        T, H, E, G, k = shape.num_tokens, shape.hidden, shape.num_experts, shape.num_groups, shape.topk
        self.shape = shape
        self.device = torch.device(device)
        nbytes = ep_workspace_bytes(shape)
        if nbytes == 0:
            raise MoeDispError("ep_workspace_bytes", ERR_INVALID_ARG, "invalid shape")
        d = self.device
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=d)
        self.tokens_per_expert = torch.empty(E, dtype=torch.int32, device=d)
        self.tokens_per_group = torch.empty(G, dtype=torch.int32, device=d)
        self.is_token_in_group = torch.empty(T, dtype=torch.int32, device=d)
        cap = T * k
        elt = 1 if shape.x_dtype == FP8_E4M3 else 2
        self.recv_x = torch.empty((cap, H * elt), dtype=torch.uint8, device=d)
        nsc = H // shape.scale_block if shape.x_dtype == FP8_E4M3 else 0
        self.recv_scales = torch.empty((cap, nsc), dtype=torch.float32, device=d) if nsc else None
        self.recv_src_idx = torch.empty(cap, dtype=torch.int32, device=d)
        self.recv_weights = torch.empty(cap, dtype=torch.float32, device=d)
        self.expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=d)
        self.slot_to_row = torch.empty((T, k), dtype=torch.int32, device=d)

    def layout(self, topk_idx, stream=None):
        ep_get_dispatch_layout(self.shape, topk_idx, self.tokens_per_expert, self.tokens_per_group,
                               self.is_token_in_group, self.ws, stream)

    def layout_notify(self, topk_idx, stream=None):
        """Layout and the dispatch's notify phase in one call; dispatch_scatter
        follows."""
        ep_get_dispatch_layout_notify(self.shape, topk_idx, self.tokens_per_expert, self.tokens_per_group,
                                      self.is_token_in_group, self.expert_offsets, self.ws, stream)

    def dispatch(self, x, x_scales, topk_idx, topk_weights, stream=None):
        ep_dispatch(self.shape, x, x_scales, topk_idx, topk_weights, self.tokens_per_expert, self.recv_x,
                    self.recv_scales, self.recv_src_idx, self.recv_weights, self.expert_offsets, self.slot_to_row,
                    self.ws, stream)

    def dispatch_notify(self, topk_idx, stream=None):
        ep_dispatch_notify(self.shape, topk_idx, self.tokens_per_expert, self.expert_offsets, self.ws, stream)

    def dispatch_scatter(self, x, x_scales, topk_idx, topk_weights, stream=None):
        ep_dispatch_scatter(self.shape, x, x_scales, topk_idx, topk_weights, self.tokens_per_expert, self.recv_x,
                            self.recv_scales, self.recv_src_idx, self.recv_weights, self.expert_offsets,
                            self.slot_to_row, self.ws, stream)

    def layout_dispatch_small(self, x, x_scales, topk_idx, topk_weights, stream=None):
        ep_layout_dispatch_small(self.shape, x, x_scales, topk_idx, topk_weights, self.tokens_per_expert,
                                 self.tokens_per_group, self.is_token_in_group, self.recv_x, self.recv_scales,
                                 self.recv_src_idx, self.recv_weights, self.expert_offsets, self.slot_to_row, self.ws,
                                 stream)

    def enable_quant(self, quant_block: int, scale_fmt: int):
        """Receive buffers of quantise-on-dispatch: E4M3 codes [T*k][H] and one
        scale per block of `quant_block` channels (float32 or uint8)."""
        T, H, k = self.shape.num_tokens, self.shape.hidden, self.shape.topk
        self.quant_block, self.scale_fmt = int(quant_block), int(scale_fmt)
        nsc = H // self.quant_block if H % self.quant_block == 0 else 0
        self.recv_q = torch.empty((T * k, H), dtype=torch.uint8, device=self.device)
        sdt = torch.float32 if scale_fmt == SCALE_FP32 else torch.uint8
        self.recv_qscales = torch.empty((T * k, nsc), dtype=sdt, device=self.device)
        return self

    def dispatch_quant(self, x, topk_idx, topk_weights, stream=None):
        ep_dispatch_quant(self.shape, self.quant_block, self.scale_fmt, x, topk_idx, topk_weights,
                          self.tokens_per_expert, self.recv_q, self.recv_qscales, self.recv_src_idx,
                          self.recv_weights, self.expert_offsets, self.slot_to_row, self.ws, stream)

    def dispatch_scatter_quant(self, x, topk_idx, topk_weights, stream=None):
        ep_dispatch_scatter_quant(self.shape, self.quant_block, self.scale_fmt, x, topk_idx, topk_weights,
                                  self.tokens_per_expert, self.recv_q, self.recv_qscales, self.recv_src_idx,
                                  self.recv_weights, self.expert_offsets, self.slot_to_row, self.ws, stream)

    def combine(self, expert_out, out, out_dtype=BF16, check_src=True, stream=None):
        ep_combine(self.shape, expert_out, self.recv_src_idx if check_src else None, self.recv_weights,
                   self.slot_to_row, out, out_dtype, self.ws, stream)

    def status(self, stream=None) -> int:
        return ep_check_status(self.ws, stream)


class EpPaddedBuffers:
    """Receive buffers of the padded (low-latency) layout (plumbing) next to an
    EpBuffers of the same shape, whose layout outputs and workspace it uses:
    E * expert_stride rows; expert e's rows start at e * expert_stride +
    row_base, at most expert_capacity of them."""

    def __init__(self, bufs: EpBuffers, expert_capacity: int, expert_stride: int = None, row_base: int = 0):
        s = bufs.shape
        self.bufs, self.shape, d = bufs, s, bufs.device
        self.capacity = int(expert_capacity)
        self.stride = int(expert_capacity if expert_stride is None else expert_stride)
        self.base = int(row_base)
        rows = s.num_experts * self.stride
        self.rows = rows
        fp8 = s.x_dtype == FP8_E4M3
        self.recv_x = torch.empty((rows, s.hidden * (1 if fp8 else 2)), dtype=torch.uint8, device=d)
        nsc = s.hidden // s.scale_block if fp8 else 0
        self.recv_scales = torch.empty((rows, nsc), dtype=torch.float32, device=d) if nsc else None
        self.recv_src_idx = torch.empty(rows, dtype=torch.int32, device=d)
        self.recv_weights = torch.empty(rows, dtype=torch.float32, device=d)
        self.slot_to_row = torch.empty((max(s.num_tokens, 1), s.topk), dtype=torch.int32, device=d)

    def dispatch(self, x, x_scales, topk_idx, topk_weights, stream=None):
        b = self.bufs
        ep_layout_dispatch_small_padded(self.shape, self.capacity, self.stride, self.base, x, x_scales, topk_idx,
                                        topk_weights, b.tokens_per_expert, b.tokens_per_group, b.is_token_in_group,
                                        self.recv_x, self.recv_scales, self.recv_src_idx, self.recv_weights,
                                        self.slot_to_row, b.ws, stream)

    def combine(self, expert_out, out, out_dtype=BF16, check_src=True, stream=None):
        ep_combine_padded(self.shape, self.stride, expert_out, self.recv_src_idx if check_src else None,
                          self.recv_weights, self.slot_to_row, out, out_dtype, self.bufs.ws, stream)


class EpGroupBuffers:
    """Device buffers of the group-deduplicated path (plumbing) on top of an
    EpBuffers of the same shape: group rows at capacity T*min(G,k), their
    restricted routing, the token -> group-row handle, and the handle of the
    local expert permutation (whose rows land in the EpBuffers' receive
    buffers)."""

    def __init__(self, bufs: EpBuffers):
        s = bufs.shape
        T, H, G, k = s.num_tokens, s.hidden, s.num_groups, s.topk
        self.bufs, self.shape, d = bufs, s, bufs.device
        cap = T * min(G, k)
        self.capacity = cap
        elt = 1 if s.x_dtype == FP8_E4M3 else 2
        self.group_x = torch.empty((cap, H * elt), dtype=torch.uint8, device=d)
        nsc = H // s.scale_block if s.x_dtype == FP8_E4M3 else 0
        self.group_scales = torch.empty((cap, nsc), dtype=torch.float32, device=d) if nsc else None
        self.group_src_idx = torch.empty(cap, dtype=torch.int32, device=d)
        self.group_topk_idx = torch.empty((cap, k), dtype=torch.int32, device=d)
        self.group_topk_weights = torch.empty((cap, k), dtype=torch.float32, device=d)
        self.group_offsets = torch.empty(G + 1, dtype=torch.int32, device=d)
        self.token_group_row = torch.empty((T, G), dtype=torch.int32, device=d)
        self.perm_src_idx = torch.empty(T * k, dtype=torch.int32, device=d)
        self.perm_slot_to_row = torch.empty((cap, k), dtype=torch.int32, device=d)

    def dispatch_groups(self, x, x_scales, topk_idx, topk_weights, stream=None):
        b = self.bufs
        ep_dispatch_groups(self.shape, x, x_scales, topk_idx, topk_weights, b.is_token_in_group,
                           b.tokens_per_group, self.group_x, self.group_scales, self.group_src_idx,
                           self.group_topk_idx, self.group_topk_weights, self.group_offsets, self.token_group_row,
                           b.ws, stream)

    def permute(self, stream=None):
        b = self.bufs
        ep_group_permute(self.shape, self.group_x, self.group_scales, self.group_topk_idx, self.group_topk_weights,
                         b.tokens_per_expert, b.recv_x, b.recv_scales, self.perm_src_idx, b.recv_weights,
                         b.expert_offsets, self.perm_slot_to_row, b.ws, stream)

    def reduce(self, expert_out, group_out, out_dtype=BF16, check_src=True, stream=None):
        b = self.bufs
        ep_group_reduce(self.shape, expert_out, self.perm_src_idx if check_src else None, b.recv_weights,
                        self.perm_slot_to_row, self.group_offsets, group_out, out_dtype, b.ws, stream)

    def combine_groups(self, group_rows, out, out_dtype=BF16, check_src=True, stream=None):
        ep_combine_groups(self.shape, group_rows, self.group_src_idx if check_src else None, self.token_group_row,
                          out, out_dtype, self.bufs.ws, stream)
