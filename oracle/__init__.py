"""Python access to the CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It loads liboracle.so, built from oracle.cpp with g++ (C++17),
and wraps
each function with numpy arrays.  Nothing here touches a GPU.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.cpp")
LIB = os.path.join(_HERE, "liboracle.so")

ERR_BAD_EXPERT = 1
ERR_DUP_EXPERT = 2

# scale formats of the quantise-on-dispatch oracle
SCALE_FP32 = 0
SCALE_UE8M0 = 1

GCC_FLAGS = ["-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra"]

# Address and undefined-behaviour sanitizers (host code only: the oracle is
# plain C++ for the CPU).  Any report aborts the process.
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]

# Environment variable naming another oracle library to load instead of
# liboracle.so (the sanitized build, for the sanitizer tests).
LIB_ENV = "MOEDISP_ORACLE_LIB"


def compile_oracle(src: str, out: str, sanitize: bool = False) -> str:
    """Compile one oracle source file (C++17) into a shared library, with the
    address and undefined-behaviour sanitizers if `sanitize`."""
    tmp = out + ".tmp"
    flags = GCC_FLAGS + (SAN_FLAGS if sanitize else [])
    subprocess.run(["g++", *flags, "-x", "c++", "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def sanitizer_env(lib: str) -> dict:
    """Environment for a child Python process that loads the sanitized oracle
    `lib`: the sanitizer runtime preloaded (it must come first in a process
    whose main program is not instrumented), leak checks off (the interpreter
    keeps its allocations at exit), and any report fatal."""
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = dict(os.environ)
    env.update({"LD_PRELOAD": asan, LIB_ENV: lib,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87"})
    return env


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        compile_oracle(SRC, LIB)
    return LIB


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


class Oracle:
    """numpy front end of one compiled oracle library."""

    def __init__(self, path: str = LIB):
        L = C.CDLL(path)
        P = C.c_void_p
        L.oracle_f32_to_bf16.argtypes = [C.c_float]
        L.oracle_f32_to_bf16.restype = C.c_uint16
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_bf16_to_double.restype = C.c_double
        L.oracle_f32_to_bf16_array.argtypes = [P, P, C.c_int64]
        L.oracle_f32_to_bf16_array.restype = None
        L.oracle_layout.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P]
        L.oracle_layout.restype = C.c_int
        L.oracle_dispatch.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int64,
                                      P, P, P, P, P, P, P, P, P, P]
        L.oracle_dispatch.restype = C.c_int
        L.oracle_combine.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int64, P, P, P, P, P]
        L.oracle_combine.restype = C.c_int
        L.oracle_f32_to_e4m3_array.argtypes = [P, P, C.c_int64]
        L.oracle_f32_to_e4m3_array.restype = None
        L.oracle_e4m3_to_double_array.argtypes = [P, P, C.c_int64]
        L.oracle_e4m3_to_double_array.restype = None
        L.oracle_ue8m0_exponent.argtypes = [C.c_float]
        L.oracle_ue8m0_exponent.restype = C.c_int
        L.oracle_quant_rows.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P]
        L.oracle_quant_rows.restype = C.c_int
        L.oracle_dispatch_quant.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                            P, P, P, P, P, P, P, P, P]
        L.oracle_dispatch_quant.restype = C.c_int
        L.oracle_dispatch_groups.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int64,
                                             P, P, P, P, P, P, P, P, P, P, P, P]
        L.oracle_dispatch_groups.restype = C.c_int
        L.oracle_combine_groups.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int64, P, P, P, P]
        L.oracle_combine_groups.restype = C.c_int
        L.oracle_dispatch_padded.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int64,
                                             C.c_int64, P, P, P, P, P, P, P, P, P]
        L.oracle_dispatch_padded.restype = C.c_int
        self.L = L
        self.path = path

    def f32_to_bf16(self, a) -> np.ndarray:
        a = _c(a, np.float32)
        out = np.empty(a.shape, np.uint16)
        self.L.oracle_f32_to_bf16_array(_p(a), _p(out), a.size)
        return out

    def layout(self, topk_idx, E: int, G: int):
        """Returns (tokens_per_expert[E], tokens_per_group[G], is_token_in_group[T], status)."""
        idx = _c(topk_idx, np.int32)
        T, k = idx.shape
        tpe = np.zeros(E, np.int32)
        tpg = np.zeros(G, np.int32)
        bm = np.zeros(T, np.uint32)
        st = self.L.oracle_layout(T, k, E, G, _p(idx), _p(tpe), _p(tpg), _p(bm))
        if st < 0:
            raise ValueError("oracle_layout: bad shape")
        return tpe, tpg, bm, st

    def dispatch(self, x, x_scales, topk_idx, topk_weights, E: int):
        """Returns a dict with recv_x [T*k][...], recv_scales, recv_src_idx [T*k],
        recv_weights [T*k], expert_offsets [E+1], slot_to_row [T][k], status.
        Rows at or past R = expert_offsets[E] stay zero (unused capacity)."""
        idx = _c(topk_idx, np.int32)
        T, k = idx.shape
        x = np.ascontiguousarray(x)
        row_bytes = int(np.prod(x.shape[1:])) * x.itemsize
        cap = T * k
        recv_x = np.zeros((cap,) + x.shape[1:], x.dtype)
        if x_scales is not None:
            xs = np.ascontiguousarray(x_scales)
            srb = int(np.prod(xs.shape[1:])) * xs.itemsize
            recv_scales = np.zeros((cap,) + xs.shape[1:], xs.dtype)
        else:
            xs, srb, recv_scales = None, 0, None
        src = np.full(cap, -1, np.int32)
        rw = np.zeros(cap, np.float32)
        off = np.zeros(E + 1, np.int32)
        s2r = np.zeros((T, k), np.int32)
        w = _c(topk_weights, np.float32)
        st = self.L.oracle_dispatch(T, k, E, row_bytes, srb, _p(x), _p(xs), _p(idx), _p(w),
                                    _p(recv_x), _p(recv_scales), _p(src), _p(rw), _p(off), _p(s2r))
        if st < 0:
            raise ValueError("oracle_dispatch: bad shape")
        return dict(recv_x=recv_x, recv_scales=recv_scales, recv_src_idx=src, recv_weights=rw,
                    expert_offsets=off, slot_to_row=s2r, status=st)

    def dispatch_padded(self, x, x_scales, topk_idx, topk_weights, E: int, C: int, S: int, B: int, fill=0):
        """Padded (low-latency) layout: returns a dict with recv_x [E*S][...],
        recv_scales, recv_src_idx [E*S], recv_weights [E*S], slot_to_row [T][k],
        status.  Rows no slot takes keep `fill` (recv_src_idx -1, weights 0)."""
        idx = _c(topk_idx, np.int32)
        T, k = idx.shape
        x = np.ascontiguousarray(x)
        row_bytes = int(np.prod(x.shape[1:])) * x.itemsize
        rows = E * S
        # one spare slab past the buffer, so that a planted off-by-one in the
        # tests' mutants writes into it instead of past the allocation
        alloc = rows + S
        recv_x = np.full((alloc,) + x.shape[1:], fill, x.dtype)
        if x_scales is not None:
            xs = np.ascontiguousarray(x_scales)
            srb = int(np.prod(xs.shape[1:])) * xs.itemsize
            recv_scales = np.zeros((alloc,) + xs.shape[1:], xs.dtype)
        else:
            xs, srb, recv_scales = None, 0, None
        src = np.full(alloc, -1, np.int32)
        rw = np.zeros(alloc, np.float32)
        s2r = np.zeros((T, k), np.int32)
        w = _c(topk_weights, np.float32)
        st = self.L.oracle_dispatch_padded(T, k, E, C, S, B, row_bytes, srb, _p(x), _p(xs), _p(idx), _p(w),
                                           _p(recv_x), _p(recv_scales), _p(src), _p(rw), _p(s2r))
        if st < 0:
            raise ValueError("oracle_dispatch_padded: bad arguments")
        return dict(recv_x=recv_x[:rows], recv_scales=None if recv_scales is None else recv_scales[:rows],
                    recv_src_idx=src[:rows], recv_weights=rw[:rows], slot_to_row=s2r, status=st)

    def combine(self, expert_out_bf16, recv_weights, slot_to_row, want_f32=True, want_bf16=True):
        """expert_out_bf16: uint16 [R][H].  Returns (out_f32 [T][H] or None, out_bf16 [T][H] or None)."""
        eo = _c(expert_out_bf16, np.uint16)
        R, H = eo.shape
        s2r = _c(slot_to_row, np.int32)
        T, k = s2r.shape
        rw = _c(recv_weights, np.float32)
        of = np.zeros((T, H), np.float32) if want_f32 else None
        ob = np.zeros((T, H), np.uint16) if want_bf16 else None
        st = self.L.oracle_combine(T, k, H, R, _p(eo), _p(rw), _p(s2r), _p(of), _p(ob))
        if st < 0:
            raise ValueError("oracle_combine: bad arguments")
        return of, ob


    # -- quantise-on-dispatch ------------------------------------------------

    def f32_to_e4m3(self, a) -> np.ndarray:
        a = _c(a, np.float32)
        out = np.empty(a.shape, np.uint8)
        self.L.oracle_f32_to_e4m3_array(_p(a), _p(out), a.size)
        return out

    def e4m3_to_f64(self, codes) -> np.ndarray:
        c = _c(codes, np.uint8)
        out = np.empty(c.shape, np.float64)
        self.L.oracle_e4m3_to_double_array(_p(c), _p(out), c.size)
        return out

    def ue8m0_exponent(self, amax: float) -> int:
        return int(self.L.oracle_ue8m0_exponent(float(amax)))

    def quant_rows(self, x_bf16, block: int, fmt: int):
        """x_bf16: uint16 [T][H].  Returns (codes uint8 [T][H], scales): scales
        float32 [T][H/block] for fmt SCALE_FP32, uint8 exponent bytes for
        SCALE_UE8M0."""
        x = _c(x_bf16, np.uint16)
        T, H = x.shape
        q = np.zeros((T, H), np.uint8)
        sc = np.zeros((T, H // block), np.float32 if fmt == SCALE_FP32 else np.uint8)
        if self.L.oracle_quant_rows(T, H, block, fmt, _p(x), _p(q), _p(sc)) < 0:
            raise ValueError("oracle_quant_rows: bad arguments")
        return q, sc

    def dispatch_quant(self, x_bf16, topk_idx, topk_weights, E: int, block: int, fmt: int):
        """Quantise-on-dispatch.  Returns the dict of dispatch() with recv_x
        holding E4M3 codes uint8 [T*k][H] and recv_scales [T*k][H/block]
        (float32, or uint8 for UE8M0)."""
        x = _c(x_bf16, np.uint16)
        idx = _c(topk_idx, np.int32)
        T, k = idx.shape
        H = x.shape[1]
        cap = T * k
        rq = np.zeros((cap, H), np.uint8)
        rs = np.zeros((cap, H // block), np.float32 if fmt == SCALE_FP32 else np.uint8)
        src = np.full(cap, -1, np.int32)
        rw = np.zeros(cap, np.float32)
        off = np.zeros(E + 1, np.int32)
        s2r = np.zeros((T, k), np.int32)
        w = _c(topk_weights, np.float32)
        st = self.L.oracle_dispatch_quant(T, k, E, H, block, fmt, _p(x), _p(idx), _p(w), _p(rq), _p(rs),
                                          _p(src), _p(rw), _p(off), _p(s2r))
        if st < 0:
            raise ValueError("oracle_dispatch_quant: bad arguments")
        return dict(recv_x=rq, recv_scales=rs, recv_src_idx=src, recv_weights=rw,
                    expert_offsets=off, slot_to_row=s2r, status=st)


    # -- group-deduplicated dispatch --------------------------------------------

    def dispatch_groups(self, x, x_scales, topk_idx, topk_weights, is_token_in_group, E: int, G: int):
        """Returns a dict: recv_x [T*min(G,k)][...], recv_scales, recv_src_idx,
        recv_topk_idx [rows][k], recv_topk_weights [rows][k], group_offsets
        [G+1], token_group_row [T][G], status.  Rows at or past
        group_offsets[G] stay zero (unused capacity)."""
        idx = _c(topk_idx, np.int32)
        T, k = idx.shape
        x = np.ascontiguousarray(x)
        row_bytes = int(np.prod(x.shape[1:])) * x.itemsize
        cap = T * min(G, k)
        recv_x = np.zeros((cap,) + x.shape[1:], x.dtype)
        if x_scales is not None:
            xs = np.ascontiguousarray(x_scales)
            srb = int(np.prod(xs.shape[1:])) * xs.itemsize
            recv_scales = np.zeros((cap,) + xs.shape[1:], xs.dtype)
        else:
            xs, srb, recv_scales = None, 0, None
        src = np.full(cap, -1, np.int32)
        rti = np.full((cap, k), -1, np.int32)
        rtw = np.zeros((cap, k), np.float32)
        goff = np.zeros(G + 1, np.int32)
        tgr = np.zeros((T, G), np.int32)
        w = _c(topk_weights, np.float32)
        bm = _c(is_token_in_group, np.uint32)
        st = self.L.oracle_dispatch_groups(T, k, E, G, row_bytes, srb, _p(x), _p(xs), _p(idx), _p(w), _p(bm),
                                           _p(recv_x), _p(recv_scales), _p(src), _p(rti), _p(rtw), _p(goff),
                                           _p(tgr))
        if st < 0:
            raise ValueError("oracle_dispatch_groups: bad shape")
        return dict(recv_x=recv_x, recv_scales=recv_scales, recv_src_idx=src, recv_topk_idx=rti,
                    recv_topk_weights=rtw, group_offsets=goff, token_group_row=tgr, status=st)

    def combine_groups(self, group_rows_bf16, token_group_row, want_f32=True, want_bf16=True):
        """group_rows_bf16: uint16 [R_g][H].  Returns (out_f32, out_bf16) [T][H]."""
        gr = _c(group_rows_bf16, np.uint16)
        Rg, H = gr.shape
        tgr = _c(token_group_row, np.int32)
        T, G = tgr.shape
        of = np.zeros((T, H), np.float32) if want_f32 else None
        ob = np.zeros((T, H), np.uint16) if want_bf16 else None
        if self.L.oracle_combine_groups(T, G, H, Rg, _p(gr), _p(tgr), _p(of), _p(ob)) < 0:
            raise ValueError("oracle_combine_groups: bad arguments")
        return of, ob


_default = None


def get() -> Oracle:
    """The oracle built from oracle.cpp (compiled on first use if missing)."""
    global _default
    if _default is None:
        other = os.environ.get(LIB_ENV)
        if other:
            _default = Oracle(other)
        else:
            if not os.path.exists(LIB):
                build()
            _default = Oracle(LIB)
    return _default


def f32_to_bf16(a):
    return get().f32_to_bf16(a)


def layout(topk_idx, E, G):
    return get().layout(topk_idx, E, G)


def dispatch(x, x_scales, topk_idx, topk_weights, E):
    return get().dispatch(x, x_scales, topk_idx, topk_weights, E)


def combine(expert_out_bf16, recv_weights, slot_to_row, want_f32=True, want_bf16=True):
    return get().combine(expert_out_bf16, recv_weights, slot_to_row, want_f32, want_bf16)


def quant_rows(x_bf16, block, fmt):
    return get().quant_rows(x_bf16, block, fmt)


def dispatch_quant(x_bf16, topk_idx, topk_weights, E, block, fmt):
    return get().dispatch_quant(x_bf16, topk_idx, topk_weights, E, block, fmt)
