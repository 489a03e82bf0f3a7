"""The C ABI without a GPU: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments on the host with
the documented codes before anything touches a device."""
import ctypes as C
import os
import re

import pytest
import torch

import combine_ep_get_dispatch_amd as M
from combine_ep_get_dispatch_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moedisp.h")
CALIB_HEADER = os.path.join(ROOT, "include", "moedisp_tools.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from combine_ep_get_dispatch_amd import build
        build.build()
    return M.load()


def declared_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTS), names
    calib = declared_functions(CALIB_HEADER)
    assert set(calib) == set(B.CALIB_EXPORTS), calib
    assert not set(names) & set(calib)
    for n in names + calib:
        assert hasattr(lib, n), f"{n} not exported"


def shape(T=4096, H=7168, E=256, G=8, k=8, dt=M.BF16, sb=0):
    return M.moedisp_shape.make(T, H, E, G, k, dt, sb)


def test_workspace_bytes(lib):
    s = shape()
    n = M.ep_workspace_bytes(s)
    # header + layout partials (32 workgroups of 128 tokens x 264 counts) + per-tile counts (256 experts x 256 tiles)
    assert n >= 256 + 32 * 264 * 4 + 256 * 256 * 4
    assert n % 256 == 0
    assert M.ep_workspace_bytes(shape(T=0)) > 0
    assert M.ep_workspace_bytes(shape(E=255)) == 0          # E % G != 0
    assert M.ep_workspace_bytes(shape(G=64, E=256)) == 0    # more groups than bitmap bits
    assert M.ep_workspace_bytes(shape(H=7)) == 0            # row not whole 16-byte units
    assert M.ep_workspace_bytes(shape(T=8, H=1 << 30)) == 0  # 2 GiB rows: 32-bit row offsets
    assert M.ep_workspace_bytes(shape(T=8, H=(1 << 30) - 8)) > 0
    assert M.ep_workspace_bytes(shape(dt=M.FP8_E4M3, sb=128)) > 0
    assert M.ep_workspace_bytes(shape(dt=M.FP8_E4M3, sb=100)) == 0


FAKE = 0x10000  # never dereferenced: every call below fails its host checks


def p(off=0):
    return C.c_void_p(FAKE + off)


def layout_rc(lib, s, ws_bytes=1 << 30, ws=None, idx=None, tpe=None, tpg=None, bm=None):
    return lib.ep_get_dispatch_layout(C.byref(s), idx or p(), tpe or p(), tpg or p(), bm or p(), ws or p(),
                                      ws_bytes, None)


def dispatch_rc(lib, s, x=None, xs=None, recv_x=None, rs=None, ws=None, ws_bytes=1 << 30, tpe=None):
    return lib.ep_dispatch(C.byref(s), x or p(), xs, p(), p(), tpe or p(), recv_x or p(), rs, p(), p(), p(), p(),
                           ws or p(), ws_bytes, None)


def noalloc_rc(lib, s, status=None, x=None):
    return lib.ep_dispatch_noalloc(C.byref(s), x or p(), None, p(), p(), p(), p(), None, p(), p(), p(), p(),
                                   status, None)


def test_host_checks_dispatch_noalloc(lib):
    """The static-workspace dispatch rejects, before any HIP call: a missing
    or misaligned status word, the usual bad arguments, and shapes whose
    workspace exceeds its 8 MiB array."""
    assert noalloc_rc(lib, shape(), status=None) == B.ERR_INVALID_ARG
    assert noalloc_rc(lib, shape(), status=p(2)) == B.ERR_MISALIGNED
    assert noalloc_rc(lib, shape(E=255), status=p()) == B.ERR_INVALID_ARG
    assert noalloc_rc(lib, shape(), status=p(), x=p(8)) == B.ERR_MISALIGNED
    for T, E, G in ((1000000, 256, 8), (345857, 256, 8), (65536, 4096, 32)):
        s = shape(T=T, E=E, G=G)
        assert lib.ep_workspace_bytes(C.byref(s)) > 8 << 20
        assert noalloc_rc(lib, s, status=p()) == B.ERR_WORKSPACE_TOO_SMALL
    # the largest fitting T of the header's example shape, and the pull shapes
    for T in (345856, 65536, 8192, 4096):
        assert lib.ep_workspace_bytes(C.byref(shape(T=T))) <= 8 << 20
    # the status word is not a workspace: no size argument, checked as 4 bytes
    with pytest.raises(M.MoeDispError, match="status"):
        sh = shape(T=4, H=64, E=8, G=2, k=2)
        z = lambda n, dt=None: torch.zeros(n, dtype=dt or torch.int32)
        M.ep_dispatch_noalloc(sh, z(4 * 128, torch.uint8), None, z(8), z(8, torch.float32), z(8),
                              z(8 * 128, torch.uint8), None, z(8), z(8, torch.float32), z(9), z(8),
                              z(0))


def combine_rc(lib, s, eo=None, out=None, out_dtype=M.BF16, ws_bytes=1 << 30):
    return lib.ep_combine(C.byref(s), eo or p(), p(), p(), p(), out or p(), out_dtype, p(), ws_bytes, None)


def test_host_checks_layout(lib):
    assert layout_rc(lib, shape(E=255)) == B.ERR_INVALID_ARG
    assert layout_rc(lib, shape(T=-1)) == B.ERR_INVALID_ARG
    assert layout_rc(lib, shape(k=0)) == B.ERR_INVALID_ARG
    assert layout_rc(lib, shape(k=9, E=8, G=8)) == B.ERR_INVALID_ARG      # k > E
    assert layout_rc(lib, shape(k=33, E=64)) == B.ERR_UNSUPPORTED
    assert layout_rc(lib, shape(G=64, E=256)) == B.ERR_UNSUPPORTED
    assert layout_rc(lib, shape(E=8192)) == B.ERR_UNSUPPORTED
    assert layout_rc(lib, shape(T=1 << 28, k=8)) == B.ERR_UNSUPPORTED     # T*k rows beyond 30 bits
    assert layout_rc(lib, shape(dt=7)) == B.ERR_UNSUPPORTED
    assert layout_rc(lib, shape(), tpe=p(2)) == B.ERR_MISALIGNED
    assert layout_rc(lib, shape(), ws=p(64)) == B.ERR_MISALIGNED           # ws needs 256-byte alignment
    assert layout_rc(lib, shape(), ws_bytes=100) == B.ERR_WORKSPACE_TOO_SMALL
    assert lib.ep_get_dispatch_layout(C.byref(shape()), None, p(), p(), p(), p(), 1 << 30, None) == B.ERR_INVALID_ARG
    assert lib.ep_get_dispatch_layout(None, p(), p(), p(), p(), p(), 1 << 30, None) == B.ERR_INVALID_ARG


def test_host_checks_layout_notify(lib):
    """The fused layout + notify call: the layout's checks, plus expert_offsets."""
    def rc(s, offs=None, tpe=None, ws_bytes=1 << 30):
        return lib.ep_get_dispatch_layout_notify(C.byref(s), p(), tpe or p(), p(), p(), offs, p(), ws_bytes, None)
    assert rc(shape(), offs=None) == B.ERR_INVALID_ARG
    assert rc(shape(), offs=p(2)) == B.ERR_MISALIGNED
    assert rc(shape(), offs=p(), tpe=p(1)) == B.ERR_MISALIGNED
    assert rc(shape(E=255), offs=p()) == B.ERR_INVALID_ARG
    assert rc(shape(k=33, E=64), offs=p()) == B.ERR_UNSUPPORTED
    assert rc(shape(), offs=p(), ws_bytes=100) == B.ERR_WORKSPACE_TOO_SMALL
    assert lib.ep_get_dispatch_layout_notify(None, p(), p(), p(), p(), p(), p(), 1 << 30, None) == B.ERR_INVALID_ARG


def test_host_checks_dispatch(lib):
    assert dispatch_rc(lib, shape(), x=p(8)) == B.ERR_MISALIGNED           # rows need 16-byte alignment
    assert dispatch_rc(lib, shape(), recv_x=p(4)) == B.ERR_MISALIGNED
    assert dispatch_rc(lib, shape(), tpe=p(1)) == B.ERR_MISALIGNED
    assert dispatch_rc(lib, shape(H=7172)) == B.ERR_UNSUPPORTED             # 14344-byte rows
    fp8 = shape(dt=M.FP8_E4M3, sb=128)
    assert dispatch_rc(lib, fp8) == B.ERR_INVALID_ARG                      # fp8 without scales
    assert dispatch_rc(lib, fp8, xs=p(), rs=None) == B.ERR_INVALID_ARG
    assert dispatch_rc(lib, shape(dt=M.FP8_E4M3, sb=0), xs=p(), rs=p()) == B.ERR_INVALID_ARG
    assert dispatch_rc(lib, shape(sb=128)) == B.ERR_INVALID_ARG             # bf16 with a scale block
    assert dispatch_rc(lib, shape(), ws_bytes=4096) == B.ERR_WORKSPACE_TOO_SMALL
    # null topk_idx
    assert lib.ep_dispatch(C.byref(shape()), p(), None, None, p(), p(), p(), None, p(), p(), p(), p(), p(),
                           1 << 30, None) == B.ERR_INVALID_ARG


def test_host_checks_dispatch_phases(lib):
    s = shape()
    # notify: null topk_idx, null expert_offsets, misaligned offsets, small ws
    assert lib.ep_dispatch_notify(C.byref(s), None, p(), p(), p(), 1 << 30, None) == B.ERR_INVALID_ARG
    assert lib.ep_dispatch_notify(C.byref(s), p(), p(), None, p(), 1 << 30, None) == B.ERR_INVALID_ARG
    assert lib.ep_dispatch_notify(C.byref(s), p(), p(), p(2), p(), 1 << 30, None) == B.ERR_MISALIGNED
    assert lib.ep_dispatch_notify(C.byref(s), p(), p(), p(), p(), 64, None) == B.ERR_WORKSPACE_TOO_SMALL
    assert lib.ep_dispatch_notify(C.byref(shape(E=255)), p(), p(), p(), p(), 1 << 30, None) == B.ERR_INVALID_ARG
    # scatter: null row buffers, misaligned rows
    assert lib.ep_dispatch_scatter(C.byref(s), None, None, p(), p(), p(), p(), None, p(), p(), p(), p(), p(),
                                   1 << 30, None) == B.ERR_INVALID_ARG
    assert lib.ep_dispatch_scatter(C.byref(s), p(8), None, p(), p(), p(), p(), None, p(), p(), p(), p(), p(),
                                   1 << 30, None) == B.ERR_MISALIGNED


def quant_rc(lib, s, block=128, fmt=M.SCALE_FP32, x=None, recv_x=None, rs=None, idx=None, ws_bytes=1 << 30):
    return lib.ep_dispatch_quant(C.byref(s), block, fmt, x or p(), idx or p(), p(), p(), recv_x or p(),
                                 rs or p(), p(), p(), p(), p(), p(), ws_bytes, None)


def test_host_checks_dispatch_quant(lib):
    s = shape()
    assert quant_rc(lib, shape(dt=M.FP8_E4M3, sb=128)) == B.ERR_UNSUPPORTED   # input must be bf16
    assert quant_rc(lib, s, fmt=2) == B.ERR_UNSUPPORTED
    assert quant_rc(lib, s, block=48) == B.ERR_UNSUPPORTED                    # not a power of two
    assert quant_rc(lib, s, block=16) == B.ERR_UNSUPPORTED                    # below 32
    assert quant_rc(lib, s, block=2048) == B.ERR_UNSUPPORTED                  # above 1024
    assert quant_rc(lib, shape(H=96), block=64) == B.ERR_INVALID_ARG          # block does not divide H
    assert quant_rc(lib, s, x=p(8)) == B.ERR_MISALIGNED
    assert quant_rc(lib, s, recv_x=p(8)) == B.ERR_MISALIGNED
    assert quant_rc(lib, s, rs=p(2)) == B.ERR_MISALIGNED                      # fp32 scales need 4 bytes
    assert quant_rc(lib, s, ws_bytes=64) == B.ERR_WORKSPACE_TOO_SMALL
    assert quant_rc(lib, shape(E=255)) == B.ERR_INVALID_ARG
    assert lib.ep_dispatch_quant(C.byref(s), 128, M.SCALE_FP32, p(), p(), p(), p(), p(), None, p(), p(), p(), p(),
                                 p(), 1 << 30, None) == B.ERR_INVALID_ARG     # null scales
    assert lib.ep_dispatch_scatter_quant(C.byref(s), 128, M.SCALE_FP32, None, p(), p(), p(), p(), p(), p(), p(),
                                         p(), p(), p(), 1 << 30, None) == B.ERR_INVALID_ARG
    assert lib.ep_dispatch_scatter_quant(C.byref(s), 96, M.SCALE_UE8M0, p(), p(), p(), p(), p(), p(), p(), p(),
                                         p(), p(), p(), 1 << 30, None) == B.ERR_UNSUPPORTED


def test_host_checks_group_path(lib):
    s = shape()
    P = p
    def groups(x=None, bm=None, tgr=None, goff=None, ws_bytes=1 << 30, sh=s):
        return lib.ep_dispatch_groups(C.byref(sh), x or P(), None, P(), P(), bm or P(), P(), P(), None, P(), P(),
                                      P(), goff or P(), tgr or P(), P(), ws_bytes, None)
    assert groups(x=P(8)) == B.ERR_MISALIGNED
    assert groups(bm=P(2)) == B.ERR_MISALIGNED
    assert groups(ws_bytes=64) == B.ERR_WORKSPACE_TOO_SMALL
    assert groups(sh=shape(E=255)) == B.ERR_INVALID_ARG
    assert lib.ep_dispatch_groups(C.byref(s), P(), None, P(), P(), None, P(), P(), None, P(), P(), P(), P(), P(),
                                  P(), 1 << 30, None) == B.ERR_INVALID_ARG          # null bitmap
    fp8 = shape(dt=M.FP8_E4M3, sb=128)
    assert groups(sh=fp8) == B.ERR_INVALID_ARG                                      # fp8 without scales
    assert lib.ep_group_permute(C.byref(s), P(8), None, P(), P(), P(), P(), None, P(), P(), P(), P(), P(),
                                1 << 30, None) == B.ERR_MISALIGNED
    assert lib.ep_group_permute(C.byref(s), P(), None, P(), P(), P(), P(), None, P(), P(), P(), P(), P(),
                                64, None) == B.ERR_WORKSPACE_TOO_SMALL
    assert lib.ep_group_reduce(C.byref(s), P(), None, P(), P(), P(), P(), M.FP8_E4M3, P(), 1 << 30,
                               None) == B.ERR_UNSUPPORTED
    assert lib.ep_group_reduce(C.byref(s), P(), None, None, P(), P(), P(), M.BF16, P(), 1 << 30,
                               None) == B.ERR_INVALID_ARG                             # null weights
    assert lib.ep_group_reduce(C.byref(s), P(), None, P(), P(), None, P(), M.BF16, P(), 1 << 30,
                               None) == B.ERR_INVALID_ARG                             # null offsets
    assert lib.ep_combine_groups(C.byref(s), P(4), None, P(), P(), M.BF16, P(), 1 << 30, None) == B.ERR_MISALIGNED
    assert lib.ep_combine_groups(C.byref(s), P(), None, None, P(), M.BF16, P(), 1 << 30, None) == B.ERR_INVALID_ARG
    assert lib.ep_combine_groups(None, P(), None, P(), P(), M.BF16, P(), 1 << 30, None) == B.ERR_INVALID_ARG


def test_workspace_covers_group_rows(lib):
    # the local permutation runs over T*min(G,k) group rows: the workspace
    # must hold their per-tile counts too
    for T, E, G, k in ((4096, 256, 8, 8), (100000, 64, 32, 8), (20000, 8, 8, 2)):
        assert M.ep_workspace_bytes(shape(T=T, E=E, G=G, k=k)) >= 256 + 64 * 4 * E


def test_host_checks_layout_dispatch_small(lib):
    def rc(sh, x=None, idx=None, tpe=None, ws_bytes=1 << 30):
        return lib.ep_layout_dispatch_small(C.byref(sh), x or p(), None, idx or p(), p(), tpe or p(), p(), p(), p(),
                                            None, p(), p(), p(), p(), p(), ws_bytes, None)
    assert rc(shape(T=4096)) == B.ERR_UNSUPPORTED                  # 32768 slots: use the two calls
    assert rc(shape(T=1025, k=8)) == B.ERR_UNSUPPORTED             # 8200 slots
    assert rc(shape(T=1000, E=4096, G=8)) == B.ERR_UNSUPPORTED     # LDS: (8000 + 8192 + 1000) * 4 > 60 KiB
    assert rc(shape(T=128), x=p(8)) == B.ERR_MISALIGNED
    assert rc(shape(T=128), tpe=p(2)) == B.ERR_MISALIGNED
    assert rc(shape(T=128), ws_bytes=64) == B.ERR_WORKSPACE_TOO_SMALL
    assert rc(shape(T=128, dt=M.FP8_E4M3, sb=128)) == B.ERR_INVALID_ARG   # fp8 without scales
    assert lib.ep_layout_dispatch_small(C.byref(shape(T=128)), p(), None, None, p(), p(), p(), p(), p(), None, p(),
                                        p(), p(), p(), p(), 1 << 30, None) == B.ERR_INVALID_ARG


def test_host_checks_layout_dispatch_small_padded(lib):
    def rc(sh, C_=128, S=128, B_=0, x=None, ws_bytes=1 << 30, tpe=None):
        return lib.ep_layout_dispatch_small_padded(C.byref(sh), C_, S, B_, x or p(), None, p(), p(), tpe or p(), p(),
                                                   p(), p(), None, p(), p(), p(), p(), ws_bytes, None)
    assert rc(shape(T=128), C_=-1) == B.ERR_INVALID_ARG           # negative capacity
    assert rc(shape(T=128), B_=-1) == B.ERR_INVALID_ARG           # negative base
    assert rc(shape(T=128), S=0, C_=0) == B.ERR_INVALID_ARG       # no slab
    assert rc(shape(T=128), C_=100, S=128, B_=29) == B.ERR_INVALID_ARG  # base + capacity past the slab
    assert rc(shape(T=128, E=256), C_=1, S=1 << 23) == B.ERR_UNSUPPORTED  # E * S >= 2^31 rows
    assert rc(shape(T=4096)) == B.ERR_UNSUPPORTED                 # the small path's own limit
    assert rc(shape(T=128), x=p(8)) == B.ERR_MISALIGNED
    assert rc(shape(T=128), ws_bytes=64) == B.ERR_WORKSPACE_TOO_SMALL
    assert rc(shape(T=128, dt=M.FP8_E4M3, sb=128)) == B.ERR_INVALID_ARG  # fp8 without scales
    # combine over the padded rows: the same host checks as ep_combine, plus the slab
    assert lib.ep_combine_padded(C.byref(shape(T=128)), 0, p(), p(), p(), p(), p(), M.BF16, p(), 1 << 30,
                                 None) == B.ERR_INVALID_ARG
    assert lib.ep_combine_padded(C.byref(shape(T=128)), 1 << 23, p(), p(), p(), p(), p(), M.BF16, p(), 1 << 30,
                                 None) == B.ERR_UNSUPPORTED
    assert lib.ep_combine_padded(C.byref(shape(T=128)), 128, p(2), p(), p(), p(), p(), M.BF16, p(), 1 << 30,
                                 None) == B.ERR_MISALIGNED


def test_host_checks_combine(lib):
    assert combine_rc(lib, shape(), out_dtype=M.FP8_E4M3) == B.ERR_UNSUPPORTED
    assert combine_rc(lib, shape(), eo=p(2)) == B.ERR_MISALIGNED
    assert combine_rc(lib, shape(), out=p(8)) == B.ERR_MISALIGNED
    assert combine_rc(lib, shape(), ws_bytes=0) == B.ERR_WORKSPACE_TOO_SMALL
    assert lib.ep_combine(C.byref(shape()), None, p(), p(), p(), p(), M.BF16, p(), 1 << 30, None) == B.ERR_INVALID_ARG


def test_host_checks_misc(lib):
    v = C.c_int32(0)
    assert lib.ep_check_status(None, 1 << 20, None, C.byref(v)) == B.ERR_INVALID_ARG
    assert lib.ep_check_status(p(), 1 << 20, None, None) == B.ERR_INVALID_ARG
    assert lib.ep_check_status(p(8), 1 << 20, None, C.byref(v)) == B.ERR_MISALIGNED
    assert lib.ep_workspace_init(p(), 16, None) == B.ERR_INVALID_ARG
    assert lib.ep_workspace_init(p(4), 1 << 20, None) == B.ERR_MISALIGNED
    assert lib.ep_probe_copy(p(), p(), 15, None) == B.ERR_UNSUPPORTED
    assert lib.ep_probe_copy(p(4), p(), 16, None) == B.ERR_MISALIGNED
    assert lib.ep_probe_fill(None, 4096, 0, None) == B.ERR_INVALID_ARG
    assert lib.ep_probe_fill(p(), 4095, 0, None) == B.ERR_UNSUPPORTED
    assert lib.ep_probe_fill(p(), 4096, 2, None) == B.ERR_UNSUPPORTED
    assert lib.ep_probe_fill(p(8), 4096, 1, None) == B.ERR_MISALIGNED
    assert lib.ep_probe_read(None, 16, p(), None) == B.ERR_INVALID_ARG
    assert lib.ep_probe_read(p(), 16, None, None) == B.ERR_INVALID_ARG
    assert lib.ep_probe_read(p(), 17, p(), None) == B.ERR_UNSUPPORTED
    assert lib.ep_probe_read(p(8), 16, p(), None) == B.ERR_MISALIGNED
    assert lib.ep_probe_read(p(), 16, p(4), None) == B.ERR_MISALIGNED
    for code in (0, -1, -2, -3, -4, -5):
        assert M.ep_status_string(code) != "unknown status"
    assert M.ep_status_string(-99) == "unknown status"


def test_python_binding_raises_without_gpu_work(lib):
    s = shape(E=255)
    with pytest.raises(M.MoeDispError):
        B._check("ep_get_dispatch_layout", layout_rc(lib, s))


def test_binding_rejects_bad_tensors_before_the_call():
    """The Python binding checks every tensor against the shape before its
    pointer reaches the library: element type, contiguity, size, device.  An
    int64 routing table (torch.topk's index type), a strided view or a buffer
    smaller than the shape needs raises MoeDispError; nothing is launched."""
    import torch
    s = shape(T=16, H=256, E=8, G=2, k=2)
    T, H, E, G, k = 16, 256, 8, 2, 2
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)

    def layout(idx=None, tpe=None, tpg=None, bm=None):
        M.ep_get_dispatch_layout(s, i32(T * k) if idx is None else idx, i32(E) if tpe is None else tpe,
                                 i32(G) if tpg is None else tpg, i32(T) if bm is None else bm, ws)

    def expect(fn, *words):
        with pytest.raises(M.MoeDispError) as e:
            fn()
        assert e.value.code == B.ERR_INVALID_ARG
        for w in words:
            assert w in str(e.value), str(e.value)

    expect(lambda: layout(idx=torch.zeros(T * k, dtype=torch.int64)), "topk_idx", "int64")
    expect(lambda: layout(idx=i32(T * k - 1)), "topk_idx", "bytes")
    expect(lambda: layout(idx=i32(2 * T * k)[::2]), "topk_idx", "contiguous")
    expect(lambda: layout(tpe=i32(E - 1)), "tokens_per_expert")
    expect(lambda: layout(idx=[0] * (T * k)), "torch.Tensor")
    expect(lambda: layout(), "expected a GPU tensor")            # right sizes and types, but host memory

    x = torch.zeros((T, H), dtype=torch.bfloat16)
    def dispatch(**kw):
        a = dict(x=x, x_scales=None, topk_idx=i32(T * k), topk_weights=f32(T * k), tokens_per_expert=i32(E),
                 recv_x=torch.zeros((T * k, H), dtype=torch.bfloat16), recv_scales=None, recv_src_idx=i32(T * k),
                 recv_weights=f32(T * k), expert_offsets=i32(E + 1), slot_to_row=i32(T * k), ws=ws)
        a.update(kw)
        M.ep_dispatch(s, **a)
    expect(lambda: dispatch(x=torch.zeros((T, H), dtype=torch.float32)), "x", "float32")
    expect(lambda: dispatch(recv_x=torch.zeros((T * k - 1, H), dtype=torch.bfloat16)), "recv_x", "bytes")
    expect(lambda: dispatch(topk_weights=torch.zeros(T * k, dtype=torch.float64)), "topk_weights")
    expect(lambda: dispatch(expert_offsets=i32(E)), "expert_offsets")
    expect(lambda: dispatch(slot_to_row=None), "slot_to_row", "required")
    expect(lambda: dispatch(), "expected a GPU tensor")

    fp8 = shape(T=T, H=H, E=E, G=G, k=k, dt=M.FP8_E4M3, sb=128)
    xq = torch.zeros((T, H), dtype=torch.uint8)
    expect(lambda: M.ep_dispatch(fp8, xq, None, i32(T * k), f32(T * k), i32(E), torch.zeros((T * k, H), dtype=torch.uint8),
                                 f32(T * k * 2), i32(T * k), f32(T * k), i32(E + 1), i32(T * k), ws),
           "x_scales", "required")

    eo = torch.zeros((T * k, H), dtype=torch.bfloat16)
    def combine(out, out_dtype, eo=eo):
        M.ep_combine(s, eo, None, f32(T * k), i32(T * k), out, out_dtype, ws)
    # bf16 rows are too small for an fp32 output
    expect(lambda: combine(torch.zeros((T, H), dtype=torch.bfloat16), M.FP32), "out", "bfloat16")
    expect(lambda: combine(torch.zeros((T, H // 2), dtype=torch.float32), M.FP32), "out", "bytes")
    expect(lambda: combine(torch.zeros((T, H), dtype=torch.bfloat16), M.BF16, eo=eo[:, : H // 2]), "expert_out")
    expect(lambda: combine(torch.zeros((T, H), dtype=torch.bfloat16), M.BF16), "expected a GPU tensor")

    expect(lambda: M.ep_probe_copy(torch.zeros(64, dtype=torch.uint8), torch.zeros(32, dtype=torch.uint8), 64),
           "src", "bytes")
