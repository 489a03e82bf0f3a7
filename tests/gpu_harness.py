"""Run one workload through libmoedisp (GPU) and through the CPU oracle, and
compare them.  Used by the GPU parity tests and the smoke check.

Stand-in expert outputs for combine are computed once on the host from the
ORACLE's received rows and uploaded, so both sides combine identical bytes
and no expected value depends on the GPU path.
"""
from __future__ import annotations

import numpy as np
import torch

import combine_ep_get_dispatch_amd as M
from combine_ep_get_dispatch_amd import workloads as W

# combine bar: bit for bit, in fp32 and in the bf16 rounding.  The kernels sum
# each token's slots in ascending order by fused multiply-add from 0, as the
# oracle does, and keep binary32 subnormals; a kernel that summed in another
# order would need a bar of about 1e-3 relative instead.
COMBINE_REL_TOL = 0.0
COMBINE_ULP_TOL = 0


def shape_of(wl: W.Workload) -> M.moedisp_shape:
    dt = M.FP8_E4M3 if wl.x_dtype == W.X_FP8 else M.BF16
    return M.moedisp_shape.make(wl.T, wl.H, wl.E, wl.G, wl.k, dt, wl.scale_block)


def x_bytes(wl: W.Workload) -> np.ndarray:
    return np.ascontiguousarray(wl.x).view(np.uint8).reshape(wl.T, wl.row_bytes)


def bits16_to_bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


class GpuInputs:
    def __init__(self, wl: W.Workload, dev):
        self.x = torch.from_numpy(x_bytes(wl)).to(dev)
        self.x_scales = torch.from_numpy(wl.x_scales).to(dev) if wl.x_scales is not None else None
        self.topk_idx = torch.from_numpy(wl.topk_idx).to(dev)
        self.topk_weights = torch.from_numpy(wl.topk_weights).to(dev)


def oracle_run(orc, wl: W.Workload):
    tpe, tpg, bm, st_l = orc.layout(wl.topk_idx, wl.E, wl.G)
    d = orc.dispatch(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E)
    d.update(tokens_per_expert=tpe, tokens_per_group=tpg, is_token_in_group=bm, layout_status=st_l)
    return d


def oracle_expert_out(wl: W.Workload, o) -> np.ndarray:
    """bf16 bits [R][H] of the stand-in experts applied to the oracle's rows."""
    R = int(o["expert_offsets"][-1])
    re = W.row_experts(o["expert_offsets"])
    rs = None if o["recv_scales"] is None else o["recv_scales"][:R]
    eo = W.expert_outputs(wl, o["recv_x"][:R], rs, re)
    return eo.view(torch.int16).numpy().view(np.uint16)


def gpu_layout_dispatch(wl: W.Workload, dev, bufs=None, inputs=None):
    shape = shape_of(wl)
    bufs = bufs or M.EpBuffers(shape, dev)
    inputs = inputs or GpuInputs(wl, dev)
    bufs.layout(inputs.topk_idx)
    bufs.dispatch(inputs.x, inputs.x_scales, inputs.topk_idx, inputs.topk_weights)
    st = bufs.status()
    return bufs, inputs, st


def fetch_dispatch(bufs: M.EpBuffers, wl: W.Workload):
    R = int(bufs.expert_offsets[-1].item())
    g = dict(
        tokens_per_expert=bufs.tokens_per_expert.cpu().numpy(),
        tokens_per_group=bufs.tokens_per_group.cpu().numpy(),
        is_token_in_group=bufs.is_token_in_group.cpu().numpy().view(np.uint32),
        expert_offsets=bufs.expert_offsets.cpu().numpy(),
        slot_to_row=bufs.slot_to_row.cpu().numpy(),
        recv_src_idx=bufs.recv_src_idx[:R].cpu().numpy(),
        recv_weights=bufs.recv_weights[:R].cpu().numpy(),
        recv_x=bufs.recv_x[:R].cpu().numpy(),
        recv_scales=None if bufs.recv_scales is None else bufs.recv_scales[:R].cpu().numpy(),
    )
    return g, R


def assert_dispatch_equal(g, o, wl: W.Workload):
    """Bit-exact: counts, bitmap, offsets, handle, rows, scales."""
    R = int(o["expert_offsets"][-1])
    np.testing.assert_array_equal(g["tokens_per_expert"], o["tokens_per_expert"], "tokens_per_expert")
    np.testing.assert_array_equal(g["tokens_per_group"], o["tokens_per_group"], "tokens_per_group")
    np.testing.assert_array_equal(g["is_token_in_group"], o["is_token_in_group"], "is_token_in_group")
    np.testing.assert_array_equal(g["expert_offsets"], o["expert_offsets"], "expert_offsets")
    np.testing.assert_array_equal(g["slot_to_row"], o["slot_to_row"], "slot_to_row")
    np.testing.assert_array_equal(g["recv_src_idx"], o["recv_src_idx"][:R], "recv_src_idx")
    np.testing.assert_array_equal(g["recv_weights"].view(np.uint32), o["recv_weights"][:R].view(np.uint32),
                                  "recv_weights")
    orx = np.ascontiguousarray(o["recv_x"][:R]).view(np.uint8).reshape(R, wl.row_bytes)
    if not np.array_equal(g["recv_x"], orx):
        bad = np.nonzero((g["recv_x"] != orx).any(axis=1))[0]
        raise AssertionError(f"recv_x differs in {bad.size} of {R} rows, first {bad[:8]}")
    if wl.x_scales is not None:
        np.testing.assert_array_equal(g["recv_scales"].view(np.uint32), o["recv_scales"][:R].view(np.uint32),
                                      "recv_scales")


def upload_expert_out(eo_bits: np.ndarray, capacity: int, H: int, dev) -> torch.Tensor:
    eo = torch.zeros((max(capacity, 1), H), dtype=torch.bfloat16, device=dev)
    R = eo_bits.shape[0]
    if R:
        eo[:R] = bits16_to_bf16_tensor(eo_bits).to(dev)
    return eo


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(u):
        u = np.asarray(u, np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def assert_combine_close(g_f32, g_bf16, o_f32, o_bf16):
    """The combine bar (bit for bit), with the relative error and ulp
    distance in the message if it fails."""
    nz = o_f32 != 0
    if nz.any():
        rel = np.abs(g_f32[nz].astype(np.float64) - o_f32[nz]) / np.abs(o_f32[nz].astype(np.float64))
        assert rel.max() <= COMBINE_REL_TOL, f"fp32 combine max rel err {rel.max():.3e}"
    assert np.all(g_f32[~nz] == 0.0), "zero sums must come out exactly zero"
    d = bf16_ulp_distance(g_bf16, o_bf16)
    assert d.size == 0 or d.max() <= COMBINE_ULP_TOL, f"bf16 combine off by {int(d.max())} ulp"
    assert np.array_equal(np.asarray(g_f32, np.float32).view(np.uint32), np.asarray(o_f32, np.float32).view(np.uint32)), \
        "fp32 combine differs in its bits (the sign of a zero)"
    assert np.array_equal(np.asarray(g_bf16, np.uint16), np.asarray(o_bf16, np.uint16)), "bf16 combine differs in its bits"
    return dict(max_ulp=int(d.max()) if d.size else 0,
                exact_f32=float(np.mean(g_f32.view(np.uint32) == o_f32.view(np.uint32))) if g_f32.size else 1.0)


def gpu_combine(bufs: M.EpBuffers, eo: torch.Tensor, wl: W.Workload, dev):
    T, H = wl.T, wl.H
    of = torch.empty((max(T, 1), H), dtype=torch.float32, device=dev)
    ob = torch.empty((max(T, 1), H), dtype=torch.bfloat16, device=dev)
    bufs.combine(eo, of, M.FP32)
    bufs.combine(eo, ob, M.BF16)
    st = bufs.status()
    return of[:T].cpu().numpy(), ob[:T].view(torch.int16).cpu().numpy().view(np.uint16), st


def full_parity(orc, wl: W.Workload, dev):
    """Layout + dispatch bit-exact; combine to the bar on every token."""
    o = oracle_run(orc, wl)
    bufs, inputs, st = gpu_layout_dispatch(wl, dev)
    assert st == o["status"], f"device status {st} != oracle status {o['status']}"
    g, R = fetch_dispatch(bufs, wl)
    assert_dispatch_equal(g, o, wl)
    eo_bits = oracle_expert_out(wl, o)
    eo = upload_expert_out(eo_bits, wl.T * wl.k, wl.H, dev)
    g_f32, g_bf16, st_c = gpu_combine(bufs, eo, wl, dev)
    assert st_c == 0
    o_f32, o_bf16 = orc.combine(eo_bits, o["recv_weights"][:R], o["slot_to_row"])
    res = assert_combine_close(g_f32, g_bf16, o_f32, o_bf16)
    return dict(R=R, **res, bufs=bufs, inputs=inputs, oracle=o, expert_out=eo)
