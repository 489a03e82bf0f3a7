"""GPU parity of quantise-on-dispatch (ep_dispatch_quant) against the CPU
oracle (needs an MI355X).

Bit-exact: E4M3 codes of every received row, the per-block scales (FP32 bits
or UE8M0 bytes), offsets and the handle.  The cases cover both scale formats,
block sizes from 32 to 1024 channels, the DeepSeek-V3 shape at full size in
the benchmark's launch configuration, decode-sized grids that split rows
across workgroups, rows wider than one pass of the workgroup, ragged token
counts, masked slots, and rows built to hit the quantiser's special cases:
all-zero and signed-zero blocks, bf16 subnormals, huge values, exact E4M3
midpoints and one dominant element per block.
"""
import numpy as np
import pytest
import torch

import combine_ep_get_dispatch_amd as M
from combine_ep_get_dispatch_amd import workloads as W
import gpu_harness as GH
import oracle_checks as K

pytestmark = pytest.mark.gpu

FP32, UE8M0 = M.SCALE_FP32, M.SCALE_UE8M0


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.load()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def gpu_quant(wl, dev, block, fmt, two_phase=False):
    bufs = M.EpBuffers(GH.shape_of(wl), dev).enable_quant(block, fmt)
    inp = GH.GpuInputs(wl, dev)
    bufs.layout(inp.topk_idx)
    if two_phase:
        bufs.dispatch_notify(inp.topk_idx)
        bufs.dispatch_scatter_quant(inp.x, inp.topk_idx, inp.topk_weights)
    else:
        bufs.dispatch_quant(inp.x, inp.topk_idx, inp.topk_weights)
    st = bufs.status()
    return bufs, inp, st


def assert_quant_equal(bufs, o, st):
    assert st == o["status"], f"device status {st} != oracle status {o['status']}"
    R = int(o["expert_offsets"][-1])
    np.testing.assert_array_equal(bufs.expert_offsets.cpu().numpy(), o["expert_offsets"], "expert_offsets")
    np.testing.assert_array_equal(bufs.slot_to_row.cpu().numpy(), o["slot_to_row"], "slot_to_row")
    np.testing.assert_array_equal(bufs.recv_src_idx[:R].cpu().numpy(), o["recv_src_idx"][:R], "recv_src_idx")
    np.testing.assert_array_equal(bufs.recv_weights[:R].cpu().numpy().view(np.uint32),
                                  o["recv_weights"][:R].view(np.uint32), "recv_weights")
    gq = bufs.recv_q[:R].cpu().numpy()
    if not np.array_equal(gq, o["recv_x"][:R]):
        bad = np.argwhere(gq != o["recv_x"][:R])
        r, h = bad[0]
        raise AssertionError(f"codes differ at {len(bad)} places, first row {r} col {h}: "
                             f"gpu {gq[r, h]:#04x} oracle {o['recv_x'][r, h]:#04x}")
    gs = bufs.recv_qscales[:R].cpu().numpy()
    np.testing.assert_array_equal(gs.view(np.uint8), o["recv_scales"][:R].view(np.uint8), "scales")
    return R


def run_case(orc, wl, dev, block, fmt, two_phase=False):
    _say(f"[quant] {wl.name} T={wl.T} H={wl.H} E={wl.E} k={wl.k} block={block} fmt={fmt} two_phase={two_phase}")
    o = orc.dispatch_quant(wl.x, wl.topk_idx, wl.topk_weights, wl.E, block, fmt)
    bufs, inp, st = gpu_quant(wl, dev, block, fmt, two_phase)
    R = assert_quant_equal(bufs, o, st)
    _say(f"[quant] {wl.name} ok R={R}")
    return bufs, inp, o


def special_workload(B):
    """Rows of quantiser special cases (oracle_checks.quant_test_rows) routed
    like any other workload."""
    x = K.quant_test_rows(seed=41 + B, B=B)
    T, H = x.shape
    wl = W.make_workload(f"special_B{B}", T, H, 8, 2, 2, seed=60 + B)
    wl.x = x
    return wl


CASES = {
    "tiny_b32_fp32": (lambda: W.config(1), 32, FP32),
    "tiny_b128_ue8m0": (lambda: W.config(1), 128, UE8M0),
    "special_b32_fp32": (lambda: special_workload(32), 32, FP32),
    "special_b32_ue8m0": (lambda: special_workload(32), 32, UE8M0),
    "special_b128_fp32": (lambda: special_workload(128), 128, FP32),
    "special_b128_ue8m0": (lambda: special_workload(128), 128, UE8M0),
    "dsv3_ragged_b128_fp32": (lambda: W.make_workload("dsv3_ragged", 601, 7168, 256, 8, 8, seed=31), 128, FP32),
    "zipf_ragged_b32_ue8m0": (lambda: W.make_workload("zipf_ragged", 777, 7168, 256, 8, 8, seed=32,
                                                      routing="zipf", mask_frac=0.05), 32, UE8M0),
    "decode_split_b128_fp32": (lambda: W.make_workload("decode", 128, 7168, 256, 8, 8, seed=34), 128, FP32),
    "decode_split_b1024_ue8m0": (lambda: W.make_workload("decode", 128, 7168, 256, 8, 8, seed=34), 1024, UE8M0),
    "wide_rows_two_passes_b64_fp32": (lambda: W.make_workload("wide", 1030, 17408, 16, 4, 4, seed=35), 64, FP32),
    "narrow_rows_b32_ue8m0": (lambda: W.make_workload("narrow", 300, 32, 16, 4, 4, seed=36, mask_frac=0.3),
                              32, UE8M0),
    "empty": (lambda: W.make_workload("empty", 0, 256, 8, 2, 2, seed=37), 32, FP32),
    "all_masked": (lambda: W.make_workload("all_masked", 40, 256, 8, 2, 2, seed=38, mask_frac=1.0), 32, UE8M0),
    "mixtral_b128_fp32": (lambda: W.make_workload("mixtral_ragged", 3001, 4096, 8, 8, 2, seed=33), 128, FP32),
}


@pytest.mark.parametrize("name", list(CASES))
def test_quant_parity(orc, dev, name):
    make, block, fmt = CASES[name]
    run_case(orc, make(), dev, block, fmt)


@pytest.mark.parametrize("block,fmt", [(128, FP32), (32, UE8M0)])
def test_quant_parity_full_size(orc, dev, block, fmt):
    """DeepSeek-V3 prefill shape (T=4096, H=7168, E=256, top-8), every row."""
    run_case(orc, W.config(2), dev, block, fmt)


def test_quant_two_phase_equals_one_call(orc, dev):
    wl = W.make_workload("two_phase", 515, 7168, 256, 8, 8, seed=39, routing="zipf", mask_frac=0.05)
    run_case(orc, wl, dev, 128, FP32, two_phase=True)


def test_quant_then_combine_round_trip(orc, dev):
    """Quantised dispatch, dequantising identity experts, combine: the GPU
    combine of the GPU rows matches the oracle combine of the oracle rows."""
    wl = W.make_workload("quant_rt", 333, 1024, 32, 4, 4, seed=40, mask_frac=0.1)
    bufs, inp, o = run_case(orc, wl, dev, 128, FP32)
    R = int(o["expert_offsets"][-1])
    codes = torch.from_numpy(o["recv_x"][:R]).view(torch.float8_e4m3fn).float()
    sc = torch.from_numpy(o["recv_scales"][:R]).repeat_interleave(128, dim=1)
    eo_bits = (codes * sc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    eo = GH.upload_expert_out(eo_bits, wl.T * wl.k, wl.H, dev)
    g_f32, g_bf16, st = GH.gpu_combine(bufs, eo, wl, dev)
    assert st == 0
    o_f32, o_bf16 = orc.combine(eo_bits, o["recv_weights"][:R], o["slot_to_row"])
    GH.assert_combine_close(g_f32, g_bf16, o_f32, o_bf16)
    # and the result is x to within the E4M3 quantisation error (weights sum to 1)
    x = K.bf16_to_f64(wl.x)
    routed = (wl.topk_idx >= 0).any(axis=1)
    err = np.abs(o_f32.astype(np.float64) - x)[routed]
    amax = np.abs(x).reshape(wl.T, -1, 128).max(-1).repeat(128, axis=1)[routed]
    assert np.all(err <= np.abs(x[routed]) * 2.0 ** -4 + amax / 448 * 2.0 ** -9 + 1e-6)


def amax_sweep_workload():
    """One 32-channel block per token, token t's block having the largest
    magnitude bf16 bits t + 1: every positive finite bf16 value (subnormals
    included) is some block's amax.  The other 31 channels hold seeded bf16
    values of random sign whose magnitude bits do not exceed the amax bits (so
    they do not exceed the amax).  E = 1 and k = 1 keep the rows in token
    order."""
    n = 0x7F7F  # bits 0x0001 .. 0x7F7F
    rng = np.random.default_rng(0xA3A3)
    amax_bits = np.arange(1, n + 1, dtype=np.uint32)
    frac = rng.random((n, 31))
    mag = np.floor(frac * (amax_bits[:, None] + 1)).astype(np.uint32)  # 0 .. amax bits
    sign = (rng.random((n, 31)) < 0.5).astype(np.uint32) << 15
    x = np.empty((n, 32), np.uint16)
    x[:, 0] = amax_bits | ((rng.random(n) < 0.5).astype(np.uint32) << 15)
    x[:, 1:] = mag | sign
    perm = rng.permuted(np.tile(np.arange(32), (n, 1)), axis=1)  # the amax anywhere in the block
    x = np.take_along_axis(x, perm, axis=1)
    wl = W.make_workload("amax_sweep", n, 32, 1, 1, 1, seed=42)
    wl.x = np.ascontiguousarray(x)
    return wl


@pytest.mark.parametrize("fmt,two_phase", [(UE8M0, False), (FP32, False), (UE8M0, True), (FP32, True)])
def test_quant_every_bf16_amax(orc, dev, fmt, two_phase):
    """Scale and codes of a block whose amax is each positive finite bf16
    value in turn, bit-exact against the oracle (whose UE8M0 exponent rule is
    itself pinned by brute force over the same values)."""
    run_case(orc, amax_sweep_workload(), dev, 32, fmt, two_phase)


@pytest.mark.parametrize("fmt", [FP32, UE8M0], ids=["fp32", "ue8m0"])
def test_quant_inconsistent_counts_are_reported(dev, fmt):
    """tokens_per_expert changed so that it disagrees with the routing (and
    its total exceeds the T*k receive rows): ep_dispatch_quant reports
    BAD_LAYOUT, writes every slot's handle entry, and names no row outside
    the receive buffer."""
    wl = W.make_workload("quant_bad_counts", 300, 512, 16, 4, 4, seed=88)
    bufs = M.EpBuffers(GH.shape_of(wl), dev).enable_quant(128, fmt)
    inp = GH.GpuInputs(wl, dev)
    bufs.layout(inp.topk_idx)
    assert bufs.status() == 0
    _say(f"[quant-err] fmt={fmt}")
    bufs.tokens_per_expert[0] += 3
    bufs.tokens_per_expert[wl.E - 1] -= 1
    bufs.slot_to_row.fill_(-7)
    bufs.dispatch_quant(inp.x, inp.topk_idx, inp.topk_weights)
    assert bufs.status() & M.binding.DEV_BAD_LAYOUT
    s = bufs.slot_to_row.cpu().numpy()
    assert s.min() >= -1 and s.max() < wl.T * wl.k
