"""The combines' summation order on the GPU (needs an MI355X): the
hand-derived binary32 cases of tests/golden/sum_order.json, whose fp32
results change under any other slot or group order, under row order, or with
the product rounded before the add.  The kernels sum a token's slots in
ascending order by fused multiply-add and its group rows in ascending group
order, as the oracle does, so here the fp32 and bf16 outputs must equal the
fixture's (and the oracle's) bit for bit.
"""
import json
import os

import numpy as np
import pytest
import torch

import combine_ep_get_dispatch_amd as M
import oracle_checks as K

pytestmark = pytest.mark.gpu

FIXTURE = os.path.join(os.path.dirname(__file__), "golden", "sum_order.json")
H = 8  # one 16-byte unit of bf16 per row; the fixture's two columns first, zeros after


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.load()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def fixture():
    with open(FIXTURE) as f:
        return json.load(f)


def _rows(values, n_rows):
    """bf16 bit patterns [n_rows][H]: the fixture's rows in the first columns."""
    a = np.zeros((n_rows, H), np.float32)
    v = np.array(values, np.float32)
    a[: v.shape[0], : v.shape[1]] = v
    return K.torch_bf16_bits(a)


def test_combine_sum_order_bit_exact(orc, dev, fixture):
    fl = fixture["flat"]
    s2r = np.array(fl["slot_to_row"], np.int32)
    T, k = s2r.shape
    shape = M.moedisp_shape.make(T, H, 4, 1, k, M.BF16, 0)
    eo_bits = _rows(fl["expert_out"], T * k)
    w = np.zeros(T * k, np.float32)
    w[: len(fl["recv_weights"])] = np.array(fl["recv_weights"], np.float32)
    bufs = M.EpBuffers(shape, dev)
    eo = torch.from_numpy(eo_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    wt = torch.from_numpy(w).to(dev)
    st = torch.from_numpy(s2r).to(dev)
    out32 = torch.full((T, H), -5.0, dtype=torch.float32, device=dev)
    out16 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    M.ep_combine(shape, eo, None, wt, st, out32, M.FP32, bufs.ws)
    M.ep_combine(shape, eo, None, wt, st, out16, M.BF16, bufs.ws)
    assert bufs.status() == 0
    g32 = out32.cpu().numpy()
    want = np.zeros((T, H))
    want[:, :2] = np.array(fl["out_f32"])
    assert g32.astype(np.float64).tolist() == want.tolist(), g32[:, :2]
    o32, o16 = orc.combine(eo_bits, w, s2r)
    assert np.array_equal(g32.view(np.uint32), o32.view(np.uint32))
    assert np.array_equal(out16.cpu().view(torch.int16).numpy().view(np.uint16), o16)


def test_combine_groups_sum_order_bit_exact(orc, dev, fixture):
    gr = fixture["groups"]
    tgr = np.array(gr["token_group_row"], np.int32)
    T, G = tgr.shape
    shape = M.moedisp_shape.make(T, H, G, G, G, M.BF16, 0)   # one expert per group, k = G
    rows_bits = _rows(gr["group_rows"], T * G)
    bufs = M.EpBuffers(shape, dev)
    rows = torch.from_numpy(rows_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    t = torch.from_numpy(tgr).to(dev)
    out32 = torch.full((T, H), -5.0, dtype=torch.float32, device=dev)
    out16 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    M.ep_combine_groups(shape, rows, None, t, out32, M.FP32, bufs.ws)
    M.ep_combine_groups(shape, rows, None, t, out16, M.BF16, bufs.ws)
    assert bufs.status() == 0
    g32 = out32.cpu().numpy()
    want = np.zeros((T, H))
    want[:, :2] = np.array(gr["out_f32"])
    assert g32.astype(np.float64).tolist() == want.tolist(), g32[:, :2]
    o32, o16 = orc.combine_groups(rows_bits, tgr)
    assert np.array_equal(g32.view(np.uint32), o32.view(np.uint32))
    assert np.array_equal(out16.cpu().view(torch.int16).numpy().view(np.uint16), o16)


def test_combine_subnormal_products_bit_exact(orc, dev):
    """Products and sums in the binary32 subnormal range (below 2^-126) and
    crossing into the normal range: the kernel keeps subnormals as the
    oracle's IEEE arithmetic does (no flush to zero), in fp32 and in the bf16
    rounding."""
    T, k = 4, 2
    shape = M.moedisp_shape.make(T, H, 4, 1, k, M.BF16, 0)
    vals = np.zeros((T * k, H), np.float32)
    w = np.zeros(T * k, np.float32)
    s2r = np.arange(T * k, dtype=np.int32).reshape(T, k)
    # token 0: 2^-100 * 2^-30 = 2^-130 twice -> 2^-129 (subnormal)
    vals[0, 0] = vals[1, 0] = 2.0 ** -30
    w[0] = w[1] = 2.0 ** -100
    # token 1: a normal product plus a subnormal one: 2^-126 + 2^-140
    vals[2, 0] = 2.0 ** -26
    w[2] = 2.0 ** -100
    vals[3, 0] = 2.0 ** -40
    w[3] = 2.0 ** -100
    # token 2: 1.5 * 2^-126 (normal) plus 2^-127 (subnormal): 2^-125
    vals[4, 0] = 1.5
    w[4] = 2.0 ** -126
    vals[5, 0] = 0.5
    w[5] = 2.0 ** -126
    # token 3: the smallest subnormal, 2^-149, and its negation: +0
    vals[6, 0] = 2.0 ** -49
    w[6] = 2.0 ** -100
    vals[7, 0] = -(2.0 ** -49)
    w[7] = 2.0 ** -100
    eo_bits = K.torch_bf16_bits(vals)
    assert np.array_equal(K.bf16_to_f64(eo_bits), vals.astype(np.float64)), "rows exact in bf16"
    o32, o16 = orc.combine(eo_bits, w, s2r)
    assert o32[0, 0] == np.float32(2.0 ** -129) and o32[2, 0] == np.float32(2.0 ** -125)
    assert o32[3, 0] == 0.0
    bufs = M.EpBuffers(shape, dev)
    eo = torch.from_numpy(eo_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    out32 = torch.full((T, H), -5.0, dtype=torch.float32, device=dev)
    out16 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    wt = torch.from_numpy(w).to(dev)
    st = torch.from_numpy(s2r).to(dev)
    M.ep_combine(shape, eo, None, wt, st, out32, M.FP32, bufs.ws)
    M.ep_combine(shape, eo, None, wt, st, out16, M.BF16, bufs.ws)
    assert bufs.status() == 0
    g32 = out32.cpu().numpy()
    assert np.array_equal(g32.view(np.uint32), o32.view(np.uint32)), (g32[:, 0], o32[:, 0])
    assert np.array_equal(out16.cpu().view(torch.int16).numpy().view(np.uint16), o16)
