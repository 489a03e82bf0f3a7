"""GPU test of ep_dispatch_noalloc, the dispatch whose workspace is the
library's static per-device array: through the C ABI, three calls in a row
(each smaller than the one before, the second with an invalid expert id),
each compared with ep_dispatch on its own workspace, bit for bit: offsets,
handle, weights, rows, scales and the status bits."""
import numpy as np
import pytest
import torch

import combine_ep_get_dispatch_amd as M
from combine_ep_get_dispatch_amd import workloads as W
import gpu_harness as GH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.load()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


CASES = [
    # block-pull scatter at the DeepSeek-V3 prefill shape
    ("dsv3", lambda: W.make_workload("na_dsv3", 4096, 7168, 256, 8, 8, seed=301)),
    # smaller, fp8 with scales, masked slots and one invalid id (pull path)
    ("fp8_bad_id", lambda: W.make_workload("na_fp8", 700, 2048, 64, 8, 6, seed=302, routing="zipf", mask_frac=0.1,
                                          x_dtype=W.X_FP8, scale_block=128)),
    # smaller still, push scatter, clean: the status must come back zero
    ("small_push", lambda: W.make_workload("na_small", 100, 512, 16, 4, 4, seed=303)),
]


class Outs:
    def __init__(self, wl, dev):
        cap = wl.T * wl.k
        self.recv_x = torch.zeros((cap, wl.row_bytes), dtype=torch.uint8, device=dev)
        nsc = 0 if wl.x_scales is None else wl.H // wl.scale_block
        self.recv_scales = torch.zeros((cap, nsc), dtype=torch.float32, device=dev) if nsc else None
        self.recv_src_idx = torch.full((cap,), -7, dtype=torch.int32, device=dev)
        self.recv_weights = torch.zeros((cap,), dtype=torch.float32, device=dev)
        self.expert_offsets = torch.full((wl.E + 1,), -7, dtype=torch.int32, device=dev)
        self.slot_to_row = torch.full((wl.T, wl.k), -7, dtype=torch.int32, device=dev)
        self.status = torch.full((1,), -1, dtype=torch.int32, device=dev)


def test_dispatch_noalloc_matches_dispatch(dev):
    runs = []
    for name, make in CASES:
        wl = make()
        if name == "fp8_bad_id":
            wl.topk_idx[5, 1] = wl.E + 3  # invalid id: a masked slot plus BAD_EXPERT_ID
        _say(f"[no_alloc] reference {name} T={wl.T} H={wl.H} E={wl.E} k={wl.k}")
        shape = GH.shape_of(wl)
        bufs = M.EpBuffers(shape, dev)
        inp = GH.GpuInputs(wl, dev)
        bufs.layout(inp.topk_idx)
        bufs.status()  # the layout's bits, cleared
        bufs.dispatch(inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights)
        ref_status = bufs.status()
        runs.append((name, wl, shape, bufs, inp, ref_status, Outs(wl, dev)))
    torch.cuda.synchronize()
    # the three calls back to back on one stream, sharing the static array
    for name, wl, shape, bufs, inp, _, o in runs:
        _say(f"[no_alloc] call {name}")
        M.ep_dispatch_noalloc(shape, inp.x, inp.x_scales, inp.topk_idx, inp.topk_weights, bufs.tokens_per_expert,
                              o.recv_x, o.recv_scales, o.recv_src_idx, o.recv_weights, o.expert_offsets,
                              o.slot_to_row, o.status)
    torch.cuda.synchronize()
    for name, wl, shape, bufs, inp, ref_status, o in runs:
        R = int(bufs.expert_offsets[-1].item())
        assert int(o.status.item()) == ref_status, (name, int(o.status.item()), ref_status)
        assert torch.equal(o.expert_offsets, bufs.expert_offsets), name
        assert torch.equal(o.slot_to_row, bufs.slot_to_row.view(wl.T, wl.k)), name
        assert torch.equal(o.recv_src_idx[:R], bufs.recv_src_idx[:R]), name
        assert torch.equal(o.recv_weights[:R].view(torch.int32), bufs.recv_weights[:R].view(torch.int32)), name
        assert torch.equal(o.recv_x[:R], bufs.recv_x[:R].view(torch.uint8).view(-1, wl.row_bytes)), name
        assert not o.recv_x[R:].any(), name  # rows past R untouched
        if o.recv_scales is not None:
            assert torch.equal(o.recv_scales[:R].view(torch.int32),
                               bufs.recv_scales[:R].view(torch.int32).view(-1, wl.H // wl.scale_block)), name
        _say(f"[no_alloc] {name} ok (R={R}, status={ref_status})")
    assert runs[1][5] & M.binding.DEV_BAD_EXPERT_ID
    assert runs[0][5] == 0 and runs[2][5] == 0
