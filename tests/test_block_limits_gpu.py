"""The block-pull copies at their block limit, against the CPU oracle (needs an
MI355X).

A block-pull copy takes its expert's prefix over the earlier blocks from one
16-byte load per lane of a wave, so a plan has at most 256 blocks, and the
compact-list copy of the group rows finds an entry's block by a scan over
the 32 blocks of its XCD.  Rows of 16384 bf16 values (32 KiB) make blocks of
112 tokens (their source rows fit one XCD's L2), so T = 28672 with k = 1 is
exactly 256 blocks, for the flat dispatch and for the group rows' local
permutation alike; one token more takes the push scatter.  Every output is
compared, bit for bit, combine included.
"""
import pytest
import torch

import combine_ep_get_dispatch_amd as M
from combine_ep_get_dispatch_amd import workloads as W
import gpu_harness as GH
from test_parity_groups_gpu import run_groups

pytestmark = pytest.mark.gpu

H = 16384
LIMIT_T = 256 * 112


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    M.load()
    return torch.device("cuda:0")


def workload(T):
    return W.make_workload(f"limit_{T}", T, H, 8, 8, 1, seed=61, expert_kind="double_odd")


def test_plans_at_the_limit():
    q = M.ep_plan_query(GH.shape_of(workload(LIMIT_T)))
    assert q["pull"] and q["pull_nblk"] == 256 and q["pull_tb"] == 112
    assert q["permute_pull"] and q["permute_pull_nblk"] == 256
    q1 = M.ep_plan_query(GH.shape_of(workload(LIMIT_T + 1)))
    assert not q1["pull"] and not q1["permute_pull"]


@pytest.mark.parametrize("T", [LIMIT_T, LIMIT_T + 1], ids=["256_blocks", "push_past_the_limit"])
def test_flat_path_at_the_block_limit(orc, dev, T):
    wl = workload(T)
    print(f"[limit] flat T={T} H={H} E=8 k=1", flush=True)
    r = GH.full_parity(orc, wl, dev)
    print(f"[limit] flat T={T} ok R={r['R']}", flush=True)


def test_group_path_at_the_block_limit(orc, dev):
    run_groups(orc, workload(LIMIT_T), dev)
