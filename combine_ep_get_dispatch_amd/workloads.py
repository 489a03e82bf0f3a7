"""Seeded synthetic workloads for MoE expert-parallel layout / dispatch / combine.

This module only draws inputs: token activations, router choices and router
weights, plus the stand-in "experts" that turn received rows into the rows the
combine step reads back.  It computes none of the layout, dispatch or combine
arithmetic; both the CPU oracle and the GPU path consume exactly the arrays it
returns.

The shapes follow the MSCCL++ EP pages ("MSCCLPP EP implementation - #852"):
the high-throughput bench shape of 256 experts with top-8 routing, the
low-latency bench shape of 128 tokens of hidden size 7168 with top-8 routing,
and hidden rows handled in 16-byte units.  Values are synthetic: activations
are N(0,1), router logits are N(0,1), expert choices are uniform (or Zipf for
the skewed case).  No dataset or trained router is involved.

Random numbers come from numpy's PCG64 generator; every array has its own
sub-stream spawned from one SeedSequence, so one array's size never shifts
another array's draws.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

X_BF16 = "bf16"
X_FP8 = "fp8_e4m3"

FP8_E4M3_MAX = 448.0
SEED_BASE = 0x5EED0000


@dataclass
class Workload:
    """One batch of routed tokens for one GPU's share of the EP path.

    Arrays are host numpy arrays in the layouts the C ABI expects:
      x            uint16 [T][H] (bf16 bit patterns) or uint8 [T][H] (OCP e4m3fn codes)
      x_scales     float32 [T][H/scale_block] or None
      topk_idx     int32 [T][k]; -1 marks a masked slot
      topk_weights float32 [T][k]; 0.0 in masked slots
    """

    name: str
    T: int
    H: int
    E: int
    G: int
    k: int
    x_dtype: str
    scale_block: int
    expert_kind: str
    x: np.ndarray
    x_scales: Optional[np.ndarray]
    topk_idx: np.ndarray
    topk_weights: np.ndarray
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def elt_bytes(self) -> int:
        return 2 if self.x_dtype == X_BF16 else 1

    @property
    def row_bytes(self) -> int:
        return self.H * self.elt_bytes

    @property
    def num_scales(self) -> int:
        return self.H // self.scale_block if self.scale_block else 0

    @property
    def num_masked(self) -> int:
        return int((self.topk_idx < 0).sum())

    @property
    def num_routed(self) -> int:
        """R: received rows = T*k minus masked slots."""
        return self.T * self.k - self.num_masked


# ---------------------------------------------------------------------------
# drawing helpers
# ---------------------------------------------------------------------------

def _streams(seed: int, n: int = 6):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    # torch's CPU float->bfloat16 cast rounds to nearest, ties to even
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _uniform_distinct(rng, T: int, E: int, k: int) -> np.ndarray:
    """k distinct experts per token, uniform; slot order = draw order.

    Each token takes the first k entries of an independent uniform random
    permutation of [0, E) (argsort of i.i.d. uniform keys).
    """
    if T == 0:
        return np.zeros((0, k), dtype=np.int32)
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def _zipf_distinct(rng, T: int, E: int, k: int, alpha: float) -> np.ndarray:
    """k distinct experts per token, drawn one by one without replacement with
    probability proportional to rank**-alpha over the ranks not yet drawn; the
    expert of rank r is perm[r-1] for one seeded permutation of the experts.

    Sequential weighted draws without replacement have the same law as sorting
    log(weight) + Gumbel noise in decreasing order (Gumbel-top-k), which is
    what is used here; slot order = draw order.
    """
    perm = rng.permutation(E).astype(np.int32)
    logw = -alpha * np.log(np.arange(1, E + 1, dtype=np.float64))
    if T == 0:
        return np.zeros((0, k), dtype=np.int32)
    g = rng.gumbel(size=(T, E))
    keys = logw[None, :] + g
    ranks = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return perm[ranks]


def _softmax_weights(rng, idx: np.ndarray) -> np.ndarray:
    """softmax of N(0,1) logits over the unmasked slots of each token (fp64,
    max-subtracted), cast to fp32; masked slots get 0.0."""
    T, k = idx.shape
    logits = rng.standard_normal((T, k))
    valid = idx >= 0
    z = np.where(valid, logits, -np.inf)
    m = np.max(z, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    ex = np.where(valid, np.exp(z - m), 0.0)
    s = ex.sum(axis=1, keepdims=True)
    w = np.divide(ex, s, out=np.zeros_like(ex), where=s > 0)
    return w.astype(np.float32)


def _quantise_e4m3(xf: np.ndarray, block: int):
    """Per-block fp32 scale = amax/448 (1.0 for an all-zero block), codes =
    round-to-nearest-even e4m3fn of x/scale clamped to +-448."""
    T, H = xf.shape
    nb = H // block
    xb = xf.reshape(T, nb, block).astype(np.float32)
    amax = np.abs(xb).max(axis=2) if T else np.zeros((0, nb), np.float32)
    scale = np.where(amax > 0, amax / np.float32(FP8_E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = np.clip(xb / scale[:, :, None], -FP8_E4M3_MAX, FP8_E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(q.reshape(T, H)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


def make_workload(name: str, T: int, H: int, E: int, G: int, k: int, *, seed: int,
                  x_dtype: str = X_BF16, scale_block: int = 0, routing: str = "uniform",
                  zipf_alpha: float = 1.2, mask_frac: float = 0.0,
                  expert_kind: str = "identity", x_kind: str = "normal") -> Workload:
    """Draw one workload.

    x_kind "normal" draws N(0,1) activations; "token_id" sets every element of
    token t to t+1 (exact in bf16 up to 256), so a misplaced row is visible.
    """
    r_x, r_route, r_logit, r_mask, r_perm, _ = _streams(seed)
    if x_kind == "normal":
        xf = r_x.standard_normal((T, H), dtype=np.float32)
    elif x_kind == "token_id":
        xf = np.repeat((np.arange(T, dtype=np.float32) + 1.0)[:, None], H, axis=1)
    else:
        raise ValueError(x_kind)

    if x_dtype == X_BF16:
        x = _f32_to_bf16_bits(xf)
        x_scales = None
        scale_block = 0
    elif x_dtype == X_FP8:
        if scale_block <= 0 or H % scale_block:
            raise ValueError("fp8 needs H divisible by a positive scale_block")
        x, x_scales = _quantise_e4m3(xf, scale_block)
    else:
        raise ValueError(x_dtype)

    if routing == "uniform":
        idx = _uniform_distinct(r_route, T, E, k)
    elif routing == "zipf":
        idx = _zipf_distinct(r_perm, T, E, k, zipf_alpha)
    else:
        raise ValueError(routing)
    idx = np.ascontiguousarray(idx, dtype=np.int32)

    if mask_frac > 0 and T * k > 0:
        m = int(round(mask_frac * T * k))
        flat = r_mask.choice(T * k, size=m, replace=False)
        idx.reshape(-1)[flat] = -1

    w = _softmax_weights(r_logit, idx)
    return Workload(name=name, T=T, H=H, E=E, G=G, k=k, x_dtype=x_dtype, scale_block=scale_block,
                    expert_kind=expert_kind, x=np.ascontiguousarray(x), x_scales=x_scales,
                    topk_idx=idx, topk_weights=np.ascontiguousarray(w), seed=seed,
                    meta=dict(routing=routing, mask_frac=mask_frac, zipf_alpha=zipf_alpha, x_kind=x_kind))


# The five workloads: tiny, DeepSeek-V3-shaped prefill, skewed (Zipf) routing,
# decode-sized fp8, Mixtral-shaped large batch.
CONFIGS = {
    1: dict(name="tiny", T=128, H=256, E=8, G=2, k=2, expert_kind="identity"),
    2: dict(name="dsv3_prefill", T=4096, H=7168, E=256, G=8, k=8, expert_kind="scale_by_id"),
    3: dict(name="skewed_zipf", T=4096, H=7168, E=256, G=8, k=8, routing="zipf", zipf_alpha=1.2,
            mask_frac=0.05, expert_kind="scale_by_id"),
    4: dict(name="decode_fp8", T=128, H=7168, E=256, G=8, k=8, x_dtype=X_FP8, scale_block=128,
            expert_kind="dequant_identity"),
    5: dict(name="mixtral_large", T=16384, H=4096, E=8, G=8, k=2, expert_kind="double_odd"),
}


def config(cid: int, seed: Optional[int] = None) -> Workload:
    spec = dict(CONFIGS[cid])
    return make_workload(seed=SEED_BASE + cid if seed is None else seed, **spec)


def config_dims(cid: int) -> dict:
    """Shape of a config without drawing it."""
    s = dict(CONFIGS[cid])
    s.setdefault("x_dtype", X_BF16)
    s.setdefault("scale_block", 0)
    return s


# ---------------------------------------------------------------------------
# stand-in experts (between dispatch and combine; not part of either)
# ---------------------------------------------------------------------------

def expert_factors(kind: str, E: int) -> np.ndarray:
    """Per-expert multiplier of the stand-in expert, as fp32.

    identity / dequant_identity: 1; scale_by_id: 1 + e/E (exact in fp32);
    double_odd: 2 for odd e, 1 for even e.
    """
    e = np.arange(E, dtype=np.float64)
    if kind in ("identity", "dequant_identity"):
        f = np.ones(E)
    elif kind == "scale_by_id":
        f = 1.0 + e / E
    elif kind == "double_odd":
        f = np.where(e % 2 == 1, 2.0, 1.0)
    else:
        raise ValueError(kind)
    return f.astype(np.float32)


def row_experts(expert_offsets: np.ndarray) -> np.ndarray:
    """Expert id of every received row, from the per-expert offsets [E+1]."""
    counts = np.diff(np.asarray(expert_offsets, dtype=np.int64))
    return np.repeat(np.arange(len(counts), dtype=np.int32), counts)


def expert_outputs(wl: Workload, recv_x, recv_scales, row_expert, device=None) -> torch.Tensor:
    """Stand-in expert outputs: bf16 [R][H] (as a torch bfloat16 tensor).

    bf16 inputs: bf16(float(row) * factor[e]) with torch's nearest-even cast.
    fp8 inputs:  bf16(decode_e4m3(code) * scale[block]) (identity expert on the
    dequantised row).  Works on host numpy arrays or device tensors.
    """
    dev = device
    if isinstance(recv_x, np.ndarray):
        rx = torch.from_numpy(recv_x)
    else:
        rx = recv_x
    if dev is not None:
        rx = rx.to(dev)
    R = rx.shape[0]
    if wl.x_dtype == X_BF16:
        f = torch.from_numpy(expert_factors(wl.expert_kind, wl.E)).to(rx.device)
        re = torch.as_tensor(np.asarray(row_expert), device=rx.device).long()
        vals = rx.view(torch.bfloat16).float() * f[re][:, None]
        return vals.to(torch.bfloat16)
    rs = torch.from_numpy(recv_scales) if isinstance(recv_scales, np.ndarray) else recv_scales
    rs = rs.to(rx.device)
    deq = rx.view(torch.float8_e4m3fn).float().view(R, wl.num_scales, wl.scale_block) * rs[:, :, None]
    return deq.view(R, wl.H).to(torch.bfloat16)
