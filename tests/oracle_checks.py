"""Checks that pin the CPU oracle to facts outside itself.

Each check takes an ``Oracle`` object (so the same checks run against
deliberately broken copies of the oracle in the mutation tests) and raises
AssertionError when a fact fails.  The facts come from the definitions of the
operations on the "MSCCLPP EP implementation - #852" page (layout counts and
token-in-rank flags; dispatch/combine as inverse directions sharing a handle;
one combine read per routed copy), from arithmetic closed forms, and from a
library routine (torch's float -> bfloat16 cast).  None of them re-types the
oracle's own loops: integer results are compared with a sort-based
formulation over every routing of tiny shapes, and sums with closed forms.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np
import torch

from combine_ep_get_dispatch_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# bf16 helpers that are not the oracle's
# ---------------------------------------------------------------------------

def torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance between bf16 encodings on the sign-magnitude ordered line."""
    def ordered(u):
        u = np.asarray(u, np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


# ---------------------------------------------------------------------------
# bf16 rounding against the library cast
# ---------------------------------------------------------------------------

def check_bf16_rounding(orc):
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        (rng.standard_normal(5000) * 1e-30).astype(np.float32),
    ]
    # exact ties: low half 0x8000 with even and odd kept parts, and near-ties
    hi = rng.integers(0, 0x7F7F, size=4000, dtype=np.uint32)
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):
        bits = (hi << 16) | np.uint32(low)
        parts.append(bits.view(np.float32))
        parts.append((bits | np.uint32(0x80000000)).view(np.float32))
    # subnormals, zero, the overflow edge, infinities
    sub = np.arange(1, 70000, 7, dtype=np.uint32)
    parts.append(sub.view(np.float32))
    edge = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.39e38, 3.3961e38, 3.4e38,
                     np.finfo(np.float32).max, 1e-45, -1e-45, 1.17549435e-38], np.float32)
    parts.append(edge)
    v = np.concatenate(parts)
    got = orc.f32_to_bf16(v)
    want = torch_bf16_bits(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"bf16 rounding differs from torch at {v[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"
    nan = orc.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x007F) != 0, "NaN must stay NaN"


# ---------------------------------------------------------------------------
# brute force over every routing of tiny shapes
# ---------------------------------------------------------------------------

def token_options(E: int, k: int):
    """Every slot assignment of one token: each slot masked (-1) or an expert,
    routed experts pairwise distinct."""
    opts = []
    for combo in itertools.product(range(-1, E), repeat=k):
        routed = [e for e in combo if e >= 0]
        if len(routed) == len(set(routed)):
            opts.append(combo)
    return opts


def sorted_key_reference(idx: np.ndarray, E: int, G: int):
    """Layout and dispatch rows by a different route than the oracle's: a
    Counter for the counts, Python sets for group membership, and one global
    sort of the (expert, token, slot) keys for the receive order."""
    T, k = idx.shape
    per_group = E // G
    tpe = np.zeros(E, np.int64)
    groups_of = []
    keys = []
    for t in range(T):
        gs = set()
        for j in range(k):
            e = int(idx[t, j])
            if e >= 0:
                tpe[e] += 1
                gs.add(e // per_group)
                keys.append((e, t, j))
        groups_of.append(gs)
    tpg = np.array([sum(1 for gs in groups_of if g in gs) for g in range(G)], np.int64)
    bm = np.array([sum(1 << g for g in gs) for gs in groups_of], np.uint64)
    keys.sort()
    s2r = -np.ones((T, k), np.int64)
    for r, (e, t, j) in enumerate(keys):
        s2r[t, j] = r
    off = np.concatenate([[0], np.cumsum(tpe)])
    return tpe, tpg, bm, off, s2r, keys


def check_bruteforce(orc, shapes=((1, 1, 2, 1), (2, 1, 2, 2), (3, 1, 4, 2), (2, 2, 4, 2),
                                  (3, 2, 4, 2), (2, 2, 4, 1), (2, 2, 4, 4), (2, 3, 3, 3))):
    H = 8
    for (T, k, E, G) in shapes:
        opts = token_options(E, k)
        # structured payload: every element of token t is t+1, every weight
        # names its slot, so a misplaced row or weight is visible
        x = torch_bf16_bits(np.repeat((np.arange(T, dtype=np.float32) + 1)[:, None], H, axis=1))
        w = (np.arange(T * k, dtype=np.float32).reshape(T, k) + 1) / 64.0
        for choice in itertools.product(range(len(opts)), repeat=T):
            idx = np.array([opts[c] for c in choice], np.int32).reshape(T, k)
            tpe, tpg, bm, off, s2r, keys = sorted_key_reference(idx, E, G)
            o_tpe, o_tpg, o_bm, st = orc.layout(idx, E, G)
            assert st == 0, (idx, st)
            assert np.array_equal(o_tpe, tpe), (idx, o_tpe, tpe)
            assert np.array_equal(o_tpg, tpg), (idx, o_tpg, tpg)
            assert np.array_equal(o_bm.astype(np.uint64), bm), (idx, o_bm, bm)
            d = orc.dispatch(x, None, idx, w, E)
            assert np.array_equal(d["expert_offsets"], off), (idx, d["expert_offsets"], off)
            assert np.array_equal(d["slot_to_row"], s2r), (idx, d["slot_to_row"], s2r)
            R = len(keys)
            for r, (e, t, j) in enumerate(keys):
                assert d["recv_src_idx"][r] == t
                assert d["recv_weights"][r] == w[t, j]
                assert np.array_equal(d["recv_x"][r], x[t])
            # identity experts: out[t] = (t+1) * sum of its routed weights,
            # exact in fp32 for these small dyadic weights
            eo = d["recv_x"][:R].reshape(R, H)
            of, ob = orc.combine(eo, d["recv_weights"][:R], d["slot_to_row"])
            for t in range(T):
                want = (t + 1) * float(sum(w[t, j] for j in range(k) if idx[t, j] >= 0))
                assert np.all(of[t] == np.float32(want)), (idx, t, of[t], want)


# ---------------------------------------------------------------------------
# invariants on config-shaped inputs
# ---------------------------------------------------------------------------

def check_layout_invariants(orc, wl):
    tpe, tpg, bm, st = orc.layout(wl.topk_idx, wl.E, wl.G)
    idx = wl.topk_idx
    assert st == 0
    assert int(tpe.sum()) == wl.T * wl.k - int((idx < 0).sum()), "expert counts must sum to T*k - masked"
    assert np.all(tpe >= 0)
    for g in range(wl.G):
        col = (bm >> np.uint32(g)) & 1
        assert int(tpg[g]) == int(col.sum()), "tokens_per_group must be the popcount of its bitmap column"
    assert np.all(tpg <= wl.T)
    assert np.all(bm < (np.uint64(1) << np.uint64(wl.G)))
    reached = int((idx >= 0).any(axis=1).sum()) if wl.T else 0
    assert int(tpg.sum()) >= reached
    assert int((bm != 0).sum()) == reached, "a token has bits iff it has a routed slot"
    # a token's bit count never exceeds its routed slots
    nslots = (idx >= 0).sum(axis=1)
    bits = np.array([bin(int(b)).count("1") for b in bm], np.int64)
    assert np.all(bits <= nslots)
    if wl.E == wl.G:
        assert np.array_equal(tpg, tpe), "one expert per group: group counts equal expert counts"
    return tpe, tpg, bm


def check_dispatch_invariants(orc, wl, d=None):
    if d is None:
        d = orc.dispatch(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E)
    tpe, _, _, _ = orc.layout(wl.topk_idx, wl.E, wl.G)
    off = d["expert_offsets"].astype(np.int64)
    s2r = d["slot_to_row"]
    idx = wl.topk_idx
    R = wl.num_routed
    assert off[0] == 0 and off[-1] == R
    assert np.all(np.diff(off) >= 0)
    assert np.array_equal(np.diff(off), tpe.astype(np.int64)), "segment sizes are the expert counts"
    assert np.all(s2r[idx < 0] == -1)
    rows = s2r[idx >= 0]
    assert np.array_equal(np.sort(rows), np.arange(R)), "slot_to_row must be a bijection onto [0,R)"
    t_of = np.broadcast_to(np.arange(wl.T)[:, None], idx.shape)[idx >= 0]
    e_of = idx[idx >= 0]
    assert np.all((off[e_of] <= rows) & (rows < off[e_of + 1])), "row lies in its expert's segment"
    assert np.array_equal(d["recv_src_idx"][rows], t_of), "src_idx names the source token"
    assert np.array_equal(d["recv_weights"][rows].view(np.uint32),
                          wl.topk_weights[idx >= 0].view(np.uint32)), "weights copied bit for bit"
    src = d["recv_src_idx"][:R]
    assert np.array_equal(d["recv_x"][:R], wl.x[src]), "every received row equals its source row"
    if wl.x_scales is not None:
        assert np.array_equal(d["recv_scales"][:R].view(np.uint32), wl.x_scales[src].view(np.uint32))
    for e in range(wl.E):
        seg = src[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0), "stable in token order (strictly increasing sources)"
    return d


# ---------------------------------------------------------------------------
# combine closed forms
# ---------------------------------------------------------------------------

def _dispatch_and_experts(orc, wl):
    d = orc.dispatch(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E)
    R = wl.num_routed
    re = W.row_experts(d["expert_offsets"])
    eo = W.expert_outputs(wl, d["recv_x"][:R], None if d["recv_scales"] is None else d["recv_scales"][:R], re)
    eo_bits = eo.view(torch.int16).numpy().view(np.uint16)
    return d, eo_bits


def check_combine_exact_dyadic(orc, T=64, H=64, E=16, G=4, k=4, seed=11):
    """Identity experts, weights 1/2, 1/4, 1/8, 1/8 in some slot order: every
    partial sum is exact in fp32, so the result is x itself, bit for bit."""
    wl = W.make_workload("dyadic", T, H, E, G, k, seed=seed, expert_kind="identity")
    rng = np.random.default_rng(seed)
    base = np.array([0.5, 0.25, 0.125, 0.125], np.float32)
    wl.topk_weights = np.stack([rng.permutation(base) for _ in range(T)]).astype(np.float32)
    d, eo = _dispatch_and_experts(orc, wl)
    of, ob = orc.combine(eo, d["recv_weights"], d["slot_to_row"])
    assert np.array_equal(of, bf16_to_f64(wl.x).astype(np.float32)), "sum of dyadic weights = 1 must return x"
    assert np.array_equal(ob, wl.x)


def check_combine_k1_inverse(orc, T=200, H=48, E=8, G=2, seed=12):
    """k = 1 with weight 1.0: combine is the inverse permutation of dispatch."""
    wl = W.make_workload("k1", T, H, E, G, 1, seed=seed, expert_kind="identity")
    wl.topk_weights = np.ones((T, 1), np.float32)
    d, eo = _dispatch_and_experts(orc, wl)
    of, ob = orc.combine(eo, d["recv_weights"], d["slot_to_row"])
    assert np.array_equal(ob, wl.x)


def check_combine_round_trip(orc, wl):
    """Identity experts and weights summing to one: combine returns x to within
    one bf16 ulp (the fp32 sum is within a few fp32 ulps of x)."""
    assert wl.expert_kind in ("identity",)
    d, eo = _dispatch_and_experts(orc, wl)
    of, ob = orc.combine(eo, d["recv_weights"], d["slot_to_row"])
    routed = (wl.topk_idx >= 0).any(axis=1)
    dist = bf16_ulp_distance(ob[routed], wl.x[routed])
    assert dist.size == 0 or int(dist.max()) <= 1, f"round trip off by {int(dist.max())} ulp"
    assert np.all(of[~routed] == 0.0)


def check_combine_closed_form(orc, wl, rel_bound):
    """out[t][h] = x[t][h] * sum_j w_j * c(e_j) for the stand-in expert
    multipliers c; compared in fp64 against a bound on the bf16 rounding of the
    expert outputs plus fp32 accumulation.  Every term has the sign of x, so
    the relative bound is well defined."""
    d, eo = _dispatch_and_experts(orc, wl)
    of, ob = orc.combine(eo, d["recv_weights"], d["slot_to_row"])
    c = W.expert_factors(wl.expert_kind, wl.E).astype(np.float64)
    idx = wl.topk_idx
    w = np.where(idx >= 0, wl.topk_weights.astype(np.float64), 0.0)
    mult = (w * c[np.maximum(idx, 0)]).sum(axis=1)
    if wl.x_dtype == W.X_BF16:
        xv = bf16_to_f64(wl.x)
    else:
        codes = torch.from_numpy(wl.x).view(torch.float8_e4m3fn).double().numpy()
        xv = (codes.reshape(wl.T, wl.num_scales, wl.scale_block)
              * wl.x_scales.astype(np.float64)[:, :, None]).reshape(wl.T, wl.H)
    exact = xv * mult[:, None]
    nz = exact != 0
    rel = np.abs(of.astype(np.float64)[nz] - exact[nz]) / np.abs(exact[nz])
    assert rel.size == 0 or rel.max() <= rel_bound, f"closed form off by {rel.max():.3e} > {rel_bound:.3e}"
    assert np.all(of[~nz] == 0.0)
    # the bf16 output is the fp32 sum rounded once
    assert np.array_equal(ob, torch_bf16_bits(of))


# ---------------------------------------------------------------------------
# hand-worked example
# ---------------------------------------------------------------------------

def check_worked_example(orc, path=os.path.join(GOLDEN, "worked_example.json")):
    with open(path) as f:
        g = json.load(f)
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_weights"], np.float32)
    x = torch_bf16_bits(np.array(g["x"], np.float32))
    E, G = g["E"], g["G"]
    tpe, tpg, bm, st = orc.layout(idx, E, G)
    assert st == 0
    assert tpe.tolist() == g["tokens_per_expert"]
    assert tpg.tolist() == g["tokens_per_group"]
    assert bm.tolist() == g["is_token_in_group"]
    d = orc.dispatch(x, None, idx, w, E)
    R = d["expert_offsets"][-1]
    assert d["expert_offsets"].tolist() == g["expert_offsets"]
    assert d["slot_to_row"].tolist() == g["slot_to_row"]
    assert d["recv_src_idx"][:R].tolist() == g["recv_src_idx"]
    assert d["recv_weights"][:R].tolist() == g["recv_weights"]
    eo = torch_bf16_bits(np.array(g["expert_out"], np.float32))
    of, ob = orc.combine(eo, d["recv_weights"][:R], d["slot_to_row"])
    assert of.tolist() == g["out"]
    assert np.array_equal(ob, torch_bf16_bits(np.array(g["out"], np.float32)))


def check_sum_order(orc, path=os.path.join(GOLDEN, "sum_order.json")):
    """Both combines sum in a fixed fp32 order: the flat one by fused
    multiply-add over ascending slots, the group one over ascending groups.
    Hand-derived cases (the fixture's derivation) whose binary32 results
    change under any other order, under row order, or with the product
    rounded before the add."""
    with open(path) as f:
        g = json.load(f)
    fl = g["flat"]
    eo = torch_bf16_bits(np.array(fl["expert_out"], np.float32))
    assert bf16_to_f64(eo).tolist() == fl["expert_out"], "rows must be exact in bf16"
    w = np.array(fl["recv_weights"], np.float32)
    assert w.astype(np.float64).tolist() == fl["recv_weights"], "weights must be exact in fp32"
    of, ob = orc.combine(eo, w, np.array(fl["slot_to_row"], np.int32))
    assert of.astype(np.float64).tolist() == fl["out_f32"], of
    assert np.array_equal(ob, torch_bf16_bits(of))
    gr = g["groups"]
    rows = torch_bf16_bits(np.array(gr["group_rows"], np.float32))
    assert bf16_to_f64(rows).tolist() == gr["group_rows"]
    of, ob = orc.combine_groups(rows, np.array(gr["token_group_row"], np.int32))
    assert of.astype(np.float64).tolist() == gr["out_f32"], of
    assert np.array_equal(ob, torch_bf16_bits(of))


def check_error_status(orc):
    idx = np.array([[0, 5], [1, 1], [-1, 2]], np.int32)   # 5 >= E: bad id; repeat in token 1
    tpe, tpg, bm, st = orc.layout(idx, 4, 2)
    assert st & 1 and st & 2
    assert tpe.tolist() == [1, 2, 1, 0], "bad id is skipped; a repeat counts as two slots"
    idx2 = np.array([[0, -7]], np.int32)
    _, _, _, st2 = orc.layout(idx2, 4, 2)
    assert st2 == 1, "a negative id other than -1 is a bad id"


# ---------------------------------------------------------------------------
# quantise-on-dispatch: E4M3 codes, FP32 and UE8M0 block scales
# ---------------------------------------------------------------------------

SCALE_FP32, SCALE_UE8M0 = 0, 1


def torch_e4m3_values() -> np.ndarray:
    """Value of every E4M3 code from torch's float8_e4m3fn type (a library
    decoding, independent of the oracle)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def torch_e4m3_codes(v: np.ndarray) -> np.ndarray:
    """torch's float -> float8_e4m3fn cast (nearest-even; only used in range)."""
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_half_spacing(v: np.ndarray) -> np.ndarray:
    """Half the E4M3 grid spacing at |v| (<= 448): 2^(p-4) in [2^p, 2^(p+1)),
    2^-10 below 2^-6."""
    a = np.abs(np.asarray(v, np.float64))
    p = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (p - 4)


def check_e4m3_codes(orc):
    """Decoding of all 256 codes equals torch's; encoding every finite value
    gives its code back; 0x7F and 0xFF are the NaNs; 448 is the largest."""
    codes = np.arange(256, dtype=np.uint8)
    dec = orc.e4m3_to_f64(codes)
    ref = torch_e4m3_values()
    nan = np.isnan(ref)
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(dec), nan)
    assert np.array_equal(dec[~nan], ref[~nan]), "E4M3 decoding differs from float8_e4m3fn"
    assert np.array_equal(np.signbit(dec[~nan]), codes[~nan] >= 0x80)
    assert dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6
    assert np.array_equal(orc.f32_to_e4m3(dec[~nan].astype(np.float32)), codes[~nan]), "encode(decode(c)) != c"


def check_e4m3_rounding(orc):
    """Nearest-even rounding against torch's cast on random values, exact
    midpoints and their neighbours; saturation beyond 448."""
    rng = np.random.default_rng(31)
    mag = 2.0 ** rng.uniform(-13, np.log2(448.0), 30000)
    v = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    assert np.array_equal(orc.f32_to_e4m3(v), torch_e4m3_codes(v)), "rounding differs from the library cast"
    vals = np.unique(torch_e4m3_values()[:0x7F])            # 0 .. 448, ascending
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)     # exact in binary32
    for sgn in (1.0, -1.0):
        m = (sgn * mid).astype(np.float32)
        c = orc.f32_to_e4m3(m)
        assert np.all((c & 1) == 0), "a tie must round to the even code"
        assert np.array_equal(c, torch_e4m3_codes(m))
        up = np.nextafter(np.abs(m), np.float32(np.inf)).astype(np.float32) * np.float32(sgn)
        dn = np.nextafter(np.abs(m), np.float32(0)).astype(np.float32) * np.float32(sgn)
        cu, cd = orc.f32_to_e4m3(up), orc.f32_to_e4m3(dn)
        assert np.array_equal(np.abs(orc.e4m3_to_f64(cu)), vals[1:]), "above a midpoint rounds up"
        assert np.array_equal(np.abs(orc.e4m3_to_f64(cd)), vals[:-1]), "below a midpoint rounds down"
    big = np.array([448.5, 463.9, 464.0, 480.0, 1e6, 3e38, np.inf], np.float32)
    assert np.all(orc.f32_to_e4m3(big) == 0x7E) and np.all(orc.f32_to_e4m3(-big) == 0xFE), "saturation"
    assert orc.f32_to_e4m3(np.array([0.0, -0.0, 2.0 ** -11, -2.0 ** -11], np.float32)).tolist() == \
        [0x00, 0x80, 0x00, 0x80], "signed zeros"


def quant_test_rows(seed=41, B=32, nblk=24):
    """bf16 rows with normal blocks, all-zero blocks, signed-zero blocks, tiny
    (subnormal) blocks, huge blocks and one dominant element per block."""
    rng = np.random.default_rng(seed)
    T, H = 6, B * nblk
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = x.reshape(T, nblk, B)
    xb[0, 1] = 0.0
    xb[0, 2] = -0.0
    xb[1, 3] *= 2.0 ** -130                     # bf16 subnormals
    xb[1, 4] = 0.0
    xb[1, 4, 5] = 2.0 ** -133                   # one tiny nonzero element
    xb[2, 5] *= 1e30
    xb[2, 6] *= 1e-20
    xb[3, :, 0] = rng.choice([-1, 1], nblk) * 2.0 ** rng.integers(-20, 20, nblk)
    xb[4] *= 448.0
    xb[5] = rng.integers(-4, 5, (nblk, B)) * 0.125    # many ties of the grid
    return torch_bf16_bits(x)


def check_quant_fp32(orc, B=32):
    x = quant_test_rows(B=B)
    T, H = x.shape
    q, sc = orc.quant_rows(x, B, SCALE_FP32)
    xf = bf16_to_f64(x).reshape(T, H // B, B)
    amax = np.abs(xf).max(axis=-1)
    s = sc.astype(np.float64)
    zero = amax == 0
    assert np.all(s[zero] == 1.0), "an all-zero block has scale 1"
    assert np.all(np.abs(s[~zero] * 448.0 - amax[~zero]) <= amax[~zero] * 2.0 ** -24 + 2.0 ** -149 * 448), \
        "scale is amax/448 to binary32 precision"
    dec = orc.e4m3_to_f64(q).reshape(xf.shape)
    assert not np.isnan(dec).any()
    v = xf / s[..., None]                        # exact quotient
    err = np.abs(dec - np.clip(v, -448, 448))
    bound = e4m3_half_spacing(np.clip(v, -448, 448)) + np.abs(v) * 2.0 ** -23
    assert np.all(err <= bound), "codes are the nearest E4M3 values of x/scale"
    arg = np.abs(xf).argmax(axis=-1)
    top = np.take_along_axis(q.reshape(xf.shape), arg[..., None], -1)[..., 0]
    normal_scale = s >= 2.0 ** -126
    assert np.all((top[~zero & normal_scale] & 0x7F) == 0x7E), "the block's largest element maps to +-448"
    assert np.array_equal(np.signbit(dec), np.signbit(xf)), "signs (zeros included) are kept"
    # blocks are independent: changing one block changes only its scale and codes
    x2 = x.copy()
    x2[0, 7 * B + 3] = torch_bf16_bits(np.array([1e4], np.float32))[0]
    q2, sc2 = orc.quant_rows(x2, B, SCALE_FP32)
    diff_blocks = np.flatnonzero((q2 != q).reshape(T, -1, B).any(-1).ravel() | (sc2 != sc).ravel())
    assert diff_blocks.tolist() == [7], "only the changed block may change"


def check_quant_ue8m0(orc, B=32):
    x = quant_test_rows(B=B)
    T, H = x.shape
    q, sc = orc.quant_rows(x, B, SCALE_UE8M0)
    xf = bf16_to_f64(x).reshape(T, H // B, B)
    amax = np.abs(xf).max(axis=-1)
    s = sc.astype(np.int64) - 127
    zero = amax == 0
    assert np.all(s[zero] == 0), "an all-zero block has scale 2^0"
    nz = ~zero
    assert np.all(448.0 * np.ldexp(1.0, s[nz]) >= amax[nz]), "no element needs saturation"
    assert np.all((s[nz] == -127) | (448.0 * np.ldexp(1.0, s[nz] - 1) < amax[nz])), "s is the smallest such"
    dec = orc.e4m3_to_f64(q).reshape(xf.shape)
    v = xf * np.ldexp(1.0, -s)[..., None]        # exact
    assert np.all(np.abs(dec - v) <= e4m3_half_spacing(v) * (1 + 2.0 ** -20)), "nearest E4M3 of x * 2^-s"
    assert np.array_equal(np.signbit(dec), np.signbit(xf))
    tiny = amax[1, 3:5]
    assert np.all(s[1, 3:5] == -127) and np.all(tiny > 0)
    assert np.all(q.reshape(xf.shape)[1, 4, 5] == 0x08), "a tiny nonzero block stays nonzero at code zero"
    # exponent choice over every positive finite bf16 amax
    a_bits = np.arange(1, 0x7F80, dtype=np.uint16)
    rows = np.zeros((a_bits.size, B), np.uint16)
    rows[:, 0] = a_bits
    _, sb = orc.quant_rows(rows, B, SCALE_UE8M0)
    a = bf16_to_f64(a_bits)
    ss = sb[:, 0].astype(np.int64) - 127
    assert np.all(448.0 * np.ldexp(1.0, ss) >= a)
    assert np.all((ss == -127) | (448.0 * np.ldexp(1.0, ss - 1) < a))


def check_quant_example(orc, path=os.path.join(GOLDEN, "quant_example.json")):
    with open(path) as f:
        g = json.load(f)
    def val(s):
        if "^" in s:
            base, ex = s.split("^")
            return (-1.0 if base.startswith("-") else 1.0) * 2.0 ** int(ex)
        return float(s)
    x = torch_bf16_bits(np.array([[val(v) for v in g["x"]]], np.float32))
    assert np.array_equal(bf16_to_f64(x)[0], [val(v) for v in g["x"]]), "example values are exact in bf16"
    q, sc = orc.quant_rows(x, g["B"], SCALE_FP32)
    assert q[0].tolist() == g["codes_fp32"]
    assert sc[0].astype(np.float64).tolist() == [m * 2.0 ** p for m, p in g["scales_fp32"]]
    q, sc = orc.quant_rows(x, g["B"], SCALE_UE8M0)
    assert q[0].tolist() == g["codes_ue8m0"]
    assert sc[0].tolist() == g["scales_ue8m0"]


def check_dispatch_quant(orc, wl, B, fmt):
    """Quantise-on-dispatch = the token's quantised row and scales, moved by
    the (separately pinned) dispatch: same handle as the bf16 dispatch, and
    every received row holds its source token's codes and scales."""
    d = orc.dispatch_quant(wl.x, wl.topk_idx, wl.topk_weights, wl.E, B, fmt)
    ref = orc.dispatch(wl.x, None, wl.topk_idx, wl.topk_weights, wl.E)
    for key in ("expert_offsets", "slot_to_row", "recv_src_idx", "recv_weights"):
        assert np.array_equal(d[key], ref[key]), key
    q, sc = orc.quant_rows(wl.x, B, fmt)
    R = wl.num_routed
    src = d["recv_src_idx"][:R]
    assert np.array_equal(d["recv_x"][:R], q[src])
    assert np.array_equal(d["recv_scales"][:R].view(np.uint8), sc[src].view(np.uint8))
    assert d["status"] == ref["status"]


def check_quant_all(orc):
    check_e4m3_codes(orc)
    check_e4m3_rounding(orc)
    check_quant_fp32(orc, 32)
    check_quant_fp32(orc, 128)
    check_quant_ue8m0(orc, 32)
    check_quant_example(orc)
    wl = W.make_workload("quant_mid", 200, 256, 32, 4, 4, seed=25, mask_frac=0.1)
    check_dispatch_quant(orc, wl, 128, SCALE_FP32)
    check_dispatch_quant(orc, wl, 32, SCALE_UE8M0)


# ---------------------------------------------------------------------------
# group-deduplicated dispatch and its combine
# ---------------------------------------------------------------------------

def group_dispatch_reference(idx, bm, E, G):
    """Second formulation: the (group, token) pairs with their bit set,
    sorted; and each pair's restricted slots from the expert -> group map."""
    T, k = idx.shape
    pairs = sorted((g, t) for t in range(T) for g in range(G) if (int(bm[t]) >> g) & 1)
    per = E // G
    rti = np.full((len(pairs), k), -1, np.int64)
    for r, (g, t) in enumerate(pairs):
        for j in range(k):
            e = int(idx[t, j])
            if 0 <= e < E and e // per == g:
                rti[r, j] = e
    return pairs, rti


def check_groups_bruteforce(orc, shapes=((2, 1, 2, 2), (3, 1, 4, 2), (2, 2, 4, 2), (2, 2, 4, 4), (1, 3, 6, 3))):
    for T, k, E, G in shapes:
        opts = token_options(E, k)
        H = 4
        for combo in itertools.product(range(len(opts)), repeat=T):
            idx = np.array([opts[c] for c in combo], np.int32).reshape(T, k)
            w = (np.arange(T * k, dtype=np.float32).reshape(T, k) + 1) / 64
            x = torch_bf16_bits(np.repeat((np.arange(T, dtype=np.float32) + 1)[:, None], H, axis=1))
            _, tpg, bm, _ = orc.layout(idx, E, G)
            d = orc.dispatch_groups(x, None, idx, w, bm, E, G)
            pairs, rti = group_dispatch_reference(idx, bm, E, G)
            Rg = len(pairs)
            assert d["group_offsets"][-1] == Rg
            assert np.array_equal(np.diff(d["group_offsets"]), tpg)
            assert d["recv_src_idx"][:Rg].tolist() == [t for _, t in pairs]
            assert np.array_equal(d["recv_topk_idx"][:Rg], rti)
            srcs = [t for _, t in pairs]
            exp_w = np.where(rti >= 0, w[srcs], 0.0) if Rg else np.zeros((0, k))
            assert np.array_equal(d["recv_topk_weights"][:Rg], exp_w)
            assert np.array_equal(d["recv_x"][:Rg], x[srcs])
            tgr = np.full((T, G), -1)
            for r, (g, t) in enumerate(pairs):
                tgr[t, g] = r
            assert np.array_equal(d["token_group_row"], tgr)


def ht_path(orc, wl):
    """layout -> group dispatch -> local permutation (dispatch of the group
    rows) -> stand-in experts -> local reduce (combine of the group rows) ->
    combine of the groups.  Returns every intermediate."""
    tpe, tpg, bm, _ = orc.layout(wl.topk_idx, wl.E, wl.G)
    gd = orc.dispatch_groups(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, bm, wl.E, wl.G)
    Rg = int(gd["group_offsets"][-1])
    gs = None if gd["recv_scales"] is None else gd["recv_scales"][:Rg]
    pm = orc.dispatch(gd["recv_x"][:Rg], gs, gd["recv_topk_idx"][:Rg], gd["recv_topk_weights"][:Rg], wl.E)
    R = int(pm["expert_offsets"][-1])
    re = W.row_experts(pm["expert_offsets"])
    eo = W.expert_outputs(wl, pm["recv_x"][:R], None if pm["recv_scales"] is None else pm["recv_scales"][:R], re)
    eo_bits = eo.view(torch.int16).numpy().view(np.uint16)
    _, part = orc.combine(eo_bits, pm["recv_weights"][:R], pm["slot_to_row"], want_f32=False)
    of, ob = orc.combine_groups(part, gd["token_group_row"])
    return dict(tpe=tpe, tpg=tpg, bm=bm, gd=gd, Rg=Rg, pm=pm, R=R, eo_bits=eo_bits, part=part, out_f32=of, out_bf16=ob)


def check_groups_invariants(orc, wl):
    h = ht_path(orc, wl)
    gd, pm, Rg = h["gd"], h["pm"], h["Rg"]
    off = gd["group_offsets"].astype(np.int64)
    assert np.array_equal(np.diff(off), h["tpg"]), "group segments are the layout's group counts"
    src = gd["recv_src_idx"][:Rg]
    for g in range(wl.G):
        assert np.all(np.diff(src[off[g]:off[g + 1]]) > 0), "token order inside a group"
    assert np.array_equal(gd["recv_x"][:Rg], wl.x[src]), "group rows are their token's row"
    tgr = gd["token_group_row"]
    assert np.array_equal(np.sort(tgr[tgr >= 0]), np.arange(Rg)), "token_group_row is a bijection onto [0,R_g)"
    assert np.array_equal(tgr >= 0, ((h["bm"][:, None] >> np.arange(wl.G)) & 1).astype(bool))
    rti = gd["recv_topk_idx"][:Rg]
    assert int((rti >= 0).sum()) == wl.num_routed, "every routed slot lands in exactly one group row"
    # the local permutation of the group rows is the flat dispatch
    flat = orc.dispatch(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E)
    R = h["R"]
    assert np.array_equal(pm["expert_offsets"], flat["expert_offsets"])
    assert np.array_equal(pm["recv_x"][:R], flat["recv_x"][:R]), "permuted rows equal the flat dispatch's"
    assert np.array_equal(src[pm["recv_src_idx"][:R]], flat["recv_src_idx"][:R])
    assert np.array_equal(pm["recv_weights"][:R].view(np.uint32), flat["recv_weights"][:R].view(np.uint32))
    per = wl.E // wl.G
    idx = wl.topk_idx
    t_of, j_of = np.nonzero(idx >= 0)
    grow = tgr[t_of, idx[t_of, j_of] // per]
    assert np.array_equal(pm["slot_to_row"][grow, j_of], flat["slot_to_row"][t_of, j_of])
    return h


def check_groups_combine_exact(orc, T=97, H=32, E=16, G=4, seed=51):
    """k = 2 with weights 1/2, 1/2 and identity experts: every group partial
    (x/2 or x) and the sum over groups are exact, so the result is x."""
    wl = W.make_workload("ht_exact", T, H, E, G, 2, seed=seed, expert_kind="identity")
    wl.topk_weights = np.full((T, 2), 0.5, np.float32)
    h = ht_path(orc, wl)
    assert np.array_equal(h["out_bf16"], wl.x)


def check_groups_combine_closed_form(orc, wl, rel_bound):
    """out = x * sum_j w_j c(e_j) in fp64, within the bound of two bf16
    roundings (expert output, group partial) plus fp32 sums."""
    h = ht_path(orc, wl)
    c = W.expert_factors(wl.expert_kind, wl.E).astype(np.float64)
    idx = wl.topk_idx
    w = np.where(idx >= 0, wl.topk_weights.astype(np.float64), 0.0)
    exact = bf16_to_f64(wl.x) * (w * c[np.maximum(idx, 0)]).sum(axis=1)[:, None]
    of = h["out_f32"].astype(np.float64)
    nz = exact != 0
    rel = np.abs(of[nz] - exact[nz]) / np.abs(exact[nz])
    assert rel.size == 0 or rel.max() <= rel_bound, f"group combine off by {rel.max():.3e} > {rel_bound:.3e}"
    assert np.all(of[~nz] == 0.0)
    assert np.array_equal(h["out_bf16"], torch_bf16_bits(h["out_f32"]))


# one rounding of each group partial on top of the flat path's bounds
GROUP_BOUND = {"identity": 2.0 ** -8 + 2.0 ** -15, "double_odd": 2.0 ** -8 + 2.0 ** -15,
               "scale_by_id": 2.0 ** -7 + 2.0 ** -15}


def group_configs():
    return [
        W.make_workload("ht_uniform", 300, 64, 64, 8, 8, seed=52, expert_kind="scale_by_id"),
        W.make_workload("ht_zipf", 300, 64, 256, 8, 8, seed=53, routing="zipf", mask_frac=0.05,
                        expert_kind="scale_by_id"),
        W.make_workload("ht_mixtral", 500, 64, 8, 8, 2, seed=54, expert_kind="double_odd"),
        W.make_workload("ht_g_lt_k", 200, 64, 16, 2, 6, seed=55, expert_kind="identity"),
    ]


def check_groups_all(orc):
    check_groups_bruteforce(orc)
    check_groups_combine_exact(orc)
    for wl in group_configs():
        check_groups_invariants(orc, wl)
        check_groups_combine_closed_form(orc, wl, GROUP_BOUND[wl.expert_kind])


# ---------------------------------------------------------------------------
# padded (low-latency) layout
# ---------------------------------------------------------------------------

def check_padded_example(orc, path=os.path.join(GOLDEN, "padded_example.json")):
    with open(path) as f:
        g = json.load(f)
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_weights"], np.float32)
    T, k = idx.shape
    x = (np.arange(T * 4, dtype=np.uint16) + 1).reshape(T, 4)
    d = orc.dispatch_padded(x, None, idx, w, g["E"], g["C"], g["S"], g["B"], fill=0xFFFF)
    assert d["status"] == g["status"]
    assert d["slot_to_row"].tolist() == g["slot_to_row"]
    for r, (t, wt) in g["rows"].items():
        r = int(r)
        assert d["recv_src_idx"][r] == t and d["recv_weights"][r] == np.float32(wt), r
        assert np.array_equal(d["recv_x"][r], x[t]), r
    for r in g["untouched_rows"]:
        assert d["recv_src_idx"][r] == -1 and np.all(d["recv_x"][r] == 0xFFFF), r


def check_padded_bruteforce(orc, shapes=((2, 1, 2, 1), (3, 1, 2, 2), (2, 2, 3, 1), (3, 2, 3, 2), (2, 3, 3, 1))):
    """Every routing of tiny shapes, against one global sort of the
    (expert, token, slot) keys: the i-th key of expert e takes row
    e*S + B + i while i < C; the status reports an expert past C."""
    H = 4
    for (T, k, E, C) in shapes:
        for (S, B) in ((C, 0), (C + 2, 1)):
            opts = token_options(E, k)
            x = (np.arange(T * H, dtype=np.uint16) + 1).reshape(T, H)
            w = (np.arange(T * k, dtype=np.float32).reshape(T, k) + 1) / 64.0
            for choice in itertools.product(range(len(opts)), repeat=T):
                idx = np.array([opts[c] for c in choice], np.int32).reshape(T, k)
                tpe, _, _, _, _, keys = sorted_key_reference(idx, E, 1)
                d = orc.dispatch_padded(x, None, idx, w, E, C, S, B, fill=0)
                want = -np.ones((T, k), np.int64)
                seen = {}
                for (e, t, j) in keys:
                    i = seen.get(e, 0)
                    seen[e] = i + 1
                    if i < C:
                        want[t, j] = e * S + B + i
                assert np.array_equal(d["slot_to_row"], want), (idx, C, S, B, d["slot_to_row"], want)
                assert d["status"] == (16 if tpe.max(initial=0) > C else 0), (idx, C, d["status"])
                taken = set(int(r) for r in want.ravel() if r >= 0)
                for t in range(T):
                    for j in range(k):
                        r = want[t, j]
                        if r >= 0:
                            assert d["recv_src_idx"][r] == t and d["recv_weights"][r] == w[t, j]
                            assert np.array_equal(d["recv_x"][r], x[t])
                for r in range(E * S):
                    if r not in taken:
                        assert d["recv_src_idx"][r] == -1 and not d["recv_x"][r].any()


def check_padded_vs_flat(orc, wl, S_extra=3, B=2):
    """Without overflow the padded layout is the flat one shifted per expert:
    the row of a slot is e*S + B + (its flat row - expert_offsets[e]); rows,
    scales, sources and weights follow the slot."""
    d = orc.dispatch(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E)
    off = d["expert_offsets"]
    C = int(np.diff(off).max(initial=0))
    S = C + B + S_extra
    p = orc.dispatch_padded(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E, C, S, B)
    assert p["status"] == d["status"]
    flat = d["slot_to_row"]
    idx = wl.topk_idx
    routed = flat >= 0
    e = np.where(routed, idx, 0).astype(np.int64)
    want = np.where(routed, e * S + B + (flat - off[e]), -1)
    assert np.array_equal(p["slot_to_row"], want)
    fr = flat[routed]
    pr = want[routed]
    assert np.array_equal(p["recv_x"][pr], d["recv_x"][fr])
    assert np.array_equal(p["recv_src_idx"][pr], d["recv_src_idx"][fr])
    assert np.array_equal(p["recv_weights"][pr].view(np.uint32), d["recv_weights"][fr].view(np.uint32))
    if d["recv_scales"] is not None:
        assert np.array_equal(p["recv_scales"][pr], d["recv_scales"][fr])
    # one capacity less than the fullest expert: exactly its last slot is dropped
    if C > 0:
        q = orc.dispatch_padded(wl.x, wl.x_scales, wl.topk_idx, wl.topk_weights, wl.E, C - 1, S, B)
        assert q["status"] & 16
        assert (q["slot_to_row"] >= 0).sum() == routed.sum() - int((np.diff(off) == C).sum())


def check_padded_all(orc):
    check_padded_example(orc)
    check_padded_bruteforce(orc)
    for wl in (W.config(1), W.config(4),
               W.make_workload("padded_zipf", 300, 64, 64, 8, 8, seed=56, routing="zipf", mask_frac=0.1)):
        check_padded_vs_flat(orc, wl)


ALL_BASIC = [check_bf16_rounding, check_bruteforce, check_combine_exact_dyadic, check_combine_k1_inverse,
             check_worked_example, check_sum_order, check_error_status, check_padded_all]


def small_configs():
    """Config-shaped workloads small enough for a quick CPU pass."""
    return [
        W.config(1),
        W.make_workload("uniform_mid", 512, 64, 64, 8, 8, seed=21, expert_kind="scale_by_id"),
        W.make_workload("zipf_mid", 512, 64, 256, 8, 8, seed=22, routing="zipf", mask_frac=0.05,
                        expert_kind="scale_by_id"),
        W.make_workload("fp8_mid", 32, 512, 32, 8, 8, seed=23, x_dtype=W.X_FP8, scale_block=128,
                        expert_kind="dequant_identity"),
        W.make_workload("mixtral_mid", 1024, 64, 8, 8, 2, seed=24, expert_kind="double_odd"),
    ]


def run_all(orc):
    """Every pin in one go (used by the mutation test)."""
    for chk in ALL_BASIC:
        chk(orc)
    check_quant_all(orc)
    check_groups_all(orc)
    for wl in small_configs():
        check_layout_invariants(orc, wl)
        check_dispatch_invariants(orc, wl)
    wl1 = W.config(1)
    check_combine_round_trip(orc, wl1)
    for wl in small_configs()[1:]:
        check_combine_closed_form(orc, wl, rel_bound=CLOSED_FORM_BOUND[wl.expert_kind])


# bf16 rounding of each stand-in expert output (<= 2^-8 relative: 8 significant
# bits, round to nearest) plus fp32
# accumulation of up to 8 same-sign terms (< 9 * 2^-24 relative)
# (the fp8 dequantisation adds one fp32 rounding before the bf16 one)
CLOSED_FORM_BOUND = {
    "scale_by_id": 2.0 ** -8 + 9 * 2.0 ** -24,
    "dequant_identity": 2.0 ** -8 + 10 * 2.0 ** -24,
    "double_odd": 9 * 2.0 ** -24,
    "identity": 9 * 2.0 ** -24,
}
