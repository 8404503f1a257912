"""GPU parity over a seeded sweep of random shapes, routings and plan options.

Each case draws its token count, hidden and intermediate sizes, expert count,
top-k, tile height, weight layout, recipe (FP8 block scales or FP8 x MXFP4),
launch flags (the ring pool has its own tests against a full-pool
control), intermediate-scale granularity, power-of-two requant scales,
activation clamp, skewed routing and a few masked or out-of-range slots, all
from one fixed seed, keeping only combinations the plan accepts.  The HIP
path runs through the C ABI and the result goes through parity_util.verify
against the oracle with the matching options, over every token; the call's
routing tables are compared bit for bit with the oracle's, and FP8 calls
that fit the no-alloc entry point's scratch are repeated through it and
compared bit for bit with the workspace forward."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import oracle
import workload as wl
from parity_util import host_copy_for_oracle, host_dict, say, verify

pytestmark = pytest.mark.gpu

NOALLOC_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES

FLAGS = {
    "none": 0,
    "direct": moe.MOE_FLAG_DIRECT_TILES,
    "single": moe.MOE_FLAG_SINGLE_LAUNCH,
    "split": moe.MOE_FLAG_SPLIT_LAUNCH,
}


def _accepted(c):
    """The plan's shape and option rules (moe_plan_create rejects the rest)."""
    H, I, mx, tile, flag = c["H"], c["I"], c["mx"], c["tile"], c["flag"]
    if c["packed"] and H % 256:
        return False
    if tile == 128 and not (H % 256 == 0 and min(H, I) // 128 >= (3 if mx else 2)):
        return False
    if mx and (c["gran"] or c["pow2"] or flag == "single"):
        return False
    if flag == "single" and c["gran"] == 64:
        return False
    return True


def _cases(n=64, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        K = int(rng.integers(1, 7))
        c = dict(
            mx=bool(rng.random() < 0.3),
            K=K,
            E=int(rng.integers(K, 25)),
            T=int(rng.choice([1, 2, 3, 7, 16, 33, 64, 100, 129, 200, 257])),
            H=int(rng.choice([256, 384, 512, 768])),
            I=int(rng.choice([128, 256, 384, 512])),
            tile=int(rng.choice([0, 16, 32, 64, 128])),
            packed=bool(rng.random() < 0.5),
            flag=str(rng.choice(list(FLAGS))),
            gran=int(rng.choice([0, 0, 64])),
            pow2=bool(rng.random() < 0.2),
            clamp=float(rng.choice([0.0, 0.0, 0.5])),
            skew=bool(rng.random() < 0.3),
            n_mask=int(rng.integers(0, 4)),
            seed=int(rng.integers(0, 1 << 30)),
        )
        if _accepted(c):
            out.append(c)
    return out


CASES = _cases()


def _name(c):
    return (f"{'mx' if c['mx'] else 'fp8'}-T{c['T']}-H{c['H']}-I{c['I']}-E{c['E']}-K{c['K']}"
            f"-t{c['tile']}-{c['flag']}{'-pk' if c['packed'] else ''}"
            f"{'-g64' if c['gran'] else ''}{'-pow2' if c['pow2'] else ''}"
            f"{'-clamp' if c['clamp'] else ''}{'-skew' if c['skew'] else ''}")


def _inputs(c):
    cfg = wl.custom_config(c["T"], c["H"], c["I"], c["E"], c["K"], c["skew"])
    inp = (wl.make_inputs_mx if c["mx"] else wl.make_inputs)(cfg, c["seed"], "cpu")
    rng = np.random.default_rng(c["seed"])
    idx = inp["topk_idx"].clone()
    for _ in range(c["n_mask"]):   # masked (-1) or out-of-range slots
        t, j = int(rng.integers(0, c["T"])), int(rng.integers(0, c["K"]))
        idx[t, j] = int(rng.choice([-1, c["E"], c["E"] + 77]))
    inp["topk_idx"] = idx
    return host_dict(inp), {k: v.cuda() for k, v in inp.items()}


@pytest.mark.parametrize("c", CASES, ids=[_name(c) for c in CASES])
def test_random_case_against_oracle(c):
    say(f"sweep {_name(c)} seed={c['seed']}")
    host, dev = _inputs(c)
    T, E, K = c["T"], c["E"], c["K"]
    flags = FLAGS[c["flag"]] | (moe.MOE_FLAG_POW2_SCALE if c["pow2"] else 0)
    r = moe.MoEForward(c["H"], c["I"], E, K, T, tile_m=c["tile"],
                       weight_layout=moe.MOE_WEIGHTS_PACKED if c["packed"] else
                       moe.MOE_WEIGHTS_ROW_MAJOR,
                       flags=flags, act_sf_gran=c["gran"], activation_clamp=c["clamp"],
                       recipe=moe.MOE_RECIPE_MXFP4 if c["mx"] else moe.MOE_RECIPE_FP8_BLOCK128)
    if c["mx"]:
        w1, w1_sf, w2, w2_sf = r.prepare_mx(dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"])
    else:
        (w1, w2), w1_sf, w2_sf = r.prepare(dev["w1"], dev["w2"]), dev["w1_sf"], dev["w2_sf"]
    y = r.forward(dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_w"], w1, w1_sf, w2, w2_sf)
    torch.cuda.synchronize()
    # the call's routing, bit for bit
    info = moe.moe_plan_info(r.plan, T)
    rc, ro, rrs, rsr, bad = oracle.route(host["idx"], E, info["tile_m"], info["pool_rows"])
    assert np.array_equal(r.view("counts", T).cpu().numpy(), rc)
    assert np.array_equal(r.view("offsets", T).cpu().numpy(), ro)
    assert np.array_equal(r.view("row_src", T).cpu().numpy(), rrs)
    assert np.array_equal(r.view("src_row", T).cpu().numpy(), rsr)
    status = moe.moe_read_status(r.plan, T, r.workspace)
    assert status[1] == bad
    # the forward, step by step
    oflags = ((oracle.ORC_POW2_SCALE if c["pow2"] else 0) |
              (oracle.ORC_SF_GRAN64 if c["gran"] == 64 else 0))
    verify(y, r, host, _name(c), oflags=oflags, clamp=c["clamp"])
    # the entry point that allocates nothing (FP8 plans whose workspace fits
    # its scratch): the same kernels, so the same bits
    if not c["mx"] and moe.moe_workspace_bytes(r.plan, T) <= NOALLOC_BYTES:
        y_na = torch.full_like(y, 0x7FC0)
        moe.moe_forward_noalloc(r.plan, T, dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_w"],
                                w1, w1_sf, w2, w2_sf, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y), "no-alloc entry point differs"


def _large_cases(n=12, seed=20261203):
    """Larger calls (many tiles per workgroup, several K blocks per tile),
    checked on sampled tokens."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        K = int(rng.integers(1, 9))
        c = dict(
            mx=bool(rng.random() < 0.3),
            K=K,
            E=int(rng.integers(max(K, 8), 65)),
            T=int(rng.integers(300, 2049)),
            H=int(rng.choice([1024, 1536, 2048])),
            I=int(rng.choice([512, 768, 1024])),
            tile=int(rng.choice([0, 16, 32, 64, 128])),
            packed=bool(rng.random() < 0.5),
            flag=str(rng.choice(list(FLAGS))),
            gran=int(rng.choice([0, 0, 64])),
            pow2=bool(rng.random() < 0.2),
            clamp=float(rng.choice([0.0, 0.0, 0.5])),
            skew=bool(rng.random() < 0.5),
            n_mask=int(rng.integers(0, 4)),
            seed=int(rng.integers(0, 1 << 30)),
        )
        if _accepted(c):
            out.append(c)
    return out


LARGE = _large_cases()


@pytest.mark.parametrize("c", LARGE, ids=[_name(c) for c in LARGE])
def test_random_large_case_sampled(c):
    say(f"sweep large {_name(c)} seed={c['seed']}")
    cfg = wl.custom_config(c["T"], c["H"], c["I"], c["E"], c["K"], c["skew"])
    inp = (wl.make_inputs_mx if c["mx"] else wl.make_inputs)(cfg, c["seed"], "cuda")
    rng = np.random.default_rng(c["seed"])
    idx = inp["topk_idx"].clone()
    for _ in range(c["n_mask"]):
        t, j = int(rng.integers(0, c["T"])), int(rng.integers(0, c["K"]))
        idx[t, j] = int(rng.choice([-1, c["E"], c["E"] + 77]))
    inp["topk_idx"] = idx
    T, E, K = c["T"], c["E"], c["K"]
    flags = FLAGS[c["flag"]] | (moe.MOE_FLAG_POW2_SCALE if c["pow2"] else 0)
    r = moe.MoEForward(c["H"], c["I"], E, K, T, tile_m=c["tile"],
                       weight_layout=moe.MOE_WEIGHTS_PACKED if c["packed"] else
                       moe.MOE_WEIGHTS_ROW_MAJOR,
                       flags=flags, act_sf_gran=c["gran"], activation_clamp=c["clamp"],
                       recipe=moe.MOE_RECIPE_MXFP4 if c["mx"] else moe.MOE_RECIPE_FP8_BLOCK128)
    if c["mx"]:
        w1, w1_sf, w2, w2_sf = r.prepare_mx(inp["w1"], inp["w1_sf"], inp["w2"], inp["w2_sf"])
    else:
        (w1, w2), w1_sf, w2_sf = r.prepare(inp["w1"], inp["w2"]), inp["w1_sf"], inp["w2_sf"]
    y = r.forward(inp["x"], inp["x_sf"], inp["topk_idx"], inp["topk_w"], w1, w1_sf, w2, w2_sf)
    torch.cuda.synchronize()
    host_idx = inp["topk_idx"].cpu().numpy()
    info = moe.moe_plan_info(r.plan, T)
    rc, ro, rrs, rsr, bad = oracle.route(host_idx, E, info["tile_m"], info["pool_rows"])
    assert np.array_equal(r.view("counts", T).cpu().numpy(), rc)
    assert np.array_equal(r.view("offsets", T).cpu().numpy(), ro)
    assert np.array_equal(r.view("row_src", T).cpu().numpy(), rrs)
    assert np.array_equal(r.view("src_row", T).cpu().numpy(), rsr)
    assert moe.moe_read_status(r.plan, T, r.workspace)[1] == bad
    toks = sorted({0, T - 1, *rng.choice(T, 14, replace=False).tolist()})
    oflags = ((oracle.ORC_POW2_SCALE if c["pow2"] else 0) |
              (oracle.ORC_SF_GRAN64 if c["gran"] == 64 else 0))
    verify(y, r, host_copy_for_oracle(inp, toks), _name(c), tokens=toks, oflags=oflags,
           clamp=c["clamp"])
