"""GPU parity of the recipe options against the oracle: per-64 intermediate
scales (dual-half L2), power-of-two requant scales, the activation clamp
(both recipes, direct and LDS tiles, split-K, single launch) -- each through
parity_util.verify with the oracle's matching option -- and the activation
quantisation entry point (codes and scales bit-exact: both sides take every
rounding decision in f32 the same way)."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import oracle
import workload as wl
from parity_util import host_copy_for_oracle, host_dict, say, small_case, verify

pytestmark = pytest.mark.gpu


def run_opts(dev, tile_m=0, flags=0, gran=0, clamp=0.0, mx=False):
    T, H = dev["x"].shape
    E, twoI, _ = dev["w1"].shape
    K = dev["topk_idx"].shape[1]
    r = moe.MoEForward(H, twoI // 2, E, K, T,
                       tile_m=tile_m, flags=flags, act_sf_gran=gran, activation_clamp=clamp,
                       recipe=moe.MOE_RECIPE_MXFP4 if mx else moe.MOE_RECIPE_FP8_BLOCK128)
    y = r.forward(dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_w"], dev["w1"], dev["w1_sf"],
                  dev["w2"], dev["w2_sf"])
    torch.cuda.synchronize()
    return y, r


@pytest.mark.parametrize("tile_m", [16, 32, 64])
def test_per64_scales_all_direct_tiles(tile_m):
    host, dev = small_case(45, 512, 384, 12, 3, 501, mask={(0, 1): -1, (7, 2): 99}, skew=True)
    y, r = run_opts(dev, tile_m=tile_m, gran=64)
    info = moe.moe_plan_info(r.plan, 45)
    assert info["act_sf_gran"] == 64 and info["l2_group_tiles"] == 1
    verify(y, r, host, f"per-64 tile {tile_m}", oflags=oracle.ORC_SF_GRAN64)
    # against the per-128 recipe: a different (still accurate) result
    y128, _ = run_opts(dev, tile_m=tile_m)
    assert not torch.equal(y, y128)


@pytest.mark.parametrize("tile_m", [64, 128])
def test_per64_scales_lds_tiles(tile_m):
    # the shared-A (64-row) and LDS-staged (128-row) tiles with per-64 h
    # scales: L1 requantises each 64-column half on its own, L2 multiplies
    # dual halves; same oracle reading as the direct tiles (bitwise equal to
    # them), and the 128-row tile on a 4-workgroup grid walks many tiles
    host, dev = small_case(300, 512, 384, 16, 4, 503, mask={(0, 1): -1, (9, 2): 77}, skew=True)
    y, r = run_opts(dev, tile_m=tile_m, gran=64)
    info = moe.moe_plan_info(r.plan, 300)
    assert info["act_sf_gran"] == 64 and info["kernel"] == (2 if tile_m == 64 else 1), info
    verify(y, r, host, f"per-64 LDS tile {tile_m}", oflags=oracle.ORC_SF_GRAN64)
    y_direct, rd = run_opts(dev, tile_m=64, gran=64, flags=moe.MOE_FLAG_DIRECT_TILES)
    assert moe.moe_plan_info(rd.plan, 300)["kernel"] == 0
    assert torch.equal(y, y_direct), "per-64: LDS tile and direct tile differ"
    if tile_m == 128:
        y_small, _ = run_opts(dev, tile_m=128, gran=64, flags=moe.MOE_FLAG_TEST_SMALL_GRID)
        assert torch.equal(y, y_small)


@pytest.mark.parametrize("name", ["flash_prefill", "pro_prefill", "skewed"])
def test_per64_full_size_sampled(name):
    # configs 3-5 with per-64 h scales on the library's prefill tiles,
    # sampled tokens through the whole chain
    cfg = wl.CONFIGS[name]
    seed = wl.default_seed(cfg)
    inp = wl.make_inputs(cfg, seed, "cuda")
    r = moe.MoEForward(cfg.H, cfg.I, cfg.E, cfg.K, cfg.T, weight_layout=moe.MOE_WEIGHTS_PACKED,
                       act_sf_gran=64)
    info = moe.moe_plan_info(r.plan, cfg.T)
    say(f"per-64 {name}: tile {info['tile_m']} kernel {info['kernel']}")
    assert info["act_sf_gran"] == 64 and info["kernel"] in (1, 2)
    w1, w2 = r.prepare(inp["w1"], inp["w2"])
    y = r.forward(inp["x"], inp["x_sf"], inp["topk_idx"], inp["topk_w"], w1, inp["w1_sf"], w2,
                  inp["w2_sf"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    toks = sorted({0, cfg.T - 1, *rng.choice(cfg.T, 16, replace=False).tolist()})
    host = host_copy_for_oracle(inp, toks)
    del w1, w2
    verify(y, r, host, f"per-64 {name} ({len(toks)} tokens)", tokens=toks,
           oflags=oracle.ORC_SF_GRAN64)
    r.close()
    del inp
    torch.cuda.empty_cache()


def test_per64_rule_and_split_k():
    # -1: the rule of PR #440 (hidden 256 is not a multiple of 512 -> 64)
    cfg = wl.CONFIGS["tiny"]
    host, dev = small_case(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, wl.default_seed(cfg))
    y, r = run_opts(dev, gran=-1)
    assert moe.moe_plan_info(r.plan, cfg.T)["act_sf_gran"] == 64
    verify(y, r, host, "tiny rule", oflags=oracle.ORC_SF_GRAN64)
    # one and two tokens at the flash shape: L1 split-K with per-64 scales
    base = wl.CONFIGS["flash_decode"]
    full = wl.make_inputs(wl.custom_config(2, base.H, base.I, base.E, base.K),
                          wl.default_seed(base), "cuda")
    for T in (1, 2):
        inp = dict(full)
        for k in ("x", "x_sf", "topk_idx", "topk_w"):
            inp[k] = full[k][:T].contiguous()
        y, r = run_opts(inp, gran=64)
        assert moe.moe_plan_info(r.plan, T)["l1_split"] > 1
        h = host_copy_for_oracle(inp, list(range(T)))
        verify(y, r, h, f"per-64 split-K T={T}", oflags=oracle.ORC_SF_GRAN64)
    del full


@pytest.mark.parametrize("tile_m", [16, 64, 128])
def test_pow2_scales(tile_m):
    host, dev = small_case(160, 512, 384, 6, 3, 502, mask={(3, 0): -1})
    y, r = run_opts(dev, tile_m=tile_m, flags=moe.MOE_FLAG_POW2_SCALE)
    verify(y, r, host, f"pow2 tile {tile_m}", oflags=oracle.ORC_POW2_SCALE)
    sf = r.view("h_sf", 160).cpu().numpy()
    used = sf[r.view("src_row", 160).cpu().numpy()[r.view("src_row", 160).cpu().numpy() >= 0]]
    m, _ = np.frexp(used.astype(np.float64))
    assert np.all(m == 0.5)  # every scale a power of two


@pytest.mark.parametrize("tile_m", [16, 64, 128])
def test_activation_clamp_fp8(tile_m):
    host, dev = small_case(160, 512, 384, 6, 3, 503)
    clamp = 0.05  # well inside the range of gate/up here: the clamp is active
    y, r = run_opts(dev, tile_m=tile_m, clamp=clamp)
    verify(y, r, host, f"clamp tile {tile_m}", clamp=clamp)
    y0, _ = run_opts(dev, tile_m=tile_m)
    assert not torch.equal(y, y0)


@pytest.mark.parametrize("tile_m", [16, 64, 128])
def test_activation_clamp_mxfp4(tile_m):
    cfg = wl.custom_config(160, 512, 384, 6, 3)
    inp = wl.make_inputs_mx(cfg, 504, "cpu")
    host = host_dict(inp)
    dev = {k: v.cuda() for k, v in inp.items()}
    y, r = run_opts(dev, tile_m=tile_m, clamp=0.05, mx=True)
    verify(y, r, host, f"MX clamp tile {tile_m}", clamp=0.05)


def test_single_launch_with_pow2_and_clamp_matches_split_launches():
    # (hidden 1024: enough L2 tiles that the split launches split no K range)
    host, dev = small_case(300, 1024, 512, 64, 4, 505)
    kw = dict(flags=moe.MOE_FLAG_POW2_SCALE, clamp=0.04)
    y_split, r1 = run_opts(dev, tile_m=16, **kw)
    info = moe.moe_plan_info(r1.plan, 300)
    assert info["l1_split"] == 1 and info["l2_split"] == 1, info
    y_one, r2 = run_opts(dev, tile_m=16, flags=kw["flags"] | moe.MOE_FLAG_SINGLE_LAUNCH,
                         clamp=kw["clamp"])
    assert moe.moe_plan_info(r2.plan, 300)["single_launch"] == 1
    assert torch.equal(y_split, y_one)
    verify(y_one, r2, host, "single launch pow2 + clamp", oflags=oracle.ORC_POW2_SCALE, clamp=0.04)


# ---------------------------------------------------- activation quantisation


def mx_quantize_reference(xf):
    T, H = xf.shape
    q = np.zeros((T, H), np.uint8)
    sf = np.zeros((T, H // 32), np.uint8)
    for t in range(T):
        for b in range(H // 32):
            q[t, 32 * b:32 * b + 32], sf[t, b] = oracle.requant_block_mx(xf[t, 32 * b:32 * b + 32])
    return q, sf


@pytest.mark.parametrize("T,H", [(1, 128), (7, 256), (300, 4096)])
@pytest.mark.parametrize("mx", [False, True])
def test_quantize_act_bit_exact(T, H, mx):
    g = torch.Generator(device="cuda").manual_seed(T * 7 + H)
    x = torch.randn(T, H, generator=g, device="cuda") * \
        torch.logspace(-4, 4, T, device="cuda")[:, None]
    x[0, :128] = 0.0  # a zero block takes the floor
    xb = x.to(torch.bfloat16).contiguous()
    plan = moe.moe_plan_create(H, 128, 4, 2, T,
                               recipe=moe.MOE_RECIPE_MXFP4 if mx else moe.MOE_RECIPE_FP8_BLOCK128)
    try:
        q = torch.empty(T, H, dtype=torch.uint8, device="cuda")
        sf = (torch.empty(T, H // 32, dtype=torch.uint8, device="cuda") if mx else
              torch.empty(T, H // 128, dtype=torch.float32, device="cuda"))
        moe.moe_quantize_act(plan, T, xb.view(torch.uint16), q, sf)
        torch.cuda.synchronize()
    finally:
        moe.moe_plan_destroy(plan)
    xf = xb.float().cpu().numpy()
    rq, rsf = mx_quantize_reference(xf) if mx else oracle.quantize_rows(xf)
    say(f"  quantize T={T} H={H} mx={mx}")
    got_q = q.cpu().numpy()
    same = (got_q == rq) | (((got_q & 0x7F) == 0) & ((rq & 0x7F) == 0))
    assert same.all()
    assert np.array_equal(sf.cpu().numpy(), rsf)
