"""GPU parity of the recipe options against the oracle: per-64 intermediate
scales (dual-half L2), power-of-two requant scales, the activation clamp
(both recipes, direct and LDS tiles, split-K, single launch), and the
activation quantisation entry point (codes and scales bit-exact: both sides
take every rounding decision in f32 the same way)."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import oracle
from fp8_grouped_gemm_amd import workload as wl
from parity_util import check_y, say, small_case

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


def oracle_opts(host, flags=0, clamp=0.0, want=(), tokens=None, mx=False):
    fn = oracle.moe_forward_mx if mx else oracle.moe_forward
    return fn(host["x"], host["x_sf"], host["idx"], host["w"], host["w1"], host["w1_sf"],
              host["w2"], host["w2_sf"], flags=flags, clamp=clamp, want=want, tokens=tokens)


def check_h(runner, host, ref, T, K, gran, what):
    # dequantised h per routed slot within the bound of the FP8 parity tests;
    # the scales agree to ~1e-3 (raw) or exactly up to one power of two
    DEC = np.array([oracle.e4m3_decode(c) for c in range(256)])
    src_row = runner.view("src_row", T).cpu().numpy()
    h = runner.view("h", T).cpu().numpy()
    h_sf = runner.view("h_sf", T).cpu().numpy()
    assert h_sf.shape[1] == h.shape[1] // gran
    for f in range(T * K):
        r = src_row[f]
        if r < 0:
            continue
        g = DEC[h[r]].reshape(-1, gran) * h_sf[r][:, None]
        o = DEC[ref["h"][f]].reshape(-1, gran) * ref["h_sf"][f][:, None]
        assert np.linalg.norm(g - o) <= 2e-2 * np.linalg.norm(o) + 1e-30, (what, f)


@pytest.mark.parametrize("tile_m", [16, 32, 64])
def test_per64_scales_all_direct_tiles(tile_m):
    host, dev = small_case(45, 512, 384, 12, 3, 501, mask={(0, 1): -1, (7, 2): 99}, skew=True)
    y, r = run_opts(dev, tile_m=tile_m, gran=64)
    info = moe.moe_plan_info(r.plan, 45)
    assert info["act_sf_gran"] == 64 and info["l2_group_tiles"] == 1
    ref = oracle_opts(host, flags=oracle.ORC_SF_GRAN64, want=("h",))
    check_y(y.cpu().numpy(), ref["y"], what=f"per-64 tile {tile_m}")
    check_h(r, host, ref, 45, 3, 64, f"per-64 tile {tile_m}")
    # against the per-128 recipe: a different (still accurate) result
    y128, _ = run_opts(dev, tile_m=tile_m)
    assert not torch.equal(y, y128)


def test_per64_rule_and_split_k():
    # -1: the rule of PR #440 (hidden 256 is not a multiple of 512 -> 64)
    cfg = wl.CONFIGS["tiny"]
    host, dev = small_case(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, wl.default_seed(cfg))
    y, r = run_opts(dev, gran=-1)
    assert moe.moe_plan_info(r.plan, cfg.T)["act_sf_gran"] == 64
    check_y(y.cpu().numpy(), oracle_opts(host, flags=oracle.ORC_SF_GRAN64)["y"], what="tiny rule")
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
        E = base.E
        idx = inp["topk_idx"].cpu().numpy()
        need = sorted({int(e) for e in idx.reshape(-1)})
        sel = lambda t: [t[e].cpu().numpy() if e in need else None for e in range(E)]
        h = dict(x=inp["x"].cpu().numpy(), x_sf=inp["x_sf"].cpu().numpy(), idx=idx,
                 w=inp["topk_w"].cpu().numpy(), w1=sel(inp["w1"]), w1_sf=sel(inp["w1_sf"]),
                 w2=sel(inp["w2"]), w2_sf=sel(inp["w2_sf"]))
        check_y(y.cpu().numpy(), oracle_opts(h, flags=oracle.ORC_SF_GRAN64)["y"],
                per_token_tol=1e-2, what=f"per-64 split-K T={T}")
    del full


@pytest.mark.parametrize("tile_m", [16, 64, 128])
def test_pow2_scales(tile_m):
    host, dev = small_case(160, 512, 384, 6, 3, 502, mask={(3, 0): -1})
    y, r = run_opts(dev, tile_m=tile_m, flags=moe.MOE_FLAG_POW2_SCALE)
    ref = oracle_opts(host, flags=oracle.ORC_POW2_SCALE, want=("h",))
    check_y(y.cpu().numpy(), ref["y"], what=f"pow2 tile {tile_m}")
    check_h(r, host, ref, 160, 3, 128, f"pow2 tile {tile_m}")
    sf = r.view("h_sf", 160).cpu().numpy()
    used = sf[r.view("src_row", 160).cpu().numpy()[r.view("src_row", 160).cpu().numpy() >= 0]]
    m, _ = np.frexp(used.astype(np.float64))
    assert np.all(m == 0.5)  # every scale a power of two


@pytest.mark.parametrize("tile_m", [16, 64, 128])
def test_activation_clamp_fp8(tile_m):
    host, dev = small_case(160, 512, 384, 6, 3, 503)
    clamp = 0.05  # well inside the range of gate/up here: the clamp is active
    y, r = run_opts(dev, tile_m=tile_m, clamp=clamp)
    ref = oracle_opts(host, clamp=clamp)
    check_y(y.cpu().numpy(), ref["y"], what=f"clamp tile {tile_m}")
    y0, _ = run_opts(dev, tile_m=tile_m)
    assert not torch.equal(y, y0)


@pytest.mark.parametrize("tile_m", [16, 64, 128])
def test_activation_clamp_mxfp4(tile_m):
    cfg = wl.custom_config(160, 512, 384, 6, 3)
    inp = wl.make_inputs_mx(cfg, 504, "cpu")
    E = cfg.E
    host = dict(x=inp["x"].numpy(), x_sf=inp["x_sf"].numpy(), idx=inp["topk_idx"].numpy(),
                w=inp["topk_w"].numpy(), w1=[inp["w1"][e].numpy() for e in range(E)],
                w1_sf=[inp["w1_sf"][e].numpy() for e in range(E)],
                w2=[inp["w2"][e].numpy() for e in range(E)],
                w2_sf=[inp["w2_sf"][e].numpy() for e in range(E)])
    dev = {k: v.cuda() for k, v in inp.items()}
    y, _ = run_opts(dev, tile_m=tile_m, clamp=0.05, mx=True)
    check_y(y.cpu().numpy(), oracle_opts(host, clamp=0.05, mx=True)["y"],
            what=f"MX clamp tile {tile_m}")


def test_single_launch_with_pow2_and_clamp_matches_split_launches():
    host, dev = small_case(300, 256, 512, 64, 4, 505)
    kw = dict(flags=moe.MOE_FLAG_POW2_SCALE, clamp=0.04)
    y_split, r1 = run_opts(dev, tile_m=16, **kw)
    y_one, r2 = run_opts(dev, tile_m=16, flags=kw["flags"] | moe.MOE_FLAG_SINGLE_LAUNCH,
                         clamp=kw["clamp"])
    assert moe.moe_plan_info(r2.plan, 300)["single_launch"] == 1
    assert torch.equal(y_split, y_one)
    check_y(y_one.cpu().numpy(),
            oracle_opts(host, flags=oracle.ORC_POW2_SCALE, clamp=0.04)["y"], what="single pow2")


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
