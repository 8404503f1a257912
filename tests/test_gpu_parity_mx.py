"""GPU parity of the FP8 x MXFP4 recipe: moe_forward_mx through the C ABI
against the oracle's MX forward on the same seeded inputs.  Routing is the
FP8 path's planner (tested bit-exact there); the rest goes through
parity_util.verify: h codes and their UE8M0 scale codes equal to the
oracle's or moved only where the measured bound of the block-scaled MFMA
allows, partials within that bound of the oracle's L2 fed the GPU's h, y
bit-exact against the combine of the GPU's partials and within relative L2
1e-2 of the oracle."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import oracle
import workload as wl
from parity_util import host_copy_for_oracle, say, verify

pytestmark = pytest.mark.gpu

def mx_case(T, H, I, E, K, seed, mask=None, skew=False):
    cfg = wl.custom_config(T, H, I, E, K, skew)
    inp = wl.make_inputs_mx(cfg, seed, "cpu")
    if mask:
        idx = inp["topk_idx"].clone()
        for (t, j), v in mask.items():
            idx[t, j] = v
        inp["topk_idx"] = idx
    host = dict(x=inp["x"].numpy(), x_sf=inp["x_sf"].numpy(), idx=inp["topk_idx"].numpy(),
                w=inp["topk_w"].numpy(),
                w1=[inp["w1"][e].numpy() for e in range(E)],
                w1_sf=[inp["w1_sf"][e].numpy() for e in range(E)],
                w2=[inp["w2"][e].numpy() for e in range(E)],
                w2_sf=[inp["w2_sf"][e].numpy() for e in range(E)])
    return host, {k: v.cuda() for k, v in inp.items()}


def run_gpu_mx(dev, tile_m=0, max_tokens=None, runner=None, weight_layout=0, flags=0):
    T, H = dev["x"].shape
    E, twoI, _ = dev["w1"].shape
    K = dev["topk_idx"].shape[1]
    if runner is None:
        runner = moe.MoEForward(H, twoI // 2, E, K, max_tokens or T, tile_m=tile_m,
                                recipe=moe.MOE_RECIPE_MXFP4, weight_layout=weight_layout,
                                flags=flags)
    w1, w1_sf, w2, w2_sf = runner.prepare_mx(dev["w1"], dev["w1_sf"], dev["w2"], dev["w2_sf"])
    y = runner.forward(dev["x"], dev["x_sf"], dev["topk_idx"], dev["topk_w"], w1, w1_sf, w2,
                       w2_sf)
    torch.cuda.synchronize()
    return y, runner


def run_oracle_mx(h, tokens=None, want=()):
    return oracle.moe_forward_mx(h["x"], h["x_sf"], h["idx"], h["w"], h["w1"], h["w1_sf"],
                                 h["w2"], h["w2_sf"], tokens=tokens, want=want)


def check_case(host, dev, tile_m, what):
    T = dev["x"].shape[0]
    K = dev["topk_idx"].shape[1]
    say(f"MX {what}: T={T} H={dev['x'].shape[1]} E={dev['w1'].shape[0]} K={K} tile {tile_m}")
    y, runner = run_gpu_mx(dev, tile_m=tile_m)
    verify(y, runner, host, f"MX {what}")
    return y, runner


@pytest.mark.parametrize("tile_m", [16, 32, 64])
def test_mx_forward_tiny_all_tiles(tile_m):
    cfg = wl.CONFIGS["tiny"]
    host, dev = mx_case(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, wl.default_seed(cfg))
    check_case(host, dev, tile_m, f"tiny tile {tile_m}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mx_forward_ragged_multi_tile(seed):
    # H % 256 == 128 (an L2 tile with two idle waves), several K blocks, hot
    # and empty experts, masked and out-of-range ids
    host, dev = mx_case(45, 640, 384, 12, 3, 300 + seed, mask={(0, 1): -1, (7, 2): 99, (44, 0): -1},
                        skew=True)
    for tile_m in (16, 64):
        check_case(host, dev, tile_m, f"ragged seed {seed} tile {tile_m}")


def test_mx_forward_masked_tokens_and_status():
    host, dev = mx_case(9, 256, 256, 5, 2, 17, mask={(3, 0): -1, (3, 1): -1, (5, 1): 5})
    y, runner = check_case(host, dev, 16, "masked")
    assert not y[3].cpu().numpy().any()
    status = moe.moe_read_status(runner.plan, 9, runner.workspace)
    assert status[0] == moe.MOE_STATUS_EXPERT_OUT_OF_RANGE and status[1] == 1


def test_mx_forward_deterministic_and_auto_tile():
    host, dev = mx_case(40, 512, 256, 6, 4, 23)
    y1, runner = run_gpu_mx(dev)
    y2, _ = run_gpu_mx(dev, runner=runner)
    assert torch.equal(y1, y2)
    info = moe.moe_plan_info(runner.plan, 40)
    assert info["tile_m"] in (16, 32, 64) and info["l1_split"] == 1
    verify(y1, runner, host, "MX auto tile")


@pytest.mark.parametrize("tile_m", [16, 32, 64, "64d"])
def test_mx_packed_weights_match_row_major_bitwise(tile_m):
    # the packed layout only changes where each operand byte is read from:
    # same MFMAs in the same order, so y is bit-identical ("64d": 64-row
    # direct-load tiles; plain 64: the shared-A 64-row tile)
    host, dev = mx_case(37, 512, 384, 16, 4, 211, mask={(5, 1): -1, (20, 3): 40})
    flags = moe.MOE_FLAG_DIRECT_TILES if tile_m == "64d" else 0
    tile_m = 64 if tile_m == "64d" else tile_m
    y_row, _ = run_gpu_mx(dev, tile_m=tile_m, flags=flags)
    y_pk, r = run_gpu_mx(dev, tile_m=tile_m, weight_layout=moe.MOE_WEIGHTS_PACKED, flags=flags)
    assert moe.moe_plan_info(r.plan, 37)["kernel"] == (0 if flags or tile_m < 64 else 2)
    assert torch.equal(y_row, y_pk)
    verify(y_pk, r, host, f"MX packed tile {tile_m}")


@pytest.mark.parametrize("tile", [64, 128])
@pytest.mark.parametrize("case", ["hot", "ragged"])
def test_mx_lds_tiles(case, tile):
    # The 64-row shared-A tile and the persistent 128-row LDS tile:
    # intermediates against the oracle, packed weights bit-identical to
    # row-major, (128) a 4-workgroup grid (each workgroup walking many tiles
    # across tile boundaries) bit-identical to the full grid, and (64) the
    # direct-load 64-row tiles bit-identical too
    if case == "hot":
        host, dev = mx_case(300, 512, 384, 4, 3, 411, skew=True)
    else:
        host, dev = mx_case(157, 768, 512, 6, 2, 412, mask={(3, 0): -1, (40, 1): 77})
    y, runner = check_case(host, dev, tile, f"LDS tile {tile} {case}")
    assert moe.moe_plan_info(runner.plan, dev["x"].shape[0])["kernel"] == (2 if tile == 64 else 1)
    y_pk, _ = run_gpu_mx(dev, tile_m=tile, weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert torch.equal(y, y_pk)
    T, H = dev["x"].shape
    E, twoI, _ = dev["w1"].shape
    small = moe.MoEForward(H, twoI // 2, E, dev["topk_idx"].shape[1], T, tile_m=tile,
                           recipe=moe.MOE_RECIPE_MXFP4, flags=moe.MOE_FLAG_TEST_SMALL_GRID)
    y_small, _ = run_gpu_mx(dev, runner=small)
    assert torch.equal(y, y_small)
    if tile == 64:
        y_direct, rd = run_gpu_mx(dev, tile_m=64, flags=moe.MOE_FLAG_DIRECT_TILES)
        assert moe.moe_plan_info(rd.plan, T)["kernel"] == 0
        assert torch.equal(y, y_direct)


def test_mx_lds_hot_expert_panel_walk():
    # The 128-row LDS tile walks experts of >= 4 row blocks in panels of
    # column tiles: against the oracle, and bit-identical to a 4-workgroup
    # grid and to packed weights.  Expert 3 holds every token's first slot
    # (1100 rows, 9 row blocks), expert 5 exactly 512 rows.
    T = 1100
    alt = [0, 1, 2, 4, 6, 7]
    mask = {(t, 0): 3 for t in range(T)}
    mask.update({(t, 1): 5 if t < 512 else alt[t % 6] for t in range(T)})
    host, dev = mx_case(T, 512, 512, 8, 2, 413, mask=mask)
    y, runner = check_case(host, dev, 128, "LDS tile 128 hot-expert panel walk")
    assert moe.moe_plan_info(runner.plan, T)["kernel"] == 1
    assert moe.moe_read_status(runner.plan, T, runner.workspace)[3] == 9 * 128
    y_pk, _ = run_gpu_mx(dev, tile_m=128, weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert torch.equal(y, y_pk)
    small = moe.MoEForward(512, 512, 8, 2, T, tile_m=128, recipe=moe.MOE_RECIPE_MXFP4,
                           flags=moe.MOE_FLAG_TEST_SMALL_GRID)
    y_small, _ = run_gpu_mx(dev, runner=small)
    assert torch.equal(y, y_small)


def _mx_full_size(cfg, seed, toks, tile=None, kernel=None, force_tile=0):
    dev = wl.make_inputs_mx(cfg, seed, "cuda")
    y, runner = run_gpu_mx(dev, tile_m=force_tile, weight_layout=moe.MOE_WEIGHTS_PACKED)
    info = moe.moe_plan_info(runner.plan, cfg.T)
    say(f"MX {cfg.name} T={cfg.T}: tile {info}")
    if tile is not None:
        assert info["tile_m"] == tile
    if kernel is not None:
        assert info["kernel"] == kernel
    host = host_copy_for_oracle(dev, toks)
    verify(y, runner, host, f"MX {cfg.name} T={cfg.T} ({len(toks)} tokens)", tokens=toks)
    del dev
    torch.cuda.empty_cache()
    return y, runner


def test_mx_flash_prefill_full_size_sampled():
    # ~48 rows per expert: the shared-A 64-row tiles
    cfg = wl.CONFIGS["flash_prefill"]
    _mx_full_size(cfg, wl.default_seed(cfg), [0, 1, 517, 1024, 1999, cfg.T - 1] + list(range(700, 716)),
                  tile=64, kernel=2)


@pytest.mark.parametrize("name,force", [("pro_prefill", 0), ("skewed", 0), ("skewed", 128)])
def test_mx_large_prefill_sampled(name, force):
    # 128 rows per expert on average (skewed: hot experts with ~4000): the
    # library's choice for MXFP4 there is the 64-row shared-A tile; the
    # persistent 128-row LDS tile (the choice between 64 and 108 rows) runs
    # the skewed workload when asked for
    cfg = wl.CONFIGS[name]
    seed = wl.default_seed(cfg)
    rng = np.random.default_rng(seed)
    toks = sorted({0, cfg.T - 1, *rng.choice(cfg.T, 14, replace=False).tolist()})
    if force:
        _mx_full_size(cfg, seed, toks, tile=128, kernel=1, force_tile=128)
    else:
        _mx_full_size(cfg, seed, toks, tile=64, kernel=2)


def test_mx_flash_decode_ep8_share_every_token():
    # one GPU's expert share under 8-way expert parallelism: 32 experts,
    # ~24 rows each (64-row shared-A tiles)
    cfg = wl.CONFIGS["flash_decode_ep8"]
    _mx_full_size(cfg, wl.default_seed(cfg), list(range(cfg.T)), tile=64, kernel=2)


@pytest.mark.parametrize("T", [1, 3, 128])
def test_mx_flash_decode_shape(T):
    # full flash-decode shape (256 experts, H 4096, I 2048) drawn on the GPU:
    # packed and row-major weights bit-identical; every token of T <= 3, a
    # 24-token sample of T = 128 against the oracle
    base = wl.CONFIGS["flash_decode"]
    cfg = wl.custom_config(T, base.H, base.I, base.E, base.K)
    dev = wl.make_inputs_mx(cfg, wl.default_seed(base), "cuda")
    y, runner = run_gpu_mx(dev)
    y_pk, _ = run_gpu_mx(dev, weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert torch.equal(y, y_pk)
    toks = list(range(T)) if T <= 8 else sorted({0, 1, 37, 64, 99, T - 1, *range(100, 118)})
    host = host_copy_for_oracle(dev, toks)
    verify(y, runner, host, f"MX flash decode T={T}", tokens=toks)
    del dev
    torch.cuda.empty_cache()
