"""GPU: the lag-ordered ring pool (MOE_FLAG_RING_POOL).

DeepGEMM PR #440 "API, Tests, Files" checks the ring bitwise against a
full-pool control, four launches per buffer with skewed routing in between,
and refuses an over-capacity bound on the host (that refusal is a CPU test in
test_abi.py).  Here the control is the full-pool single launch with the same
tiles: the ring changes where h / h_sf rows live and the order of the tiles,
never their arithmetic, so y and the partials are bit-identical.  The control
itself is checked against the oracle step by step (parity_util.verify), which
the ring arm's bit-identical y then meets too.  Each ring slot is also
checked to hold its last row block's h and h_sf."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import workload as wl
from parity_util import say, small_case, verify

pytestmark = pytest.mark.gpu

RING = moe.MOE_FLAG_RING_POOL
CONTROL = moe.MOE_FLAG_SINGLE_LAUNCH | moe.MOE_FLAG_DIRECT_TILES

# name: (T, H, I, E, K, tile_m, weight layout)
SHAPES = {
    "t16": (600, 512, 256, 64, 4, 16, moe.MOE_WEIGHTS_ROW_MAJOR),
    "t16_packed": (600, 512, 256, 64, 4, 16, moe.MOE_WEIGHTS_PACKED),
    "t32": (2048, 1024, 512, 32, 6, 32, moe.MOE_WEIGHTS_ROW_MAJOR),
    "t64": (4096, 1024, 1024, 16, 2, 64, moe.MOE_WEIGHTS_PACKED),
}


def _routing(kind, T, H, I, E, K, seed, device):
    """topk ids of one launch: the router draw, its Zipf-skewed variant, or
    every token on a few hot experts."""
    if kind in ("uniform", "skewed"):
        cfg = wl.custom_config(T, H, I, E, K, skew=kind == "skewed")
        idx, _ = wl.make_routing(cfg, seed, "cpu")
        return idx.to(device)
    rng = np.random.default_rng(seed)
    hot = rng.choice(E, size=max(K, 3), replace=False)
    idx = np.stack([rng.choice(hot, size=K, replace=False) for _ in range(T)])
    return torch.from_numpy(idx.astype(np.int32)).to(device)


def _used_blocks(runner, T, tile):
    counts = runner.view("counts", T).cpu().numpy().astype(np.int64)
    return int(np.sum((counts + tile - 1) // tile))


def _forward(runner, dev, idx, w1, w2):
    y = runner.forward(dev["x"], dev["x_sf"], idx, dev["topk_w"], w1, dev["w1_sf"], w2,
                       dev["w2_sf"])
    torch.cuda.synchronize()
    return y


def _check_ring_slots(ring, ctrl, T, tile):
    """Slot s of the ring holds the h / h_sf rows of the last used row block
    mb with mb % ring_blocks == s (its valid rows)."""
    info = moe.moe_plan_info(ring.plan, T)
    rb = info["ring_blocks"]
    used = _used_blocks(ctrl, T, tile)
    row_src = ctrl.view("row_src", T).cpu().numpy()
    h_r, h_c = ring.view("h", T).cpu().numpy(), ctrl.view("h", T).cpu().numpy()
    s_r, s_c = ring.view("h_sf", T).cpu().numpy(), ctrl.view("h_sf", T).cpu().numpy()
    for s in range(min(rb, used)):
        mb = s + rb * ((used - 1 - s) // rb)
        rows = np.arange(mb * tile, (mb + 1) * tile)
        ok = row_src[rows] >= 0
        slot_rows = np.arange(s * tile, (s + 1) * tile)[ok]
        assert np.array_equal(h_r[slot_rows], h_c[rows[ok]]), (s, mb)
        assert np.array_equal(s_r[slot_rows].view(np.uint32), s_c[rows[ok]].view(np.uint32))


@pytest.mark.parametrize("name", list(SHAPES))
def test_ring_bitwise_vs_full_pool_four_launches(name):
    T, H, I, E, K, tile, layout = SHAPES[name]
    host, dev = small_case(T, H, I, E, K, 40 + T)
    ring = moe.MoEForward(H, I, E, K, T, tile_m=tile, weight_layout=layout, flags=RING)
    ctrl = moe.MoEForward(H, I, E, K, T, tile_m=tile, weight_layout=layout, flags=CONTROL)
    info = moe.moe_plan_info(ring.plan, T)
    assert info["ring_blocks"] > 0 and info["single_launch"] == 1, info
    assert moe.moe_plan_info(ctrl.plan, T)["single_launch"] == 1
    assert moe.moe_workspace_bytes(ring.plan, T) < moe.moe_workspace_bytes(ctrl.plan, T)
    w1, w2 = ring.prepare(dev["w1"], dev["w2"])
    wrapped = 0
    for i, kind in enumerate(("uniform", "skewed", "hot", "skewed")):
        idx = dev["topk_idx"] if i == 0 else _routing(kind, T, H, I, E, K, 7 * i + T, "cuda")
        say(f"ring {name} launch {i} ({kind}): T={T} H={H} I={I} E={E} K={K} tile={tile} "
            f"ring_blocks={info['ring_blocks']} lag={info['l2_lag_units']}")
        y_c = _forward(ctrl, dev, idx, w1, w2)
        y_r = _forward(ring, dev, idx, w1, w2)
        for r in (ring, ctrl):
            st = moe.moe_read_status(r.plan, T, r.workspace)
            assert not (st[0] & moe.MOE_STATUS_WAIT_TIMEOUT), (name, i)
        used = _used_blocks(ctrl, T, tile)
        wrapped += used > info["ring_blocks"]
        assert torch.equal(y_r, y_c), (name, i, kind)
        assert torch.equal(ring.view("partial", T), ctrl.view("partial", T)), (name, i)
        _check_ring_slots(ring, ctrl, T, tile)
        if i < 2 and name == "t16":
            h = dict(host)
            h["idx"] = idx.cpu().numpy()
            verify(y_c, ctrl, h, f"ring control {name} launch {i}")
    assert wrapped >= 3, (name, wrapped)  # the ring wraps on most launches
    ring.close()
    ctrl.close()


def test_ring_single_wave_order_when_blocks_fit():
    # the ring is engaged for this T, but every token goes to 8 experts: the
    # used row blocks fit the ring and the stream takes the single-wave order
    # (I = 512: 300 tokens already make 256 L1 tiles, so the control does not
    # split K either and runs as one launch with the same arithmetic)
    T, H, I, E, K, tile = 300, 512, 512, 64, 4, 16
    host, dev = small_case(T, H, I, E, K, 77)
    idx = _routing("hot8", T, H, I, E, K, 5, "cuda")
    hot = np.unique(idx.cpu().numpy())
    assert hot.size <= 8
    ring = moe.MoEForward(H, I, E, K, 600, tile_m=tile, flags=RING)
    ctrl = moe.MoEForward(H, I, E, K, 600, tile_m=tile, flags=CONTROL)
    info = moe.moe_plan_info(ring.plan, T)
    assert info["ring_blocks"] > 0
    cinfo = moe.moe_plan_info(ctrl.plan, T)
    assert cinfo["single_launch"] == 1 and cinfo["l1_split"] == 1, cinfo
    w1, w2 = ring.prepare(dev["w1"], dev["w2"])
    y_c = _forward(ctrl, dev, idx, w1, w2)
    y_r = _forward(ring, dev, idx, w1, w2)
    assert _used_blocks(ctrl, T, tile) <= info["ring_blocks"]
    st = moe.moe_read_status(ring.plan, T, ring.workspace)
    assert not (st[0] & moe.MOE_STATUS_WAIT_TIMEOUT)
    assert torch.equal(y_r, y_c)
    h = dict(host)
    h["idx"] = idx.cpu().numpy()
    verify(y_c, ctrl, h, "ring single-wave control")
    ring.close()
    ctrl.close()


def test_ring_small_grid_matches_control():
    # four workgroups walk the whole stream: every wait is for an earlier
    # item, so the ring's waits end with any grid
    T, H, I, E, K, tile, layout = SHAPES["t32"]
    _, dev = small_case(T, H, I, E, K, 91)
    ring = moe.MoEForward(H, I, E, K, T, tile_m=tile, flags=RING | moe.MOE_FLAG_TEST_SMALL_GRID)
    ctrl = moe.MoEForward(H, I, E, K, T, tile_m=tile, flags=CONTROL)
    assert moe.moe_plan_info(ctrl.plan, T)["single_launch"] == 1
    w1, w2 = ring.prepare(dev["w1"], dev["w2"])
    idx = _routing("skewed", T, H, I, E, K, 3, "cuda")
    y_c = _forward(ctrl, dev, idx, w1, w2)
    y_r = _forward(ring, dev, idx, w1, w2)
    assert _used_blocks(ctrl, T, tile) > moe.moe_plan_info(ring.plan, T)["ring_blocks"]
    st = moe.moe_read_status(ring.plan, T, ring.workspace)
    assert not (st[0] & moe.MOE_STATUS_WAIT_TIMEOUT)
    assert torch.equal(y_r, y_c)
    ring.close()
    ctrl.close()


def test_ring_full_size_flash_prefill_bitwise():
    # the flash prefill layer (2048 tokens, 64-row direct tiles): a 124-block
    # ring for ~320 used blocks, uniform then Zipf-skewed routing
    cfg = wl.CONFIGS["flash_prefill"]
    inp = wl.make_inputs(cfg, wl.default_seed(cfg), "cuda")
    T = cfg.T
    ring = moe.MoEForward(cfg.H, cfg.I, cfg.E, cfg.K, T, weight_layout=moe.MOE_WEIGHTS_PACKED,
                          flags=RING)
    info = moe.moe_plan_info(ring.plan, T)
    ctrl = moe.MoEForward(cfg.H, cfg.I, cfg.E, cfg.K, T, tile_m=info["tile_m"],
                          weight_layout=moe.MOE_WEIGHTS_PACKED, flags=CONTROL)
    say(f"ring flash_prefill: tile {info['tile_m']} ring_blocks {info['ring_blocks']} "
        f"lag {info['l2_lag_units']}")
    assert info["ring_blocks"] > 0
    assert moe.moe_plan_info(ctrl.plan, T)["single_launch"] == 1
    w1, w2 = ring.prepare(inp["w1"], inp["w2"])
    for i, kind in enumerate(("uniform", "skewed")):
        idx = inp["topk_idx"] if i == 0 else _routing(kind, T, cfg.H, cfg.I, cfg.E, cfg.K, 11,
                                                       "cuda")
        y_c = _forward(ctrl, inp, idx, w1, w2)
        y_r = _forward(ring, inp, idx, w1, w2)
        assert _used_blocks(ctrl, T, info["tile_m"]) > info["ring_blocks"]
        st = moe.moe_read_status(ring.plan, T, ring.workspace)
        assert not (st[0] & moe.MOE_STATUS_WAIT_TIMEOUT)
        assert torch.equal(y_r, y_c), kind
    ring.close()
    ctrl.close()
    del inp, w1, w2
    torch.cuda.empty_cache()


def test_ring_wait_timeout_is_reported_and_next_call_is_clean():
    # The test flag makes every wait of the ring's single launch give up at
    # once (L1 tiles waiting for a slot's previous L2 tiles included): the
    # call completes and flags MOE_STATUS_WAIT_TIMEOUT; a normal ring plan on
    # the same inputs then runs clean and matches the full-pool control.
    T, H, I, E, K, tile, layout = SHAPES["t16"]
    _, dev = small_case(T, H, I, E, K, 93)
    bad = moe.MoEForward(H, I, E, K, T, tile_m=tile, flags=RING | moe.MOE_FLAG_TEST_NO_WAIT)
    assert moe.moe_plan_info(bad.plan, T)["ring_blocks"] > 0
    _forward(bad, dev, dev["topk_idx"], dev["w1"], dev["w2"])
    st = moe.moe_read_status(bad.plan, T, bad.workspace)
    assert st[0] & moe.MOE_STATUS_WAIT_TIMEOUT
    ring = moe.MoEForward(H, I, E, K, T, tile_m=tile, flags=RING)
    ctrl = moe.MoEForward(H, I, E, K, T, tile_m=tile, flags=CONTROL)
    y_r = _forward(ring, dev, dev["topk_idx"], dev["w1"], dev["w2"])
    y_c = _forward(ctrl, dev, dev["topk_idx"], dev["w1"], dev["w2"])
    st = moe.moe_read_status(ring.plan, T, ring.workspace)
    assert not (st[0] & moe.MOE_STATUS_WAIT_TIMEOUT)
    assert torch.equal(y_r, y_c)
    for r in (bad, ring, ctrl):
        r.close()
