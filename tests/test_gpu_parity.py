"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs.  Routing is compared bit for bit; the rest with
parity_util.verify, which follows the path step by step: h and its scales
equal to the oracle's or moved only where the measured MFMA error bound
allows, partials within that bound of the oracle's L2 fed the GPU's own h, y
bit-exact against the combine of the GPU's partials and within relative L2
1e-2 of the oracle (per case and per token)."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import oracle
import workload as wl
from parity_util import (cpu_inputs_to_gpu, gpu_inputs, host_copy_for_oracle, host_dict, run_gpu,
                         say, small_case, verify)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ routing


def gpu_route(idx_np, E, K, row_align):
    T = idx_np.shape[0]
    p = moe.moe_plan_create(128, 128, E, K, max(T, 1))
    try:
        idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
        r_cap = T * K + E * (row_align - 1)
        counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
        offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
        row_src = torch.full((max(r_cap, 1),), -7, dtype=torch.int32, device="cuda")
        src_row = torch.full((max(T * K, 1),), -7, dtype=torch.int32, device="cuda")
        ws = torch.empty(moe.moe_route_workspace_bytes(p, T), dtype=torch.uint8, device="cuda")
        moe.moe_route(p, T, idx, row_align, counts, offsets, row_src, src_row, ws)
        status = moe.moe_read_status(p, T, ws)
        torch.cuda.synchronize()
        return (counts.cpu().numpy(), offsets.cpu().numpy(), row_src.cpu().numpy()[:r_cap],
                src_row.cpu().numpy()[:T * K], status)
    finally:
        moe.moe_plan_destroy(p)


def assert_route_equal(idx, E, K, ra, what):
    T = idx.shape[0]
    r_cap = T * K + E * (ra - 1)
    say(f"route {what}: T={T} K={K} E={E} row_align={ra}")
    c, o, rs, sr, status = gpu_route(idx, E, K, ra)
    rc, ro, rrs, rsr, bad = oracle.route(idx, E, ra, r_cap)
    assert np.array_equal(c, rc), what
    assert np.array_equal(o, ro), what
    assert np.array_equal(rs, rrs), what
    assert np.array_equal(sr, rsr), what
    assert status[1] == bad and status[0] == (1 if bad else 0), what
    # pool rows used, and the largest aligned segment (from the oracle's offsets)
    assert status[2] == ro[E], what
    assert status[3] == (int(np.diff(ro).max()) if E > 0 else 0), what


@pytest.mark.parametrize("name", ["tiny", "flash_decode", "flash_prefill", "pro_prefill", "skewed",
                                  "flash_decode_ep8"])
@pytest.mark.parametrize("ra", [16, 64, 128])
def test_route_bitexact_workloads(name, ra):
    cfg = wl.CONFIGS[name]
    for seed in (wl.default_seed(cfg), 0):
        idx, _ = wl.make_routing(cfg, seed, "cpu")
        assert_route_equal(idx.numpy(), cfg.E, cfg.K, ra, f"{name} seed {seed}")


def test_route_bitexact_adversarial():
    rng = np.random.default_rng(5)
    cases = {
        "all_one_expert": np.full((3000, 6), 7, np.int32),
        "masks_and_out_of_range": rng.integers(-3, 300, (777, 8)).astype(np.int32),
        "single_token": np.array([[5, 1, 5]], np.int32),
        "dups_in_token": np.tile(np.array([[2, 2, 3, 3]], np.int32), (1500, 1)),
        "ragged_chunks": rng.integers(0, 256, (1023, 3)).astype(np.int32),
        "all_masked": -np.ones((50, 4), np.int32),
        "max_experts": rng.integers(0, 1024, (4096, 8)).astype(np.int32),
    }
    for what, idx in cases.items():
        E = 1024 if what == "max_experts" else 256
        for ra in (1, 16, 128):
            assert_route_equal(idx, E, idx.shape[1], ra, what)


def test_route_zero_tokens():
    c, o, rs, sr, status = gpu_route(np.zeros((0, 4), np.int32), 32, 4, 16)
    assert not c.any() and not o.any()
    assert np.all(rs == -1)
    assert status[1] == 0


# ---------------------------------------------------------------- forward


def check_plan(runner, host, T, E, what):
    """counts, offsets, row_src, src_row of the call bit-exact against the oracle."""
    info = moe.moe_plan_info(runner.plan, T)
    rc, ro, rrs, rsr, _ = oracle.route(host["idx"], E, info["tile_m"], info["pool_rows"])
    assert np.array_equal(runner.view("counts", T).cpu().numpy(), rc), what
    assert np.array_equal(runner.view("offsets", T).cpu().numpy(), ro), what
    assert np.array_equal(runner.view("row_src", T).cpu().numpy(), rrs), what
    assert np.array_equal(runner.view("src_row", T).cpu().numpy(), rsr), what


def forward_and_check(host, dev, tile_m, what, flags=0):
    say(f"forward {what}: tile_m={tile_m} flags={flags}")
    y, runner = run_gpu(dev, tile_m=tile_m, flags=flags)
    T = dev["x"].shape[0]
    check_plan(runner, host, T, dev["w1"].shape[0], what)
    verify(y, runner, host, what)
    return runner


@pytest.mark.parametrize("tile_m", [16, 32, 64])
def test_forward_tiny_all_tiles(tile_m):
    cfg = wl.CONFIGS["tiny"]
    host, dev = small_case(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, wl.default_seed(cfg))
    forward_and_check(host, dev, tile_m, f"tiny tile {tile_m}")


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
def test_forward_tiny_seeds_auto_tile(seed):
    cfg = wl.CONFIGS["tiny"]
    host, dev = small_case(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, seed)
    forward_and_check(host, dev, 0, f"tiny seed {seed}")


def test_forward_edge_masks_out_of_range_and_empty_tokens():
    mask = {(0, 0): -1, (0, 1): -1, (0, 2): -1,      # token 0 fully masked -> y = 0
            (3, 1): 40, (5, 2): 9999,                  # ids >= E: skipped + flagged
            (7, 0): -5}
    host, dev = small_case(37, 384, 256, 12, 3, 11, mask=mask)   # H % 256 == 128, I = 2 n-tiles
    for tile_m in (16, 64):
        runner = forward_and_check(host, dev, tile_m, f"edge tile {tile_m}")
        status = moe.moe_read_status(runner.plan, 37, runner.workspace)
        assert status[0] == moe.MOE_STATUS_EXPERT_OUT_OF_RANGE and status[1] == 2


def test_forward_ragged_multi_tile_shapes():
    # several K blocks, several n tiles, T*K not a multiple of the tile or 1024
    host, dev = small_case(203, 512, 384, 16, 4, 12)
    for tile_m in (16, 32, 64, 128):
        forward_and_check(host, dev, tile_m, f"ragged tile {tile_m}")
    forward_and_check(host, dev, 64, "ragged tile 64 direct", flags=moe.MOE_FLAG_DIRECT_TILES)


def test_forward_single_token_and_hot_expert():
    host, dev = small_case(1, 256, 128, 4, 2, 13)
    forward_and_check(host, dev, 0, "single token")
    # every token on expert 2: one long segment, many row tiles
    T = 150
    host, dev = small_case(T, 256, 256, 8, 2, 14, mask={(t, 0): 2 for t in range(T)})
    for tile_m in (16, 64, 128):
        forward_and_check(host, dev, tile_m, f"hot expert tile {tile_m}")
    forward_and_check(host, dev, 64, "hot expert tile 64 direct", flags=moe.MOE_FLAG_DIRECT_TILES)


def test_forward_deterministic_and_workspace_reuse():
    host, dev = small_case(90, 256, 256, 8, 3, 15)
    y1, runner = run_gpu(dev, tile_m=32, max_tokens=200)
    # a different, larger call in between leaves stale state in the workspace
    host2, dev2 = small_case(200, 256, 256, 8, 3, 16)
    y2, _ = run_gpu(dev2, runner=runner)
    verify(y2, runner, host2, "reuse, larger call")
    y3, _ = run_gpu(dev, runner=runner)
    assert torch.equal(y1, y3)
    verify(y3, runner, host, "reuse, first call again")


@pytest.mark.parametrize("tile_m", [16, 32, 64, 128, "64d"])
def test_packed_weights_match_row_major_bitwise(tile_m):
    # packed weights only change where the kernels read each fragment from:
    # same arithmetic in the same order, so y is bit-identical
    host, dev = small_case(203, 512, 384, 16, 4, 17)
    flags = moe.MOE_FLAG_DIRECT_TILES if tile_m == "64d" else 0  # 64-row direct-load tiles
    tile_m = 64 if tile_m == "64d" else tile_m
    y_row, _ = run_gpu(dev, tile_m=tile_m, flags=flags)
    y_pk, runner = run_gpu(dev, tile_m=tile_m, weight_layout=moe.MOE_WEIGHTS_PACKED, flags=flags)
    want = 0 if flags or tile_m < 64 else (2 if tile_m == 64 else 1)  # 2: shared-A, 1: LDS
    assert moe.moe_plan_info(runner.plan, 203)["kernel"] == want
    assert torch.equal(y_row, y_pk)
    verify(y_pk, runner, host, f"packed tile {tile_m}")


def test_packed_weights_full_size_decode_bitwise():
    cfg = wl.CONFIGS["flash_decode"]
    inp = gpu_inputs(cfg, wl.default_seed(cfg))
    y_row, _ = run_gpu(inp)
    y_pk, _ = run_gpu(inp, weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert torch.equal(y_row, y_pk)
    del inp
    torch.cuda.empty_cache()


def test_forward_small_token_counts_split_k():
    # Flash-decode shapes with one or two tokens: fewer (row block, column
    # tile) pairs than compute units, so each L1 tile's K range is split
    # over 4 or 2 workgroups, and at one token each L2 tile's over 4 (f32
    # partials per routed slot, added in slice order by the slice counted
    # last); from three tokens on there is no split.  At 32 tokens the L2 workgroups each take two column tiles.
    # Every token is checked against the oracle; packed and row-major
    # weights must agree bit for bit.
    base = wl.CONFIGS["flash_decode"]
    full = gpu_inputs(wl.custom_config(32, base.H, base.I, base.E, base.K), wl.default_seed(base))
    for T, (split, l2g) in {1: (4, 1), 2: (2, 1), 3: (1, 1), 8: (1, 1), 32: (1, 2)}.items():
        inp = dict(full)
        for k in ("x", "x_sf", "topk_idx", "topk_w"):
            inp[k] = full[k][:T].contiguous()
        y_row, runner = run_gpu(inp)
        info = moe.moe_plan_info(runner.plan, T)
        say(f"  T={T}: tile {info['tile_m']}, L1 split {info['l1_split']}, "
            f"L2 split {info['l2_split']}, L2 tiles/workgroup {info['l2_group_tiles']}")
        assert info["tile_m"] == 16 and info["l1_split"] == split
        assert info["l2_split"] == (4 if T == 1 else 1) and info["l2_group_tiles"] == l2g
        y_pk, r_pk = run_gpu(inp, weight_layout=moe.MOE_WEIGHTS_PACKED)
        assert torch.equal(y_row, y_pk), T
        host = host_copy_for_oracle(inp, list(range(T)))
        verify(y_pk, r_pk, host, f"T={T} L1 split {split}")
        del runner, r_pk
    del full, inp
    torch.cuda.empty_cache()


# ---------------- 128-row tiles (persistent LDS kernel), 64-row shared-A tiles


@pytest.mark.parametrize("tile", [128])
@pytest.mark.parametrize("case", ["ragged", "hot", "many_blocks", "tiny_rows"])
def test_lds_tiles_persistent_small_grid_matches_full_grid(case, tile):
    # With the test flag the persistent kernels run on 4 workgroups, so each
    # walks many tiles (copies of the next tile overlap the current tile's
    # epilogue, metadata slots rotate); the arithmetic per tile is the same,
    # so y is bit-identical to the full grid, and both match the oracle.
    if case == "ragged":
        host, dev = small_case(203, 512, 384, 16, 4, 12)
    elif case == "hot":
        T = 150
        host, dev = small_case(T, 256, 256, 8, 2, 14, mask={(t, 0): 2 for t in range(T)})
    elif case == "many_blocks":
        host, dev = small_case(600, 512, 512, 16, 4, 22)
    else:  # one K block more than the minimum, masked slots, a token with no slot
        host, dev = small_case(45, 256, 256, 6, 3, 23, mask={(0, 0): -1, (0, 1): -1, (0, 2): -1,
                                                             (5, 1): -3})
    y_full, r_full = _run_flags(dev, 0, tile)
    y_small, r_small = _run_flags(dev, moe.MOE_FLAG_TEST_SMALL_GRID, tile)
    T = dev["x"].shape[0]
    assert moe.moe_plan_info(r_small.plan, T)["kernel"] == 1
    assert torch.equal(y_full, y_small), case
    verify(y_small, r_small, host, f"tile {tile} small grid {case}")


@pytest.mark.parametrize("case", ["ragged", "hot", "tiny_rows"])
def test_tile64_shared_a_matches_direct_tiles_and_tile128_bitwise(case):
    # Every kernel computes each row with the same MFMAs, the same per-K-block
    # promotion and the same epilogue arithmetic; only the tiling (and hence
    # the padding rows) differs, so y is bit-identical across them.
    if case == "ragged":
        host, dev = small_case(203, 512, 384, 16, 4, 12)
    elif case == "hot":
        T = 150
        host, dev = small_case(T, 256, 256, 8, 2, 14, mask={(t, 0): 2 for t in range(T)})
    else:
        host, dev = small_case(45, 256, 256, 6, 3, 23, mask={(0, 0): -1, (5, 1): -3})
    T = dev["x"].shape[0]
    y64, r64 = _run_flags(dev, 0, 64)
    assert moe.moe_plan_info(r64.plan, T)["kernel"] == 2
    y64d, r64d = _run_flags(dev, moe.MOE_FLAG_DIRECT_TILES, 64)
    assert moe.moe_plan_info(r64d.plan, T)["kernel"] == 0
    y128, _ = _run_flags(dev, 0, 128)
    assert torch.equal(y64, y64d), case
    assert torch.equal(y64, y128), case
    y64p, _ = _run_flags(dev, 0, 64, weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert torch.equal(y64, y64p), case
    verify(y64, r64, host, f"tile 64 shared-A {case}")


def _hot_mask(T):
    # every token's first slot on expert 3 (T rows), the second slot of
    # tokens 0-511 on expert 5 (exactly 4 row blocks of 128), the others on
    # the remaining experts in turn
    alt = [0, 1, 2, 4, 6, 7]
    mask = {(t, 0): 3 for t in range(T)}
    mask.update({(t, 1): 5 if t < 512 else alt[t % 6] for t in range(T)})
    return mask


def test_lds_hot_expert_panel_walk_bitwise():
    # Experts spanning >= 4 row blocks of 128 rows are walked in panels of
    # column tiles (the planner's status[3], the largest segment, switches
    # it on).  Only the order of the tiles changes, so y is bit-identical to
    # the 64-row shared-A tiles (which never reorder) and to a 4-workgroup
    # grid, and it matches the oracle.  Expert 3: 1100 rows (9 row blocks,
    # not a multiple of the panel), expert 5: 512 rows (the threshold).
    T = 1100
    host, dev = small_case(T, 512, 512, 8, 2, 31, mask=_hot_mask(T))
    y128, r128 = _run_flags(dev, 0, 128)
    assert moe.moe_plan_info(r128.plan, T)["kernel"] == 1
    st = moe.moe_read_status(r128.plan, T, r128.workspace)
    assert st[3] == 9 * 128, st
    y_small, _ = _run_flags(dev, moe.MOE_FLAG_TEST_SMALL_GRID, 128)
    assert torch.equal(y128, y_small)
    y64, r64 = _run_flags(dev, 0, 64)
    assert moe.moe_plan_info(r64.plan, T)["kernel"] == 2
    assert torch.equal(y128, y64)
    y128p, _ = _run_flags(dev, 0, 128, weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert torch.equal(y128, y128p)
    verify(y128, r128, host, "tile 128 hot-expert panel walk")


def test_lds_tile_padding_row_halves_bitwise():
    # Experts of 1, 63, 64, 65, 127, 128 and 129 routed rows: in the 128-row
    # tile the waves of a row half that holds only padding skip their MFMAs
    # (first tiles of <= 64 rows, the 129-row expert's second tile), while a
    # half with one routed row (65) multiplies.  y is bitwise that of the
    # 64-row shared-A tile, and matches the oracle.
    sizes = [1, 63, 64, 65, 127, 128, 129, 0]
    T = sum(sizes)
    owner = [e for e, n in enumerate(sizes) for _ in range(n)]
    host, dev = small_case(T, 256, 256, len(sizes), 1, 41, mask={(t, 0): owner[t] for t in range(T)})
    y128, r128 = _run_flags(dev, 0, 128)
    assert moe.moe_plan_info(r128.plan, T)["kernel"] == 1
    counts = r128.view("counts", T).cpu().numpy()
    assert counts.tolist() == sizes
    y64, r64 = _run_flags(dev, 0, 64)
    assert moe.moe_plan_info(r64.plan, T)["kernel"] == 2
    assert torch.equal(y128, y64)
    verify(y128, r128, host, "tile 128 padding row halves")


def test_lds_tiles_full_size_packed_small_grid():
    # The flash-prefill workload on 128-row tiles on 4 workgroups (every
    # workgroup walks ~700 L1 tiles) against the full grid, packed weights,
    # and both against the library's choice there (64-row shared-A tiles,
    # ~48 rows per expert): the same arithmetic per row, so bit-identical.
    cfg = wl.CONFIGS["flash_prefill"]
    inp = gpu_inputs(cfg, wl.default_seed(cfg))
    y_full, r = _run_flags(inp, 0, 128, weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert moe.moe_plan_info(r.plan, cfg.T)["kernel"] == 1
    y_small, _ = _run_flags(inp, moe.MOE_FLAG_TEST_SMALL_GRID, 128,
                            weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert torch.equal(y_full, y_small)
    y_auto, ra = _run_flags(inp, 0, 0, weight_layout=moe.MOE_WEIGHTS_PACKED)
    info = moe.moe_plan_info(ra.plan, cfg.T)
    assert info["kernel"] == 2 and info["tile_m"] == 64
    assert torch.equal(y_full, y_auto)
    del inp
    torch.cuda.empty_cache()


# -------------------------------------------- single launch (a6 variant)


def _run_flags(inp, flags, tile_m=0, weight_layout=0):
    T, H = inp["x"].shape
    E, twoI, _ = inp["w1"].shape
    K = inp["topk_idx"].shape[1]
    runner = moe.MoEForward(H, twoI // 2, E, K, T, tile_m=tile_m, weight_layout=weight_layout,
                            flags=flags)
    return run_gpu(inp, runner=runner)


@pytest.mark.parametrize("case", ["wide16", "wide32", "wide64", "tiny32", "ragged32",
                                  "ragged64", "edge64", "hot32"])
def test_single_launch_matches_split_launch_bitwise(case):
    # Same tiles, same arithmetic in the same order; only the hand-off
    # between L1, L2 and the combine changes, so y is bit-identical.  (The
    # single launch runs when neither GEMM splits K, i.e. 16-row tiles need
    # at least 256 L1 and 256 L2 tiles: hence the wide case.)
    cfg = wl.CONFIGS["tiny"]
    tile = int(case[-2:])
    if case.startswith("wide"):
        host, dev = small_case(300, 1024, 512, 64, 4, 21)
    elif case.startswith("tiny"):
        host, dev = small_case(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, wl.default_seed(cfg))
    elif case.startswith("ragged"):
        host, dev = small_case(203, 512, 384, 16, 4, 12)
    elif case.startswith("edge"):
        host, dev = small_case(37, 384, 256, 12, 3, 11, mask={(0, 0): -1, (0, 1): -1, (0, 2): -1,
                                                               (3, 1): 40, (7, 0): -5})
    else:
        T = 150
        host, dev = small_case(T, 256, 256, 8, 2, 14, mask={(t, 0): 2 for t in range(T)})
    # (64-row tiles: the direct-load kernels, which the single launch is built from)
    direct = moe.MOE_FLAG_DIRECT_TILES if tile == 64 else 0
    y_split, r_split = _run_flags(dev, moe.MOE_FLAG_SPLIT_LAUNCH | direct, tile)
    y_one, r_one = _run_flags(dev, moe.MOE_FLAG_SINGLE_LAUNCH | direct, tile)
    T = dev["x"].shape[0]
    assert moe.moe_plan_info(r_split.plan, T)["single_launch"] == 0
    assert moe.moe_plan_info(r_one.plan, T)["single_launch"] == 1
    st = moe.moe_read_status(r_one.plan, T, r_one.workspace)
    assert not (st[0] & moe.MOE_STATUS_WAIT_TIMEOUT)
    assert torch.equal(y_split, y_one), case
    verify(y_one, r_one, host, f"single launch {case}")


def test_single_launch_full_size_decode_bitwise_and_repeat():
    cfg = wl.CONFIGS["flash_decode"]
    inp = gpu_inputs(cfg, wl.default_seed(cfg))
    y_split, _ = _run_flags(inp, moe.MOE_FLAG_SPLIT_LAUNCH, weight_layout=moe.MOE_WEIGHTS_PACKED)
    y_one, runner = _run_flags(inp, moe.MOE_FLAG_SINGLE_LAUNCH,
                               weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert moe.moe_plan_info(runner.plan, cfg.T)["single_launch"] == 1
    assert torch.equal(y_split, y_one)
    # the counters are reset by every call's planner: repeated calls agree
    w1, w2 = runner.prepare(inp["w1"], inp["w2"])
    for _ in range(3):
        y = runner.forward(inp["x"], inp["x_sf"], inp["topk_idx"], inp["topk_w"], w1,
                           inp["w1_sf"], w2, inp["w2_sf"])
        assert torch.equal(y, y_one)
    st = moe.moe_read_status(runner.plan, cfg.T, runner.workspace)
    assert not (st[0] & moe.MOE_STATUS_WAIT_TIMEOUT)
    del inp, w1, w2
    torch.cuda.empty_cache()


def test_single_launch_wait_timeout_is_reported():
    # The test flag makes every wait give up at once (no kernel spins): the
    # call still completes and flags MOE_STATUS_WAIT_TIMEOUT; the next call
    # on a normal plan with the same inputs is clean and correct.
    cfg = wl.CONFIGS["tiny"]
    host, dev = small_case(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, wl.default_seed(cfg))
    _, bad = _run_flags(dev, moe.MOE_FLAG_SINGLE_LAUNCH | moe.MOE_FLAG_TEST_NO_WAIT, 32)
    assert moe.moe_plan_info(bad.plan, cfg.T)["single_launch"] == 1
    st = moe.moe_read_status(bad.plan, cfg.T, bad.workspace)
    assert st[0] & moe.MOE_STATUS_WAIT_TIMEOUT
    y, good = _run_flags(dev, moe.MOE_FLAG_SINGLE_LAUNCH, 32)
    st = moe.moe_read_status(good.plan, cfg.T, good.workspace)
    assert not (st[0] & moe.MOE_STATUS_WAIT_TIMEOUT)
    verify(y, good, host, "single launch after a timeout run")


def test_forward_zero_tokens_is_noop():
    runner = moe.MoEForward(256, 128, 8, 2, 16)
    y = torch.full((0, 256), 7, dtype=torch.uint16, device="cuda")
    z = torch.empty(0, dtype=torch.uint8, device="cuda")
    moe.moe_forward(runner.plan, 0, z, z, z, z, z, z, z, z, y, runner.workspace)
    torch.cuda.synchronize()


# -------------------------------------------------- full-size workloads


def _full_size(name, tokens=None):
    cfg = wl.CONFIGS[name]
    seed = wl.default_seed(cfg)
    say(f"full size {name}: drawing inputs on the GPU")
    inp = gpu_inputs(cfg, seed)
    torch.cuda.synchronize()
    y, runner = run_gpu(inp, weight_layout=moe.MOE_WEIGHTS_PACKED)
    info = moe.moe_plan_info(runner.plan, cfg.T)
    say(f"  tile {info}")
    if tokens is None:
        toks = list(range(cfg.T))
    else:
        rng = np.random.default_rng(seed)
        toks = sorted({0, cfg.T - 1, *rng.choice(cfg.T, tokens, replace=False).tolist()})
        if cfg.skew:  # tokens routed to the hottest expert
            idx = inp["topk_idx"].cpu().numpy()
            hot = np.bincount(idx.reshape(-1), minlength=cfg.E).argmax()
            toks = sorted(set(toks) | set(np.nonzero((idx == hot).any(1))[0][:3].tolist()))
    host = host_copy_for_oracle(inp, toks)
    # the plan of the whole workload, bit-exact
    check_plan(runner, host, cfg.T, cfg.E, name)
    st = verify(y, runner, host, f"{name} ({len(toks)} tokens)", tokens=toks)
    del inp
    torch.cuda.empty_cache()
    return st


@pytest.mark.parametrize("name", ["flash_decode", "flash_prefill"])
def test_forward_full_size_every_token(name):
    # every token of the workload: its h, h_sf and partials (all 768 resp.
    # 12288 routed slots) and y
    _full_size(name)


@pytest.mark.parametrize("name", ["pro_prefill", "skewed", "flash_decode_ep8"])
def test_forward_full_size_sampled(name):
    _full_size(name, tokens=24)


@pytest.mark.parametrize("tile_m", [16, 64, 128])
def test_forward_zero_blocks_and_outlier_rows(tile_m):
    # Inputs the seeded generator never draws: all-zero activation blocks
    # (their scale takes the 1e-10 floor), a token whose row is all zero (its
    # h blocks are all zero, take the floor too, and its y is exactly zero),
    # rows scaled by 1e4 and 1e-4, a zero 128x128 block of W1 and zero rows
    # of W2 (zero partial columns).
    T, H, I, E, K = 96, 512, 384, 6, 3
    cfg = wl.custom_config(T, H, I, E, K)
    inp = wl.make_inputs(cfg, 601, "cpu")
    g = torch.Generator().manual_seed(601)
    x = torch.randn(T, H, generator=g)
    x[3, 128:256] = 0.0
    x[10] = 0.0
    x[20] *= 1e4
    x[21] *= 1e-4
    x[22, :128] *= 1e3
    inp["x"], inp["x_sf"] = wl.quantize_blocks(x, 1, 128)
    w1 = inp["w1"].clone()
    w1_sf = inp["w1_sf"].clone()
    w1[1, 128:256, 256:384] = 0          # gate block (1, 2) of expert 1
    w1_sf[1, 1, 2] = 1e-10 / 448.0
    w2 = inp["w2"].clone()
    w2[2, 5:40] = 0                      # output columns 5..39 of expert 2
    inp.update(w1=w1, w1_sf=w1_sf, w2=w2)
    host = host_dict(inp)
    dev = cpu_inputs_to_gpu(inp)
    assert float(inp["x_sf"][10].max()) == np.float32(1e-10) / np.float32(448.0)
    runner = forward_and_check(host, dev, tile_m, f"zero blocks / outliers tile {tile_m}")
    y = runner.view("h_sf", T)  # the zero token's intermediate scales took the floor
    src_row = runner.view("src_row", T).cpu().numpy()
    floor = np.float32(1e-10) / np.float32(448.0)
    for j in range(K):
        if host["idx"][10, j] >= 0:
            assert np.all(y[src_row[10 * K + j]].cpu().numpy() == floor)
