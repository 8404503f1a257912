"""GPU: the 160-row LDS tile (gemm_lds160.hip) against the 128-row LDS tile
and the oracle.  Both tiles compute every row with the same MFMAs, the same
per-128-K promotion and the same epilogue arithmetic; only the tiling (and
the padding rows) differs, so y is bit-identical, and each case also passes
the step-by-step chain check against the oracle."""
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import workload as wl
from parity_util import gpu_inputs, say, small_case, verify

pytestmark = pytest.mark.gpu

PACKED = moe.MOE_WEIGHTS_PACKED


def _run(inp, tile_m, flags=0):
    T, H = inp["x"].shape
    E, twoI, _ = inp["w1"].shape
    K = inp["topk_idx"].shape[1]
    r = moe.MoEForward(H, twoI // 2, E, K, T, tile_m=tile_m, weight_layout=PACKED, flags=flags)
    w1, w2 = r.prepare(inp["w1"], inp["w2"])
    y = r.forward(inp["x"], inp["x_sf"], inp["topk_idx"], inp["topk_w"], w1, inp["w1_sf"], w2,
                  inp["w2_sf"])
    torch.cuda.synchronize()
    return y, r


def _sizes_case(sizes, H, I, seed):
    T = sum(sizes)
    owner = [e for e, n in enumerate(sizes) for _ in range(n)]
    return small_case(T, H, I, len(sizes), 1, seed, mask={(t, 0): owner[t] for t in range(T)})


def _hot_mask(T):
    # every token's first slot on expert 3 (T rows), the second slot of
    # tokens 0-639 on expert 5 (exactly 4 row blocks of 160), the others on
    # the remaining experts in turn
    alt = [0, 1, 2, 4, 6, 7]
    mask = {(t, 0): 3 for t in range(T)}
    mask.update({(t, 1): 5 if t < 640 else alt[t % 6] for t in range(T)})
    return mask


CASES = ["ragged", "hot", "many_blocks", "tiny_rows", "padding_halves", "hot_panels"]


@pytest.mark.parametrize("case", CASES)
def test_tile160_matches_tile128_bitwise_and_oracle(case):
    if case == "ragged":
        host, dev = small_case(203, 512, 384, 16, 4, 12)
    elif case == "hot":
        T = 150
        host, dev = small_case(T, 256, 256, 8, 2, 14, mask={(t, 0): 2 for t in range(T)})
    elif case == "many_blocks":
        host, dev = small_case(600, 512, 512, 16, 4, 22)
    elif case == "tiny_rows":  # the minimum K blocks, masked slots, a token with no slot
        host, dev = small_case(45, 256, 256, 6, 3, 23, mask={(0, 0): -1, (0, 1): -1, (0, 2): -1,
                                                             (5, 1): -3})
    elif case == "padding_halves":
        # experts of 1, 79, 80, 81, 159, 160, 161 rows: the second row half
        # (rows 80-159) holds only padding for <= 80 rows and skips its MFMAs
        host, dev = _sizes_case([1, 79, 80, 81, 159, 160, 161, 0], 256, 256, 41)
    else:  # experts of 7 and 4 row blocks: the hot-expert panel walk
        T = 1100
        host, dev = small_case(T, 512, 512, 8, 2, 31, mask=_hot_mask(T))
    T = dev["x"].shape[0]
    say(f"tile160 {case}: T={T}")
    y160, r160 = _run(dev, 160)
    info = moe.moe_plan_info(r160.plan, T)
    assert info["kernel"] == 3 and info["tile_m"] == 160 and info["row_align"] == 160
    if case == "hot_panels":
        st = moe.moe_read_status(r160.plan, T, r160.workspace)
        assert st[3] == 7 * 160, st
    y128, r128 = _run(dev, 128)
    assert moe.moe_plan_info(r128.plan, T)["kernel"] == 1
    assert torch.equal(y160, y128), case
    # 4 workgroups: each walks many tiles (slots rotate, copies of the next
    # tile overlap the current tile's epilogue); same arithmetic per tile
    y_small, _ = _run(dev, 160, moe.MOE_FLAG_TEST_SMALL_GRID)
    assert torch.equal(y160, y_small), case
    verify(y160, r160, host, f"tile 160 {case}")


@pytest.mark.parametrize("name", ["pro_prefill", "skewed"])
def test_tile160_full_size_matches_tile128_bitwise(name):
    # The full workloads (every token, every slot): the 160-row tile against
    # the 128-row tile, whose output the full-size oracle tests check on
    # sampled tokens; the h intermediate and its scales are compared too.
    cfg = wl.CONFIGS[name]
    inp = gpu_inputs(cfg, wl.default_seed(cfg))
    say(f"tile160 full size {name}")
    y160, r160 = _run(inp, 160)
    assert moe.moe_plan_info(r160.plan, cfg.T)["kernel"] == 3
    h160 = r160.view("h", cfg.T).clone()
    sf160 = r160.view("h_sf", cfg.T).clone()
    rs160 = r160.view("row_src", cfg.T).clone()
    del r160
    y128, r128 = _run(inp, 128)
    assert torch.equal(y160, y128), name
    # h rows by routed slot: the pools differ in alignment, the slots' rows not
    h128 = r128.view("h", cfg.T)
    sf128 = r128.view("h_sf", cfg.T)
    rs128 = r128.view("row_src", cfg.T)
    TK = cfg.T * cfg.K
    for rs, h, sf, tag in ((rs160, h160, sf160, "160"), (rs128, h128, sf128, "128")):
        m = (rs >= 0) & (rs < TK)
        order = torch.argsort(rs[m])
        if tag == "160":
            a_h, a_sf = h[m][order], sf[m][order]
        else:
            b_h, b_sf = h[m][order], sf[m][order]
    assert torch.equal(a_h, b_h) and torch.equal(a_sf, b_sf), name
    del inp, r128
    torch.cuda.empty_cache()
