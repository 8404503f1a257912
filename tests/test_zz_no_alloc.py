"""moe_forward_noalloc (the forward for callers that cannot allocate: its
workspace is the library's static per-GPU scratch array) against
moe_forward with a caller workspace: the same kernels on the same inputs,
so y must be bit-identical -- on two calls in a row, the second with fewer
tokens (the array keeps the first call's contents), at the flash-decode
shape (256 experts, hidden 4096, intermediate 2048, top-6) and on a small
ragged case with masked and out-of-range ids; the first call is also held
to the oracle through the chain check."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import workload as wl
from parity_util import host_copy_for_oracle, say, verify

pytestmark = pytest.mark.gpu


def _noalloc(runner, inp, T, w1, w2):
    y = torch.full((T, inp["x"].shape[1]), 0x7FC0, dtype=torch.uint16, device="cuda")
    moe.moe_forward_noalloc(runner.plan, T, inp["x"][:T], inp["x_sf"][:T], inp["topk_idx"][:T],
                            inp["topk_w"][:T], w1, inp["w1_sf"], w2, inp["w2_sf"], y)
    return y


def _with_workspace(runner, inp, T, w1, w2):
    return runner.forward(inp["x"][:T], inp["x_sf"][:T], inp["topk_idx"][:T], inp["topk_w"][:T],
                          w1, inp["w1_sf"], w2, inp["w2_sf"])


@pytest.mark.parametrize("case", ["flash_decode", "ragged"])
def test_noalloc_matches_forward_two_calls(case):
    if case == "flash_decode":
        cfg = wl.CONFIGS["flash_decode"]
        inp = wl.make_inputs(cfg, wl.default_seed(cfg), "cuda")
        layout, T1, T2 = moe.MOE_WEIGHTS_PACKED, 128, 37
    else:
        cfg = wl.custom_config(203, 512, 384, 16, 4)
        inp = wl.make_inputs(cfg, 12, "cuda")
        idx = inp["topk_idx"].clone()
        idx[0] = -1
        idx[5, 1] = 999
        inp["topk_idx"] = idx
        layout, T1, T2 = moe.MOE_WEIGHTS_ROW_MAJOR, 203, 40
    runner = moe.MoEForward(cfg.H, cfg.I, cfg.E, cfg.K, cfg.T, weight_layout=layout)
    w1, w2 = runner.prepare(inp["w1"], inp["w2"])
    for T in (T1, T2):
        say(f"no-alloc {case}: T={T}")
        y_na = _noalloc(runner, inp, T, w1, w2)
        torch.cuda.synchronize()
        y_ws = _with_workspace(runner, inp, T, w1, w2)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), (case, T)
        if T == T1:  # the reference path itself against the oracle
            verify(y_ws, runner, host_copy_for_oracle(inp, list(range(T))), f"no-alloc {case}")
    del inp, w1, w2
    torch.cuda.empty_cache()


def test_noalloc_rejects_calls_beyond_its_scratch():
    # pro shape: 8192 tokens need far more than the static array holds; the
    # call is refused on the host and enqueues nothing
    cfg = wl.CONFIGS["pro_prefill"]
    p = moe.moe_plan_create(cfg.H, cfg.I, cfg.E, cfg.K, cfg.T)
    try:
        assert moe.moe_workspace_bytes(p, cfg.T) > moe.MOE_NOALLOC_SCRATCH_BYTES
        t = torch.zeros(256, dtype=torch.uint8, device="cuda")
        with pytest.raises(moe.MoEError) as e:
            moe.moe_forward_noalloc(p, cfg.T, t, t, t, t, t, t, t, t, t)
        assert e.value.code == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    finally:
        moe.moe_plan_destroy(p)
