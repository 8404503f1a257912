"""The GPU parity checker (parity_util.verify) on the CPU.

A stand-in for a forward's workspace is filled from the oracle itself (its
plan, h, h_sf and partials placed in pool order), so verify must pass with
nothing moved; then single planted mistakes -- an h code moved where the
arithmetic cannot move it, a scale off by more than the bound, a wrong
partial, a y that is not the combine of its partials -- must each be
rejected.  The checker's arithmetic (bounds, index mapping, codecs) is thus
exercised before any GPU run relies on it.  CPU only.
"""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import oracle
import workload as wl
from parity_util import ORD, host_dict, verify


class StubRunner:
    """The attributes verify reads from a moe.MoEForward, backed by host
    arrays laid out as a forward leaves them in the workspace."""

    def __init__(self, H, I, E, K, T, mx, oflags, views):
        self.recipe = moe.MOE_RECIPE_MXFP4 if mx else moe.MOE_RECIPE_FP8_BLOCK128
        self.shape = (H, I, E, K, T, 16)
        gran = 64 if oflags & oracle.ORC_SF_GRAN64 else 0
        self.plan = moe.moe_plan_create(H, I, E, K, T, 16, recipe=self.recipe, act_sf_gran=gran)
        self.views = views

    def view(self, name, num_tokens):
        return torch.from_numpy(self.views[name])


def make_case(mx, oflags, seed=5):
    T, H, I, E, K = 11, 256, 256, 4, 2
    cfg = wl.custom_config(T, H, I, E, K)
    inp = (wl.make_inputs_mx if mx else wl.make_inputs)(cfg, seed, "cpu")
    idx = inp["topk_idx"].clone()
    idx[2, 0] = -1
    idx[2, 1] = -1      # a token with no slot
    idx[6, 1] = 9       # out of range
    inp["topk_idx"] = idx
    host = host_dict(inp)
    fwd = oracle.moe_forward_mx if mx else oracle.moe_forward
    ref = fwd(host["x"], host["x_sf"], host["idx"], host["w"], host["w1"], host["w1_sf"],
              host["w2"], host["w2_sf"], flags=oflags, want=("h", "partial"))
    ra = 16
    R = T * K + E * (ra - 1)
    R = (R + ra - 1) // ra * ra
    _, _, row_src, src_row, _ = oracle.route(host["idx"], E, ra, R)
    h = np.full((R, I), 0x55, np.uint8)
    sf = np.full((R,) + ref["h_sf"].shape[1:], 7, ref["h_sf"].dtype)
    part = np.full((K, T, H), 0x1234, np.uint16)
    for f in range(T * K):
        r = src_row[f]
        if r >= 0:
            h[r], sf[r] = ref["h"][f], ref["h_sf"][f]
            part[f % K, f // K] = ref["partial"][f]
    views = dict(src_row=src_row.astype(np.int32), h=h, h_sf=sf, partial=part.view(np.int16))
    runner = StubRunner(H, I, E, K, T, mx, oflags, views)
    y = torch.from_numpy(ref["y"].astype(np.int16))
    return y, runner, host, src_row


CASES = [(False, 0), (False, oracle.ORC_SF_GRAN64), (False, oracle.ORC_POW2_SCALE), (True, 0)]


@pytest.mark.parametrize("mx,oflags", CASES)
def test_checker_accepts_the_oracle_itself(mx, oflags):
    y, runner, host, _ = make_case(mx, oflags)
    st = verify(y, runner, host, "stub", oflags=oflags)
    assert st["moved"] == 0 and st["y_l2_fed"] == 0.0


@pytest.mark.parametrize("mx,oflags", CASES)
def test_checker_rejects_a_moved_h_code(mx, oflags):
    y, runner, host, src_row = make_case(mx, oflags)
    r = src_row[1]
    h = runner.views["h"]
    # move the largest-magnitude code of the row one step towards zero: far
    # from any rounding boundary the MFMA error could reach
    c = int(np.argmax(np.abs(ORD[h[r].astype(np.int64)])))
    h[r, c] = h[r, c] - 1
    with pytest.raises(AssertionError):
        verify(y, runner, host, "planted h", oflags=oflags, check_y_full=False)


def test_checker_rejects_a_scale_outside_the_bound():
    y, runner, host, src_row = make_case(False, 0)
    runner.views["h_sf"][src_row[3], 1] *= 1.02
    with pytest.raises(AssertionError):
        verify(y, runner, host, "planted scale", check_y_full=False)


def test_checker_rejects_a_pow2_scale_off_by_two():
    y, runner, host, src_row = make_case(False, oracle.ORC_POW2_SCALE)
    runner.views["h_sf"][src_row[3], 0] *= 2
    with pytest.raises(AssertionError):
        verify(y, runner, host, "planted pow2 scale", oflags=oracle.ORC_POW2_SCALE,
               check_y_full=False)


def test_checker_rejects_a_wrong_partial_and_a_wrong_y():
    y, runner, host, src_row = make_case(False, 0)
    part = runner.views["partial"]
    part[1, 4, 17] ^= 0x0004  # four bf16 ulps of one value
    with pytest.raises(AssertionError):
        verify(y, runner, host, "planted partial", check_y_full=False)
    y, runner, host, _ = make_case(False, 0)
    y[5, 3] ^= 1  # one ulp of one output
    with pytest.raises(AssertionError):
        verify(y, runner, host, "planted y", check_y_full=False)


def test_checker_ignores_rows_of_skipped_slots():
    # stale contents of rows and partials no routed slot owns are never read
    y, runner, host, src_row = make_case(False, 0)
    part = runner.views["partial"]
    part[0, 2] = 0x7F7F     # token 2 has no slot
    part[1, 6] = 0x7F7F     # slot (6, 1) is out of range
    st = verify(y, runner, host, "stale rows")
    assert st["moved"] == 0
