"""Pins of the oracle's auxiliary outputs, the ones the GPU parity tests use
to decide which differences from the oracle the hardware's arithmetic can
explain:

  - moe_l2_combine / moe_l2_combine_mx: steps 5-6 (L2 + combine) started
    from a given intermediate; fed the forward's own h and h_sf they must
    give the forward's partials and y bit for bit (both recipes, every
    intermediate-scale option, masked and out-of-range slots, token lists);
  - acc1_mag / o_mag: sum over K blocks of |scale product| x (sum of
    |products| in the block), against an fp64 numpy model written here from
    the closed-form e4m3 / e2m1 tables;
  - hval: the SwiGLU x top-k weight output before requantisation, against an
    fp64 numpy SiLU, and re-encoded with torch's e4m3 cast it gives h.
CPU only.
"""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_pins import DEC, small_inputs, run_oracle
from test_oracle_pins_mx import DEC4, DEC8, small_inputs_mx, run_mx, unpack_e2m1


def _l2_fp8(d, ref, toks=None, flags=0):
    return oracle.moe_l2_combine(d["idx"], d["w2"], d["w2_sf"], ref["h"], ref["h_sf"],
                                 tokens=toks, flags=flags, want=("partial", "o_mag"))


@pytest.mark.parametrize("flags", [0, oracle.ORC_SF_GRAN64, oracle.ORC_POW2_SCALE,
                                   oracle.ORC_SF_GRAN64 | oracle.ORC_POW2_SCALE])
def test_l2_combine_fed_own_h_reproduces_forward_bitwise(flags):
    mask = {(0, 0): -1, (0, 1): -1, (2, 1): 7, (4, 0): -2}  # masked token, id >= E
    d = small_inputs(T=9, H=256, I=384, E=4, K=2, seed=31, mask=mask)
    ref = run_oracle(d, flags=flags, want=("h", "partial"))
    got = _l2_fp8(d, ref, flags=flags)
    assert got["n_bad"] == ref["n_bad"] == 1
    assert np.array_equal(got["y"], ref["y"])
    valid = (d["idx"].reshape(-1) >= 0) & (d["idx"].reshape(-1) < d["E"])
    assert np.array_equal(got["partial"][valid], ref["partial"][valid])
    # a token list: rows of h follow the listed tokens
    toks = [5, 0, 8]
    ref_t = run_oracle(d, flags=flags, tokens=toks, want=("h",))
    got_t = _l2_fp8(d, ref_t, toks=toks, flags=flags)
    assert np.array_equal(got_t["y"], ref_t["y"])
    assert np.array_equal(got_t["y"], ref["y"][toks])


def test_l2_combine_uses_the_given_h():
    # a changed code moves the partial of that slot only, by the exact amount
    # its weight column says (one code, one 128-block, one scale product)
    d = small_inputs(T=4, H=256, I=256, E=2, K=2, seed=32)
    ref = run_oracle(d, want=("h",))
    h = ref["h"].copy()
    f = 3
    e = d["idx"].reshape(-1)[f]
    col = 130  # block 1
    old = int(h[f, col])
    h[f, col] = 0x38 if old != 0x38 else 0x30  # 1.0 or 0.5
    base = oracle.moe_l2_combine(d["idx"], d["w2"], d["w2_sf"], ref["h"], ref["h_sf"],
                                 want=("partial",))
    got = oracle.moe_l2_combine(d["idx"], d["w2"], d["w2_sf"], h, ref["h_sf"],
                                want=("partial",))
    others = [g for g in range(8) if g != f]
    assert np.array_equal(got["partial"][others], base["partial"][others])
    bf = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    delta = (DEC[h[f, col]] - DEC[old]) * ref["h_sf"][f, 1] * \
        DEC[d["w2"][e][:, col]] * np.repeat(d["w2_sf"][e][:, 1], 128)
    diff = bf(got["partial"][f]) - bf(base["partial"][f])
    # both sides are bf16 roundings of values delta apart
    assert np.allclose(diff, delta, rtol=2e-2, atol=4e-3 * np.abs(bf(base["partial"][f])).max())


def _mag_model_fp8(a_codes, a_sf, w, w_sf):
    """sum_kb |sa*sb| * sum_c |a_c * b_c| for every output row of w."""
    A = np.abs(DEC[a_codes.astype(np.int64)]).reshape(-1, 128)      # [KB,128]
    B = np.abs(DEC[w.astype(np.int64)]).reshape(w.shape[0], -1, 128)  # [N,KB,128]
    blk = np.einsum("kc,nkc->nk", A, B)
    s = np.abs(a_sf.astype(np.float64)[None, :] *
               np.repeat(w_sf.astype(np.float64), 128, axis=0))
    return (blk * s).sum(1)


def test_acc1_mag_and_o_mag_match_fp64_model():
    d = small_inputs(T=5, H=384, I=256, E=3, K=2, seed=33)
    ref = run_oracle(d, want=("acc1", "acc1_mag", "h"))
    l2 = _l2_fp8(d, ref)
    K = d["K"]
    for f in range(d["T"] * K):
        t, e = f // K, d["idx"].reshape(-1)[f]
        m1 = _mag_model_fp8(d["x"][t], d["x_sf"][t], d["w1"][e], d["w1_sf"][e])
        assert np.allclose(ref["acc1_mag"][f], m1, rtol=1e-6, atol=0)
        assert np.all(ref["acc1_mag"][f] >= np.abs(ref["acc1"][f]) * (1 - 1e-6))
        m2 = _mag_model_fp8(ref["h"][f], ref["h_sf"][f], d["w2"][e], d["w2_sf"][e])
        assert np.allclose(l2["o_mag"][f], m2, rtol=1e-6, atol=0)


def test_o_mag_per64_halves():
    d = small_inputs(T=3, H=256, I=256, E=2, K=2, seed=34)
    ref = run_oracle(d, flags=oracle.ORC_SF_GRAN64, want=("h",))
    l2 = _l2_fp8(d, ref, flags=oracle.ORC_SF_GRAN64)
    for f in range(6):
        e = d["idx"].reshape(-1)[f]
        A = np.abs(DEC[ref["h"][f].astype(np.int64)]) * np.repeat(ref["h_sf"][f], 64)
        B = np.abs(DEC[d["w2"][e].astype(np.int64)]) * \
            np.repeat(np.repeat(d["w2_sf"][e], 128, axis=0), 128, axis=1)
        assert np.allclose(l2["o_mag"][f], B @ A, rtol=1e-6, atol=0)


def test_hval_is_the_swiglu_output_and_encodes_to_h():
    d = small_inputs(T=6, H=256, I=256, E=3, K=2, seed=35)
    ref = run_oracle(d, want=("acc1", "hval", "h"))
    I, K = d["I"], d["K"]
    g = ref["acc1"][:, :I].astype(np.float64)
    u = ref["acc1"][:, I:].astype(np.float64)
    w = d["w"].reshape(-1).astype(np.float64)[:, None]
    model = g / (1.0 + np.exp(-g)) * u * w
    assert np.allclose(ref["hval"], model, rtol=1e-5, atol=1e-7 * np.abs(model).max())
    hv = ref["hval"].reshape(-1, I // 128, 128)
    sf = (np.maximum(np.abs(hv).max(-1), np.float32(1e-10)) / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(sf, ref["h_sf"])
    q = torch.from_numpy((hv / sf[..., None]).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(q.view(torch.uint8).numpy().reshape(-1, I), ref["h"])


def test_mx_l2_combine_fed_own_h_reproduces_forward_bitwise():
    mask = {(1, 0): -1, (3, 1): 9}
    d = small_inputs_mx(T=7, H=256, I=256, E=3, K=2, seed=36, mask=mask)
    ref = run_mx(d, want=("h", "partial"))
    got = oracle.moe_l2_combine_mx(d["idx"], d["w2"], d["w2_sf"], ref["h"], ref["h_sf"],
                                   want=("partial", "o_mag"))
    assert np.array_equal(got["y"], ref["y"])
    valid = (d["idx"].reshape(-1) >= 0) & (d["idx"].reshape(-1) < d["E"])
    assert np.array_equal(got["partial"][valid], ref["partial"][valid])


def test_mx_magnitudes_match_fp64_model():
    d = small_inputs_mx(T=4, H=256, I=256, E=2, K=2, seed=37)
    ref = run_mx(d, want=("acc1", "acc1_mag", "h"))
    l2 = oracle.moe_l2_combine_mx(d["idx"], d["w2"], d["w2_sf"], ref["h"], ref["h_sf"],
                                  want=("o_mag",))

    def model(a, a_sf, w, w_sf):
        A = np.abs(DEC8[a.astype(np.int64)]) * np.repeat(np.ldexp(1.0, a_sf.astype(np.int64) - 127), 32)
        B = np.abs(DEC4[unpack_e2m1(w)]) * np.repeat(np.ldexp(1.0, w_sf.astype(np.int64) - 127), 32, axis=1)
        return B @ A

    for f in range(8):
        t, e = f // 2, d["idx"].reshape(-1)[f]
        m1 = model(d["x"][t], d["x_sf"][t], d["w1"][e], d["w1_sf"][e])
        assert np.allclose(ref["acc1_mag"][f], m1, rtol=1e-6, atol=0)
        assert np.all(ref["acc1_mag"][f] >= np.abs(ref["acc1"][f]) * (1 - 1e-6))
        m2 = model(ref["h"][f], ref["h_sf"][f], d["w2"][e], d["w2_sf"][e])
        assert np.allclose(l2["o_mag"][f], m2, rtol=1e-6, atol=0)
