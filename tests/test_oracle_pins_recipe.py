"""Pins of the oracle's recipe options (FP8 recipe): power-of-two requant
scales, per-64 intermediate scales with the dual-half L2 of the design doc
§5.4, the activation clamp of §10.1, and the per-1x128 input quantisation.
Each is checked against a library routine, an independent fp64 model, a
closed form, or exact rational arithmetic at every rounding point.  CPU only.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workload as wl
from test_oracle_pins import (DEC, _bf16_bits, _e4m3, _f32, bf16_bits_to_f64, dequant_blocks,
                              rel_l2, small_inputs)


def run(d, **kw):
    return oracle.moe_forward(d["x"], d["x_sf"], d["idx"], d["w"], d["w1"], d["w1_sf"],
                              d["w2"], d["w2_sf"], **kw)


# -------------------------------------------------------- power-of-two scale


def test_pow2_requant_closed_forms_and_torch_cast():
    rng = np.random.default_rng(41)
    for k in (-9, 0, 4):
        codes = rng.integers(0, 0x7F, 128)
        codes[3] = 0x7E  # 448: amax = 448 * 2^k, scale exactly 2^k
        v = (DEC[codes] * 2.0 ** k).astype(np.float32)
        q, sf = oracle.requant_block(v, pow2=True)
        assert sf == 2.0 ** k and np.array_equal(DEC[q], DEC[codes])
    for _ in range(200):
        v = (rng.standard_t(3, 128) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        q, sf = oracle.requant_block(v, pow2=True)
        _, raw = oracle.requant_block(v)
        m, e = np.frexp(np.float64(sf))
        assert m == 0.5 and raw <= sf < 2 * raw  # the power of two just above
        ref = torch.from_numpy((v.astype(np.float64) / sf).astype(np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q & 0x7F, ref & 0x7F) and np.array_equal(q[q & 0x7F != 0],
                                                                       ref[q & 0x7F != 0])


# ------------------------------------------------------- input quantisation


def test_quantize_rows_matches_torch_and_the_generator():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(7, 512, generator=g) * torch.logspace(-3, 3, 7)[:, None]
    x[2, 128:256] = 0.0  # an all-zero block takes the 1e-10 floor
    xb = x.to(torch.bfloat16).to(torch.float32)  # bf16 inputs, exact in f32
    q, sf = oracle.quantize_rows(xb.numpy())
    blk = xb.reshape(7, 4, 128)
    want_sf = torch.clamp(blk.abs().amax(-1), min=1e-10) / 448.0
    assert np.array_equal(sf, want_sf.numpy())
    want_q = (blk / want_sf[..., None]).reshape(7, 512).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(q, want_q.numpy())
    gq, gsf = wl.quantize_blocks(xb, 1, 128)  # the input generator's own quantiser
    assert np.array_equal(q, gq.numpy()) and np.array_equal(sf, gsf.numpy())


# --------------------------------------------------------- fp64 models


def numpy_moe(d, gran=128, pow2=False, clamp=0.0):
    H, I, K, E = d["H"], d["I"], d["K"], d["E"]
    x = dequant_blocks(d["x"], d["x_sf"], 1, 128)
    y = np.zeros((d["T"], H))
    for t in range(d["T"]):
        for j in range(K):
            e = d["idx"][t, j]
            if e < 0 or e >= E:
                continue
            w1 = dequant_blocks(d["w1"][e], d["w1_sf"][e], 128, 128)
            w2 = dequant_blocks(d["w2"][e], d["w2_sf"][e], 128, 128)
            a = w1 @ x[t]
            g, u = a[:I], a[I:]
            if clamp > 0:
                g, u = np.clip(g, -clamp, clamp), np.clip(u, -clamp, clamp)
            hv = g / (1.0 + np.exp(-g)) * u * float(d["w"][t, j])
            hb = hv.reshape(-1, gran)
            sf = np.maximum(np.abs(hb).max(1), 1e-10) / 448.0
            if pow2:
                sf = 2.0 ** np.ceil(np.log2(sf))
            q = torch.from_numpy((hb / sf[:, None]).astype(np.float32)).to(
                torch.float8_e4m3fn).to(torch.float64).numpy()
            y[t] += w2 @ (q * sf[:, None]).reshape(-1)
    return y


@pytest.mark.parametrize("gran,pow2,clamp", [(64, False, 0.0), (128, True, 0.0), (64, True, 0.0),
                                             (128, False, 0.05), (64, False, 0.02)])
def test_options_match_fp64_model(gran, pow2, clamp):
    d = small_inputs(T=6, H=256, I=384, E=4, K=3, seed=51, mask={(2, 1): -1})
    flags = (oracle.ORC_SF_GRAN64 if gran == 64 else 0) | (oracle.ORC_POW2_SCALE if pow2 else 0)
    y = bf16_bits_to_f64(run(d, flags=flags, clamp=clamp)["y"])
    ref = numpy_moe(d, gran, pow2, clamp)
    for t in range(d["T"]):
        assert rel_l2(y[t], ref[t]) <= 1e-2, (t, rel_l2(y[t], ref[t]))
    if clamp > 0:  # the clamp is active: it changes y
        base = bf16_bits_to_f64(run(d, flags=flags)["y"])
        assert rel_l2(y, base) > 1e-2


def test_clamp_above_every_value_is_the_identity():
    d = small_inputs(T=5, H=256, I=256, E=3, K=2, seed=52)
    a = run(d, want=("acc1",))
    big = float(np.abs(a["acc1"]).max()) * 2
    assert np.array_equal(run(d, clamp=big)["y"], a["y"])


def test_per64_scales_cover_64_columns():
    d = small_inputs(T=4, H=256, I=384, E=3, K=2, seed=53)
    out = run(d, flags=oracle.ORC_SF_GRAN64, want=("h",))
    assert out["h_sf"].shape == (4 * 2, 384 // 64)
    for f in range(8):
        if (d["idx"].reshape(-1)[f] < 0):
            continue
        for b in range(6):
            codes = out["h"][f, 64 * b:64 * b + 64]
            # the block's largest magnitude maps to (224, 448]
            assert 224.0 < np.abs(DEC[codes]).max() <= 448.0, (f, b)


# ------------------------------------------- whole layer in exact arithmetic


def _pow2_at_least(q: Fraction) -> Fraction:
    e = 0
    while Fraction(2) ** e < q:
        e += 1
    while Fraction(2) ** (e - 1) >= q:
        e -= 1
    return Fraction(2) ** e


@pytest.mark.parametrize("gran,pow2,clamp", [(64, False, 0.0), (128, True, 0.0), (64, True, 0.03)])
def test_options_whole_layer_in_exact_arithmetic_tiny(gran, pow2, clamp):
    # As the FP8 exact-layer pin, with the option's rounding points: clamp
    # of gate/up (exact), per-64 requant blocks, power-of-two scales (the
    # f32 quotient by a power of two is exact), and the dual-half L2 (two
    # 64-term exact sums per 128-K block, each rounded once to f32, two fmas).
    T, H, I, E, K = 3, 256, 256, 2, 2
    d = small_inputs(T=T, H=H, I=I, E=E, K=K, seed=61, mask={(2, 1): -1})
    flags = (oracle.ORC_SF_GRAN64 if gran == 64 else 0) | (oracle.ORC_POW2_SCALE if pow2 else 0)
    out = run(d, flags=flags, clamp=clamp, want=("acc1", "h", "partial"))
    F = lambda v: Fraction(float(v))
    one_e10 = F(np.float32(1e-10))
    c = F(np.float32(clamp))
    xi = (DEC[d["x"].astype(np.int64)] * 512).astype(np.int64)
    y_exact = np.zeros((T, H), np.uint16)
    for t in range(T):
        a_sum = [Fraction(0)] * H
        for j in range(K):
            e = int(d["idx"][t, j])
            if e < 0:
                continue
            f = t * K + j
            acc = [F(v) for v in out["acc1"][f]]  # L1 is pinned by the FP8 exact test
            cl = (lambda v: min(max(v, -c), c)) if clamp > 0 else (lambda v: v)
            hv = [F(oracle.swiglu(float(cl(acc[i])), float(cl(acc[I + i])), float(d["w"][t, j])))
                  for i in range(I)]
            q, sfs = [], []
            for ib in range(I // gran):
                blk = hv[ib * gran:(ib + 1) * gran]
                sf = _f32(max(max(abs(v) for v in blk), one_e10) / 448)
                if pow2:
                    sf = _pow2_at_least(sf)
                sfs.append(sf)
                q += [_e4m3(_f32(v / sf)) for v in blk]
                assert sf == F(out["h_sf"][f, ib]), (t, j, ib)
            got = out["h"][f].astype(np.int64)
            want = np.array(q, np.int64)
            assert np.array_equal(np.where((got & 0x7F) == 0, 0, got),
                                  np.where((want & 0x7F) == 0, 0, want)), (t, j)
            hi = (DEC[want] * 512).astype(np.int64)
            w2i = (DEC[d["w2"][e].astype(np.int64)] * 512).astype(np.int64)
            for n in range(H):
                a = Fraction(0)
                for kb in range(I // 128):
                    sb = F(d["w2_sf"][e][n // 128, kb])
                    halves = ((0, 128),) if gran == 128 else ((0, 64), (64, 128))
                    for hh, (lo, up) in enumerate(halves):
                        p = Fraction(int(w2i[n, kb * 128 + lo:kb * 128 + up] @
                                         hi[kb * 128 + lo:kb * 128 + up]), 2 ** 18)
                        sa = sfs[kb] if gran == 128 else sfs[2 * kb + hh]
                        a = _f32(_f32(sa * sb) * _f32(p) + a)
                bits = _bf16_bits(a)
                assert bits == int(out["partial"][f, n]), (t, j, n)
                a_sum[n] = _f32(a_sum[n] + F(bf16_bits_to_f64(np.array([bits]))[0]))
        for n in range(H):
            y_exact[t, n] = _bf16_bits(a_sum[n])
    assert np.array_equal(out["y"], y_exact)
