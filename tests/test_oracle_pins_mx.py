"""Pins of the oracle's FP8 x MXFP4 recipe against things other than itself:
the OCP MX value tables, torch's UE8M0 codec, exact rational arithmetic, an
independently written fp64 numpy model, and exact invariants.  CPU only.

Recipe (the SM100 MegaMoE kernel as the "07 · MegaMoE" page §0 describes it:
e4m3 activations, e2m1 weights, one UE8M0 scale per 32 K values, recipe
(1,1,32)); the readings the pages leave open are stated in the oracle's
header and repeated where a test depends on them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workload as wl

# OCP Microscaling Formats (MX) v1.0, E2M1 element values for codes 0..7
E2M1_TABLE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(code: int) -> float:
    v = E2M1_TABLE[code & 7]
    return -v if code & 8 else v


def e4m3_value(code: int) -> float:
    """OCP E4M3FN (1-4-3, bias 7, no inf, S.1111.111 = NaN)."""
    s = -1.0 if code & 0x80 else 1.0
    E, M = (code >> 3) & 0xF, code & 0x7
    if E == 0xF and M == 0x7:
        return float("nan")
    if E == 0:
        return s * (M / 8.0) * 2.0 ** -6
    return s * (1.0 + M / 8.0) * 2.0 ** (E - 7)


DEC8 = np.array([e4m3_value(c) for c in range(256)])
DEC4 = np.array([e2m1_value(c) for c in range(16)])


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """[R, C/2] bytes -> [R, C] codes; element k in byte k/2, even k low nibble."""
    p = packed.astype(np.int64)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def scale_rep(codes: np.ndarray) -> np.ndarray:
    """[..., C/32] UE8M0 codes -> [..., C] float64 scales."""
    return np.repeat(np.ldexp(1.0, codes.astype(np.int64) - 127), 32, axis=-1)


def small_inputs_mx(T=6, H=256, I=256, E=3, K=2, seed=7, mask=None):
    cfg = wl.custom_config(T, H, I, E, K)
    x, x_sf = wl.make_x_mx(cfg, seed)
    idx, w = wl.make_routing(cfg, seed)
    ex = [wl.make_expert_mx(cfg, seed, e) for e in range(E)]
    idx = idx.numpy().copy()
    for (t, j), v in (mask or {}).items():
        idx[t, j] = v
    return dict(x=x.numpy(), x_sf=x_sf.numpy(), idx=idx, w=w.numpy(),
                w1=[e[0].numpy() for e in ex], w1_sf=[e[1].numpy() for e in ex],
                w2=[e[2].numpy() for e in ex], w2_sf=[e[3].numpy() for e in ex],
                H=H, I=I, E=E, K=K, T=T)


def run_mx(d, **kw):
    return oracle.moe_forward_mx(d["x"], d["x_sf"], d["idx"], d["w"], d["w1"], d["w1_sf"],
                                 d["w2"], d["w2_sf"], **kw)


def bf16_f64(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ----------------------------------------------------------------- codecs


def test_e2m1_decode_matches_ocp_table_all_codes():
    for c in range(16):
        got = oracle.e2m1_decode(c)
        assert got == e2m1_value(c), c
        assert math.copysign(1.0, got) == (-1.0 if c & 8 else 1.0), c
    # only the low nibble is a code
    assert oracle.e2m1_decode(0x35) == e2m1_value(5)


def test_e8m0_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e8m0_decode(c)
        if c == 255:
            assert math.isnan(got) and math.isnan(ref[c])
        else:
            assert got == ref[c] == 2.0 ** (c - 127), c


def test_e8m0_ceil_is_the_smallest_power_of_two_at_or_above():
    rng = np.random.default_rng(3)
    vals = np.concatenate([np.exp(rng.uniform(-80, 80, 2000)),
                           [2.0 ** k for k in range(-120, 120, 7)],
                           [np.float32(1e-10) / np.float32(448)]]).astype(np.float32)
    for v in vals:
        c = oracle.e8m0_ceil(float(v))
        m, e = math.frexp(float(v))  # v = m 2^e, 0.5 <= m < 1
        want = e - 1 if m == 0.5 else e
        assert c == want + 127, (v, c, want)


# ------------------------------------------------------------ requantise


def test_requant_mx_closed_forms():
    rng = np.random.default_rng(5)
    # (a) amax exactly 448 * 2^k, every value an e4m3 value times 2^k: scale 2^k,
    # codes re-encode exactly
    for k in (-12, -3, 0, 5):
        codes = rng.integers(0, 0x7F, 32)
        codes[7] = 0x7E  # 448
        v = np.array([e4m3_value(int(c)) for c in codes]) * 2.0 ** k
        q, sc = oracle.requant_block_mx(v.astype(np.float32))
        assert sc == 127 + k
        assert [e4m3_value(int(c)) for c in q] == [e4m3_value(int(c)) for c in codes]
    # (b) amax just above 448 * 2^k: the next power of two; the amax element's
    # quotient lies in (224, 448], so its code is 224 or above
    for k in (-6, 0, 3):
        v = rng.normal(size=32).astype(np.float32)
        v[11] = np.float32(448.0 * 2.0 ** k * (1 + 2.0 ** -20))
        q, sc = oracle.requant_block_mx(v)
        assert sc == 128 + k
        assert 224.0 <= abs(e4m3_value(int(q[11]))) <= 448.0
        assert all(abs(e4m3_value(int(c))) <= 448.0 for c in q)
    # (c) scaling the block by 2^j keeps the codes and moves the scale by j
    v = rng.normal(size=32).astype(np.float32) * np.float32(3.7)
    q0, s0 = oracle.requant_block_mx(v)
    for j in (-9, -1, 1, 6):
        q1, s1 = oracle.requant_block_mx((v * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q0, q1) and s1 == s0 + j
    # (d) all-zero block: floor 1e-10 -> scale 2^-42, codes zero
    q, sc = oracle.requant_block_mx(np.zeros(32, np.float32))
    assert sc == 127 - 42 and not q.any()


def test_requant_mx_matches_torch_cast_after_power_of_two_scaling():
    # q = e4m3(v / sf) with sf a power of two: torch's RNE e4m3 cast of the
    # exactly scaled values must give the same codes (within +-448)
    rng = np.random.default_rng(9)
    for _ in range(200):
        v = (rng.standard_t(3, size=32) * 10.0 ** rng.uniform(-8, 8)).astype(np.float32)
        q, sc = oracle.requant_block_mx(v)
        sf = 2.0 ** (sc - 127)
        ref = torch.from_numpy((v.astype(np.float64) / sf).astype(np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        same = (q == ref) | (((q & 0x7F) == 0) & ((ref & 0x7F) == 0))
        assert same.all()


# ----------------------------------------------------------------- MX GEMM


def exact_mx_dot(a, sa, b_codes, sb) -> Fraction:
    """Exact rational sum: e4m3 values are multiples of 2^-9, e2m1 of 2^-1."""
    ai = [int(round(e4m3_value(int(c)) * 512)) for c in a]
    bi = [int(round(e2m1_value(int(c)) * 2)) for c in b_codes]
    s = Fraction(0)
    for blk in range(len(a) // 32):
        p = sum(ai[k] * bi[k] for k in range(32 * blk, 32 * blk + 32))
        s += Fraction(p) * Fraction(2) ** (int(sa[blk]) + int(sb[blk]) - 254 - 10)
    return s


def test_mx_dot_matches_exact_rationals_and_fp64():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = 32 * int(rng.integers(1, 9))
        a = rng.integers(0, 256, n)
        a[(a & 0x7F) == 0x7F] = 0  # no NaN codes
        b = rng.integers(0, 16, n)
        spread = 8 if trial % 2 else 40
        sa = rng.integers(127 - spread, 127 + spread, n // 32)
        sb = rng.integers(127 - spread, 127 + spread, n // 32)
        got = oracle.mx_dot(a, sa, pack_e2m1(b), sb)
        # reading: blocks added in ascending order in binary64; each block's
        # value is exact in binary64, so Python float addition reproduces it
        seq = 0.0
        for blk in range(n // 32):
            seq += float(exact_mx_dot(a[32 * blk:32 * blk + 32], sa[blk:blk + 1],
                                      b[32 * blk:32 * blk + 32], sb[blk:blk + 1]))
        assert got == seq, trial
        if spread == 8:  # terms span < 53 bits: the exact sum
            assert Fraction(got) == exact_mx_dot(a, sa, b, sb), trial
        va = DEC8[a] * scale_rep(sa)
        vb = DEC4[b] * scale_rep(sb)
        ref = float(va @ vb)
        assert abs(got - ref) <= 1e-12 * float(np.abs(va) @ np.abs(vb)) + 1e-300, trial
    # a NaN scale code poisons the sum
    assert math.isnan(oracle.mx_dot(np.zeros(32), [255], np.zeros(16), [127]))


def test_mx_dot_reads_the_even_element_from_the_low_nibble():
    a = np.zeros(32, np.int64)
    a[0] = 0x38  # 1.0 at k = 0 only
    b = np.zeros(32, np.int64)
    b[0], b[1] = 2, 7  # 1.0 at k = 0, 6.0 at k = 1
    assert oracle.mx_dot(a, [127], pack_e2m1(b), [127]) == 1.0
    a[0], a[1] = 0, 0x38
    assert oracle.mx_dot(a, [127], pack_e2m1(b), [127]) == 6.0


# ------------------------------------------------------------ whole oracle


def numpy_moe_mx(d, requant=True):
    """Independent fp64 model of the MX forward; the optional per-32
    power-of-two requantisation goes through torch's e4m3 cast."""
    H, I, K, E = d["H"], d["I"], d["K"], d["E"]
    x = DEC8[d["x"].astype(np.int64)] * scale_rep(d["x_sf"])
    y = np.zeros((d["T"], H))
    for t in range(d["T"]):
        for j in range(K):
            e = d["idx"][t, j]
            if e < 0 or e >= E:
                continue
            w1 = DEC4[unpack_e2m1(d["w1"][e])] * scale_rep(d["w1_sf"][e])
            w2 = DEC4[unpack_e2m1(d["w2"][e])] * scale_rep(d["w2_sf"][e])
            a = w1 @ x[t]
            g, u = a[:I], a[I:]
            hval = g / (1.0 + np.exp(-g)) * u * float(d["w"][t, j])
            if requant:
                hb = hval.reshape(-1, 32)
                s = np.maximum(np.abs(hb).max(1), 1e-10) / 448.0
                sf = 2.0 ** np.ceil(np.log2(s))
                q = torch.from_numpy((hb / sf[:, None]).astype(np.float32)).to(
                    torch.float8_e4m3fn).to(torch.float64).numpy()
                hval = (q * sf[:, None]).reshape(-1)
            y[t] += w2 @ hval
    return y


def test_mx_unquantised_switches_match_fp64_moe():
    d = small_inputs_mx(T=6, H=256, I=384, E=4, K=3, seed=21, mask={(1, 2): -1, (4, 0): 9})
    out = run_mx(d, flags=oracle.ORC_NO_REQUANT | oracle.ORC_NO_BF16, want=("y_f32",))
    ref = numpy_moe_mx(d, requant=False)
    assert out["n_bad"] == 1
    for t in range(d["T"]):
        assert rel_l2(out["y_f32"][t].astype(np.float64), ref[t]) <= 1e-5, t


def test_mx_full_oracle_within_quantisation_budget_of_fp64_moe():
    d = small_inputs_mx(T=6, H=256, I=384, E=4, K=3, seed=22, mask={(2, 1): -1})
    y = bf16_f64(run_mx(d)["y"])
    ref_q = numpy_moe_mx(d, requant=True)
    ref_f = numpy_moe_mx(d, requant=False)
    for t in range(d["T"]):
        assert rel_l2(y[t], ref_q[t]) <= 1e-2, t
        r = rel_l2(y[t], ref_f[t])
        assert 1e-4 <= r <= 0.1, (t, r)


def test_mx_dense_ffn_reduction():
    """E=1, K=1, w=1: a dense SwiGLU FFN on the same operands."""
    d = small_inputs_mx(T=4, H=256, I=256, E=1, K=1, seed=23)
    d["w"] = np.ones_like(d["w"])
    y = bf16_f64(run_mx(d)["y"])
    x = DEC8[d["x"].astype(np.int64)] * scale_rep(d["x_sf"])
    w1 = DEC4[unpack_e2m1(d["w1"][0])] * scale_rep(d["w1_sf"][0])
    w2 = DEC4[unpack_e2m1(d["w2"][0])] * scale_rep(d["w2_sf"][0])
    gate, up = x @ w1[:256].T, x @ w1[256:].T
    hid = gate / (1 + np.exp(-gate)) * up
    blocks = hid.reshape(4, -1, 32)
    sf = 2.0 ** np.ceil(np.log2(np.maximum(np.abs(blocks).max(-1, keepdims=True), 1e-10) / 448.0))
    q = torch.from_numpy((blocks / sf).astype(np.float32)).to(torch.float8_e4m3fn)
    ref = (q.to(torch.float64).numpy() * sf).reshape(4, -1) @ w2.T
    for t in range(4):
        assert rel_l2(y[t], ref[t]) <= 5e-3, t


def test_mx_exact_invariants_bitwise():
    d = small_inputs_mx(T=6, H=256, I=256, E=4, K=2, seed=24)
    y0 = run_mx(d)["y"]
    # (i) router weights x2 -> y x2
    d2 = dict(d, w=d["w"] * np.float32(2))
    assert np.array_equal(bf16_f64(run_mx(d2)["y"]), 2 * bf16_f64(y0))
    # (ii) every L2 weight scale code + 1 -> y x2
    d3 = dict(d, w2_sf=[(s + 1).astype(np.uint8) for s in d["w2_sf"]])
    assert np.array_equal(bf16_f64(run_mx(d3)["y"]), 2 * bf16_f64(y0))
    # (iii) one L1 weight block's scale code + 1 equals that block's values x2
    # (e2m1 codes 1..5 double to codes 3..7 exactly: 0.5->1, 1->2, 1.5->3, 2->4, 3->6)
    dbl = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 5: 7}
    e, n, blk = 1, 5, 2
    codes = unpack_e2m1(d["w1"][e])
    seg = codes[n, 32 * blk:32 * blk + 32]
    if np.all(np.isin(seg & 7, list(dbl))):
        w1a = [w.copy() for w in d["w1"]]
        c2 = codes.copy()
        c2[n, 32 * blk:32 * blk + 32] = [dbl[c & 7] | (c & 8) for c in seg]
        w1a[e] = pack_e2m1(c2)
        s1b = [s.copy() for s in d["w1_sf"]]
        s1b[e][n, blk] += 1
        ya = run_mx(dict(d, w1=w1a))["y"]
        yb = run_mx(dict(d, w1_sf=s1b))["y"]
        assert np.array_equal(ya, yb)
    # (iv) permuting tokens permutes y; (v) relabelling experts leaves y
    perm = np.array([3, 0, 5, 1, 4, 2])
    d4 = dict(d, x=d["x"][perm].copy(), x_sf=d["x_sf"][perm].copy(), idx=d["idx"][perm].copy(),
              w=d["w"][perm].copy())
    assert np.array_equal(run_mx(d4)["y"], y0[perm])
    rel = np.array([2, 0, 3, 1])
    inv = np.argsort(rel)
    d5 = dict(d, idx=rel[d["idx"]].astype(np.int32),
              w1=[d["w1"][inv[e]] for e in range(4)], w1_sf=[d["w1_sf"][inv[e]] for e in range(4)],
              w2=[d["w2"][inv[e]] for e in range(4)], w2_sf=[d["w2_sf"][inv[e]] for e in range(4)])
    assert np.array_equal(run_mx(d5)["y"], y0)
    assert np.array_equal(run_mx(d, tokens=[4, 1])["y"], y0[[4, 1]])


def test_mx_masked_token_gives_zero():
    d = small_inputs_mx(T=4, H=256, I=128, E=3, K=2, seed=25,
                        mask={(1, 0): -1, (1, 1): -1, (2, 1): 7})
    out = run_mx(d)
    assert out["n_bad"] == 1
    assert not out["y"][1].any()
    # token 2 = its slot 0 alone
    d1 = dict(d, idx=np.array([[d["idx"][2, 0], -1]], np.int32), x=d["x"][2:3].copy(),
              x_sf=d["x_sf"][2:3].copy(), w=d["w"][2:3].copy())
    assert np.array_equal(run_mx(d1)["y"][0], out["y"][2])


# ------------------------------------------- whole layer in exact arithmetic


def _round_binary(q: Fraction, mant: int, emin: int) -> Fraction:
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, emin) - mant)
    m = a / ulp
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return (n * ulp) if q > 0 else -(n * ulp)


def _f32(q):
    return _round_binary(q, 23, -126)


def _bf16_bits(q):
    v = np.float32(float(_round_binary(q, 7, -126)))
    return int(np.array([v]).view(np.uint32)[0] >> 16)


_E4M3_CODE = {Fraction(float(DEC8[c])): c for c in range(0x7F)}


def _e4m3(q):
    r = _round_binary(q, 3, -6)
    r = max(min(r, Fraction(448)), Fraction(-448))
    return _E4M3_CODE[abs(r)] | (0x80 if r < 0 else 0)


def _pow2_ceil(q: Fraction) -> int:
    e = 0
    while Fraction(2) ** e < q:
        e += 1
    while Fraction(2) ** (e - 1) >= q:
        e -= 1
    return e


def test_mx_whole_layer_in_exact_arithmetic_tiny():
    # Every rounding point written out with exact rationals: each GEMM value
    # is the exact sum over K (integer block sums times powers of two)
    # rounded once to f32, the requant scale the smallest power of two at or
    # above f32(max(amax, 1e-10)/448), codes by exact scaling and e4m3
    # rounding, bf16 partials, f32 combine, bf16 y.  SiLU comes from the
    # oracle's pinned routine.
    T, H, I, E, K = 3, 128, 128, 2, 2
    d = small_inputs_mx(T=T, H=H, I=I, E=E, K=K, seed=31, mask={(2, 1): -1})
    out = run_mx(d, want=("acc1", "h", "partial"))
    F = lambda v: Fraction(float(v))
    floor = F(np.float32(1e-10))
    xi = np.rint(DEC8[d["x"].astype(np.int64)] * 512).astype(np.int64)
    y_exact = np.zeros((T, H), np.uint16)

    def gemm_exact(ai, asc, bi, bsc):
        s = Fraction(0)
        for blk in range(len(ai) // 32):
            p = int(ai[32 * blk:32 * blk + 32] @ bi[32 * blk:32 * blk + 32])
            s += Fraction(p) * Fraction(2) ** (int(asc[blk]) + int(bsc[blk]) - 254 - 10)
        return _f32(s)

    for t in range(T):
        a_sum = [Fraction(0)] * H
        for j in range(K):
            e = int(d["idx"][t, j])
            if e < 0:
                continue
            f = t * K + j
            w1i = np.rint(DEC4[unpack_e2m1(d["w1"][e])] * 2).astype(np.int64)
            acc = []
            for n in range(2 * I):
                a = gemm_exact(xi[t], d["x_sf"][t], w1i[n], d["w1_sf"][e][n])
                acc.append(a)
                assert a == F(out["acc1"][f, n]), (t, j, n)
            hv = [F(oracle.swiglu(float(acc[i]), float(acc[I + i]), float(d["w"][t, j])))
                  for i in range(I)]
            q, codes = [], []
            for ib in range(I // 32):
                blk = hv[32 * ib:32 * ib + 32]
                s = _f32(max(max(abs(v) for v in blk), floor) / 448)
                k = _pow2_ceil(s)
                codes.append(127 + k)
                q += [_e4m3(v / Fraction(2) ** k) for v in blk]
            assert codes == [int(c) for c in out["h_sf"][f]], (t, j)
            got = out["h"][f].astype(np.int64)
            want = np.array(q, np.int64)
            assert np.array_equal(np.where((got & 0x7F) == 0, 0, got),
                                  np.where((want & 0x7F) == 0, 0, want)), (t, j)
            hi = np.rint(DEC8[want] * 512).astype(np.int64)
            w2i = np.rint(DEC4[unpack_e2m1(d["w2"][e])] * 2).astype(np.int64)
            for n in range(H):
                a = gemm_exact(hi, codes, w2i[n], d["w2_sf"][e][n])
                bits = _bf16_bits(a)
                assert bits == int(out["partial"][f, n]), (t, j, n)
                a_sum[n] = _f32(a_sum[n] + F(bf16_f64(np.array([bits]))[0]))
        for n in range(H):
            y_exact[t, n] = _bf16_bits(a_sum[n])
    assert np.array_equal(out["y"], y_exact)
