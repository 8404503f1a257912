"""Shared helpers for the GPU parity tests: run the HIP path through the
C ABI and the oracle on the same seeded inputs, and compare.

The comparison (verify) follows the path step by step and accepts a
difference from the oracle only where the arithmetic explains it:

  1. plan: counts, offsets, row_src and src_row bit-exact (a separate check
     in the tests, oracle.route);
  2. h and h_sf (steps 2-4): the oracle sums every 128-wide K block exactly;
     the gfx950 MFMA accumulates inside one instruction with limited
     precision, |MFMA - exact| <= BETA * sum|products| (BETA_FP8, BETA_MX:
     measured in test_gpu_mfma_bound.py).  Carried through the f32
     promotion, the SwiGLU and the requantisation this bounds, per element,
     how far the GPU's pre-rounding quotient h/sf can be from the oracle's.
     A GPU code must be the e4m3 rounding of some value within that bound of
     the oracle's quotient (taken with the GPU's scale): the oracle's own
     code, or a neighbour when the quotient lies within the bound of a
     rounding boundary (or, for a quotient near zero, a small code of the
     other sign).  A scale must be within the bound of the
     oracle's (raw scales), or equal it (power-of-two scales) unless the
     oracle's raw scale lies within the bound of the power of two between
     them;
  3. the partials (step 5): against the oracle's L2 fed the GPU's own h and
     h_sf (oracle.moe_l2_combine), within BETA * (the L2 magnitude) plus one
     bf16 ulp (two correct roundings of values that close can straddle one
     rounding boundary);
  4. y (step 6): bit-exact against the combine of the GPU's own partials
     (f32 sum over slots in ascending order, one bf16 rounding), and within
     per-token relative L2 1e-2 of the oracle's L2 + combine fed the GPU's
     h; against the full oracle, relative L2 <= 1e-2 over the case, per token
     <= 1e-2 for every token whose h codes all equal the oracle's (a token
     with a moved code is held by the step-by-step chain instead), and exact
     zeros where the oracle's token is zero.
"""
import sys

import numpy as np
import torch

import fp8_grouped_gemm_amd as moe
import oracle
import workload as wl

Y_TOL = 1e-2   # relative L2 of y against the oracle (case and token)

# |one 16x16x128 MFMA - the exact sum of its products| / sum |products|,
# held by test_gpu_mfma_bound.py (measured maxima: 2.05e-4 for e4m3 x e4m3 on
# codes drawn uniformly from all finite values, 2.5e-4 for e4m3 x e2m1 with
# block scales 2^31 apart)
BETA_FP8 = 2.0 ** -11    # e4m3 x e4m3
BETA_MX = 2.0 ** -10     # e4m3 x e2m1 with UE8M0 block scales


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _e4m3_closed(c):
    """OCP E4M3FN value of code c (closed form)."""
    s = -1.0 if c & 0x80 else 1.0
    E, M = (c >> 3) & 0xF, c & 0x7
    if E == 0xF and M == 0x7:
        return float("nan")
    return s * ((M / 8.0) * 2.0 ** -6 if E == 0 else (1.0 + M / 8.0) * 2.0 ** (E - 7))


DEC = np.array([_e4m3_closed(c) for c in range(256)])
# value * 2^9 as an integer (every finite e4m3 value is a multiple of 2^-9)
E4M3_INT = np.array([0 if np.isnan(v) else int(round(v * 512)) for v in DEC], np.int64)
# position on the value line: codes c and c' are neighbours iff |ORD| differ by 1
ORD = np.array([(c & 0x7F) * (-1 if c & 0x80 else 1) for c in range(256)], np.int64)


def bf16_to_f64(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(v):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def e4m3_codes(q):
    """torch's e4m3 cast (RNE) of f32 values already within +-448."""
    t = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def per_token_rel_l2(y_gpu_bits, y_ref_bits):
    a = bf16_to_f64(y_gpu_bits)
    b = bf16_to_f64(y_ref_bits)
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    zero = den == 0
    rel = np.where(zero, 0.0, num / np.where(zero, 1.0, den))
    return rel, zero, a, b


def check_y(y_gpu_bits, y_ref_bits, what="", strict_tokens=None):
    """y against the full oracle: relative L2 <= Y_TOL over the case; per
    token <= Y_TOL on strict_tokens (a boolean mask; default all tokens);
    tokens with a zero reference exactly zero."""
    rel, zero, a, b = per_token_rel_l2(y_gpu_bits, y_ref_bits)
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    assert np.all(a[zero] == 0), f"{what}: token with zero reference is not zero"
    if strict_tokens is None:
        strict_tokens = np.ones(rel.shape, bool)
    glob = float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
    worst = float(rel.max()) if rel.size else 0.0
    worst_strict = float(rel[strict_tokens].max()) if strict_tokens.any() else 0.0
    say(f"  {what}: y vs oracle rel L2 {glob:.3e}; per token max {worst:.3e} "
        f"({int(strict_tokens.sum())} tokens with the oracle's codes: max {worst_strict:.3e})")
    assert glob <= Y_TOL, f"{what}: rel L2 {glob} > {Y_TOL}"
    assert worst_strict <= Y_TOL, f"{what}: per-token rel L2 {worst_strict} > {Y_TOL}"
    return glob


# ----------------------------------------------------------- the chain check


def _silu(g):
    return g * 0.5 * (1.0 + np.tanh(0.5 * g))  # g * sigmoid(g), no overflow


def _h_bound(ref, w_slots, I, nkb, beta, clamp):
    """Per element of h: a bound on |GPU - oracle| of the SwiGLU output."""
    acc, mag = ref["acc1"].astype(np.float64), ref["acc1_mag"].astype(np.float64)
    # f32 promotion over nkb blocks (+ up to 4 split-K slices) on both sides
    dacc = (beta + (nkb + 4) * 2.0 ** -23) * mag
    g, u = acc[:, :I], acc[:, I:]
    dg, du = dacc[:, :I], dacc[:, I:]
    if clamp > 0:  # clamping is 1-Lipschitz
        g, u = np.clip(g, -clamp, clamp), np.clip(u, -clamp, clamp)
    sg = _silu(g)
    w = np.abs(w_slots.astype(np.float64))[:, None]
    hv = np.abs(ref["hval"].astype(np.float64))
    # |silu'| <= 1.1; the GPU's SiLU (hardware exp2 and reciprocal) is within
    # 2^-18 relative of the oracle's; a few f32 roundings on either side
    return w * (1.1 * np.abs(u) * dg + (np.abs(sg) + 1.1 * dg) * du
                + 2.0 ** -18 * np.abs(sg * u)) + 2.0 ** -20 * hv + 1e-38


def _check_scales(sf_g, sf_o, amax_o, damax, pow2, what):
    """sf_g, sf_o: [m, nb] scale values (f64)."""
    if not pow2:
        ok = np.abs(sf_g - sf_o) <= damax / 448.0 * 1.0001 + 2.0 ** -22 * sf_o
        assert ok.all(), f"{what}: {int((~ok).sum())} h scales outside the bound"
        return 0
    s = np.maximum(amax_o, 1e-10) / 448.0
    same = sf_g == sf_o
    up = (sf_g == 2 * sf_o) & (sf_o - s <= damax / 448.0 * 1.0001)
    down = (sf_g == sf_o / 2) & (s - sf_o / 2 <= damax / 448.0 * 1.0001)
    ok = same | up | down
    assert ok.all(), f"{what}: {int((~ok).sum())} power-of-two h scales not explained"
    return int((~same).sum())


def _check_codes(h_g, sf_g_el, hval, dh, what):
    """h_g [m, I] GPU codes; sf_g_el [m, I] the GPU's scale per element.  A
    code is accepted when it is the e4m3 rounding of some value within the
    bound of the oracle's quotient: rounding is monotone, so those codes are
    the ones between the roundings of the bound's two ends (which is the
    oracle's own code, or a neighbour -- or, for a quotient near zero, the
    small codes of either sign)."""
    q = (hval.astype(np.float32) / sf_g_el.astype(np.float32)).astype(np.float32)
    q = np.clip(q, -448.0, 448.0)
    c_ref = e4m3_codes(q)
    o_g, o_ref = ORD[h_g.astype(np.int64)], ORD[c_ref.astype(np.int64)]
    moved = o_g != o_ref
    n_moved = int(moved.sum())
    if n_moved:
        qv = q[moved].astype(np.float64)
        tau = 2.0 * dh[moved] / sf_g_el[moved] + 2.0 ** -20 * np.abs(qv) + 1e-30
        lo = ORD[e4m3_codes(np.clip(qv - tau, -448.0, 448.0)).astype(np.int64)]
        hi = ORD[e4m3_codes(np.clip(qv + tau, -448.0, 448.0)).astype(np.int64)]
        og = o_g[moved]
        inside = (og >= lo) & (og <= hi)
        if not inside.all():
            k = np.nonzero(~inside)[0][:5]
            ex = [(float(qv[i]), float(tau[i]), int(h_g[moved][i]), int(c_ref[moved][i]))
                  for i in k]
            raise AssertionError(f"{what}: {int((~inside).sum())} of {n_moved} moved h codes are "
                                 f"not a rounding of any value within the MFMA bound of the "
                                 f"oracle's quotient; (q, bound, gpu code, oracle code): {ex}")
    return moved


def verify(y, runner, host, what, tokens=None, oflags=0, clamp=0.0, check_y_full=True):
    """The chain check above for one forward (y: device bf16 [T,H] written by
    runner).  host: the oracle's inputs (x, x_sf, idx, w, per-expert w1,
    w1_sf, w2, w2_sf; experts no listed token uses may be None).  tokens:
    the tokens to check (default all).  Returns a dict of statistics."""
    mx = runner.recipe == moe.MOE_RECIPE_MXFP4
    H, I, E, K = runner.shape[:4]
    T = y.shape[0]
    toks = list(range(T)) if tokens is None else list(tokens)
    n = len(toks)
    info = moe.moe_plan_info(runner.plan, T)
    G = 32 if mx else info["act_sf_gran"]
    pow2 = mx or bool(oflags & oracle.ORC_POW2_SCALE)
    beta = BETA_MX if mx else BETA_FP8
    fwd = oracle.moe_forward_mx if mx else oracle.moe_forward
    ref = fwd(host["x"], host["x_sf"], host["idx"], host["w"], host["w1"], host["w1_sf"],
              host["w2"], host["w2_sf"], tokens=toks, flags=oflags, clamp=clamp,
              want=("acc1", "acc1_mag", "hval", "h"))
    idx = np.asarray(host["idx"])
    slots = np.array([t * K + j for t in toks for j in range(K)], np.int64)
    ids = idx.reshape(-1)[slots]
    valid = (ids >= 0) & (ids < E)
    src_row = runner.view("src_row", T).cpu().numpy()[slots]
    assert np.all(src_row[valid] >= 0) and np.all(src_row[~valid] < 0), what
    rows = src_row[valid]
    h_all = runner.view("h", T).cpu().numpy()
    sf_all = runner.view("h_sf", T).cpu().numpy()
    m = int(valid.sum())
    h_g = np.zeros((n * K, I), np.uint8)
    sf_g = np.zeros((n * K, I // G), sf_all.dtype)
    h_g[valid] = h_all[rows]
    sf_g[valid] = sf_all[rows]

    # ---- step 2-4: h and its scales
    w_slots = np.asarray(host["w"]).reshape(-1)[slots]
    dh = _h_bound({k: ref[k][valid] for k in ("acc1", "acc1_mag", "hval")}, w_slots[valid], I,
                  H // 128, beta, clamp)
    hv = ref["hval"][valid]
    to_val = (lambda c: np.ldexp(1.0, c.astype(np.int64) - 127)) if mx else \
        (lambda s: s.astype(np.float64))
    sfg_v, sfo_v = to_val(sf_g[valid]), to_val(ref["h_sf"][valid])
    nb = I // G
    amax_o = np.abs(hv.astype(np.float64)).reshape(m, nb, G).max(-1)
    damax = dh.reshape(m, nb, G).max(-1)
    moved_sf = _check_scales(sfg_v, sfo_v, amax_o, damax, pow2, what)
    moved = _check_codes(h_g[valid], np.repeat(sfg_v, G, axis=1), hv, dh, what)
    # slots with a code unlike the oracle's own (from a moved rounding or a
    # moved scale; a scale that moved without changing a code changes y by
    # no more than its own bound, checked above)
    differs = (ORD[h_g[valid].astype(np.int64)] != ORD[ref["h"][valid].astype(np.int64)]).any(1)
    moved_slot = np.zeros(n * K, bool)
    moved_slot[np.nonzero(valid)[0]] = differs
    moved_tok = moved_slot.reshape(n, K).any(1)

    # ---- step 5: partials against the oracle's L2 fed the GPU's h
    if mx:
        l2 = oracle.moe_l2_combine_mx(idx, host["w2"], host["w2_sf"], h_g, sf_g, tokens=toks,
                                      want=("partial", "o_mag"))
    else:
        l2 = oracle.moe_l2_combine(idx, host["w2"], host["w2_sf"], h_g, sf_g, tokens=toks,
                                   flags=oflags & oracle.ORC_SF_GRAN64, want=("partial", "o_mag"))
    part = runner.view("partial", T).cpu().numpy().astype(np.uint16)   # [K, T, H]
    tt, jj = slots // K, slots % K
    p_g = np.zeros((n * K, H), np.uint16)
    p_g[valid] = part[jj[valid], tt[valid]]
    a, b = bf16_to_f64(p_g[valid]), bf16_to_f64(l2["partial"][valid])
    nkb2 = (I // 128) * (2 if G == 64 else 1)
    # the two f32 values differ by at most the MFMA bound; their bf16
    # roundings by that plus one bf16 ulp (8 significant bits) of the larger
    _, ex = np.frexp(np.maximum(np.abs(a), np.abs(b)))
    dp = (beta + (nkb2 + 2) * 2.0 ** -23) * l2["o_mag"][valid].astype(np.float64) + \
        np.ldexp(1.0, ex - 8) + 1e-38
    bad = np.abs(a - b) > dp
    assert not bad.any(), (f"{what}: {int(bad.sum())} partial values outside the L2 bound "
                           f"(worst {float((np.abs(a - b) / dp).max()):.2f} x bound)")

    # ---- step 6: y is the combine of the GPU's own partials, bit for bit
    yg = y.cpu().numpy().astype(np.uint16)[toks]
    acc = np.zeros((n, H), np.float32)
    pf = bf16_to_f64(p_g).astype(np.float32).reshape(n, K, H)
    vm = valid.reshape(n, K)
    for j in range(K):
        acc = np.where(vm[:, j:j + 1], (acc + pf[:, j]).astype(np.float32), acc)
    assert np.array_equal(yg, f32_to_bf16_bits(acc)), f"{what}: y is not the combine of its partials"
    rel2, _, _, _ = per_token_rel_l2(yg, l2["y"])
    say(f"  {what}: {m} routed slots; h codes moved {int(moved.sum())}/{m * I}, "
        f"h scales moved {moved_sf}, {int(moved_tok.sum())}/{n} tokens with a code unlike "
        f"the oracle's; "
        f"y vs oracle L2 fed the GPU's h: per token max {float(rel2.max()):.3e}")
    assert float(rel2.max()) <= Y_TOL, f"{what}: y vs oracle L2 on the GPU's h {rel2.max()}"
    stats = dict(slots=m, moved=int(moved.sum()), moved_tokens=int(moved_tok.sum()),
                 y_l2_fed=float(rel2.max()))
    if check_y_full:
        stats["y_full"] = check_y(yg, ref["y"], what=what, strict_tokens=~moved_tok)
    return stats


# ------------------------------------------------------------ running cases


def gpu_inputs(cfg, seed, device="cuda"):
    """Seeded inputs drawn directly on the device (large workloads)."""
    return wl.make_inputs(cfg, seed, device)


def host_copy_for_oracle(inp, tokens):
    """Move what the oracle needs for `tokens` to the host: token data plus the
    weights of the experts those tokens use (others stay None)."""
    E = inp["w1"].shape[0]
    idx = inp["topk_idx"].cpu().numpy()
    need = sorted({int(e) for e in idx[tokens].reshape(-1) if 0 <= e < E})
    sel = lambda t: [t[e].cpu().numpy() if e in need else None for e in range(E)]
    return dict(x=inp["x"].cpu().numpy(), x_sf=inp["x_sf"].cpu().numpy(), idx=idx,
                w=inp["topk_w"].cpu().numpy(), w1=sel(inp["w1"]), w1_sf=sel(inp["w1_sf"]),
                w2=sel(inp["w2"]), w2_sf=sel(inp["w2_sf"]))


def run_oracle(h, tokens=None, want=()):
    return oracle.moe_forward(h["x"], h["x_sf"], h["idx"], h["w"], h["w1"], h["w1_sf"],
                              h["w2"], h["w2_sf"], tokens=tokens, want=want)


def run_gpu(inp, tile_m=0, max_tokens=None, runner=None, weight_layout=0, flags=0):
    T, H = inp["x"].shape
    E, twoI, _ = inp["w1"].shape
    K = inp["topk_idx"].shape[1]
    if runner is None:
        runner = moe.MoEForward(H, twoI // 2, E, K, max_tokens or T, tile_m=tile_m,
                                weight_layout=weight_layout, flags=flags)
    w1, w2 = runner.prepare(inp["w1"], inp["w2"])
    y = runner.forward(inp["x"], inp["x_sf"], inp["topk_idx"], inp["topk_w"], w1,
                       inp["w1_sf"], w2, inp["w2_sf"])
    torch.cuda.synchronize()
    return y, runner


def cpu_inputs_to_gpu(inp):
    return {k: v.cuda() for k, v in inp.items()}


def host_dict(inp):
    E = inp["w1"].shape[0]
    return dict(x=inp["x"].numpy(), x_sf=inp["x_sf"].numpy(), idx=inp["topk_idx"].numpy(),
                w=inp["topk_w"].numpy(),
                w1=[inp["w1"][e].numpy() for e in range(E)],
                w1_sf=[inp["w1_sf"][e].numpy() for e in range(E)],
                w2=[inp["w2"][e].numpy() for e in range(E)],
                w2_sf=[inp["w2_sf"][e].numpy() for e in range(E)])


def small_case(T, H, I, E, K, seed, mask=None, skew=False):
    """Inputs drawn on the CPU (oracle runs on all tokens); returns (host
    numpy dict for the oracle, device tensor dict for the HIP path)."""
    cfg = wl.custom_config(T, H, I, E, K, skew)
    inp = wl.make_inputs(cfg, seed, "cpu")
    if mask:
        idx = inp["topk_idx"].clone()
        for (t, j), v in mask.items():
            idx[t, j] = v
        inp["topk_idx"] = idx
    return host_dict(inp), cpu_inputs_to_gpu(inp)
