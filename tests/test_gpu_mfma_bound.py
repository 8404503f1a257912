"""The one hardware-arithmetic constant the parity tests rely on, measured.

The oracle sums each 128-wide K block exactly (the pages' block-scaled GEMM
with its one rounding to f32).  The gfx950 matrix instruction the GEMM
kernels use does not: inside one 16x16x128 MFMA the products are accumulated
with limited precision.  The parity tests accept a difference from the
oracle only when it fits

    |MFMA result - exact block sum| <= BETA * (sum of |products| of the block)

with BETA_FP8 for e4m3 x e4m3 and BETA_MX for the block-scaled e4m3 x e2m1
form.  This test measures the left side on random and adversarial operands,
loaded exactly as the GEMM kernels load them (moe_probe_mfma_block), against
exact integer arithmetic, and holds it to those constants.
"""
import numpy as np
import pytest
import torch

from fp8_grouped_gemm_amd import peaks
from parity_util import BETA_FP8, BETA_MX, E4M3_INT, say

pytestmark = pytest.mark.gpu

# e2m1 magnitudes times 2 (integers), OCP MX element table
E2M1_INT2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def exact_fp8(a, b):
    """[n,16,128] x [n,16,128] codes -> exact sums and sums of |products| (f64)."""
    ia = E4M3_INT[a.astype(np.int64)]  # value * 2^9
    ib = E4M3_INT[b.astype(np.int64)]
    s = np.matmul(ia, ib.transpose(0, 2, 1))               # int64, < 2^43
    m = np.matmul(np.abs(ia), np.abs(ib).transpose(0, 2, 1))
    return np.ldexp(s.astype(np.float64), -18), np.ldexp(m.astype(np.float64), -18)


def exact_mx(a, b_packed, sa, sb):
    """Block-scaled e4m3 x e2m1 sums, exact in int64 then rounded once."""
    ia = E4M3_INT[a.astype(np.int64)]                        # [n,16,128] * 2^9
    bp = b_packed.astype(np.int64)
    codes = np.empty(bp.shape[:-1] + (128,), np.int64)
    codes[..., 0::2] = bp & 15
    codes[..., 1::2] = bp >> 4
    ib = E2M1_INT2[codes]                                    # [n,16,128] * 2
    n = a.shape[0]
    shift = sa.astype(np.int64)[:, :, None, :] + sb.astype(np.int64)[:, None, :, :]  # [n,16,16,4]
    lo = shift.min(-1, keepdims=True)
    s = np.zeros((n, 16, 16), np.int64)
    m = np.zeros((n, 16, 16), np.int64)
    for blk in range(4):
        ka, kb = ia[..., 32 * blk:32 * blk + 32], ib[..., 32 * blk:32 * blk + 32]
        ps = np.matmul(ka, kb.transpose(0, 2, 1))            # < 2^27
        pm = np.matmul(np.abs(ka), np.abs(kb).transpose(0, 2, 1))
        up = np.left_shift(1, shift[..., blk] - lo[..., 0])
        s += ps * up
        m += pm * up
    e = lo[..., 0] - 254 - 10
    return np.ldexp(s.astype(np.float64), e), np.ldexp(m.astype(np.float64), e)


def run_probe(mode, a, b, sa=None, sb=None):
    dev = lambda v: None if v is None else torch.from_numpy(np.ascontiguousarray(v)).cuda()
    out = torch.full((a.shape[0], 16, 16), float("nan"), dtype=torch.float32, device="cuda")
    peaks.probe_mfma_block(mode, dev(a), dev(b), out, sa=dev(sa), sb=dev(sb))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def rel_err(got, exact, mag):
    assert np.all(np.isfinite(got))
    zero = mag == 0
    assert np.all(got[zero] == 0)
    return np.abs(got - exact)[~zero] / mag[~zero]


def fp8_cases(rng, n):
    uni = lambda shape: FINITE[rng.integers(0, FINITE.size, shape)]
    yield "uniform codes", uni((n, 16, 128)), uni((n, 16, 128))
    g = lambda shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * 40) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    yield "gaussian", g((n, 16, 128)), g((n, 16, 128))
    # one dominant product per row/column pair, the rest 2^-20..2^-26 of it,
    # all positive: the small terms sit where limited precision drops them
    a = rng.integers(0x01, 0x10, (n, 16, 128)).astype(np.uint8)   # 2^-9 .. 2^-6 range
    b = rng.integers(0x30, 0x40, (n, 16, 128)).astype(np.uint8)   # 0.5 .. 1.875
    k0 = rng.integers(0, 128, n)
    a[np.arange(n), :, k0] = 0x7E                                  # 448
    b[np.arange(n), :, k0] = 0x7E
    yield "one dominant product", a, b
    # cancellation: equal and opposite halves plus a small remainder
    a = uni((n, 16, 128))
    b = uni((n, 16, 128))
    a[..., 64:] = a[..., :64] ^ 0x80
    b[..., 64:] = b[..., :64]
    a[..., 127] = rng.integers(1, 8, (n, 16)).astype(np.uint8)
    yield "cancellation", a, b


def test_mfma_e4m3_block_error_within_stated_bound():
    rng = np.random.default_rng(20261202)
    worst = 0.0
    for what, a, b in fp8_cases(rng, 512):
        say(f"mfma probe e4m3: {what}")
        got = run_probe(peaks.MOE_PROBE_E4M3, a, b)
        exact, mag = exact_fp8(a, b)
        r = rel_err(got, exact, mag)
        say(f"  max |mfma - exact| / sum|ab| = {r.max():.3e} (mean {r.mean():.3e}); "
            f"exact in {np.mean(got == exact.astype(np.float32)) * 100:.1f} % of outputs")
        worst = max(worst, float(r.max()))
    say(f"  e4m3 worst {worst:.3e} against BETA_FP8 = {BETA_FP8:.3e}")
    assert worst <= BETA_FP8


def test_mfma_e4m3_e2m1_block_error_within_stated_bound():
    rng = np.random.default_rng(20261203)
    worst = 0.0
    n = 512
    cases = []
    uni = lambda shape: FINITE[rng.integers(0, FINITE.size, shape)]
    cases.append(("uniform, scales 120..134", uni((n, 16, 128)),
                  rng.integers(0, 256, (n, 16, 64)).astype(np.uint8),
                  rng.integers(120, 135, (n, 16, 4)), rng.integers(120, 135, (n, 16, 4))))
    sa = np.full((n, 16, 4), 127)
    sb = np.full((n, 16, 4), 127)
    sa[..., 0] = 136                                   # one block far above the others
    sb[..., 0] = 134
    sa[..., 1:] = 112                                  # (spread 31: the int64 sums stay exact)
    cases.append(("block scales 2^31 apart", uni((n, 16, 128)),
                  rng.integers(0, 256, (n, 16, 64)).astype(np.uint8), sa, sb))
    for what, a, b, sa, sb in cases:
        say(f"mfma probe e4m3 x e2m1: {what}")
        got = run_probe(peaks.MOE_PROBE_E4M3_E2M1, a, b, sa.astype(np.uint8), sb.astype(np.uint8))
        exact, mag = exact_mx(a, b, sa, sb)
        r = rel_err(got, exact, mag)
        say(f"  max |mfma - exact| / sum|ab| = {r.max():.3e} (mean {r.mean():.3e})")
        worst = max(worst, float(r.max()))
    say(f"  e4m3 x e2m1 worst {worst:.3e} against BETA_MX = {BETA_MX:.3e}")
    assert worst <= BETA_MX
