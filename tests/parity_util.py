"""Shared helpers for the GPU parity tests: run the HIP path through the
C ABI and the oracle on the same seeded inputs, and compare."""
import sys

import numpy as np
import torch

import fp8_grouped_gemm_amd as moe
import oracle
from fp8_grouped_gemm_amd import workload as wl

# Parity bar for y: relative L2 error of y against the oracle <= 1e-2 for
# every case; tokens whose oracle output is exactly zero must be exactly zero.
# Per-token relative L2 is reported and held to PER_TOKEN_TOL.
Y_TOL = 1e-2
PER_TOKEN_TOL = 5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_f64(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def per_token_rel_l2(y_gpu_bits, y_ref_bits):
    a = bf16_to_f64(y_gpu_bits)
    b = bf16_to_f64(y_ref_bits)
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    zero = den == 0
    rel = np.where(zero, 0.0, num / np.where(zero, 1.0, den))
    return rel, zero, a, b


def check_y(y_gpu_bits, y_ref_bits, tol=Y_TOL, per_token_tol=PER_TOKEN_TOL, what=""):
    rel, zero, a, b = per_token_rel_l2(y_gpu_bits, y_ref_bits)
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    assert np.all(a[zero] == 0), f"{what}: token with zero reference is not zero"
    worst = float(rel.max()) if rel.size else 0.0
    glob = float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
    n_over = int((rel > 1e-2).sum())
    say(f"  {what}: rel L2 {glob:.3e}; per token max {worst:.3e}, median "
        f"{float(np.median(rel)) if rel.size else 0:.3e}, {n_over}/{rel.size} tokens > 1e-2")
    assert glob <= tol, f"{what}: rel L2 {glob} > {tol}"
    assert worst <= per_token_tol, f"{what}: per-token rel L2 {worst} > {per_token_tol}"
    return glob


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
    host = dict(x=inp["x"].numpy(), x_sf=inp["x_sf"].numpy(), idx=inp["topk_idx"].numpy(),
                w=inp["topk_w"].numpy(),
                w1=[inp["w1"][e].numpy() for e in range(E)],
                w1_sf=[inp["w1_sf"][e].numpy() for e in range(E)],
                w2=[inp["w2"][e].numpy() for e in range(E)],
                w2_sf=[inp["w2_sf"][e].numpy() for e in range(E)])
    return host, cpu_inputs_to_gpu(inp)
