"""Seeded synthetic inputs for the FP8 MoE expert forward.

This module only draws inputs.  It holds none of the forward's arithmetic:
the FP8 quantisation of the inputs uses torch's own float8_e4m3fn cast, and
both the CPU oracle and the HIP path consume exactly the bytes it returns.

Recipe (one per workload, all synthetic, standing in for the model shapes
the DeepGEMM MegaMoE pages benchmark: DeepSeek "Flash" 4096/2048/256/top-6,
"Pro" 7168/3072/384/top-6, a skewed-routing stress, and one GPU's expert
share of the flash layer under 8-way expert parallelism):
  x        f32 N(0,1) [T,H], quantised per 1x128 block
  W1[e]    f32 N(0, 1/sqrt(H)) [2I,H] (gate rows, then up rows), per 128x128
  W2[e]    f32 N(0, 1/sqrt(I)) [H,I], per 128x128
  block quantisation: sf = max(amax, 1e-10)/448, q = e4m3(clamp(v/sf, +-448))
  router   logits N(0,1) [T,E]; the skewed workload adds a Zipf(1.2)-ranked
           bias -1.2*ln(rank_e) with rank_e = 1 + (a seeded permutation)[e];
           top-K by logit (ties: lower expert id first), topk_w = softmax over
           the K selected logits.
Every tensor comes from its own torch.Generator seeded from (seed, tag,
expert), so any expert's weights can be redrawn alone.

The FP8 x MXFP4 inputs (make_inputs_mx) quantise the same f32 draws with
one power-of-two (UE8M0) scale per 1x32 block: x to e4m3 with
sf = 2^ceil(log2(max(amax, 1e-10)/448)), weights to e2m1 (round to nearest,
ties to the even code) with sf = 2^ceil(log2(max(amax, 1e-10)/6)), packed
two per byte with the even element in the low nibble.
"""
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    K: int
    skew: bool = False

    @property
    def flops(self) -> float:
        """Algorithmic FLOP if every slot is active: 2*(T*K)*3*H*I."""
        return 2.0 * self.T * self.K * 3.0 * self.H * self.I


CONFIGS = {
    "tiny": MoEConfig("tiny", 64, 256, 128, 8, 2),
    "flash_decode": MoEConfig("flash_decode", 128, 4096, 2048, 256, 6),
    "flash_prefill": MoEConfig("flash_prefill", 2048, 4096, 2048, 256, 6),
    "pro_prefill": MoEConfig("pro_prefill", 8192, 7168, 3072, 384, 6),
    "skewed": MoEConfig("skewed", 4096, 4096, 2048, 256, 8, skew=True),
    # one GPU's share of the flash layer under 8-way expert parallelism at
    # 128 tokens per rank: 32 resident experts receiving 768 routed rows
    # (~24 per expert, 805 MB of FP8 weights)
    "flash_decode_ep8": MoEConfig("flash_decode_ep8", 128, 4096, 2048, 32, 6),
}

TAG_LOGITS, TAG_X, TAG_W1, TAG_W2, TAG_PERM = 0, 1, 2, 3, 4


def default_seed(cfg: MoEConfig) -> int:
    return 20261202 + list(CONFIGS).index(cfg.name) + 1 if cfg.name in CONFIGS else 20261202


def _gen(device, seed: int, tag: int, e: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + tag * 7919 + e * 104729) % (2 ** 63))
    return g


def quantize_blocks(v: torch.Tensor, br: int, bc: int):
    """Quantise a 2-D f32 tensor in br x bc blocks to e4m3 codes + f32 scales."""
    R, C = v.shape
    assert R % br == 0 and C % bc == 0
    blk = v.reshape(R // br, br, C // bc, bc)
    amax = blk.abs().amax(dim=(1, 3))
    sf = torch.clamp(amax, min=1e-10) / 448.0
    q = torch.clamp(blk / sf[:, None, :, None], -448.0, 448.0)
    q = q.reshape(R, C).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.contiguous(), sf.to(torch.float32).contiguous()


_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)  # midpoints of 0,.5,1,1.5,2,3,4,6


def _pow2_ceil_code(s: torch.Tensor) -> torch.Tensor:
    """UE8M0 code (int32) of the smallest power of two >= s, for s > 0."""
    m, e = torch.frexp(s)  # s = m * 2^e, 0.5 <= m < 1
    return torch.where(m == 0.5, e - 1, e).to(torch.int32) + 127


def quantize_mx_e4m3(v: torch.Tensor):
    """[R,C] f32 -> e4m3 codes [R,C] u8 + UE8M0 scale codes [R,C/32] u8."""
    R, C = v.shape
    blk = v.reshape(R, C // 32, 32)
    code = _pow2_ceil_code(torch.clamp(blk.abs().amax(-1), min=1e-10) / 448.0)
    sf = torch.ldexp(torch.ones_like(blk[..., 0]), code - 127)
    q = torch.clamp(blk / sf[..., None], -448.0, 448.0).reshape(R, C)
    return (q.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(),
            code.to(torch.uint8).contiguous())


def quantize_mx_e2m1(v: torch.Tensor):
    """[R,C] f32 -> packed e2m1 [R,C/2] u8 + UE8M0 scale codes [R,C/32] u8."""
    R, C = v.shape
    blk = v.reshape(R, C // 32, 32)
    code = _pow2_ceil_code(torch.clamp(blk.abs().amax(-1), min=1e-10) / 6.0)
    sf = torch.ldexp(torch.ones_like(blk[..., 0]), code - 127)
    a = (blk / sf[..., None]).reshape(R, C)
    mag = a.abs().clamp(max=6.0)
    mid = torch.tensor(_E2M1_MID, dtype=a.dtype, device=a.device)
    lo = torch.bucketize(mag, mid)  # number of midpoints below mag
    tie = (lo < 7) & (mag == mid[lo.clamp(max=6)]) & (lo % 2 == 1)
    c4 = (lo + tie.to(lo.dtype)) | ((a < 0).to(lo.dtype) << 3)
    packed = (c4[:, 0::2] | (c4[:, 1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), code.to(torch.uint8).contiguous()


def make_routing(cfg: MoEConfig, seed: int, device="cpu"):
    g = _gen(device, seed, TAG_LOGITS)
    logits = torch.randn(cfg.T, cfg.E, generator=g, device=device, dtype=torch.float32)
    if cfg.skew:
        gp = _gen(device, seed, TAG_PERM)
        rank = 1 + torch.randperm(cfg.E, generator=gp, device=device)
        logits = logits + (-1.2 * torch.log(rank.to(torch.float32)))[None, :]
    order = torch.sort(logits, dim=1, descending=True, stable=True)
    idx = order.indices[:, :cfg.K].to(torch.int32).contiguous()
    sel = order.values[:, :cfg.K]
    w = torch.softmax(sel, dim=1).to(torch.float32).contiguous()
    return idx, w


def make_x(cfg: MoEConfig, seed: int, device="cpu"):
    g = _gen(device, seed, TAG_X)
    x = torch.randn(cfg.T, cfg.H, generator=g, device=device, dtype=torch.float32)
    return quantize_blocks(x, 1, 128)


def make_expert(cfg: MoEConfig, seed: int, e: int, device="cpu"):
    """(w1 [2I,H] u8, w1_sf [2I/128,H/128], w2 [H,I] u8, w2_sf [H/128,I/128])."""
    g1 = _gen(device, seed, TAG_W1, e)
    w1 = torch.randn(2 * cfg.I, cfg.H, generator=g1, device=device,
                     dtype=torch.float32) * (1.0 / cfg.H ** 0.5)
    q1, s1 = quantize_blocks(w1, 128, 128)
    del w1
    g2 = _gen(device, seed, TAG_W2, e)
    w2 = torch.randn(cfg.H, cfg.I, generator=g2, device=device,
                     dtype=torch.float32) * (1.0 / cfg.I ** 0.5)
    q2, s2 = quantize_blocks(w2, 128, 128)
    return q1, s1, q2, s2


def make_weights(cfg: MoEConfig, seed: int, device="cpu"):
    """All experts stacked: w1 [E,2I,H] u8, w1_sf, w2 [E,H,I] u8, w2_sf."""
    E, H, I = cfg.E, cfg.H, cfg.I
    w1 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device=device)
    w1_sf = torch.empty(E, 2 * I // 128, H // 128, dtype=torch.float32, device=device)
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device=device)
    w2_sf = torch.empty(E, H // 128, I // 128, dtype=torch.float32, device=device)
    for e in range(E):
        q1, s1, q2, s2 = make_expert(cfg, seed, e, device)
        w1[e].copy_(q1)
        w1_sf[e].copy_(s1)
        w2[e].copy_(q2)
        w2_sf[e].copy_(s2)
    return w1, w1_sf, w2, w2_sf


def make_inputs(cfg: MoEConfig, seed: int, device="cpu"):
    x, x_sf = make_x(cfg, seed, device)
    idx, w = make_routing(cfg, seed, device)
    w1, w1_sf, w2, w2_sf = make_weights(cfg, seed, device)
    return dict(x=x, x_sf=x_sf, topk_idx=idx, topk_w=w, w1=w1, w1_sf=w1_sf,
                w2=w2, w2_sf=w2_sf)


def make_x_mx(cfg: MoEConfig, seed: int, device="cpu"):
    g = _gen(device, seed, TAG_X)
    x = torch.randn(cfg.T, cfg.H, generator=g, device=device, dtype=torch.float32)
    return quantize_mx_e4m3(x)


def make_expert_mx(cfg: MoEConfig, seed: int, e: int, device="cpu"):
    """(w1 [2I,H/2] u8, w1_sf [2I,H/32] u8, w2 [H,I/2] u8, w2_sf [H,I/32] u8)."""
    g1 = _gen(device, seed, TAG_W1, e)
    w1 = torch.randn(2 * cfg.I, cfg.H, generator=g1, device=device,
                     dtype=torch.float32) * (1.0 / cfg.H ** 0.5)
    q1, s1 = quantize_mx_e2m1(w1)
    del w1
    g2 = _gen(device, seed, TAG_W2, e)
    w2 = torch.randn(cfg.H, cfg.I, generator=g2, device=device,
                     dtype=torch.float32) * (1.0 / cfg.I ** 0.5)
    q2, s2 = quantize_mx_e2m1(w2)
    return q1, s1, q2, s2


def make_weights_mx(cfg: MoEConfig, seed: int, device="cpu"):
    """All experts stacked: w1 [E,2I,H/2], w1_sf [E,2I,H/32], w2 [E,H,I/2], w2_sf [E,H,I/32]."""
    E, H, I = cfg.E, cfg.H, cfg.I
    w1 = torch.empty(E, 2 * I, H // 2, dtype=torch.uint8, device=device)
    w1_sf = torch.empty(E, 2 * I, H // 32, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I // 2, dtype=torch.uint8, device=device)
    w2_sf = torch.empty(E, H, I // 32, dtype=torch.uint8, device=device)
    for e in range(E):
        q1, s1, q2, s2 = make_expert_mx(cfg, seed, e, device)
        w1[e].copy_(q1)
        w1_sf[e].copy_(s1)
        w2[e].copy_(q2)
        w2_sf[e].copy_(s2)
    return w1, w1_sf, w2, w2_sf


def make_inputs_mx(cfg: MoEConfig, seed: int, device="cpu"):
    x, x_sf = make_x_mx(cfg, seed, device)
    idx, w = make_routing(cfg, seed, device)
    w1, w1_sf, w2, w2_sf = make_weights_mx(cfg, seed, device)
    return dict(x=x, x_sf=x_sf, topk_idx=idx, topk_w=w, w1=w1, w1_sf=w1_sf,
                w2=w2, w2_sf=w2_sf)


def custom_config(T, H, I, E, K, skew=False, name="custom") -> MoEConfig:
    return MoEConfig(name, T, H, I, E, K, skew)
