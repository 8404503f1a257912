"""GPU: a forward captured in a HIP graph and replayed.  The library records
only kernel launches inside a forward (no allocation, memset or copy), so a
replay must give exactly the eager result for whatever the input buffers
hold at replay time.  Several replays, with eager forwards of other inputs
on the same plan and workspace between them, are each compared bitwise."""
import pytest
import torch

import fp8_grouped_gemm_amd as moe
import workload as wl
from parity_util import say

pytestmark = pytest.mark.gpu


def _tokens(cfg, seed):
    """Activations and routing of another seed (the weights stay shared)."""
    x, x_sf = wl.make_x(cfg, seed, "cuda")
    idx, w = wl.make_routing(cfg, seed, "cuda")
    return dict(x=x, x_sf=x_sf, topk_idx=idx, topk_w=w)


# 16-row direct tiles with split-K (1 and 3 tokens), without (128), the
# 64-row shared-A tile (2048) and the 160-row LDS tile (5461: 128 rows per
# expert)
@pytest.mark.parametrize("name,T", [("flash_decode", 1), ("flash_decode", 3), ("flash_decode", 128),
                                    ("flash_prefill", 2048), ("flash_prefill", 5461)])
def test_graph_replay_matches_eager_bitwise(name, T):
    base = wl.CONFIGS[name]
    cfg = wl.custom_config(T, base.H, base.I, base.E, base.K, base.skew)
    say(f"graph replay {name} T={T}")
    a = wl.make_inputs(cfg, 101, "cuda")
    b = _tokens(cfg, 202)
    r = moe.MoEForward(cfg.H, cfg.I, cfg.E, cfg.K, T, weight_layout=moe.MOE_WEIGHTS_PACKED)
    w1, w2 = r.prepare(a["w1"], a["w2"])  # the weights stay those of input set a
    stream = torch.cuda.current_stream()

    def eager(inp, y):
        moe.moe_forward(r.plan, T, inp["x"], inp["x_sf"], inp["topk_idx"], inp["topk_w"], w1,
                        a["w1_sf"], w2, a["w2_sf"], y, r.workspace, stream=stream)

    # the buffers the graph reads and writes
    x, x_sf = a["x"].clone(), a["x_sf"].clone()
    idx, tw = a["topk_idx"].clone(), a["topk_w"].clone()
    y_g = torch.empty(T, cfg.H, dtype=torch.uint16, device="cuda")
    y_a = torch.empty_like(y_g)
    y_b = torch.empty_like(y_g)
    eager(a, y_a)
    eager(b, y_b)
    torch.cuda.synchronize()
    assert not torch.equal(y_a, y_b)

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(g, stream=cap):
        moe.moe_forward(r.plan, T, x, x_sf, idx, tw, w1, a["w1_sf"], w2, a["w2_sf"], y_g,
                        r.workspace, stream=cap)
    torch.cuda.synchronize()
    for rep in range(3):
        y_g.fill_(0x7FC0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_a), (name, T, rep)
        # eager work on the same plan and workspace between replays
        y_e = torch.empty_like(y_g)
        eager(b, y_e)
        torch.cuda.synchronize()
        assert torch.equal(y_e, y_b), (name, T, rep)
    # the graph reads the buffers' contents at replay time
    x.copy_(b["x"])
    x_sf.copy_(b["x_sf"])
    idx.copy_(b["topk_idx"])
    tw.copy_(b["topk_w"])
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_b), (name, T, "inputs b", rep)
    del g
    r.close()
