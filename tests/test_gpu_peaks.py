"""The ceiling-measurement kernels (libmoe_peaks.so) compute what they claim:
the streaming read touches every 32-bit word of the buffer exactly once (the
XOR of its per-wave results equals the XOR of all words, for every load
mode, unroll and grid, including sizes with a partial final round), and the
FP8 MFMA loop runs exactly the instructions its FLOP count assumes (each
lane's result is exactly 8 * 4 * 64 * iters)."""
import numpy as np
import pytest
import torch

from fp8_grouped_gemm_amd import peaks
from parity_util import say

pytestmark = pytest.mark.gpu


def xor_words(t):
    return int(np.bitwise_xor.reduce(t.cpu().numpy().view(np.uint32)))


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (64 << 20) + 48])
def test_stream_read_touches_every_word_once(nbytes):
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    want = xor_words(buf)
    for mode in (peaks.MOE_PEAK_READ_PLAIN, peaks.MOE_PEAK_READ_NONTEMPORAL):
        for unroll in (4, 8):
            for blocks in (1, 7, 300):
                say(f"stream read: {nbytes} B, mode {mode}, unroll {unroll}, {blocks} blocks")
                out = torch.full((4 * blocks,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
                peaks.stream_read(buf, blocks, out, unroll=unroll, mode=mode)
                torch.cuda.synchronize()
                assert xor_words(out) == want, (mode, unroll, blocks)


def test_mfma_loop_counts_every_instruction():
    for blocks, iters in ((1, 1), (3, 5), (64, 2048)):
        say(f"mfma loop: {blocks} blocks x {iters} rounds")
        out = torch.full((256 * blocks,), -1.0, dtype=torch.float32, device="cuda")
        peaks.mfma_fp8(blocks, iters, out)
        torch.cuda.synchronize()
        assert torch.all(out == float(8 * 4 * 64 * iters)), (blocks, iters)
