"""The ceiling-measurement kernels (libmoe_peaks.so) compute what they claim:
the streaming read touches every 32-bit word of the buffer exactly once (the
XOR of its per-wave results equals the XOR of all words, for every load
mode, unroll and grid, including sizes with a partial final round), and the
FP8 MFMA loop runs exactly the instructions its FLOP count assumes (each
lane's result is exactly 8 * 4 * 64 * iters).  The conversion probe pins the
two conversions the epilogues use to their integer definitions on every
f32 bit pattern."""
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


def test_conversions_match_their_definitions_on_every_f32():
    # f32 -> bf16 (hardware) against round to nearest even on the bits, and
    # the hardware f32 -> e4m3 against the integer encoder: 2^32 patterns
    blocks = 4096
    say(f"conversion probe: every f32 pattern over {blocks} workgroups")
    counts = torch.full((2 * 256 * blocks,), -1, dtype=torch.int32, device="cuda")
    peaks.probe_conversions(blocks, counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy().astype(np.int64).reshape(2, -1)
    assert c[0].sum() == 0, f"bf16: {c[0].sum()} patterns differ"
    assert c[1].sum() == 0, f"e4m3: {c[1].sum()} patterns differ"
