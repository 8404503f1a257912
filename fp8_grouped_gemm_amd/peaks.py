"""Binding of libmoe_peaks.so (include/moe_peaks.h): the streaming-read and
FP8 MFMA kernels that measure the ceilings the MoE kernels are compared to.

Argument marshalling only; raises if the library has not been built.
"""
import ctypes
import os

from . import MoEError, MOE_OK, _stream
from .build import PEAKS_LIB

MOE_PEAK_READ_PLAIN = 0
MOE_PEAK_READ_NONTEMPORAL = 1
MOE_PROBE_E4M3 = 0
MOE_PROBE_E4M3_E2M1 = 1
EXPORTED_SYMBOLS = ("moe_peak_stream_read", "moe_peak_mfma_fp8", "moe_probe_mfma_block",
                    "moe_probe_conversions")
MFMA_FLOP_PER_WAVE_ROUND = 8 * 2 * 16 * 16 * 128

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PEAKS_LIB):
            raise ImportError(f"{PEAKS_LIB} is missing: build it with "
                              "`python -m fp8_grouped_gemm_amd.build`")
        L = ctypes.CDLL(PEAKS_LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.moe_peak_stream_read.argtypes = [vp, ctypes.c_size_t, i32, i32, i32, vp, vp]
        L.moe_peak_mfma_fp8.argtypes = [i32, i32, vp, vp]
        L.moe_probe_mfma_block.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp]
        L.moe_probe_conversions.argtypes = [i32, vp, vp]
        for name in EXPORTED_SYMBOLS:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def stream_read(buf, blocks, out, unroll=8, mode=MOE_PEAK_READ_NONTEMPORAL, stream=None,
                nbytes=None):
    """Read all of `buf` (a device tensor); out: uint32-sized tensor of 4*blocks."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    rc = lib().moe_peak_stream_read(_ptr(buf), n, blocks, unroll, mode, _ptr(out),
                                    _stream(stream))
    if rc != MOE_OK:
        raise MoEError(rc, "moe_peak_stream_read")


def mfma_fp8(blocks, iters, out, stream=None):
    """Dense e4m3 MFMA loop; out: float32 tensor of 256*blocks."""
    rc = lib().moe_peak_mfma_fp8(blocks, iters, _ptr(out), _stream(stream))
    if rc != MOE_OK:
        raise MoEError(rc, "moe_peak_mfma_fp8")


def mfma_flop(blocks, iters):
    return blocks * 4 * iters * MFMA_FLOP_PER_WAVE_ROUND


def probe_mfma_block(mode, a, b, out, sa=None, sb=None, stream=None):
    """One 16x16x128 MFMA per tile (moe_probe_mfma_block); a, b, sa, sb, out
    device tensors shaped as the header documents."""
    n_tiles = a.shape[0]
    rc = lib().moe_probe_mfma_block(mode, n_tiles, _ptr(a), _ptr(b), _ptr(sa), _ptr(sb),
                                    _ptr(out), _stream(stream))
    if rc != MOE_OK:
        raise MoEError(rc, "moe_probe_mfma_block")


def probe_conversions(blocks, counts, stream=None):
    """Mismatch counts of the bf16 and e4m3 conversions over every f32
    pattern; counts: int32/uint32-sized tensor of 2 * 256 * blocks."""
    rc = lib().moe_probe_conversions(blocks, _ptr(counts), _stream(stream))
    if rc != MOE_OK:
        raise MoEError(rc, "moe_probe_conversions")
