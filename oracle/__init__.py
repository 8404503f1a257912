"""ctypes wrapper of the CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, the smoke entry and the benchmark's
CPU-baseline leg may import this module; the product package never does,
and this module imports nothing from the product package.  All arrays are
numpy arrays on the host.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

ORC_NO_REQUANT = 1
ORC_NO_BF16 = 2
ORC_POW2_SCALE = 4
ORC_SF_GRAN64 = 8

_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_e4m3_decode.restype = ctypes.c_float
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_route.restype = ctypes.c_int
        L.orc_route.argtypes = [ctypes.c_int] * 4 + [_i32p, _i32p, _i32p, _i32p,
                                                     ctypes.c_int, _i32p]
        L.orc_block_dot_e4m3.restype = ctypes.c_double
        L.orc_block_dot_e4m3.argtypes = [_u8p, _u8p, ctypes.c_int]
        L.orc_swiglu.restype = ctypes.c_float
        L.orc_swiglu.argtypes = [ctypes.c_float] * 3
        L.orc_requant_block.restype = None
        L.orc_requant_block.argtypes = [_f32p, ctypes.c_int, _u8p, _f32p]
        L.orc_moe_forward.restype = ctypes.c_int
        L.orc_moe_forward.argtypes = (
            [ctypes.c_int] * 5
            + [_u8p, _f32p, _i32p, _f32p]
            + [ctypes.POINTER(ctypes.c_void_p)] * 4
            + [ctypes.c_int, _i32p, _u16p, _f32p, _f32p, _f32p, _f32p, _u8p, _f32p, _u16p,
               ctypes.c_int, ctypes.c_float, ctypes.c_int])
        L.orc_moe_l2_combine.restype = ctypes.c_int
        L.orc_moe_l2_combine.argtypes = (
            [ctypes.c_int] * 5 + [_i32p] + [ctypes.POINTER(ctypes.c_void_p)] * 2
            + [ctypes.c_int, _i32p, _u8p, _f32p, _u16p, _u16p, _f32p, ctypes.c_int,
               ctypes.c_int])
        L.orc_moe_l2_combine_mx.restype = ctypes.c_int
        L.orc_moe_l2_combine_mx.argtypes = (
            [ctypes.c_int] * 5 + [_i32p] + [ctypes.POINTER(ctypes.c_void_p)] * 2
            + [ctypes.c_int, _i32p, _u8p, _u8p, _u16p, _u16p, _f32p, ctypes.c_int,
               ctypes.c_int])
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_requant_block_pow2.restype = None
        L.orc_requant_block_pow2.argtypes = [_f32p, ctypes.c_int, _u8p, _f32p]
        L.orc_quantize_rows.restype = None
        L.orc_quantize_rows.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, _u8p, _f32p]
        L.orc_e2m1_decode.restype = ctypes.c_float
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_decode.restype = ctypes.c_double
        L.orc_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_ceil.restype = ctypes.c_uint8
        L.orc_e8m0_ceil.argtypes = [ctypes.c_float]
        L.orc_mx_dot.restype = ctypes.c_double
        L.orc_mx_dot.argtypes = [_u8p, _u8p, _u8p, _u8p, ctypes.c_int]
        L.orc_requant_block_mx.restype = None
        L.orc_requant_block_mx.argtypes = [_f32p, ctypes.c_int, _u8p, _u8p]
        L.orc_moe_forward_mx.restype = ctypes.c_int
        L.orc_moe_forward_mx.argtypes = (
            [ctypes.c_int] * 5
            + [_u8p, _u8p, _i32p, _f32p]
            + [ctypes.POINTER(ctypes.c_void_p)] * 4
            + [ctypes.c_int, _i32p, _u16p, _f32p, _f32p, _f32p, _f32p, _u8p, _u8p, _u16p,
               ctypes.c_int, ctypes.c_float, ctypes.c_int])
        _lib = L
    return _lib


def _p(a, t):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def bf16_rne(v: float) -> int:
    return lib().orc_bf16_rne(float(v))


def bf16_to_f32(b: int) -> float:
    return lib().orc_bf16_to_f32(int(b) & 0xFFFF)


def block_dot(a: np.ndarray, b: np.ndarray) -> float:
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return lib().orc_block_dot_e4m3(_p(a, _u8p), _p(b, _u8p), a.size)


def swiglu(g: float, u: float, w: float) -> float:
    return lib().orc_swiglu(float(g), float(u), float(w))


def requant_block(v: np.ndarray, pow2=False):
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.zeros(v.size, np.uint8)
    sf = ctypes.c_float(0)
    fn = lib().orc_requant_block_pow2 if pow2 else lib().orc_requant_block
    fn(_p(v, _f32p), v.size, _p(q, _u8p), ctypes.byref(sf))
    return q, sf.value


def quantize_rows(x: np.ndarray):
    """Per-1x128 e4m3 quantisation of [T,H] activations: (codes, f32 scales)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    q = np.zeros((T, H), np.uint8)
    sf = np.zeros((T, H // 128), np.float32)
    lib().orc_quantize_rows(_p(x, _f32p), T, H, _p(q, _u8p), _p(sf, _f32p))
    return q, sf


def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(int(code) & 0xF)


def e8m0_decode(code: int) -> float:
    return lib().orc_e8m0_decode(int(code) & 0xFF)


def e8m0_ceil(s: float) -> int:
    return lib().orc_e8m0_ceil(float(s))


def mx_dot(a, sa, b_packed, sb) -> float:
    """MX GEMM element: e4m3 a [n], UE8M0 sa [n/32], packed e2m1 b [n/2], sb [n/32]."""
    a, sa, b, sb = (np.ascontiguousarray(v, dtype=np.uint8) for v in (a, sa, b_packed, sb))
    assert a.size % 32 == 0 and b.size * 2 == a.size and sa.size == sb.size == a.size // 32
    return lib().orc_mx_dot(_p(a, _u8p), _p(sa, _u8p), _p(b, _u8p), _p(sb, _u8p), a.size)


def requant_block_mx(v: np.ndarray):
    """Power-of-two-scaled e4m3 requantisation: (codes, UE8M0 scale code)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.zeros(v.size, np.uint8)
    sf = ctypes.c_uint8(0)
    lib().orc_requant_block_mx(_p(v, _f32p), v.size, _p(q, _u8p), ctypes.byref(sf))
    return q, sf.value


def route(topk_idx: np.ndarray, num_experts: int, row_align: int, r_cap: int):
    """Plan: returns (counts[E], offsets[E+1], row_src[r_cap], src_row[T*K], n_bad)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = idx.shape
    E = num_experts
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    row_src = np.zeros(max(r_cap, 1), np.int32)
    src_row = np.zeros(max(T * K, 1), np.int32)
    bad = lib().orc_route(T, K, E, row_align, _p(idx, _i32p), _p(counts, _i32p),
                          _p(offsets, _i32p), _p(row_src, _i32p), r_cap,
                          _p(src_row, _i32p))
    return counts, offsets, row_src[:r_cap], src_row[:T * K], bad


def moe_forward(x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, *, tokens=None,
                flags=0, want=(), nthreads=0, clamp=0.0):
    """Oracle forward.

    w1, w1_sf, w2, w2_sf: sequences indexed by expert (arrays or None for
    experts no listed token uses).  tokens: optional list of token ids.
    want: subset of {"acc1", "acc1_mag", "hval", "h", "partial", "y_f32"} extra
    outputs ("acc1_mag": per L1 output the sum over K blocks of |scale product|
    times the block's sum of |products|, the magnitude a bound on rounding
    inside a block scales with; "hval": the f32 SwiGLU output before
    requantisation).
    Returns dict with "y" (uint16 bf16 bits [n,H]) and requested extras,
    indexed by position in the token list (slot-major: row p*K + j).
    """
    x = np.ascontiguousarray(x, dtype=np.uint8)
    x_sf = np.ascontiguousarray(x_sf, dtype=np.float32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    wts = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, H = x.shape
    K = idx.shape[1]
    E = len(w1)
    I = None
    keep = []

    def ptrs(seq, dt):
        arr = (ctypes.c_void_p * E)()
        for e, a in enumerate(seq):
            if a is None:
                arr[e] = None
            else:
                a = np.ascontiguousarray(a, dtype=dt)
                keep.append(a)
                arr[e] = a.ctypes.data
        return arr

    for a in w2:
        if a is not None:
            I = a.shape[-1]
            break
    if I is None:
        for a in w1:
            if a is not None:
                I = a.shape[0] // 2
                break
    if I is None:
        I = 128
    p1, p1s = ptrs(w1, np.uint8), ptrs(w1_sf, np.float32)
    p2, p2s = ptrs(w2, np.uint8), ptrs(w2_sf, np.float32)
    if tokens is None:
        toks = None
        n = T
    else:
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        n = toks.size
    y = np.zeros((n, H), np.uint16)
    y_f32 = np.zeros((n, H), np.float32) if "y_f32" in want else None
    acc1 = np.zeros((n * K, 2 * I), np.float32) if "acc1" in want else None
    acc1_mag = np.zeros((n * K, 2 * I), np.float32) if "acc1_mag" in want else None
    hval = np.zeros((n * K, I), np.float32) if "hval" in want else None
    h = np.zeros((n * K, I), np.uint8) if "h" in want else None
    G = 64 if flags & ORC_SF_GRAN64 else 128
    h_sf = np.zeros((n * K, I // G), np.float32) if "h" in want else None
    partial = np.zeros((n * K, H), np.uint16) if "partial" in want else None
    rc = lib().orc_moe_forward(
        T, H, I, E, K, _p(x, _u8p), _p(x_sf, _f32p), _p(idx, _i32p), _p(wts, _f32p),
        p1, p1s, p2, p2s, n, _p(toks, _i32p), _p(y, _u16p), _p(y_f32, _f32p),
        _p(acc1, _f32p), _p(acc1_mag, _f32p), _p(hval, _f32p), _p(h, _u8p), _p(h_sf, _f32p),
        _p(partial, _u16p), int(flags), float(clamp), int(nthreads))
    if rc < 0:
        raise ValueError("oracle: invalid shape or missing expert weights")
    out = {"y": y, "n_bad": rc}
    for k, v in (("y_f32", y_f32), ("acc1", acc1), ("acc1_mag", acc1_mag), ("hval", hval),
                 ("h", h), ("h_sf", h_sf), ("partial", partial)):
        if v is not None:
            out[k] = v
    return out


def _ptr_array(seq, dt, keep):
    arr = (ctypes.c_void_p * len(seq))()
    for e, a in enumerate(seq):
        if a is None:
            arr[e] = None
        else:
            a = np.ascontiguousarray(a, dtype=dt)
            keep.append(a)
            arr[e] = a.ctypes.data
    return arr


def moe_l2_combine(topk_idx, w2, w2_sf, h, h_sf, *, tokens=None, flags=0, want=(),
                   nthreads=0):
    """Oracle steps 5-6 (L2 + combine) from a given intermediate.

    h [n*K, I] e4m3 codes and h_sf [n*K, I/G] f32 scales (G = 64 with
    ORC_SF_GRAN64, else 128), rows indexed like moe_forward's outputs (slot j
    of the p-th listed token at row p*K + j; rows of skipped slots unread).
    w2, w2_sf: per-expert sequences as for moe_forward.  want: subset of
    {"partial", "o_mag"}.  Returns dict with "y" [n,H] bf16 bits and extras.
    """
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = idx.shape
    E = len(w2)
    h = np.ascontiguousarray(h, dtype=np.uint8)
    h_sf = np.ascontiguousarray(h_sf, dtype=np.float32)
    I = h.shape[1]
    H = next(a.shape[0] for a in w2 if a is not None)
    keep = []
    p2, p2s = _ptr_array(w2, np.uint8, keep), _ptr_array(w2_sf, np.float32, keep)
    toks = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if toks is None else toks.size
    assert h.shape[0] == n * K and h_sf.shape[0] == n * K
    y = np.zeros((n, H), np.uint16)
    partial = np.zeros((n * K, H), np.uint16) if "partial" in want else None
    o_mag = np.zeros((n * K, H), np.float32) if "o_mag" in want else None
    rc = lib().orc_moe_l2_combine(T, H, I, E, K, _p(idx, _i32p), p2, p2s, n, _p(toks, _i32p),
                                  _p(h, _u8p), _p(h_sf, _f32p), _p(y, _u16p),
                                  _p(partial, _u16p), _p(o_mag, _f32p), int(flags),
                                  int(nthreads))
    if rc < 0:
        raise ValueError("oracle: invalid shape or missing expert weights")
    out = {"y": y, "n_bad": rc}
    if partial is not None:
        out["partial"] = partial
    if o_mag is not None:
        out["o_mag"] = o_mag
    return out


def moe_l2_combine_mx(topk_idx, w2, w2_sf, h, h_sf, *, tokens=None, want=(), nthreads=0):
    """moe_l2_combine for the MXFP4 recipe: h_sf [n*K, I/32] UE8M0 codes,
    per expert w2 [H, I/2] packed e2m1 and w2_sf [H, I/32] codes."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = idx.shape
    E = len(w2)
    h = np.ascontiguousarray(h, dtype=np.uint8)
    h_sf = np.ascontiguousarray(h_sf, dtype=np.uint8)
    I = h.shape[1]
    H = next(a.shape[0] for a in w2 if a is not None)
    keep = []
    p2, p2s = _ptr_array(w2, np.uint8, keep), _ptr_array(w2_sf, np.uint8, keep)
    toks = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if toks is None else toks.size
    assert h.shape[0] == n * K and h_sf.shape[0] == n * K
    y = np.zeros((n, H), np.uint16)
    partial = np.zeros((n * K, H), np.uint16) if "partial" in want else None
    o_mag = np.zeros((n * K, H), np.float32) if "o_mag" in want else None
    rc = lib().orc_moe_l2_combine_mx(T, H, I, E, K, _p(idx, _i32p), p2, p2s, n,
                                     _p(toks, _i32p), _p(h, _u8p), _p(h_sf, _u8p),
                                     _p(y, _u16p), _p(partial, _u16p), _p(o_mag, _f32p), 0,
                                     int(nthreads))
    if rc < 0:
        raise ValueError("oracle: invalid shape or missing expert weights")
    out = {"y": y, "n_bad": rc}
    if partial is not None:
        out["partial"] = partial
    if o_mag is not None:
        out["o_mag"] = o_mag
    return out


def moe_forward_mx(x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, *, tokens=None,
                   flags=0, want=(), nthreads=0, clamp=0.0):
    """Oracle forward of the FP8 x MXFP4 recipe (see moe_oracle.c).

    x [T,H] e4m3, x_sf [T,H/32] UE8M0; per expert w1 [2I,H/2] packed e2m1,
    w1_sf [2I,H/32], w2 [H,I/2], w2_sf [H,I/32] (None for unused experts).
    Same outputs as moe_forward; "h" comes with "h_sf" [n*K, I/32] UE8M0.
    """
    x = np.ascontiguousarray(x, dtype=np.uint8)
    x_sf = np.ascontiguousarray(x_sf, dtype=np.uint8)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    wts = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, H = x.shape
    K = idx.shape[1]
    E = len(w1)
    keep = []

    def ptrs(seq):
        arr = (ctypes.c_void_p * E)()
        for e, a in enumerate(seq):
            if a is None:
                arr[e] = None
            else:
                a = np.ascontiguousarray(a, dtype=np.uint8)
                keep.append(a)
                arr[e] = a.ctypes.data
        return arr

    I = next((a.shape[-1] * 2 for a in w2 if a is not None), None)
    if I is None:
        I = next((a.shape[0] // 2 for a in w1 if a is not None), 128)
    p1, p1s, p2, p2s = ptrs(w1), ptrs(w1_sf), ptrs(w2), ptrs(w2_sf)
    if tokens is None:
        toks, n = None, T
    else:
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        n = toks.size
    y = np.zeros((n, H), np.uint16)
    y_f32 = np.zeros((n, H), np.float32) if "y_f32" in want else None
    acc1 = np.zeros((n * K, 2 * I), np.float32) if "acc1" in want else None
    acc1_mag = np.zeros((n * K, 2 * I), np.float32) if "acc1_mag" in want else None
    hval = np.zeros((n * K, I), np.float32) if "hval" in want else None
    h = np.zeros((n * K, I), np.uint8) if "h" in want else None
    h_sf = np.zeros((n * K, I // 32), np.uint8) if "h" in want else None
    partial = np.zeros((n * K, H), np.uint16) if "partial" in want else None
    rc = lib().orc_moe_forward_mx(
        T, H, I, E, K, _p(x, _u8p), _p(x_sf, _u8p), _p(idx, _i32p), _p(wts, _f32p),
        p1, p1s, p2, p2s, n, _p(toks, _i32p), _p(y, _u16p), _p(y_f32, _f32p),
        _p(acc1, _f32p), _p(acc1_mag, _f32p), _p(hval, _f32p), _p(h, _u8p), _p(h_sf, _u8p),
        _p(partial, _u16p), int(flags), float(clamp), int(nthreads))
    if rc < 0:
        raise ValueError("oracle: invalid shape or missing expert weights")
    out = {"y": y, "n_bad": rc}
    for k, v in (("y_f32", y_f32), ("acc1", acc1), ("acc1_mag", acc1_mag), ("hval", hval),
                 ("h", h), ("h_sf", h_sf), ("partial", partial)):
        if v is not None:
            out[k] = v
    return out


def max_threads() -> int:
    return lib().orc_max_threads()
