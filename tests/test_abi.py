"""The C-ABI library loads, exports every declared symbol, and rejects invalid
calls on the host before any HIP call (CPU only: no compute call is made)."""
import ctypes
import math
import os
import re

import pytest

import fp8_grouped_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp8.h")
PEAKS_HEADER = os.path.join(ROOT, "include", "moe_peaks.h")


def declared_symbols(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^(?:int|const char\*|size_t)\s+(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert declared_symbols() == sorted(moe.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert L.moe_version() >= 1


def test_peaks_library_exports_every_declared_symbol():
    from fp8_grouped_gemm_amd import peaks
    assert declared_symbols(PEAKS_HEADER) == sorted(peaks.EXPORTED_SYMBOLS)
    L = peaks.lib()
    for name in peaks.EXPORTED_SYMBOLS:
        assert hasattr(L, name), name


def test_peaks_reject_invalid_arguments_on_host():
    # every case fails the host checks, before the device is queried
    from fp8_grouped_gemm_amd import peaks
    L = peaks.lib()
    buf, out = ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20)
    bad_reads = [
        (None, 1 << 20, 256, 8, 1, out),                   # null buffer
        (buf, 1 << 20, 256, 8, 1, None),                   # null out
        (ctypes.c_void_p((1 << 20) + 8), 1 << 20, 256, 8, 1, out),  # misaligned
        (buf, 0, 256, 8, 1, out), (buf, 1000, 256, 8, 1, out),      # size
        (buf, 1 << 20, 0, 8, 1, out), (buf, 1 << 20, 65537, 8, 1, out),  # blocks
        (buf, 1 << 20, 256, 2, 1, out), (buf, 1 << 20, 256, 16, 1, out),  # unroll
        (buf, 1 << 20, 256, 8, 2, out), (buf, 1 << 20, 256, 8, -1, out),  # mode
    ]
    for a in bad_reads:
        assert L.moe_peak_stream_read(*a, None) == moe.MOE_ERR_INVALID_ARG, a
    for blocks, iters, o in [(0, 16, out), (65537, 16, out), (256, 0, out), (256, 2049, out),
                             (256, 16, None)]:
        assert L.moe_peak_mfma_fp8(blocks, iters, o, None) == moe.MOE_ERR_INVALID_ARG
    for blocks, o in [(0, out), (65537, out), (-1, out), (256, None)]:
        assert L.moe_probe_conversions(blocks, o, None) == moe.MOE_ERR_INVALID_ARG


def test_strerror_names_every_code():
    for code in (0, -1, -2, -3, -4, -5):
        assert moe.strerror(code) != "unknown error"
    assert moe.strerror(-99) == "unknown error"


@pytest.mark.parametrize("shape,code", [
    ((250, 128, 8, 2, 64, 0), moe.MOE_ERR_UNSUPPORTED_SHAPE),   # H % 128
    ((256, 100, 8, 2, 64, 0), moe.MOE_ERR_UNSUPPORTED_SHAPE),   # I % 128
    ((256, 128, 8, 9, 64, 0), moe.MOE_ERR_INVALID_ARG),         # K > E
    ((256, 128, 2048, 2, 64, 0), moe.MOE_ERR_UNSUPPORTED_SHAPE),  # E > 1024
    ((256, 128, 8, 2, -1, 0), moe.MOE_ERR_INVALID_ARG),         # max_tokens < 0
    ((256, 128, 8, 2, 64, 48), moe.MOE_ERR_UNSUPPORTED_SHAPE),  # tile_m
    ((0, 128, 8, 2, 64, 0), moe.MOE_ERR_INVALID_ARG),
    ((256, 128, 8, 8, 1 << 21, 0), moe.MOE_ERR_UNSUPPORTED_SHAPE),  # T*K >= 2^24
])
def test_plan_create_rejects(shape, code):
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_plan_create(*shape)
    assert ei.value.code == code


def test_packed_layout_validation():
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_plan_create(384, 128, 8, 2, 64, 0, moe.MOE_WEIGHTS_PACKED)  # H % 256
    assert ei.value.code == moe.MOE_ERR_UNSUPPORTED_SHAPE
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_plan_create(256, 128, 8, 2, 64, 0, 7)
    assert ei.value.code == moe.MOE_ERR_INVALID_ARG
    L = moe.lib()
    a, b, c, d = (ctypes.c_void_p(x) for x in (0x10000, 0x20000000, 0x40000000, 0x60000000))
    row = moe.moe_plan_create(256, 128, 8, 2, 64)
    pk = moe.moe_plan_create(256, 128, 8, 2, 64, 0, moe.MOE_WEIGHTS_PACKED)
    try:
        # a row-major plan has nothing to prepare
        assert L.moe_prepare_weights(row, a, b, c, d, None) == moe.MOE_ERR_INVALID_ARG
        # null or overlapping buffers are rejected before any HIP call
        assert L.moe_prepare_weights(pk, None, b, c, d, None) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_prepare_weights(pk, a, b, ctypes.c_void_p(0x10000 + 4096), d, None) == \
            moe.MOE_ERR_INVALID_ARG
    finally:
        moe.moe_plan_destroy(row)
        moe.moe_plan_destroy(pk)


def test_plan_create_null_shape():
    h = ctypes.c_void_p()
    assert moe.lib().moe_plan_create(None, ctypes.byref(h)) == moe.MOE_ERR_INVALID_ARG


def test_plan_info_tile_choice_and_workspace_monotone():
    p = moe.moe_plan_create(4096, 2048, 256, 6, 8192)
    try:
        assert moe.moe_plan_info(p, 128)["tile_m"] == 16      # 3 rows / expert
        assert moe.moe_plan_info(p, 853)["tile_m"] == 32      # 20 rows / expert
        assert moe.moe_plan_info(p, 1024)["tile_m"] == 64     # 24 rows / expert
        assert moe.moe_plan_info(p, 8192)["tile_m"] >= 64
        last = 0
        for T in (0, 1, 17, 128, 500, 1024, 2048, 4096, 8192):
            b = moe.moe_workspace_bytes(p, T)
            assert b >= last
            last = b
        info = moe.moe_plan_info(p, 128)
        assert info["pool_rows"] >= 128 * 6 + 256 * 15
        assert info["pool_rows"] % info["tile_m"] == 0
        lay = moe.moe_workspace_layout(p, 128)
        assert lay["total"] == moe.moe_workspace_bytes(p, 128)
        assert all(lay[k] % 256 == 0 for k in lay if k != "total")
        with pytest.raises(moe.MoEError):
            moe.moe_plan_info(p, 8193)
    finally:
        moe.moe_plan_destroy(p)


def test_tile128_needs_two_k_blocks_per_layer():
    # the persistent 128-row-tile kernels need H % 256 == 0 and I >= 256
    for shape in ((256, 128, 8, 2), (384, 256, 8, 2)):
        with pytest.raises(moe.MoEError) as e:
            moe.moe_plan_create(*shape, 64, tile_m=128)
        assert e.value.code == moe.MOE_ERR_UNSUPPORTED_SHAPE
    p = moe.moe_plan_create(256, 128, 8, 2, 4096)   # auto choice never picks them there
    try:
        assert moe.moe_plan_info(p, 4096)["tile_m"] == 64
        assert moe.moe_plan_info(p, 4096)["kernel"] == 0
    finally:
        moe.moe_plan_destroy(p)
    moe.moe_plan_destroy(moe.moe_plan_create(256, 256, 8, 2, 64, tile_m=128))


def test_tile160_validation_and_info():
    # the 160-row LDS tile: FP8 recipe, per-128 intermediate scales, packed
    # weights, two K blocks per layer, 31-bit copy offsets; no ring pool
    P = moe.MOE_WEIGHTS_PACKED
    bad = [((512, 384, 16, 4, 256), dict()),                                  # row-major
           ((512, 384, 16, 4, 256), dict(weight_layout=P, recipe=moe.MOE_RECIPE_MXFP4)),
           ((512, 384, 16, 4, 256), dict(weight_layout=P, act_sf_gran=64)),
           ((512, 384, 16, 4, 256), dict(weight_layout=P, flags=moe.MOE_FLAG_RING_POOL)),
           ((256, 128, 8, 2, 64), dict(weight_layout=P)),                      # one K block of I
           ((7168, 3072, 384, 6, 1 << 19), dict(weight_layout=P))]             # T*H >= 2^31
    for shape, kw in bad:
        with pytest.raises(moe.MoEError) as e:
            moe.moe_plan_create(*shape, tile_m=160, **kw)
        assert e.value.code == moe.MOE_ERR_UNSUPPORTED_SHAPE, (shape, kw)
    p = moe.moe_plan_create(512, 384, 16, 4, 256, tile_m=160, weight_layout=P)
    try:
        info = moe.moe_plan_info(p, 256)
        assert (info["tile_m"], info["row_align"], info["kernel"]) == (160, 160, 3)
        # pool capacity: T*K + E*(160 - 1) rounded up to 160 rows
        assert info["pool_rows"] == -(-(256 * 4 + 16 * 159) // 160) * 160
    finally:
        moe.moe_plan_destroy(p)


def test_tile160_auto_choice_follows_the_measured_sweep():
    # the expected-row-tiles rule against the measured faster tile (pro and
    # flash prefill shapes, packed FP8 weights): 160 rows from ~120 to ~170
    # rows per expert and at 256, 128 rows at 96, 112 and 192; row-major
    # weights and per-64 scales keep the 128-row tile
    P = moe.MOE_WEIGHTS_PACKED
    cases = [((7168, 3072, 384, 6), 6144, 128), ((7168, 3072, 384, 6), 7168, 128),
             ((7168, 3072, 384, 6), 8192, 160), ((7168, 3072, 384, 6), 9216, 160),
             ((7168, 3072, 384, 6), 10240, 160), ((7168, 3072, 384, 6), 12288, 128),
             ((7168, 3072, 384, 6), 16384, 160), ((4096, 2048, 256, 6), 4096, 128),
             ((4096, 2048, 256, 6), 5461, 160), ((4096, 2048, 256, 6), 6827, 160),
             ((4096, 2048, 256, 6), 8192, 128)]
    for shape, T, tile in cases:
        p = moe.moe_plan_create(*shape, T, weight_layout=P)
        try:
            info = moe.moe_plan_info(p, T)
            assert info["tile_m"] == tile, (shape, T, info["tile_m"])
            assert info["kernel"] == (3 if tile == 160 else 1)
        finally:
            moe.moe_plan_destroy(p)
    for kw in (dict(), dict(weight_layout=P, act_sf_gran=64)):
        p = moe.moe_plan_create(7168, 3072, 384, 6, 8192, **kw)
        try:
            assert moe.moe_plan_info(p, 8192)["tile_m"] == 128, kw
        finally:
            moe.moe_plan_destroy(p)


def test_tile64_kernel_choice():
    # 64-row tiles run on the shared-A kernel where the LDS tiles fit (per-64
    # scales included), on the direct-load kernel where they do not (H % 256
    # != 0, too few K blocks) or when the plan asks for direct tiles
    cases = [((512, 384, 16, 4), {}, 2),
             ((512, 384, 16, 4), dict(flags=moe.MOE_FLAG_DIRECT_TILES), 0),
             ((384, 256, 8, 2), {}, 0),
             ((256, 128, 8, 2), {}, 0),
             ((512, 384, 16, 4), dict(act_sf_gran=64), 2),
             ((512, 384, 16, 4), dict(recipe=moe.MOE_RECIPE_MXFP4), 2),
             ((512, 256, 16, 4), dict(recipe=moe.MOE_RECIPE_MXFP4), 0)]  # MX: 3 K blocks
    for shape, kw, kernel in cases:
        p = moe.moe_plan_create(*shape, 256, tile_m=64, **kw)
        try:
            assert moe.moe_plan_info(p, 256)["kernel"] == kernel, (shape, kw)
        finally:
            moe.moe_plan_destroy(p)


def test_plan_flags_and_single_launch_choice():
    with pytest.raises(moe.MoEError) as e:
        moe.moe_plan_create(256, 128, 8, 2, 64, flags=1 << 5)            # unknown bit
    assert e.value.code == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoEError):
        moe.moe_plan_create(256, 128, 8, 2, 64,
                            flags=moe.MOE_FLAG_SINGLE_LAUNCH | moe.MOE_FLAG_SPLIT_LAUNCH)
    p = moe.moe_plan_create(4096, 2048, 256, 6, 8192, flags=moe.MOE_FLAG_SINGLE_LAUNCH)
    q = moe.moe_plan_create(4096, 2048, 256, 6, 8192, flags=moe.MOE_FLAG_SPLIT_LAUNCH)
    try:
        assert moe.moe_plan_info(p, 128)["single_launch"] == 1   # 16-row direct tiles
        assert moe.moe_plan_info(p, 853)["single_launch"] == 1   # 32-row direct tiles
        assert moe.moe_plan_info(p, 1)["single_launch"] == 0     # L1 split-K: split launches
        assert moe.moe_plan_info(p, 8192)["single_launch"] == 0  # LDS tiles: split launches
        assert all(moe.moe_plan_info(q, T)["single_launch"] == 0 for T in (1, 128, 1024, 8192))
        assert moe.moe_workspace_bytes(p, 128) == moe.moe_workspace_bytes(q, 128)
    finally:
        moe.moe_plan_destroy(p)
        moe.moe_plan_destroy(q)


@pytest.mark.parametrize("shape", [(4096, 2048, 256, 6, 0), (256, 128, 8, 2, 16),
                                   (512, 384, 16, 4, 16), (7168, 3072, 384, 6, 0)])
def test_split_k_choice_and_workspace_monotone_every_T(shape):
    # L1 split-K only where the 16-row tiles number fewer than the compute
    # units (256): S in {1, 2, 4}, nonincreasing in T, at most the K blocks;
    # the workspace never shrinks as T grows, for every T.
    H, I, E, K, tile = shape
    p = moe.moe_plan_create(H, I, E, K, 300, tile_m=tile)
    try:
        last_b, last_s = 0, 4
        for T in range(0, 301):
            info = moe.moe_plan_info(p, T)
            S = info["l1_split"]
            assert S in (1, 2, 4) and S <= max(1, H // 128) and S <= last_s, (T, S)
            if info["tile_m"] != 16 or T == 0:
                assert S == 1
            else:
                rows = max((T * K + 15) // 16, min(T * K, E))
                tiles = rows * (I // 128)
                assert (S == 1) == (tiles >= 256) or S == min(4, H // 128), (T, S, tiles)
            # 16-row L2 tiles pair up in 8-wave workgroups once at least
            # 1024 such workgroups are expected
            g = info["l2_group_tiles"]
            if info["tile_m"] == 16 and T > 0:
                rows = max((T * K + 15) // 16, min(T * K, E))
                assert (g == 2) == (rows * ((H // 256 + 1) // 2) >= 1024), (T, g)
            else:
                assert g == 1
            # L2 splits K by the same rule over its 256-column tiles
            S2 = info["l2_split"]
            assert S2 in (1, 2, 4) and S2 <= max(1, I // 128), (T, S2)
            if info["tile_m"] != 16 or T == 0:
                assert S2 == 1
            else:
                rows = max((T * K + 15) // 16, min(T * K, E))
                tiles2 = rows * ((H + 255) // 256)
                assert (S2 == 1) == (2 * tiles2 >= 256 or I // 128 < 2), (T, S2, tiles2)
                if S2 > 1:  # the smallest power of two reaching 256 items, within limits
                    assert tiles2 * S2 >= 256 or S2 == 4 or 2 * S2 > I // 128, (T, S2, tiles2)
                if S2 > 1:
                    assert g == 1 and info["single_launch"] == 0
            b = moe.moe_workspace_bytes(p, T)
            assert b >= last_b, T
            last_b = b
            if T > 0:
                last_s = S
    finally:
        moe.moe_plan_destroy(p)


class FakeTensor:
    """Stand-in carrying an address; these calls fail before touching it."""

    def __init__(self, addr=0x1000, nbytes=1 << 20):
        self.addr, self.nbytes = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def _forward_rc(plan, T, **over):
    args = dict(x=FakeTensor(), x_sf=FakeTensor(), topk_idx=FakeTensor(), topk_w=FakeTensor(),
                w1=FakeTensor(), w1_sf=FakeTensor(), w2=FakeTensor(), w2_sf=FakeTensor(),
                y=FakeTensor(), workspace=FakeTensor())
    args.update(over)
    try:
        moe.moe_forward(plan, T, args["x"], args["x_sf"], args["topk_idx"], args["topk_w"],
                        args["w1"], args["w1_sf"], args["w2"], args["w2_sf"], args["y"],
                        args["workspace"], stream=0)
        return 0
    except moe.MoEError as e:
        return e.code


def test_forward_host_validation_without_gpu():
    p = moe.moe_plan_create(256, 128, 8, 2, 64)
    try:
        assert _forward_rc(p, 65) == moe.MOE_ERR_INVALID_ARG       # T > max_tokens
        assert _forward_rc(p, -1) == moe.MOE_ERR_INVALID_ARG
        assert _forward_rc(p, 0) == moe.MOE_OK                      # no-op, no HIP call
        for name in ("x", "x_sf", "topk_idx", "topk_w", "w1", "w1_sf", "w2", "w2_sf", "y",
                     "workspace"):
            assert _forward_rc(p, 8, **{name: None}) == moe.MOE_ERR_INVALID_ARG, name
        # alignment: 16 bytes for x, w1, w2, y; 256 for the workspace
        for name in ("x", "w1", "w2", "y"):
            assert _forward_rc(p, 8, **{name: FakeTensor(addr=0x1008)}) == \
                moe.MOE_ERR_INVALID_ARG, name
        assert _forward_rc(p, 8, workspace=FakeTensor(addr=0x1080)) == moe.MOE_ERR_INVALID_ARG
        small = FakeTensor(nbytes=moe.moe_workspace_bytes(p, 8) - 1)
        assert _forward_rc(p, 8, workspace=small) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
        rc = moe.lib().moe_forward(None, 8, *([ctypes.c_void_p(0x1000)] * 10), 1 << 30, None)
        assert rc == moe.MOE_ERR_INVALID_ARG
    finally:
        moe.moe_plan_destroy(p)


def test_route_host_validation_without_gpu():
    p = moe.moe_plan_create(256, 128, 8, 2, 64)
    L = moe.lib()
    a = ctypes.c_void_p(0x1000)
    big = 1 << 30
    try:
        # row_align out of range
        assert L.moe_route(p, 8, a, 0, a, a, a, 1000, a, a, big, None) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_route(p, 8, a, 2048, a, a, a, 10 ** 6, a, a, big, None) == moe.MOE_ERR_INVALID_ARG
        # row_src too short for T*K + E*(row_align-1)
        assert L.moe_route(p, 8, a, 16, a, a, a, 16 + 8 * 15 - 1, a, a, big, None) == \
            moe.MOE_ERR_INVALID_ARG
        # workspace too small
        assert L.moe_route(p, 8, a, 16, a, a, a, 1000, a, a, 8, None) == \
            moe.MOE_ERR_WORKSPACE_TOO_SMALL
        # null outputs
        assert L.moe_route(p, 8, a, 16, None, a, a, 1000, a, a, big, None) == moe.MOE_ERR_INVALID_ARG
    finally:
        moe.moe_plan_destroy(p)


def test_mx_recipe_validation_and_choices():
    # recipe values, and what an MXFP4 plan accepts
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_plan_create(256, 256, 4, 2, 8, recipe=2)
    assert ei.value.code == moe.MOE_ERR_INVALID_ARG
    # the MXFP4 LDS tile keeps three K blocks in flight: H, I >= 384
    for H, I in ((256, 256), (512, 256)):
        with pytest.raises(moe.MoEError) as ei:
            moe.moe_plan_create(H, I, 4, 2, 8, tile_m=128, recipe=moe.MOE_RECIPE_MXFP4)
        assert ei.value.code == moe.MOE_ERR_UNSUPPORTED_SHAPE
    moe.moe_plan_destroy(moe.moe_plan_create(512, 384, 4, 2, 8, tile_m=128,
                                             recipe=moe.MOE_RECIPE_MXFP4))
    with pytest.raises(moe.MoEError) as ei:  # x must be addressable with 32-bit offsets
        moe.moe_plan_create(65536, 256, 4, 2, 32768, recipe=moe.MOE_RECIPE_MXFP4)
    assert ei.value.code == moe.MOE_ERR_UNSUPPORTED_SHAPE
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_plan_create(256, 256, 4, 2, 8, recipe=moe.MOE_RECIPE_MXFP4,
                            flags=moe.MOE_FLAG_SINGLE_LAUNCH)
    assert ei.value.code == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoEError) as ei:  # packed needs whole 256-row L2 tiles
        moe.moe_plan_create(384, 256, 4, 2, 8, recipe=moe.MOE_RECIPE_MXFP4,
                            weight_layout=moe.MOE_WEIGHTS_PACKED)
    assert ei.value.code == moe.MOE_ERR_UNSUPPORTED_SHAPE
    # moe_prepare_weights_mx: only packed MXFP4 plans, no overlaps, aligned
    # weights; moe_prepare_weights refuses MXFP4 plans (no HIP call is made)
    L = moe.lib()
    pk = moe.moe_plan_create(256, 256, 4, 2, 8, recipe=moe.MOE_RECIPE_MXFP4,
                             weight_layout=moe.MOE_WEIGHTS_PACKED)
    rm = moe.moe_plan_create(256, 256, 4, 2, 8, recipe=moe.MOE_RECIPE_MXFP4)
    fp = moe.moe_plan_create(256, 256, 4, 2, 8, weight_layout=moe.MOE_WEIGHTS_PACKED)
    try:
        M = 1 << 24
        bufs = [ctypes.c_void_p(M * (i + 1)) for i in range(8)]
        for plan in (rm, fp):
            assert L.moe_prepare_weights_mx(plan, *bufs, None) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_prepare_weights(pk, bufs[0], bufs[2], bufs[4], bufs[6], None) == \
            moe.MOE_ERR_INVALID_ARG
        same = list(bufs)
        same[4] = bufs[0]  # packed w1 over the input w1
        assert L.moe_prepare_weights_mx(pk, *same, None) == moe.MOE_ERR_INVALID_ARG
        mis = list(bufs)
        mis[6] = ctypes.c_void_p(M * 7 + 8)  # packed w2 not 16-byte aligned
        assert L.moe_prepare_weights_mx(pk, *mis, None) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_prepare_weights_mx(pk, None, *bufs[1:], None) == moe.MOE_ERR_INVALID_ARG
    finally:
        for plan in (pk, rm, fp):
            moe.moe_plan_destroy(plan)
    p = moe.moe_plan_create(4096, 2048, 256, 6, 8192, recipe=moe.MOE_RECIPE_MXFP4)
    q = moe.moe_plan_create(4096, 2048, 256, 6, 8192)
    try:
        for T in (1, 2, 8, 128, 1024, 8192):
            info = moe.moe_plan_info(p, T)
            # at these token counts the same tile choice as FP8 up to 1024
            # tokens (MXFP4 leaves 32-row tiles out where the shared-A tile
            # fits, and takes it again beyond 108 rows per expert), no
            # split-K, one L2 tile per workgroup
            want = (64, 2) if T == 8192 else (moe.moe_plan_info(q, T)["tile_m"],
                                                moe.moe_plan_info(q, T)["kernel"])
            assert (info["tile_m"], info["kernel"]) == want, T
            assert info["l1_split"] == 1 and info["l2_group_tiles"] == 1 and \
                info["single_launch"] == 0, T
            # same workspace as the FP8 plan (h_sf: I/32 bytes = I/128 floats per row)
            assert moe.moe_workspace_bytes(p, T) <= moe.moe_workspace_bytes(q, T) or \
                moe.moe_plan_info(q, T)["tile_m"] != info["tile_m"]
        # each forward entry point rejects the other recipe's plan before any
        # HIP call (fake pointers are never touched)
        fake = [ctypes.c_void_p(4096 * (i + 1)) for i in range(10)]
        L = moe.lib()
        args = [fake[0], fake[1], fake[2], fake[3], fake[4], fake[5], fake[6], fake[7], fake[8],
                fake[9], 1 << 30, None]
        assert L.moe_forward(p, 4, *args) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_forward_mx(q, 4, *args) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_forward_mx(p, -1, *args) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_forward_mx(p, 4, None, *args[1:]) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_forward_mx(p, 0, *args) == moe.MOE_OK  # T == 0: no-op
    finally:
        moe.moe_plan_destroy(p)
        moe.moe_plan_destroy(q)


def test_recipe_options_validation_and_rule():
    # act_sf_gran: 0/128, 64, -1 (PR #440 rule); per-64 plans: no single
    # launch; MXFP4 plans: no per-64 or power-of-two flag; NaN clamp
    for kw, code in ((dict(act_sf_gran=32), moe.MOE_ERR_INVALID_ARG),
                     (dict(act_sf_gran=64, flags=moe.MOE_FLAG_SINGLE_LAUNCH), moe.MOE_ERR_INVALID_ARG),
                     (dict(activation_clamp=float("nan")), moe.MOE_ERR_INVALID_ARG),
                     (dict(act_sf_gran=64, recipe=moe.MOE_RECIPE_MXFP4), moe.MOE_ERR_INVALID_ARG),
                     (dict(flags=moe.MOE_FLAG_POW2_SCALE, recipe=moe.MOE_RECIPE_MXFP4),
                      moe.MOE_ERR_INVALID_ARG)):
        with pytest.raises(moe.MoEError) as ei:
            moe.moe_plan_create(4096, 2048, 256, 6, 8192, **kw)
        assert ei.value.code == code, kw
    for (H, I), want in (((4096, 2048), 128), ((7168, 3072), 128), ((256, 128), 64),
                         ((640, 384), 64)):
        p = moe.moe_plan_create(H, I, 16, 2, 4096, act_sf_gran=-1)
        try:
            info = moe.moe_plan_info(p, 4096)
            assert info["act_sf_gran"] == want, (H, I)
        finally:
            moe.moe_plan_destroy(p)
    # per-64 plans take the LDS tiles where they fit (128 rows at 4096 tokens)
    p = moe.moe_plan_create(4096, 2048, 256, 6, 8192, act_sf_gran=64)
    try:
        assert moe.moe_plan_info(p, 8192)["kernel"] == 1
        assert moe.moe_plan_info(p, 2048)["kernel"] == 2
    finally:
        moe.moe_plan_destroy(p)
    # per-64 needs twice the h_sf bytes; the workspace grows accordingly
    a = moe.moe_plan_create(4096, 2048, 256, 6, 128)
    b = moe.moe_plan_create(4096, 2048, 256, 6, 128, act_sf_gran=64)
    try:
        la, lb = moe.moe_workspace_layout(a, 128), moe.moe_workspace_layout(b, 128)
        assert lb["h"] - lb["h_sf"] >= 2 * (la["h"] - la["h_sf"]) - 256
        assert moe.moe_plan_info(b, 128)["single_launch"] == 0
    finally:
        moe.moe_plan_destroy(a)
        moe.moe_plan_destroy(b)


def test_quantize_act_rejects_invalid_calls_on_host():
    L = moe.lib()
    p = moe.moe_plan_create(256, 128, 4, 2, 8)
    try:
        x, q, sf = ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20)
        assert L.moe_quantize_act(p, 9, x, q, sf, None) == moe.MOE_ERR_INVALID_ARG  # T > max
        assert L.moe_quantize_act(p, 4, None, q, sf, None) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_quantize_act(p, 4, ctypes.c_void_p((1 << 20) + 2), q, sf, None) == \
            moe.MOE_ERR_INVALID_ARG
        assert L.moe_quantize_act(p, 4, x, q, ctypes.c_void_p((3 << 20) + 1), None) == \
            moe.MOE_ERR_INVALID_ARG
        assert L.moe_quantize_act(p, 0, x, q, sf, None) == moe.MOE_OK  # no-op
        assert L.moe_quantize_act(None, 4, x, q, sf, None) == moe.MOE_ERR_INVALID_ARG
    finally:
        moe.moe_plan_destroy(p)


def test_noalloc_host_validation_without_gpu():
    # every rejection of moe_forward_noalloc happens before its first HIP call
    L = moe.lib()
    a = ctypes.c_void_p(0x1000)
    p = moe.moe_plan_create(4096, 2048, 256, 6, 8192)
    pmx = moe.moe_plan_create(4096, 2048, 256, 6, 64, recipe=moe.MOE_RECIPE_MXFP4)
    try:
        assert L.moe_forward_noalloc(p, 8193, *([a] * 9), None) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_forward_noalloc(p, -1, *([a] * 9), None) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_forward_noalloc(p, 0, *([None] * 9), None) == moe.MOE_OK  # no-op
        for i in range(9):
            args = [a] * 9
            args[i] = None
            assert L.moe_forward_noalloc(p, 8, *args, None) == moe.MOE_ERR_INVALID_ARG, i
        for i in (0, 4, 6, 8):  # x, w1, w2, y need 16-byte alignment
            args = [a] * 9
            args[i] = ctypes.c_void_p(0x1008)
            assert L.moe_forward_noalloc(p, 8, *args, None) == moe.MOE_ERR_INVALID_ARG, i
        # the static scratch holds the workspace of up to 404 flash-decode tokens
        assert moe.moe_workspace_bytes(p, 404) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        assert moe.moe_workspace_bytes(p, 405) > moe.MOE_NOALLOC_SCRATCH_BYTES
        assert L.moe_forward_noalloc(p, 405, *([a] * 9), None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
        assert L.moe_forward_noalloc(pmx, 8, *([a] * 9), None) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_forward_noalloc(None, 8, *([a] * 9), None) == moe.MOE_ERR_INVALID_ARG
    finally:
        moe.moe_plan_destroy(p)
        moe.moe_plan_destroy(pmx)


def _ring_expect(T, K, tile):
    # DeepGEMM PR #440 "How it works": units of up to 8 row blocks, lag =
    # clamp(round(0.45 units), 8, 64); "Ring sizing": 8 (lag + 4) + 4 slots
    units = max(1, -(-(T * K) // (8 * tile)))
    lag = min(64, max(8, math.floor(0.45 * units + 0.5)))
    return 8 * (lag + 4) + 4, lag


def test_ring_pool_plan_info_sizes_and_workspace():
    H, I, E, K = 4096, 2048, 256, 6
    ring = moe.moe_plan_create(H, I, E, K, 8192, flags=moe.MOE_FLAG_RING_POOL)
    try:
        last = 0
        for T in (1, 2, 17, 128, 300, 1024, 2048, 4096, 5000, 8192):
            info = moe.moe_plan_info(ring, T)
            # the single launch with direct-load tiles, one L2 tile per workgroup
            assert info["kernel"] == 0 and info["l1_split"] == 1, T
            assert info["single_launch"] == 1 and info["l2_group_tiles"] == 1, T
            blocks = info["pool_rows"] // info["tile_m"]
            rb, lag = _ring_expect(T, K, info["tile_m"])
            if rb < blocks:
                assert (info["ring_blocks"], info["l2_lag_units"]) == (rb, lag), T
                # the ring holds the live set 8 (lag + group) + 1
                assert info["ring_blocks"] >= 8 * (info["l2_lag_units"] + 4) + 1
            else:  # a ring the size of the pool never wraps
                assert (info["ring_blocks"], info["l2_lag_units"]) == (0, 0), T
            b = moe.moe_workspace_bytes(ring, T)
            assert b >= last, T
            last = b
            if info["ring_blocks"] > 0:
                # against the full pool with the same tiles, h and h_sf shrink
                # from pool_rows to ring_blocks * tile_m rows
                full = moe.moe_plan_create(H, I, E, K, 8192, tile_m=info["tile_m"],
                                           flags=moe.MOE_FLAG_SINGLE_LAUNCH |
                                           moe.MOE_FLAG_DIRECT_TILES)
                try:
                    saved = ((info["pool_rows"] - info["ring_blocks"] * info["tile_m"]) *
                             (I + 4 * I // 128))
                    assert moe.moe_workspace_bytes(full, T) - b >= saved // 2, T
                finally:
                    moe.moe_plan_destroy(full)
        assert moe.moe_plan_info(ring, 2048)["ring_blocks"] == 124       # lag 11 at 64-row tiles
        assert moe.moe_plan_info(ring, 8192)["l2_lag_units"] == 43
    finally:
        moe.moe_plan_destroy(ring)


def test_ring_pool_flag_rejections():
    R = moe.MOE_FLAG_RING_POOL
    for kw, err in ((dict(flags=R | moe.MOE_FLAG_SPLIT_LAUNCH), moe.MOE_ERR_INVALID_ARG),
                    (dict(flags=R, recipe=moe.MOE_RECIPE_MXFP4), moe.MOE_ERR_INVALID_ARG),
                    (dict(flags=R, act_sf_gran=64), moe.MOE_ERR_INVALID_ARG),
                    (dict(flags=R, act_sf_gran=-1), moe.MOE_ERR_INVALID_ARG),  # 2I % 512 != 0
                    (dict(flags=R, tile_m=128), moe.MOE_ERR_UNSUPPORTED_SHAPE)):
        H, I = (4096, 2048 + 128) if kw.get("act_sf_gran") == -1 else (4096, 2048)
        with pytest.raises(moe.MoEError) as ex:
            moe.moe_plan_create(H, I, 256, 6, 64, **kw)
        assert ex.value.code == err, kw
    # the shape rule that gives per-128 scales keeps the ring
    p = moe.moe_plan_create(4096, 2048, 256, 6, 64, flags=R, act_sf_gran=-1)
    moe.moe_plan_destroy(p)


def test_ring_pool_over_capacity_rejected_before_any_launch():
    # a token count one alignment above the plan's bound is refused on the
    # host, before any HIP call (DeepGEMM PR #440 "API, Tests, Files")
    L = moe.lib()
    a = ctypes.c_void_p(0x1000)
    p = moe.moe_plan_create(4096, 2048, 256, 6, 1024, flags=moe.MOE_FLAG_RING_POOL)
    try:
        for T in (1025, 1024 + 16, 1024 + 64):
            assert L.moe_forward(p, T, *([a] * 9), a, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
            with pytest.raises(moe.MoEError):
                moe.moe_plan_info(p, T)
            with pytest.raises(moe.MoEError):
                moe.moe_workspace_bytes(p, T)
        # a workspace one byte short is refused before any HIP call too
        need = moe.moe_workspace_bytes(p, 1024)
        assert L.moe_forward(p, 1024, *([a] * 9), ctypes.c_void_p(0x100000), need - 1,
                             None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    finally:
        moe.moe_plan_destroy(p)


@pytest.mark.parametrize("shape", [(4096, 2048, 256, 6), (7168, 3072, 384, 6)])
def test_mxfp4_tile_choice_and_workspace_monotone(shape):
    # MXFP4 takes the 128-row LDS tile only between 64 and 108 routed rows per
    # expert and the 64-row shared-A tile on both sides, yet a workspace sized
    # for a token count serves every smaller one
    H, I, E, K = shape
    p = moe.moe_plan_create(H, I, E, K, 16384, recipe=moe.MOE_RECIPE_MXFP4)
    try:
        last = 0
        for T in list(range(1, 16385, 61)) + [16384]:
            info = moe.moe_plan_info(p, T)
            rows = T * K / E
            if 64 < rows <= 108:
                assert (info["tile_m"], info["kernel"]) == (128, 1), T
            elif rows > 108:
                assert (info["tile_m"], info["kernel"]) == (64, 2), T
            b = moe.moe_workspace_bytes(p, T)
            assert b >= last, T
            last = b
    finally:
        moe.moe_plan_destroy(p)
