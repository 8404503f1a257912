"""FP8 MoE expert forward on MI355X (gfx950): Python binding of libmoe_fp8.so.

The binding only marshals arguments: every step of the forward runs in the
HIP kernels of the library (include/moe_fp8.h documents the ABI).  torch
supplies device memory and the stream.  Importing this package does not
load the library; the first call does, and it raises if the library has not
been built (python -m fp8_grouped_gemm_amd.build) -- there is no fallback.
"""
import ctypes
import os

from .build import LIB as LIB_PATH

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED_SHAPE = -2
MOE_ERR_WORKSPACE_TOO_SMALL = -3
MOE_ERR_HIP = -4
MOE_ERR_NOT_GFX950 = -5
MOE_STATUS_EXPERT_OUT_OF_RANGE = 1
MOE_STATUS_WAIT_TIMEOUT = 2
MOE_WEIGHTS_ROW_MAJOR = 0
MOE_WEIGHTS_PACKED = 1
MOE_FLAG_SINGLE_LAUNCH = 1
MOE_FLAG_SPLIT_LAUNCH = 2
MOE_FLAG_POW2_SCALE = 4
MOE_FLAG_DIRECT_TILES = 8
MOE_FLAG_RING_POOL = 16
MOE_FLAG_TEST_NO_WAIT = 256
MOE_FLAG_TEST_SMALL_GRID = 512
MOE_RECIPE_FP8_BLOCK128 = 0
MOE_RECIPE_MXFP4 = 1

EXPORTED_SYMBOLS = (
    "moe_plan_create", "moe_plan_destroy", "moe_plan_info", "moe_workspace_bytes",
    "moe_workspace_layout", "moe_forward", "moe_forward_timed", "moe_forward_mx",
    "moe_forward_mx_timed", "moe_forward_noalloc", "moe_route",
    "moe_route_workspace_bytes", "moe_prepare_weights", "moe_prepare_weights_mx",
    "moe_quantize_act",
    "moe_read_status", "moe_strerror", "moe_version",
)


class MoEError(RuntimeError):
    def __init__(self, code, what=""):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


class moe_shape_t(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("recipe", ctypes.c_int32), ("act_sf_gran", ctypes.c_int32),
                ("activation_clamp", ctypes.c_float)]


class moe_tile_info_t(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int32), ("row_align", ctypes.c_int32),
                ("pool_rows", ctypes.c_int32), ("l1_tile_n", ctypes.c_int32),
                ("l2_tile_n", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("l1_split", ctypes.c_int32), ("single_launch", ctypes.c_int32),
                ("l2_group_tiles", ctypes.c_int32), ("act_sf_gran", ctypes.c_int32),
                ("l2_split", ctypes.c_int32),
                ("ring_blocks", ctypes.c_int32), ("l2_lag_units", ctypes.c_int32)]


class moe_ws_layout_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("counts", "offsets", "row_src", "src_row", "h", "h_sf", "partial",
                 "status", "total")]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


def lib():
    """Load libmoe_fp8.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m fp8_grouped_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_plan_create.argtypes = [ctypes.POINTER(moe_shape_t), ctypes.POINTER(_vp)]
        L.moe_plan_destroy.argtypes = [_vp]
        L.moe_plan_info.argtypes = [_vp, _i32, ctypes.POINTER(moe_tile_info_t)]
        L.moe_workspace_bytes.argtypes = [_vp, _i32, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_workspace_layout.argtypes = [_vp, _i32, ctypes.POINTER(moe_ws_layout_t)]
        L.moe_forward.argtypes = [_vp, _i32] + [_vp] * 10 + [ctypes.c_size_t, _vp]
        L.moe_forward_timed.argtypes = [_vp, _i32] + [_vp] * 10 + [ctypes.c_size_t, _vp,
                                                                   ctypes.POINTER(_vp)]
        L.moe_forward_noalloc.argtypes = [_vp, _i32] + [_vp] * 10
        L.moe_forward_mx.argtypes = L.moe_forward.argtypes
        L.moe_forward_mx_timed.argtypes = L.moe_forward_timed.argtypes
        L.moe_route.argtypes = ([_vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp,
                                 ctypes.c_size_t, _vp])
        L.moe_route_workspace_bytes.argtypes = [_vp, _i32, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_prepare_weights.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_prepare_weights_mx.argtypes = [_vp] * 10
        L.moe_quantize_act.argtypes = [_vp, _i32, _vp, _vp, _vp, _vp]
        L.moe_read_status.argtypes = [_vp, _i32, _vp, ctypes.c_size_t,
                                      ctypes.POINTER(ctypes.c_int32), _vp]
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        for name in EXPORTED_SYMBOLS:
            if name not in ("moe_strerror",):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    try:
        return lib().moe_strerror(int(code)).decode()
    except ImportError:
        return "library not built"


def _check(rc, what):
    if rc != MOE_OK:
        raise MoEError(rc, what)


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# --- the C ABI, one Python function per entry point -----------------------

def moe_plan_create(hidden, intermediate, num_experts, top_k, max_tokens, tile_m=0,
                    weight_layout=MOE_WEIGHTS_ROW_MAJOR, flags=0,
                    recipe=MOE_RECIPE_FP8_BLOCK128, act_sf_gran=0, activation_clamp=0.0):
    shape = moe_shape_t(hidden, intermediate, num_experts, top_k, max_tokens, tile_m,
                        weight_layout, flags, recipe, act_sf_gran, activation_clamp)
    h = ctypes.c_void_p()
    _check(lib().moe_plan_create(ctypes.byref(shape), ctypes.byref(h)), "moe_plan_create")
    return h


def moe_plan_destroy(plan):
    _check(lib().moe_plan_destroy(plan), "moe_plan_destroy")


def moe_plan_info(plan, num_tokens):
    info = moe_tile_info_t()
    _check(lib().moe_plan_info(plan, num_tokens, ctypes.byref(info)), "moe_plan_info")
    return {f: getattr(info, f) for f, _ in moe_tile_info_t._fields_}


def moe_workspace_bytes(plan, num_tokens):
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_bytes(plan, num_tokens, ctypes.byref(n)), "moe_workspace_bytes")
    return n.value


def moe_workspace_layout(plan, num_tokens):
    lay = moe_ws_layout_t()
    _check(lib().moe_workspace_layout(plan, num_tokens, ctypes.byref(lay)), "moe_workspace_layout")
    return {f: getattr(lay, f) for f, _ in moe_ws_layout_t._fields_}


def moe_forward(plan, num_tokens, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y,
                workspace, stream=None):
    """All tensors are device tensors (see include/moe_fp8.h for layouts)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().moe_forward(plan, num_tokens, _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                           _ptr(topk_w), _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                           _ptr(y), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "moe_forward")


def moe_forward_timed(plan, num_tokens, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y,
                      workspace, stream, step_events):
    """moe_forward that also records step_events (5 torch.cuda.Event, or None
    entries) on `stream` before the planner and after each step.  The events
    must already exist (torch creates them on their first record())."""
    ws_bytes = workspace.numel() * workspace.element_size()
    ev = (_vp * 5)()
    for i, e in enumerate(step_events):
        if e is not None and not e.cuda_event:
            raise ValueError("step event has no HIP event yet: record() it once first")
        ev[i] = None if e is None else e.cuda_event
    rc = lib().moe_forward_timed(plan, num_tokens, _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                                 _ptr(topk_w), _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                                 _ptr(y), _ptr(workspace), ws_bytes, _stream(stream), ev)
    _check(rc, "moe_forward_timed")


MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_forward_noalloc(plan, num_tokens, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y,
                        stream=None):
    """moe_forward with the library's static per-GPU scratch instead of a
    workspace (no device allocation; calls overlapping on one GPU race)."""
    rc = lib().moe_forward_noalloc(plan, num_tokens, _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                                   _ptr(topk_w), _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                                   _ptr(y), _stream(stream))
    _check(rc, "moe_forward_noalloc")


def moe_forward_mx(plan, num_tokens, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y,
                   workspace, stream=None):
    """FP8 x MXFP4 forward: UE8M0 scale codes (uint8) and packed e2m1 weights."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().moe_forward_mx(plan, num_tokens, _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                              _ptr(topk_w), _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                              _ptr(y), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "moe_forward_mx")


def moe_forward_mx_timed(plan, num_tokens, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y,
                         workspace, stream, step_events):
    ws_bytes = workspace.numel() * workspace.element_size()
    ev = (_vp * 5)()
    for i, e in enumerate(step_events):
        if e is not None and not e.cuda_event:
            raise ValueError("step event has no HIP event yet: record() it once first")
        ev[i] = None if e is None else e.cuda_event
    rc = lib().moe_forward_mx_timed(plan, num_tokens, _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                                    _ptr(topk_w), _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                                    _ptr(y), _ptr(workspace), ws_bytes, _stream(stream), ev)
    _check(rc, "moe_forward_mx_timed")


def moe_prepare_weights(plan, w1, w2, w1_packed, w2_packed, stream=None):
    """Write the packed (MFMA operand order) copies of w1/w2 for a packed plan."""
    rc = lib().moe_prepare_weights(plan, _ptr(w1), _ptr(w2), _ptr(w1_packed), _ptr(w2_packed),
                                   _stream(stream))
    _check(rc, "moe_prepare_weights")


def moe_prepare_weights_mx(plan, w1, w1_sf, w2, w2_sf, w1_packed, w1_sf_packed, w2_packed,
                           w2_sf_packed, stream=None):
    """Packed copies of MXFP4 weights and their scale codes for a packed MXFP4 plan."""
    rc = lib().moe_prepare_weights_mx(plan, _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf),
                                      _ptr(w1_packed), _ptr(w1_sf_packed), _ptr(w2_packed),
                                      _ptr(w2_sf_packed), _stream(stream))
    _check(rc, "moe_prepare_weights_mx")


def moe_quantize_act(plan, num_tokens, x_bf16, x, x_sf, stream=None):
    """bf16 activations -> e4m3 codes + scales for the plan's recipe."""
    rc = lib().moe_quantize_act(plan, num_tokens, _ptr(x_bf16), _ptr(x), _ptr(x_sf),
                                _stream(stream))
    _check(rc, "moe_quantize_act")


def moe_route_workspace_bytes(plan, num_tokens):
    n = ctypes.c_size_t()
    _check(lib().moe_route_workspace_bytes(plan, num_tokens, ctypes.byref(n)),
           "moe_route_workspace_bytes")
    return n.value


def moe_route(plan, num_tokens, topk_idx, row_align, counts, offsets, row_src, src_row,
              workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().moe_route(plan, num_tokens, _ptr(topk_idx), row_align, _ptr(counts),
                         _ptr(offsets), _ptr(row_src), row_src.numel(), _ptr(src_row),
                         _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "moe_route")


def moe_read_status(plan, num_tokens, workspace, stream=None):
    out = (ctypes.c_int32 * 4)()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_read_status(plan, num_tokens, _ptr(workspace), ws_bytes, out,
                                 _stream(stream)), "moe_read_status")
    return list(out)


# --- convenience wrapper ---------------------------------------------------

class MoEForward:
    """Plan + workspace holder.  forward() writes y for T tokens."""

    def __init__(self, hidden, intermediate, num_experts, top_k, max_tokens, tile_m=0,
                 device="cuda", weight_layout=MOE_WEIGHTS_ROW_MAJOR, flags=0,
                 recipe=MOE_RECIPE_FP8_BLOCK128, act_sf_gran=0, activation_clamp=0.0):
        import torch
        self.shape = (hidden, intermediate, num_experts, top_k, max_tokens, tile_m)
        self.weight_layout = weight_layout
        self.recipe = recipe
        self.plan = moe_plan_create(hidden, intermediate, num_experts, top_k, max_tokens,
                                    tile_m, weight_layout, flags, recipe, act_sf_gran,
                                    activation_clamp)
        self.ws_bytes = moe_workspace_bytes(self.plan, max_tokens)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def prepare(self, w1, w2, stream=None):
        """Packed copies of w1/w2 for this plan (identity for row-major plans)."""
        import torch
        if self.weight_layout != MOE_WEIGHTS_PACKED:
            return w1, w2
        p1 = torch.empty_like(w1)
        p2 = torch.empty_like(w2)
        moe_prepare_weights(self.plan, w1, w2, p1, p2, stream)
        return p1, p2

    def prepare_mx(self, w1, w1_sf, w2, w2_sf, stream=None):
        """Packed copies of MXFP4 weights and scales (identity for row-major plans)."""
        import torch
        if self.weight_layout != MOE_WEIGHTS_PACKED:
            return w1, w1_sf, w2, w2_sf
        out = [torch.empty_like(t) for t in (w1, w1_sf, w2, w2_sf)]
        moe_prepare_weights_mx(self.plan, w1, w1_sf, w2, w2_sf, *out, stream=stream)
        return tuple(out)

    def forward(self, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y=None, stream=None):
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty(T, self.shape[0], dtype=torch.uint16, device=x.device)
        fwd = moe_forward_mx if self.recipe == MOE_RECIPE_MXFP4 else moe_forward
        fwd(self.plan, T, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y,
            self.workspace, stream)
        return y

    def view(self, name, num_tokens):
        """A typed view of one workspace section after a forward of num_tokens."""
        import torch
        lay = moe_workspace_layout(self.plan, num_tokens)
        info = moe_plan_info(self.plan, num_tokens)
        H, I, E, K = self.shape[:4]
        R = info["pool_rows"]
        # ring-pool calls: h / h_sf hold ring_blocks row blocks
        HR = info["ring_blocks"] * info["tile_m"] if info["ring_blocks"] > 0 else R
        spec = {
            "counts": (torch.int32, (E,)),
            "offsets": (torch.int32, (E + 1,)),
            "row_src": (torch.int32, (R,)),
            "src_row": (torch.int32, (num_tokens * K,)),
            "h": (torch.uint8, (HR, I)),
            "h_sf": ((torch.uint8, (HR, I // 32)) if self.recipe == MOE_RECIPE_MXFP4
                     else (torch.float32, (HR, I // info["act_sf_gran"]))),
            "partial": (torch.int16, (K, num_tokens, H)),
            "status": (torch.int32, (4,)),
        }[name]
        dt, shp = spec
        n = 1
        for s in shp:
            n *= s
        nbytes = n * torch.tensor([], dtype=dt).element_size()
        raw = self.workspace[lay[name]:lay[name] + nbytes]
        return raw.view(dt).view(shp)

    def close(self):
        if self.plan is not None:
            moe_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
