"""ctypes binding of libbeam_moe.so (argument marshalling only).

Every step of the MoE block runs in the library's HIP kernels; this module
checks tensor dtypes, shapes and devices, allocates outputs and the workspace
with torch, and passes raw device pointers plus the current HIP stream.  There
is no fallback: if the library is missing or a call fails, it raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbeam_moe.so")
#: the debug build with the kernels' index checks (include/beam_moe_debug.h)
LIB_CHECKED_PATH = os.path.join(_PKG, "libbeam_moe_checked.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_TOO_LARGE = -5

#: check bits of the debug build (include/beam_moe_debug.h)
CHECK_BITS = {"permute_row": 1 << 0, "plan_capacity": 1 << 1, "plan_rows": 1 << 2,
              "gather_index": 1 << 3, "token_index": 1 << 4, "weight_offset": 1 << 5,
              "combine_row": 1 << 6}

ENTRY_ROUTE = 0
ENTRY_PERMUTE = 1
ENTRY_EXPERT_FFN = 2
ENTRY_LAYER = 3
ENTRY_EXPERT_STAGE = 4
ENTRY_EXPERT_FFN_LORA = 5
ENTRY_LAYER_LORA = 6

LAYOUT_ROW_MAJOR = 0
LAYOUT_PACKED = 1
LAYOUT_FP8_PACKED = 2

#: Every symbol include/beam_moe.h declares.
EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_route_replay", "moe_permute",
           "moe_expert_ffn", "moe_expert_gate_up", "moe_expert_down", "moe_combine",
           "moe_layer_forward", "moe_pack_weights", "moe_quantize_fp8", "moe_expert_ffn_fp8",
           "moe_expert_gate_up_fp8", "moe_expert_down_fp8", "moe_layer_forward_fp8",
           "moe_expert_ffn_lora", "moe_layer_forward_lora", "moe_layer_forward_noalloc",
           "moe_debug_check_flags", "moe_status_string")


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("topk_groups", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("routed_scaling", ctypes.c_float),
        ("weight_layout", ctypes.c_int32),
    ]


class MoeLora(ctypes.Structure):
    _fields_ = [
        ("a_gate_up", ctypes.c_void_p),
        ("b_gate_up", ctypes.c_void_p),
        ("a_down", ctypes.c_void_p),
        ("b_down", ctypes.c_void_p),
        ("rank", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {status_string(code)} ({code})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """Loads one build of the library (normal or checked) with its argument
    types declared (raises if it is missing)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m grouped_top_routing_amd.build`")
    L = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    CP = ctypes.POINTER(MoeConfig)
    L.moe_workspace_bytes.argtypes = [CP, I, ctypes.POINTER(Z)]
    L.moe_route.argtypes = [CP, P, P, P, P, P, P, Z, P]
    L.moe_route_replay.argtypes = [CP, P, P, P, P, P, Z, P]
    L.moe_permute.argtypes = [CP, P, P, P, P, P, P, Z, P]
    L.moe_expert_ffn.argtypes = [CP, P, P, P, P, P, P, P, Z, P]
    L.moe_expert_gate_up.argtypes = [CP, P, P, P, P, P, P, Z, P]
    L.moe_expert_down.argtypes = [CP, P, P, P, P, P, Z, P]
    L.moe_combine.argtypes = [CP, P, P, P, P, P]
    L.moe_pack_weights.argtypes = [CP, P, P, P, P, P]
    L.moe_layer_forward.argtypes = [CP, P, P, P, P, P, P, P, P, P, Z, P]
    L.moe_layer_forward_noalloc.argtypes = [CP, P, P, P, P, P, P, P, P, P]
    L.moe_quantize_fp8.argtypes = [CP, P, P, P, P, P, P, P]
    L.moe_expert_ffn_fp8.argtypes = [CP, P, P, P, P, P, P, P, P, P, Z, P]
    L.moe_expert_gate_up_fp8.argtypes = [CP, P, P, P, P, P, P, P, Z, P]
    L.moe_expert_down_fp8.argtypes = [CP, P, P, P, P, P, P, Z, P]
    L.moe_layer_forward_fp8.argtypes = [CP, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    LP = ctypes.POINTER(MoeLora)
    L.moe_expert_ffn_lora.argtypes = [CP, P, P, P, P, P, LP, P, P, Z, P]
    L.moe_layer_forward_lora.argtypes = [CP, P, P, P, P, P, LP, P, P, P, P, Z, P]
    L.moe_debug_check_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    L.moe_status_string.argtypes = [I]
    L.moe_status_string.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name != "moe_status_string":
            getattr(L, name).restype = I
    return L


class use_library:
    """Context manager: the binding's calls go to another build of the
    library (e.g. the checked one) inside the block."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = lib()
        _lib = load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def check_flags() -> dict:
    """moe_debug_check_flags of the library in use: {check name: bool} of the
    bits recorded since the last call (the checked build only)."""
    f = ctypes.c_uint32(0)
    _call("moe_debug_check_flags", lib().moe_debug_check_flags(ctypes.byref(f)))
    return {k: bool(f.value & b) for k, b in CHECK_BITS.items()}


def status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()


def make_config(num_tokens, hidden, intermediate, *, num_experts=256, num_groups=8,
                topk_groups=4, topk=8, renormalize=True, routed_scaling=2.5,
                weight_layout=LAYOUT_ROW_MAJOR) -> MoeConfig:
    return MoeConfig(int(num_tokens), int(hidden), int(intermediate), int(num_experts),
                     int(num_groups), int(topk_groups), int(topk), int(bool(renormalize)),
                     float(routed_scaling), int(weight_layout))


def workspace_bytes(cfg: MoeConfig, entry: int) -> int:
    n = ctypes.c_size_t(0)
    st = lib().moe_workspace_bytes(ctypes.byref(cfg), int(entry), ctypes.byref(n))
    if st != MOE_OK:
        raise MoeError(st, "moe_workspace_bytes")
    return int(n.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class Workspace:
    """A reusable device workspace (a torch uint8 buffer grown on demand).

    Calls that share one Workspace must be ordered: issue them on one stream,
    or synchronise between streams yourself.  Each use records the current
    stream on the buffer, so a buffer replaced when the workspace grows is
    not reused by torch's allocator before the work queued on it is done."""

    def __init__(self):
        self._buf = None

    def get(self, nbytes: int, device) -> torch.Tensor | None:
        if nbytes == 0:
            return None
        if self._buf is None or self._buf.numel() < nbytes or self._buf.device != device:
            self._buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self._buf.record_stream(torch.cuda.current_stream(device))
        return self._buf


# default workspaces, one per (device, stream): calls on different streams
# never share scratch memory
_default_ws: dict = {}


def _ws(workspace, device):
    if workspace is None:
        key = (device, torch.cuda.current_stream(device).cuda_stream)
        workspace = _default_ws.setdefault(key, Workspace())
    return workspace


def _call(name, code):
    if code != MOE_OK:
        raise MoeError(code, name)


def route(x, w_router, *, sel_bias=None, num_groups=8, topk_groups=4, topk=8, renormalize=True,
          workspace=None):
    """Router: returns (topk_ids int32 [T, k], topk_w fp32 [T, k])."""
    T, H = x.shape
    E = w_router.shape[0]
    _check(x, "x", torch.bfloat16)
    _check(w_router, "w_router", torch.float32, (E, H), x.device)
    if sel_bias is not None:
        _check(sel_bias, "sel_bias", torch.float32, (E,), x.device)
    cfg = make_config(T, H, 128, num_experts=E, num_groups=num_groups, topk_groups=topk_groups,
                      topk=topk, renormalize=renormalize)
    ids = torch.empty(T, topk, dtype=torch.int32, device=x.device)
    w = torch.empty(T, topk, dtype=torch.float32, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_ROUTE)
    ws = _ws(workspace, x.device).get(nb, x.device)
    _call("moe_route", lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(sel_bias),
                                       _ptr(ids), _ptr(w), _ptr(ws), nb, _stream(x.device)))
    return ids, w


def route_replay(x, w_router, topk_ids, *, renormalize=True, workspace=None):
    """Combine weights for caller-supplied expert ids: fp32 [T, k]."""
    T, H = x.shape
    E = w_router.shape[0]
    k = topk_ids.shape[1]
    _check(x, "x", torch.bfloat16)
    _check(w_router, "w_router", torch.float32, (E, H), x.device)
    _check(topk_ids, "topk_ids", torch.int32, (T, k), x.device)
    cfg = make_config(T, H, 128, num_experts=E, num_groups=1, topk_groups=1, topk=k,
                      renormalize=renormalize)
    w = torch.empty(T, k, dtype=torch.float32, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_ROUTE)
    ws = _ws(workspace, x.device).get(nb, x.device)
    _call("moe_route_replay", lib().moe_route_replay(ctypes.byref(cfg), _ptr(x), _ptr(w_router),
                                                     _ptr(topk_ids), _ptr(w), _ptr(ws), nb,
                                                     _stream(x.device)))
    return w


def permute(topk_ids, *, num_experts=256, workspace=None):
    """Returns (counts [E], offsets [E+1], perm_src [T*k], perm_dst [T*k]), all int32."""
    T, k = topk_ids.shape
    _check(topk_ids, "topk_ids", torch.int32)
    dev = topk_ids.device
    cfg = make_config(T, 256, 128, num_experts=num_experts, num_groups=1, topk_groups=1, topk=k)
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    psrc = torch.empty(T * k, dtype=torch.int32, device=dev)
    pdst = torch.empty(T * k, dtype=torch.int32, device=dev)
    nb = workspace_bytes(cfg, ENTRY_PERMUTE)
    ws = _ws(workspace, dev).get(nb, dev)
    _call("moe_permute", lib().moe_permute(ctypes.byref(cfg), _ptr(topk_ids), _ptr(counts),
                                           _ptr(offsets), _ptr(psrc), _ptr(pdst), _ptr(ws), nb,
                                           _stream(dev)))
    return counts, offsets, psrc, pdst


def expert_ffn(x, perm_src, offsets, w_gate_up, w_down, *, topk=8, weight_layout=LAYOUT_ROW_MAJOR,
               workspace=None):
    """Expert SwiGLU MLPs over the permuted rows: y_perm bf16 [T*k, H]."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    _check(x, "x", torch.bfloat16)
    _check(perm_src, "perm_src", torch.int32, (T * topk,), x.device)
    _check(offsets, "offsets", torch.int32, (E + 1,), x.device)
    _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * I, H), x.device)
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=topk,
                      weight_layout=weight_layout)
    y = torch.empty(T * topk, H, dtype=torch.bfloat16, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_EXPERT_FFN)
    ws = _ws(workspace, x.device).get(nb, x.device)
    _call("moe_expert_ffn", lib().moe_expert_ffn(ctypes.byref(cfg), _ptr(x), _ptr(perm_src),
                                                 _ptr(offsets), _ptr(w_gate_up), _ptr(w_down),
                                                 _ptr(y), _ptr(ws), nb, _stream(x.device)))
    return y


def expert_gate_up(x, perm_src, offsets, w_gate_up, *, topk=8, weight_layout=LAYOUT_ROW_MAJOR,
                   workspace=None):
    """First expert GEMM with the fused SwiGLU: h bf16 [T*k, I]."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    _check(x, "x", torch.bfloat16)
    _check(perm_src, "perm_src", torch.int32, (T * topk,), x.device)
    _check(offsets, "offsets", torch.int32, (E + 1,), x.device)
    _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * I, H), x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=topk,
                      weight_layout=weight_layout)
    h = torch.empty(T * topk, I, dtype=torch.bfloat16, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_EXPERT_STAGE)
    ws = _ws(workspace, x.device).get(nb, x.device)
    _call("moe_expert_gate_up", lib().moe_expert_gate_up(
        ctypes.byref(cfg), _ptr(x), _ptr(perm_src), _ptr(offsets), _ptr(w_gate_up), _ptr(h),
        _ptr(ws), nb, _stream(x.device)))
    return h


def expert_down(h, offsets, w_down, *, topk=8, weight_layout=LAYOUT_ROW_MAJOR, workspace=None):
    """Second expert GEMM: y_perm bf16 [T*k, H]."""
    R, I = h.shape
    E, H, _ = w_down.shape
    T = R // topk
    _check(h, "h", torch.bfloat16, (T * topk, I))
    _check(offsets, "offsets", torch.int32, (E + 1,), h.device)
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), h.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=topk,
                      weight_layout=weight_layout)
    y = torch.empty(T * topk, H, dtype=torch.bfloat16, device=h.device)
    nb = workspace_bytes(cfg, ENTRY_EXPERT_STAGE)
    ws = _ws(workspace, h.device).get(nb, h.device)
    _call("moe_expert_down", lib().moe_expert_down(
        ctypes.byref(cfg), _ptr(h), _ptr(offsets), _ptr(w_down), _ptr(y), _ptr(ws), nb,
        _stream(h.device)))
    return y


def combine(y_perm, perm_dst, topk_w, *, routed_scaling=2.5):
    """Weighted un-permute: out bf16 [T, H]."""
    T, k = topk_w.shape
    H = y_perm.shape[1]
    _check(y_perm, "y_perm", torch.bfloat16)
    _check(perm_dst, "perm_dst", torch.int32, (T * k,), y_perm.device)
    _check(topk_w, "topk_w", torch.float32, (T, k), y_perm.device)
    cfg = make_config(T, H, 128, num_groups=1, topk_groups=1, topk=k,
                      routed_scaling=routed_scaling)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=y_perm.device)
    _call("moe_combine", lib().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(perm_dst),
                                           _ptr(topk_w), _ptr(out), _stream(y_perm.device)))
    return out


def layer_forward(x, w_router, w_gate_up, w_down, *, sel_bias=None, num_groups=8, topk_groups=4,
                  topk=8, renormalize=True, routed_scaling=2.5, weight_layout=LAYOUT_ROW_MAJOR,
                  return_routing=False, out=None, workspace=None):
    """The whole MoE block.  Returns out bf16 [T, H] (and (ids, w) if asked)."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    _check(x, "x", torch.bfloat16)
    _check(w_router, "w_router", torch.float32, (E, H), x.device)
    _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * I, H), x.device)
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), x.device)
    if sel_bias is not None:
        _check(sel_bias, "sel_bias", torch.float32, (E,), x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=num_groups, topk_groups=topk_groups,
                      topk=topk, renormalize=renormalize, routed_scaling=routed_scaling,
                      weight_layout=weight_layout)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    else:
        _check(out, "out", torch.bfloat16, (T, H), x.device)
    ids = w = None
    if return_routing:
        ids = torch.empty(T, topk, dtype=torch.int32, device=x.device)
        w = torch.empty(T, topk, dtype=torch.float32, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_LAYER)
    ws = _ws(workspace, x.device).get(nb, x.device)
    _call("moe_layer_forward",
          lib().moe_layer_forward(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(sel_bias),
                                  _ptr(w_gate_up), _ptr(w_down), _ptr(out), _ptr(ids), _ptr(w),
                                  _ptr(ws), nb, _stream(x.device)))
    return (out, ids, w) if return_routing else out


def layer_forward_noalloc(x, w_router, w_gate_up, w_down, *, sel_bias=None, num_groups=8,
                          topk_groups=4, topk=8, renormalize=True, routed_scaling=2.5,
                          weight_layout=LAYOUT_ROW_MAJOR, out=None, ids=None, w=None):
    """moe_layer_forward_noalloc: the whole block with the library's static
    scratch array instead of a workspace.  ``out`` (bf16 [T, H]) and the
    optional routing outputs ``ids`` (int32 [T, k]) and ``w`` (fp32 [T, k])
    may be passed preallocated; the library call itself allocates nothing.
    Returns out, or (out, ids, w) when ids or w are given."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    _check(x, "x", torch.bfloat16)
    _check(w_router, "w_router", torch.float32, (E, H), x.device)
    _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * I, H), x.device)
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), x.device)
    if sel_bias is not None:
        _check(sel_bias, "sel_bias", torch.float32, (E,), x.device)
    for t, name, dt in ((ids, "ids", torch.int32), (w, "w", torch.float32)):
        if t is not None:
            _check(t, name, dt, (T, topk), x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=num_groups, topk_groups=topk_groups,
                      topk=topk, renormalize=renormalize, routed_scaling=routed_scaling,
                      weight_layout=weight_layout)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    else:
        _check(out, "out", torch.bfloat16, (T, H), x.device)
    _call("moe_layer_forward_noalloc",
          lib().moe_layer_forward_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(w_router),
                                          _ptr(sel_bias), _ptr(w_gate_up), _ptr(w_down),
                                          _ptr(out), _ptr(ids), _ptr(w), _stream(x.device)))
    return out if ids is None and w is None else (out, ids, w)


def pack_weights(w_gate_up=None, w_down=None):
    """Fragment-packed copies of the expert weights (MOE_LAYOUT_PACKED), same
    shapes and dtype as the inputs.  Either argument may be None."""
    ref = w_gate_up if w_gate_up is not None else w_down
    if ref is None:
        raise ValueError("pack_weights: nothing to pack")
    if w_gate_up is not None:
        E, I2, H = w_gate_up.shape
        I = I2 // 2
        _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * I, H))
    if w_down is not None:
        E, H, I = w_down.shape
        _check(w_down, "w_down", torch.bfloat16, (E, H, I), ref.device)
        if w_gate_up is not None and tuple(w_gate_up.shape) != (E, 2 * I, H):
            raise ValueError("w_gate_up and w_down shapes disagree")
    cfg = make_config(0, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=1)
    pgu = torch.empty_like(w_gate_up) if w_gate_up is not None else None
    pd = torch.empty_like(w_down) if w_down is not None else None
    _call("moe_pack_weights", lib().moe_pack_weights(ctypes.byref(cfg), _ptr(w_gate_up),
                                                     _ptr(w_down), _ptr(pgu), _ptr(pd),
                                                     _stream(ref.device)))
    return pgu, pd


# ---------------------------------------------------------------------------
# FP8 (E4M3FN) per-channel expert weights
class Fp8Weights:
    """Quantised expert weights: codes uint8 in the fp8 fragment layout
    (q_gate_up [E, 2I, H], q_down [E, H, I]) and fp32 per-row scales
    (s_gate_up [E, 2I], s_down [E, H])."""

    def __init__(self, q_gate_up, s_gate_up, q_down, s_down):
        self.q_gate_up, self.s_gate_up = q_gate_up, s_gate_up
        self.q_down, self.s_down = q_down, s_down

    @property
    def shape(self):
        """(E, H, I)."""
        E, I2, H = self.q_gate_up.shape
        return E, H, I2 // 2

    def check(self, device):
        E, H, I = self.shape
        _check(self.q_gate_up, "q_gate_up", torch.uint8, (E, 2 * I, H), device)
        _check(self.s_gate_up, "s_gate_up", torch.float32, (E, 2 * I), device)
        _check(self.q_down, "q_down", torch.uint8, (E, H, I), device)
        _check(self.s_down, "s_down", torch.float32, (E, H), device)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.q_gate_up, self.s_gate_up, self.q_down, self.s_down))


def quantize_fp8(w_gate_up, w_down) -> Fp8Weights:
    """Per-channel FP8 quantisation of row-major bf16 expert weights."""
    E, I2, H = w_gate_up.shape
    I = I2 // 2
    _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * I, H))
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), w_gate_up.device)
    dev = w_gate_up.device
    cfg = make_config(0, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=1)
    f = Fp8Weights(torch.empty(E, 2 * I, H, dtype=torch.uint8, device=dev),
                   torch.empty(E, 2 * I, dtype=torch.float32, device=dev),
                   torch.empty(E, H, I, dtype=torch.uint8, device=dev),
                   torch.empty(E, H, dtype=torch.float32, device=dev))
    _call("moe_quantize_fp8", lib().moe_quantize_fp8(
        ctypes.byref(cfg), _ptr(w_gate_up), _ptr(w_down), _ptr(f.q_gate_up), _ptr(f.s_gate_up),
        _ptr(f.q_down), _ptr(f.s_down), _stream(dev)))
    return f


def expert_ffn_fp8(x, perm_src, offsets, w: Fp8Weights, *, topk=8, workspace=None):
    """expert_ffn with FP8 weights: y_perm bf16 [T*k, H]."""
    T, H = x.shape
    E, _, I = w.shape
    _check(x, "x", torch.bfloat16, (T, H))
    w.check(x.device)
    _check(perm_src, "perm_src", torch.int32, (T * topk,), x.device)
    _check(offsets, "offsets", torch.int32, (E + 1,), x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=topk,
                      weight_layout=LAYOUT_FP8_PACKED)
    y = torch.empty(T * topk, H, dtype=torch.bfloat16, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_EXPERT_FFN)
    ws = _ws(workspace, x.device).get(nb, x.device)
    _call("moe_expert_ffn_fp8", lib().moe_expert_ffn_fp8(
        ctypes.byref(cfg), _ptr(x), _ptr(perm_src), _ptr(offsets), _ptr(w.q_gate_up),
        _ptr(w.s_gate_up), _ptr(w.q_down), _ptr(w.s_down), _ptr(y), _ptr(ws), nb,
        _stream(x.device)))
    return y


def expert_gate_up_fp8(x, perm_src, offsets, w: Fp8Weights, *, topk=8, workspace=None):
    """expert_gate_up with FP8 weights: h bf16 [T*k, I]."""
    T, H = x.shape
    E, _, I = w.shape
    _check(x, "x", torch.bfloat16, (T, H))
    w.check(x.device)
    _check(perm_src, "perm_src", torch.int32, (T * topk,), x.device)
    _check(offsets, "offsets", torch.int32, (E + 1,), x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=topk,
                      weight_layout=LAYOUT_FP8_PACKED)
    h = torch.empty(T * topk, I, dtype=torch.bfloat16, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_EXPERT_STAGE)
    ws = _ws(workspace, x.device).get(nb, x.device)
    _call("moe_expert_gate_up_fp8", lib().moe_expert_gate_up_fp8(
        ctypes.byref(cfg), _ptr(x), _ptr(perm_src), _ptr(offsets), _ptr(w.q_gate_up),
        _ptr(w.s_gate_up), _ptr(h), _ptr(ws), nb, _stream(x.device)))
    return h


def expert_down_fp8(h, offsets, w: Fp8Weights, *, topk=8, workspace=None):
    """expert_down with FP8 weights: y_perm bf16 [T*k, H]."""
    R, I = h.shape
    E, H, _ = w.shape
    T = R // topk
    _check(h, "h", torch.bfloat16, (T * topk, I))
    w.check(h.device)
    _check(offsets, "offsets", torch.int32, (E + 1,), h.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=topk,
                      weight_layout=LAYOUT_FP8_PACKED)
    y = torch.empty(T * topk, H, dtype=torch.bfloat16, device=h.device)
    nb = workspace_bytes(cfg, ENTRY_EXPERT_STAGE)
    ws = _ws(workspace, h.device).get(nb, h.device)
    _call("moe_expert_down_fp8", lib().moe_expert_down_fp8(
        ctypes.byref(cfg), _ptr(h), _ptr(offsets), _ptr(w.q_down), _ptr(w.s_down), _ptr(y),
        _ptr(ws), nb, _stream(h.device)))
    return y


def layer_forward_fp8(x, w_router, w: Fp8Weights, *, sel_bias=None, num_groups=8, topk_groups=4,
                      topk=8, renormalize=True, routed_scaling=2.5, return_routing=False,
                      out=None, workspace=None):
    """layer_forward with FP8 expert weights."""
    T, H = x.shape
    E, _, I = w.shape
    _check(x, "x", torch.bfloat16, (T, H))
    _check(w_router, "w_router", torch.float32, (E, H), x.device)
    w.check(x.device)
    if sel_bias is not None:
        _check(sel_bias, "sel_bias", torch.float32, (E,), x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=num_groups, topk_groups=topk_groups,
                      topk=topk, renormalize=renormalize, routed_scaling=routed_scaling,
                      weight_layout=LAYOUT_FP8_PACKED)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    else:
        _check(out, "out", torch.bfloat16, (T, H), x.device)
    ids = tw = None
    if return_routing:
        ids = torch.empty(T, topk, dtype=torch.int32, device=x.device)
        tw = torch.empty(T, topk, dtype=torch.float32, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_LAYER)
    ws = _ws(workspace, x.device).get(nb, x.device)
    _call("moe_layer_forward_fp8", lib().moe_layer_forward_fp8(
        ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(w.q_gate_up),
        _ptr(w.s_gate_up), _ptr(w.q_down), _ptr(w.s_down), _ptr(out), _ptr(ids), _ptr(tw),
        _ptr(ws), nb, _stream(x.device)))
    return (out, ids, tw) if return_routing else out


# ---------------------------------------------------------------------------
# Expert LoRA on the bf16 expert weights
class LoraWeights:
    """One adapter per expert weight: a_gate_up [E, r, H], b_gate_up [E, 2I, r],
    a_down [E, r, I], b_down [E, H, r] (bf16), applied as W a + scale * B (A a)."""

    def __init__(self, a_gate_up, b_gate_up, a_down, b_down, scale):
        self.a_gate_up, self.b_gate_up = a_gate_up, b_gate_up
        self.a_down, self.b_down = a_down, b_down
        self.scale = float(scale)

    @property
    def rank(self):
        return int(self.a_gate_up.shape[1])

    def check(self, E, H, I, device):
        r = self.rank
        _check(self.a_gate_up, "a_gate_up", torch.bfloat16, (E, r, H), device)
        _check(self.b_gate_up, "b_gate_up", torch.bfloat16, (E, 2 * I, r), device)
        _check(self.a_down, "a_down", torch.bfloat16, (E, r, I), device)
        _check(self.b_down, "b_down", torch.bfloat16, (E, H, r), device)

    def struct(self):
        return MoeLora(self.a_gate_up.data_ptr(), self.b_gate_up.data_ptr(),
                       self.a_down.data_ptr(), self.b_down.data_ptr(), self.rank, self.scale)


def expert_ffn_lora(x, perm_src, offsets, w_gate_up, w_down, lora: LoraWeights, *, topk=8,
                    weight_layout=LAYOUT_ROW_MAJOR, workspace=None):
    """expert_ffn with expert LoRA: y_perm bf16 [T*k, H]."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    _check(x, "x", torch.bfloat16)
    _check(perm_src, "perm_src", torch.int32, (T * topk,), x.device)
    _check(offsets, "offsets", torch.int32, (E + 1,), x.device)
    _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * I, H), x.device)
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), x.device)
    lora.check(E, H, I, x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=1, topk_groups=1, topk=topk,
                      weight_layout=weight_layout)
    y = torch.empty(T * topk, H, dtype=torch.bfloat16, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_EXPERT_FFN_LORA)
    ws = _ws(workspace, x.device).get(nb, x.device)
    ls = lora.struct()
    _call("moe_expert_ffn_lora", lib().moe_expert_ffn_lora(
        ctypes.byref(cfg), _ptr(x), _ptr(perm_src), _ptr(offsets), _ptr(w_gate_up), _ptr(w_down),
        ctypes.byref(ls), _ptr(y), _ptr(ws), nb, _stream(x.device)))
    return y


def layer_forward_lora(x, w_router, w_gate_up, w_down, lora: LoraWeights, *, sel_bias=None,
                       num_groups=8, topk_groups=4, topk=8, renormalize=True, routed_scaling=2.5,
                       weight_layout=LAYOUT_ROW_MAJOR, return_routing=False, out=None,
                       workspace=None):
    """layer_forward with expert LoRA."""
    T, H = x.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    _check(x, "x", torch.bfloat16)
    _check(w_router, "w_router", torch.float32, (E, H), x.device)
    _check(w_gate_up, "w_gate_up", torch.bfloat16, (E, 2 * I, H), x.device)
    _check(w_down, "w_down", torch.bfloat16, (E, H, I), x.device)
    lora.check(E, H, I, x.device)
    if sel_bias is not None:
        _check(sel_bias, "sel_bias", torch.float32, (E,), x.device)
    cfg = make_config(T, H, I, num_experts=E, num_groups=num_groups, topk_groups=topk_groups,
                      topk=topk, renormalize=renormalize, routed_scaling=routed_scaling,
                      weight_layout=weight_layout)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    else:
        _check(out, "out", torch.bfloat16, (T, H), x.device)
    ids = tw = None
    if return_routing:
        ids = torch.empty(T, topk, dtype=torch.int32, device=x.device)
        tw = torch.empty(T, topk, dtype=torch.float32, device=x.device)
    nb = workspace_bytes(cfg, ENTRY_LAYER_LORA)
    ws = _ws(workspace, x.device).get(nb, x.device)
    ls = lora.struct()
    _call("moe_layer_forward_lora", lib().moe_layer_forward_lora(
        ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(w_gate_up), _ptr(w_down),
        ctypes.byref(ls), _ptr(out), _ptr(ids), _ptr(tw), _ptr(ws), nb, _stream(x.device)))
    return (out, ids, tw) if return_routing else out
