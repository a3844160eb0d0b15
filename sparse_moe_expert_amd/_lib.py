"""ctypes binding to libsparse_moe_expert_amd.so (argument marshalling only).

Every step of the routed-MoE path runs in the HIP library; this module checks
tensor dtypes, devices and contiguity, passes data pointers and torch's
current HIP stream, and turns status codes into exceptions.  There is no
fallback: if the library is missing the import of a call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libsparse_moe_expert_amd.so")

MOE_STATUS = {
    0: "MOE_OK",
    1: "MOE_ERR_NULL_POINTER",
    2: "MOE_ERR_INVALID_SHAPE",
    3: "MOE_ERR_UNSUPPORTED",
    4: "MOE_ERR_MISALIGNED",
    5: "MOE_ERR_WORKSPACE_TOO_SMALL",
    6: "MOE_ERR_HIP",
    7: "MOE_ERR_SCRATCH_TOO_SMALL",
}

# Exported C symbols and their ctypes signatures.
_P = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "moe_router_logits": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "moe_route_topk": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "moe_bucket_routes": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "moe_route_bucket": (_I, [_P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_router_route_bucket": (_I, [_P, _P, _P] + [_I] * 4 + [_P] * 11),
    "moe_expert_ffn_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "moe_expert_ffn": (_I, [_P] * 15 + [_I] * 5 + [_P, ctypes.c_size_t, _P, _P]),
    "moe_expert_ffn_stage": (_I, [_I] + [_P] * 15 + [_I] * 5 + [_P, ctypes.c_size_t, _P, _P]),
    "moe_step_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "moe_step": (_I, [_P, _P, _P] + [_P] * 7 + [_I] * 5 + [_P] * 8 + [_P, ctypes.c_size_t, _P, _P]),
    "moe_step_stage": (_I, [_I, _P, _P, _P] + [_P] * 7 + [_P] + [_I] * 5 + [_P] * 8 + [_P, ctypes.c_size_t, _P, _P]),
    "moe_packed_weights_size": (ctypes.c_size_t, [_I, _I, _I]),
    "moe_pack_weights": (_I, [_P] * 6 + [_I] * 3 + [_P, _P]),
    "moe_step_packed": (_I, [_P, _P, _P] + [_P] * 7 + [_P] + [_I] * 5 + [_P] * 8 + [_P, ctypes.c_size_t, _P, _P]),
    "moe_shared_expert_workspace_size": (ctypes.c_size_t, [_I, _I, _I]),
    "moe_shared_expert": (_I, [_P] * 4 + [_I] * 3 + [_P, ctypes.c_size_t, _P, _P]),
    "moe_step_shared": (_I, [_P, _P, _P] + [_P] * 7 + [_P] + [_I] * 5 + [_P] * 8 + [_P, ctypes.c_size_t, _P]
                        + [_P] * 3 + [_I, _P, ctypes.c_size_t, _P, _P]),
    "moe_expert_ffn_per_route": (_I, [_P] * 10 + [_I] * 5 + [_P, ctypes.c_size_t, _P, _P]),
    "moe_step_noalloc": (_I, [_P, _P, _P] + [_P] * 7 + [_P] + [_I] * 5 + [_P] * 8 + [_P, _P]),
    "moe_status_string": (ctypes.c_char_p, [_I]),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {MOE_STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build it with `python -m sparse_moe_expert_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        msg = load_library().moe_status_string(status).decode()
        raise MoeError(fn, status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def moe_router_logits(x: torch.Tensor, w_router: torch.Tensor,
                      logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Router logits fp32 [T,E] = fl32(x @ w_router^T) from bf16 x [T,H] (or its
    uint16 bits) and fp32 w_router [E,H], summed in fp64 on the GPU."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    x = _check_x(x)
    _need(w_router, "w_router", torch.float32, (E, H), dev)
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    _need(logits, "logits", torch.float32, (T, E), dev)
    st = load_library().moe_router_logits(_ptr(x), _ptr(w_router), T, H, E, _ptr(logits), _stream(dev))
    _check("moe_router_logits", st)
    return logits


def moe_shared_expert(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                      y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The dense shared expert: bf16 y [T,H] = W_down (SiLU(W_gate x) * (W_up x))
    for every token, bf16 weights w_gate/w_up [Is,H] and w_down [H,Is]."""
    T, H = x.shape
    Is = w_gate.shape[0]
    dev = x.device
    x = _check_x(x)
    for t, name, shape in ((w_gate, "w_gate", (Is, H)), (w_up, "w_up", (Is, H)), (w_down, "w_down", (H, Is))):
        _need(t, name, torch.bfloat16, shape, dev)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, (T, H), dev)
    lib = load_library()
    ws_bytes = lib.moe_shared_expert_workspace_size(T, H, Is)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    st = lib.moe_shared_expert(_ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), T, H, Is, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(y), _stream(dev))
    _check("moe_shared_expert", st)
    return y


def moe_route_topk(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                   topk_idx: Optional[torch.Tensor] = None,
                   topk_w: Optional[torch.Tensor] = None):
    """Top-k expert ids (int32 [T,k]) and renormalised weights (fp32 [T,k])."""
    T, E = logits.shape
    dev = logits.device
    _need(logits, "logits", torch.float32)
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    st = load_library().moe_route_topk(_ptr(logits), _ptr(bias), T, E, k, _ptr(topk_idx),
                                       _ptr(topk_w), _stream(dev))
    _check("moe_route_topk", st)
    return topk_idx, topk_w


class Buckets(NamedTuple):
    expert_count: torch.Tensor    # int32 [E]
    expert_offset: torch.Tensor   # int32 [E+1]
    active_experts: torch.Tensor  # int32 [E]
    n_active: torch.Tensor        # int32 [1]
    route_src: torch.Tensor       # int32 [R]
    route_pos: torch.Tensor       # int32 [R]


def empty_buckets(T: int, E: int, k: int, device) -> Buckets:
    R = T * k
    mk = lambda n: torch.empty((n,), dtype=torch.int32, device=device)  # noqa: E731
    return Buckets(mk(E), mk(E + 1), mk(E), mk(1), mk(R), mk(R))


def moe_bucket_routes(topk_idx: torch.Tensor, E: int, out: Optional[Buckets] = None) -> Buckets:
    """Routes grouped by expert, stable in flat route id t*k+j."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    _need(topk_idx, "topk_idx", torch.int32)
    b = out if out is not None else empty_buckets(T, E, k, dev)
    for name, t, n in zip(Buckets._fields, b, (E, E + 1, E, 1, T * k, T * k)):
        _need(t, name, torch.int32, (n,), dev)
    st = load_library().moe_bucket_routes(_ptr(topk_idx), T, E, k, *(_ptr(t) for t in b),
                                          _stream(dev))
    _check("moe_bucket_routes", st)
    return b


def moe_route_bucket(logits: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                     topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
                     out: Optional[Buckets] = None):
    """moe_route_topk and moe_bucket_routes in one call (one kernel for T <= 64)."""
    T, E = logits.shape
    dev = logits.device
    _need(logits, "logits", torch.float32)
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    b = out if out is not None else empty_buckets(T, E, k, dev)
    for name, t, n in zip(Buckets._fields, b, (E, E + 1, E, 1, T * k, T * k)):
        _need(t, name, torch.int32, (n,), dev)
    st = load_library().moe_route_bucket(_ptr(logits), _ptr(bias), T, E, k, _ptr(topk_idx), _ptr(topk_w),
                                         *(_ptr(t) for t in b), _stream(dev))
    _check("moe_route_bucket", st)
    return topk_idx, topk_w, b


def moe_router_route_bucket(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor], k: int,
                            logits: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                            buckets: "Buckets", counter: torch.Tensor) -> None:
    """Router projection, top-k and buckets in one call (one launch for small
    batches); `counter` is an int32 [1] device tensor, zero before the first
    call and left zero by every call."""
    x = _check_x(x)
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    _need(w_router, "w_router", torch.float32, (E, H), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), dev)
    _need(logits, "logits", torch.float32, (T, E), dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    for name, t, n in zip(Buckets._fields, buckets, (E, E + 1, E, 1, T * k, T * k)):
        _need(t, name, torch.int32, (n,), dev)
    _need(counter, "counter", torch.int32, (1,), dev)
    st = load_library().moe_router_route_bucket(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, _ptr(logits),
                                                _ptr(topk_idx), _ptr(topk_w), *(_ptr(t) for t in buckets),
                                                _ptr(counter), _stream(dev))
    _check("moe_router_route_bucket", st)


class ExpertWeights(NamedTuple):
    w_gate: torch.Tensor   # uint8 [E, I, H/2]
    s_gate: torch.Tensor   # uint8 [E, I, H/16]
    w_up: torch.Tensor     # uint8 [E, I, H/2]
    s_up: torch.Tensor     # uint8 [E, I, H/16]
    w_down: torch.Tensor   # uint8 [E, H, I/2]
    s_down: torch.Tensor   # uint8 [E, H, I/16]
    g_scale: torch.Tensor  # fp32  [E, 3]

    @property
    def shape(self):
        E, I, H2 = self.w_gate.shape
        return E, 2 * H2, I


def moe_expert_ffn_workspace_size(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(load_library().moe_expert_ffn_workspace_size(T, H, I, E, k))


def make_workspace(T: int, H: int, I: int, E: int, k: int, device) -> torch.Tensor:
    """Workspace of the size moe_expert_ffn needs (reusable across calls)."""
    n = max(moe_expert_ffn_workspace_size(T, H, I, E, k), 256)
    return torch.empty((n,), dtype=torch.uint8, device=device)


def moe_expert_ffn(x: torch.Tensor, weights: ExpertWeights, topk_w: torch.Tensor,
                   buckets: Buckets, workspace: torch.Tensor,
                   y: Optional[torch.Tensor] = None, stage: int = 3) -> torch.Tensor:
    """bf16 [T,H] output of the routed experts.  x is bf16 [T,H] (or its uint16 bits).

    stage 3 runs the whole FFN; 1 runs only gate/up (h stays in the workspace);
    2 runs only down + unroute on the workspace's h."""
    T, H = x.shape
    E, H_w, I = weights.shape
    k = topk_w.shape[1]
    dev = x.device
    x = _check_x(x)
    if H_w != H:
        raise ValueError(f"weights are for H={H_w}, x has H={H}")
    shapes = [(E, I, H // 2), (E, I, H // 16), (E, I, H // 2), (E, I, H // 16),
              (E, H, I // 2), (E, H, I // 16)]
    for name, t, shp in zip(ExpertWeights._fields, weights, shapes):
        _need(t, name, torch.uint8, shp, dev)
    _need(weights.g_scale, "g_scale", torch.float32, (E, 3), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if y.dtype != torch.bfloat16 or tuple(y.shape) != (T, H) or not y.is_contiguous() or y.device != dev:
        raise ValueError("y must be a contiguous bfloat16 [T, H] tensor on x's device")
    args = (_ptr(x), *(_ptr(t) for t in weights), _ptr(topk_w), *(_ptr(t) for t in buckets),
            T, H, I, E, k, _ptr(workspace), ctypes.c_size_t(workspace.numel()), _ptr(y), _stream(dev))
    if stage == 3:
        st = load_library().moe_expert_ffn(*args)
        _check("moe_expert_ffn", st)
    else:
        st = load_library().moe_expert_ffn_stage(stage, *args)
        _check("moe_expert_ffn_stage", st)
    return y


def _check_x(x: torch.Tensor) -> torch.Tensor:
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    if x.dtype not in (torch.int16, torch.uint16):
        raise TypeError("x must be bfloat16 (or its 16-bit patterns)")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    return x


def moe_step_workspace_size(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(load_library().moe_step_workspace_size(T, H, I, E, k))


def moe_packed_weights_size(E: int, H: int, I: int) -> int:
    return int(load_library().moe_packed_weights_size(E, H, I))


def pack_weights(weights: ExpertWeights) -> torch.Tensor:
    """The weights in MFMA tile order (moe_pack_weights), for moe_step(..., packed=)."""
    E, H, I = weights.shape
    n = moe_packed_weights_size(E, H, I)
    if n == 0:
        raise ValueError(f"packed weights need H and I multiples of 64 (H={H}, I={I})")
    dev = weights.w_gate.device
    packed = torch.empty((n,), dtype=torch.uint8, device=dev)
    st = load_library().moe_pack_weights(*(_ptr(t) for t in weights[:6]), E, H, I, _ptr(packed), _stream(dev))
    _check("moe_pack_weights", st)
    return packed


def moe_step(x: torch.Tensor, logits: torch.Tensor, bias: Optional[torch.Tensor], weights: ExpertWeights,
             k: int, topk_idx: torch.Tensor, topk_w: torch.Tensor, buckets: Buckets,
             workspace: torch.Tensor, y: torch.Tensor, packed: Optional[torch.Tensor] = None,
             stage: int = 3) -> torch.Tensor:
    """One whole step (route, bucket, expert FFN) in one call; fills every output.  With `packed`
    (from pack_weights of the same weights) it runs moe_step_packed.  stage 1 or 2 runs one part
    of it (moe_step_stage)."""
    x = _check_x(x)
    T, H = x.shape
    E, H_w, I = weights.shape
    dev = x.device
    if H_w != H:
        raise ValueError(f"weights are for H={H_w}, x has H={H}")
    _need(logits, "logits", torch.float32, (T, E), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), dev)
    shapes = [(E, I, H // 2), (E, I, H // 16), (E, I, H // 2), (E, I, H // 16),
              (E, H, I // 2), (E, H, I // 16)]
    for name, t, shp in zip(ExpertWeights._fields, weights, shapes):
        _need(t, name, torch.uint8, shp, dev)
    _need(weights.g_scale, "g_scale", torch.float32, (E, 3), dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    for name, t, n in zip(Buckets._fields, buckets, (E, E + 1, E, 1, T * k, T * k)):
        _need(t, name, torch.int32, (n,), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    if y.dtype != torch.bfloat16 or tuple(y.shape) != (T, H) or not y.is_contiguous() or y.device != dev:
        raise ValueError("y must be a contiguous bfloat16 [T, H] tensor on x's device")
    if stage != 3:
        if packed is not None:
            _need(packed, "packed", torch.uint8, (moe_packed_weights_size(E, H, I),), dev)
        st = load_library().moe_step_stage(stage, _ptr(x), _ptr(logits), _ptr(bias), *(_ptr(t) for t in weights),
                                           _ptr(packed), T, H, I, E, k, _ptr(topk_idx), _ptr(topk_w),
                                           *(_ptr(t) for t in buckets), _ptr(workspace),
                                           ctypes.c_size_t(workspace.numel()), _ptr(y), _stream(dev))
        _check("moe_step_stage", st)
        return y
    if packed is None:
        st = load_library().moe_step(_ptr(x), _ptr(logits), _ptr(bias), *(_ptr(t) for t in weights),
                                     T, H, I, E, k, _ptr(topk_idx), _ptr(topk_w), *(_ptr(t) for t in buckets),
                                     _ptr(workspace), ctypes.c_size_t(workspace.numel()), _ptr(y), _stream(dev))
        _check("moe_step", st)
        return y
    _need(packed, "packed", torch.uint8, (moe_packed_weights_size(E, H, I),), dev)
    st = load_library().moe_step_packed(_ptr(x), _ptr(logits), _ptr(bias), *(_ptr(t) for t in weights),
                                        _ptr(packed), T, H, I, E, k, _ptr(topk_idx), _ptr(topk_w),
                                        *(_ptr(t) for t in buckets), _ptr(workspace),
                                        ctypes.c_size_t(workspace.numel()), _ptr(y), _stream(dev))
    _check("moe_step_packed", st)
    return y


def moe_expert_ffn_per_route(x: torch.Tensor, weights: ExpertWeights, topk_idx: torch.Tensor,
                             topk_w: torch.Tensor, workspace: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """The expert FFN without unique-expert reuse (every route streams its own
    expert's weights): the baseline beside moe_expert_ffn."""
    x = _check_x(x)
    T, H = x.shape
    E, H_w, I = weights.shape
    dev = x.device
    if H_w != H:
        raise ValueError(f"weights are for H={H_w}, x has H={H}")
    k = topk_idx.shape[1]
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need(y, "y", torch.bfloat16, (T, H), dev)
    st = load_library().moe_expert_ffn_per_route(_ptr(x), *(_ptr(t) for t in weights), _ptr(topk_idx), _ptr(topk_w),
                                                 T, H, I, E, k, _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                                 _ptr(y), _stream(dev))
    _check("moe_expert_ffn_per_route", st)
    return y


NOALLOC_SCRATCH_BYTES = 8 << 20    # MOE_NOALLOC_SCRATCH_BYTES


def moe_step_noalloc(x: torch.Tensor, logits: torch.Tensor, bias: Optional[torch.Tensor], weights: ExpertWeights,
                     k: int, topk_idx: torch.Tensor, topk_w: torch.Tensor, buckets: Buckets, y: torch.Tensor,
                     packed: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_step (moe_step_packed with `packed`) with the library's static
    scratch as its workspace: no workspace argument, nothing allocated."""
    x = _check_x(x)
    T, H = x.shape
    E, H_w, I = weights.shape
    dev = x.device
    if H_w != H:
        raise ValueError(f"weights are for H={H_w}, x has H={H}")
    _need(logits, "logits", torch.float32, (T, E), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), dev)
    shapes = [(E, I, H // 2), (E, I, H // 16), (E, I, H // 2), (E, I, H // 16),
              (E, H, I // 2), (E, H, I // 16)]
    for name, t, shp in zip(ExpertWeights._fields, weights, shapes):
        _need(t, name, torch.uint8, shp, dev)
    _need(weights.g_scale, "g_scale", torch.float32, (E, 3), dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    for name, t, n in zip(Buckets._fields, buckets, (E, E + 1, E, 1, T * k, T * k)):
        _need(t, name, torch.int32, (n,), dev)
    _need(y, "y", torch.bfloat16, (T, H), dev)
    if packed is not None:
        _need(packed, "packed", torch.uint8, (moe_packed_weights_size(E, H, I),), dev)
    st = load_library().moe_step_noalloc(_ptr(x), _ptr(logits), _ptr(bias), *(_ptr(t) for t in weights),
                                         _ptr(packed), T, H, I, E, k, _ptr(topk_idx), _ptr(topk_w),
                                         *(_ptr(t) for t in buckets), _ptr(y), _stream(dev))
    _check("moe_step_noalloc", st)
    return y


def moe_step_shared(x: torch.Tensor, logits: torch.Tensor, bias: Optional[torch.Tensor], weights: ExpertWeights,
                    k: int, topk_idx: torch.Tensor, topk_w: torch.Tensor, buckets: Buckets,
                    workspace: torch.Tensor, y: torch.Tensor, shared: tuple, y_shared: torch.Tensor,
                    se_workspace: torch.Tensor, packed: Optional[torch.Tensor] = None) -> tuple:
    """moe_step (moe_step_packed with `packed`) and the dense shared expert
    `shared` = (w_gate [Is,H], w_up [Is,H], w_down [H,Is], bf16) of the same
    tokens in one call: y = the routed output, y_shared = the shared expert's."""
    x = _check_x(x)
    T, H = x.shape
    E, H_w, I = weights.shape
    dev = x.device
    if H_w != H:
        raise ValueError(f"weights are for H={H_w}, x has H={H}")
    _need(logits, "logits", torch.float32, (T, E), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,), dev)
    shapes = [(E, I, H // 2), (E, I, H // 16), (E, I, H // 2), (E, I, H // 16),
              (E, H, I // 2), (E, H, I // 16)]
    for name, t, shp in zip(ExpertWeights._fields, weights, shapes):
        _need(t, name, torch.uint8, shp, dev)
    _need(weights.g_scale, "g_scale", torch.float32, (E, 3), dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, k), dev)
    _need(topk_w, "topk_w", torch.float32, (T, k), dev)
    for name, t, n in zip(Buckets._fields, buckets, (E, E + 1, E, 1, T * k, T * k)):
        _need(t, name, torch.int32, (n,), dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _need(y, "y", torch.bfloat16, (T, H), dev)
    w_g, w_u, w_d = shared
    Is = w_g.shape[0]
    for t, name, shape in ((w_g, "w_gate", (Is, H)), (w_u, "w_up", (Is, H)), (w_d, "w_down", (H, Is))):
        _need(t, name, torch.bfloat16, shape, dev)
    _need(y_shared, "y_shared", torch.bfloat16, (T, H), dev)
    _need(se_workspace, "se_workspace", torch.uint8, None, dev)
    if packed is not None:
        _need(packed, "packed", torch.uint8, (moe_packed_weights_size(E, H, I),), dev)
    st = load_library().moe_step_shared(_ptr(x), _ptr(logits), _ptr(bias), *(_ptr(t) for t in weights),
                                        _ptr(packed), T, H, I, E, k, _ptr(topk_idx), _ptr(topk_w),
                                        *(_ptr(t) for t in buckets), _ptr(workspace),
                                        ctypes.c_size_t(workspace.numel()), _ptr(y), _ptr(w_g), _ptr(w_u),
                                        _ptr(w_d), Is, _ptr(se_workspace), ctypes.c_size_t(se_workspace.numel()),
                                        _ptr(y_shared), _stream(dev))
    _check("moe_step_shared", st)
    return y, y_shared


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()
