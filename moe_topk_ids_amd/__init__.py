"""Thin Python binding over the C ABI of ``libmoe_topk_ids.so``.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and torch's current HIP stream are passed
through ctypes, and every step of the computation runs in the library's HIP
kernels. The entry points carry the C names (see include/moe_topk_ids.h for
the contract of each). If the library has not been built the calls raise;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_HIP = -3
MOE_ERR_ALLOC = -4
MOE_ERR_WORKSPACE = -5

FLAG_ATOMIC_COMBINE = 1
FLAG_FORCE_GROUPED = 2
FLAG_FORCE_DECODE = 4
FLAG_DEBUG_SYNC = 8
FLAG_VALIDATE_IDS = 16
FLAG_FORCE_SMALL_BATCH = 32
FLAG_FP8_WEIGHTS = 64
FLAG_BF16_Y = 128
FLAG_FP32_Y = 256
FLAG_NO_TAIL_SPLIT = 512

ACT_SILU = 0
ACT_GELU_TANH = 1
ACT_SWIGLUOAI = 2
ACT_GELU_ERF = 3
ACTIVATIONS = {"silu": ACT_SILU, "gelu_tanh": ACT_GELU_TANH, "swigluoai": ACT_SWIGLUOAI,
               "gelu_erf": ACT_GELU_ERF}

NOALLOC_SCRATCH_BYTES = 128 << 20  # MOE_NOALLOC_SCRATCH_BYTES

PATH_GROUPED = 0
PATH_DECODE = 1
PATH_SMALL_BATCH = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_topk_ids.so")

_lib = None


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


def load_library():
    """Load the HIP library (after torch, so one HIP runtime serves both)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (maps torch's HIP runtime before the library's)

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library missing: {LIB_PATH}; build it with "
                           "`python -m moe_topk_ids_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32, u32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                            ctypes.c_size_t)
    lib.moe_forward.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, p, p]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_ex.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, p, u32, p, sz, p]
    lib.moe_forward_ex.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.moe_forward_act.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32, f32, f32, p, p,
                                    p, u32, p, sz, p]
    lib.moe_forward_act.restype = ctypes.c_int
    lib.moe_forward_fp8.argtypes = [p, p, p, p, p, i64, p, p, i64, i64, i64, i64, i64, i32, f32,
                                    f32, p, p, p, u32, p, sz, p]
    lib.moe_forward_fp8.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, p, u32, p]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, u32]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_m_tile.argtypes = [i64, i64, i64, i64, i64, u32]
    lib.moe_m_tile.restype = i32
    lib.moe_uses_decode_path.argtypes = [i64, i64, i64, i64, i64, u32]
    lib.moe_uses_decode_path.restype = ctypes.c_int
    lib.moe_path.argtypes = [i64, i64, i64, i64, i64, u32]
    lib.moe_path.restype = ctypes.c_int
    lib.moe_y_bf16.argtypes = [i64, i64, i64, i64, i64, u32]
    lib.moe_y_bf16.restype = ctypes.c_int
    lib.moe_down_tail_split.argtypes = [i64, i64, i64, i64, i64, u32]
    lib.moe_down_tail_split.restype = ctypes.c_int
    lib.moe_route.argtypes = [p, i64, i64, i64, i32, p, p, p, p, p, p, i64, p, p]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route_scratch_bytes.argtypes = [i64, i64, i64]
    lib.moe_route_scratch_bytes.restype = sz
    lib.moe_gemm1_silu.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i32, i64, p, p]
    lib.moe_gemm1_silu.restype = ctypes.c_int
    lib.moe_gemm1_silu_fp8.argtypes = [p, p, p, i64, p, p, p, i64, i64, i64, i64, i64, i32, i64,
                                       p, p]
    lib.moe_gemm1_silu_fp8.restype = ctypes.c_int
    lib.moe_fp8_widens_in_gemm.argtypes = [i64, i64, i64, i64, i64, i64]
    lib.moe_fp8_widens_in_gemm.restype = ctypes.c_int
    lib.moe_topk_softmax.argtypes = [p, i64, i64, i64, ctypes.c_int, p, p, p]
    lib.moe_topk_softmax.restype = ctypes.c_int
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_release.argtypes = []
    lib.moe_release.restype = None
    _lib = lib
    return lib


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, load_library().moe_last_error().decode())


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype, ndim):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def moe_forward(hidden_states, w1, w2, topk_weights, topk_ids, out=None, flags=None,
                workspace=None, stream=None, activation="silu", alpha=1.702, limit=7.0,
                b1=None, b2=None):
    """out[T,H] fp32 = sum_k topk_weights[:,k] * expert_{topk_ids[:,k]}(hidden_states).

    ``flags=None`` calls ``moe_forward`` (internal workspace, MOE_COMBINE from
    the environment); otherwise ``moe_forward_ex`` with these flags and the
    optional ``workspace`` (a uint8 device tensor). An activation other than
    "silu" ("gelu_tanh", "gelu_erf", "swigluoai" with ``alpha``/``limit``) or
    expert biases (fp32 ``b1`` [E, 2I], ``b2`` [E, H]) call ``moe_forward_act``.
    """
    import torch

    lib = load_library()
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(w1, "w1", torch.bfloat16, 3)
    _need(w2, "w2", torch.bfloat16, 3)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, H = hidden_states.shape
    E, I2, H1 = w1.shape
    I = I2 // 2
    K = topk_ids.shape[1]
    if H1 != H or I2 % 2 or tuple(w2.shape) != (E, H, I) or tuple(topk_weights.shape) != (T, K) \
            or topk_ids.shape[0] != T:
        raise ValueError("inconsistent shapes: hidden %s w1 %s w2 %s weights %s ids %s" % (
            tuple(hidden_states.shape), tuple(w1.shape), tuple(w2.shape),
            tuple(topk_weights.shape), tuple(topk_ids.shape)))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=hidden_states.device)
    else:
        _need(out, "out", torch.float32, 2)
        if tuple(out.shape) != (T, H):
            raise ValueError("out must be [T, H]")
    args = (_ptr(hidden_states), _ptr(w1), _ptr(w2), _ptr(topk_weights), _ptr(topk_ids),
            T, H, I, E, K, _ptr(out))
    if activation != "silu" or b1 is not None or b2 is not None:
        if activation not in ACTIVATIONS:
            raise ValueError(f"unknown activation {activation!r}")
        if b1 is not None:
            _need(b1, "b1", torch.float32, 2)
            if tuple(b1.shape) != (E, 2 * I):
                raise ValueError("b1 must be [E, 2I]")
        if b2 is not None:
            _need(b2, "b2", torch.float32, 2)
            if tuple(b2.shape) != (E, H):
                raise ValueError("b2 must be [E, H]")
        ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
        if workspace is not None:
            _need(workspace, "workspace", torch.uint8, 1)
            ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
        _check(lib.moe_forward_act(
            *args[:10], ACTIVATIONS[activation], ctypes.c_float(alpha), ctypes.c_float(limit),
            None if b1 is None else _ptr(b1), None if b2 is None else _ptr(b2), args[10],
            ctypes.c_uint32(flags or 0), ws_ptr, ctypes.c_size_t(ws_bytes), _stream(stream)))
        return out
    if flags is None and workspace is None:
        _check(lib.moe_forward(*args, _stream(stream)))
    else:
        ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
        if workspace is not None:
            _need(workspace, "workspace", torch.uint8, 1)
            ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
        _check(lib.moe_forward_ex(*args, ctypes.c_uint32(flags or 0), ws_ptr,
                                  ctypes.c_size_t(ws_bytes), _stream(stream)))
    return out


def moe_forward_fp8(hidden_states, w1q, w1_scale, w2q, w2_scale, block, topk_weights, topk_ids,
                    out=None, flags=0, workspace=None, stream=None, activation="silu",
                    alpha=1.702, limit=7.0, b1=None, b2=None):
    """The forward with FP8 E4M3 expert weights: uint8 codes w1q [E,2I,H] and
    w2q [E,H,I] with fp32 scales w1_scale [E,2I,H/block], w2_scale
    [E,H,I/block] (see moe_forward_fp8 in the header)."""
    import torch

    lib = load_library()
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(w1q, "w1q", torch.uint8, 3)
    _need(w2q, "w2q", torch.uint8, 3)
    _need(w1_scale, "w1_scale", torch.float32, 3)
    _need(w2_scale, "w2_scale", torch.float32, 3)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, H = hidden_states.shape
    E, I2, H1 = w1q.shape
    I = I2 // 2
    K = topk_ids.shape[1]
    if H1 != H or tuple(w2q.shape) != (E, H, I) or block <= 0 or H % block or I % block \
            or tuple(w1_scale.shape) != (E, 2 * I, H // block) \
            or tuple(w2_scale.shape) != (E, H, I // block) \
            or tuple(topk_weights.shape) != (T, K) or topk_ids.shape[0] != T:
        raise ValueError("inconsistent shapes for the FP8 forward")
    if activation not in ACTIVATIONS:
        raise ValueError(f"unknown activation {activation!r}")
    for b, name, shape in ((b1, "b1", (E, 2 * I)), (b2, "b2", (E, H))):
        if b is not None:
            _need(b, name, torch.float32, 2)
            if tuple(b.shape) != shape:
                raise ValueError(f"{name} must be {shape}")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=hidden_states.device)
    else:
        _need(out, "out", torch.float32, 2)
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    _check(lib.moe_forward_fp8(
        _ptr(hidden_states), _ptr(w1q), _ptr(w1_scale), _ptr(w2q), _ptr(w2_scale), block,
        _ptr(topk_weights), _ptr(topk_ids), T, H, I, E, K, ACTIVATIONS[activation],
        ctypes.c_float(alpha), ctypes.c_float(limit), None if b1 is None else _ptr(b1),
        None if b2 is None else _ptr(b2), _ptr(out), ctypes.c_uint32(flags or 0), ws_ptr,
        ctypes.c_size_t(ws_bytes), _stream(stream)))
    return out


def moe_workspace_bytes(T, H, I, E, K, flags=0) -> int:
    return int(load_library().moe_workspace_bytes(T, H, I, E, K, flags))


def moe_m_tile(T, H, I, E, K, flags=0) -> int:
    v = int(load_library().moe_m_tile(T, H, I, E, K, flags))
    if v < 0:
        _check(v)
    return v


def moe_uses_decode_path(T, H, I, E, K, flags=0) -> bool:
    v = int(load_library().moe_uses_decode_path(T, H, I, E, K, flags))
    if v < 0:
        _check(v)
    return bool(v)


def moe_path(T, H, I, E, K, flags=0) -> int:
    """PATH_GROUPED, PATH_DECODE or PATH_SMALL_BATCH for these sizes and flags."""
    v = int(load_library().moe_path(T, H, I, E, K, flags))
    if v < 0:
        _check(v)
    return v


def moe_y_bf16(T, H, I, E, K, flags=0) -> bool:
    """Whether the forward rounds each expert output y_{t,k} to bf16 before
    the weighted sum for these sizes and flags."""
    v = int(load_library().moe_y_bf16(T, H, I, E, K, flags))
    if v < 0:
        _check(v)
    return bool(v)


def moe_down_tail_split(T, H, I, E, K, flags=0) -> bool:
    """Whether the forward plans the down projection's last partial round
    as column halves in a second launch for these sizes and flags."""
    v = int(load_library().moe_down_tail_split(T, H, I, E, K, flags))
    if v < 0:
        _check(v)
    return bool(v)


def moe_route(topk_ids, E, m_tile, stream=None) -> dict:
    """Routing arrays (device int32 tensors); see moe_route in the header."""
    import torch

    lib = load_library()
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, K = topk_ids.shape
    n = T * K
    cap = n + min(E, n) * (m_tile - 1)
    cap = -(-cap // m_tile) * m_tile
    dev = topk_ids.device
    r = {
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "sorted": torch.empty(max(cap, 1), dtype=torch.int32, device=dev),
        "slot_of": torch.empty(max(n, 1), dtype=torch.int32, device=dev),
        "tile_expert": torch.empty(max(cap // m_tile, 1), dtype=torch.int32, device=dev),
        "num_tiles": torch.empty(1, dtype=torch.int32, device=dev),
    }
    scratch = torch.empty(max(int(lib.moe_route_scratch_bytes(T, K, E)), 4), dtype=torch.uint8,
                          device=dev)
    _check(lib.moe_route(_ptr(topk_ids), T, K, E, m_tile, _ptr(r["counts"]), _ptr(r["offsets"]),
                         _ptr(r["sorted"]), _ptr(r["slot_of"]), _ptr(r["tile_expert"]),
                         _ptr(r["num_tiles"]), cap, _ptr(scratch), _stream(stream)))
    r["capacity"] = cap
    r["E"], r["K"], r["m_tile"], r["T"] = E, K, m_tile, T
    r["_scratch"] = scratch  # keep alive until the stream passes the work
    return r


def _check_route(route: dict, T: int, E: int, K: int, m_tile: int):
    """The routing arrays must come from moe_route for these sizes: the
    GEMMs index w1 by the tile experts and read ``capacity`` rows."""
    got = (route.get("T"), route.get("E"), route.get("K"), route.get("m_tile"))
    if got != (T, E, K, m_tile):
        raise ValueError(f"route was built for (T, E, K, m_tile) = {got}, this call needs "
                         f"{(T, E, K, m_tile)}")


def moe_gemm1_silu(hidden_states, w1, route: dict, K: int, m_tile: int, act=None, stream=None):
    """bf16 intermediate [capacity, I] of the grouped gate/up GEMM + SiLU
    (written into ``act`` if given)."""
    import torch

    lib = load_library()
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(w1, "w1", torch.bfloat16, 3)
    T, H = hidden_states.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_route(route, T, E, K, m_tile)
    cap = route["capacity"]
    if act is None:
        act = torch.zeros((max(cap, 1), I), dtype=torch.bfloat16, device=hidden_states.device)
    else:
        _need(act, "act", torch.bfloat16, 2)
        if act.shape[0] < cap or act.shape[1] != I:
            raise ValueError("act must be at least [capacity, I]")
    _check(lib.moe_gemm1_silu(_ptr(hidden_states), _ptr(w1), _ptr(route["sorted"]),
                              _ptr(route["tile_expert"]), _ptr(route["num_tiles"]), T, H, I, E, K,
                              m_tile, cap // m_tile, _ptr(act), _stream(stream)))
    return act


def moe_gemm1_silu_fp8(hidden_states, w1q, w1_scale, block: int, route: dict, K: int,
                       m_tile: int, act=None, stream=None):
    """moe_gemm1_silu with FP8 E4M3 gate/up weights (uint8 codes [E,2I,H],
    fp32 scales [E,2I,H/block]) widened in registers."""
    import torch

    lib = load_library()
    _need(hidden_states, "hidden_states", torch.bfloat16, 2)
    _need(w1q, "w1q", torch.uint8, 3)
    _need(w1_scale, "w1_scale", torch.float32, 3)
    T, H = hidden_states.shape
    E, I2, _ = w1q.shape
    I = I2 // 2
    if tuple(w1q.shape) != (E, 2 * I, H) or tuple(w1_scale.shape) != (E, 2 * I, H // block):
        raise ValueError("w1q must be [E,2I,H] and w1_scale [E,2I,H/block]")
    _check_route(route, T, E, K, m_tile)
    cap = route["capacity"]
    if act is None:
        act = torch.zeros((max(cap, 1), I), dtype=torch.bfloat16, device=hidden_states.device)
    else:
        _need(act, "act", torch.bfloat16, 2)
        if act.shape[0] < cap or act.shape[1] != I:
            raise ValueError("act must be at least [capacity, I]")
    _check(lib.moe_gemm1_silu_fp8(_ptr(hidden_states), _ptr(w1q), _ptr(w1_scale), block,
                                  _ptr(route["sorted"]), _ptr(route["tile_expert"]),
                                  _ptr(route["num_tiles"]), T, H, I, E, K, m_tile, cap // m_tile,
                                  _ptr(act), _stream(stream)))
    return act


def moe_fp8_widens_in_gemm(T: int, H: int, I: int, E: int, K: int, block: int) -> bool:
    """True when the grouped path widens FP8 fragments inside its GEMMs, False
    when it first widens the weights to bf16 in the workspace."""
    rc = load_library().moe_fp8_widens_in_gemm(T, H, I, E, K, block)
    if rc < 0:
        _check(rc)
    return rc == 1


def moe_topk_softmax(router_logits, top_k: int, renormalize: bool = True, topk_weights=None,
                     topk_ids=None, stream=None):
    """(topk_weights fp32 [T,K], topk_ids int32 [T,K]) from fp32 logits [T,E]."""
    import torch

    lib = load_library()
    _need(router_logits, "router_logits", torch.float32, 2)
    T, E = router_logits.shape
    dev = router_logits.device
    if topk_weights is None:
        topk_weights = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    _need(topk_weights, "topk_weights", torch.float32, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    if tuple(topk_weights.shape) != (T, top_k) or tuple(topk_ids.shape) != (T, top_k):
        raise ValueError("outputs must be [T, top_k]")
    _check(lib.moe_topk_softmax(_ptr(router_logits), T, E, top_k, 1 if renormalize else 0,
                                _ptr(topk_weights), _ptr(topk_ids), _stream(stream)))
    return topk_weights, topk_ids


def moe_release():
    load_library().moe_release()
