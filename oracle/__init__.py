"""Python access to the plain CPU oracle in ``moe_oracle.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers. The GPU library never
imports this package and this package imports nothing from the GPU library.

bf16 tensors travel as ``numpy.uint16`` arrays holding the raw bf16 bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc: IEEE fp32, no contraction, no fast-math."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
           "-fPIC", "-std=c11", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_route.argtypes = [p, i64, i64, i64, i64, p, p, p, i64, p, p, i64, p]
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_moe_forward.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, ctypes.c_int, p]
    lib.oracle_moe_forward.restype = None
    lib.oracle_moe_forward_f64.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, p]
    lib.oracle_moe_forward_f64.restype = None
    f32, f64 = ctypes.c_float, ctypes.c_double
    lib.oracle_moe_forward_act.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, ctypes.c_int,
                                           f32, f32, p, p, ctypes.c_int, p]
    lib.oracle_moe_forward_act.restype = None
    lib.oracle_moe_forward_act_f64.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64,
                                               ctypes.c_int, f64, f64, p, p, p]
    lib.oracle_moe_forward_act_f64.restype = None
    lib.oracle_slot_act_bf16.argtypes = [p, p, p, i64, i64, i64, i64, i64, p]
    lib.oracle_slot_act_bf16.restype = None
    lib.oracle_moe_forward_q.argtypes = [p, p, p, p, p, i64, p, p, i64, i64, i64, i64, i64,
                                         ctypes.c_int, f32, f32, p, p, ctypes.c_int, p]
    lib.oracle_moe_forward_q.restype = None
    lib.oracle_fp8_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3_to_f32.restype = ctypes.c_float
    lib.oracle_topk_softmax.argtypes = [p, i64, i64, i64, ctypes.c_int, p, p]
    lib.oracle_topk_softmax.restype = None
    lib.oracle_f32_to_bf16.argtypes = [p, p, i64]
    lib.oracle_bf16_to_f32.argtypes = [p, p, i64]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def route(ids: np.ndarray, E: int, M: int):
    """Routing oracle: counts, offsets, sorted, slot_of, tile_expert, num_tiles.

    ``ids`` is int32 [T,K]. ``sorted`` has length P = offsets[E] and
    ``tile_expert`` length P // M.
    """
    lib = _load()
    ids = _c(ids, np.int32)
    T, K = ids.shape
    n = T * K
    cap = n + E * (M - 1)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_ = np.zeros(max(cap, 1), np.int32)
    slot_of = np.zeros(max(n, 1), np.int32)
    tile_expert = np.zeros(max(cap // M, 1), np.int32)
    num_tiles = np.zeros(1, np.int32)
    rc = lib.oracle_route(_ptr(ids), T, K, E, M, _ptr(counts), _ptr(offsets), _ptr(sorted_),
                          cap, _ptr(slot_of), _ptr(tile_expert), cap // M, _ptr(num_tiles))
    if rc != 0:
        raise RuntimeError("oracle_route: capacity exceeded")
    P = int(offsets[E])
    return dict(counts=counts, offsets=offsets, sorted=sorted_[:P].copy(),
                slot_of=slot_of[:n].copy(), tile_expert=tile_expert[:P // M].copy(),
                num_tiles=int(num_tiles[0]))


def _mode(bf16_inter: bool, bf16_y: bool) -> int:
    """The C oracle's mode bits: 1 rounds the activation to bf16, 2 rounds
    each expert's down-projection result y_{t,k} to bf16 (before b2 and the
    routing weight)."""
    return (1 if bf16_inter else 0) | (2 if bf16_y else 0)


def moe_forward(x, w1, w2, topk_weights, topk_ids, bf16_inter: bool = False,
                bf16_y: bool = False) -> np.ndarray:
    """fp32 oracle forward. x uint16 [T,H]; w1 uint16 [E,2I,H]; w2 uint16 [E,H,I]."""
    lib = _load()
    x, w1, w2 = _c(x, np.uint16), _c(w1, np.uint16), _c(w2, np.uint16)
    tw, ids = _c(topk_weights, np.float32), _c(topk_ids, np.int32)
    T, H = x.shape
    E, I2, H2 = w1.shape
    I = I2 // 2
    K = ids.shape[1] if ids.ndim == 2 else 0
    assert H2 == H and w2.shape == (E, H, I) and tw.shape == ids.shape == (T, K)
    out = np.zeros((T, H), np.float32)
    lib.oracle_moe_forward(_ptr(x), _ptr(w1), _ptr(w2), _ptr(tw), _ptr(ids), T, H, I, E, K,
                           _mode(bf16_inter, bf16_y), _ptr(out))
    return out


def moe_forward_f64(x, w1, w2, topk_weights, topk_ids) -> np.ndarray:
    """Same definition evaluated in fp64 (weights widened from fp32)."""
    lib = _load()
    x, w1, w2 = _c(x, np.uint16), _c(w1, np.uint16), _c(w2, np.uint16)
    tw, ids = _c(topk_weights, np.float64), _c(topk_ids, np.int32)
    T, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    K = ids.shape[1]
    out = np.zeros((T, H), np.float64)
    lib.oracle_moe_forward_f64(_ptr(x), _ptr(w1), _ptr(w2), _ptr(tw), _ptr(ids), T, H, I, E, K,
                               _ptr(out))
    return out


ACTIVATIONS = {"silu": 0, "gelu_tanh": 1, "swigluoai": 2, "gelu_erf": 3}


def _opt(a, dtype):
    return None if a is None else _c(a, dtype)


def _optptr(a):
    return None if a is None else _ptr(a)


def moe_forward_act(x, w1, w2, topk_weights, topk_ids, act: str = "silu", alpha: float = 1.702,
                    limit: float = 7.0, b1=None, b2=None, bf16_inter: bool = False,
                    bf16_y: bool = False) -> np.ndarray:
    """fp32 oracle forward with an activation variant and optional fp32
    biases b1 [E, 2I] (gate, then up) and b2 [E, H]."""
    lib = _load()
    x, w1, w2 = _c(x, np.uint16), _c(w1, np.uint16), _c(w2, np.uint16)
    tw, ids = _c(topk_weights, np.float32), _c(topk_ids, np.int32)
    b1, b2 = _opt(b1, np.float32), _opt(b2, np.float32)
    T, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    K = ids.shape[1]
    assert b1 is None or b1.shape == (E, 2 * I)
    assert b2 is None or b2.shape == (E, H)
    out = np.zeros((T, H), np.float32)
    lib.oracle_moe_forward_act(_ptr(x), _ptr(w1), _ptr(w2), _ptr(tw), _ptr(ids), T, H, I, E, K,
                               ACTIVATIONS[act], alpha, limit, _optptr(b1), _optptr(b2),
                               _mode(bf16_inter, bf16_y), _ptr(out))
    return out


def moe_forward_act_f64(x, w1, w2, topk_weights, topk_ids, act: str = "silu",
                        alpha: float = 1.702, limit: float = 7.0, b1=None, b2=None) -> np.ndarray:
    """The same definition in fp64 (weights and biases widened)."""
    lib = _load()
    x, w1, w2 = _c(x, np.uint16), _c(w1, np.uint16), _c(w2, np.uint16)
    tw, ids = _c(topk_weights, np.float64), _c(topk_ids, np.int32)
    b1, b2 = _opt(b1, np.float64), _opt(b2, np.float64)
    T, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    K = ids.shape[1]
    out = np.zeros((T, H), np.float64)
    lib.oracle_moe_forward_act_f64(_ptr(x), _ptr(w1), _ptr(w2), _ptr(tw), _ptr(ids), T, H, I, E,
                                   K, ACTIVATIONS[act], alpha, limit, _optptr(b1), _optptr(b2),
                                   _ptr(out))
    return out


def moe_forward_q(x, w1q, w1s, w2q, w2s, block: int, topk_weights, topk_ids, act: str = "silu",
                  alpha: float = 1.702, limit: float = 7.0, b1=None, b2=None,
                  bf16_inter: bool = False, bf16_y: bool = False) -> np.ndarray:
    """fp32 oracle forward with FP8 E4M3 weights (uint8 codes) and fp32
    per-block scales: w1q [E,2I,H], w1s [E,2I,H/block], w2q [E,H,I],
    w2s [E,H,I/block]."""
    lib = _load()
    x = _c(x, np.uint16)
    w1q, w2q = _c(w1q, np.uint8), _c(w2q, np.uint8)
    w1s, w2s = _c(w1s, np.float32), _c(w2s, np.float32)
    tw, ids = _c(topk_weights, np.float32), _c(topk_ids, np.int32)
    b1, b2 = _opt(b1, np.float32), _opt(b2, np.float32)
    T, H = x.shape
    E, I2, _ = w1q.shape
    I = I2 // 2
    K = ids.shape[1]
    assert w1q.shape == (E, 2 * I, H) and w2q.shape == (E, H, I)
    assert w1s.shape == (E, 2 * I, H // block) and w2s.shape == (E, H, I // block)
    out = np.zeros((T, H), np.float32)
    lib.oracle_moe_forward_q(_ptr(x), _ptr(w1q), _ptr(w1s), _ptr(w2q), _ptr(w2s), block,
                             _ptr(tw), _ptr(ids), T, H, I, E, K, ACTIVATIONS[act], alpha, limit,
                             _optptr(b1), _optptr(b2), _mode(bf16_inter, bf16_y), _ptr(out))
    return out


def fp8_e4m3_to_f32(codes) -> np.ndarray:
    lib = _load()
    return np.array([lib.oracle_fp8_e4m3_to_f32(int(c)) for c in np.asarray(codes).ravel()],
                    np.float32).reshape(np.shape(codes))


def slot_act_bf16(x, w1, topk_ids) -> np.ndarray:
    """Per-slot activation silu(g)*u rounded to bf16, as uint16 [T*K, I]."""
    lib = _load()
    x, w1, ids = _c(x, np.uint16), _c(w1, np.uint16), _c(topk_ids, np.int32)
    T, H = x.shape
    E, I2, _ = w1.shape
    I = I2 // 2
    K = ids.shape[1]
    out = np.zeros((T * K, I), np.uint16)
    lib.oracle_slot_act_bf16(_ptr(x), _ptr(w1), _ptr(ids), T, H, I, E, K, _ptr(out))
    return out


def topk_softmax(logits, K: int, renormalize: bool = True):
    """Router oracle: (weights fp32 [T,K], ids int32 [T,K]) from fp32 logits [T,E]."""
    lib = _load()
    logits = _c(logits, np.float32)
    T, E = logits.shape
    w = np.zeros((T, K), np.float32)
    ids = np.zeros((T, K), np.int32)
    lib.oracle_topk_softmax(_ptr(logits), T, E, K, 1 if renormalize else 0, _ptr(w), _ptr(ids))
    return w, ids


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    lib = _load()
    a = _c(a, np.float32)
    out = np.zeros(a.shape, np.uint16)
    lib.oracle_f32_to_bf16(_ptr(a), _ptr(out), a.size)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    lib = _load()
    a = _c(a, np.uint16)
    out = np.zeros(a.shape, np.float32)
    lib.oracle_bf16_to_f32(_ptr(a), _ptr(out), a.size)
    return out


def omp_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS, else the
    runtime's default)."""
    lib = _load()
    lib.omp_get_max_threads.restype = ctypes.c_int
    return int(lib.omp_get_max_threads())


def set_omp_threads(n: int) -> None:
    """Threads for the oracle's later OpenMP loops started from this thread."""
    lib = _load()
    lib.omp_set_num_threads.argtypes = [ctypes.c_int]
    lib.omp_set_num_threads(int(n))
