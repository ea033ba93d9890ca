"""moe_forward_noalloc (the forward with its workspace in a static device
array, for callers that cannot allocate) against moe_forward_ex through the
C ABI: the same kernels on the same inputs, so the same bits, over
consecutive calls that reuse the array, the second with a smaller input."""
import ctypes

import numpy as np
import pytest
import torch

import moe_topk_ids_amd as moe
from gpu_helpers import cpu_inputs, require_gpu, say, shape_inputs, to_device

pytestmark = pytest.mark.gpu


def _lib():
    lib = moe.load_library()
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.moe_forward_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, p,
                                        ctypes.c_uint32, p]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    return lib


def _noalloc(dd, flags):
    lib = _lib()
    T, H = dd["hidden_states"].shape
    E, I2, _ = dd["w1"].shape
    K = dd["topk_ids"].shape[1]
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.moe_forward_noalloc(P(dd["hidden_states"]), P(dd["w1"]), P(dd["w2"]),
                                 P(dd["topk_weights"]), P(dd["topk_ids"]), T, H, I2 // 2, E, K,
                                 P(out), flags,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == moe.MOE_OK, lib.moe_last_error().decode()
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ex(dd, flags):
    out = moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                          dd["topk_ids"], flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("flags,label", [
    (moe.FLAG_FORCE_GROUPED, "grouped"),
    (0, "default path"),
    (moe.FLAG_FORCE_GROUPED | moe.FLAG_ATOMIC_COMBINE, "grouped, atomic combine"),
])
def test_noalloc_equals_forward_ex_on_consecutive_calls(flags, label):
    """The prefill workload (the largest the array holds on the grouped path),
    then the tiny one: both bitwise equal to moe_forward_ex's output."""
    require_gpu()
    big = to_device(shape_inputs("prefill"))
    small = to_device(shape_inputs("tiny"))
    for name, dd in (("prefill", big), ("tiny", small)):
        say(f"noalloc {label} {name}")
        a = _noalloc(dd, flags)
        b = _ex(dd, flags)
        assert np.all(np.isfinite(a)), name
        assert np.array_equal(a, b), f"{label}/{name}"


def test_noalloc_streaming_paths_then_grouped():
    """The per-token and small-batch paths, then a grouped call, then the
    per-token path again with a smaller input."""
    require_gpu()
    dec = to_device(shape_inputs("decode"))
    mid = to_device(cpu_inputs(40, 2048, 768, 128, 8, seed=9))
    tiny = to_device(shape_inputs("tiny"))
    for dd, fl, label in ((mid, moe.FLAG_FORCE_SMALL_BATCH, "small batch T=40"),
                          (mid, moe.FLAG_FORCE_DECODE, "per-token T=40"),
                          (tiny, moe.FLAG_FORCE_GROUPED, "grouped tiny"),
                          (dec, 0, "decode T=1")):
        say(f"noalloc {label}")
        assert np.array_equal(_noalloc(dd, fl), _ex(dd, fl)), label


def test_noalloc_rejects_sizes_beyond_the_array():
    """The large workload needs more than the static array: a clear error,
    nothing launched, and the next call still works."""
    require_gpu()
    lib = _lib()
    p = ctypes.c_void_p(0)
    rc = lib.moe_forward_noalloc(p, p, p, p, p, 15381, 4096, 4096, 8, 2, p, 0, p)
    assert rc == moe.MOE_ERR_WORKSPACE
    msg = lib.moe_last_error().decode()
    assert "static scratch" in msg and str(moe.NOALLOC_SCRATCH_BYTES) in msg
    tiny = to_device(shape_inputs("tiny"))
    assert np.array_equal(_noalloc(tiny, 0), _ex(tiny, 0))
