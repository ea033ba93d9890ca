"""Activation variants and expert biases on the GPU against the oracle
(the later tpu-inference fused_moe kernel.py: activation_fn, swigluoai,
ref_moe's b1/b2), on every path, through the C ABI."""
import numpy as np
import pytest
import torch

import moe_topk_ids_amd as moe
import oracle
from gpu_helpers import (MAX_ABS, REL_L2, REL_L2_BF16_INTER, cpu_inputs, random_shapes, rel_l2,
                         require_gpu, sample_rows, say, shape_inputs, to_device, y_bf16_for)
from moe_topk_ids_amd.inputs import SHAPES, bf16_bits, make_biases

pytestmark = pytest.mark.gpu

PATHS = {
    "slot": moe.FLAG_FORCE_GROUPED,
    "atomic": moe.FLAG_FORCE_GROUPED | moe.FLAG_ATOMIC_COMBINE,
    "decode": moe.FLAG_FORCE_DECODE,
    "small_batch": moe.FLAG_FORCE_SMALL_BATCH,
}
# swigluoai with a limit inside the spread of the projections, so that both
# clips are active on a good share of the elements
ACTS = [("silu", {}), ("gelu_tanh", {}), ("gelu_erf", {}),
        ("swigluoai", {"alpha": 1.702, "limit": 0.1}), ("swigluoai", {"alpha": 1.702, "limit": 7.0})]


def _oracle(d, rows, act, kw, b, bf16_inter=False, bf16_y=False):
    return oracle.moe_forward_act(
        bf16_bits(d["hidden_states"])[rows], bf16_bits(d["w1"]), bf16_bits(d["w2"]),
        d["topk_weights"].numpy()[rows], d["topk_ids"].numpy()[rows], act=act,
        b1=None if b is None else b["b1"].numpy(), b2=None if b is None else b["b2"].numpy(),
        bf16_inter=bf16_inter, bf16_y=bf16_y, **kw)


def _check(got, want, want_b16, label):
    err = float(np.max(np.abs(got.astype(np.float64) - want)))
    r, rb = rel_l2(got, want), rel_l2(got, want_b16)
    say(f"{label}: max-abs {err:.3e} rel-L2 {r:.3e} rel-L2(bf16-inter oracle) {rb:.3e}")
    assert np.all(np.isfinite(got)), label
    assert err <= MAX_ABS and r <= REL_L2 and rb <= REL_L2_BF16_INTER, label


def _run(dd, flags, act, kw, bd):
    out = moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                          dd["topk_ids"], flags=flags, activation=act,
                          b1=None if bd is None else bd["b1"], b2=None if bd is None else bd["b2"],
                          **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("act,kw", ACTS)
@pytest.mark.parametrize("bias", [False, True])
def test_variant_on_every_path(path, act, kw, bias):
    """A ragged shape (T not a multiple of any tile, several row tiles per
    expert, several 128-wide column tiles)."""
    require_gpu()
    T, H, I, E, K = 77, 256, 384, 8, 2
    d = cpu_inputs(T, H, I, E, K, seed=21)
    b = make_biases(H, I, E, seed=21) if bias else None
    dd = to_device(d)
    bd = None if b is None else to_device(b)
    rows = np.arange(T)
    got = _run(dd, PATHS[path], act, kw, bd)
    _check(got, _oracle(d, rows, act, kw, b),
           _oracle(d, rows, act, kw, b, True, y_bf16_for(d, PATHS[path])),
           f"{act}{kw}/bias={bias}/{path}")


@pytest.mark.parametrize("name,act,kw", [
    ("prefill", "swigluoai", {"alpha": 1.702, "limit": 0.1}),
    ("decode", "gelu_tanh", {}),
    ("wide", "gelu_erf", {}),
    ("large", "swigluoai", {"alpha": 1.702, "limit": 7.0}),
])
def test_variant_at_workload_size(name, act, kw):
    """Full-size workloads on the default path, with biases; the oracle on
    256 seeded token rows (every row of decode)."""
    require_gpu()
    s = SHAPES[name]
    d = shape_inputs(name)
    b = make_biases(s.H, s.I, s.E, seed=2)
    dd, bd = to_device(d), to_device(b)
    say(f"variant {act} at {name}")
    got = _run(dd, None, act, kw, bd)
    rows = sample_rows(s.T, 256, seed=4)
    _check(got[rows], _oracle(d, rows, act, kw, b),
           _oracle(d, rows, act, kw, b, True, y_bf16_for(d, None)), f"{name}/{act}")


# seeded shapes over every route and row tile (a third draw), each with the
# next activation in turn and biases on every other shape; half of them on
# the default route, half forced grouped
RANDOM_SHAPES = random_shapes(15, seed=20261207)


@pytest.mark.parametrize("idx", range(len(RANDOM_SHAPES)))
def test_variants_on_random_shapes(idx):
    require_gpu()
    T, H, I, E, K = RANDOM_SHAPES[idx]
    act, kw = ACTS[idx % len(ACTS)]
    d = cpu_inputs(T, H, I, E, K, seed=200 + idx)
    b = make_biases(H, I, E, seed=200 + idx) if idx % 2 else None
    dd = to_device(d)
    bd = None if b is None else to_device(b)
    fl = PATHS["slot"] if idx % 4 >= 2 else None
    say(f"variant random shape {idx}: T={T} H={H} I={I} E={E} K={K} act={act}{kw} "
        f"bias={b is not None} route={moe.moe_path(T, H, I, E, K, fl or 0)}")
    got = _run(dd, fl, act, kw, bd)
    rows = sample_rows(T, 32, seed=idx)
    _check(got[rows], _oracle(d, rows, act, kw, b),
           _oracle(d, rows, act, kw, b, True, y_bf16_for(d, fl)),
           f"variant random {idx} {T},{H},{I},{E},{K}/{act}")


def test_silu_variant_entry_equals_plain_entry():
    """moe_forward_act with silu and no biases is the plain forward, bit for
    bit, on every path."""
    require_gpu()
    dd = to_device(shape_inputs("tiny"))
    for path, fl in PATHS.items():
        a = moe.moe_forward(dd["hidden_states"], dd["w1"], dd["w2"], dd["topk_weights"],
                            dd["topk_ids"], flags=fl)
        lib = moe.load_library()
        b = torch.empty_like(a)
        import ctypes
        s = SHAPES["tiny"]
        rc = lib.moe_forward_act(
            ctypes.c_void_p(dd["hidden_states"].data_ptr()), ctypes.c_void_p(dd["w1"].data_ptr()),
            ctypes.c_void_p(dd["w2"].data_ptr()), ctypes.c_void_p(dd["topk_weights"].data_ptr()),
            ctypes.c_void_p(dd["topk_ids"].data_ptr()), s.T, s.H, s.I, s.E, s.K, moe.ACT_SILU,
            ctypes.c_float(1.702), ctypes.c_float(7.0), None, None,
            ctypes.c_void_p(b.data_ptr()), fl, None, 0,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == moe.MOE_OK
        torch.cuda.synchronize()
        assert torch.equal(a, b), path
