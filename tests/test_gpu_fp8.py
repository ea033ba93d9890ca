"""FP8 E4M3 expert weights with per-block fp32 scales (the later
tpu-inference fused_moe kernel.py's sub-channel quantisation) on the GPU,
against the oracle's quantised forward, on every path, through the C ABI."""
import numpy as np
import pytest
import torch

import moe_topk_ids_amd as moe
import oracle
from gpu_helpers import (MAX_ABS, REL_L2, REL_L2_BF16_INTER, cpu_inputs, random_shapes, rel_l2,
                         require_gpu, sample_rows, say, shape_inputs, to_device, y_bf16_for)
from moe_topk_ids_amd.inputs import SHAPES, bf16_bits, make_biases, make_fp8_weights

pytestmark = pytest.mark.gpu

PATHS = {
    "decode": moe.FLAG_FORCE_DECODE,
    "small_batch": moe.FLAG_FORCE_SMALL_BATCH,
    "slot": moe.FLAG_FORCE_GROUPED,
    "atomic": moe.FLAG_FORCE_GROUPED | moe.FLAG_ATOMIC_COMBINE,
}


def _widened(q, block):
    """The grouped path's bf16 weights: fp8 value times scale, rounded to
    bf16 (computed here with torch on the CPU)."""
    def one(codes, scales):
        v = codes.view(torch.float8_e4m3fn).float()
        return (v * scales.repeat_interleave(block, dim=-1)).to(torch.bfloat16)
    return one(q["w1q"], q["w1s"]), one(q["w2q"], q["w2s"])


def _oracle(d, q, rows, kw, b, bf16_inter=False):
    return oracle.moe_forward_q(
        bf16_bits(d["hidden_states"])[rows], q["w1q"].numpy(), q["w1s"].numpy(),
        q["w2q"].numpy(), q["w2s"].numpy(), q["block"], d["topk_weights"].numpy()[rows],
        d["topk_ids"].numpy()[rows], b1=None if b is None else b["b1"].numpy(),
        b2=None if b is None else b["b2"].numpy(), bf16_inter=bf16_inter, **kw)


def _oracle_widened(d, q, rows, kw, b, flags):
    """The grouped path's tight oracle: bf16-widened weights, bf16 activation,
    expert outputs rounded to bf16 where the forward does."""
    w1, w2 = _widened(q, q["block"])
    return oracle.moe_forward_act(
        bf16_bits(d["hidden_states"])[rows], bf16_bits(w1), bf16_bits(w2),
        d["topk_weights"].numpy()[rows], d["topk_ids"].numpy()[rows],
        b1=None if b is None else b["b1"].numpy(), b2=None if b is None else b["b2"].numpy(),
        bf16_inter=True, bf16_y=y_bf16_for(d, (flags or 0) | moe.FLAG_FP8_WEIGHTS), **kw)


def _run(dd, qd, flags, kw, bd):
    out = moe.moe_forward_fp8(dd["hidden_states"], qd["w1q"], qd["w1s"], qd["w2q"], qd["w2s"],
                              qd["block"], dd["topk_weights"], dd["topk_ids"], flags=flags,
                              b1=None if bd is None else bd["b1"],
                              b2=None if bd is None else bd["b2"], **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(got, want, want_tight, label):
    err = float(np.max(np.abs(got.astype(np.float64) - want)))
    r, rt = rel_l2(got, want), rel_l2(got, want_tight)
    say(f"{label}: max-abs {err:.3e} rel-L2 {r:.3e} rel-L2(tight oracle) {rt:.3e}")
    assert np.all(np.isfinite(got)), label
    assert err <= MAX_ABS and r <= REL_L2 and rt <= REL_L2_BF16_INTER, label


def _to_dev(q):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in q.items()}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("act,kw,bias", [("silu", {}, False),
                                         ("swigluoai", {"alpha": 1.702, "limit": 0.1}, True),
                                         ("gelu_tanh", {}, True)])
@pytest.mark.parametrize("block", [128, 256])
def test_fp8_on_every_path(path, act, kw, bias, block):
    require_gpu()
    T, H, I, E, K = 77, 512, 768, 8, 2
    d = cpu_inputs(T, H, I, E, K, seed=31)
    q = make_fp8_weights(d, block)
    b = make_biases(H, I, E, seed=31) if bias else None
    dd, qd = to_device(d), _to_dev(q)
    bd = None if b is None else to_device(b)
    kw = dict(kw, activation=act)
    okw = {k: v for k, v in kw.items() if k != "activation"}
    okw["act"] = act
    got = _run(dd, qd, PATHS[path], kw, bd)
    rows = np.arange(T)
    want = _oracle(d, q, rows, okw, b)
    # the streaming paths read the codes themselves; the grouped path works
    # on the bf16-widened weights
    tight = (_oracle(d, q, rows, okw, b, True) if path in ("decode", "small_batch")
             else _oracle_widened(d, q, rows, okw, b, PATHS[path]))
    _check(got, want, tight, f"fp8/{act}/bias={bias}/block={block}/{path}")


# seeded shapes over every route and row tile (a different draw from the bf16
# sweep), each with one of the activations, biases on every other shape, and
# scale blocks of 128 or 256 where 256 divides H and I
RANDOM_SHAPES = random_shapes(12, seed=20261204)
RANDOM_ACTS = [("silu", {}), ("gelu_tanh", {}), ("swigluoai", {"alpha": 1.702, "limit": 0.1}),
               ("gelu_erf", {})]


@pytest.mark.parametrize("idx", range(len(RANDOM_SHAPES)))
def test_fp8_and_variants_on_random_shapes(idx):
    require_gpu()
    T, H, I, E, K = RANDOM_SHAPES[idx]
    act, kw = RANDOM_ACTS[idx % len(RANDOM_ACTS)]
    block = 256 if idx % 3 == 0 and H % 256 == 0 and I % 256 == 0 else 128
    d = cpu_inputs(T, H, I, E, K, seed=100 + idx)
    q = make_fp8_weights(d, block)
    b = make_biases(H, I, E, seed=100 + idx) if idx % 2 else None
    dd, qd = to_device(d), _to_dev(q)
    bd = None if b is None else to_device(b)
    route = moe.moe_path(T, H, I, E, K, moe.FLAG_FP8_WEIGHTS)
    say(f"fp8 random shape {idx}: T={T} H={H} I={I} E={E} K={K} act={act} bias={b is not None} "
        f"block={block} route={route}")
    kw = dict(kw, activation=act)
    okw = {k: v for k, v in kw.items() if k != "activation"}
    okw["act"] = act
    got = _run(dd, qd, None, kw, bd)
    rows = sample_rows(T, 32, seed=idx)
    want = _oracle(d, q, rows, okw, b)
    tight = (_oracle(d, q, rows, okw, b, True) if route != moe.PATH_GROUPED
             else _oracle_widened(d, q, rows, okw, b, None))
    _check(got[rows], want, tight, f"fp8 random {idx} {T},{H},{I},{E},{K}/{act}")


@pytest.mark.parametrize("name", ["decode", "prefill", "wide"])
def test_fp8_at_workload_size(name):
    """Default path at the workload's full size; the oracle on 256 seeded
    token rows (every row of decode)."""
    require_gpu()
    s = SHAPES[name]
    d = shape_inputs(name)
    q = make_fp8_weights(d, 128 if s.I % 256 else 256)
    dd, qd = to_device(d), _to_dev(q)
    say(f"fp8 forward at {name}")
    got = _run(dd, qd, 0, {}, None)
    rows = sample_rows(s.T, 256, seed=6)
    want = _oracle(d, q, rows, {"act": "silu"}, None)
    path = moe.moe_path(s.T, s.H, s.I, s.E, s.K, moe.FLAG_FP8_WEIGHTS)
    tight = (_oracle(d, q, rows, {"act": "silu"}, None, True) if path != moe.PATH_GROUPED
             else _oracle_widened(d, q, rows, {"act": "silu"}, None, 0))
    _check(got[rows], want, tight, f"fp8/{name}")


@pytest.mark.parametrize("H,I,block,native", [(4096, 256, 128, True),    # 32 scale blocks
                                               (4224, 384, 128, False),   # 33: widened first
                                               (4224, 256, 128, False)])
def test_fp8_grouped_at_the_scale_block_limit(H, I, block, native):
    """The grouped GEMMs keep a tile's scales in LDS for up to 32 blocks per
    row; longer rows go through the bf16 widening pass. Both against the
    oracle."""
    require_gpu()
    T, E, K = 150, 4, 2
    d = cpu_inputs(T, H, I, E, K, seed=33)
    q = make_fp8_weights(d, block)
    dd, qd = to_device(d), _to_dev(q)
    say(f"fp8 grouped H={H} I={I} block={block} native={native}")
    got = _run(dd, qd, moe.FLAG_FORCE_GROUPED, {}, None)
    rows = np.arange(T)
    want = _oracle(d, q, rows, {"act": "silu"}, None)
    tight = _oracle_widened(d, q, rows, {"act": "silu"}, None, moe.FLAG_FORCE_GROUPED)
    _check(got, want, tight, f"fp8/grouped H={H} I={I}")


@pytest.mark.parametrize("name,m_tile", [("tiny", None), ("wide", None), ("tiny", 192),
                                         ("tiny", 64)])
def test_fp8_gemm1_intermediate(name, m_tile):
    """moe_gemm1_silu_fp8 (codes widened in registers) vs the oracle's per-slot
    bf16 activation on the bf16-widened weights: at most one bf16 ulp apart
    (the k order inside a stage differs), nearly all identical. At the
    workload's own row tile and at the other tile shapes."""
    require_gpu()
    s = SHAPES[name]
    d = shape_inputs(name)
    q = make_fp8_weights(d, 128)
    dd, qd = to_device(d), _to_dev(q)
    M = m_tile or moe.moe_m_tile(s.T, s.H, s.I, s.E, s.K)
    say(f"fp8 intermediate {name} M={M}")
    r = moe.moe_route(dd["topk_ids"], s.E, M)
    act = moe.moe_gemm1_silu_fp8(dd["hidden_states"], qd["w1q"], qd["w1s"], 128, r, s.K, M)
    torch.cuda.synchronize()
    slot_of = r["slot_of"].cpu().numpy()
    rows = sample_rows(s.T, 48, seed=4)
    slots = (rows[:, None] * s.K + np.arange(s.K)[None, :]).ravel()
    got = act.cpu().view(torch.int16).numpy().view(np.uint16)[slot_of[slots]]
    w1, _ = _widened(q, 128)
    want = oracle.slot_act_bf16(bf16_bits(d["hidden_states"])[rows], bf16_bits(w1),
                                d["topk_ids"].numpy()[rows])
    gf = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy()
    wf = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
    tol = 2.0 ** -7 * np.maximum(np.abs(gf), np.abs(wf)) + 1e-7
    exact = float(np.mean(got == want))
    say(f"  identical {exact:.4f}, max |diff| {np.max(np.abs(gf - wf)):.3e}")
    assert np.all(np.abs(gf - wf) <= tol)
    assert exact >= 0.97


def test_fp8_caller_workspace_for_the_grouped_path():
    require_gpu()
    T, H, I, E, K = 200, 256, 256, 4, 2
    d = cpu_inputs(T, H, I, E, K, seed=32)
    q = make_fp8_weights(d, 128)
    dd, qd = to_device(d), _to_dev(q)
    fl = moe.FLAG_FORCE_GROUPED
    ref = _run(dd, qd, fl, {}, None)
    n = moe.moe_workspace_bytes(T, H, I, E, K, fl | moe.FLAG_FP8_WEIGHTS)
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    out = moe.moe_forward_fp8(dd["hidden_states"], qd["w1q"], qd["w1s"], qd["w2q"], qd["w2s"],
                              128, dd["topk_weights"], dd["topk_ids"], flags=fl, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)
    too_small = torch.empty(n - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_fp8(dd["hidden_states"], qd["w1q"], qd["w1s"], qd["w2q"], qd["w2s"], 128,
                            dd["topk_weights"], dd["topk_ids"], flags=fl, workspace=too_small)
    assert ei.value.code == moe.MOE_ERR_WORKSPACE
