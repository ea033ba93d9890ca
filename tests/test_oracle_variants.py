"""Pins for the oracle's activation variants and expert biases (the later
tpu-inference fused_moe kernel.py: activation_fn, swigluoai, ref_moe's b1 and
b2): hand-worked values, library special cases, reductions between variants,
and closed forms for the biases."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from moe_topk_ids_amd.inputs import bf16_bits, make_biases, make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))
VARIANTS = ["silu", "gelu_tanh", "gelu_erf", "swigluoai"]


def _bits(a):
    return bf16_bits(torch.tensor(a, dtype=torch.float32).to(torch.bfloat16))


def _np(d):
    return (bf16_bits(d["hidden_states"]), bf16_bits(d["w1"]), bf16_bits(d["w2"]),
            d["topk_weights"].numpy(), d["topk_ids"].numpy())


def test_handworked_variants():
    g = json.load(open(os.path.join(HERE, "golden", "activation_handworked.json")))
    c = g["common"]
    for case in g["cases"]:
        kw = dict(act=case["act"])
        if "alpha" in case:
            kw.update(alpha=case["alpha"], limit=case["limit"])
        if "b1" in case:
            kw.update(b1=np.array(case["b1"], np.float32), b2=np.array(case["b2"], np.float32))
        args = (_bits(c["x"]), _bits(case["w1"]), _bits(c["w2"]),
                np.array(c["topk_weights"], np.float32), np.array(c["topk_ids"], np.int32))
        got = oracle.moe_forward_act(*args, **kw)
        np.testing.assert_allclose(got, np.array(case["out"]), rtol=2e-6, err_msg=case["name"])
        got64 = oracle.moe_forward_act_f64(*args, **kw)
        np.testing.assert_allclose(got64, np.array(case["out"]), rtol=1e-9, err_msg=case["name"])


@pytest.mark.parametrize("act,approx", [("gelu_tanh", "tanh"), ("gelu_erf", "none"),
                                        ("silu", None)])
def test_single_expert_is_a_dense_gated_mlp(act, approx):
    """E = K = 1 with weight 1: a dense gated MLP, checked against torch's
    own gelu / silu and linear layers in fp64."""
    d = make_inputs(16, 128, 64, 1, 1, seed=3)
    d["hidden_states"] = d["hidden_states"] * 30  # reach the non-linear range
    d["topk_weights"] = torch.ones(16, 1)
    x, w1, w2, tw, ids = _np(d)
    got = oracle.moe_forward_act_f64(x, w1, w2, tw, ids, act=act)
    xt = d["hidden_states"].double()
    g = F.linear(xt, d["w1"][0, :64].double())
    u = F.linear(xt, d["w1"][0, 64:].double())
    a = (F.silu(g) if approx is None else F.gelu(g, approximate=approx)) * u
    want = F.linear(a, d["w2"][0].double()).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-13)


def test_swigluoai_reduces_to_silu():
    """alpha = 1, no clipping (huge limit) and an up bias of -1 make
    (u - 1 + 1) * g * sigmoid(g) = silu(g) * u."""
    d = make_inputs(24, 128, 64, 4, 2, seed=4)
    d["hidden_states"] = d["hidden_states"] * 20
    args = _np(d)
    b1 = np.zeros((4, 128), np.float32)
    b1[:, 64:] = -1.0
    got = oracle.moe_forward_act_f64(*args, act="swigluoai", alpha=1.0, limit=1e30, b1=b1)
    want = oracle.moe_forward_act_f64(*args, act="silu")
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-14)


def test_swigluoai_limit_clips():
    """Past the limit nothing changes: gate values above it and up values
    outside [-limit, limit] give the output of inputs sitting at the limit.
    Scaling the gate weights up (all gates >= limit) leaves the result equal
    to the closed form (clip(u) + 1) * L * sigmoid(alpha * L)."""
    d = make_inputs(8, 128, 64, 1, 1, seed=5)
    d["topk_weights"] = torch.ones(8, 1)
    w1 = d["w1"].float().clone()
    w1[0, :64] = w1[0, :64].abs() * 50  # every gate far above the limit
    d["w1"] = w1.to(torch.bfloat16)
    d["hidden_states"] = d["hidden_states"].abs()
    x, w1b, w2, tw, ids = _np(d)
    L, alpha = 0.05, 1.702
    got = oracle.moe_forward_act_f64(x, w1b, w2, tw, ids, act="swigluoai", alpha=alpha, limit=L)
    xt = d["hidden_states"].double()
    u = F.linear(xt, d["w1"][0, 64:].double())
    a = (u.clamp(-L, L) + 1) * (L * torch.sigmoid(torch.tensor(alpha * L, dtype=torch.float64)))
    want = F.linear(a, d["w2"][0].double()).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-14)


def test_b1_is_a_constant_input_feature():
    """A gate/up bias equals one more input feature fixed at 1 whose weights
    are the biases (bf16-representable biases, fp64 sums)."""
    T, H, I, E, K = 12, 128, 64, 4, 2
    d = make_inputs(T, H, I, E, K, seed=6)
    b1 = make_biases(H, I, E, seed=6)["b1"].to(torch.bfloat16).float()
    x, w1, w2, tw, ids = _np(d)
    got = oracle.moe_forward_act_f64(x, w1, w2, tw, ids, act="gelu_tanh", b1=b1.numpy())
    # the hidden size is both the contraction of w1 and the output width, so
    # the extra feature also adds an output column, fed by zero w2 rows
    xa = torch.cat([d["hidden_states"], torch.ones(T, 1, dtype=torch.bfloat16)], dim=1)
    w1a = torch.cat([d["w1"], b1.to(torch.bfloat16).unsqueeze(-1)], dim=2)
    w2a = torch.cat([d["w2"], torch.zeros(E, 1, I, dtype=torch.bfloat16)], dim=1)
    want = oracle.moe_forward_act_f64(bf16_bits(xa), bf16_bits(w1a), bf16_bits(w2a), tw, ids,
                                      act="gelu_tanh")
    assert np.all(want[:, H] == 0)
    np.testing.assert_allclose(got, want[:, :H], rtol=1e-11, atol=1e-15)


def test_b2_adds_the_weighted_biases():
    """out(b2) - out(no b2) = sum_k w[t,k] * b2[e_k] (fp64)."""
    T, H, I, E, K = 20, 128, 64, 8, 3
    d = make_inputs(T, H, I, E, K, seed=7)
    b2 = make_biases(H, I, E, seed=7)["b2"].numpy()
    args = _np(d)
    diff = (oracle.moe_forward_act_f64(*args, act="swigluoai", b2=b2)
            - oracle.moe_forward_act_f64(*args, act="swigluoai"))
    tw, ids = args[3].astype(np.float64), args[4]
    want = np.einsum("tk,tkh->th", tw, b2[ids].astype(np.float64))
    np.testing.assert_allclose(diff, want, rtol=1e-9, atol=1e-14)


@pytest.mark.parametrize("act", VARIANTS)
def test_fp32_oracle_close_to_fp64(act):
    T, H, I, E, K = 32, 256, 128, 8, 2
    d = make_inputs(T, H, I, E, K, seed=8)
    b = make_biases(H, I, E, seed=8)
    args = _np(d)
    kw = dict(act=act, b1=b["b1"].numpy(), b2=b["b2"].numpy())
    if act == "swigluoai":
        kw.update(alpha=1.702, limit=0.1)  # small limit: both clips active
    got = oracle.moe_forward_act(*args, **kw).astype(np.float64)
    want = oracle.moe_forward_act_f64(*args, **kw)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) < 1e-6


def test_silu_entry_point_is_the_variant_entry_point():
    d = make_inputs(16, 128, 128, 4, 2, seed=9)
    args = _np(d)
    assert np.array_equal(oracle.moe_forward(*args), oracle.moe_forward_act(*args, act="silu"))
    assert np.array_equal(oracle.moe_forward(*args, bf16_inter=True),
                          oracle.moe_forward_act(*args, act="silu", bf16_inter=True))
